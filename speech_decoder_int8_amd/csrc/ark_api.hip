// C ABI of the decoder step: host-side validation, workspace planning and
// kernel sequencing.  Validation touches no HIP API, so every error path can
// be exercised without a GPU; a call that fails validation enqueues nothing.
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/ark.h"
#include "common.hpp"
#include "kernels.hpp"

using namespace ark;

// Scratch of ark_decode_step_noalloc, for callers that cannot allocate
// device memory (code under graph capture, tight serving loops, harnesses
// that forbid hipMalloc): one copy per device, held until the process ends.
// In host code the name is a stand-in, not a device address: the device
// address comes from hipGetSymbolAddress, once per device.
constexpr size_t kNoAllocBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

struct Plan {
  size_t x, rs, codes, qkv, q, attn, a, stats, qs, qz, part, done, rowpart, gsk, mega, hn, total;
};

bool use_mega(const ark_dims& d, int B, int S) {
  if (B != 1 || S != 1) return false;
  if (!decode_mega_supported(d.hidden, d.n_heads, d.n_kv_heads, d.head_dim, d.intermediate,
                             d.max_total_len, d.n_layers))
    return false;
  const char* e = getenv("ARK_DECODE_PATH");
  return !(e && strcmp(e, "multi") == 0);
}

Plan plan(const ark_dims& d, int B, int S) {
  const size_t R = (size_t)B * S;
  const size_t H = d.hidden, Q = (size_t)d.n_heads * d.head_dim;
  const size_t KV = (size_t)d.n_kv_heads * d.head_dim, I = d.intermediate;
  const size_t Kmax = std::max(std::max(H, Q), I);
  Plan p;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes);
    return at;
  };
  p.x = take(R * H * 4);
  p.rs = take(R * 8);
  p.codes = take(R * Kmax);
  p.qkv = take(R * (Q + 2 * KV) * 4);
  p.q = take(R * Q * 4);
  p.attn = take(R * Q * 4);
  p.a = take(R * I * 4);
  p.stats = take(2 * (size_t)kStatsSetInts * 4);
  p.qs = take((size_t)std::max(B, 64) * 4);
  p.qz = take((size_t)std::max(B, 64) * 4);
  // decode-only regions are always reserved, so a workspace sized for a
  // prefill of B sequences also serves their decode steps
  p.part = take(std::max(attention_ws_bytes(B, 1, d.n_heads, d.max_total_len),
                         attention_ws_bytes(B, S, d.n_heads, d.max_total_len)));
  p.done = take((size_t)kMaxBatch * 4);
  // split sums of the decode GEMMs that run their epilogue per row
  p.rowpart = take(gemm_rows_part_bytes((int)std::min<size_t>(B, 64), (int)H));
  p.gsk = take(gemm_ws_bytes(R));
  p.mega = take(B == 1 ? decode_mega_ws_bytes(d.n_layers, d.max_total_len) : 0);
  p.hn = take((size_t)B * H * 4);  // final-normed rows of the int4 LM tier
  p.total = o;
  return p;
}

// Re-anchored parity record layout (ark_dump_layout): per recorded layer
// the fields of ark_dump_field, each 256-byte aligned; after the layer
// records the LM-head record.
struct DumpLayout {
  size_t f[ARK_DUMP_NFIELDS];
  size_t rec;
  size_t head[4];  // relative to the head record
  size_t head_bytes;
};

DumpLayout dump_layout(const ark_dims& d, int B, int S) {
  const size_t R = (size_t)B * S, H = d.hidden, Q = (size_t)d.n_heads * d.head_dim;
  const size_t KV = (size_t)d.n_kv_heads * d.head_dim, I = d.intermediate;
  const size_t sz[ARK_DUMP_NFIELDS] = {R * H * 4, R * (Q + 2 * KV) * 4, R * Q * 4, R * H * 4,
                                       R * H * 4, R * I * 4,            R * H * 4, R * H,
                                       R * Q,     R * H,                R * I,     4 * (size_t)B * 4,
                                       4 * (size_t)B * 4};
  DumpLayout L;
  size_t o = 0;
  for (int i = 0; i < ARK_DUMP_NFIELDS; ++i) {
    L.f[i] = o;
    o += align_up(sz[i]);
  }
  L.rec = o;
  const size_t hs[4] = {(size_t)B * H * 4, (size_t)B * H, (size_t)B * 4, (size_t)B * 4};
  o = 0;
  for (int i = 0; i < 4; ++i) {
    L.head[i] = o;
    o += align_up(hs[i]);
  }
  L.head_bytes = o;
  return L;
}

int popcount_below(uint64_t mask, int l) {
  return __builtin_popcountll(l >= 64 ? mask : (mask & ((1ull << l) - 1)));
}

size_t dump_total(const ark_dims& d, int B, int S, uint64_t mask) {
  const DumpLayout L = dump_layout(d, B, S);
  return (size_t)popcount_below(mask, d.n_layers) * L.rec + L.head_bytes;
}

DumpRec dump_rec(const ark_dims& d, int B, int S, uint64_t mask, void* base) {
  const DumpLayout L = dump_layout(d, B, S);
  DumpRec r;
  r.base = (char*)base;
  r.mask = d.n_layers >= 64 ? mask : (mask & ((1ull << d.n_layers) - 1));
  r.rec = L.rec;
  for (int i = 0; i < ARK_DUMP_NFIELDS; ++i) r.f[i] = L.f[i];
  const size_t h0 = (size_t)popcount_below(r.mask, d.n_layers) * L.rec;
  for (int i = 0; i < 4; ++i) r.head[i] = h0 + L.head[i];
  return r;
}

bool dims_ok(const ark_dims& d) {
  if (d.n_layers < 1 || d.n_layers > kMaxLayers) return false;
  if (d.head_dim != kHeadDim) return false;
  if (d.n_heads < 1 || d.n_kv_heads < 1 || d.n_heads % d.n_kv_heads) return false;
  if (d.n_heads / d.n_kv_heads > 8) return false;
  if (d.hidden < 256 || d.hidden % 256) return false;
  if (d.intermediate < 64 || d.intermediate % 64) return false;
  if (d.max_total_len < 32 || d.max_total_len % 32 || d.max_total_len > 8192) return false;
  if (d.vocab < 1) return false;
  if (!(d.rms_eps >= 0.0) || !(d.rope_theta > 0.0)) return false;
  return true;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_qlinear(const ark_qlinear& q, int n, int k, bool bias_allowed) {
  if (!q.w || !q.scale || !q.colsum) return ARK_E_NULL;
  if (q.n != n || q.k != k) return ARK_E_SHAPE;
  if (q.bias && !bias_allowed) return ARK_E_SHAPE;
  if (!aligned(q.w, 16)) return ARK_E_ALIGN;
  return ARK_OK;
}

int check_qlinear4(const ark_qlinear4& q, int n, int k) {
  if (!q.w || !q.scale || !q.zp) return ARK_E_NULL;
  if (q.n != n || q.k != k || !lm4_supported(k)) return ARK_E_SHAPE;
  if (!aligned(q.w, 16) || !aligned(q.scale, 4)) return ARK_E_ALIGN;
  return ARK_OK;
}

bool has_head(const ark_model* m) { return m->lm_head.w || m->lm_head4.w; }

int check_model(const ark_model* m, bool need_embed) {
  if (!m) return ARK_E_NULL;
  const ark_dims& d = m->d;
  if (!dims_ok(d)) return ARK_E_SHAPE;
  if (!m->layers || !m->rope_cos || !m->rope_sin) return ARK_E_NULL;
  if (need_embed && !m->embed_f16) return ARK_E_NULL;
  const int H = d.hidden, Q = d.n_heads * d.head_dim, KV = d.n_kv_heads * d.head_dim;
  const int I = d.intermediate;
  for (int l = 0; l < d.n_layers; ++l) {
    const ark_layer& L = m->layers[l];
    if (!L.ln1 || !L.ln2) return ARK_E_NULL;
    int e;
    if ((e = check_qlinear(L.q, Q, H, true))) return e;
    if ((e = check_qlinear(L.k, KV, H, true))) return e;
    if ((e = check_qlinear(L.v, KV, H, true))) return e;
    if ((e = check_qlinear(L.o, H, Q, false))) return e;
    if ((e = check_qlinear(L.gate, I, H, false))) return e;
    if ((e = check_qlinear(L.up, I, H, false))) return e;
    if ((e = check_qlinear(L.down, H, I, false))) return e;
  }
  if (m->lm_head.w && m->lm_head4.w) return ARK_E_SHAPE;
  if (m->lm_head.w) {
    if (!m->final_norm) return ARK_E_NULL;
    int e;
    if ((e = check_qlinear(m->lm_head, d.vocab, H, false))) return e;
  }
  if (m->lm_head4.w) {
    if (!m->final_norm) return ARK_E_NULL;
    if (!norm_quant_row_supported(H)) return ARK_E_SHAPE;
    int e;
    if ((e = check_qlinear4(m->lm_head4, d.vocab, H))) return e;
  }
  return ARK_OK;
}

int check_step(const ark_model* m, int B, int S, const int32_t* pos, const float* const* kc,
               const float* const* vc, const float* kd, const float* vd, const float* logits,
               const void* ws, size_t ws_bytes) {
  if (B < 1 || B > kMaxBatch || S < 1) return ARK_E_SHAPE;
  if (!pos || !kc || !vc || !kd || !vd || !ws) return ARK_E_NULL;
  const ark_dims& d = m->d;
  for (int l = 0; l < d.n_layers; ++l)
    if (!kc[l] || !vc[l]) return ARK_E_NULL;
  if (logits && !has_head(m)) return ARK_E_SHAPE;
  for (int b = 0; b < B; ++b)
    if (pos[b] < 0 || (int64_t)pos[b] + S > d.max_total_len) return ARK_E_RANGE;
  if (!aligned(ws, kAlign) || !aligned(kd, 16) || !aligned(vd, 16)) return ARK_E_ALIGN;
  for (int l = 0; l < d.n_layers; ++l)
    if (!aligned(kc[l], 16) || !aligned(vc[l], 16)) return ARK_E_ALIGN;
  if (ws_bytes < plan(d, B, S).total) return ARK_E_WORKSPACE;
  return ARK_OK;
}

inline Seg seg_of(const ark_qlinear& q, float* out, int ldo) {
  Seg s;
  s.w = q.w;
  s.sw = q.scale;
  s.cs = q.colsum;
  s.bias = q.bias;
  s.n = q.n;
  s.out = out;
  s.ldo = ldo;
  return s;
}

// Benchmark instrumentation (see ark_profile_arm).
// Process-wide and meant for one benchmarking thread; the members are
// atomic so that decode calls on other threads, which only read them while
// nothing is armed, never race with the arming.
struct Profiler {
  std::atomic<hipEvent_t*> ev{nullptr};
  std::atomic<int> n{0};
  std::atomic<int> count{0};
};
Profiler g_prof;

// The event pair of the next recorded launch, or false when not armed or full.
inline bool prof_claim(hipEvent_t& b, hipEvent_t& e) {
  hipEvent_t* ev = g_prof.ev.load();
  if (!ev) return false;
  const int i = g_prof.count.load();
  if (i >= g_prof.n.load()) return false;
  g_prof.count.store(i + 1);
  b = ev[2 * i];
  e = ev[2 * i + 1];
  return true;
}

#define HIP_TRY(expr)                       \
  do {                                      \
    if ((expr) != hipSuccess) return ARK_E_HIP; \
  } while (0)

// The int4 tier's LM head over B rows (row b at last + b * ldx): the final
// RMSNorm into the workspace's hn rows (its uint8 quantisation, which the
// fused row kernel also writes, goes to the code scratch and is not used),
// then the weight-only int4 head.  A parity record gets the normed rows.
int head_int4(const ark_model* m, int B, const float* last, int ldx, float* logits, char* ws,
              const Plan& p, hipStream_t st, const DumpRec* dr) {
  const ark_dims& d = m->d;
  const int H = d.hidden;
  float* hn = (float*)(ws + p.hn);
  if (launch_norm_quant_row(st, B, H, last, ldx, m->final_norm, d.rms_eps, (int8_t*)(ws + p.codes),
                            (float*)(ws + p.qs), (int*)(ws + p.qz), hn) != hipSuccess)
    return ARK_E_HIP;
  if (dr && dr->base &&
      hipMemcpyAsync(dr->base + dr->head[0], hn, (size_t)B * H * 4, hipMemcpyDeviceToDevice, st) !=
          hipSuccess)
    return ARK_E_HIP;
  const ark_qlinear4& W = m->lm_head4;
  return launch_lm4(st, B, H, d.vocab, hn, H, W.w, W.scale, W.zp, logits, d.vocab) == hipSuccess
             ? ARK_OK
             : ARK_E_HIP;
}

// All layers and the LM head over the rows already in x ([B*S][H]).
#define D2D(dst, src, bytes)                                                                  \
  do {                                                                                        \
    char* dst_ = (dst);                                                                       \
    if (dst_) HIP_TRY(hipMemcpyAsync(dst_, (src), (bytes), hipMemcpyDeviceToDevice, st));     \
  } while (0)

// All layers and the LM head over the rows already in x ([B*S][H]).  dr
// (optional): the parity record to fill (copies of the workspace tensors
// after each step; the quantisers also write the values they quantised).
int run_forward(const ark_model* m, int B, int S, float* x, const int32_t* pos_host,
                const float* const* kc, const float* const* vc, float* kd, float* vd,
                float* logits, char* ws, hipStream_t st, const DumpRec* dr = nullptr) {
  const ark_dims& d = m->d;
  const Plan p = plan(d, B, S);
  // field f of layer l's record, or nullptr when layer l is not recorded
  auto dptr = [&](int l, int f) -> char* {
    if (!dr || !dr->base || !((dr->mask >> l) & 1)) return nullptr;
    return dr->base + (size_t)popcount_below(dr->mask, l) * dr->rec + dr->f[f];
  };
  // quantisation record of point pt (0: h1, 1: attention, 2: h2, 3: SwiGLU)
  QDump qd[4];
  auto qdp = [&](int l, int pt) -> const QDump* {
    char* c = dptr(l, ARK_DUMP_C1 + pt);
    if (!c) return nullptr;
    const int hf[4] = {ARK_DUMP_H1, -1, ARK_DUMP_H2, -1};
    qd[pt].h = hf[pt] >= 0 ? (float*)dptr(l, hf[pt]) : nullptr;
    qd[pt].codes = (int8_t*)c;
    qd[pt].s = (float*)dptr(l, ARK_DUMP_S) + (size_t)pt * B;
    qd[pt].z = (int*)dptr(l, ARK_DUMP_Z) + (size_t)pt * B;
    return &qd[pt];
  };
  // after a workspace quantiser: its codes [R][K] and (s, z)
  auto qcopy = [&](int l, int pt, const int8_t* codes, const float* qs, const int* qz, int K) {
    const QDump* q = qdp(l, pt);
    if (!q) return (int)ARK_OK;
    const size_t R = (size_t)B * S;
    if (hipMemcpyAsync(q->codes, codes, R * K, hipMemcpyDeviceToDevice, st) != hipSuccess ||
        hipMemcpyAsync(q->s, qs, (size_t)B * 4, hipMemcpyDeviceToDevice, st) != hipSuccess ||
        hipMemcpyAsync(q->z, qz, (size_t)B * 4, hipMemcpyDeviceToDevice, st) != hipSuccess)
      return (int)ARK_E_HIP;
    return (int)ARK_OK;
  };
#define QCOPY(l, pt, K) HIP_TRY(qcopy((l), (pt), codes, qs, qz, (K)) == ARK_OK ? hipSuccess : hipErrorUnknown)
  const int R = B * S, H = d.hidden, NH = d.n_heads, NKV = d.n_kv_heads;
  const int Q = NH * kHeadDim, KV = NKV * kHeadDim, I = d.intermediate, T = d.max_total_len;
  const bool gemv = (S == 1 && B <= 4);
  // one row per sequence: norm and quantisation fused per row
  const bool rowq = S == 1 && norm_quant_row_supported(H) && norm_quant_row_supported(Q) &&
                    norm_quant_row_supported(I);
  double* rs = (double*)(ws + p.rs);
  int8_t* codes = (int8_t*)(ws + p.codes);
  float* qkv = (float*)(ws + p.qkv);
  float* q = (float*)(ws + p.q);
  float* attn = (float*)(ws + p.attn);
  float* a = (float*)(ws + p.a);
  // per-sequence activation ranges: two sets filled in turn, each producer
  // clearing the other set for the producer after it
  int* stw = (int*)(ws + p.stats);
  const SeqStats sa = {stw, stw + kStatsSetInts, B};
  const SeqStats sb = {stw + kStatsSetInts, stw, B};
  float* qs = (float*)(ws + p.qs);
  int* qz = (int*)(ws + p.qz);
  void* part = ws + p.part;
  void* gsk = ws + p.gsk;  // GEMM scratch (few-row blocks, split-K blocks)
  HIP_TRY(gemm_scratch_reset(st, gsk, (size_t)R));
  if (!gemv && !rowq) HIP_TRY(launch_seq_stats_init(st, sa.cur));
  // one row per sequence: the o and down GEMMs store their split sums and a
  // row kernel runs the epilogue together with the RMSNorm and quantiser
  // that follow (RMSNorm 2; the next layer's RMSNorm 1 or the final norm)
  int32_t* rpart = (int32_t*)(ws + p.rowpart);
  bool h1_ready = false;  // layer l's RMSNorm 1 codes came from layer l-1's down step
  PosArgs pos;
  memset(&pos, 0, sizeof(pos));
  int pmax = 0;
  for (int b = 0; b < B; ++b) {
    pos.p[b] = pos_host[b];
    pmax = std::max(pmax, pos_host[b]);
  }
  const int ldqkv = Q + 2 * KV;

  for (int l = 0; l < d.n_layers; ++l) {
    const ark_layer& L = m->layers[l];
    float* kdl = kd + (size_t)l * R * KV;
    float* vdl = vd + (size_t)l * R * KV;
    Seg qkvs[3] = {seg_of(L.q, qkv, ldqkv), seg_of(L.k, qkv + Q, ldqkv),
                   seg_of(L.v, qkv + Q + KV, ldqkv)};
    Seg os[1] = {seg_of(L.o, x, H)};
    Seg gus[2] = {seg_of(L.gate, a, I), seg_of(L.up, a, I)};
    Seg ds[1] = {seg_of(L.down, x, H)};
    if (gemv) {
      HIP_TRY(launch_gemv(st, B, H, x, H, L.ln1, d.rms_eps, qkvs, 3, EPI_STORE, qdp(l, 0)));
    } else if (rowq) {
      if (!h1_ready)
        HIP_TRY(launch_norm_quant_row(st, B, H, x, H, L.ln1, d.rms_eps, codes, qs, qz,
                                      (float*)dptr(l, ARK_DUMP_H1)));
      QCOPY(l, 0, H);
      // q|k|v keep the split GEMM's own epilogue (faster here than the split
      // sums through the row kernel: nothing follows it to fuse)
      HIP_TRY(launch_gemm(st, R, H, codes, qs, qz, S, qkvs, 3, EPI_STORE, nullptr, gsk));
    } else {
      HIP_TRY(launch_row_stats(st, R, H, S, x, H, L.ln1, d.rms_eps, rs, sa));
      HIP_TRY(launch_quant_seq(st, R, H, S, x, H, rs, L.ln1, sa.cur, codes, nullptr, qs, qz,
                               (float*)dptr(l, ARK_DUMP_H1)));
      QCOPY(l, 0, H);
      HIP_TRY(launch_gemm(st, R, H, codes, qs, qz, S, qkvs, 3, EPI_STORE, nullptr, gsk));
    }
    D2D(dptr(l, ARK_DUMP_QKV), qkv, (size_t)R * ldqkv * 4);
    // decode: the rotary step runs inside the attention kernel
    const bool rope_in_attn = S == 1 && NH / NKV <= 8;
    if (!rope_in_attn)
      HIP_TRY(launch_rope(st, B, S, NH, NKV, qkv, m->rope_cos, m->rope_sin, pos, q, kdl, vdl));
    const RopeIn ri = {qkv, ldqkv, m->rope_cos, m->rope_sin, kdl, vdl};
    const bool att_stats = !gemv && !rowq && attention_stats(B, S, NH, NKV, T, pmax);
    HIP_TRY(launch_attention(st, B, S, NH, NKV, T, q, kc[l], vc[l], kdl, vdl, pos, attn, part,
                             att_stats ? &sb : nullptr, rope_in_attn ? &ri : nullptr));
    D2D(dptr(l, ARK_DUMP_ATTN), attn, (size_t)R * Q * 4);
    if (gemv) {
      HIP_TRY(launch_gemv(st, B, Q, attn, Q, nullptr, 0.0, os, 1, EPI_RESID, qdp(l, 1)));
      D2D(dptr(l, ARK_DUMP_X1), x, (size_t)R * H * 4);
      hipEvent_t eb = nullptr, ee = nullptr;
      const bool prof = B == 1 && prof_claim(eb, ee);
      if (prof) HIP_TRY(hipEventRecord(eb, st));
      HIP_TRY(launch_gemv(st, B, H, x, H, L.ln2, d.rms_eps, gus, 2, EPI_SWIGLU, qdp(l, 2)));
      if (prof) HIP_TRY(hipEventRecord(ee, st));
      D2D(dptr(l, ARK_DUMP_A), a, (size_t)R * I * 4);
      HIP_TRY(launch_gemv(st, B, I, a, I, nullptr, 0.0, ds, 1, EPI_RESID, qdp(l, 3)));
    } else if (rowq) {
      HIP_TRY(launch_norm_quant_row(st, B, Q, attn, Q, nullptr, 0.0, codes, qs, qz));
      QCOPY(l, 1, Q);
      if (gemm_rows_supported(R, Q, EPI_RESID, H)) {
        const RowNorm n2 = {L.ln2, d.rms_eps, codes, qs, qz, (float*)dptr(l, ARK_DUMP_H2)};
        HIP_TRY(launch_gemm_rows(st, R, Q, codes, qs, qz, os, 1, EPI_RESID, rpart, &n2));
        D2D(dptr(l, ARK_DUMP_X1), x, (size_t)R * H * 4);
      } else {
        HIP_TRY(launch_gemm(st, R, Q, codes, qs, qz, S, os, 1, EPI_RESID, nullptr, gsk));
        D2D(dptr(l, ARK_DUMP_X1), x, (size_t)R * H * 4);
        HIP_TRY(launch_norm_quant_row(st, B, H, x, H, L.ln2, d.rms_eps, codes, qs, qz,
                                      (float*)dptr(l, ARK_DUMP_H2)));
      }
      QCOPY(l, 2, H);
      HIP_TRY(launch_gemm(st, R, H, codes, qs, qz, S, gus, 2, EPI_SWIGLU, nullptr, gsk));
      D2D(dptr(l, ARK_DUMP_A), a, (size_t)R * I * 4);
      HIP_TRY(launch_norm_quant_row(st, B, I, a, I, nullptr, 0.0, codes, qs, qz));
      QCOPY(l, 3, I);
      // the down step also runs the next RMSNorm: layer l+1's, or the final
      // norm of the int8 LM head over more than 4 rows
      const bool last = l + 1 == d.n_layers;
      const bool head_rows = last && logits && !m->lm_head4.w && B > 4;
      if (gemm_rows_supported(R, I, EPI_RESID, H)) {
        float* h_dump = last ? nullptr : (float*)dptr(l + 1, ARK_DUMP_H1);
        if (last && dr && dr->base) h_dump = (float*)(dr->base + dr->head[0]);
        const RowNorm n1 = {last ? m->final_norm : m->layers[l + 1].ln1, d.rms_eps, codes, qs, qz,
                            h_dump};
        h1_ready = !last || head_rows;
        HIP_TRY(launch_gemm_rows(st, R, I, codes, qs, qz, ds, 1, EPI_RESID, rpart,
                                 h1_ready ? &n1 : nullptr));
      } else {
        h1_ready = false;
        HIP_TRY(launch_gemm(st, R, I, codes, qs, qz, S, ds, 1, EPI_RESID, nullptr, gsk));
      }
    } else {
      if (!att_stats) HIP_TRY(launch_row_stats(st, R, Q, S, attn, Q, nullptr, 0.0, nullptr, sb));
      HIP_TRY(launch_quant_seq(st, R, Q, S, attn, Q, nullptr, nullptr, sb.cur, codes, nullptr, qs,
                               qz));
      QCOPY(l, 1, Q);
      HIP_TRY(launch_gemm(st, R, Q, codes, qs, qz, S, os, 1, EPI_RESID, nullptr, gsk));
      D2D(dptr(l, ARK_DUMP_X1), x, (size_t)R * H * 4);
      HIP_TRY(launch_row_stats(st, R, H, S, x, H, L.ln2, d.rms_eps, rs, sa));
      HIP_TRY(launch_quant_seq(st, R, H, S, x, H, rs, L.ln2, sa.cur, codes, nullptr, qs, qz,
                               (float*)dptr(l, ARK_DUMP_H2)));
      QCOPY(l, 2, H);
      const bool gu_stats = gemm_swiglu_stats(R, H, gsk);
      HIP_TRY(launch_gemm(st, R, H, codes, qs, qz, S, gus, 2, EPI_SWIGLU, nullptr, gsk, false,
                          gu_stats ? &sb : nullptr));
      D2D(dptr(l, ARK_DUMP_A), a, (size_t)R * I * 4);
      if (!gu_stats) HIP_TRY(launch_row_stats(st, R, I, S, a, I, nullptr, 0.0, nullptr, sb));
      HIP_TRY(launch_quant_seq(st, R, I, S, a, I, nullptr, nullptr, sb.cur, codes, nullptr, qs, qz));
      QCOPY(l, 3, I);
      HIP_TRY(launch_gemm(st, R, I, codes, qs, qz, S, ds, 1, EPI_RESID, nullptr, gsk));
    }
    D2D(dptr(l, ARK_DUMP_X2), x, (size_t)R * H * 4);
  }

  if (logits && m->lm_head4.w)
    return head_int4(m, B, x + (size_t)(S - 1) * H, S * H, logits, ws, p, st, dr);
  if (logits) {
    Seg lm[1] = {seg_of(m->lm_head, logits, d.vocab)};
    const float* last = x + (size_t)(S - 1) * H;  // row S-1 of each sequence, stride S*H
    QDump hq = {nullptr, nullptr, nullptr, nullptr};
    if (dr && dr->base) {
      hq.h = (float*)(dr->base + dr->head[0]);
      hq.codes = (int8_t*)(dr->base + dr->head[1]);
      hq.s = (float*)(dr->base + dr->head[2]);
      hq.z = (int*)(dr->base + dr->head[3]);
    }
    if (B <= 4) {
      HIP_TRY(launch_gemv(st, B, H, last, S * H, m->final_norm, d.rms_eps, lm, 1, EPI_STORE,
                          hq.codes ? &hq : nullptr));
    } else {
      if (rowq && h1_ready) {
        // the last down step ran the final norm and its quantiser
      } else if (norm_quant_row_supported(H)) {
        HIP_TRY(launch_norm_quant_row(st, B, H, last, S * H, m->final_norm, d.rms_eps, codes, qs,
                                      qz, hq.h));
      } else {
        // set A is clear here: the last producer of the layers (if any) filled B
        HIP_TRY(launch_row_stats(st, B, H, 1, last, S * H, m->final_norm, d.rms_eps, rs, sa));
        HIP_TRY(launch_quant_seq(st, B, H, 1, last, S * H, rs, m->final_norm, sa.cur, codes,
                                 nullptr, qs, qz, hq.h));
      }
      if (hq.codes) {
        HIP_TRY(hipMemcpyAsync(hq.codes, codes, (size_t)B * H, hipMemcpyDeviceToDevice, st));
        HIP_TRY(hipMemcpyAsync(hq.s, qs, (size_t)B * 4, hipMemcpyDeviceToDevice, st));
        HIP_TRY(hipMemcpyAsync(hq.z, qz, (size_t)B * 4, hipMemcpyDeviceToDevice, st));
      }
      HIP_TRY(launch_gemm(st, B, H, codes, qs, qz, 1, lm, 1, EPI_STORE, nullptr, gsk));
    }
  }
  return ARK_OK;
}
#undef QCOPY

int mega_upload(const ark_model* m, const float* const* kc, const float* const* vc, char* ws,
                hipStream_t st) {
  const ark_dims& d = m->d;
  MegaLayer tab[kMaxLayers];
  for (int l = 0; l < d.n_layers; ++l) {
    const ark_layer& L = m->layers[l];
    const ark_qlinear* q[7] = {&L.q, &L.k, &L.v, &L.o, &L.gate, &L.up, &L.down};
    for (int i = 0; i < 7; ++i) {
      tab[l].w[i] = q[i]->w;
      tab[l].sw[i] = q[i]->scale;
      tab[l].cs[i] = q[i]->colsum;
    }
    tab[l].bias[0] = L.q.bias;
    tab[l].bias[1] = L.k.bias;
    tab[l].bias[2] = L.v.bias;
    tab[l].ln1 = L.ln1;
    tab[l].ln2 = L.ln2;
    tab[l].kc = kc[l];
    tab[l].vc = vc[l];
  }
  const Plan p = plan(d, 1, 1);
  return decode_mega_upload(st, ws + p.mega, d.n_layers, d.max_total_len, tab) == hipSuccess
             ? ARK_OK
             : ARK_E_HIP;
}

// Bound of the persistent kernel's waits: the default, or the value of
// ARK_TEST_SPIN_LIMIT (tests of the time-out report set it, e.g. to 0).
int64_t mega_spin_limit() {
  const char* e = getenv("ARK_TEST_SPIN_LIMIT");
  if (!e || !*e) return -1;
  char* end = nullptr;
  const long long v = strtoll(e, &end, 10);
  return (end && *end == 0 && v >= 0) ? (int64_t)v : -1;
}

int mega_step(const ark_model* m, const int32_t* token, int pos, float* kd, float* vd,
              float* logits, float* hidden_out, const uint8_t* mask, int32_t* out_token, char* ws,
              hipStream_t st, const DumpRec* dr = nullptr, bool prep = true) {
  const ark_dims& d = m->d;
  const Plan p = plan(d, 1, 1);
  // int4 tier: the kernel's tail runs the final norm, the int4 head and
  // the masked argmax in place of the int8 head
  const bool h4 = logits && m->lm_head4.w;
  MegaStep S;
  S.L = d.n_layers;
  S.T = d.max_total_len;
  S.V = d.vocab;
  S.pos = pos;
  S.eps = d.rms_eps;
  S.token = token;
  S.table = m->embed_f16;
  S.final_norm = logits ? m->final_norm : nullptr;
  S.lm_w = (logits && !h4) ? m->lm_head.w : nullptr;
  S.lm4_w = h4 ? m->lm_head4.w : nullptr;
  S.lm4_s = m->lm_head4.scale;
  S.lm4_z = m->lm_head4.zp;
  S.lm_sw = m->lm_head.scale;
  S.lm_cs = m->lm_head.colsum;
  S.rcos = m->rope_cos;
  S.rsin = m->rope_sin;
  S.kdelta = kd;
  S.vdelta = vd;
  S.logits = logits;
  S.hidden_out = hidden_out;
  S.mask = logits ? mask : nullptr;
  S.out_token = out_token;
  memset(&S.dump, 0, sizeof(S.dump));
  if (dr) S.dump = *dr;
  S.spin_limit = mega_spin_limit();
  hipEvent_t eb = nullptr, ee = nullptr;
  prof_claim(eb, ee);
  const hipError_t e = decode_mega_launch(st, ws + p.mega, S, eb, ee, prep);
  return e == hipSuccess ? ARK_OK : ARK_E_HIP;
}

// After a greedy step on the persistent path: cache write-back of its
// deltas, the stop rule, and (prep) the next step's preparation.
int mega_between(const ark_model* m, int32_t* token, int pos, float* kd, float* vd,
                 float* const* kc, float* const* vc, int32_t* out_row, int32_t end_id,
                 int32_t* done, char* ws, hipStream_t st, bool prep) {
  const ark_dims& d = m->d;
  const Plan p = plan(d, 1, 1);
  MegaStep S;
  memset(&S, 0, sizeof(S));
  S.L = d.n_layers;
  S.T = d.max_total_len;
  S.V = d.vocab;
  S.pos = pos;
  S.token = token;
  S.table = m->embed_f16;
  S.kdelta = kd;
  S.vdelta = vd;
  const hipError_t e = decode_mega_between(st, ws + p.mega, S, kc, vc, out_row, end_id, done, prep);
  return e == hipSuccess ? ARK_OK : ARK_E_HIP;
}

bool mega_ready(const ark_model* m, int B) {
  return use_mega(m->d, B, 1) && decode_mega_init() == hipSuccess;
}

// Synchronise the stream, then read the persistent kernel's error word.
int mega_check(const ark_model* m, const char* ws, hipStream_t st) {
  const Plan p = plan(m->d, 1, 1);
  uint32_t word = 0;
  const uint32_t* w = decode_mega_err_word(ws + p.mega, m->d.n_layers, m->d.max_total_len);
  if (hipStreamSynchronize(st) != hipSuccess ||
      hipMemcpy(&word, w, 4, hipMemcpyDeviceToHost) != hipSuccess)
    return ARK_E_HIP;
  return word ? ARK_E_TIMEOUT : ARK_OK;
}

int prefill_impl(const ark_model* m, int32_t B, int32_t S, const float* embeds,
                 const int32_t* cache_position, const float* const* k_cache,
                 const float* const* v_cache, float* k_delta, float* v_delta, float* logits,
                 float* hidden_out, void* workspace, size_t workspace_bytes, void* stream,
                 const DumpRec* dr) {
  int e = check_model(m, false);
  if (e) return e;
  if (!embeds) return ARK_E_NULL;
  e = check_step(m, B, S, cache_position, k_cache, v_cache, k_delta, v_delta, logits, workspace,
                 workspace_bytes);
  if (e) return e;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const Plan p = plan(m->d, B, S);
  float* x = hidden_out ? hidden_out : (float*)(ws + p.x);
  const size_t xb = (size_t)B * S * m->d.hidden * 4;
  if (hipMemcpyAsync(x, embeds, xb, hipMemcpyDeviceToDevice, st) != hipSuccess) return ARK_E_HIP;
  return run_forward(m, B, S, x, cache_position, k_cache, v_cache, k_delta, v_delta, logits, ws,
                     st, dr);
}

int decode_impl(const ark_model* m, int32_t B, const int32_t* token_ids,
                const int32_t* cache_position, const float* const* k_cache,
                const float* const* v_cache, float* k_delta, float* v_delta, float* logits,
                float* hidden_out, void* workspace, size_t workspace_bytes, void* stream,
                const DumpRec* dr) {
  int e = check_model(m, true);
  if (e) return e;
  if (!token_ids) return ARK_E_NULL;
  e = check_step(m, B, 1, cache_position, k_cache, v_cache, k_delta, v_delta, logits, workspace,
                 workspace_bytes);
  if (e) return e;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  if (mega_ready(m, B)) {
    if ((e = mega_upload(m, k_cache, v_cache, ws, st))) return e;
    return mega_step(m, token_ids, cache_position[0], k_delta, v_delta, logits, hidden_out, nullptr,
                     nullptr, ws, st, dr);
  }
  const Plan p = plan(m->d, B, 1);
  float* x = hidden_out ? hidden_out : (float*)(ws + p.x);
  if (launch_embed(st, B, 1, m->d.hidden, m->d.vocab, token_ids, m->embed_f16, nullptr, 0, 0, x) !=
      hipSuccess)
    return ARK_E_HIP;
  return run_forward(m, B, 1, x, cache_position, k_cache, v_cache, k_delta, v_delta, logits, ws,
                     st, dr);
}

// ---- audio adapter
struct AdapterPlan {
  size_t merged, codes, y, rs, stats, qs, qz, gsk, total;
};

// Workspace layout of ark_audio_adapter; `compact`: the merged rows are
// copied together first (frames not a multiple of merge, several sequences).
AdapterPlan adapter_plan(const ark_adapter& A, int B, int frames, bool* compact = nullptr) {
  const size_t n = (size_t)(frames / A.merge), R = (size_t)B * n;
  const size_t K1 = (size_t)A.merge * A.frame_dim, I = (size_t)A.up.n;
  const bool c = B > 1 && frames % A.merge != 0;
  if (compact) *compact = c;
  AdapterPlan p;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes);
    return at;
  };
  p.merged = take(c ? R * K1 * 4 : 0);
  p.codes = take(R * std::max(K1, I));
  p.y = take(R * I * 4);
  p.rs = take(R * 8);
  p.stats = take(2 * (size_t)kStatsSetInts * 4);
  p.qs = take((size_t)kMaxBatch * 4);
  p.qz = take((size_t)kMaxBatch * 4);
  p.gsk = take(gemm_ws_bytes(R));
  p.total = o;
  return p;
}

int check_adapter(const ark_adapter* A, int B, int frames) {
  if (!A) return ARK_E_NULL;
  if (B < 1 || B > kMaxBatch || A->merge < 1 || A->frame_dim < 1) return ARK_E_SHAPE;
  if (frames < A->merge) return ARK_E_SHAPE;
  if ((int64_t)B * (frames / A->merge) > 65535) return ARK_E_SHAPE;
  const int K1 = A->merge * A->frame_dim;
  int e;
  if ((e = check_qlinear(A->up, A->up.n, K1, true))) return e;
  if ((e = check_qlinear(A->down, A->down.n, A->up.n, true))) return e;
  if (!A->up.bias || !A->down.bias) return ARK_E_NULL;
  // both GEMMs take K in whole 64-byte steps
  if (A->up.n < 1 || A->down.n < 1 || K1 % 64 || A->up.n % 64) return ARK_E_SHAPE;
  return ARK_OK;
}

// ---- audio encoder
struct EncoderPlan {
  size_t cols, a1, x, h, qkv, attn, f, codes, rs, stats, qs, qz, gsk, part, total;
};

EncoderPlan encoder_plan(const ark_encoder& E, int B, int M) {
  const size_t F = (size_t)(M - 1) / 2 + 1, R1 = (size_t)B * M, R = (size_t)B * F;
  const size_t D = E.d_model, C = E.n_mels, FF = E.ffn;
  EncoderPlan p;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes);
    return at;
  };
  p.cols = take(std::max(R1 * 3 * C, R * 3 * D) * 4);
  p.a1 = take(R1 * D * 4);
  p.x = take(R * D * 4);
  p.h = take(R * D * 4);
  p.qkv = take(R * 3 * D * 4);
  p.attn = take(R * D * 4);
  p.f = take(R * FF * 4);
  p.codes = take(std::max(std::max(R1 * 3 * C, R * 3 * D), R * std::max(FF, D)));
  p.rs = take(std::max(R1, R) * 8);
  p.stats = take(2 * (size_t)kStatsSetInts * 4);
  p.qs = take((size_t)kMaxBatch * 4);
  p.qz = take((size_t)kMaxBatch * 4);
  p.gsk = take(gemm_ws_bytes(std::max(R1, R)));
  p.part = take(enc_attention_ws_bytes(B, (int)F, E.n_heads));  // split attention states
  p.total = o;
  return p;
}

int check_encoder(const ark_encoder* E, int B, int M) {
  if (!E) return ARK_E_NULL;
  const int D = E->d_model, C = E->n_mels, FF = E->ffn;
  if (B < 1 || B > kMaxBatch || M < 1 || (int64_t)B * M > (1 << 24)) return ARK_E_SHAPE;
  // every GEMM here takes K in whole 64-byte steps: 3 n_mels, 3 d, d, ffn
  if (E->n_heads < 1 || D != 64 * E->n_heads || C < 64 || C % 64 || FF < 64 || FF % 64 ||
      E->n_layers < 1 || E->max_pos < 1 || !(E->ln_eps >= 0.0))
    return ARK_E_SHAPE;
  if ((M - 1) / 2 + 1 > E->max_pos) return ARK_E_SHAPE;
  if (!E->pos || !E->layers || !E->lnf_g || !E->lnf_b || !E->rope_cos || !E->rope_sin)
    return ARK_E_NULL;
  int e;
  if ((e = check_qlinear(E->conv1, D, 3 * C, true))) return e;
  if ((e = check_qlinear(E->conv2, D, 3 * D, true))) return e;
  if (!E->conv1.bias || !E->conv2.bias) return ARK_E_NULL;
  for (int l = 0; l < E->n_layers; ++l) {
    const ark_enc_layer& L = E->layers[l];
    if (!L.ln1_g || !L.ln1_b || !L.ln2_g || !L.ln2_b) return ARK_E_NULL;
    if ((e = check_qlinear(L.q, D, D, true))) return e;
    if ((e = check_qlinear(L.k, D, D, false))) return e;
    if ((e = check_qlinear(L.v, D, D, true))) return e;
    if ((e = check_qlinear(L.o, D, D, true))) return e;
    if ((e = check_qlinear(L.fc1, FF, D, true))) return e;
    if ((e = check_qlinear(L.fc2, D, FF, true))) return e;
    if (!L.q.bias || !L.v.bias || !L.o.bias || !L.fc1.bias || !L.fc2.bias) return ARK_E_NULL;
  }
  return ARK_OK;
}

// ---- bf16 serving variant
struct PlanBf16 {
  size_t x, h, qkv, q, attn, a, part, total;
};

PlanBf16 plan_bf16(const ark_dims& d, int B, int S) {
  const size_t R = (size_t)B * S, H = d.hidden, Q = (size_t)d.n_heads * d.head_dim;
  const size_t KV = (size_t)d.n_kv_heads * d.head_dim, I = d.intermediate;
  PlanBf16 p;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes);
    return at;
  };
  p.x = take(R * H * 2);
  p.h = take(R * H * 2);
  p.qkv = take(R * (Q + 2 * KV) * 2);
  p.q = take(R * Q * 2);
  p.attn = take(R * Q * 2);
  p.a = take(R * I * 2);
  p.part = take(attention_ws_bytes(B, S, d.n_heads, d.max_total_len));  // split partials
  p.total = o;
  return p;
}

int check_linear_bf16(const ark_linear_bf16& q, int n, int k, bool bias_allowed) {
  if (!q.w) return ARK_E_NULL;
  if (q.n != n || q.k != k || !gemm_bf16_supported(k)) return ARK_E_SHAPE;
  if (q.bias && !bias_allowed) return ARK_E_SHAPE;
  if (!aligned(q.w, 16)) return ARK_E_ALIGN;
  return ARK_OK;
}

int check_model_bf16(const ark_model_bf16* m, bool need_embed) {
  if (!m) return ARK_E_NULL;
  const ark_dims& d = m->d;
  if (!dims_ok(d) || !attn_bf16_supported(d.n_heads, d.n_kv_heads)) return ARK_E_SHAPE;
  if (!m->layers || !m->rope_cos || !m->rope_sin) return ARK_E_NULL;
  if (need_embed && !m->embed) return ARK_E_NULL;
  const int H = d.hidden, Q = d.n_heads * d.head_dim, KV = d.n_kv_heads * d.head_dim;
  const int I = d.intermediate;
  for (int l = 0; l < d.n_layers; ++l) {
    const ark_layer_bf16& L = m->layers[l];
    if (!L.ln1 || !L.ln2) return ARK_E_NULL;
    int e;
    if ((e = check_linear_bf16(L.q, Q, H, true))) return e;
    if ((e = check_linear_bf16(L.k, KV, H, true))) return e;
    if ((e = check_linear_bf16(L.v, KV, H, true))) return e;
    if ((e = check_linear_bf16(L.o, H, Q, false))) return e;
    if ((e = check_linear_bf16(L.gate, I, H, false))) return e;
    if ((e = check_linear_bf16(L.up, I, H, false))) return e;
    if ((e = check_linear_bf16(L.down, H, I, false))) return e;
  }
  if (m->lm_head.w) {
    if (!m->final_norm) return ARK_E_NULL;
    int e;
    if ((e = check_linear_bf16(m->lm_head, d.vocab, H, false))) return e;
  }
  return ARK_OK;
}

int check_step_bf16(const ark_model_bf16* m, int B, int S, const int32_t* pos,
                    const uint16_t* const* kc, const uint16_t* const* vc, const uint16_t* kd,
                    const uint16_t* vd, const float* logits, const void* ws, size_t ws_bytes) {
  if (B < 1 || B > kMaxBatch || S < 1) return ARK_E_SHAPE;
  if (!pos || !kc || !vc || !kd || !vd || !ws) return ARK_E_NULL;
  const ark_dims& d = m->d;
  for (int l = 0; l < d.n_layers; ++l)
    if (!kc[l] || !vc[l]) return ARK_E_NULL;
  if (logits && !m->lm_head.w) return ARK_E_SHAPE;
  for (int b = 0; b < B; ++b)
    if (pos[b] < 0 || (int64_t)pos[b] + S > d.max_total_len) return ARK_E_RANGE;
  if (!aligned(ws, kAlign) || !aligned(kd, 16) || !aligned(vd, 16)) return ARK_E_ALIGN;
  for (int l = 0; l < d.n_layers; ++l)
    if (!aligned(kc[l], 16) || !aligned(vc[l], 16)) return ARK_E_ALIGN;
  if (ws_bytes < plan_bf16(d, B, S).total) return ARK_E_WORKSPACE;
  return ARK_OK;
}

inline BSeg bseg(const ark_linear_bf16& q, void* out, int ldo) {
  BSeg s;
  s.w = q.w;
  s.bias = q.bias;
  s.out = out;
  s.n = q.n;
  s.ldo = ldo;
  return s;
}

// All layers and the LM head of the bf16 variant over the rows in x.
int run_forward_bf16(const ark_model_bf16* m, int B, int S, uint16_t* x, const int32_t* pos_host,
                     const uint16_t* const* kc, const uint16_t* const* vc, uint16_t* kd,
                     uint16_t* vd, float* logits, char* ws, hipStream_t st) {
  const ark_dims& d = m->d;
  const PlanBf16 p = plan_bf16(d, B, S);
  const int R = B * S, H = d.hidden, NH = d.n_heads, NKV = d.n_kv_heads;
  const int Q = NH * kHeadDim, KV = NKV * kHeadDim, I = d.intermediate, W = Q + 2 * KV;
  uint16_t* h = (uint16_t*)(ws + p.h);
  uint16_t* qkv = (uint16_t*)(ws + p.qkv);
  uint16_t* q = (uint16_t*)(ws + p.q);
  uint16_t* attn = (uint16_t*)(ws + p.attn);
  uint16_t* a = (uint16_t*)(ws + p.a);
  PosArgs pos;
  memset(&pos, 0, sizeof(pos));
  for (int b = 0; b < B; ++b) pos.p[b] = pos_host[b];
  for (int l = 0; l < d.n_layers; ++l) {
    const ark_layer_bf16& L = m->layers[l];
    uint16_t* kdl = kd + (size_t)l * R * KV;
    uint16_t* vdl = vd + (size_t)l * R * KV;
    HIP_TRY(launch_rmsnorm_bf16(st, R, H, x, H, L.ln1, d.rms_eps, h));
    BSeg qs3[3] = {bseg(L.q, qkv, W), bseg(L.k, qkv + Q, W), bseg(L.v, qkv + Q + KV, W)};
    HIP_TRY(launch_gemm_bf16(st, R, H, h, H, qs3, 3, BE_STORE));
    HIP_TRY(launch_rope_bf16(st, B, S, NH, NKV, qkv, m->rope_cos, m->rope_sin, pos, q, kdl, vdl));
    AttnBf16Params A;
    A.B = B;
    A.S = S;
    A.NH = NH;
    A.NKV = NKV;
    A.T = d.max_total_len;
    A.q = q;
    A.kc = kc[l];
    A.vc = vc[l];
    A.kd = kdl;
    A.vd = vdl;
    A.pos = pos;
    A.out = attn;
    HIP_TRY(launch_attn_bf16(st, A, ws + p.part));
    BSeg os[1] = {bseg(L.o, x, H)};
    HIP_TRY(launch_gemm_bf16(st, R, Q, attn, Q, os, 1, BE_RESID));
    HIP_TRY(launch_rmsnorm_bf16(st, R, H, x, H, L.ln2, d.rms_eps, h));
    BSeg gu[2] = {bseg(L.gate, a, I), bseg(L.up, a, I)};
    HIP_TRY(launch_gemm_bf16(st, R, H, h, H, gu, 2, BE_SWIGLU));
    BSeg ds[1] = {bseg(L.down, x, H)};
    HIP_TRY(launch_gemm_bf16(st, R, I, a, I, ds, 1, BE_RESID));
  }
  if (logits) {
    HIP_TRY(launch_rmsnorm_bf16(st, B, H, x + (size_t)(S - 1) * H, S * H, m->final_norm,
                                d.rms_eps, h));
    BSeg lm[1] = {bseg(m->lm_head, logits, d.vocab)};
    HIP_TRY(launch_gemm_bf16(st, B, H, h, H, lm, 1, BE_F32));
  }
  return ARK_OK;
}

// Validate a parity record request and build its descriptor.
int dump_check(const ark_model* m, int B, int S, void* dump, size_t dump_bytes, uint64_t mask,
               DumpRec* out) {
  if (!m) return ARK_E_NULL;
  if (!dump) return ARK_E_NULL;
  if (!dims_ok(m->d) || B < 1 || B > kMaxBatch || S < 1) return ARK_E_SHAPE;
  if (!aligned(dump, kAlign)) return ARK_E_ALIGN;
  if (dump_bytes < dump_total(m->d, B, S, mask)) return ARK_E_WORKSPACE;
  *out = dump_rec(m->d, B, S, mask, dump);
  return ARK_OK;
}

// Device address of `scratch` on each device (resolved on the entry
// point's first call there, with that device current) and the kind of the
// last call made with it: a persistent-kernel step of one layout, or not.
constexpr int kMaxDevices = 64;
struct DeviceScratch {
  char* ptr = nullptr;
  uint64_t last = 0;
};
DeviceScratch g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_of_device(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ARK_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev].ptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ARK_E_HIP;
    g_scratch[dev].ptr = (char*)p;
  }
  *out = g_scratch[dev].ptr;
  return ARK_OK;
}

// Record the kind of this call on the current device; true when the
// persistent kernel's exchange area must be re-initialised (the array last
// served another layout or the multi-kernel path, whose buffers overlap it).
bool scratch_switch(uint64_t key) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return true;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  const bool changed = key != 0 && g_scratch[dev].last != key;
  g_scratch[dev].last = key;
  return changed;
}

}  // namespace

extern "C" {

size_t ark_noalloc_max_bytes(void) { return kNoAllocBytes; }

int ark_decode_step_noalloc(const ark_model* m, int32_t B, const int32_t* token_ids,
                            const int32_t* cache_position, const float* const* k_cache,
                            const float* const* v_cache, float* k_delta, float* v_delta,
                            float* logits, float* hidden_out, void* stream) {
  if (!m) return ARK_E_NULL;
  if (!dims_ok(m->d) || B < 1 || B > kMaxBatch) return ARK_E_SHAPE;
  const size_t need = plan(m->d, B, 1).total;
  if (need > kNoAllocBytes) return ARK_E_NOALLOC;
  int e = check_model(m, true);
  if (e) return e;
  if (!token_ids) return ARK_E_NULL;
  char* ws = nullptr;
  if ((e = scratch_of_device(&ws))) return e;
  e = check_step(m, B, 1, cache_position, k_cache, v_cache, k_delta, v_delta, logits, ws, need);
  if (e) return e;
  hipStream_t st = (hipStream_t)stream;
  const bool mega = mega_ready(m, B);
  const uint64_t key =
      mega ? ((1ull << 63) | ((uint64_t)m->d.n_layers << 32) | (uint32_t)m->d.max_total_len) : 0;
  if (scratch_switch(key)) {
    const Plan p = plan(m->d, 1, 1);
    uint64_t* marker = decode_mega_marker(ws + p.mega, m->d.n_layers, m->d.max_total_len);
    if (launch_zero_u32(st, (uint32_t*)marker, 2) != hipSuccess) return ARK_E_HIP;
  }
  return decode_impl(m, B, token_ids, cache_position, k_cache, v_cache, k_delta, v_delta, logits,
                     hidden_out, ws, need, stream, nullptr);
}

const char* ark_status_string(int status) {
  switch (status) {
    case ARK_OK: return "ok";
    case ARK_E_NULL: return "a required pointer is NULL";
    case ARK_E_SHAPE: return "a size is invalid, inconsistent or unsupported";
    case ARK_E_RANGE: return "cache_position out of range for the static cache";
    case ARK_E_WORKSPACE: return "workspace too small";
    case ARK_E_HIP: return "HIP launch failed";
    case ARK_E_ALIGN: return "pointer misaligned";
    case ARK_E_NOALLOC:
      return "the call needs more scratch than the library's static array holds "
             "(ark_noalloc_max_bytes)";
    case ARK_E_TIMEOUT:
      return "a bounded wait of the persistent decode kernel timed out; that step's outputs are invalid";
    default: return "unknown status";
  }
}

size_t ark_workspace_bytes(const ark_dims* d, int32_t B, int32_t S) {
  if (!d || !dims_ok(*d) || B < 1 || B > kMaxBatch || S < 1) return 0;
  return plan(*d, B, S).total;
}

int ark_prep_weight(const float* w, int32_t n, int32_t k, int8_t* codes, float* scale,
                    int32_t* colsum, void* stream) {
  if (!w || !codes || !scale || !colsum) return ARK_E_NULL;
  if (n < 1 || k < 16 || k % 16) return ARK_E_SHAPE;
  return launch_prep_weight((hipStream_t)stream, w, n, k, codes, scale, colsum) == hipSuccess
             ? ARK_OK
             : ARK_E_HIP;
}

int ark_prep_weight_int4(const float* w, int32_t n, int32_t k, uint8_t* codes, float* scale,
                         uint8_t* zp, void* stream) {
  if (!w || !codes || !scale || !zp) return ARK_E_NULL;
  if (n < 1 || k < 256 || k % 256) return ARK_E_SHAPE;
  if (!aligned(w, 16) || !aligned(codes, 16) || !aligned(scale, 16) || !aligned(zp, 16))
    return ARK_E_ALIGN;
  return launch_prep_w4((hipStream_t)stream, w, n, k, codes, scale, zp) == hipSuccess ? ARK_OK
                                                                                      : ARK_E_HIP;
}

int ark_lm_head_int4(int32_t B, const float* h, int32_t ldh, const ark_qlinear4* W,
                     float* logits, int32_t ldl, void* stream) {
  if (!h || !W || !logits) return ARK_E_NULL;
  if (B < 1 || B > kMaxBatch || W->n < 1) return ARK_E_SHAPE;
  int e = check_qlinear4(*W, W->n, W->k);
  if (e) return e;
  if (ldh < W->k || ldl < W->n) return ARK_E_SHAPE;
  if (!aligned(h, 16)) return ARK_E_ALIGN;
  return launch_lm4((hipStream_t)stream, B, W->k, W->n, h, ldh, W->w, W->scale, W->zp, logits,
                    ldl) == hipSuccess
             ? ARK_OK
             : ARK_E_HIP;
}

size_t ark_adapter_workspace_bytes(const ark_adapter* A, int32_t B, int32_t frames) {
  if (check_adapter(A, B, frames) != ARK_OK) return 0;
  return adapter_plan(*A, B, frames).total;
}

int ark_audio_adapter(const ark_adapter* A, int32_t B, int32_t frames, const float* enc,
                      float* out, float* mid, void* workspace, size_t workspace_bytes,
                      void* stream) {
  int e = check_adapter(A, B, frames);
  if (e) return e;
  if (!enc || !out || !workspace) return ARK_E_NULL;
  if (!aligned(enc, 16) || !aligned(out, 16) || (mid && !aligned(mid, 16)) ||
      !aligned(workspace, kAlign))
    return ARK_E_ALIGN;
  bool compact = false;
  const AdapterPlan p = adapter_plan(*A, B, frames, &compact);
  if (workspace_bytes < p.total) return ARK_E_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const int n = frames / A->merge, R = B * n, K1 = A->merge * A->frame_dim, I = A->up.n;
  const int H = A->down.n;
  // merged rows: row i of sequence b is frames merge*i .. merge*i + merge - 1
  // of that sequence side by side, i.e. enc + (b * frames + merge * i) *
  // frame_dim read K1 wide; with frames % merge == 0 (or one sequence) every
  // row is K1 floats after the one before
  const float* x = enc;
  if (compact) {
    float* m = (float*)(ws + p.merged);
    if (hipMemcpy2DAsync(m, (size_t)n * K1 * 4, enc, (size_t)frames * A->frame_dim * 4,
                         (size_t)n * K1 * 4, B, hipMemcpyDeviceToDevice, st) != hipSuccess)
      return ARK_E_HIP;
    x = m;
  }
  int8_t* codes = (int8_t*)(ws + p.codes);
  float* y = mid ? mid : (float*)(ws + p.y);
  double* rs = (double*)(ws + p.rs);
  int* stw = (int*)(ws + p.stats);
  const SeqStats sa = {stw, stw + kStatsSetInts, B};
  const SeqStats sb = {stw + kStatsSetInts, stw, B};
  float* qs = (float*)(ws + p.qs);
  int* qz = (int*)(ws + p.qz);
  void* gsk = ws + p.gsk;
  HIP_TRY(gemm_scratch_reset(st, gsk, (size_t)R));
  HIP_TRY(launch_seq_stats_init(st, sa.cur));
  // merged rows: range per sequence, codes, up projection (+ bias)
  HIP_TRY(launch_row_stats(st, R, K1, n, x, K1, nullptr, 0.0, rs, sa));
  HIP_TRY(launch_quant_seq(st, R, K1, n, x, K1, nullptr, nullptr, sa.cur, codes, nullptr, qs, qz));
  Seg up[1] = {seg_of(A->up, y, I)};
  HIP_TRY(launch_gemm(st, R, K1, codes, qs, qz, n, up, 1, EPI_STORE, nullptr, gsk));
  // GELU in place with its range, codes, down projection (+ bias)
  HIP_TRY(launch_gelu_stats(st, R, I, n, y, I, sb));
  HIP_TRY(launch_quant_seq(st, R, I, n, y, I, nullptr, nullptr, sb.cur, codes, nullptr, qs, qz));
  Seg dn[1] = {seg_of(A->down, out, H)};
  HIP_TRY(launch_gemm(st, R, I, codes, qs, qz, n, dn, 1, EPI_STORE, nullptr, gsk));
  return ARK_OK;
}

size_t ark_encoder_workspace_bytes(const ark_encoder* E, int32_t B, int32_t mel_frames) {
  if (check_encoder(E, B, mel_frames) != ARK_OK) return 0;
  return encoder_plan(*E, B, mel_frames).total;
}

int ark_audio_encoder(const ark_encoder* E, int32_t B, int32_t mel_frames, const float* mel,
                      float* out, void* workspace, size_t workspace_bytes, void* stream) {
  int e = check_encoder(E, B, mel_frames);
  if (e) return e;
  if (!mel || !out || !workspace) return ARK_E_NULL;
  if (!aligned(mel, 16) || !aligned(out, 16) || !aligned(workspace, kAlign)) return ARK_E_ALIGN;
  const EncoderPlan p = encoder_plan(*E, B, mel_frames);
  if (workspace_bytes < p.total) return ARK_E_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const int M = mel_frames, F = (M - 1) / 2 + 1, R1 = B * M, R = B * F;
  const int D = E->d_model, C = E->n_mels, FF = E->ffn, H = E->n_heads;
  float* cols = (float*)(ws + p.cols);
  float* a1 = (float*)(ws + p.a1);
  float* x = (float*)(ws + p.x);
  float* h = (float*)(ws + p.h);
  float* qkv = (float*)(ws + p.qkv);
  float* attn = (float*)(ws + p.attn);
  float* f = (float*)(ws + p.f);
  int8_t* codes = (int8_t*)(ws + p.codes);
  double* rs = (double*)(ws + p.rs);
  int* stw = (int*)(ws + p.stats);
  const SeqStats sa = {stw, stw + kStatsSetInts, B};
  const SeqStats sb = {stw + kStatsSetInts, stw, B};
  const SeqStats none = {nullptr, nullptr, B};
  float* qs = (float*)(ws + p.qs);
  int* qz = (int*)(ws + p.qz);
  void* gsk = ws + p.gsk;
  HIP_TRY(gemm_scratch_reset(st, gsk, (size_t)std::max(R1, R)));
  HIP_TRY(launch_seq_stats_init(st, sa.cur));
  // conv1: tap-major rows of the mel frames, their range and codes per clip,
  // the int8 GEMM (+ bias), GELU with its range (for conv2's codes)
  HIP_TRY(launch_im2col(st, B, M, C, 1, mel, cols));
  HIP_TRY(launch_row_stats(st, R1, 3 * C, M, cols, 3 * C, nullptr, 0.0, rs, sa));
  HIP_TRY(launch_quant_seq(st, R1, 3 * C, M, cols, 3 * C, nullptr, nullptr, sa.cur, codes, nullptr,
                           qs, qz));
  Seg c1[1] = {seg_of(E->conv1, a1, D)};
  HIP_TRY(launch_gemm(st, R1, 3 * C, codes, qs, qz, M, c1, 1, EPI_STORE, nullptr, gsk));
  HIP_TRY(launch_gelu_stats(st, R1, D, M, a1, D, sb));
  // conv2 (stride 2): its rows hold the GELU values (and zero padding), so
  // the GELU's range is theirs; GELU, then the positional rows
  HIP_TRY(launch_im2col(st, B, M, D, 2, a1, cols));
  HIP_TRY(launch_quant_seq(st, R, 3 * D, F, cols, 3 * D, nullptr, nullptr, sb.cur, codes, nullptr,
                           qs, qz));
  Seg c2[1] = {seg_of(E->conv2, x, D)};
  HIP_TRY(launch_gemm(st, R, 3 * D, codes, qs, qz, F, c2, 1, EPI_STORE, nullptr, gsk));
  HIP_TRY(launch_gelu_stats(st, R, D, F, x, D, none, E->pos, D));
  // the layers; ranges alternate between the two sets (each producer clears
  // the other for the producer after it)
  for (int l = 0; l < E->n_layers; ++l) {
    const ark_enc_layer& L = E->layers[l];
    HIP_TRY(launch_layernorm(st, R, D, F, x, L.ln1_g, L.ln1_b, E->ln_eps, h, sa));
    HIP_TRY(launch_quant_seq(st, R, D, F, h, D, nullptr, nullptr, sa.cur, codes, nullptr, qs, qz));
    Seg qkvs[3] = {seg_of(L.q, qkv, 3 * D), seg_of(L.k, qkv + D, 3 * D),
                   seg_of(L.v, qkv + 2 * D, 3 * D)};
    HIP_TRY(launch_gemm(st, R, D, codes, qs, qz, F, qkvs, 3, EPI_STORE, nullptr, gsk));
    HIP_TRY(launch_enc_attention(st, B, F, H, qkv, E->rope_cos, E->rope_sin, attn, sb, ws + p.part));
    HIP_TRY(launch_quant_seq(st, R, D, F, attn, D, nullptr, nullptr, sb.cur, codes, nullptr, qs,
                             qz));
    Seg os[1] = {seg_of(L.o, x, D)};
    HIP_TRY(launch_gemm(st, R, D, codes, qs, qz, F, os, 1, EPI_RESID, nullptr, gsk));
    HIP_TRY(launch_layernorm(st, R, D, F, x, L.ln2_g, L.ln2_b, E->ln_eps, h, sa));
    HIP_TRY(launch_quant_seq(st, R, D, F, h, D, nullptr, nullptr, sa.cur, codes, nullptr, qs, qz));
    Seg f1[1] = {seg_of(L.fc1, f, FF)};
    HIP_TRY(launch_gemm(st, R, D, codes, qs, qz, F, f1, 1, EPI_STORE, nullptr, gsk));
    HIP_TRY(launch_gelu_stats(st, R, FF, F, f, FF, sb));
    HIP_TRY(launch_quant_seq(st, R, FF, F, f, FF, nullptr, nullptr, sb.cur, codes, nullptr, qs, qz));
    Seg f2[1] = {seg_of(L.fc2, x, D)};
    HIP_TRY(launch_gemm(st, R, FF, codes, qs, qz, F, f2, 1, EPI_RESID, nullptr, gsk));
  }
  HIP_TRY(launch_layernorm(st, R, D, F, x, E->lnf_g, E->lnf_b, E->ln_eps, out, none));
  return ARK_OK;
}

int ark_to_bf16(const float* x, int64_t n, uint16_t* out, void* stream) {
  if (!x || !out) return ARK_E_NULL;
  if (n < 0) return ARK_E_SHAPE;
  return launch_to_bf16((hipStream_t)stream, n, x, out) == hipSuccess ? ARK_OK : ARK_E_HIP;
}

size_t ark_workspace_bytes_bf16(const ark_dims* d, int32_t B, int32_t S) {
  if (!d || !dims_ok(*d) || B < 1 || B > kMaxBatch || S < 1) return 0;
  return plan_bf16(*d, B, S).total;
}

int ark_prefill_bf16(const ark_model_bf16* m, int32_t B, int32_t S, const uint16_t* embeds,
                     const int32_t* cache_position, const uint16_t* const* k_cache,
                     const uint16_t* const* v_cache, uint16_t* k_delta, uint16_t* v_delta,
                     float* logits, uint16_t* hidden_out, void* workspace,
                     size_t workspace_bytes, void* stream) {
  int e = check_model_bf16(m, false);
  if (e) return e;
  if (!embeds) return ARK_E_NULL;
  e = check_step_bf16(m, B, S, cache_position, k_cache, v_cache, k_delta, v_delta, logits,
                      workspace, workspace_bytes);
  if (e) return e;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const PlanBf16 p = plan_bf16(m->d, B, S);
  uint16_t* x = hidden_out ? hidden_out : (uint16_t*)(ws + p.x);
  if (hipMemcpyAsync(x, embeds, (size_t)B * S * m->d.hidden * 2, hipMemcpyDeviceToDevice, st) !=
      hipSuccess)
    return ARK_E_HIP;
  return run_forward_bf16(m, B, S, x, cache_position, k_cache, v_cache, k_delta, v_delta, logits,
                          ws, st);
}

int ark_decode_step_bf16(const ark_model_bf16* m, int32_t B, const int32_t* token_ids,
                         const int32_t* cache_position, const uint16_t* const* k_cache,
                         const uint16_t* const* v_cache, uint16_t* k_delta, uint16_t* v_delta,
                         float* logits, uint16_t* hidden_out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  int e = check_model_bf16(m, true);
  if (e) return e;
  if (!token_ids) return ARK_E_NULL;
  e = check_step_bf16(m, B, 1, cache_position, k_cache, v_cache, k_delta, v_delta, logits,
                      workspace, workspace_bytes);
  if (e) return e;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const PlanBf16 p = plan_bf16(m->d, B, 1);
  uint16_t* x = hidden_out ? hidden_out : (uint16_t*)(ws + p.x);
  if (launch_embed_bf16(st, B, m->d.hidden, m->d.vocab, token_ids, m->embed, x) != hipSuccess)
    return ARK_E_HIP;
  return run_forward_bf16(m, B, 1, x, cache_position, k_cache, v_cache, k_delta, v_delta, logits,
                          ws, st);
}

int ark_cache_write_bf16(const ark_dims* d, int32_t B, int32_t S, const int32_t* cache_position,
                         uint16_t* const* k_cache, uint16_t* const* v_cache,
                         const uint16_t* k_delta, const uint16_t* v_delta, void* stream) {
  if (!d || !cache_position || !k_cache || !v_cache || !k_delta || !v_delta) return ARK_E_NULL;
  if (!dims_ok(*d) || B < 1 || B > kMaxBatch || S < 1) return ARK_E_SHAPE;
  CacheBf16Args A;
  for (int l = 0; l < d->n_layers; ++l) {
    if (!k_cache[l] || !v_cache[l]) return ARK_E_NULL;
    if (!aligned(k_cache[l], 16) || !aligned(v_cache[l], 16)) return ARK_E_ALIGN;
    A.k[l] = k_cache[l];
    A.v[l] = v_cache[l];
  }
  if (!aligned(k_delta, 16) || !aligned(v_delta, 16)) return ARK_E_ALIGN;
  PosArgs pos;
  memset(&pos, 0, sizeof(pos));
  for (int b = 0; b < B; ++b) {
    if (cache_position[b] < 0 || (int64_t)cache_position[b] + S > d->max_total_len)
      return ARK_E_RANGE;
    pos.p[b] = cache_position[b];
  }
  return launch_cache_write_bf16((hipStream_t)stream, d->n_layers, B, S, d->max_total_len,
                                 d->n_kv_heads * d->head_dim, pos, A, k_delta, v_delta) == hipSuccess
             ? ARK_OK
             : ARK_E_HIP;
}

int ark_rope_table(int32_t T, int32_t head_dim, double theta, double* cos_out, double* sin_out,
                   void* stream) {
  if (!cos_out || !sin_out) return ARK_E_NULL;
  if (T < 1 || head_dim < 2 || head_dim % 2 || !(theta > 0.0)) return ARK_E_SHAPE;
  return launch_rope_table((hipStream_t)stream, T, head_dim, theta, cos_out, sin_out) == hipSuccess
             ? ARK_OK
             : ARK_E_HIP;
}

int ark_embed_splice(const ark_dims* d, int32_t B, int32_t S, const int32_t* ids,
                     const uint16_t* embed_f16, const float* audio, int32_t a0, int32_t N,
                     float* out, void* stream) {
  if (!d || !ids || !embed_f16 || !out) return ARK_E_NULL;
  if (B < 1 || S < 1 || d->hidden < 1 || d->vocab < 1) return ARK_E_SHAPE;
  if (N < 0 || a0 < 0 || (int64_t)a0 + N > S) return ARK_E_SHAPE;
  if ((N > 0) != (audio != nullptr)) return N > 0 ? ARK_E_NULL : ARK_E_SHAPE;
  return launch_embed((hipStream_t)stream, B, S, d->hidden, d->vocab, ids, embed_f16, audio, a0,
                      N, out) == hipSuccess
             ? ARK_OK
             : ARK_E_HIP;
}

int ark_prefill(const ark_model* m, int32_t B, int32_t S, const float* embeds,
                const int32_t* cache_position, const float* const* k_cache,
                const float* const* v_cache, float* k_delta, float* v_delta, float* logits,
                float* hidden_out, void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_impl(m, B, S, embeds, cache_position, k_cache, v_cache, k_delta, v_delta, logits,
                      hidden_out, workspace, workspace_bytes, stream, nullptr);
}

int ark_decode_step(const ark_model* m, int32_t B, const int32_t* token_ids,
                    const int32_t* cache_position, const float* const* k_cache,
                    const float* const* v_cache, float* k_delta, float* v_delta, float* logits,
                    float* hidden_out, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(m, B, token_ids, cache_position, k_cache, v_cache, k_delta, v_delta, logits,
                     hidden_out, workspace, workspace_bytes, stream, nullptr);
}

int ark_decode_check(const ark_model* m, int32_t B, const void* workspace, size_t workspace_bytes,
                     void* stream) {
  if (!m || !workspace) return ARK_E_NULL;
  if (!dims_ok(m->d) || B < 1 || B > kMaxBatch) return ARK_E_SHAPE;
  if (workspace_bytes < plan(m->d, B, 1).total) return ARK_E_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  if (!mega_ready(m, B)) return hipStreamSynchronize(st) == hipSuccess ? ARK_OK : ARK_E_HIP;
  return mega_check(m, (const char*)workspace, st);
}

int ark_decode_path(const ark_model* m, int32_t B) {
  if (!m) return ARK_E_NULL;
  if (!dims_ok(m->d) || B < 1 || B > kMaxBatch) return ARK_E_SHAPE;
  return mega_ready(m, B) ? 1 : 0;
}

size_t ark_dump_layout(const ark_dims* d, int32_t B, int32_t S, uint64_t layer_mask,
                       size_t* field_off, size_t* record_bytes, size_t* head_off) {
  if (!d || !dims_ok(*d) || B < 1 || B > kMaxBatch || S < 1) return 0;
  const DumpRec r = dump_rec(*d, B, S, layer_mask, nullptr);
  if (field_off)
    for (int i = 0; i < ARK_DUMP_NFIELDS; ++i) field_off[i] = r.f[i];
  if (record_bytes) *record_bytes = r.rec;
  if (head_off)
    for (int i = 0; i < 4; ++i) head_off[i] = r.head[i];
  return dump_total(*d, B, S, layer_mask);
}

int ark_prefill_dump(const ark_model* m, int32_t B, int32_t S, const float* embeds,
                     const int32_t* cache_position, const float* const* k_cache,
                     const float* const* v_cache, float* k_delta, float* v_delta, float* logits,
                     float* hidden_out, void* workspace, size_t workspace_bytes, void* stream,
                     void* dump, size_t dump_bytes, uint64_t layer_mask) {
  DumpRec dr;
  const int e = dump_check(m, B, S, dump, dump_bytes, layer_mask, &dr);
  if (e) return e;
  return prefill_impl(m, B, S, embeds, cache_position, k_cache, v_cache, k_delta, v_delta, logits,
                      hidden_out, workspace, workspace_bytes, stream, &dr);
}

int ark_decode_step_dump(const ark_model* m, int32_t B, const int32_t* token_ids,
                         const int32_t* cache_position, const float* const* k_cache,
                         const float* const* v_cache, float* k_delta, float* v_delta,
                         float* logits, float* hidden_out, void* workspace,
                         size_t workspace_bytes, void* stream, void* dump, size_t dump_bytes,
                         uint64_t layer_mask) {
  DumpRec dr;
  const int e = dump_check(m, B, 1, dump, dump_bytes, layer_mask, &dr);
  if (e) return e;
  return decode_impl(m, B, token_ids, cache_position, k_cache, v_cache, k_delta, v_delta, logits,
                     hidden_out, workspace, workspace_bytes, stream, &dr);
}

int ark_masked_argmax(int32_t B, int32_t V, const float* logits, const uint8_t* mask,
                      int32_t* out_ids, void* stream) {
  if (!logits || !mask || !out_ids) return ARK_E_NULL;
  if (B < 1 || V < 1) return ARK_E_SHAPE;
  return launch_masked_argmax((hipStream_t)stream, B, V, logits, mask, out_ids) == hipSuccess
             ? ARK_OK
             : ARK_E_HIP;
}

int ark_cache_write(const ark_dims* d, int32_t B, int32_t S, const int32_t* cache_position,
                    float* const* k_cache, float* const* v_cache, const float* k_delta,
                    const float* v_delta, void* stream) {
  if (!d || !cache_position || !k_cache || !v_cache || !k_delta || !v_delta) return ARK_E_NULL;
  if (!dims_ok(*d) || B < 1 || B > kMaxBatch || S < 1) return ARK_E_SHAPE;
  for (int l = 0; l < d->n_layers; ++l) {
    if (!k_cache[l] || !v_cache[l]) return ARK_E_NULL;
    if (!aligned(k_cache[l], 16) || !aligned(v_cache[l], 16)) return ARK_E_ALIGN;
  }
  if (!aligned(k_delta, 16) || !aligned(v_delta, 16)) return ARK_E_ALIGN;
  for (int b = 0; b < B; ++b)
    if (cache_position[b] < 0 || (int64_t)cache_position[b] + S > d->max_total_len)
      return ARK_E_RANGE;
  return launch_cache_write((hipStream_t)stream, d->n_layers, B, S, d->max_total_len,
                            d->n_kv_heads * d->head_dim, cache_position, k_cache, v_cache,
                            k_delta, v_delta) == hipSuccess
             ? ARK_OK
             : ARK_E_HIP;
}

int ark_greedy_decode(const ark_model* m, int32_t B, int32_t* token_ids, int32_t* cache_position,
                      float* const* k_cache, float* const* v_cache, float* k_delta, float* v_delta,
                      float* logits, const uint8_t* mask, int32_t end_id, int32_t max_steps,
                      int32_t check_every, int32_t* out_tokens, void* workspace,
                      size_t workspace_bytes, void* stream) {
  int e = check_model(m, true);
  if (e) return e;
  if (!token_ids || !logits || !mask || !out_tokens) return ARK_E_NULL;
  if (!has_head(m)) return ARK_E_SHAPE;
  if (max_steps < 0 || check_every < 1) return ARK_E_SHAPE;
  e = check_step(m, B, 1, cache_position, (const float* const*)k_cache,
                 (const float* const*)v_cache, k_delta, v_delta, logits, workspace,
                 workspace_bytes);
  if (e) return e;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const Plan p = plan(m->d, B, 1);
  int32_t* done = (int32_t*)(ws + p.done);
  if (hipMemsetAsync(done, 0, (size_t)kMaxBatch * 4, st) != hipSuccess) return ARK_E_HIP;
  std::vector<int32_t> pos(cache_position, cache_position + B);
  std::vector<int32_t> flags(B);
  const int T = m->d.max_total_len;
  const bool mega = mega_ready(m, B);
  if (mega && (e = mega_upload(m, (const float* const*)k_cache, (const float* const*)v_cache, ws, st)))
    return e;
  int steps = 0;
  bool prepared = false;  // the next persistent launch is prepared already
  for (int t = 0; t < max_steps; ++t) {
    bool room = true;
    for (int b = 0; b < B; ++b) room = room && pos[b] + 1 <= T;
    if (!room) break;
    if (mega) {
      // one persistent kernel computes the logits and the masked greedy id;
      // one small kernel then writes its deltas back, applies the stop rule
      // and prepares the next launch
      e = mega_step(m, token_ids, pos[0], k_delta, v_delta, logits, nullptr, mask, token_ids, ws,
                    st, nullptr, !prepared);
      if (e) return e;
      const bool next = t + 1 < max_steps && pos[0] + 2 <= T;
      e = mega_between(m, token_ids, pos[0], k_delta, v_delta, k_cache, v_cache,
                       out_tokens + (size_t)t * B, end_id, done, ws, st, next);
      if (e) return e;
      prepared = next;
    } else {
      e = ark_decode_step(m, B, token_ids, pos.data(), (const float* const*)k_cache,
                          (const float* const*)v_cache, k_delta, v_delta, logits, nullptr,
                          workspace, workspace_bytes, stream);
      if (e) return e;
      if (launch_masked_argmax(st, B, m->d.vocab, logits, mask, token_ids) != hipSuccess)
        return ARK_E_HIP;
      if (launch_greedy_post(st, B, token_ids, out_tokens + (size_t)t * B, end_id, done) !=
          hipSuccess)
        return ARK_E_HIP;
      if (launch_cache_write(st, m->d.n_layers, B, 1, T, m->d.n_kv_heads * m->d.head_dim,
                             pos.data(), k_cache, v_cache, k_delta, v_delta) != hipSuccess)
        return ARK_E_HIP;
    }
    for (int b = 0; b < B; ++b) pos[b] += 1;
    ++steps;
    if ((t + 1) % check_every == 0 || t + 1 == max_steps) {
      if (hipMemcpyAsync(flags.data(), done, (size_t)B * 4, hipMemcpyDeviceToHost, st) !=
              hipSuccess ||
          hipStreamSynchronize(st) != hipSuccess)
        return ARK_E_HIP;
      // a timed-out wait of the persistent kernel invalidates its step (and
      // every token fed back after it): report it instead of the count
      if (mega && (e = mega_check(m, ws, st))) return e;
      bool all = true;
      for (int b = 0; b < B; ++b) all = all && flags[b];
      if (all) break;
    }
  }
  // the loop may have ended on the room check without a final sync
  if (mega && steps > 0 && (e = mega_check(m, ws, st))) return e;
  for (int b = 0; b < B; ++b) cache_position[b] = pos[b];
  return steps;
}

int ark_profile_arm(void* const* events, int32_t n_pairs) {
  if (events && n_pairs < 1) return ARK_E_SHAPE;
  if (events) {
    g_prof.ev.store(nullptr);
    g_prof.n.store(n_pairs);
    g_prof.count.store(0);
    g_prof.ev.store((hipEvent_t*)events);
  } else {
    g_prof.ev.store(nullptr);  // disarming keeps the count of the last armed run
  }
  return ARK_OK;
}

int32_t ark_profile_count(void) { return g_prof.count.load(); }

size_t ark_decode_trace_offset(const ark_dims* d) {
  if (!d || !dims_ok(*d)) return 0;
  return plan(*d, 1, 1).mega + decode_mega_trace_offset(d->n_layers, d->max_total_len);
}

const char* ark_dominant_kernel(void) {
  const char* e = getenv("ARK_DECODE_PATH");
  if (e && strcmp(e, "multi") == 0) return "ark::k_gemv<1, 2, 2>";
  return "ark::mk::k_decode";
}

size_t ark_test_dynquant_workspace_bytes(void) { return 2 * (size_t)kStatsSetInts * 4; }

int ark_test_dynquant(int32_t B, int32_t R, int32_t K, const float* x, uint8_t* codes,
                      float* scale, int32_t* zp, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (!x || !codes || !scale || !zp || !workspace) return ARK_E_NULL;
  if (B < 1 || R < 1 || K < 1) return ARK_E_SHAPE;
  if (workspace_bytes < ark_test_dynquant_workspace_bytes()) return ARK_E_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  if (B > kMaxBatch) return ARK_E_SHAPE;
  int* stw = (int*)workspace;
  const SeqStats sa = {stw, stw + kStatsSetInts, B};
  if (launch_seq_stats_init(st, sa.cur) != hipSuccess) return ARK_E_HIP;
  if (launch_row_stats(st, B * R, K, R, x, K, nullptr, 0.0, nullptr, sa) != hipSuccess)
    return ARK_E_HIP;
  if (launch_quant_seq(st, B * R, K, R, x, K, nullptr, nullptr, sa.cur, nullptr, codes, scale,
                       zp) != hipSuccess)
    return ARK_E_HIP;
  return ARK_OK;
}

int ark_test_layernorm(int32_t B, int32_t S, int32_t D, const float* x, const float* g,
                       const float* b, double eps, float* y, float* lo, float* hi,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (!x || !g || !b || !y || !lo || !hi || !workspace) return ARK_E_NULL;
  if (B < 1 || B > kMaxBatch || S < 1 || D < 1 || !(eps >= 0.0)) return ARK_E_SHAPE;
  if (workspace_bytes < ark_test_dynquant_workspace_bytes()) return ARK_E_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  int* stw = (int*)workspace;
  const SeqStats sa = {stw, stw + kStatsSetInts, B};
  HIP_TRY(launch_seq_stats_init(st, sa.cur));
  HIP_TRY(launch_layernorm(st, B * S, D, S, x, g, b, eps, y, sa));
  HIP_TRY(launch_seq_stats_read(st, sa.cur, B, lo, hi));
  return ARK_OK;
}

size_t ark_test_enc_attention_workspace_bytes(int32_t B, int32_t F, int32_t H) {
  if (B < 1 || F < 1 || H < 1) return 0;
  return align_up(ark_test_dynquant_workspace_bytes()) + enc_attention_ws_bytes(B, F, H);
}

int ark_test_enc_attention(int32_t B, int32_t F, int32_t H, const float* qkv,
                           const double* rope_cos, const double* rope_sin, float* out, float* lo,
                           float* hi, void* workspace, size_t workspace_bytes, void* stream) {
  if (!qkv || !rope_cos || !rope_sin || !out || !lo || !hi || !workspace) return ARK_E_NULL;
  if (B < 1 || B > kMaxBatch || F < 1 || H < 1) return ARK_E_SHAPE;
  if (!aligned(qkv, 16)) return ARK_E_ALIGN;
  if (workspace_bytes < ark_test_dynquant_workspace_bytes()) return ARK_E_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  int* stw = (int*)workspace;
  const SeqStats sa = {stw, stw + kStatsSetInts, B};
  // the split form when the workspace holds its states
  void* part = workspace_bytes >= ark_test_enc_attention_workspace_bytes(B, F, H) &&
                       enc_attention_ws_bytes(B, F, H) > 0
                   ? (char*)workspace + align_up(ark_test_dynquant_workspace_bytes())
                   : nullptr;
  HIP_TRY(launch_seq_stats_init(st, sa.cur));
  HIP_TRY(launch_enc_attention(st, B, F, H, qkv, rope_cos, rope_sin, out, sa, part));
  HIP_TRY(launch_seq_stats_read(st, sa.cur, B, lo, hi));
  return ARK_OK;
}

size_t ark_test_qlinear_workspace_bytes(int32_t rows, int32_t k, int32_t use_gemm) {
  if (rows < 1 || k < 1) return 0;
  return align_up((size_t)rows * (k + 8) + 256) + (use_gemm == 1 ? gemm_ws_bytes(rows) : 0);
}

int ark_test_qlinear(int32_t B, int32_t R, const uint8_t* codes, const float* scale,
                     const uint8_t* zp, const ark_qlinear* W, int32_t* acc, float* y,
                     int32_t use_gemm, void* workspace, size_t workspace_bytes, void* stream) {
  if (!codes || !scale || !zp || !W || !y || !workspace) return ARK_E_NULL;
  if (!W->w || !W->scale || !W->colsum) return ARK_E_NULL;
  if (B < 1 || R < 1 || W->n < 1 || W->k < 64 || W->k % 64) return ARK_E_SHAPE;
  const int rows = B * R;
  if (!use_gemm && rows > 4) return ARK_E_SHAPE;
  if (use_gemm < 0 || use_gemm > 2) return ARK_E_SHAPE;
  const size_t base = align_up((size_t)rows * (W->k + 8) + 256);
  const size_t need = base + (use_gemm == 1 ? gemm_ws_bytes(rows) : 0);
  if (workspace_bytes < need) return ARK_E_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  int8_t* sc = (int8_t*)ws;
  float* srow = (float*)(ws + align_up((size_t)rows * W->k));
  int* zrow = (int*)(srow + rows);
  if (launch_test_codes(st, rows, W->k, R, codes, sc, scale, zp, srow, zrow) != hipSuccess)
    return ARK_E_HIP;
  Seg s = seg_of(*W, y, W->n);
  hipError_t err;
  if (use_gemm == 1) {
    void* gsk = ws + base;
    err = gemm_scratch_reset(st, gsk, rows);
    if (err == hipSuccess)
      err = launch_gemm(st, rows, W->k, sc, srow, zrow, 1, &s, 1, EPI_STORE, acc, gsk);
  } else if (use_gemm == 2) {
    err = launch_gemm(st, rows, W->k, sc, srow, zrow, 1, &s, 1, EPI_STORE, acc, nullptr, true);
  } else {
    err = launch_gemv_codes(st, rows, W->k, sc, srow, zrow, &s, 1, EPI_STORE, acc);
  }
  return err == hipSuccess ? ARK_OK : ARK_E_HIP;
}

size_t ark_test_gate_up_workspace_bytes(int32_t B, int32_t R, int32_t k) {
  if (B < 1 || R < 1 || k < 1) return 0;
  const size_t rows = (size_t)B * R;
  return align_up(rows * k) + 2 * align_up(rows * 4) + 3 * align_up((size_t)B * 4) +
         ark_test_dynquant_workspace_bytes() + gemm_ws_bytes(rows);
}

int ark_test_swiglu(int64_t n, const float* g, const float* u, float* y, void* stream) {
  if (n < 0) return ARK_E_SHAPE;
  if (n > 0 && (!g || !u || !y)) return ARK_E_NULL;
  return launch_swiglu((hipStream_t)stream, n, g, u, y) == hipSuccess ? ARK_OK : ARK_E_HIP;
}

int ark_test_gate_up(int32_t B, int32_t R, const uint8_t* codes, const float* scale,
                     const uint8_t* zp, const ark_qlinear* gate, const ark_qlinear* up, float* y,
                     float* seq_min, float* seq_max, void* workspace, size_t workspace_bytes,
                     void* stream) {
  if (!codes || !scale || !zp || !gate || !up || !y || !seq_min || !seq_max || !workspace)
    return ARK_E_NULL;
  if (!gate->w || !gate->scale || !gate->colsum || !up->w || !up->scale || !up->colsum)
    return ARK_E_NULL;
  if (B < 1 || R < 1 || B > kMaxBatch) return ARK_E_SHAPE;
  const int n = gate->n, k = gate->k;
  if (up->n != n || up->k != k || n < 1 || k < 64 || k % 64) return ARK_E_SHAPE;
  if (workspace_bytes < ark_test_gate_up_workspace_bytes(B, R, k)) return ARK_E_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const int rows = B * R;
  char* ws = (char*)workspace;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    char* at = ws + o;
    o += align_up(bytes);
    return at;
  };
  int8_t* sc = (int8_t*)take((size_t)rows * k);
  float* srow = (float*)take((size_t)rows * 4);
  int* zrow = (int*)take((size_t)rows * 4);
  float* sseq = (float*)take((size_t)B * 4);
  int* zseq = (int*)take((size_t)B * 4);
  int8_t* junk = (int8_t*)take((size_t)B * 4);
  int* stw = (int*)take(ark_test_dynquant_workspace_bytes());
  void* gsk = take(gemm_ws_bytes(rows));
  const SeqStats sa = {stw, stw + kStatsSetInts, B};
  // shifted codes, then the per-sequence (s, z) as one-column "rows"
  HIP_TRY(launch_test_codes(st, rows, k, R, codes, sc, scale, zp, srow, zrow));
  HIP_TRY(launch_test_codes(st, B, 1, 1, codes, junk, scale, zp, sseq, zseq));
  HIP_TRY(gemm_scratch_reset(st, gsk, rows));
  HIP_TRY(launch_seq_stats_init(st, sa.cur));
  Seg gus[2] = {seg_of(*gate, y, n), seg_of(*up, y, n)};
  const bool fused = gemm_swiglu_stats(rows, k, gsk);
  HIP_TRY(launch_gemm(st, rows, k, sc, sseq, zseq, R, gus, 2, EPI_SWIGLU, nullptr, gsk, false,
                      fused ? &sa : nullptr));
  if (!fused) HIP_TRY(launch_row_stats(st, rows, n, R, y, n, nullptr, 0.0, nullptr, sa));
  HIP_TRY(launch_seq_stats_read(st, sa.cur, B, seq_min, seq_max));
  return ARK_OK;
}

size_t ark_test_attention_workspace_bytes(int32_t B, int32_t S, int32_t n_heads, int32_t T) {
  if (B < 1 || S < 1 || n_heads < 1 || T < 1) return 0;
  return align_up(attention_ws_bytes(B, S, n_heads, T)) + ark_test_dynquant_workspace_bytes();
}

int ark_test_attention(int32_t B, int32_t S, int32_t n_heads, int32_t n_kv_heads, int32_t T,
                       const int32_t* cache_position, const float* q, const float* k_cache,
                       const float* v_cache, const float* k_delta, const float* v_delta,
                       float* out, float* seq_min, float* seq_max, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (!cache_position || !q || !k_cache || !v_cache || !k_delta || !v_delta || !out || !seq_min ||
      !seq_max || !workspace)
    return ARK_E_NULL;
  if (B < 1 || B > kMaxBatch || S < 1 || n_kv_heads < 1 || n_heads % n_kv_heads ||
      n_heads / n_kv_heads > 8 || T < 32 || T % 32 || T > 8192)
    return ARK_E_SHAPE;
  for (int b = 0; b < B; ++b)
    if (cache_position[b] < 0 || cache_position[b] + S > T) return ARK_E_RANGE;
  if (workspace_bytes < ark_test_attention_workspace_bytes(B, S, n_heads, T))
    return ARK_E_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  int* stw = (int*)(ws + align_up(attention_ws_bytes(B, S, n_heads, T)));
  const SeqStats sa = {stw, stw + kStatsSetInts, B};
  PosArgs pos;
  memset(&pos, 0, sizeof(pos));
  int pmax = 0;
  for (int b = 0; b < B; ++b) {
    pos.p[b] = cache_position[b];
    pmax = std::max(pmax, cache_position[b]);
  }
  HIP_TRY(launch_seq_stats_init(st, sa.cur));
  const bool fused = attention_stats(B, S, n_heads, n_kv_heads, T, pmax);
  HIP_TRY(launch_attention(st, B, S, n_heads, n_kv_heads, T, q, k_cache, v_cache, k_delta,
                           v_delta, pos, out, ws, fused ? &sa : nullptr));
  const int Q = n_heads * kHeadDim;
  if (!fused) HIP_TRY(launch_row_stats(st, B * S, Q, S, out, Q, nullptr, 0.0, nullptr, sa));
  HIP_TRY(launch_seq_stats_read(st, sa.cur, B, seq_min, seq_max));
  return ARK_OK;
}

}  // extern "C"
