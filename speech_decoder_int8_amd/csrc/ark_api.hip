// C ABI of the decoder step: host-side validation, workspace planning and
// kernel sequencing.  Validation touches no HIP API, so every error path can
// be exercised without a GPU; a call that fails validation enqueues nothing.
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "../../include/ark.h"
#include "common.hpp"
#include "kernels.hpp"

using namespace ark;

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

struct Plan {
  size_t x, rs, codes, qkv, q, attn, a, stats, qs, qz, part, done, gsk, mega, total;
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
  p.part = take(attention_ws_bytes(B, 1, d.n_heads, d.max_total_len));
  p.done = take((size_t)kMaxBatch * 4);
  p.gsk = take(gemm_skinny_ws_bytes());
  p.mega = take(B == 1 ? decode_mega_ws_bytes(d.n_layers, d.max_total_len) : 0);
  p.total = o;
  return p;
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
  if (m->lm_head.w) {
    if (!m->final_norm) return ARK_E_NULL;
    int e;
    if ((e = check_qlinear(m->lm_head, d.vocab, H, false))) return e;
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
  if (logits && !m->lm_head.w) return ARK_E_SHAPE;
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
struct Profiler {
  hipEvent_t* ev = nullptr;
  int n = 0;
  int count = 0;
};
Profiler g_prof;

inline void prof_begin(hipStream_t st, bool dominant) {
  if (dominant && g_prof.ev && g_prof.count < g_prof.n) hipEventRecord(g_prof.ev[2 * g_prof.count], st);
}
inline void prof_end(hipStream_t st, bool dominant) {
  if (dominant && g_prof.ev && g_prof.count < g_prof.n) {
    hipEventRecord(g_prof.ev[2 * g_prof.count + 1], st);
    ++g_prof.count;
  }
}

#define HIP_TRY(expr)                       \
  do {                                      \
    if ((expr) != hipSuccess) return ARK_E_HIP; \
  } while (0)

// All layers and the LM head over the rows already in x ([B*S][H]).
int run_forward(const ark_model* m, int B, int S, float* x, const int32_t* pos_host,
                const float* const* kc, const float* const* vc, float* kd, float* vd,
                float* logits, char* ws, hipStream_t st) {
  const ark_dims& d = m->d;
  const Plan p = plan(d, B, S);
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
  void* gsk = ws + p.gsk;  // few-row GEMM scratch
  HIP_TRY(gemm_skinny_reset(st, gsk));
  if (!gemv && !rowq) HIP_TRY(launch_seq_stats_init(st, sa.cur));
  PosArgs pos;
  memset(&pos, 0, sizeof(pos));
  for (int b = 0; b < B; ++b) pos.p[b] = pos_host[b];
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
      HIP_TRY(launch_gemv(st, B, H, x, H, L.ln1, d.rms_eps, qkvs, 3, EPI_STORE));
    } else if (rowq) {
      HIP_TRY(launch_norm_quant_row(st, B, H, x, H, L.ln1, d.rms_eps, codes, qs, qz));
      HIP_TRY(launch_gemm(st, R, H, codes, qs, qz, S, qkvs, 3, EPI_STORE, nullptr, gsk));
    } else {
      HIP_TRY(launch_row_stats(st, R, H, S, x, H, L.ln1, d.rms_eps, rs, sa));
      HIP_TRY(launch_quant_seq(st, R, H, S, x, H, rs, L.ln1, sa.cur, codes, nullptr, qs, qz));
      HIP_TRY(launch_gemm(st, R, H, codes, qs, qz, S, qkvs, 3, EPI_STORE, nullptr, gsk));
    }
    // decode: the rotary step runs inside the attention kernel
    const bool rope_in_attn = S == 1 && NH / NKV <= 8;
    if (!rope_in_attn)
      HIP_TRY(launch_rope(st, B, S, NH, NKV, qkv, m->rope_cos, m->rope_sin, pos, q, kdl, vdl));
    const RopeIn ri = {qkv, ldqkv, m->rope_cos, m->rope_sin, kdl, vdl};
    const bool att_stats = !gemv && !rowq && attention_stats(S, NH, NKV);
    HIP_TRY(launch_attention(st, B, S, NH, NKV, T, q, kc[l], vc[l], kdl, vdl, pos, attn, part,
                             att_stats ? &sb : nullptr, rope_in_attn ? &ri : nullptr));
    if (gemv) {
      HIP_TRY(launch_gemv(st, B, Q, attn, Q, nullptr, 0.0, os, 1, EPI_RESID));
      prof_begin(st, B == 1);
      HIP_TRY(launch_gemv(st, B, H, x, H, L.ln2, d.rms_eps, gus, 2, EPI_SWIGLU));
      prof_end(st, B == 1);
      HIP_TRY(launch_gemv(st, B, I, a, I, nullptr, 0.0, ds, 1, EPI_RESID));
    } else if (rowq) {
      HIP_TRY(launch_norm_quant_row(st, B, Q, attn, Q, nullptr, 0.0, codes, qs, qz));
      HIP_TRY(launch_gemm(st, R, Q, codes, qs, qz, S, os, 1, EPI_RESID, nullptr, gsk));
      HIP_TRY(launch_norm_quant_row(st, B, H, x, H, L.ln2, d.rms_eps, codes, qs, qz));
      HIP_TRY(launch_gemm(st, R, H, codes, qs, qz, S, gus, 2, EPI_SWIGLU, nullptr, gsk));
      HIP_TRY(launch_norm_quant_row(st, B, I, a, I, nullptr, 0.0, codes, qs, qz));
      HIP_TRY(launch_gemm(st, R, I, codes, qs, qz, S, ds, 1, EPI_RESID, nullptr, gsk));
    } else {
      if (!att_stats) HIP_TRY(launch_row_stats(st, R, Q, S, attn, Q, nullptr, 0.0, nullptr, sb));
      HIP_TRY(launch_quant_seq(st, R, Q, S, attn, Q, nullptr, nullptr, sb.cur, codes, nullptr, qs,
                               qz));
      HIP_TRY(launch_gemm(st, R, Q, codes, qs, qz, S, os, 1, EPI_RESID, nullptr, gsk));
      HIP_TRY(launch_row_stats(st, R, H, S, x, H, L.ln2, d.rms_eps, rs, sa));
      HIP_TRY(launch_quant_seq(st, R, H, S, x, H, rs, L.ln2, sa.cur, codes, nullptr, qs, qz));
      const bool gu_stats = gemm_swiglu_stats(R, H, gsk);
      HIP_TRY(launch_gemm(st, R, H, codes, qs, qz, S, gus, 2, EPI_SWIGLU, nullptr, gsk, false,
                          gu_stats ? &sb : nullptr));
      if (!gu_stats) HIP_TRY(launch_row_stats(st, R, I, S, a, I, nullptr, 0.0, nullptr, sb));
      HIP_TRY(launch_quant_seq(st, R, I, S, a, I, nullptr, nullptr, sb.cur, codes, nullptr, qs, qz));
      HIP_TRY(launch_gemm(st, R, I, codes, qs, qz, S, ds, 1, EPI_RESID, nullptr, gsk));
    }
  }

  if (logits) {
    Seg lm[1] = {seg_of(m->lm_head, logits, d.vocab)};
    const float* last = x + (size_t)(S - 1) * H;  // row S-1 of each sequence, stride S*H
    if (B <= 4) {
      HIP_TRY(launch_gemv(st, B, H, last, S * H, m->final_norm, d.rms_eps, lm, 1, EPI_STORE));
    } else {
      if (norm_quant_row_supported(H)) {
        HIP_TRY(launch_norm_quant_row(st, B, H, last, S * H, m->final_norm, d.rms_eps, codes, qs,
                                      qz));
      } else {
        // set A is clear here: the last producer of the layers (if any) filled B
        HIP_TRY(launch_row_stats(st, B, H, 1, last, S * H, m->final_norm, d.rms_eps, rs, sa));
        HIP_TRY(launch_quant_seq(st, B, H, 1, last, S * H, rs, m->final_norm, sa.cur, codes,
                                 nullptr, qs, qz));
      }
      HIP_TRY(launch_gemm(st, B, H, codes, qs, qz, 1, lm, 1, EPI_STORE, nullptr, gsk));
    }
  }
  return ARK_OK;
}

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

int mega_step(const ark_model* m, const int32_t* token, int pos, float* kd, float* vd,
              float* logits, float* hidden_out, const uint8_t* mask, int32_t* out_token, char* ws,
              hipStream_t st) {
  const ark_dims& d = m->d;
  const Plan p = plan(d, 1, 1);
  MegaStep S;
  S.L = d.n_layers;
  S.T = d.max_total_len;
  S.V = d.vocab;
  S.pos = pos;
  S.eps = d.rms_eps;
  S.token = token;
  S.table = m->embed_f16;
  S.final_norm = logits ? m->final_norm : nullptr;
  S.lm_w = logits ? m->lm_head.w : nullptr;
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
  hipEvent_t eb = nullptr, ee = nullptr;
  if (g_prof.ev && g_prof.count < g_prof.n) {
    eb = g_prof.ev[2 * g_prof.count];
    ee = g_prof.ev[2 * g_prof.count + 1];
    ++g_prof.count;
  }
  const hipError_t e = decode_mega_launch(st, ws + p.mega, S, eb, ee);
  return e == hipSuccess ? ARK_OK : ARK_E_HIP;
}

bool mega_ready(const ark_model* m, int B) {
  return use_mega(m->d, B, 1) && decode_mega_init() == hipSuccess;
}

}  // namespace

extern "C" {

const char* ark_status_string(int status) {
  switch (status) {
    case ARK_OK: return "ok";
    case ARK_E_NULL: return "a required pointer is NULL";
    case ARK_E_SHAPE: return "a size is invalid, inconsistent or unsupported";
    case ARK_E_RANGE: return "cache_position out of range for the static cache";
    case ARK_E_WORKSPACE: return "workspace too small";
    case ARK_E_HIP: return "HIP launch failed";
    case ARK_E_ALIGN: return "pointer misaligned";
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
                     st);
}

int ark_decode_step(const ark_model* m, int32_t B, const int32_t* token_ids,
                    const int32_t* cache_position, const float* const* k_cache,
                    const float* const* v_cache, float* k_delta, float* v_delta, float* logits,
                    float* hidden_out, void* workspace, size_t workspace_bytes, void* stream) {
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
                     nullptr, ws, st);
  }
  const Plan p = plan(m->d, B, 1);
  float* x = hidden_out ? hidden_out : (float*)(ws + p.x);
  if (launch_embed(st, B, 1, m->d.hidden, m->d.vocab, token_ids, m->embed_f16, nullptr, 0, 0, x) !=
      hipSuccess)
    return ARK_E_HIP;
  return run_forward(m, B, 1, x, cache_position, k_cache, v_cache, k_delta, v_delta, logits, ws,
                     st);
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
  if (!m->lm_head.w) return ARK_E_SHAPE;
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
  for (int t = 0; t < max_steps; ++t) {
    bool room = true;
    for (int b = 0; b < B; ++b) room = room && pos[b] + 1 <= T;
    if (!room) break;
    if (mega) {
      // one persistent kernel computes the logits and the masked greedy id
      e = mega_step(m, token_ids, pos[0], k_delta, v_delta, logits, nullptr, mask, token_ids, ws,
                    st);
      if (e) return e;
    } else {
      e = ark_decode_step(m, B, token_ids, pos.data(), (const float* const*)k_cache,
                          (const float* const*)v_cache, k_delta, v_delta, logits, nullptr,
                          workspace, workspace_bytes, stream);
      if (e) return e;
      if (launch_masked_argmax(st, B, m->d.vocab, logits, mask, token_ids) != hipSuccess)
        return ARK_E_HIP;
    }
    if (launch_greedy_post(st, B, token_ids, out_tokens + (size_t)t * B, end_id, done) !=
        hipSuccess)
      return ARK_E_HIP;
    if (launch_cache_write(st, m->d.n_layers, B, 1, T, m->d.n_kv_heads * m->d.head_dim,
                           pos.data(), k_cache, v_cache, k_delta, v_delta) != hipSuccess)
      return ARK_E_HIP;
    for (int b = 0; b < B; ++b) pos[b] += 1;
    ++steps;
    if ((t + 1) % check_every == 0 || t + 1 == max_steps) {
      if (hipMemcpyAsync(flags.data(), done, (size_t)B * 4, hipMemcpyDeviceToHost, st) !=
              hipSuccess ||
          hipStreamSynchronize(st) != hipSuccess)
        return ARK_E_HIP;
      bool all = true;
      for (int b = 0; b < B; ++b) all = all && flags[b];
      if (all) break;
    }
  }
  for (int b = 0; b < B; ++b) cache_position[b] = pos[b];
  return steps;
}

int ark_profile_arm(void* const* events, int32_t n_pairs) {
  if (events && n_pairs < 1) return ARK_E_SHAPE;
  g_prof.ev = events ? (hipEvent_t*)events : nullptr;
  g_prof.n = events ? n_pairs : 0;
  if (events) g_prof.count = 0;  // disarming keeps the count of the last armed run
  return ARK_OK;
}

int32_t ark_profile_count(void) { return g_prof.count; }

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

size_t ark_test_qlinear_workspace_bytes(int32_t rows, int32_t k, int32_t use_gemm) {
  if (rows < 1 || k < 1) return 0;
  return align_up((size_t)rows * (k + 8) + 256) + (use_gemm == 1 ? gemm_skinny_ws_bytes() : 0);
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
  const size_t need = base + (use_gemm == 1 ? gemm_skinny_ws_bytes() : 0);
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
    err = gemm_skinny_reset(st, gsk);
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
         ark_test_dynquant_workspace_bytes() + gemm_skinny_ws_bytes();
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
  void* gsk = take(gemm_skinny_ws_bytes());
  const SeqStats sa = {stw, stw + kStatsSetInts, B};
  // shifted codes, then the per-sequence (s, z) as one-column "rows"
  HIP_TRY(launch_test_codes(st, rows, k, R, codes, sc, scale, zp, srow, zrow));
  HIP_TRY(launch_test_codes(st, B, 1, 1, codes, junk, scale, zp, sseq, zseq));
  HIP_TRY(gemm_skinny_reset(st, gsk));
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
  for (int b = 0; b < B; ++b) pos.p[b] = cache_position[b];
  HIP_TRY(launch_seq_stats_init(st, sa.cur));
  const bool fused = attention_stats(S, n_heads, n_kv_heads);
  HIP_TRY(launch_attention(st, B, S, n_heads, n_kv_heads, T, q, k_cache, v_cache, k_delta,
                           v_delta, pos, out, ws, fused ? &sa : nullptr));
  const int Q = n_heads * kHeadDim;
  if (!fused) HIP_TRY(launch_row_stats(st, B * S, Q, S, out, Q, nullptr, 0.0, nullptr, sa));
  HIP_TRY(launch_seq_stats_read(st, sa.cur, B, seq_min, seq_max));
  return ARK_OK;
}

}  // extern "C"
