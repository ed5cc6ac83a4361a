// Prefill attention on fp64 matrix cores (v_mfma_f64_16x16x4f64).
//
// Same computation as the prefill path of k_attn (model card
// "ark-asr-3b-onnx", section "Shapes": every query row attends the whole
// static cache, masked beyond its own position; rows [p, p + S) come from
// this call's deltas): scores q.k * (1/sqrt(128)), softmax and the weighted
// sum in fp64, fp32 out.  Only the 64-key chunks that hold a key some row of
// the tile may see are visited; keys past p + S are staged as zeros (their
// cache contents never reach a product), and every masked score is selected
// out before the exponential.
//
// One workgroup = one (sequence, KV head g, 16-row query tile), one wave per
// query head of g (the K/V chunk is staged in LDS once for all of them); a
// launch of few workgroups gives each half of g's heads, and may deal the
// tile's key chunks over several workgroups whose softmax states a merge
// kernel combines (attention_prefill_split).  A
// wave computes S^T = K Q^T as 16x16 blocks (A = 16 keys x 4 dims of K,
// B = 4 dims x 16 rows of Q^T, kept in registers), the online-softmax update
// per row, and O^T += V^T P^T (A = 16 dims x 4 keys of V^T, B = 4 keys x 16
// rows of P^T).  Fragment layout (16x16x4 f64): lane l supplies
// A[l % 16][l / 16] and B[l / 16][l % 16]; the 16x16 result holds
// C[4 i + l / 16][l % 16] in register i.  So the score block kb leaves
// P^T[16 kb + 4 i + l / 16][l % 16] in lane l's register i, which is the B
// operand that lane supplies for keys 4 t .. 4 t + 3 with t = 4 kb + i: the
// weights never leave the registers.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace ark {

typedef double f64x4 __attribute__((ext_vector_type(4)));

namespace a2 {
constexpr int KC = 64;    // keys per chunk
// The chunk is staged widened to fp64 once for all waves (the matrix
// operands are then read as they are, without a conversion per wave).
// Row pitches in doubles: an 8-byte fragment read of K (16 keys x 2 dims
// per half wave) and of V (16 dims x 2 keys per half wave) touches each
// LDS bank once per half wave.
constexpr int KP = 130;
constexpr int VP = 144;
constexpr int QT = 16;    // query rows per workgroup
constexpr int GMAX = 8;   // query heads per KV head
constexpr int LDS_BYTES = KC * KP * 8 + KC * VP * 8;
}  // namespace a2

struct Attn2Params {
  int B, S, NH, NKV, G, T, nqt;
  const float* q;
  const float* kc;
  const float* vc;
  const float* kd;
  const float* vd;
  PosArgs pos;
  float* out;
  SeqStats stats;  // per-sequence min/max of out (cur == nullptr: off)
  // nsplit > 1: the key chunks of a query tile are dealt over nsplit
  // workgroups (chunk c to split c % nsplit), each writing its unnormalised
  // softmax state per row and head to part ([B][NH][S][nsplit][2 + 128]:
  // max, sum, weighted values); the split merge writes out
  int nsplit;
  double* part;
  int hsplit;  // query heads of a KV head dealt over hsplit workgroups
};

// four fp32 values widened into LDS (exact)
__device__ __forceinline__ void put4(double* dst, float4 v) {
  *(double2*)dst = double2{(double)v.x, (double)v.y};
  *(double2*)(dst + 2) = double2{(double)v.z, (double)v.w};
}

// BF: the bf16 serving variant (q, caches, deltas and the output in bf16,
// the output rounded once more from the fp32 value; no range).
template <bool BF>
__global__ __launch_bounds__(512) void k_attn_prefill(Attn2Params P) {
  using namespace a2;
  extern __shared__ __align__(16) unsigned char smem[];
  double* Ks = (double*)smem;                    // [KC][KP]
  double* Vs = Ks + KC * KP;                     // [KC][VP]
  if (!BF && P.stats.cur) stats_clear_other(P.stats);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nthr = blockDim.x;
  // heavy (late) query tiles first
  const int ns = max(P.nsplit, 1), hs = max(P.hsplit, 1);
  const int split = (int)blockIdx.x % ns, hsel = ((int)blockIdx.x / ns) % hs;
  const int tix = (int)blockIdx.x / (ns * hs);
  const int nbg = P.B * P.NKV;
  const int qt = P.nqt - 1 - tix / nbg;
  const int bg = tix % nbg;
  const int b = bg / P.NKV, g = bg % P.NKV;
  const int i0 = qt * QT;
  const int p = P.pos.p[b];
  const int S = P.S, T = P.T;
  const int h = g * P.G + hsel * (P.G / hs) + wave;
  const int c16 = lane & 15, q4 = lane >> 4;
  const int qrow = i0 + c16;                     // this lane's query row
  const bool rowok = qrow < S;
  const int qpos = p + qrow;
  const int maxq = p + min(i0 + QT - 1, S - 1);  // last key any row of the tile sees
  const int live_end = min(p + S, T);            // rows at or past it are never seen

  // B operand of S^T = K Q^T: Q[qrow][4s + q4], s = 0..31
  // (all 32 loads issued before the first use; a row past S loads row S - 1
  // and is zeroed)
  double qv[32];
  {
    const size_t qoff = ((size_t)(b * S + min(qrow, S - 1)) * P.NH + h) * kHeadDim;
    float qf[32];
    if constexpr (BF) {
      const gptr<const uint16_t> src = uniform_ptr((const uint16_t*)P.q) + qoff;
#pragma unroll
      for (int s = 0; s < 32; ++s) qf[s] = bf2f(src[4 * s + q4]);
    } else {
      const gptr<const float> src = uniform_ptr(P.q) + qoff;
#pragma unroll
      for (int s = 0; s < 32; ++s) qf[s] = src[4 * s + q4];
    }
#pragma unroll
    for (int s = 0; s < 32; ++s) qv[s] = rowok ? (double)qf[s] : 0.0;
  }
  f64x4 o[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) o[d] = f64x4{0.0, 0.0, 0.0, 0.0};
  double m = -INFINITY, l = 0.0;
  const double scale = 1.0 / sqrt((double)kHeadDim);
  const SwigluK EK = swiglu_consts();  // constants of the exponential below

  const int nch = maxq / KC + 1;
  // float4 e of a chunk (key jj = e / 32, dims 4 (e % 32) ..) from the cache
  // or this call's deltas; zero past the rows any query sees
  // (the four base pointers are wave-uniform values: a per-lane choice
  // between them is a select, not a load of the parameter block)
  const gptr<const float> kcp = uniform_ptr(P.kc), vcp = uniform_ptr(P.vc);
  const gptr<const float> kdp = uniform_ptr(P.kd), vdp = uniform_ptr(P.vd);
  auto fetch = [&](int j0, int e, float4& kv, float4& vv) {
    const int jj = e >> 5, d4 = e & 31;
    const int j = j0 + jj;
    kv = make_float4(0.f, 0.f, 0.f, 0.f);
    vv = kv;
    if (j < live_end) {
      const bool dl = j >= p;  // this call's rows come from the deltas
      const size_t off = dl ? ((size_t)(b * S + (j - p)) * P.NKV + g) * kHeadDim
                            : ((size_t)(b * T + j) * P.NKV + g) * kHeadDim;
      kv = ld4e<BF>(dl ? kdp : kcp, off, d4);
      vv = ld4e<BF>(dl ? vdp : vcp, off, d4);
    }
  };
  // with 512 threads (8 query heads) each thread holds 4 float4 of K and of V
  // of the next chunk in registers while the current one is computed
  constexpr int PF = KC * (kHeadDim / 4) / 512;
  const bool piped = nthr == 512;
  float4 kn[PF], vn[PF];
  if (piped)
#pragma unroll
    for (int u = 0; u < PF; ++u) fetch(split * KC, tid + 512 * u, kn[u], vn[u]);
  for (int c = split; c < nch; c += ns) {
    const int j0 = c * KC;
    __syncthreads();  // the previous chunk's K, V and P are used
    if (piped) {
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        const int e = tid + 512 * u, jj = e >> 5, d4 = e & 31;
        put4(Ks + jj * KP + 4 * d4, kn[u]);
        put4(Vs + jj * VP + 4 * d4, vn[u]);
      }
      if (c + ns < nch)
#pragma unroll
        for (int u = 0; u < PF; ++u) fetch(j0 + ns * KC, tid + 512 * u, kn[u], vn[u]);
    } else {
      for (int e = tid; e < KC * (kHeadDim / 4); e += nthr) {
        float4 kv, vv;
        fetch(j0, e, kv, vv);
        const int jj = e >> 5, d4 = e & 31;
        put4(Ks + jj * KP + 4 * d4, kv);
        put4(Vs + jj * VP + 4 * d4, vv);
      }
    }
    __syncthreads();

    // scores: sc[kb][i] = S^T[key j0 + 16 kb + 4 i + q4][qrow]
    f64x4 sc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      sc[kb] = f64x4{0.0, 0.0, 0.0, 0.0};
      const double* kr = Ks + (16 * kb + c16) * KP + q4;
#pragma unroll
      for (int s = 0; s < 32; ++s)
        sc[kb] = __builtin_amdgcn_mfma_f64_16x16x4f64(kr[4 * s], qv[s], sc[kb], 0, 0, 0);
    }
    double cmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + 16 * kb + 4 * i + q4;
        const double v = (rowok && j <= qpos) ? sc[kb][i] * scale : -INFINITY;
        sc[kb][i] = v;
        cmax = fmax(cmax, v);
      }
    cmax = fmax(cmax, __shfl_xor(cmax, 16, kWave));
    cmax = fmax(cmax, __shfl_xor(cmax, 32, kWave));
    const double mnew = fmax(m, cmax);
    // every argument of the exponential is <= 0 (m, scores <= mnew)
    const double alpha = (m == -INFINITY) ? 0.0 : exp_nonpos_f64(m - mnew, EK);
    double lsum = 0.0;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double e = (sc[kb][i] == -INFINITY) ? 0.0 : exp_nonpos_f64(sc[kb][i] - mnew, EK);
        lsum += e;
        sc[kb][i] = e;  // P^T[key 16 kb + 4 i + q4][qrow]
      }
    lsum += __shfl_xor(lsum, 16, kWave);
    lsum += __shfl_xor(lsum, 32, kWave);
    l = l * alpha + lsum;
    m = mnew;
#pragma unroll
    for (int d = 0; d < 8; ++d) o[d] *= alpha;
    // O^T[dim][row] += V^T[dim][key] P^T[key][row], 16 steps of 4 keys
#pragma unroll
    for (int t = 0; t < KC / 4; ++t) {
      const double pb = sc[t >> 2][t & 3];
      const double* vr = Vs + (4 * t + q4) * VP + c16;
#pragma unroll
      for (int d = 0; d < 8; ++d)
        o[d] = __builtin_amdgcn_mfma_f64_16x16x4f64(vr[16 * d], pb, o[d], 0, 0, 0);
    }
  }
  // o[d][i] = O^T[dim 16 d + 4 i + q4][qrow]
  if (ns > 1) {
    // this split's state of row qrow, head h (a split that saw no chunk
    // leaves the empty state: m = -inf, l = 0, o = 0)
    if (rowok) {
      double* dst = P.part + ((((size_t)b * P.NH + h) * S + qrow) * ns + split) * (2 + kHeadDim);
      if (q4 == 0) {
        dst[0] = m;
        dst[1] = l;
      }
#pragma unroll
      for (int d = 0; d < 8; ++d)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[2 + 16 * d + 4 * i + q4] = o[d][i];
    }
    return;
  }
  const size_t doff = ((size_t)(b * S + qrow) * P.NH + h) * kHeadDim;
  float lo = INFINITY, hi = -INFINITY;
  if (rowok) {
#pragma unroll
    for (int d = 0; d < 8; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float y = (float)(o[d][i] / l);
        if constexpr (BF)
          ((uint16_t*)P.out)[doff + 16 * d + 4 * i + q4] = f2bf(y);
        else
          P.out[doff + 16 * d + 4 * i + q4] = y;
        lo = fminf(lo, y);
        hi = fmaxf(hi, y);
      }
  }
  if (!BF && P.stats.cur) {
    lo = wave_min(lo);
    hi = wave_max(hi);
    if (lane == 0) stats_fold(P.stats, blockIdx.x * 8 + wave, b, lo, hi);
  }
}

bool attention_prefill_supported(int NH, int NKV) {
  return NKV >= 1 && NH % NKV == 0 && NH / NKV <= a2::GMAX;
}

// A launch of few workgroups (a single prompt) also deals the query heads
// of a KV head over two workgroups of half the waves, so that a wave has a
// SIMD's matrix core to itself.
static int head_split(int B, int S, int NH, int NKV) {
  return B * NKV * ((S + a2::QT - 1) / a2::QT) < 128 && (NH / NKV) % 2 == 0 ? 2 : 1;
}

int attention_prefill_split(int B, int S, int NH, int NKV, int T, int pmax) {
  const int nwg = B * NKV * ((S + a2::QT - 1) / a2::QT) * head_split(B, S, NH, NKV);
  if (S < 2 || nwg >= 128) return 1;
  const int nch = (std::min(pmax + S, T) - 1) / a2::KC + 1;  // chunks of the last tile
  return std::max(1, std::min(std::min((512 + nwg - 1) / nwg, 8), nch));
}

static int max_pos(int B, const PosArgs& pos) {
  int m = 0;
  for (int b = 0; b < B; ++b) m = std::max(m, pos.p[b]);
  return m;
}

hipError_t launch_attention_prefill(hipStream_t st, int B, int S, int NH, int NKV, int T,
                                    const float* q, const float* k_cache, const float* v_cache,
                                    const float* k_delta, const float* v_delta,
                                    const PosArgs& pos, float* out, const SeqStats* stats,
                                    void* part) {
  // one-time attribute set-up (a function-local static: initialised once,
  // thread-safe)
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)k_attn_prefill<false>, hipFuncAttributeMaxDynamicSharedMemorySize, a2::LDS_BYTES);
  if (attr != hipSuccess) return attr;
  Attn2Params P = {};
  P.B = B;
  P.S = S;
  P.NH = NH;
  P.NKV = NKV;
  P.G = NH / NKV;
  P.T = T;
  P.nqt = (S + a2::QT - 1) / a2::QT;
  P.q = q;
  P.kc = k_cache;
  P.vc = v_cache;
  P.kd = k_delta;
  P.vd = v_delta;
  P.pos = pos;
  P.out = out;
  P.nsplit = part ? attention_prefill_split(B, S, NH, NKV, T, max_pos(B, pos)) : 1;
  P.part = (double*)part;
  P.hsplit = head_split(B, S, NH, NKV);
  if (stats && P.nsplit == 1) P.stats = *stats;
  const int lds = a2::LDS_BYTES;
  hipLaunchKernelGGL(k_attn_prefill<false>, dim3(B * NKV * P.nqt * P.hsplit * P.nsplit),
                     dim3(64 * P.G / P.hsplit), lds, st, P);
  if (P.nsplit > 1) return launch_attention_merge(st, B, S, NH, P.nsplit, P.part, out, false);
  return hipGetLastError();
}

hipError_t launch_attention_prefill_bf16(hipStream_t st, const AttnBf16Params& Q, void* part) {
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)k_attn_prefill<true>, hipFuncAttributeMaxDynamicSharedMemorySize, a2::LDS_BYTES);
  if (attr != hipSuccess) return attr;
  if (Q.S < 1 || !attention_prefill_supported(Q.NH, Q.NKV)) return hipErrorInvalidValue;
  Attn2Params P = {};
  P.B = Q.B;
  P.S = Q.S;
  P.NH = Q.NH;
  P.NKV = Q.NKV;
  P.G = Q.NH / Q.NKV;
  P.T = Q.T;
  P.nqt = (Q.S + a2::QT - 1) / a2::QT;
  P.q = (const float*)Q.q;  // bf16 storage, read as such
  P.kc = (const float*)Q.kc;
  P.vc = (const float*)Q.vc;
  P.kd = (const float*)Q.kd;
  P.vd = (const float*)Q.vd;
  P.pos = Q.pos;
  P.out = (float*)Q.out;
  P.nsplit = part ? attention_prefill_split(Q.B, Q.S, Q.NH, Q.NKV, Q.T, max_pos(Q.B, Q.pos)) : 1;
  P.part = (double*)part;
  P.hsplit = head_split(Q.B, Q.S, Q.NH, Q.NKV);
  hipLaunchKernelGGL(k_attn_prefill<true>, dim3(P.B * P.NKV * P.nqt * P.hsplit * P.nsplit),
                     dim3(64 * P.G / P.hsplit), a2::LDS_BYTES, st, P);
  if (P.nsplit > 1) return launch_attention_merge(st, Q.B, Q.S, Q.NH, P.nsplit, P.part, Q.out, true);
  return hipGetLastError();
}

}  // namespace ark
