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
// query head of g (the K/V chunk is staged in LDS once for all of them).  A
// wave computes S^T = K Q^T as 16x16 blocks (A = 16 keys x 4 dims of K,
// B = 4 dims x 16 rows of Q^T, kept in registers), the online-softmax update
// per row, and O^T += V^T P^T (A = 16 dims x 4 keys of V^T, B = 4 keys x 16
// rows of P^T).  Fragment layout (16x16x4 f64): lane l supplies
// A[l % 16][l / 16] and B[l / 16][l % 16]; the 16x16 result holds
// C[4 i + l / 16][l % 16] in register i.  So the score block kb leaves
// P^T[16 kb + 4 i + l / 16][l % 16] in lane l's register i, which is the B
// operand that lane supplies for keys 4 t .. 4 t + 3 with t = 4 kb + i: the
// weights never leave the registers.
#include "common.hpp"
#include "kernels.hpp"

namespace ark {

typedef double f64x4 __attribute__((ext_vector_type(4)));

namespace a2 {
constexpr int KC = 64;    // keys per chunk
constexpr int KP = 132;   // K row pitch (floats): 16 keys x 4 dims reads hit distinct banks
constexpr int VP = 128;   // V row pitch (floats)
constexpr int QT = 16;    // query rows per workgroup
constexpr int GMAX = 8;   // query heads per KV head
constexpr int LDS_BYTES = KC * KP * 4 + KC * VP * 4;
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
};

__global__ __launch_bounds__(512) void k_attn_prefill(Attn2Params P) {
  using namespace a2;
  extern __shared__ __align__(16) unsigned char smem[];
  float* Ks = (float*)smem;                      // [KC][KP]
  float* Vs = Ks + KC * KP;                      // [KC][VP]
  if (P.stats.cur) stats_clear_other(P.stats);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nthr = blockDim.x;
  // heavy (late) query tiles first
  const int nbg = P.B * P.NKV;
  const int qt = P.nqt - 1 - (int)blockIdx.x / nbg;
  const int bg = blockIdx.x % nbg;
  const int b = bg / P.NKV, g = bg % P.NKV;
  const int i0 = qt * QT;
  const int p = P.pos.p[b];
  const int S = P.S, T = P.T;
  const int h = g * P.G + wave;
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
    const gptr<const float> src =
        uniform_ptr(P.q) + ((size_t)(b * S + min(qrow, S - 1)) * P.NH + h) * kHeadDim;
    float qf[32];
#pragma unroll
    for (int s = 0; s < 32; ++s) qf[s] = src[4 * s + q4];
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
  for (int c = 0; c < nch; ++c) {
    const int j0 = c * KC;
    __syncthreads();  // the previous chunk's K, V and P are used
    for (int e = tid; e < KC * (kHeadDim / 4); e += nthr) {
      const int jj = e >> 5, d4 = e & 31;
      const int j = j0 + jj;
      float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
      if (j < live_end) {
        size_t off;
        const float *ks, *vs;
        if (j >= p) {
          off = ((size_t)(b * S + (j - p)) * P.NKV + g) * kHeadDim;
          ks = P.kd;
          vs = P.vd;
        } else {
          off = ((size_t)(b * T + j) * P.NKV + g) * kHeadDim;
          ks = P.kc;
          vs = P.vc;
        }
        kv = ((const float4*)(ks + off))[d4];
        vv = ((const float4*)(vs + off))[d4];
      }
      *(float4*)(Ks + jj * KP + 4 * d4) = kv;
      *(float4*)(Vs + jj * VP + 4 * d4) = vv;
    }
    __syncthreads();

    // scores: sc[kb][i] = S^T[key j0 + 16 kb + 4 i + q4][qrow]
    f64x4 sc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      sc[kb] = f64x4{0.0, 0.0, 0.0, 0.0};
      const float* kr = Ks + (16 * kb + c16) * KP + q4;
#pragma unroll
      for (int s = 0; s < 32; ++s)
        sc[kb] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)kr[4 * s], qv[s], sc[kb], 0, 0, 0);
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
      const float* vr = Vs + (4 * t + q4) * VP + c16;
#pragma unroll
      for (int d = 0; d < 8; ++d)
        o[d] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)vr[16 * d], pb, o[d], 0, 0, 0);
    }
  }
  // o[d][i] = O^T[dim 16 d + 4 i + q4][qrow]
  float* dst = P.out + ((size_t)(b * S + qrow) * P.NH + h) * kHeadDim;
  float lo = INFINITY, hi = -INFINITY;
  if (rowok) {
#pragma unroll
    for (int d = 0; d < 8; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float y = (float)(o[d][i] / l);
        dst[16 * d + 4 * i + q4] = y;
        lo = fminf(lo, y);
        hi = fmaxf(hi, y);
      }
  }
  if (P.stats.cur) {
    lo = wave_min(lo);
    hi = wave_max(hi);
    if (lane == 0) stats_fold(P.stats, blockIdx.x * 8 + wave, b, lo, hi);
  }
}

bool attention_prefill_supported(int NH, int NKV) {
  return NKV >= 1 && NH % NKV == 0 && NH / NKV <= a2::GMAX;
}

hipError_t launch_attention_prefill(hipStream_t st, int B, int S, int NH, int NKV, int T,
                                    const float* q, const float* k_cache, const float* v_cache,
                                    const float* k_delta, const float* v_delta,
                                    const PosArgs& pos, float* out, const SeqStats* stats) {
  static bool attr = false;
  if (!attr) {
    const hipError_t e = hipFuncSetAttribute((const void*)k_attn_prefill,
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             a2::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr = true;
  }
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
  if (stats) P.stats = *stats;
  const int lds = a2::LDS_BYTES;
  hipLaunchKernelGGL(k_attn_prefill, dim3(B * NKV * P.nqt), dim3(64 * P.G), lds, st, P);
  return hipGetLastError();
}

}  // namespace ark
