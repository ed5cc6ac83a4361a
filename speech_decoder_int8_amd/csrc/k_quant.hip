// Row-parallel RMSNorm statistics and per-sequence dynamic quantisation
// (prefill and batched paths).  The decode GEMV fuses the same arithmetic into its
// prologue; both use the helpers of common.hpp so the results agree.
#include <float.h>

#include "common.hpp"
#include "kernels.hpp"

namespace ark {

__global__ void k_seq_stats_init(int* set) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < kStatsSetInts) set[t] = (t % (2 * kMaxBatch)) < kMaxBatch ? kOrdPosInf : kOrdNegInf;
}

hipError_t launch_seq_stats_init(hipStream_t st, int* set) {
  hipLaunchKernelGGL(k_seq_stats_init, dim3((kStatsSetInts + 255) / 256), dim3(256), 0, st, set);
  return hipGetLastError();
}

// one wave per sequence
__global__ void k_seq_stats_read(const int* set, int n, float* flo, float* fhi) {
  const int b = blockIdx.x;
  float lo, hi;
  stats_range(set, b, lo, hi);
  if (threadIdx.x == 0) {
    flo[b] = lo;
    fhi[b] = hi;
  }
}

hipError_t launch_seq_stats_read(hipStream_t st, const int* set, int n, float* flo, float* fhi) {
  hipLaunchKernelGGL(k_seq_stats_read, dim3(n), dim3(64), 0, st, set, n, flo, fhi);
  return hipGetLastError();
}

// Row kernels.  Statistics: rows of K <= 256 * RV floats (16-byte aligned)
// take one wave each, four rows per workgroup, the row held in registers as
// float4 per lane (columns 4 * lane + 256 * c); other rows take a workgroup
// each and read the row again where they need it twice.  Quantisation: one
// wave per row when there are many rows, else a workgroup per row.
constexpr int kRowsPerBlock = 4;
constexpr int kStatsRV = 8;  // float4 per lane: rows up to 2048 floats

__device__ __forceinline__ float4 ld4(const float* p) { return *(const float4*)p; }

// Qwen2 RMSNorm (cookbook "ARK-ASR-3B" introduction: dense Qwen2 decoder):
// h = x / sqrt(mean(x^2) + eps) * g, fp64 inside, fp32 out.  Statistics
// pass: rs = 1 / sqrt(mean(x^2) + eps) per row and the sequence's min/max of
// h (or, without g, of x itself).
template <int RV>
__global__ __launch_bounds__(256) void k_row_stats(int R, int K, int rps,
                                                   const float* __restrict__ x, int ldx,
                                                   const float* __restrict__ g, double eps,
                                                   double* __restrict__ rs_out, SeqStats S) {
  stats_clear_other(S);
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (r >= R) return;
  const float* xr = x + (size_t)r * ldx;
  float lo = INFINITY, hi = -INFINITY;
  {
    float4 v[RV];
#pragma unroll
    for (int c = 0; c < RV; ++c) {
      const int i = 4 * lane + 256 * c;
      v[c] = i < K ? ld4(xr + i) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (g) {
      double ss = 0.0;
#pragma unroll
      for (int c = 0; c < RV; ++c)
        ss += (double)v[c].x * v[c].x + (double)v[c].y * v[c].y + (double)v[c].z * v[c].z +
              (double)v[c].w * v[c].w;
      ss = wave_sum(ss);
      const double rs = 1.0 / sqrt(ss / (double)K + eps);
      if (lane == 0) rs_out[r] = rs;
#pragma unroll
      for (int c = 0; c < RV; ++c) {
        const int i = 4 * lane + 256 * c;
        if (i < K) {
          const float4 gg = ld4(g + i);
          v[c].x = (float)(((double)v[c].x * rs) * (double)gg.x);
          v[c].y = (float)(((double)v[c].y * rs) * (double)gg.y);
          v[c].z = (float)(((double)v[c].z * rs) * (double)gg.z);
          v[c].w = (float)(((double)v[c].w * rs) * (double)gg.w);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < RV; ++c)
      if (4 * lane + 256 * c < K) {
        lo = fminf(lo, fminf(fminf(v[c].x, v[c].y), fminf(v[c].z, v[c].w)));
        hi = fmaxf(hi, fmaxf(fmaxf(v[c].x, v[c].y), fmaxf(v[c].z, v[c].w)));
      }
  }
  lo = wave_min(lo);
  hi = wave_max(hi);
  if (lane == 0) stats_fold(S, r, r / rps, lo, hi);
}

// workgroup per row: any K, stride and alignment (float4 accesses when VEC)
template <bool VEC>
__global__ __launch_bounds__(256) void k_row_stats_wide(int K, int rps,
                                                        const float* __restrict__ x, int ldx,
                                                        const float* __restrict__ g, double eps,
                                                        double* __restrict__ rs_out, SeqStats S) {
  __shared__ double redd[4];
  __shared__ float redf[8];
  stats_clear_other(S);
  const int r = blockIdx.x, t = threadIdx.x;
  const float* xr = x + (size_t)r * ldx;
  double rs = 1.0;
  if (g) {
    double ss = 0.0;
    if constexpr (VEC) {
      for (int i = 4 * t; i < K; i += 1024) {
        const float4 v = ld4(xr + i);
        ss += (double)v.x * v.x + (double)v.y * v.y + (double)v.z * v.z + (double)v.w * v.w;
      }
    } else {
      for (int i = t; i < K; i += 256) ss += (double)xr[i] * (double)xr[i];
    }
    ss = block_sum<256>(ss, redd);
    rs = 1.0 / sqrt(ss / (double)K + eps);
    if (t == 0) rs_out[r] = rs;
  }
  float lo = INFINITY, hi = -INFINITY;
  if constexpr (VEC) {
    for (int i = 4 * t; i < K; i += 1024) {
      float4 v = ld4(xr + i);
      if (g) {
        const float4 gg = ld4(g + i);
        v.x = (float)(((double)v.x * rs) * (double)gg.x);
        v.y = (float)(((double)v.y * rs) * (double)gg.y);
        v.z = (float)(((double)v.z * rs) * (double)gg.z);
        v.w = (float)(((double)v.w * rs) * (double)gg.w);
      }
      lo = fminf(lo, fminf(fminf(v.x, v.y), fminf(v.z, v.w)));
      hi = fmaxf(hi, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
    }
  } else {
    for (int i = t; i < K; i += 256) {
      const float y = g ? (float)(((double)xr[i] * rs) * (double)g[i]) : xr[i];
      lo = fminf(lo, y);
      hi = fmaxf(hi, y);
    }
  }
  block_minmax<256>(lo, hi, redf);
  if (t == 0) stats_fold(S, r, r / rps, lo, hi);
}

static bool vec_ok(const void* p, int K, int ld) {
  return ((uintptr_t)p % 16) == 0 && K % 4 == 0 && ld % 4 == 0;
}

hipError_t launch_row_stats(hipStream_t st, int R, int K, int rps, const float* x, int ldx,
                            const float* gain, double eps, double* rs_out, const SeqStats& S) {
  const bool vec = vec_ok(x, K, ldx) && (!gain || (uintptr_t)gain % 16 == 0);
  if (vec && K <= 256 * kStatsRV)
    hipLaunchKernelGGL((k_row_stats<kStatsRV>), dim3((R + kRowsPerBlock - 1) / kRowsPerBlock),
                       dim3(256), 0, st, R, K, rps, x, ldx, gain, eps, rs_out, S);
  else if (vec)
    hipLaunchKernelGGL((k_row_stats_wide<true>), dim3(R), dim3(256), 0, st, K, rps, x, ldx, gain,
                       eps, rs_out, S);
  else
    hipLaunchKernelGGL((k_row_stats_wide<false>), dim3(R), dim3(256), 0, st, K, rps, x, ldx, gain,
                       eps, rs_out, S);
  return hipGetLastError();
}

__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
  return (uint32_t)(a & 255) | ((uint32_t)(b & 255) << 8) | ((uint32_t)(c & 255) << 16) |
         ((uint32_t)(d & 255) << 24);
}

// Dynamic uint8 quantisation with one (s, z) per sequence (model card "Files":
// activations are quantised at run time; one scale per tensor, here per
// sequence), from the sequence's min/max; h = fp32((x * rs) * g) is
// recomputed with the statistics pass's arithmetic when rs is given.
template <bool VEC, int WPR>
__global__ __launch_bounds__(256) void k_quant_seq(int R, int K, int rps,
                                                   const float* __restrict__ x, int ldx,
                                                   const double* __restrict__ rs,
                                                   const float* __restrict__ g,
                                                   const int* __restrict__ set,
                                                   int8_t* __restrict__ codes,
                                                   uint8_t* __restrict__ codes_u8,
                                                   float* __restrict__ s_out,
                                                   int* __restrict__ z_out,
                                                   float* __restrict__ h_out) {
  constexpr int TPR = 64 * WPR;  // threads per row
  const int lt = threadIdx.x % TPR;
  const int r = blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  if (r >= R) return;
  const int b = r / rps;
  float lo, hi;
  stats_range(set, b, lo, hi);
  const QParam p = quant_param(lo, hi);
  if (lt == 0 && r == b * rps) {
    s_out[b] = p.s;
    z_out[b] = p.z;
  }
  const float* xr = x + (size_t)r * ldx;
  const double rr = rs ? rs[r] : 0.0;
  if constexpr (VEC) {
    // four float4 loads in flight per thread
    for (int i0 = 4 * lt; i0 < K; i0 += 16 * TPR) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (i0 + 4 * TPR * u < K) v[u] = ld4(xr + i0 + 4 * TPR * u);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + 4 * TPR * u;
        if (i >= K) continue;
        if (rs) {
          const float4 gg = ld4(g + i);
          v[u].x = (float)(((double)v[u].x * rr) * (double)gg.x);
          v[u].y = (float)(((double)v[u].y * rr) * (double)gg.y);
          v[u].z = (float)(((double)v[u].z * rr) * (double)gg.z);
          v[u].w = (float)(((double)v[u].w * rr) * (double)gg.w);
        }
        if (h_out) *(float4*)(h_out + (size_t)r * K + i) = v[u];
        const int c0 = quant_code(v[u].x, p), c1 = quant_code(v[u].y, p);
        const int c2 = quant_code(v[u].z, p), c3 = quant_code(v[u].w, p);
        if (codes)
          *(uint32_t*)(codes + (size_t)r * K + i) =
              pack4(shift_code(c0), shift_code(c1), shift_code(c2), shift_code(c3));
        if (codes_u8) *(uint32_t*)(codes_u8 + (size_t)r * K + i) = pack4(c0, c1, c2, c3);
      }
    }
  } else {
    for (int i = lt; i < K; i += TPR) {
      const float y = rs ? (float)(((double)xr[i] * rr) * (double)g[i]) : xr[i];
      if (h_out) h_out[(size_t)r * K + i] = y;
      const int c = quant_code(y, p);
      if (codes) codes[(size_t)r * K + i] = shift_code(c);
      if (codes_u8) codes_u8[(size_t)r * K + i] = (uint8_t)c;
    }
  }
}

hipError_t launch_quant_seq(hipStream_t st, int R, int K, int rps, const float* x, int ldx,
                            const double* rs, const float* gain, const int* set, int8_t* codes,
                            uint8_t* codes_u8, float* s_out, int* z_out, float* h_out) {
  const bool vec = vec_ok(x, K, ldx) && (!codes || (uintptr_t)codes % 4 == 0) &&
                   (!codes_u8 || (uintptr_t)codes_u8 % 4 == 0) &&
                   (!rs || (uintptr_t)gain % 16 == 0);
  // a wave per row once the rows fill the chip, else a workgroup per row
  const bool wide = R < 1024;
#define ARK_QUANT_LAUNCH(V, W)                                                                   \
  hipLaunchKernelGGL((k_quant_seq<V, W>), dim3((R * W + 3) / 4), dim3(256), 0, st, R, K, rps, x, \
                     ldx, rs, gain, set, codes, codes_u8, s_out, z_out, h_out)
  if (vec && wide)
    ARK_QUANT_LAUNCH(true, 4);
  else if (vec)
    ARK_QUANT_LAUNCH(true, 1);
  else if (wide)
    ARK_QUANT_LAUNCH(false, 4);
  else
    ARK_QUANT_LAUNCH(false, 1);
#undef ARK_QUANT_LAUNCH
  return hipGetLastError();
}

// Decode form (one row per sequence, so the row is the whole tensor of its
// sequence): RMSNorm (when g != nullptr) and the dynamic quantiser in one
// pass, values kept in registers.  One workgroup of 1024 threads per row
// (four waves per SIMD: with a few dozen rows per launch, one wave per SIMD
// would leave every latency exposed); K <= 1024 * QMAX.  The gain is
// requested together with the row.  Same arithmetic as k_row_stats +
// k_quant_seq.
constexpr int QNT = 1024, QMAX = 12;
__global__ __launch_bounds__(QNT) void k_norm_quant_row(int K, const float* __restrict__ x, int ldx,
                                                        const float* __restrict__ g, double eps,
                                                        int8_t* __restrict__ codes,
                                                        float* __restrict__ s_out,
                                                        int* __restrict__ z_out,
                                                        float* __restrict__ h_out) {
  __shared__ double redd[QNT / 64];
  __shared__ float redf[2 * (QNT / 64)];
  const int r = blockIdx.x, t = threadIdx.x;
  const float* xr = x + (size_t)r * ldx;
  const float* gp = g ? g : xr;  // without a gain these loads are not used
  float v[QMAX], gv[QMAX];
#pragma unroll
  for (int k = 0; k < QMAX; ++k) {
    const bool in = t + QNT * k < K;
    v[k] = in ? xr[t + QNT * k] : 0.f;
    gv[k] = in ? gp[t + QNT * k] : 0.f;
  }
  if (g) {
    double ss = 0.0;
#pragma unroll
    for (int k = 0; k < QMAX; ++k) ss += (double)v[k] * (double)v[k];
    ss = block_sum<QNT>(ss, redd);
    const double rs = 1.0 / sqrt(ss / (double)K + eps);
#pragma unroll
    for (int k = 0; k < QMAX; ++k)
      if (t + QNT * k < K) v[k] = (float)(((double)v[k] * rs) * (double)gv[k]);
  }
  float lo = INFINITY, hi = -INFINITY;
#pragma unroll
  for (int k = 0; k < QMAX; ++k)
    if (t + QNT * k < K) {
      lo = fminf(lo, v[k]);
      hi = fmaxf(hi, v[k]);
    }
  block_minmax<QNT>(lo, hi, redf);
  const QParam p = quant_param(lo, hi);
  if (t == 0) {
    s_out[r] = p.s;
    z_out[r] = p.z;
  }
  int8_t* cr = codes + (size_t)r * K;
#pragma unroll
  for (int k = 0; k < QMAX; ++k)
    if (t + QNT * k < K) cr[t + QNT * k] = shift_code(quant_code(v[k], p));
  if (h_out)
#pragma unroll
    for (int k = 0; k < QMAX; ++k)
      if (t + QNT * k < K) h_out[(size_t)r * K + t + QNT * k] = v[k];
}

bool norm_quant_row_supported(int K) { return K >= 1 && K <= QNT * QMAX; }

// Epilogue of a split few-row GEMM, one workgroup of 1024 threads per row
// (sequence): adds the ks int32 partial sums of every output column
// (part [ks][M][ncols], exact), dequantises as the GEMM epilogues do
// (fp32(fp32(acc + (128 - z) * colsum) * fp32(s * sw)), + bias, + the
// residual input), stores the row and, given a gain, runs RMSNorm and the
// dynamic quantiser on it in registers exactly as k_norm_quant_row does
// (same thread layout t + 1024 k, sums and reductions), so the codes are
// those a separate k_norm_quant_row launch would give.  VPT values per
// thread (ncols <= 1024 * VPT).
struct RowEpiParams {
  int M, ncols, ks, nseg, resid;
  const int32_t* part;
  const float* qs;
  const int* qz;
  Seg seg[3];
  int seg_start[4];
  RowNorm nrm;
  int has_norm;
};

template <int VPT>
__global__ __launch_bounds__(QNT) void k_row_epi(RowEpiParams P) {
  static_assert(VPT <= QMAX, "row longer than the quantiser's registers");
  __shared__ double redd[QNT / 64];
  __shared__ float redf[2 * (QNT / 64)];
  const int r = blockIdx.x, t = threadIdx.x;
  const int ncols = P.ncols;
  // every split's sums of this thread's columns requested together
  int acc[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) acc[k] = 0;
  {
    int pv[8][VPT];
#pragma unroll
    for (int sp = 0; sp < 8; ++sp)
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        const int n = t + QNT * k;
        pv[sp][k] = (sp < P.ks && n < ncols) ? P.part[((size_t)sp * P.M + r) * ncols + n] : 0;
      }
#pragma unroll
    for (int sp = 0; sp < 8; ++sp)
#pragma unroll
      for (int k = 0; k < VPT; ++k) acc[k] += pv[sp][k];
  }
  const float rs = P.qs[r];
  const int rz = 128 - P.qz[r];
  const int sb1 = P.nseg > 1 ? P.seg_start[1] : ncols, sb2 = P.nseg > 2 ? P.seg_start[2] : ncols;
  int cs[VPT];
  float sw[VPT], bv[VPT], old[VPT];
  float* dst[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int n = min(t + QNT * k, ncols - 1);
    const int si = n >= sb2 ? 2 : (n >= sb1 ? 1 : 0);
    const Seg& S = P.seg[si];
    const int nn = n - P.seg_start[si];
    cs[k] = S.cs[nn];
    sw[k] = S.sw[nn];
    bv[k] = S.bias ? S.bias[nn] : 0.f;
    dst[k] = S.out + (size_t)r * S.ldo + nn;
    old[k] = P.resid ? *dst[k] : 0.f;
  }
  float v[QMAX];
#pragma unroll
  for (int k = 0; k < QMAX; ++k) v[k] = 0.f;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int n = t + QNT * k;
    const int si = n >= sb2 ? 2 : (n >= sb1 ? 1 : 0);
    float y = dequant(acc[k] + rz * cs[k], rs, sw[k]);
    if (P.seg[si].bias) y = y + bv[k];
    if (P.resid) y = old[k] + y;
    v[k] = y;
    if (n < ncols) *dst[k] = y;
  }
  if (!P.has_norm) return;
  const RowNorm& N = P.nrm;
  const int K = ncols;
  float gv[QMAX];
#pragma unroll
  for (int k = 0; k < QMAX; ++k) gv[k] = (k < VPT && t + QNT * k < K) ? N.g[t + QNT * k] : 0.f;
#pragma unroll
  for (int k = 0; k < QMAX; ++k)
    if (!(t + QNT * k < K)) v[k] = 0.f;
  double ss = 0.0;
#pragma unroll
  for (int k = 0; k < QMAX; ++k) ss += (double)v[k] * (double)v[k];
  ss = block_sum<QNT>(ss, redd);
  const double rsn = 1.0 / sqrt(ss / (double)K + N.eps);
#pragma unroll
  for (int k = 0; k < QMAX; ++k)
    if (t + QNT * k < K) v[k] = (float)(((double)v[k] * rsn) * (double)gv[k]);
  float lo = INFINITY, hi = -INFINITY;
#pragma unroll
  for (int k = 0; k < QMAX; ++k)
    if (t + QNT * k < K) {
      lo = fminf(lo, v[k]);
      hi = fmaxf(hi, v[k]);
    }
  block_minmax<QNT>(lo, hi, redf);
  const QParam p = quant_param(lo, hi);
  if (t == 0) {
    N.s[r] = p.s;
    N.z[r] = p.z;
  }
  int8_t* cr = N.codes + (size_t)r * K;
#pragma unroll
  for (int k = 0; k < QMAX; ++k)
    if (t + QNT * k < K) cr[t + QNT * k] = shift_code(quant_code(v[k], p));
  if (N.h_out)
#pragma unroll
    for (int k = 0; k < QMAX; ++k)
      if (t + QNT * k < K) N.h_out[(size_t)r * K + t + QNT * k] = v[k];
}

bool row_epi_supported(int ncols) { return ncols >= 1 && ncols <= QNT * 4; }

hipError_t launch_row_epi(hipStream_t st, int M, int ks, const int32_t* part, const float* s,
                          const int* z, const Seg* segs, int nseg, Epi epi, const RowNorm* norm) {
  RowEpiParams P = {};
  P.M = M;
  P.ks = ks;
  P.nseg = nseg;
  P.resid = epi == EPI_RESID;
  P.part = part;
  P.qs = s;
  P.qz = z;
  P.seg_start[0] = 0;
  for (int i = 0; i < nseg; ++i) {
    P.seg[i] = segs[i];
    P.seg_start[i + 1] = P.seg_start[i] + segs[i].n;
  }
  P.ncols = P.seg_start[nseg];
  if (norm) {
    P.nrm = *norm;
    P.has_norm = 1;
  }
  if (ks < 1 || ks > 8 || nseg < 1 || nseg > 3 || epi == EPI_SWIGLU || !row_epi_supported(P.ncols))
    return hipErrorInvalidValue;
  const int vpt = (P.ncols + QNT - 1) / QNT;
  if (vpt <= 2)
    hipLaunchKernelGGL(k_row_epi<2>, dim3(M), dim3(QNT), 0, st, P);
  else if (vpt <= 3)
    hipLaunchKernelGGL(k_row_epi<3>, dim3(M), dim3(QNT), 0, st, P);
  else
    hipLaunchKernelGGL(k_row_epi<4>, dim3(M), dim3(QNT), 0, st, P);
  return hipGetLastError();
}

hipError_t launch_norm_quant_row(hipStream_t st, int B, int K, const float* x, int ldx,
                                 const float* gain, double eps, int8_t* codes, float* s_out,
                                 int* z_out, float* h_out) {
  hipLaunchKernelGGL(k_norm_quant_row, dim3(B), dim3(QNT), 0, st, K, x, ldx, gain, eps, codes,
                     s_out, z_out, h_out);
  return hipGetLastError();
}

}  // namespace ark
