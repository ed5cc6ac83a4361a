// Row-parallel RMSNorm and per-sequence dynamic quantisation (prefill and
// batched paths).  The decode GEMV fuses the same arithmetic into its
// prologue; both use the helpers of common.hpp so the results agree.
#include <float.h>

#include "common.hpp"
#include "kernels.hpp"

namespace ark {

// Qwen2 RMSNorm (cookbook "ARK-ASR-3B" introduction: dense Qwen2 decoder):
// h = x / sqrt(mean(x^2) + eps) * g, fp64 inside, fp32 out; also the row's
// min and max of h for the quantiser.  One workgroup per row.
__global__ __launch_bounds__(256) void k_rmsnorm_rows(int H, const float* __restrict__ x, int ldx,
                                                      const float* __restrict__ g, double eps,
                                                      float* __restrict__ h,
                                                      float* __restrict__ rmin,
                                                      float* __restrict__ rmax) {
  __shared__ double redd[4];
  __shared__ float redf[8];
  const int r = blockIdx.x;
  const float* xr = x + (size_t)r * ldx;
  double ss = 0.0;
  for (int i = threadIdx.x; i < H; i += 256) {
    const double v = xr[i];
    ss += v * v;
  }
  ss = block_sum<256>(ss, redd);
  const double rs = 1.0 / sqrt(ss / (double)H + eps);
  float lo = INFINITY, hi = -INFINITY;
  float* hr = h + (size_t)r * H;
  for (int i = threadIdx.x; i < H; i += 256) {
    const float y = (float)(((double)xr[i] * rs) * (double)g[i]);
    hr[i] = y;
    lo = fminf(lo, y);
    hi = fmaxf(hi, y);
  }
  block_minmax<256>(lo, hi, redf);
  if (threadIdx.x == 0) {
    rmin[r] = lo;
    rmax[r] = hi;
  }
}

hipError_t launch_rmsnorm_rows(hipStream_t st, int R, int H, const float* x, int ldx,
                               const float* gain, double eps, float* h, float* rmin, float* rmax) {
  hipLaunchKernelGGL(k_rmsnorm_rows, dim3(R), dim3(256), 0, st, H, x, ldx, gain, eps, h, rmin,
                     rmax);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_rowminmax(int K, const float* __restrict__ x,
                                                   float* __restrict__ rmin,
                                                   float* __restrict__ rmax) {
  __shared__ float redf[8];
  const int r = blockIdx.x;
  const float* xr = x + (size_t)r * K;
  float lo = INFINITY, hi = -INFINITY;
  for (int i = threadIdx.x; i < K; i += 256) {
    const float v = xr[i];
    lo = fminf(lo, v);
    hi = fmaxf(hi, v);
  }
  block_minmax<256>(lo, hi, redf);
  if (threadIdx.x == 0) {
    rmin[r] = lo;
    rmax[r] = hi;
  }
}

hipError_t launch_rowminmax(hipStream_t st, int R, int K, const float* x, float* rmin,
                            float* rmax) {
  hipLaunchKernelGGL(k_rowminmax, dim3(R), dim3(256), 0, st, K, x, rmin, rmax);
  return hipGetLastError();
}

// Dynamic uint8 quantisation with one (s, z) per sequence (model card "Files":
// activations are quantised at run time; one scale per tensor, here per
// sequence): reduce the row min/max of the sequence, then quantise row r.
__global__ __launch_bounds__(256) void k_quant_rows(int S, int K, const float* __restrict__ x,
                                                    const float* __restrict__ rmin,
                                                    const float* __restrict__ rmax,
                                                    int8_t* __restrict__ codes,
                                                    uint8_t* __restrict__ codes_u8,
                                                    float* __restrict__ s_out,
                                                    int* __restrict__ z_out) {
  __shared__ float redf[8];
  const int r = blockIdx.x;
  const int b = r / S;
  float lo = INFINITY, hi = -INFINITY;
  for (int i = threadIdx.x; i < S; i += 256) {
    lo = fminf(lo, rmin[b * S + i]);
    hi = fmaxf(hi, rmax[b * S + i]);
  }
  block_minmax<256>(lo, hi, redf);
  const QParam p = quant_param(lo, hi);
  if (threadIdx.x == 0 && r == b * S) {
    s_out[b] = p.s;
    z_out[b] = p.z;
  }
  const float* xr = x + (size_t)r * K;
  int8_t* cr = codes ? codes + (size_t)r * K : nullptr;
  for (int i = threadIdx.x; i < K; i += 256) {
    const int c = quant_code(xr[i], p);
    if (codes) cr[i] = shift_code(c);
    if (codes_u8) codes_u8[(size_t)r * K + i] = (uint8_t)c;
  }
}

hipError_t launch_quant_rows(hipStream_t st, int B, int S, int K, const float* x,
                             const float* rmin, const float* rmax, int8_t* codes,
                             uint8_t* codes_u8, float* s_out, int* z_out) {
  hipLaunchKernelGGL(k_quant_rows, dim3(B * S), dim3(256), 0, st, S, K, x, rmin, rmax, codes,
                     codes_u8, s_out, z_out);
  return hipGetLastError();
}

// Decode form (one row per sequence, so the row is the whole tensor of its
// sequence): RMSNorm (when g != nullptr) and the dynamic quantiser in one
// pass, values kept in registers.  One workgroup of 256 threads per row;
// K <= 256 * QMAX.  Same arithmetic as k_rmsnorm_rows + k_quant_rows.
constexpr int QMAX = 48;
__global__ __launch_bounds__(256) void k_norm_quant_row(int K, const float* __restrict__ x, int ldx,
                                                        const float* __restrict__ g, double eps,
                                                        int8_t* __restrict__ codes,
                                                        float* __restrict__ s_out,
                                                        int* __restrict__ z_out) {
  __shared__ double redd[4];
  __shared__ float redf[8];
  const int r = blockIdx.x, t = threadIdx.x;
  const float* xr = x + (size_t)r * ldx;
  float v[QMAX];
#pragma unroll
  for (int k = 0; k < QMAX; ++k) v[k] = (t + 256 * k < K) ? xr[t + 256 * k] : 0.f;
  if (g) {
    double ss = 0.0;
#pragma unroll
    for (int k = 0; k < QMAX; ++k) ss += (double)v[k] * (double)v[k];
    ss = block_sum<256>(ss, redd);
    const double rs = 1.0 / sqrt(ss / (double)K + eps);
#pragma unroll
    for (int k = 0; k < QMAX; ++k)
      if (t + 256 * k < K) v[k] = (float)(((double)v[k] * rs) * (double)g[t + 256 * k]);
  }
  float lo = INFINITY, hi = -INFINITY;
#pragma unroll
  for (int k = 0; k < QMAX; ++k)
    if (t + 256 * k < K) {
      lo = fminf(lo, v[k]);
      hi = fmaxf(hi, v[k]);
    }
  block_minmax<256>(lo, hi, redf);
  const QParam p = quant_param(lo, hi);
  if (t == 0) {
    s_out[r] = p.s;
    z_out[r] = p.z;
  }
  int8_t* cr = codes + (size_t)r * K;
#pragma unroll
  for (int k = 0; k < QMAX; ++k)
    if (t + 256 * k < K) cr[t + 256 * k] = shift_code(quant_code(v[k], p));
}

bool norm_quant_row_supported(int K) { return K >= 1 && K <= 256 * QMAX; }

hipError_t launch_norm_quant_row(hipStream_t st, int B, int K, const float* x, int ldx,
                                 const float* gain, double eps, int8_t* codes, float* s_out,
                                 int* z_out) {
  hipLaunchKernelGGL(k_norm_quant_row, dim3(B), dim3(256), 0, st, K, x, ldx, gain, eps, codes,
                     s_out, z_out);
  return hipGetLastError();
}

}  // namespace ark
