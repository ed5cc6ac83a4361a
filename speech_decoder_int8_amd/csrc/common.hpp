// Internal device helpers shared by the gfx950 kernels.
//
// Exactness rules (they make GPU results reproduce the host reference
// bit for bit on the integer paths):
//   * compiled with -ffp-contract=off, so a*b+c is two rounded operations
//     unless fma() is written explicitly;
//   * fp32 '/' is the correctly rounded IEEE division (hipcc default);
//   * rintf() rounds half to even; (float)int rounds to nearest even.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ark {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef long i64x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kHeadDim = 128;

// Wave-wide reductions, result in every lane (all 64 lanes must be active).
// Within each row of 16 lanes: DPP exchanges with lane^1, lane^2 (quad
// permutes), the mirror lane of the 8-lane half and of the 16-lane row, so
// every lane holds its row's result; the four rows are then combined in the
// fixed order 0, 16, 32, 48 from lane reads.  Integer sums and min/max are
// exact; a double sum is rounded in that fixed order.
namespace dpp {
constexpr int kXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kHalfMirror = 0x141; // row_half_mirror
constexpr int kMirror = 0x140;     // row_mirror
template <int C>
__device__ __forceinline__ int mov(int v) {
  return __builtin_amdgcn_update_dpp(0, v, C, 0xF, 0xF, false);
}
template <int C>
__device__ __forceinline__ float mov(float v) {
  return __int_as_float(mov<C>(__float_as_int(v)));
}
template <int C>
__device__ __forceinline__ double mov(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = mov<C>((int)b), hi = mov<C>((int)(b >> 32));
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}
__device__ __forceinline__ int lane_read(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float lane_read(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ double lane_read(double v, int l) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)b, l), hi = __builtin_amdgcn_readlane((int)(b >> 32), l);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}
template <typename T, typename Op>
__device__ __forceinline__ T all_reduce(T v, Op op) {
  v = op(v, mov<kXor1>(v));
  v = op(v, mov<kXor2>(v));
  v = op(v, mov<kHalfMirror>(v));
  v = op(v, mov<kMirror>(v));
  return op(op(op(lane_read(v, 0), lane_read(v, 16)), lane_read(v, 32)), lane_read(v, 48));
}
}  // namespace dpp

__device__ __forceinline__ double wave_sum(double v) {
  return dpp::all_reduce(v, [](double a, double b) { return a + b; });
}
// fp32 sum over the wave (the same reduction tree wherever it is used, so
// two kernels that feed it the same lane values agree bit for bit).
__device__ __forceinline__ float wave_sum_f32(float v) {
  return dpp::all_reduce(v, [](float a, float b) { return a + b; });
}
__device__ __forceinline__ int wave_sum(int v) {
  return dpp::all_reduce(v, [](int a, int b) { return a + b; });
}
__device__ __forceinline__ float wave_min(float v) {
  return dpp::all_reduce(v, [](float a, float b) { return fminf(a, b); });
}
__device__ __forceinline__ float wave_max(float v) {
  return dpp::all_reduce(v, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ double wave_max(double v) {
  return dpp::all_reduce(v, [](double a, double b) { return fmax(a, b); });
}

// Block-wide reductions for blockDim.x == NT (multiple of 64).  `red` must
// hold NT/64 elements of the type; all threads get the result.
template <int NT>
__device__ __forceinline__ double block_sum(double v, double* red) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int i = 0; i < NT / kWave; ++i) t += red[i];
  return t;
}
template <int NT>
__device__ __forceinline__ int block_sum(int v, int* red) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int i = 0; i < NT / kWave; ++i) t += red[i];
  return t;
}
template <int NT>
__device__ __forceinline__ void block_minmax(float& lo, float& hi, float* red) {
  lo = wave_min(lo);
  hi = wave_max(hi);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  __syncthreads();
  if (l == 0) { red[2 * w] = lo; red[2 * w + 1] = hi; }
  __syncthreads();
  lo = red[0];
  hi = red[1];
#pragma unroll
  for (int i = 1; i < NT / kWave; ++i) { lo = fminf(lo, red[2 * i]); hi = fmaxf(hi, red[2 * i + 1]); }
}

// Dynamic uint8 quantisation parameters of a tensor whose min/max are lo/hi
// (range widened to include 0): s = (hi - lo) / 255, z = sat(rne(-lo / s)).
struct QParam {
  float s;
  int z;
};
__device__ __forceinline__ QParam quant_param(float lo, float hi) {
  lo = fminf(lo, 0.0f);
  hi = fmaxf(hi, 0.0f);
  QParam p;
  p.s = (hi - lo) / 255.0f;
  if (p.s == 0.0f) {
    p.z = 0;
    return p;
  }
  float zf = rintf(-lo / p.s);
  zf = fminf(fmaxf(zf, 0.0f), 255.0f);
  p.z = (int)zf;
  return p;
}
// uint8 code of x: sat(rne(x / s) + z); 0 when s == 0.
__device__ __forceinline__ int quant_code(float x, QParam p) {
  if (p.s == 0.0f) return 0;
  float q = rintf(x / p.s) + (float)p.z;
  q = fminf(fmaxf(q, 0.0f), 255.0f);
  return (int)q;
}
// The kernels keep codes shifted to signed int8 (code - 128) so the signed
// int8 dot/MFMA instructions apply; sum_k (code-z)*w is then recovered as
// sum_k (code-128)*w + (128-z)*colsum (exact in int32).
__device__ __forceinline__ int8_t shift_code(int code) { return (int8_t)(code - 128); }

// Dequantised output: fp32(fp32(acc) * fp32(s * sw)) (+ bias), no FMA.
__device__ __forceinline__ float dequant(int acc, float s, float sw) {
  const float mult = s * sw;
  return (float)acc * mult;
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  return __half2float(__ushort_as_half(h));
}

// Ordered-int encoding of floats so integer atomics give float min/max.
__device__ __forceinline__ int float_to_ordered(float f) {
  int i = __float_as_int(f);
  return i >= 0 ? i : i ^ 0x7fffffff;
}
__device__ __forceinline__ float ordered_to_float(int i) {
  return __int_as_float(i >= 0 ? i : i ^ 0x7fffffff);
}
constexpr int kOrdPosInf = 0x7f800000;         // float_to_ordered(+inf)
constexpr int kOrdNegInf = (int)0x807fffffu;  // float_to_ordered(-inf)

}  // namespace ark
