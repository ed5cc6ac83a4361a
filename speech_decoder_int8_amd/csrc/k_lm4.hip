// Weight-only int4 LM head (the "int4 LM tier" of the model card
// "ark-asr-3b-onnx", section "Revision history").
//
// Format: codes are uint4 in blocks of 128 consecutive weights along K,
// packed two per byte (byte i of a row holds k = 2i in its low nibble and
// k = 2i + 1 in its high nibble); every block has an fp32 scale and a uint4
// zero point, packed two per byte like the codes (blocks 2j and 2j + 1).  A block is quantised like a dynamic
// activation tensor with 15 levels: range widened to include 0,
// s = (max - min) / 15, z = sat(rne(-min / s)), q = sat(rne(w / s) + z).
// The weights multiplied are w' = fp32((q - z) * s); the activations (the
// final-normed last rows) stay fp32: logits = h . w'^T, fp32 sums.
//
// At K == 2048 every lane keeps its 32 activation values of up to 4 rows
// in registers and a wave streams whole weight rows (16 bytes per lane =
// one 2048-wide row), four rows in flight; batches of more than 4 rows take
// several passes over the weights.  Other K read the activation rows from
// LDS.
#include "common.hpp"
#include "kernels.hpp"

namespace ark {

constexpr int kLm4Block = 128;
constexpr int kLm4MaxRows = 16;  // activation rows per pass

// One wave per (row, pair of blocks): 2 weights per lane and block; the
// pair's zero points share one byte.
__global__ __launch_bounds__(256) void k_prep_w4(const float* __restrict__ w, int n, int k,
                                                 uint8_t* __restrict__ codes,
                                                 float* __restrict__ scale,
                                                 uint8_t* __restrict__ zp) {
  const int lane = threadIdx.x & 63;
  const int nb = k / kLm4Block, np = nb / 2;
  const long item = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= (long)n * np) return;
  const int row = (int)(item / np), pair = (int)(item % np);
  int zz[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int blk = 2 * pair + h;
    const float2 v = *(const float2*)(w + (size_t)row * k + blk * kLm4Block + 2 * lane);
    float lo = fminf(fminf(v.x, v.y), 0.0f), hi = fmaxf(fmaxf(v.x, v.y), 0.0f);
    lo = wave_min(lo);
    hi = wave_max(hi);
    const float s = (hi - lo) / 15.0f;
    int z = 0, q0 = 0, q1 = 0;
    if (s != 0.0f) {
      z = (int)fminf(fmaxf(rintf(-lo / s), 0.0f), 15.0f);
      q0 = (int)fminf(fmaxf(rintf(v.x / s) + (float)z, 0.0f), 15.0f);
      q1 = (int)fminf(fmaxf(rintf(v.y / s) + (float)z, 0.0f), 15.0f);
    }
    codes[(size_t)row * (k / 2) + blk * (kLm4Block / 2) + lane] = (uint8_t)(q0 | (q1 << 4));
    if (lane == 0) scale[(size_t)row * nb + blk] = s;
    zz[h] = z;
  }
  if (lane == 0) zp[(size_t)row * np + pair] = (uint8_t)(zz[0] | (zz[1] << 4));
}

hipError_t launch_prep_w4(hipStream_t st, const float* w, int n, int k, uint8_t* codes,
                          float* scale, uint8_t* zp) {
  const long items = (long)n * (k / (2 * kLm4Block));
  hipLaunchKernelGGL(k_prep_w4, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, st, w, n, k,
                     codes, scale, zp);
  return hipGetLastError();
}

// The 32 weights of a 16-byte chunk (codes of k = 32 c .. 32 c + 31 of one
// row, all in block c / 4), dequantised: w'[i] = fp32((q_i - z) * s).
__device__ __forceinline__ void dequant32(const i32x4 v, float s, int z, float (&wq)[32]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t x = (uint32_t)v[j];
#pragma unroll
    for (int i = 0; i < 8; ++i) wq[8 * j + i] = (float)((int)((x >> (4 * i)) & 15u) - z) * s;
  }
}

constexpr int kLm4Rows = 4;  // weight rows a wave requests together

// Byte m of x as a float (one v_cvt_f32_ubyte<m>).
__device__ __forceinline__ float ubyte_f(uint32_t x, int m) { return (float)((x >> (8 * m)) & 0xffu); }

// K == 2048, RB activation rows (1, 2 or 4) in registers: lane l owns the
// 32-weight chunk l of every weight row (all in block l / 4); wave w of the
// grid takes weight rows w * kLm4Rows, (w + nwaves) * kLm4Rows, ...
// kLm4Rows at a time.  Per chunk the lane forms A = sum_i h_i q_i over the
// raw codes (a code is one byte-to-float conversion after two mask
// operations per 8 codes) and contributes s (A - z sum_i h_i): the same
// value as sum_i h_i (q_i - z) s in exact arithmetic, at about 2.5
// instructions per weight instead of 5, which keeps the kernel on the HBM
// stream rather than the vector ALU.  Its rounding error is bounded by
// (32 + 12) u sum_i s |h_i| (q_i + z) per logit (the entry point's
// contract).
template <int RB>
__global__ __launch_bounds__(256) void k_lm4_k2048(int N, const float* __restrict__ h, int ldh,
                                                   const uint8_t* __restrict__ w,
                                                   const float* __restrict__ sc,
                                                   const uint8_t* __restrict__ zp,
                                                   float* __restrict__ logits, int ldl) {
  constexpr int K = 2048, NB = K / kLm4Block, RB2 = K / 2;
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6), nw = gridDim.x * 4;
  float hv[RB][32], hsum[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
#pragma unroll
    for (int i = 0; i < 32; i += 4) {
      const float4 t = *(const float4*)(h + (size_t)b * ldh + 32 * lane + i);
      hv[b][i] = t.x;
      hv[b][i + 1] = t.y;
      hv[b][i + 2] = t.z;
      hv[b][i + 3] = t.w;
    }
    float t = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) t += hv[b][i];
    hsum[b] = t;
  }
  const int blk = lane / 4;
  for (int n0 = gw * kLm4Rows; n0 < N; n0 += nw * kLm4Rows) {
    i32x4 v[kLm4Rows];
    float s[kLm4Rows];
    uint32_t zb[kLm4Rows];
#pragma unroll
    for (int r = 0; r < kLm4Rows; ++r) {
      const int n = min(n0 + r, N - 1);
      v[r] = __builtin_nontemporal_load((const i32x4*)(w + (size_t)n * RB2 + 16 * lane));
      s[r] = sc[(size_t)n * NB + blk];
      zb[r] = zp[(size_t)n * (NB / 2) + blk / 2];
    }
#pragma unroll
    for (int r = 0; r < kLm4Rows; ++r) {
      float a[RB];
#pragma unroll
      for (int b = 0; b < RB; ++b) a[b] = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t x = (uint32_t)v[r][j];
        uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;
        // opaque to the compiler: knowing each byte holds 4 bits, it would
        // extract every nibble (v_bfe) before a byte-0 conversion
        asm volatile("" : "+v"(lo), "+v"(hi));
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float q0 = ubyte_f(lo, m), q1 = ubyte_f(hi, m);
#pragma unroll
          for (int b = 0; b < RB; ++b) {
            a[b] = fmaf(hv[b][8 * j + 2 * m], q0, a[b]);
            a[b] = fmaf(hv[b][8 * j + 2 * m + 1], q1, a[b]);
          }
        }
      }
      const float zf = (float)((zb[r] >> (4 * (blk & 1))) & 15u);
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        const float t = wave_sum_f32(s[r] * (a[b] - zf * hsum[b]));
        if (lane == 0 && n0 + r < N) logits[(size_t)b * ldl + n0 + r] = t;
      }
    }
  }
}

template <int RB>
hipError_t launch_k2048(hipStream_t st, int N, const float* h, int ldh, const uint8_t* w,
                        const float* sc, const uint8_t* zp, float* logits, int ldl) {
  const int grid = std::min(2048, (N + 4 * kLm4Rows - 1) / (4 * kLm4Rows));
  hipLaunchKernelGGL(k_lm4_k2048<RB>, dim3(grid), dim3(256), 0, st, N, h, ldh, w, sc, zp, logits,
                     ldl);
  return hipGetLastError();
}

// Any batch of B <= kLm4MaxRows rows and any K % 256 == 0: the rows in
// LDS, each lane a chunk of 32 weights per step along K.
__global__ __launch_bounds__(256) void k_lm4_rows(int B, int K, int N,
                                                  const float* __restrict__ h, int ldh,
                                                  const uint8_t* __restrict__ w,
                                                  const float* __restrict__ sc,
                                                  const uint8_t* __restrict__ zp,
                                                  float* __restrict__ logits, int ldl) {
  extern __shared__ __align__(16) float hs[];  // [B][K]
  for (int i = threadIdx.x; i < B * K; i += blockDim.x) hs[i] = h[(size_t)(i / K) * ldh + i % K];
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6), nw = gridDim.x * 4;
  const int NB = K / kLm4Block, RB = K / 2, NC = K / 32;
  for (int n = gw; n < N; n += nw) {
    float acc[kLm4MaxRows];
#pragma unroll
    for (int b = 0; b < kLm4MaxRows; ++b) acc[b] = 0.0f;
    for (int c = lane; c < NC; c += 64) {
      const i32x4 v = __builtin_nontemporal_load((const i32x4*)(w + (size_t)n * RB + 16 * c));
      float wq[32];
      const int blk = c / 4;
      dequant32(v, sc[(size_t)n * NB + blk], (zp[(size_t)n * (NB / 2) + blk / 2] >> (4 * (blk & 1))) & 15,
                wq);
#pragma unroll
      for (int b = 0; b < kLm4MaxRows; ++b) {
        if (b < B) {
          const float* hb = hs + b * K + 32 * c;
          float a = acc[b];
#pragma unroll
          for (int i = 0; i < 32; ++i) a = fmaf(hb[i], wq[i], a);
          acc[b] = a;
        }
      }
    }
#pragma unroll
    for (int b = 0; b < kLm4MaxRows; ++b) {
      if (b < B) {
        const float t = wave_sum_f32(acc[b]);
        if (lane == 0) logits[(size_t)b * ldl + n] = t;
      }
    }
  }
}

bool lm4_supported(int K) { return K >= 256 && K % 256 == 0 && K <= 16384; }

// Rows of h are 16-byte aligned when h is and ldh % 4 == 0.
hipError_t launch_lm4(hipStream_t st, int B, int K, int N, const float* h, int ldh,
                      const uint8_t* w, const float* sc, const uint8_t* zp, float* logits,
                      int ldl) {
  if (K == 2048 && ((uintptr_t)h % 16) == 0 && ldh % 4 == 0) {
    for (int b0 = 0; b0 < B; b0 += 4) {
      const int nb = std::min(4, B - b0);
      const float* hb = h + (size_t)b0 * ldh;
      float* lb = logits + (size_t)b0 * ldl;
      const hipError_t e = nb == 4   ? launch_k2048<4>(st, N, hb, ldh, w, sc, zp, lb, ldl)
                           : nb >= 2 ? launch_k2048<2>(st, N, hb, ldh, w, sc, zp, lb, ldl)
                                     : launch_k2048<1>(st, N, hb, ldh, w, sc, zp, lb, ldl);
      if (e != hipSuccess) return e;
      if (nb == 3) {  // the third row of a pass of 3
        const hipError_t e3 =
            launch_k2048<1>(st, N, hb + 2 * (size_t)ldh, ldh, w, sc, zp, lb + 2 * (size_t)ldl, ldl);
        if (e3 != hipSuccess) return e3;
      }
    }
    return hipSuccess;
  }
  // rows per pass: as many as fit 64 KiB of LDS, at most kLm4MaxRows
  const int per = std::max(1, std::min(kLm4MaxRows, (64 * 1024) / (K * 4)));
  for (int b0 = 0; b0 < B; b0 += per) {
    const int nb = std::min(per, B - b0);
    const size_t lds = (size_t)nb * K * 4;
    const int grid = std::min(1024, (N + 3) / 4);
    hipLaunchKernelGGL(k_lm4_rows, dim3(grid), dim3(256), lds, st, nb, K, N,
                       h + (size_t)b0 * ldh, ldh, w, sc, zp, logits + (size_t)b0 * ldl, ldl);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ark
