// Small kernels of the decoder step: weight preparation, rotary tables,
// embedding gather/splice, masked greedy argmax and the cache write-back.
#include <float.h>
#include <limits.h>

#include "common.hpp"
#include "kernels.hpp"

namespace ark {

// ---------------------------------------------------------------- prep --
// Per-channel symmetric int8 weights (model card "Files"): one workgroup per
// output row; scale = max|w| / 127, code = clamp(rne(w / scale), -127, 127),
// plus the row's code sum used by the shifted-activation correction.
__global__ __launch_bounds__(256) void k_prep_weight(const float* __restrict__ w, int k,
                                                      int8_t* __restrict__ codes,
                                                      float* __restrict__ scale,
                                                      int32_t* __restrict__ colsum) {
  __shared__ float redf[8];
  __shared__ int redi[4];
  const size_t n = blockIdx.x;
  const float* row = w + n * (size_t)k;
  float amax = 0.0f, dummy = 0.0f;
  for (int i = threadIdx.x; i < k; i += 256) amax = fmaxf(amax, fabsf(row[i]));
  block_minmax<256>(dummy, amax, redf);
  const float s = amax / 127.0f;
  int cs = 0;
  for (int i = threadIdx.x; i < k; i += 256) {
    int c = 0;
    if (s != 0.0f) {
      float q = rintf(row[i] / s);
      q = fminf(fmaxf(q, -127.0f), 127.0f);
      c = (int)q;
    }
    codes[n * (size_t)k + i] = (int8_t)c;
    cs += c;
  }
  cs = block_sum<256>(cs, redi);
  if (threadIdx.x == 0) {
    scale[n] = s;
    colsum[n] = cs;
  }
}

hipError_t launch_prep_weight(hipStream_t st, const float* w, int n, int k, int8_t* codes,
                              float* scale, int32_t* colsum) {
  hipLaunchKernelGGL(k_prep_weight, dim3(n), dim3(256), 0, st, w, k, codes, scale, colsum);
  return hipGetLastError();
}

// Rotary angles pos * theta^(-2j/D) in fp64.
__global__ void k_rope_table(int T, int half, int D, double theta, double* c, double* s) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= T * half) return;
  const int pos = idx / half, j = idx % half;
  const double inv = pow(theta, -(2.0 * (double)j) / (double)D);
  const double ang = (double)pos * inv;
  c[idx] = cos(ang);
  s[idx] = sin(ang);
}

hipError_t launch_rope_table(hipStream_t st, int T, int D, double theta, double* c, double* s) {
  const int n = T * (D / 2);
  hipLaunchKernelGGL(k_rope_table, dim3((n + 255) / 256), dim3(256), 0, st, T, D / 2, D, theta,
                     c, s);
  return hipGetLastError();
}

// ------------------------------------------------------------- embedding --
// out[r] = fp32(table[ids[r]]) or the audio row for slots [a0, a0 + N).  An id
// outside [0, V) yields a NaN row instead of an out-of-bounds read.
__global__ __launch_bounds__(256) void k_embed(int S, int H, int V, const int32_t* __restrict__ ids,
                                               const uint16_t* __restrict__ table,
                                               const float* __restrict__ audio, int a0, int N,
                                               float* __restrict__ out) {
  const int r = blockIdx.x;
  const int b = r / S, i = r % S;
  float* dst = out + (size_t)r * H;
  if (i >= a0 && i < a0 + N) {
    const float* src = audio + ((size_t)b * N + (i - a0)) * H;
    for (int e = threadIdx.x; e < H; e += 256) dst[e] = src[e];
    return;
  }
  const int id = ids[r];
  if (id < 0 || id >= V) {
    for (int e = threadIdx.x; e < H; e += 256) dst[e] = __int_as_float(0x7fc00000);
    return;
  }
  const uint16_t* src = table + (size_t)id * H;
  for (int e = threadIdx.x; e < H; e += 256) dst[e] = half_bits_to_float(src[e]);
}

hipError_t launch_embed(hipStream_t st, int B, int S, int H, int V, const int32_t* ids,
                        const uint16_t* table, const float* audio, int a0, int N, float* out) {
  hipLaunchKernelGGL(k_embed, dim3(B * S), dim3(256), 0, st, S, H, V, ids, table, audio, a0, N,
                     out);
  return hipGetLastError();
}

// --------------------------------------------------------- masked argmax --
// Candidate order: larger logit wins; equal logits go to the lower id; NaN and
// masked ids never win.  Deterministic two-pass reduction.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// One 1024-thread workgroup per row: the row (<= 0.6 MB) streams once.
// Where the rows are 16-byte aligned, ids are taken in groups of 4 (one
// 16-byte logit load and one 4-byte mask load), four groups per thread
// requested together (indices clamped, so no branch separates the loads);
// the comparison breaks ties by id, so the visiting order does not matter.
__global__ __launch_bounds__(1024) void k_masked_argmax(int V, const float* __restrict__ logits,
                                                        const uint8_t* __restrict__ mask,
                                                        int32_t* __restrict__ out) {
  __shared__ float sv[16];
  __shared__ int si[16];
  const int b = blockIdx.x;
  const float* row = logits + (size_t)b * V;
  float bv = -INFINITY;
  int bi = INT_MAX;
  const bool vec = (V & 3) == 0 && (((uintptr_t)logits | (uintptr_t)mask) & 15) == 0;
  if (vec) {
    const int n4 = V >> 2;
    const float4* r4 = (const float4*)row;
    const uint32_t* m4 = (const uint32_t*)mask;
    for (int g0 = threadIdx.x; g0 < n4; g0 += 4 * 1024) {
      float4 v[4];
      uint32_t mk[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int g = min(g0 + u * 1024, n4 - 1);
        v[u] = r4[g];
        mk[u] = m4[g];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int g = g0 + u * 1024;
        if (g >= n4) continue;
        const float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int i = 4 * g + c;
          if (((mk[u] >> (8 * c)) & 0xff) == 0 && !isnan(e[c]) && better(e[c], i, bv, bi)) {
            bv = e[c];
            bi = i;
          }
        }
      }
    }
  } else {
    for (int i = threadIdx.x; i < V; i += 1024) {
      const float v = row[i];
      if (mask[i] == 0 && !isnan(v) && better(v, i, bv, bi)) {
        bv = v;
        bi = i;
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float v = __shfl_xor(bv, o, 64);
    const int i = __shfl_xor(bi, o, 64);
    if (i != INT_MAX && better(v, i, bv, bi)) {
      bv = v;
      bi = i;
    }
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sv[w] = bv;
    si[w] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < 16; ++k)
      if (si[k] != INT_MAX && better(sv[k], si[k], bv, bi)) {
        bv = sv[k];
        bi = si[k];
      }
    out[b] = (bi == INT_MAX) ? -1 : bi;
  }
}

hipError_t launch_masked_argmax(hipStream_t st, int B, int V, const float* logits,
                                const uint8_t* mask, int32_t* out_ids) {
  hipLaunchKernelGGL(k_masked_argmax, dim3(B), dim3(1024), 0, st, V, logits, mask, out_ids);
  return hipGetLastError();
}

// Test helper: uint8 codes -> shifted int8 codes; per-sequence (s, z) ->
// per-row arrays (row r belongs to sequence r / R).
__global__ void k_test_codes(size_t n, int K, int R, const uint8_t* __restrict__ in,
                             int8_t* __restrict__ out, const float* __restrict__ s_in,
                             const uint8_t* __restrict__ z_in, float* __restrict__ s_row,
                             int* __restrict__ z_row) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = shift_code(in[i]);
  if (i < n && i % K == 0) {
    const size_t r = i / K;
    s_row[r] = s_in[r / R];
    z_row[r] = z_in[r / R];
  }
}

hipError_t launch_test_codes(hipStream_t st, int rows, int K, int R, const uint8_t* in,
                             int8_t* out, const float* s_in, const uint8_t* z_in, float* s_row,
                             int* z_row) {
  const size_t n = (size_t)rows * K;
  hipLaunchKernelGGL(k_test_codes, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, n, K, R,
                     in, out, s_in, z_in, s_row, z_row);
  return hipGetLastError();
}

// ---------------------------------------------------------- cache write --
// cache[l][b][p_b + i] = delta[l][b][i] for keys and values (model card
// "Shapes": the host copies the returned rows in at cache_position).
struct CacheWriteArgs {
  float* k[kMaxLayers];
  float* v[kMaxLayers];
  int32_t p[kMaxBatch];
};

__global__ __launch_bounds__(128) void k_cache_write(CacheWriteArgs A, int B, int S, int T,
                                                     int row4, const float4* __restrict__ kd,
                                                     const float4* __restrict__ vd) {
  const int idx = blockIdx.x;              // ((l * B) + b) * S + i
  const int i = idx % S;
  const int b = (idx / S) % B;
  const int l = idx / (S * B);
  const size_t dst = ((size_t)b * T + A.p[b] + i) * row4;
  const size_t src = (size_t)idx * row4;
  float4* kc = (float4*)A.k[l];
  float4* vc = (float4*)A.v[l];
  for (int e = threadIdx.x; e < row4; e += 128) {
    kc[dst + e] = kd[src + e];
    vc[dst + e] = vd[src + e];
  }
}

hipError_t launch_cache_write(hipStream_t st, int L, int B, int S, int T, int row_floats,
                              const int32_t* pos_host, float* const* k_cache,
                              float* const* v_cache, const float* k_delta, const float* v_delta) {
  CacheWriteArgs A;
  for (int l = 0; l < L; ++l) {
    A.k[l] = k_cache[l];
    A.v[l] = v_cache[l];
  }
  for (int b = 0; b < B; ++b) A.p[b] = pos_host[b];
  hipLaunchKernelGGL(k_cache_write, dim3(L * B * S), dim3(128), 0, st, A, B, S, T, row_floats / 4,
                     (const float4*)k_delta, (const float4*)v_delta);
  return hipGetLastError();
}

// ----------------------------------------------------------- greedy loop --
__global__ void k_greedy_post(int B, int32_t* tokens, int32_t* out_row, int32_t end_id,
                              int32_t* done) {
  const int b = threadIdx.x;
  if (b >= B) return;
  int t = tokens[b];
  if (done[b]) t = end_id;
  tokens[b] = t;
  out_row[b] = t;
  if (t == end_id) done[b] = 1;
}

hipError_t launch_greedy_post(hipStream_t st, int B, int32_t* tokens, int32_t* out_row,
                              int32_t end_id, int32_t* done) {
  hipLaunchKernelGGL(k_greedy_post, dim3(1), dim3(64), 0, st, B, tokens, out_row, end_id, done);
  return hipGetLastError();
}

}  // namespace ark
