// Decode-time int8 GEMV (B <= 4 input rows) for gfx950.
//
// The projection weights dominate decode traffic, so each wavefront streams
// whole weight rows with 16-byte loads (one 1 KiB contiguous segment per
// instruction) and reduces its 64 lane partials once per row.  Every
// workgroup rebuilds the quantised input vector in LDS from the fp32
// activations (RMSNorm first when a gain is given), so no separate
// quantisation kernel or grid-wide reduction precedes the GEMV; all
// workgroups run the same arithmetic and obtain identical codes.
#include <float.h>

#include "common.hpp"
#include "kernels.hpp"

namespace ark {

struct GemvParams {
  int B, K;
  const float* x;  // fp32 input rows (or nullptr: use codes/qs/qz)
  int ldx;
  const float* gain;  // RMSNorm gain, or nullptr
  double eps;
  const int8_t* codes;  // shifted codes [B][K]
  const float* qs;
  const int* qz;
  Seg seg[3];
  int seg_start[4];
  int nseg;
  int rows_total;  // output rows iterated (gate rows for SWIGLU)
  int epi;
  int32_t* acc_out;  // optional [B][rows_total] accumulators (tests)
  QDump dump;        // optional record of the prologue's quantisation (workgroup 0)
};

__device__ __forceinline__ int dot16(const i32x4 w, const i32x4 a, int acc) {
  acc = __builtin_amdgcn_sdot4(w[0], a[0], acc, false);
  acc = __builtin_amdgcn_sdot4(w[1], a[1], acc, false);
  acc = __builtin_amdgcn_sdot4(w[2], a[2], acc, false);
  acc = __builtin_amdgcn_sdot4(w[3], a[3], acc, false);
  return acc;
}

template <int BMAX, int NR, int EPI>
__global__ __launch_bounds__(256) void k_gemv(GemvParams P) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float qs_l[BMAX];
  __shared__ int qz_l[BMAX];
  __shared__ double redd[4];
  __shared__ float redf[8];
  const int B = P.B, K = P.K;
  int8_t* cl = (int8_t*)smem;                  // [BMAX][K] shifted codes
  float* hb = (float*)(smem + BMAX * K);       // [BMAX][K] normalised rows
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // ---- prologue: quantised input rows in LDS
  if (P.x) {
    for (int b = 0; b < B; ++b) {
      const float* xr = P.x + (size_t)b * P.ldx;
      float lo = INFINITY, hi = -INFINITY;
      if (P.gain) {
        double ss = 0.0;
        for (int i = tid; i < K; i += 256) {
          const double v = xr[i];
          ss += v * v;
        }
        ss = block_sum<256>(ss, redd);
        const double rs = 1.0 / sqrt(ss / (double)K + P.eps);
        for (int i = tid; i < K; i += 256) {
          const float y = (float)(((double)xr[i] * rs) * (double)P.gain[i]);
          hb[b * K + i] = y;
          lo = fminf(lo, y);
          hi = fmaxf(hi, y);
        }
      } else {
        for (int i = tid; i < K; i += 256) {
          const float v = xr[i];
          lo = fminf(lo, v);
          hi = fmaxf(hi, v);
        }
      }
      block_minmax<256>(lo, hi, redf);
      const QParam q = quant_param(lo, hi);
      if (tid == 0) {
        qs_l[b] = q.s;
        qz_l[b] = q.z;
      }
      const float* src = P.gain ? hb + b * K : xr;
      for (int i = tid; i < K; i += 256) cl[b * K + i] = shift_code(quant_code(src[i], q));
      if (P.dump.codes && blockIdx.x == 0) {
        for (int i = tid; i < K; i += 256) {
          P.dump.codes[(size_t)b * K + i] = cl[b * K + i];
          if (P.dump.h && P.gain) P.dump.h[(size_t)b * K + i] = src[i];
        }
        if (tid == 0) {
          P.dump.s[b] = q.s;
          P.dump.z[b] = q.z;
        }
      }
    }
  } else {
    const int n16 = (B * K) >> 4;
    for (int i = tid; i < n16; i += 256) ((i32x4*)cl)[i] = ((const i32x4*)P.codes)[i];
    if (tid < B) {
      qs_l[tid] = P.qs[tid];
      qz_l[tid] = P.qz[tid];
    }
  }
  __syncthreads();

  // ---- weight rows of this wave
  constexpr bool swiglu = EPI == EPI_SWIGLU;
  constexpr int NW = 2 * NR;
  const int row0 = (blockIdx.x * 4 + wave) * NR;
  const int8_t* wp[NW];
  int nw = swiglu ? 2 * NR : NR;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    int row = row0 + r;
    if (row >= P.rows_total) row = 0;  // in-bounds dummy; result discarded
    if (swiglu) {
      wp[r] = P.seg[0].w + (size_t)row * K;
      wp[NR + r] = P.seg[1].w + (size_t)row * K;
    } else {
      int s = 0;
      while (s + 1 < P.nseg && row >= P.seg_start[s + 1]) ++s;
      wp[r] = P.seg[s].w + (size_t)(row - P.seg_start[s]) * K;
      wp[NR + r] = wp[r];
    }
  }

  int acc[NW][BMAX];
#pragma unroll
  for (int r = 0; r < NW; ++r)
#pragma unroll
    for (int b = 0; b < BMAX; ++b) acc[r][b] = 0;

  const int nchunk = K >> 4;
#pragma unroll 2
  for (int c = lane; c < nchunk; c += 64) {
    i32x4 a[BMAX];
#pragma unroll
    for (int b = 0; b < BMAX; ++b)
      a[b] = (b < B) ? *(const i32x4*)(cl + b * K + c * 16) : i32x4{0, 0, 0, 0};
    i32x4 w[NW];
#pragma unroll
    for (int r = 0; r < NW; ++r) {
      w[r] = i32x4{0, 0, 0, 0};
      if (r < nw) w[r] = __builtin_nontemporal_load((const i32x4*)(wp[r] + (size_t)c * 16));
    }
#pragma unroll
    for (int r = 0; r < NW; ++r) {
      if (r < nw) {
#pragma unroll
        for (int b = 0; b < BMAX; ++b)
          if (b < B) acc[r][b] = dot16(w[r], a[b], acc[r][b]);
      }
    }
  }

#pragma unroll
  for (int r = 0; r < NW; ++r)
#pragma unroll
    for (int b = 0; b < BMAX; ++b) acc[r][b] = wave_sum(acc[r][b]);

  // ---- epilogue (lane 0 of each wave)
  if (lane != 0) return;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int row = row0 + r;
    if (row >= P.rows_total) continue;
#pragma unroll
    for (int b = 0; b < BMAX; ++b) {
      if (b >= B) continue;
      const float s = qs_l[b];
      const int zc = 128 - qz_l[b];
      if (swiglu) {
        const Seg& G = P.seg[0];
        const Seg& U = P.seg[1];
        const int ag = acc[r][b] + zc * G.cs[row];
        const int au = acc[NR + r][b] + zc * U.cs[row];
        const float g = dequant(ag, s, G.sw[row]);
        const float u = dequant(au, s, U.sw[row]);
        G.out[(size_t)b * G.ldo + row] = swiglu_f64(g, u, swiglu_consts_literal());
        if (P.acc_out) P.acc_out[(size_t)b * P.rows_total + row] = ag;
      } else {
        int si = 0;
        while (si + 1 < P.nseg && row >= P.seg_start[si + 1]) ++si;
        const Seg& S = P.seg[si];
        const int n = row - P.seg_start[si];
        const int at = acc[r][b] + zc * S.cs[n];
        float y = dequant(at, s, S.sw[n]);
        if (S.bias) y = y + S.bias[n];
        float* o = S.out + (size_t)b * S.ldo + n;
        if (EPI == EPI_RESID)
          *o = *o + y;
        else
          *o = y;
        if (P.acc_out) P.acc_out[(size_t)b * P.rows_total + row] = at;
      }
    }
  }
}

template <int BMAX, int NR>
static void launch_epi(hipStream_t st, Epi epi, int grid, size_t lds, const GemvParams& P) {
  if (epi == EPI_STORE)
    hipLaunchKernelGGL((k_gemv<BMAX, NR, EPI_STORE>), dim3(grid), dim3(256), lds, st, P);
  else if (epi == EPI_RESID)
    hipLaunchKernelGGL((k_gemv<BMAX, NR, EPI_RESID>), dim3(grid), dim3(256), lds, st, P);
  else
    hipLaunchKernelGGL((k_gemv<BMAX, NR, EPI_SWIGLU>), dim3(grid), dim3(256), lds, st, P);
}

template <int NR>
static hipError_t launch_bmax(hipStream_t st, int bmax, Epi epi, int grid, size_t lds,
                              const GemvParams& P) {
  if (bmax == 1)
    launch_epi<1, NR>(st, epi, grid, lds, P);
  else if (bmax == 2)
    launch_epi<2, NR>(st, epi, grid, lds, P);
  else
    launch_epi<4, NR>(st, epi, grid, lds, P);
  return hipGetLastError();
}

static hipError_t gemv_dispatch(hipStream_t st, GemvParams& P, const Seg* segs, int nseg, Epi epi) {
  P.nseg = nseg;
  P.epi = epi;
  P.seg_start[0] = 0;
  for (int i = 0; i < nseg; ++i) {
    P.seg[i] = segs[i];
    P.seg_start[i + 1] = P.seg_start[i] + segs[i].n;
  }
  P.rows_total = (epi == EPI_SWIGLU) ? segs[0].n : P.seg_start[nseg];
  constexpr int NR = 2;
  const int grid = (P.rows_total + 4 * NR - 1) / (4 * NR);
  const int bmax = P.B <= 1 ? 1 : (P.B <= 2 ? 2 : 4);
  const size_t lds = (size_t)bmax * P.K + ((P.x && P.gain) ? (size_t)bmax * P.K * 4 : 0);
  return launch_bmax<NR>(st, bmax, epi, grid, lds, P);
}

hipError_t launch_gemv(hipStream_t st, int B, int K, const float* x, int ldx, const float* gain,
                       double eps, const Seg* segs, int nseg, Epi epi, const QDump* qd) {
  GemvParams P = {};
  if (qd) P.dump = *qd;
  P.B = B;
  P.K = K;
  P.x = x;
  P.ldx = ldx;
  P.gain = gain;
  P.eps = eps;
  return gemv_dispatch(st, P, segs, nseg, epi);
}

hipError_t launch_gemv_codes(hipStream_t st, int B, int K, const int8_t* codes, const float* s,
                             const int* z, const Seg* segs, int nseg, Epi epi, int32_t* acc_out) {
  GemvParams P = {};
  P.B = B;
  P.K = K;
  P.codes = codes;
  P.qs = s;
  P.qz = z;
  P.acc_out = acc_out;
  return gemv_dispatch(st, P, segs, nseg, epi);
}

}  // namespace ark
