// int8 x int8 -> int32 GEMM on gfx950 matrix cores (v_mfma_i32_16x16x64_i8)
// for prefill and batched decode, with the dequantising epilogues of the
// decoder: store (+bias), residual add, and SwiGLU over paired gate/up tiles.
//
// Operands: A = activation codes shifted to signed int8 (code - 128), [M][K];
// B = weight codes [N][K] (K contiguous for both).  Tiles of BM x BN x 64 are
// staged through LDS (rows padded to 80 bytes: conflict-free 16-byte reads).
// Each wavefront owns an (FM*16) x (FN*16) block of 16x16 accumulators.
//
// Fragment layout: lane l supplies row (l % 16) of its A fragment and row
// (l % 16) of its B fragment, both with the 16 K-bytes [16*(l/16), +16) of
// the 64-wide K step.  Because A and B use the same lane->K assignment, the
// product is sum_k A[i][k] * B[j][k] whatever order the instruction walks K.
// The 16x16 result sits in lane (j + 16*(i/4)), register i % 4.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace ark {

struct GemmParams {
  int M, K;
  const int8_t* A;
  const float* qs;
  const int* qz;
  int rows_per_seq;
  Seg seg[3];
  int seg_start[4];
  int nseg;
  int ncols;  // concatenated output columns (gate columns for SWIGLU)
  int epi;
  int32_t* acc_out;  // optional [M][ncols]
};

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(256) void k_gemm(GemmParams P) {
  constexpr int BK = 64, LW = BK + 16;
  constexpr int FM = BM / (16 * WM), FN = BN / (16 * WN);
  constexpr int ACH = BM * 4, BCH = BN * 4;  // 16-byte chunks per tile
  constexpr int AP = (ACH + 255) / 256, BP = (BCH + 255) / 256;
  __shared__ __align__(16) int8_t As[BM * LW];
  __shared__ __align__(16) int8_t Bs[BN * LW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const bool swiglu = P.epi == EPI_SWIGLU;
  const int m0 = blockIdx.y * BM;
  const int nb = blockIdx.x * (swiglu ? BN / 2 : BN);
  const int K = P.K;

  // Global sources of this thread's A and B chunks (nullptr: zero fill).
  const int8_t* asrc[AP];
  int aoff[AP];
#pragma unroll
  for (int p = 0; p < AP; ++p) {
    const int c = tid + p * 256;
    asrc[p] = nullptr;
    aoff[p] = -1;
    if (c < ACH) {
      const int tr = c >> 2, q = c & 3;
      aoff[p] = tr * LW + q * 16;
      if (m0 + tr < P.M) asrc[p] = P.A + (size_t)(m0 + tr) * K + q * 16;
    }
  }
  const int8_t* bsrc[BP];
  int boff[BP];
#pragma unroll
  for (int p = 0; p < BP; ++p) {
    const int c = tid + p * 256;
    bsrc[p] = nullptr;
    boff[p] = -1;
    if (c < BCH) {
      const int tr = c >> 2, q = c & 3;
      boff[p] = tr * LW + q * 16;
      if (swiglu) {
        const int half = BN / 2;
        const int n = nb + (tr < half ? tr : tr - half);
        if (n < P.ncols) bsrc[p] = (tr < half ? P.seg[0].w : P.seg[1].w) + (size_t)n * K + q * 16;
      } else {
        const int n = nb + tr;
        if (n < P.ncols) {
          int s = 0;
          while (s + 1 < P.nseg && n >= P.seg_start[s + 1]) ++s;
          bsrc[p] = P.seg[s].w + (size_t)(n - P.seg_start[s]) * K + q * 16;
        }
      }
    }
  }

  i32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = i32x4{0, 0, 0, 0};

  // B-tile row of fragment fn for this lane
  int brow[FN];
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) {
    if (swiglu) {
      const int h = FN / 2;
      brow[fn] = (fn < h ? 0 : BN / 2) + wn * h * 16 + (fn % h) * 16 + (lane & 15);
    } else {
      brow[fn] = wn * FN * 16 + fn * 16 + (lane & 15);
    }
  }
  const int kq = (lane >> 4) * 16;

  for (int k0 = 0; k0 < K; k0 += BK) {
    i32x4 ra[AP], rb[BP];
#pragma unroll
    for (int p = 0; p < AP; ++p)
      ra[p] = asrc[p] ? *(const i32x4*)(asrc[p] + k0) : i32x4{0, 0, 0, 0};
#pragma unroll
    for (int p = 0; p < BP; ++p)
      rb[p] = bsrc[p] ? __builtin_nontemporal_load((const i32x4*)(bsrc[p] + k0))
                      : i32x4{0, 0, 0, 0};
    __syncthreads();
#pragma unroll
    for (int p = 0; p < AP; ++p)
      if (aoff[p] >= 0) *(i32x4*)(As + aoff[p]) = ra[p];
#pragma unroll
    for (int p = 0; p < BP; ++p)
      if (boff[p] >= 0) *(i32x4*)(Bs + boff[p]) = rb[p];
    __syncthreads();
    i32x4 fa[FM], fb[FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
      fa[fm] = *(const i32x4*)(As + (wm * FM * 16 + fm * 16 + (lane & 15)) * LW + kq);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) fb[fn] = *(const i32x4*)(Bs + brow[fn] * LW + kq);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        acc[fm][fn] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[fm], fb[fn], acc[fm][fn], 0, 0, 0);
  }

  // ---- epilogue
  const SwigluK SK = swiglu_consts();
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = m0 + wm * FM * 16 + fm * 16 + (lane >> 4) * 4 + v;
      if (row >= P.M) continue;
      const int b = row / P.rows_per_seq;
      const float s = P.qs[b];
      const int zc = 128 - P.qz[b];
      if (swiglu) {
        const Seg& G = P.seg[0];
        const Seg& U = P.seg[1];
#pragma unroll
        for (int fn = 0; fn < FN / 2; ++fn) {
          const int n = nb + wn * (FN / 2) * 16 + fn * 16 + (lane & 15);
          if (n >= P.ncols) continue;
          const int ag = acc[fm][fn][v] + zc * G.cs[n];
          const int au = acc[fm][fn + FN / 2][v] + zc * U.cs[n];
          const float g = dequant(ag, s, G.sw[n]);
          const float u = dequant(au, s, U.sw[n]);
          G.out[(size_t)row * G.ldo + n] = swiglu_f64(g, u, SK);
          if (P.acc_out) P.acc_out[(size_t)row * P.ncols + n] = ag;
        }
      } else {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const int col = nb + wn * FN * 16 + fn * 16 + (lane & 15);
          if (col >= P.ncols) continue;
          int si = 0;
          while (si + 1 < P.nseg && col >= P.seg_start[si + 1]) ++si;
          const Seg& S = P.seg[si];
          const int n = col - P.seg_start[si];
          const int at = acc[fm][fn][v] + zc * S.cs[n];
          float y = dequant(at, s, S.sw[n]);
          if (S.bias) y = y + S.bias[n];
          float* o = S.out + (size_t)row * S.ldo + n;
          if (P.epi == EPI_RESID)
            *o = *o + y;
          else
            *o = y;
          if (P.acc_out) P.acc_out[(size_t)row * P.ncols + col] = at;
        }
      }
    }
  }
}

__global__ __launch_bounds__(256) void k_swiglu(int64_t n, const float* g, const float* u,
                                                float* y) {
  const SwigluK SK = swiglu_consts();
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    y[i] = swiglu_f64(g[i], u[i], SK);
}

hipError_t launch_swiglu(hipStream_t st, int64_t n, const float* g, const float* u, float* y) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(k_swiglu, dim3((unsigned)blocks), dim3(256), 0, st, n, g, u, y);
  return hipGetLastError();
}

bool gemm_swiglu_stats(int M, int K, const void* scratch) {
  return !(scratch && gemm_skinny_supported(M, K)) && gemm_big_supported(M, K);
}

hipError_t launch_gemm(hipStream_t st, int M, int K, const int8_t* codes, const float* s,
                       const int* z, int rows_per_seq, const Seg* segs, int nseg, Epi epi,
                       int32_t* acc_out, void* scratch, bool tiled_only, const SeqStats* stats) {
  if (!tiled_only && scratch && gemm_skinny_supported(M, K))
    return launch_gemm_skinny(st, M, K, codes, s, z, rows_per_seq, segs, nseg, epi, acc_out,
                              scratch);
  GemmParams P = {};
  P.M = M;
  P.K = K;
  P.A = codes;
  P.qs = s;
  P.qz = z;
  P.rows_per_seq = rows_per_seq;
  P.nseg = nseg;
  P.epi = epi;
  P.acc_out = acc_out;
  P.seg_start[0] = 0;
  for (int i = 0; i < nseg; ++i) {
    P.seg[i] = segs[i];
    P.seg_start[i + 1] = P.seg_start[i] + segs[i].n;
  }
  P.ncols = (epi == EPI_SWIGLU) ? segs[0].n : P.seg_start[nseg];
  if (!tiled_only && gemm_big_supported(M, K))
    return launch_gemm_big(st, M, K, codes, s, z, rows_per_seq, segs, nseg, epi, acc_out, stats,
                           scratch ? (char*)scratch + gemm_skinny_ws_bytes() : nullptr);
  if (M <= 32) {
    constexpr int BM = 32, BN = 128;
    const int tn = epi == EPI_SWIGLU ? BN / 2 : BN;
    dim3 grid((P.ncols + tn - 1) / tn, (M + BM - 1) / BM);
    hipLaunchKernelGGL((k_gemm<BM, BN, 1, 4>), grid, dim3(256), 0, st, P);
  } else {
    constexpr int BM = 128, BN = 128;
    const int tn = epi == EPI_SWIGLU ? BN / 2 : BN;
    dim3 grid((P.ncols + tn - 1) / tn, (M + BM - 1) / BM);
    hipLaunchKernelGGL((k_gemm<BM, BN, 2, 2>), grid, dim3(256), 0, st, P);
  }
  return hipGetLastError();
}

}  // namespace ark
