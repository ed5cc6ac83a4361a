// Kernels of the bf16 serving variant of the decoder (cookbook "ARK-ASR-3B",
// "dtype": bfloat16 is the default serving dtype): weights, activations and
// the KV cache in bf16, every operation rounding its output once to bf16
// (round to nearest even), fp32 logits.  Products of bf16 values are exact
// in fp32; sums run in fp32 (matrix cores) or fp64 (norms, rotary step,
// attention).
//   * k_to_bf16        fp32 -> bf16 of weights and inputs
//   * k_gemv_bf16      up to 8 activation rows: one wave per pair of weight
//                      rows, the rows of x read from cache
//   * k_gemm_bf16      more rows: v_mfma_f32_16x16x32_bf16 tiles (the byte
//                      layout of the int8 tiled GEMM: a 64-byte K step is
//                      one matrix instruction per fragment pair)
//   * k_rmsnorm_bf16, k_rope_bf16, k_embed_bf16, k_cache_write_bf16
//   * attention: the int8 path's kernels (k_attn2.hip, k_attn.hip) on bf16
//     storage
#include "common.hpp"
#include "kernels.hpp"

namespace ark {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// 8 bf16 in a 16-byte word -> floats
__device__ __forceinline__ void unpack8(const i32x4 v, float (&f)[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w = (uint32_t)v[j];
    f[2 * j] = __uint_as_float(w << 16);
    f[2 * j + 1] = __uint_as_float(w & 0xffff0000u);
  }
}

// ---- fp32 -> bf16
__global__ __launch_bounds__(256) void k_to_bf16(int64_t n, const float* __restrict__ x,
                                                 uint16_t* __restrict__ y) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    y[i] = f2bf(x[i]);
}

hipError_t launch_to_bf16(hipStream_t st, int64_t n, const float* x, uint16_t* y) {
  if (n <= 0) return hipSuccess;
  const int64_t g = std::min<int64_t>((n + 255) / 256, 16384);
  hipLaunchKernelGGL(k_to_bf16, dim3((unsigned)g), dim3(256), 0, st, n, x, y);
  return hipGetLastError();
}

// ---- few rows: one wave per RB weight rows (per RB gate + RB up rows), or
// with KW = 4 (long rows: the down projection) the four waves of a
// workgroup on the same rows, each over a quarter of K, their sums added
// in LDS in a fixed order.  A lane takes 16-byte chunks of K; U chunks of
// every row (and of the MM rows of x) are requested before any is used, so
// a wave keeps U x rows x 1 KB of weights in flight.
constexpr int kGvMaxRows = 8;
constexpr int kGvRB = 2;

template <int MM, int KW>
__global__ __launch_bounds__(256) void k_gemv_bf16(GemvBf16Params P) {
  constexpr int U = MM <= 2 ? 4 : (MM <= 4 ? 2 : 1);
  constexpr int NR = 2 * kGvRB;
  static_assert(KW == 1 || KW == 4, "waves per row group");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wv = KW == 1 ? blockIdx.x * 4 + wave : blockIdx.x;
  const bool swiglu = P.epi == BE_SWIGLU;
  const int n0 = wv * kGvRB;
  if (n0 >= P.ncols) return;
  const int K = P.K, NC = K / 8, M = P.M;
  const uint16_t* wr[NR];
#pragma unroll
  for (int r = 0; r < kGvRB; ++r) {
    const int col = min(n0 + r, P.ncols - 1);
    if (swiglu) {
      wr[r] = P.seg[0].w + (size_t)col * K;
      wr[kGvRB + r] = P.seg[1].w + (size_t)col * K;
    } else {
      int si = 0;
      while (si + 1 < P.nseg && col >= P.seg_start[si + 1]) ++si;
      wr[r] = P.seg[si].w + (size_t)(col - P.seg_start[si]) * K;
      wr[kGvRB + r] = wr[r];
    }
  }
  const int nr = swiglu ? NR : kGvRB;
  float acc[NR][MM];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int m = 0; m < MM; ++m) acc[r][m] = 0.0f;
  // this wave's chunks of K: [cb, ce)
  const int cq = KW == 1 ? NC : (NC + KW - 1) / KW;
  const int cb = KW == 1 ? 0 : min(NC, wave * cq), ce = KW == 1 ? NC : min(NC, cb + cq);
  for (int c0 = cb + lane; c0 < ce; c0 += 64 * U) {
    i32x4 wq[U][NR], xq[U][MM];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = min(c0 + 64 * u, ce - 1);
#pragma unroll
      for (int r = 0; r < NR; ++r)
        if (r < nr) wq[u][r] = __builtin_nontemporal_load((const i32x4*)(wr[r] + 8 * c));
#pragma unroll
      for (int m = 0; m < MM; ++m)
        xq[u][m] = *(const i32x4*)(P.x + (size_t)min(m, M - 1) * P.ldx + 8 * c);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c0 + 64 * u >= ce) break;
      float xf[MM][8];
#pragma unroll
      for (int m = 0; m < MM; ++m) unpack8(xq[u][m], xf[m]);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        if (r < nr) {
          float wf[8];
          unpack8(wq[u][r], wf);
#pragma unroll
          for (int m = 0; m < MM; ++m) {
            float a = acc[r][m];
#pragma unroll
            for (int i = 0; i < 8; ++i) a = fmaf(xf[m][i], wf[i], a);
            acc[r][m] = a;
          }
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int m = 0; m < MM; ++m)
      if (r < nr) acc[r][m] = wave_sum_f32(acc[r][m]);
  if constexpr (KW > 1) {
    // the K quarters' sums, added in wave order by wave 0
    __shared__ float part[KW][NR][MM];
    if (lane == 0)
#pragma unroll
      for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int m = 0; m < MM; ++m) part[wave][r][m] = acc[r][m];
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int m = 0; m < MM; ++m) {
        float a = part[0][r][m];
#pragma unroll
        for (int w = 1; w < KW; ++w) a += part[w][r][m];
        acc[r][m] = a;
      }
  }
  if (lane != 0) return;
#pragma unroll
  for (int r = 0; r < kGvRB; ++r) {
    const int col = n0 + r;
    if (col >= P.ncols) continue;
#pragma unroll
    for (int m = 0; m < MM; ++m) {
      if (m >= M) continue;
      if (swiglu) {
        ((uint16_t*)P.seg[0].out)[(size_t)m * P.seg[0].ldo + col] =
            bf_swiglu(acc[r][m], acc[kGvRB + r][m]);
      } else {
        int si = 0;
        while (si + 1 < P.nseg && col >= P.seg_start[si + 1]) ++si;
        bf_out(P.epi, P.seg[si], m, col - P.seg_start[si], acc[r][m]);
      }
    }
  }
}

// ---- more rows: matrix-core tiles (BM x BN x 32 bf16 per step)
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(256) void k_gemm_bf16(GemvBf16Params P) {
  constexpr int BKB = 64, LW = BKB + 16;  // bytes per K step, LDS row pitch
  constexpr int FM = BM / (16 * WM), FN = BN / (16 * WN);
  constexpr int ACH = BM * 4, BCH = BN * 4;
  constexpr int AP = (ACH + 255) / 256, BP = (BCH + 255) / 256;
  __shared__ __align__(16) unsigned char As[BM * LW];
  __shared__ __align__(16) unsigned char Bs[BN * LW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const bool swiglu = P.epi == BE_SWIGLU;
  const int m0 = blockIdx.y * BM;
  const int nb = blockIdx.x * (swiglu ? BN / 2 : BN);
  const size_t KB = (size_t)P.K * 2;  // bytes per row

  const unsigned char* asrc[AP];
  int aoff[AP];
#pragma unroll
  for (int p = 0; p < AP; ++p) {
    const int c = tid + p * 256;
    asrc[p] = nullptr;
    aoff[p] = -1;
    if (c < ACH) {
      const int tr = c >> 2, q = c & 3;
      aoff[p] = tr * LW + q * 16;
      if (m0 + tr < P.M) asrc[p] = (const unsigned char*)(P.x + (size_t)(m0 + tr) * P.ldx) + q * 16;
    }
  }
  const unsigned char* bsrc[BP];
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
        if (n < P.ncols)
          bsrc[p] = (const unsigned char*)((tr < half ? P.seg[0].w : P.seg[1].w)) + (size_t)n * KB + q * 16;
      } else {
        const int n = nb + tr;
        if (n < P.ncols) {
          int s = 0;
          while (s + 1 < P.nseg && n >= P.seg_start[s + 1]) ++s;
          bsrc[p] = (const unsigned char*)P.seg[s].w + (size_t)(n - P.seg_start[s]) * KB + q * 16;
        }
      }
    }
  }
  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
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
  // the next step's operands are requested before this step's products, so
  // one step of loads is always in flight behind the matrix instructions
  i32x4 ra[AP], rb[BP];
  auto load = [&](size_t k0) {
#pragma unroll
    for (int p = 0; p < AP; ++p) ra[p] = asrc[p] ? *(const i32x4*)(asrc[p] + k0) : i32x4{0, 0, 0, 0};
#pragma unroll
    for (int p = 0; p < BP; ++p)
      rb[p] = bsrc[p] ? __builtin_nontemporal_load((const i32x4*)(bsrc[p] + k0)) : i32x4{0, 0, 0, 0};
  };
  load(0);
  for (size_t k0 = 0; k0 < KB; k0 += BKB) {
    __syncthreads();
#pragma unroll
    for (int p = 0; p < AP; ++p)
      if (aoff[p] >= 0) *(i32x4*)(As + aoff[p]) = ra[p];
#pragma unroll
    for (int p = 0; p < BP; ++p)
      if (boff[p] >= 0) *(i32x4*)(Bs + boff[p]) = rb[p];
    __syncthreads();
    if (k0 + BKB < KB) load(k0 + BKB);
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
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8_t, fa[fm]), __builtin_bit_cast(bf16x8_t, fb[fn]), acc[fm][fn],
            0, 0, 0);
  }
  // C[4 (lane / 16) + v][lane % 16] of each 16x16 block
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = m0 + wm * FM * 16 + fm * 16 + (lane >> 4) * 4 + v;
      if (row >= P.M) continue;
      if (swiglu) {
#pragma unroll
        for (int fn = 0; fn < FN / 2; ++fn) {
          const int n = nb + wn * (FN / 2) * 16 + fn * 16 + (lane & 15);
          if (n >= P.ncols) continue;
          ((uint16_t*)P.seg[0].out)[(size_t)row * P.seg[0].ldo + n] =
              bf_swiglu(acc[fm][fn][v], acc[fm][fn + FN / 2][v]);
        }
      } else {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const int col = nb + wn * FN * 16 + fn * 16 + (lane & 15);
          if (col >= P.ncols) continue;
          int si = 0;
          while (si + 1 < P.nseg && col >= P.seg_start[si + 1]) ++si;
          bf_out(P.epi, P.seg[si], row, col - P.seg_start[si], acc[fm][fn][v]);
        }
      }
    }
  }
}

bool gemm_bf16_supported(int K) { return K >= 32 && K % 32 == 0; }

hipError_t launch_gemm_bf16(hipStream_t st, int M, int K, const uint16_t* x, int ldx,
                            const BSeg* segs, int nseg, int epi) {
  GemvBf16Params P = {};
  P.M = M;
  P.K = K;
  P.x = x;
  P.ldx = ldx;
  P.nseg = nseg;
  P.epi = epi;
  P.seg_start[0] = 0;
  for (int i = 0; i < nseg; ++i) {
    P.seg[i] = segs[i];
    P.seg_start[i + 1] = P.seg_start[i] + segs[i].n;
  }
  P.ncols = (epi == BE_SWIGLU) ? segs[0].n : P.seg_start[nseg];
  if (M >= 128 && ldx == K && (2 * K) % 64 == 0) return launch_gemm_big_bf16(st, M, K, x, segs, nseg, epi);
  if (M <= kGvMaxRows) {
    const int groups = (P.ncols + kGvRB - 1) / kGvRB;  // row groups of one wave
    // long rows (K >= 4096: the down projection) take a workgroup per group
    if (K >= 4096) {
      const dim3 g(groups);
      if (M == 1)
        hipLaunchKernelGGL((k_gemv_bf16<1, 4>), g, dim3(256), 0, st, P);
      else if (M == 2)
        hipLaunchKernelGGL((k_gemv_bf16<2, 4>), g, dim3(256), 0, st, P);
      else if (M <= 4)
        hipLaunchKernelGGL((k_gemv_bf16<4, 4>), g, dim3(256), 0, st, P);
      else
        hipLaunchKernelGGL((k_gemv_bf16<8, 4>), g, dim3(256), 0, st, P);
      return hipGetLastError();
    }
    const dim3 g((groups + 3) / 4);
    if (M == 1)
      hipLaunchKernelGGL((k_gemv_bf16<1, 1>), g, dim3(256), 0, st, P);
    else if (M == 2)
      hipLaunchKernelGGL((k_gemv_bf16<2, 1>), g, dim3(256), 0, st, P);
    else if (M <= 4)
      hipLaunchKernelGGL((k_gemv_bf16<4, 1>), g, dim3(256), 0, st, P);
    else
      hipLaunchKernelGGL((k_gemv_bf16<8, 1>), g, dim3(256), 0, st, P);
  } else if (M <= 32) {
    constexpr int BM = 32, BN = 64;
    const int tn = epi == BE_SWIGLU ? BN / 2 : BN;
    hipLaunchKernelGGL((k_gemm_bf16<BM, BN, 2, 2>), dim3((P.ncols + tn - 1) / tn, (M + BM - 1) / BM),
                       dim3(256), 0, st, P);
  } else {
    constexpr int BM = 128, BN = 128;
    const int tn = epi == BE_SWIGLU ? BN / 2 : BN;
    hipLaunchKernelGGL((k_gemm_bf16<BM, BN, 2, 2>), dim3((P.ncols + tn - 1) / tn, (M + BM - 1) / BM),
                       dim3(256), 0, st, P);
  }
  return hipGetLastError();
}

// ---- RMSNorm: one workgroup per row, 16-byte loads;
// bf16(g * bf16(x / sqrt(mean(x^2) + eps)))
__global__ __launch_bounds__(256) void k_rmsnorm_bf16(int R, int H, const uint16_t* __restrict__ x,
                                                      int ldx, const uint16_t* __restrict__ g,
                                                      double eps, uint16_t* __restrict__ y) {
  __shared__ double red[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  const uint16_t* xr = x + (size_t)row * ldx;
  const int NC = H / 8;
  double s = 0.0;
  for (int c = tid; c < NC; c += 256) {
    float f[8];
    unpack8(*(const i32x4*)(xr + 8 * c), f);
#pragma unroll
    for (int i = 0; i < 8; ++i) s += (double)f[i] * (double)f[i];
  }
  s = block_sum<256>(s, red);
  const double r = 1.0 / sqrt(s / (double)H + eps);
  uint16_t* yr = y + (size_t)row * H;
  for (int c = tid; c < NC; c += 256) {
    float f[8], gf[8];
    unpack8(*(const i32x4*)(xr + 8 * c), f);
    unpack8(*(const i32x4*)(g + 8 * c), gf);
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint16_t lo = f2bf((float)((double)rbf((float)((double)f[2 * i] * r)) * (double)gf[2 * i]));
      const uint16_t hi =
          f2bf((float)((double)rbf((float)((double)f[2 * i + 1] * r)) * (double)gf[2 * i + 1]));
      o[i] = (uint32_t)lo | ((uint32_t)hi << 16);
    }
    *(i32x4*)(yr + 8 * c) = i32x4{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
  }
}

hipError_t launch_rmsnorm_bf16(hipStream_t st, int R, int H, const uint16_t* x, int ldx,
                               const uint16_t* g, double eps, uint16_t* y) {
  hipLaunchKernelGGL(k_rmsnorm_bf16, dim3(R), dim3(256), 0, st, R, H, x, ldx, g, eps, y);
  return hipGetLastError();
}

// ---- rotary step: q rotated into q_out; rotated keys and the values into
// the deltas [B][S][NKV][128]; pairs (j, j + 64), fp64, one rounding
__global__ __launch_bounds__(256) void k_rope_bf16(int B, int S, int NH, int NKV,
                                                   const uint16_t* __restrict__ qkv,
                                                   const double* __restrict__ cosT,
                                                   const double* __restrict__ sinT, PosArgs pos,
                                                   uint16_t* __restrict__ q_out,
                                                   uint16_t* __restrict__ kd,
                                                   uint16_t* __restrict__ vd) {
  constexpr int D = 128, HD = 64;
  const int Q = NH * D, KV = NKV * D, W = Q + 2 * KV;
  const int heads = NH + NKV;  // rotated heads per row
  const long n = (long)B * S * heads * HD;
  for (long e = (long)blockIdx.x * 256 + threadIdx.x; e < n; e += (long)gridDim.x * 256) {
    const int j = (int)(e % HD);
    const long rh = e / HD;
    const int hh = (int)(rh % heads);
    const int r = (int)(rh / heads);
    const int b = r / S, i = r % S;
    const int p = pos.p[b] + i;
    const double c = cosT[(size_t)p * HD + j], s = sinT[(size_t)p * HD + j];
    const uint16_t* src = qkv + (size_t)r * W + (hh < NH ? hh * D : Q + (hh - NH) * D);
    const double a = bf2f(src[j]), bb = bf2f(src[j + HD]);
    const uint16_t ra = f2bf((float)(a * c - bb * s)), rb = f2bf((float)(bb * c + a * s));
    uint16_t* dst = hh < NH ? q_out + (size_t)r * Q + hh * D
                            : kd + ((size_t)r * NKV + (hh - NH)) * D;
    dst[j] = ra;
    dst[j + HD] = rb;
    if (hh >= NH) {  // the value row of this KV head, copied once per pair slot
      const uint16_t* vs = qkv + (size_t)r * W + Q + KV + (hh - NH) * D;
      uint16_t* vdst = vd + ((size_t)r * NKV + (hh - NH)) * D;
      vdst[j] = vs[j];
      vdst[j + HD] = vs[j + HD];
    }
  }
}

hipError_t launch_rope_bf16(hipStream_t st, int B, int S, int NH, int NKV, const uint16_t* qkv,
                            const double* cosT, const double* sinT, const PosArgs& pos,
                            uint16_t* q_out, uint16_t* kd, uint16_t* vd) {
  const long n = (long)B * S * (NH + NKV) * 64;
  const int g = (int)std::min<long>((n + 255) / 256, 16384);
  hipLaunchKernelGGL(k_rope_bf16, dim3(g), dim3(256), 0, st, B, S, NH, NKV, qkv, cosT, sinT, pos,
                     q_out, kd, vd);
  return hipGetLastError();
}

// ---- attention over the bf16 cache: the int8 path's kernels on bf16
// storage (loads widen bf16 to fp32, sums in fp64, the output rounded once
// to bf16 from the fp32 value).  Prefill rows: the fp64 matrix-core kernel;
// a decode row: 32-key splits and their merge (part: the partial states).
hipError_t launch_attn_bf16(hipStream_t st, const AttnBf16Params& P, void* part) {
  if (!attn_bf16_supported(P.NH, P.NKV)) return hipErrorInvalidValue;
  if (P.S == 1) return launch_attention_dec_bf16(st, P, part);
  return launch_attention_prefill_bf16(st, P, part);
}

bool attn_bf16_supported(int NH, int NKV) {
  return NKV >= 1 && NH % NKV == 0 && NH / NKV <= 8;
}

// ---- embedding rows from the bf16 table; ids out of range give NaN rows
__global__ __launch_bounds__(256) void k_embed_bf16(int R, int H, int V, const int32_t* __restrict__ ids,
                                                    const uint16_t* __restrict__ table,
                                                    uint16_t* __restrict__ x) {
  const long n = (long)R * H;
  for (long e = (long)blockIdx.x * 256 + threadIdx.x; e < n; e += (long)gridDim.x * 256) {
    const int r = (int)(e / H), i = (int)(e % H);
    const int id = ids[r];
    x[e] = (id >= 0 && id < V) ? table[(size_t)id * H + i] : (uint16_t)0x7fc0;
  }
}

hipError_t launch_embed_bf16(hipStream_t st, int R, int H, int V, const int32_t* ids,
                             const uint16_t* table, uint16_t* x) {
  const long n = (long)R * H;
  const int g = (int)std::min<long>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(k_embed_bf16, dim3(g), dim3(256), 0, st, R, H, V, ids, table, x);
  return hipGetLastError();
}

// ---- deltas into the bf16 caches at each sequence's position
__global__ __launch_bounds__(256) void k_cache_write_bf16(CacheBf16Args A, int B, int S, int T,
                                                          int KVW, PosArgs pos,
                                                          const uint16_t* __restrict__ kd,
                                                          const uint16_t* __restrict__ vd) {
  const int l = blockIdx.y;
  const int units = KVW / 8;  // 16-byte units per row
  const long n = (long)B * S * units;
  uint16_t* kc = A.k[l];
  uint16_t* vc = A.v[l];
  const uint16_t* kdl = kd + (size_t)l * B * S * KVW;
  const uint16_t* vdl = vd + (size_t)l * B * S * KVW;
  for (long e = (long)blockIdx.x * 256 + threadIdx.x; e < n; e += (long)gridDim.x * 256) {
    const int u = (int)(e % units);
    const int r = (int)(e / units);
    const int b = r / S, i = r % S;
    const size_t dst = ((size_t)b * T + pos.p[b] + i) * KVW + 8 * u;
    const size_t src = (size_t)r * KVW + 8 * u;
    *(i32x4*)(kc + dst) = *(const i32x4*)(kdl + src);
    *(i32x4*)(vc + dst) = *(const i32x4*)(vdl + src);
  }
}

hipError_t launch_cache_write_bf16(hipStream_t st, int L, int B, int S, int T, int KVW,
                                   const PosArgs& pos, const CacheBf16Args& A, const uint16_t* kd,
                                   const uint16_t* vd) {
  const long n = (long)B * S * (KVW / 8);
  const int g = (int)std::min<long>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(k_cache_write_bf16, dim3(g, L), dim3(256), 0, st, A, B, S, T, KVW, pos, kd, vd);
  return hipGetLastError();
}

}  // namespace ark
