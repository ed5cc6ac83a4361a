// Kernels of the Whisper-style audio encoder (model card "ark-asr-3b-onnx",
// "Inference" step 1 and "Files"; cookbook "ARK-ASR-3B" introduction: a
// Whisper-style audio tower with rotary self-attention; Audio8 article,
// "What arkasr actually is": the encoder's parameter count, which fixes the
// Whisper large structure).  The int8 projections and convolutions run on
// the library's GEMMs; this file holds the pieces around them:
//   * im2col of the width-3 convolutions (tap-major rows),
//   * LayerNorm in fp64 with the per-sequence range of its output,
//   * bidirectional rotary self-attention on fp64 matrix cores.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace ark {

typedef double f64x4_t __attribute__((ext_vector_type(4)));

// ---- im2col: one thread per 4 floats of an output row
__global__ __launch_bounds__(256) void k_im2col(int B, int T, int C, int To, int stride,
                                                const float* __restrict__ x,
                                                float* __restrict__ rows) {
  const int C4 = C / 4;
  const long n = (long)B * To * 3 * C4;
  for (long e = (long)blockIdx.x * 256 + threadIdx.x; e < n; e += (long)gridDim.x * 256) {
    const int c4 = (int)(e % C4);
    const long rest = e / C4;
    const int j = (int)(rest % 3);
    const long bt = rest / 3;
    const int t = (int)(bt % To), b = (int)(bt / To);
    const int src = t * stride - 1 + j;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (src >= 0 && src < T) v = ((const float4*)(x + ((size_t)b * T + src) * C))[c4];
    ((float4*)(rows + (size_t)bt * 3 * C + (size_t)j * C))[c4] = v;
  }
}

hipError_t launch_im2col(hipStream_t st, int B, int T, int C, int stride, const float* x,
                         float* rows) {
  const int To = (T - 1) / stride + 1;
  const long n = (long)B * To * 3 * (C / 4);
  const int grid = (int)std::min<long>(16384, (n + 255) / 256);
  hipLaunchKernelGGL(k_im2col, dim3(grid), dim3(256), 0, st, B, T, C, To, stride, x, rows);
  return hipGetLastError();
}

// ---- LayerNorm: one wave per row, four rows per workgroup.  With NPL > 0
// (D <= 64 NPL) the row is read once into registers, every load requested
// before the first sum; NPL = 0 reads it three times (any D).
template <int NPL>
__global__ __launch_bounds__(256) void k_layernorm(int R, int D, int rows_per_seq,
                                                   const float* __restrict__ x,
                                                   const float* __restrict__ g,
                                                   const float* __restrict__ bb, double eps,
                                                   float* __restrict__ y, SeqStats S) {
  const bool stats = S.cur != nullptr;
  if (stats) stats_clear_other(S);
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= R) return;
  const float* xr = x + (size_t)row * D;
  float lo = INFINITY, hi = -INFINITY;
  float* yr = y + (size_t)row * D;
  if constexpr (NPL > 0) {
    float xv[NPL];
#pragma unroll
    for (int k = 0; k < NPL; ++k) {
      const int i = lane + 64 * k;
      xv[k] = i < D ? xr[i] : 0.0f;
    }
    double s = 0.0;
#pragma unroll
    for (int k = 0; k < NPL; ++k) s += (double)xv[k];
    const double mu = wave_sum(s) / (double)D;
    double v = 0.0;
#pragma unroll
    for (int k = 0; k < NPL; ++k) {
      const double c = lane + 64 * k < D ? (double)xv[k] - mu : 0.0;
      v += c * c;
    }
    const double r = 1.0 / sqrt(wave_sum(v) / (double)D + eps);
#pragma unroll
    for (int k = 0; k < NPL; ++k) {
      const int i = lane + 64 * k;
      if (i < D) {
        const float o = (float)((((double)xv[k] - mu) * r) * (double)g[i] + (double)bb[i]);
        yr[i] = o;
        lo = fminf(lo, o);
        hi = fmaxf(hi, o);
      }
    }
  } else {
    double s = 0.0;
    for (int i = lane; i < D; i += 64) s += (double)xr[i];
    const double mu = wave_sum(s) / (double)D;
    double v = 0.0;
    for (int i = lane; i < D; i += 64) {
      const double c = (double)xr[i] - mu;
      v += c * c;
    }
    const double r = 1.0 / sqrt(wave_sum(v) / (double)D + eps);
    for (int i = lane; i < D; i += 64) {
      const float o = (float)((((double)xr[i] - mu) * r) * (double)g[i] + (double)bb[i]);
      yr[i] = o;
      lo = fminf(lo, o);
      hi = fmaxf(hi, o);
    }
  }
  if (stats) {
    lo = wave_min(lo);
    hi = wave_max(hi);
    if (lane == 0) stats_fold(S, row, row / rows_per_seq, lo, hi);
  }
}

hipError_t launch_layernorm(hipStream_t st, int R, int D, int rows_per_seq, const float* x,
                            const float* g, const float* b, double eps, float* y,
                            const SeqStats& S) {
  if (D <= 64 * 20)
    hipLaunchKernelGGL(k_layernorm<20>, dim3((R + 3) / 4), dim3(256), 0, st, R, D, rows_per_seq, x,
                       g, b, eps, y, S);
  else
    hipLaunchKernelGGL(k_layernorm<0>, dim3((R + 3) / 4), dim3(256), 0, st, R, D, rows_per_seq, x,
                       g, b, eps, y, S);
  return hipGetLastError();
}

// ---- bidirectional rotary self-attention on fp64 matrix cores
//
// One workgroup = one (clip b, head h, group of 8 query tiles of 16 rows),
// one wave per query tile; each 64-key chunk of K (rotated) and V is staged
// in LDS once for the 8 waves.  A wave forms S^T = K Q^T in 16x16 blocks
// (v_mfma_f64_16x16x4f64: lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16]; the result holds C[4 i + l / 16][l % 16] in register
// i), the online softmax per query row, and O^T += V^T P^T with P^T taken
// straight from the score registers (register i of score block kb is the B
// operand the lane supplies for keys 4 t .. 4 t + 3, t = 4 kb + i).
// Keys past the clip's F frames score -inf (no other mask: every frame sees
// every frame).  Rotary pairs are (d, d + 32); q and k are rotated in fp64
// and rounded to fp32 (the tensors the method's rotary step produces), then
// widened: the chunk is staged in LDS as fp64 once for the 8 waves, and the
// next chunk's rows are fetched into registers while the current one is
// used.
namespace ea {
constexpr int DH = 64;    // head dim
constexpr int KC = 64;    // keys per chunk
// row pitches in doubles: an 8-byte fragment read of K (16 keys x 2 dims per
// half wave) and of V (16 dims x 2 keys per half wave) touches each LDS bank
// once per half wave
constexpr int KP = 66;
constexpr int VP = 80;
constexpr int QT = 16;    // query rows per wave
constexpr int NW = 8;     // waves (query tiles) per workgroup
}  // namespace ea

struct EncAttnParams {
  int B, F, H, ngrp;
  const float* qkv;
  const double* cos;
  const double* sin;
  float* out;
  SeqStats stats;
  // nsplit > 1 (a clip of few query tiles): chunk c of the keys goes to
  // split c % nsplit, which writes its unnormalised softmax state per row
  // and head to part ([B][H][F][nsplit][2 + 64]: max, sum, weighted
  // values); k_enc_merge writes out and folds the range
  int nsplit;
  double* part;
};

constexpr int ENC_ATTN_LDS = (ea::KC * ea::KP + ea::KC * ea::VP) * 8;

__global__ __launch_bounds__(512) void k_enc_attn(EncAttnParams P) {
  using namespace ea;
  extern __shared__ __align__(16) unsigned char esm[];
  double* Ks = (double*)esm;       // [KC][KP]
  double* Vs = Ks + KC * KP;       // [KC][VP]
  if (P.stats.cur) stats_clear_other(P.stats);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ns = max(P.nsplit, 1);
  const int split = blockIdx.x % ns;
  const int grp = (blockIdx.x / ns) % P.ngrp;
  const int bh = blockIdx.x / ns / P.ngrp;
  const int b = bh / P.H, h = bh % P.H;
  const int F = P.F, W3 = 3 * P.H * DH;
  const int c16 = lane & 15, q4 = lane >> 4;
  const int qrow = (grp * NW + wave) * QT + c16;
  const bool rowok = qrow < F;
  const float* base = P.qkv + (size_t)b * F * W3;

  // this lane's query dims 4 s + q4, s = 0..15, rotated: dim d < 32 pairs
  // with d + 32, held at s + 8
  double qv[16];
  {
    const int qr = min(qrow, F - 1);
    const float* src = base + (size_t)qr * W3 + h * DH;
    float qf[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) qf[s] = src[4 * s + q4];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int d = 4 * s + q4;
      const double c = P.cos[(size_t)qr * (DH / 2) + d], sn = P.sin[(size_t)qr * (DH / 2) + d];
      const double a = qf[s], bq = qf[s + 8];
      const float ra = (float)(a * c - bq * sn), rb = (float)(bq * c + a * sn);
      qv[s] = rowok ? (double)ra : 0.0;
      qv[s + 8] = rowok ? (double)rb : 0.0;
    }
  }
  f64x4_t o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) o[d] = f64x4_t{0.0, 0.0, 0.0, 0.0};
  double m = -INFINITY, l = 0.0;
  const double scale = 0.125;  // 1 / sqrt(64), exact
  const SwigluK EK = swiglu_consts();

  const int nch = (F + KC - 1) / KC;
  // 64 keys x 8 pairs of float4 (dims 4 p .. 4 p + 3 with their partners 32
  // on): one item per thread, fetched a chunk ahead
  const int jj = tid >> 3, p4 = tid & 7;
  float4 k0, k1, va, vb;
  double cc[4], sn[4];
  auto fetch = [&](int j0) {
    const int j = min(j0 + jj, F - 1);  // rows past F are zeroed when staged
    const float* kr = base + (size_t)j * W3 + P.H * DH + h * DH;
    const float* vr = kr + P.H * DH;
    k0 = ((const float4*)kr)[p4];
    k1 = ((const float4*)kr)[p4 + 8];
    va = ((const float4*)vr)[p4];
    vb = ((const float4*)vr)[p4 + 8];
    const double* cr = P.cos + (size_t)j * (DH / 2) + 4 * p4;
    const double* sr = P.sin + (size_t)j * (DH / 2) + 4 * p4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      cc[e] = cr[e];
      sn[e] = sr[e];
    }
  };
  fetch(split * KC);
  for (int c = split; c < nch; c += ns) {
    const int j0 = c * KC;
    __syncthreads();  // the previous chunk's K and V are used
    {
      const bool live = j0 + jj < F;
      const float a[4] = {k0.x, k0.y, k0.z, k0.w}, bq[4] = {k1.x, k1.y, k1.z, k1.w};
      const float v0[4] = {va.x, va.y, va.z, va.w}, v1[4] = {vb.x, vb.y, vb.z, vb.w};
      double ka[4], kb[4], wa[4], wb[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ka[e] = live ? (double)(float)((double)a[e] * cc[e] - (double)bq[e] * sn[e]) : 0.0;
        kb[e] = live ? (double)(float)((double)bq[e] * cc[e] + (double)a[e] * sn[e]) : 0.0;
        wa[e] = live ? (double)v0[e] : 0.0;
        wb[e] = live ? (double)v1[e] : 0.0;
      }
      double* kd = Ks + jj * KP + 4 * p4;
      double* vd = Vs + jj * VP + 4 * p4;
      *(double2*)kd = double2{ka[0], ka[1]};
      *(double2*)(kd + 2) = double2{ka[2], ka[3]};
      *(double2*)(kd + 32) = double2{kb[0], kb[1]};
      *(double2*)(kd + 34) = double2{kb[2], kb[3]};
      *(double2*)vd = double2{wa[0], wa[1]};
      *(double2*)(vd + 2) = double2{wa[2], wa[3]};
      *(double2*)(vd + 32) = double2{wb[0], wb[1]};
      *(double2*)(vd + 34) = double2{wb[2], wb[3]};
    }
    if (c + ns < nch) fetch(j0 + ns * KC);
    __syncthreads();

    f64x4_t sc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      sc[kb] = f64x4_t{0.0, 0.0, 0.0, 0.0};
      const double* kr = Ks + (16 * kb + c16) * KP + q4;
#pragma unroll
      for (int s = 0; s < 16; ++s)
        sc[kb] = __builtin_amdgcn_mfma_f64_16x16x4f64(kr[4 * s], qv[s], sc[kb], 0, 0, 0);
    }
    double cmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + 16 * kb + 4 * i + q4;
        const double v = (rowok && j < F) ? sc[kb][i] * scale : -INFINITY;
        sc[kb][i] = v;
        cmax = fmax(cmax, v);
      }
    cmax = fmax(cmax, __shfl_xor(cmax, 16, kWave));
    cmax = fmax(cmax, __shfl_xor(cmax, 32, kWave));
    const double mnew = fmax(m, cmax);
    const double alpha = (m == -INFINITY) ? 0.0 : exp_nonpos_f64(m - mnew, EK);
    double lsum = 0.0;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double e = (sc[kb][i] == -INFINITY) ? 0.0 : exp_nonpos_f64(sc[kb][i] - mnew, EK);
        lsum += e;
        sc[kb][i] = e;
      }
    lsum += __shfl_xor(lsum, 16, kWave);
    lsum += __shfl_xor(lsum, 32, kWave);
    l = l * alpha + lsum;
    m = mnew;
#pragma unroll
    for (int d = 0; d < 4; ++d) o[d] *= alpha;
#pragma unroll
    for (int t = 0; t < KC / 4; ++t) {
      const double pb = sc[t >> 2][t & 3];
      const double* vr = Vs + (4 * t + q4) * VP + c16;
#pragma unroll
      for (int d = 0; d < 4; ++d)
        o[d] = __builtin_amdgcn_mfma_f64_16x16x4f64(vr[16 * d], pb, o[d], 0, 0, 0);
    }
  }
  // o[d][i] = O^T[dim 16 d + 4 i + q4][qrow]
  if (ns > 1) {
    if (rowok) {
      double* dst = P.part + ((((size_t)b * P.H + h) * F + qrow) * ns + split) * (2 + DH);
      if (q4 == 0) {
        dst[0] = m;
        dst[1] = l;
      }
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[2 + 16 * d + 4 * i + q4] = o[d][i];
    }
    return;
  }
  float lo = INFINITY, hi = -INFINITY;
  if (rowok) {
    float* dst = P.out + ((size_t)b * F + qrow) * (P.H * DH) + h * DH;
#pragma unroll
    for (int d = 0; d < 4; ++d)
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
    if (lane == 0) stats_fold(P.stats, blockIdx.x * NW + wave, b, lo, hi);
  }
}

// Merge of the split states of one (clip, head, row): one wave, a lane per
// dim; each split weighted by exp(m_s - M) with M the largest m_s (a split
// that saw no key of the row is skipped); the row's range folded into the
// clip's.
__global__ __launch_bounds__(64) void k_enc_merge(int F, int H, int ns, const double* __restrict__ part,
                                                  float* __restrict__ out, SeqStats S) {
  using namespace ea;
  if (S.cur) stats_clear_other(S);
  const int idx = blockIdx.x;  // (b H + h) F + row
  const int row = idx % F, h = (idx / F) % H, b = idx / (F * H);
  const int d = threadIdx.x;
  const double* src = part + (size_t)idx * ns * (2 + DH);
  double M = -INFINITY;
  for (int u = 0; u < ns; ++u) M = fmax(M, src[(size_t)u * (2 + DH)]);
  double L = 0.0, O = 0.0;
  for (int u = 0; u < ns; ++u) {
    const double* q = src + (size_t)u * (2 + DH);
    const double mu = q[0];
    if (mu == -INFINITY) continue;
    const double w = exp(mu - M);
    L += q[1] * w;
    O += q[2 + d] * w;
  }
  const float y = (float)(O / L);
  out[((size_t)b * F + row) * (H * DH) + h * DH + d] = y;
  if (S.cur) {
    const float lo = wave_min(y), hi = wave_max(y);
    if (d == 0) stats_fold(S, idx, b, lo, hi);
  }
}

// key-chunk splits of a launch of few workgroups (a short clip)
int enc_attention_split(int B, int F, int H) {
  const int nqt = (F + ea::QT - 1) / ea::QT;
  const int nwg = B * H * ((nqt + ea::NW - 1) / ea::NW);
  const int nch = (F + ea::KC - 1) / ea::KC;
  if (nwg >= 128) return 1;
  return std::max(1, std::min(std::min((256 + nwg - 1) / nwg, 8), nch));
}

size_t enc_attention_ws_bytes(int B, int F, int H) {
  const int ns = enc_attention_split(B, F, H);
  return ns > 1 ? (size_t)B * H * F * ns * (2 + ea::DH) * sizeof(double) : 0;
}

hipError_t launch_enc_attention(hipStream_t st, int B, int F, int H, const float* qkv,
                                const double* cos, const double* sin, float* out,
                                const SeqStats& S, void* part) {
  // one-time attribute set-up (a function-local static: initialised once,
  // thread-safe)
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)k_enc_attn, hipFuncAttributeMaxDynamicSharedMemorySize, ENC_ATTN_LDS);
  if (attr != hipSuccess) return attr;
  EncAttnParams P = {};
  P.B = B;
  P.F = F;
  P.H = H;
  const int nqt = (F + ea::QT - 1) / ea::QT;
  P.ngrp = (nqt + ea::NW - 1) / ea::NW;
  P.qkv = qkv;
  P.cos = cos;
  P.sin = sin;
  P.out = out;
  P.stats = S;
  P.nsplit = part ? enc_attention_split(B, F, H) : 1;
  P.part = (double*)part;
  if (P.nsplit > 1) P.stats.cur = nullptr;  // the merge folds the range
  hipLaunchKernelGGL(k_enc_attn, dim3(B * H * P.ngrp * P.nsplit), dim3(64 * ea::NW), ENC_ATTN_LDS, st,
                     P);
  if (P.nsplit > 1)
    hipLaunchKernelGGL(k_enc_merge, dim3(B * H * F), dim3(64), 0, st, F, H, P.nsplit, P.part, out, S);
  return hipGetLastError();
}

}  // namespace ark
