// Rotary embedding and grouped-query attention over the static cache.
//
// Model card "ark-asr-3b-onnx", section "Shapes": 16 query heads share 2 KV
// heads of dimension 128; the cache is [T, 2, 128] per sequence and layer and
// every query attends over ALL T positions, masked beyond its own position.
// Rows [p, p + S) come from this call's deltas, all other rows from the
// cache; masked rows are removed by selection (their contents, even NaN,
// never reach a result).  Scores, softmax and the weighted sum run in fp64.
//
// One workgroup serves the 8 query heads of one KV head, so each K/V chunk is
// staged in LDS once for all of them.  Decode (S = 1) splits T across
// workgroups and merges the partial softmax states in a second kernel.

#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace ark {

// ------------------------------------------------------------------ rope --
__global__ __launch_bounds__(256) void k_rope(int S, int NH, int NKV, const float* __restrict__ qkv,
                                              const double* __restrict__ cosT,
                                              const double* __restrict__ sinT, PosArgs P,
                                              float* __restrict__ q, float* __restrict__ kd,
                                              float* __restrict__ vd) {
  const int r = blockIdx.x;
  const int b = r / S, i = r % S;
  const int pos = P.p[b] + i;
  const int ld = (NH + 2 * NKV) * kHeadDim;
  const float* src = qkv + (size_t)r * ld;
  for (int t = threadIdx.x; t < (NH + NKV) * 64; t += 256) {
    const int head = t >> 6, j = t & 63;
    const float* x = src + head * kHeadDim;
    const double c = cosT[pos * 64 + j], s = sinT[pos * 64 + j];
    const double x1 = x[j], x2 = x[j + 64];
    const float o1 = (float)(x1 * c - x2 * s);
    const float o2 = (float)(x2 * c + x1 * s);
    float* dst = head < NH ? q + (size_t)r * NH * kHeadDim + head * kHeadDim
                           : kd + (size_t)r * NKV * kHeadDim + (head - NH) * kHeadDim;
    dst[j] = o1;
    dst[j + 64] = o2;
  }
  const float* vs = src + (NH + NKV) * kHeadDim;
  for (int e = threadIdx.x; e < NKV * kHeadDim; e += 256) vd[(size_t)r * NKV * kHeadDim + e] = vs[e];
}

hipError_t launch_rope(hipStream_t st, int B, int S, int NH, int NKV, const float* qkv,
                       const double* cosT, const double* sinT, const PosArgs& pos, float* q,
                       float* k_delta, float* v_delta) {
  hipLaunchKernelGGL(k_rope, dim3(B * S), dim3(256), 0, st, S, NH, NKV, qkv, cosT, sinT, pos, q,
                     k_delta, v_delta);
  return hipGetLastError();
}

// ------------------------------------------------------------- attention --
struct AttnParams {
  int B, S, NH, NKV, G, T;
  const float* q;
  const float* kc;
  const float* vc;
  const float* kd;
  const float* vd;
  PosArgs pos;
  float* out;
  int nsplit, tsplit;
  double* part;  // [B][NH][S][nsplit][2 + 128]
  RopeIn rope;   // decode with the rotary step folded in (rope.qkv != nullptr)
};

constexpr int kPart = 2 + kHeadDim;

template <int QT, int KC>
__global__ __launch_bounds__(256) void k_attn(AttnParams P) {
  constexpr int NQ = QT * 8;        // query vectors per workgroup (8 heads x QT rows)
  constexpr int TPQ = 256 / NQ;     // threads per query vector
  constexpr int KPT = KC / TPQ;     // scores per thread per chunk
  constexpr int DPT = kHeadDim / TPQ;  // output dims per thread
  static_assert(KPT >= 1 && DPT >= 1, "tile shape");
  __shared__ __align__(16) float Qs[NQ][kHeadDim];
  __shared__ __align__(16) float Ks[KC][kHeadDim];
  __shared__ __align__(16) float Vs[KC][kHeadDim];
  __shared__ double Ps[NQ][KC];

  const int tid = threadIdx.x;
  const int b = blockIdx.y / P.NKV, g = blockIdx.y % P.NKV;
  const int qtile = blockIdx.x / P.nsplit, split = blockIdx.x % P.nsplit;
  const int i0 = qtile * QT;
  const int p = P.pos.p[b];
  const int S = P.S, T = P.T, NH = P.NH, NKV = P.NKV;
  const int qv = tid / TPQ, sub = tid % TPQ;
  const int qi = qv >> 3, hh = qv & 7;
  const bool active = hh < P.G && i0 + qi < S;
  const int h = g * P.G + hh;
  const int qpos = p + i0 + qi;  // absolute position of this query row

  // stage the queries of this workgroup (every load requested before the
  // first store, so the loads overlap)
  {
    constexpr int QIT = NQ * kHeadDim / 256;
    static_assert(QIT * 256 == NQ * kHeadDim, "query staging split");
    float qvals[QIT];
#pragma unroll
    for (int k = 0; k < QIT; ++k) {
      const int e = tid + 256 * k;
      const int v = e / kHeadDim, d = e % kHeadDim;
      const int vqi = v >> 3, vhh = v & 7;
      qvals[k] = (vhh < P.G && i0 + vqi < S)
                     ? P.q[((size_t)(b * S + i0 + vqi) * NH + g * P.G + vhh) * kHeadDim + d]
                     : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < QIT; ++k) {
      const int e = tid + 256 * k;
      Qs[e / kHeadDim][e % kHeadDim] = qvals[k];
    }
  }

  const double scale = 1.0 / sqrt((double)kHeadDim);
  double m = -INFINITY, l = 0.0;
  double o[DPT];
#pragma unroll
  for (int e = 0; e < DPT; ++e) o[e] = 0.0;

  // keys past the last query row's position carry zero weight: they are
  // neither loaded nor scored (a split that starts past it leaves an empty
  // state, which the merge skips)
  const int jbeg = split * P.tsplit;
  const int jend = min(min(T, jbeg + P.tsplit), p + min(S, i0 + QT));
  for (int j0 = jbeg; j0 < jend; j0 += KC) {
    __syncthreads();
    // K/V rows j0 .. j0 + KC - 1 (cache or this call's deltas); every load
    // is requested before the first store
    constexpr int KIT = KC * (kHeadDim / 4) / 256;
    static_assert(KIT * 256 == KC * (kHeadDim / 4), "K/V staging split");
    float4 kvs[KIT], vvs[KIT];
#pragma unroll
    for (int k = 0; k < KIT; ++k) {
      const int e = tid + 256 * k;
      const int jj = e / (kHeadDim / 4), d4 = e % (kHeadDim / 4);
      const int j = j0 + jj;
      kvs[k] = make_float4(0.f, 0.f, 0.f, 0.f);
      vvs[k] = kvs[k];
      if (j < jend) {
        size_t off;
        const float *ks, *vs;
        if (j >= p && j < p + S) {
          off = ((size_t)(b * S + (j - p)) * NKV + g) * kHeadDim;
          ks = P.kd;
          vs = P.vd;
        } else {
          off = ((size_t)(b * T + j) * NKV + g) * kHeadDim;
          ks = P.kc;
          vs = P.vc;
        }
        kvs[k] = ((const float4*)(ks + off))[d4];
        vvs[k] = ((const float4*)(vs + off))[d4];
      }
    }
#pragma unroll
    for (int k = 0; k < KIT; ++k) {
      const int e = tid + 256 * k;
      const int jj = e / (kHeadDim / 4), d4 = e % (kHeadDim / 4);
      ((float4*)Ks[jj])[d4] = kvs[k];
      ((float4*)Vs[jj])[d4] = vvs[k];
    }
    __syncthreads();

    // scores of this thread's keys
    double sc[KPT];
    double cmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < KPT; ++t) {
      const int jj = sub + t * TPQ;
      const int j = j0 + jj;
      double s = -INFINITY;
      if (active && j < jend && j <= qpos) {
        // the threads of a query vector read different key rows: each walks
        // the dimensions from its own offset, so their reads of one step
        // fall on different LDS banks (rows are 512 bytes, a whole number of
        // bank rounds)
        double dot = 0.0;
#pragma unroll 8
        for (int dd = 0; dd < kHeadDim; ++dd) {
          const int d = (dd + sub) & (kHeadDim - 1);
          dot = fma((double)Qs[qv][d], (double)Ks[jj][d], dot);
        }
        s = dot * scale;
      }
      sc[t] = s;
      cmax = fmax(cmax, s);
    }
#pragma unroll
    for (int off = TPQ / 2; off > 0; off >>= 1) cmax = fmax(cmax, __shfl_xor(cmax, off, kWave));
    const double mnew = fmax(m, cmax);
    double alpha = 1.0, lsum = 0.0;
    if (mnew != -INFINITY) {
      alpha = (m == -INFINITY) ? 0.0 : exp(m - mnew);
#pragma unroll
      for (int t = 0; t < KPT; ++t) {
        const double e = (sc[t] == -INFINITY) ? 0.0 : exp(sc[t] - mnew);
        Ps[qv][sub + t * TPQ] = e;
        lsum += e;
      }
    } else {
#pragma unroll
      for (int t = 0; t < KPT; ++t) Ps[qv][sub + t * TPQ] = 0.0;
    }
#pragma unroll
    for (int off = TPQ / 2; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off, kWave);
    l = l * alpha + lsum;
    m = mnew;
    __syncthreads();

    // weighted values: a masked row's value is replaced by 0 before the
    // product (its contents never reach a result; o starts at +0, so the
    // added 0 * 0 changes nothing).  Four keys' weights and values are read
    // before the first product, with no branch between them.
    static_assert(KC % 4 == 0, "weighted-sum key groups");
#pragma unroll
    for (int e = 0; e < DPT; ++e) o[e] *= alpha;
#pragma unroll 2
    for (int jj = 0; jj < KC; jj += 4) {
      double w[4];
      float vf[4][DPT];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w[i] = Ps[qv][jj + i];
#pragma unroll
        for (int e = 0; e < DPT; ++e) vf[i][e] = Vs[jj + i][sub + e * TPQ];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < DPT; ++e) {
          const double v = (w[i] != 0.0) ? (double)vf[i][e] : 0.0;
          o[e] = fma(w[i], v, o[e]);
        }
    }
  }

  if (!active) return;
  const int row = b * S + i0 + qi;
  if (P.nsplit == 1) {
    float* dst = P.out + ((size_t)row * NH + h) * kHeadDim;
#pragma unroll
    for (int e = 0; e < DPT; ++e) dst[sub + e * TPQ] = (float)(o[e] / l);
  } else {
    double* dst = P.part + ((((size_t)b * NH + h) * S + i0 + qi) * P.nsplit + split) * kPart;
    if (sub == 0) {
      dst[0] = m;
      dst[1] = l;
    }
#pragma unroll
    for (int e = 0; e < DPT; ++e) dst[2 + sub + e * TPQ] = o[e];
  }
}

// Decode form (one query row per sequence): one workgroup per (sequence b,
// KV head g, 32-key split of the cache), 256 threads = 8 query heads x 32
// lanes.  The heads' query rows are widened to fp64 once, in LDS, and read
// as broadcasts; key rows are padded to 132 floats so that the 16-byte reads
// of 16 lanes (one key each) fall in distinct banks; in the weighted sum a
// lane owns 4 consecutive dims and reads them with one 16-byte load per key.
// Only rows at or before the position are staged (the rest of the split's
// rows are zero and carry zero weight), so no row needs selecting out.  A
// split past the position leaves an empty state, which the merge skips.
// With P.rope.qkv set, q, k and v come unrotated from the projection rows:
// the workgroup rotates its heads' q rows in LDS, and the split holding the
// position rotates this call's key row and writes the key and value deltas
// (the arithmetic of k_rope: fp64 products, rounded once to fp32).
// BF: the bf16 serving variant (q, the caches and the deltas held as bf16 and
// widened on load; the merge rounds the output to bf16; no rotary step).
namespace ad {
constexpr int DK = 32;       // keys per split
constexpr int KPITCH = 132;  // floats per staged key row
}  // namespace ad

template <bool BF>
__global__ __launch_bounds__(256) void k_attn_dec(AttnParams P) {
  using namespace ad;
  __shared__ __align__(16) double Qd[8][kHeadDim];  // reused for the weights
  __shared__ __align__(16) float Ks[DK][KPITCH];
  __shared__ __align__(16) float Vs[DK][kHeadDim];
  double(*Ps)[DK] = (double(*)[DK])&Qd[0][0];

  const int tid = threadIdx.x, hh = tid >> 5, sub = tid & 31;
  const int b = blockIdx.y / P.NKV, g = blockIdx.y % P.NKV;
  const int split = blockIdx.x;
  const int p = P.pos.p[b];
  const int NH = P.NH, NKV = P.NKV, G = P.G, T = P.T;
  const bool active = hh < G;
  const int h = g * G + hh;
  const int jbeg = split * DK;
  const int nk = min(min(T, jbeg + DK), p + 1) - jbeg;  // live keys of this split
  double* dst = P.part + ((size_t)(b * NH + h) * P.nsplit + split) * kPart;
  if (nk <= 0) {  // past the position: the empty state
    if (active && sub == 0) {
      dst[0] = -INFINITY;
      dst[1] = 0.0;
    }
    if (active)
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[2 + 4 * sub + e] = 0.0;
    return;
  }

  // stage q (8 heads x 128), the keys and the values: every load is issued,
  // with no branch or wait between them, before the first store (sources
  // are wave-uniform pointers chosen per lane with selects; rows past the
  // live keys load a live row and are zeroed afterwards)
  const bool raw = !BF && P.rope.qkv != nullptr;
  const gptr<const float> kcp = uniform_ptr(P.kc), vcp = uniform_ptr(P.vc);
  // q rows of heads g G .. and this call's k / v rows of KV head g
  const gptr<const float> qp = uniform_ptr(raw ? P.rope.qkv : P.q);
  const gptr<const float> kdp = uniform_ptr(raw ? P.rope.qkv : P.kd);
  const gptr<const float> vdp = uniform_ptr(raw ? P.rope.qkv : P.vd);
  const size_t qbase = raw ? (size_t)b * P.rope.ld + (size_t)g * G * kHeadDim
                           : ((size_t)b * NH + g * G) * kHeadDim;
  const size_t dko = raw ? (size_t)b * P.rope.ld + (size_t)(NH + g) * kHeadDim
                         : ((size_t)b * NKV + g) * kHeadDim;
  const size_t dvo = raw ? (size_t)b * P.rope.ld + (size_t)(NH + NKV + g) * kHeadDim : dko;
  float qf[4];
  float4 kv[4], vv[4];
  double rc = 0.0, rsn = 0.0;  // rotation of pair (tid & 63) at position p
  if (raw) {
    rc = uniform_ptr(P.rope.cosT)[(size_t)p * (kHeadDim / 2) + (tid & 63)];
    rsn = uniform_ptr(P.rope.sinT)[(size_t)p * (kHeadDim / 2) + (tid & 63)];
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int e = tid + 256 * k;
    const int qh = min(e >> 7, G - 1), d = e & (kHeadDim - 1);
    const size_t qo = qbase + (size_t)qh * kHeadDim + d;
    if constexpr (BF)
      qf[k] = bf2f(((gptr<const uint16_t>)qp)[qo]);
    else
      qf[k] = qp[qo];
    const int jj = e >> 5, d4 = e & 31;
    const int j = jbeg + min(jj, nk - 1);
    const bool dl = j == p;  // this call's row replaces cache row p
    const size_t off = ((size_t)(b * T + j) * NKV + g) * kHeadDim;
    kv[k] = ld4e<BF>(dl ? kdp : kcp, dl ? dko : off, d4);
    vv[k] = ld4e<BF>(dl ? vdp : vcp, dl ? dvo : off, d4);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int e = tid + 256 * k;
    if ((e >> 7) >= G) qf[k] = 0.f;
    if ((e >> 5) >= nk) {
      kv[k] = make_float4(0.f, 0.f, 0.f, 0.f);
      vv[k] = kv[k];
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int e = tid + 256 * k;
    Qd[e >> 7][e & (kHeadDim - 1)] = (double)qf[k];
    const int jj = e >> 5, d4 = e & 31;
    *(float4*)&Ks[jj][4 * d4] = kv[k];
    *(float4*)&Vs[jj][4 * d4] = vv[k];
  }
  __syncthreads();
  if (raw) {
    // rotary at position p: pair (jj, jj + 64) of each q row (two rows per
    // thread), and of this call's key row in the split that holds it
    const int jj = tid & 63;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int qh = (tid >> 6) + 4 * k;
      const double x1 = Qd[qh][jj], x2 = Qd[qh][jj + 64];
      Qd[qh][jj] = (double)(float)(x1 * rc - x2 * rsn);
      Qd[qh][jj + 64] = (double)(float)(x2 * rc + x1 * rsn);
    }
    const int r = p - jbeg;
    if (r < nk && tid < 64) {
      const double x1 = Ks[r][jj], x2 = Ks[r][jj + 64];
      const float o1 = (float)(x1 * rc - x2 * rsn), o2 = (float)(x2 * rc + x1 * rsn);
      Ks[r][jj] = o1;
      Ks[r][jj + 64] = o2;
      float* kd = P.rope.kd_out + ((size_t)b * NKV + g) * kHeadDim;
      float* vd = P.rope.vd_out + ((size_t)b * NKV + g) * kHeadDim;
      kd[jj] = o1;
      kd[jj + 64] = o2;
      vd[jj] = Vs[r][jj];
      vd[jj + 64] = Vs[r][jj + 64];
    }
    __syncthreads();
  }

  // score of key sub for head hh
  double dot = 0.0;
  {
    const float4* kr = (const float4*)&Ks[sub][0];
    const double2* qr = (const double2*)&Qd[hh][0];
#pragma unroll 8
    for (int d4 = 0; d4 < kHeadDim / 4; ++d4) {
      const float4 k4 = kr[d4];
      const double2 qa = qr[2 * d4], qb = qr[2 * d4 + 1];
      dot = fma(qa.x, (double)k4.x, dot);
      dot = fma(qa.y, (double)k4.y, dot);
      dot = fma(qb.x, (double)k4.z, dot);
      dot = fma(qb.y, (double)k4.w, dot);
    }
  }
  const double sc = sub < nk ? dot * (1.0 / sqrt((double)kHeadDim)) : -INFINITY;
  double m = sc;
#pragma unroll
  for (int off = 16; off > 0; off >>= 1) m = fmax(m, __shfl_xor(m, off, kWave));
  const double ev = sub < nk ? exp(sc - m) : 0.0;
  double l = ev;
#pragma unroll
  for (int off = 16; off > 0; off >>= 1) l += __shfl_xor(l, off, kWave);
  __syncthreads();  // every query read is done: the weights take its place
  Ps[hh][sub] = ev;
  __syncthreads();

  // weighted values of dims 4 sub .. 4 sub + 3, four keys per group (the
  // rows past nk are zero and their weights 0)
  double o[4] = {0.0, 0.0, 0.0, 0.0};
  for (int jj = 0; jj < nk; jj += 4) {
    double w[4];
    float4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w[i] = Ps[hh][jj + i];
      v[i] = *(const float4*)&Vs[jj + i][4 * sub];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[0] = fma(w[i], (double)v[i].x, o[0]);
      o[1] = fma(w[i], (double)v[i].y, o[1]);
      o[2] = fma(w[i], (double)v[i].z, o[2]);
      o[3] = fma(w[i], (double)v[i].w, o[3]);
    }
  }
  if (!active) return;
  if (sub == 0) {
    dst[0] = m;
    dst[1] = l;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) dst[2 + 4 * sub + e] = o[e];
}

// Merge the split partial softmax states of one (sequence, head, row).
// BF: out holds bf16, rounded from the fp32 value.
template <bool BF>
__global__ __launch_bounds__(128) void k_attn_combine(int S, int NH, int nsplit,
                                                      const double* __restrict__ part,
                                                      float* __restrict__ out) {
  const int idx = blockIdx.x;  // (b * NH + h) * S + i
  const int i = idx % S, h = (idx / S) % NH, b = idx / (S * NH);
  const double* src = part + (size_t)idx * nsplit * kPart;
  const int d = threadIdx.x;
  // the states of up to 16 splits are requested together before any is
  // used (one round trip for a 512-row cache); each split is weighted by
  // exp(m_s - M) with M the maximum of the m_s seen so far, and a later
  // group with a larger maximum rescales what was summed before it
  constexpr int U = 16;
  double M = -INFINITY, L = 0.0, O = 0.0;
  for (int s0 = 0; s0 < nsplit; s0 += U) {
    double ms[U], ls[U], os[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = s0 + u < nsplit;
      const double* q = src + (size_t)(ok ? s0 + u : 0) * kPart;
      ms[u] = q[0];
      ls[u] = q[1];
      os[u] = q[2 + d];
    }
    // every load is out before any value is used (not sunk into the
    // per-split branches below, each with its own wait)
#pragma unroll
    for (int u = 0; u < U; ++u) asm volatile("" : "+v"(ms[u]), "+v"(ls[u]), "+v"(os[u]));
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (s0 + u >= nsplit) ms[u] = -INFINITY;
    double Mg = M;
#pragma unroll
    for (int u = 0; u < U; ++u) Mg = fmax(Mg, ms[u]);
    if (Mg != M && M != -INFINITY) {
      const double a = exp(M - Mg);
      L *= a;
      O *= a;
    }
    M = Mg;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ms[u] == -INFINITY) continue;
      const double w = exp(ms[u] - M);
      L += ls[u] * w;
      O += os[u] * w;
    }
  }
  const size_t oi = ((size_t)(b * S + i) * NH + h) * kHeadDim + d;
  if constexpr (BF)
    ((uint16_t*)out)[oi] = f2bf((float)(O / L));
  else
    out[oi] = (float)(O / L);
}

static int decode_split(int T) { return T / 32; }
// the splits a decode launch needs: those holding a key at or before the
// largest position (later ones would only write empty states)
static int decode_split(int T, int B, const PosArgs& pos) {
  int pmax = 0;
  for (int b = 0; b < B; ++b) pmax = std::max(pmax, pos.p[b]);
  return std::min(T / 32, pmax / ad::DK + 1);
}

size_t attention_ws_bytes(int B, int S, int NH, int T) {
  if (S == 1) return (size_t)B * NH * decode_split(T) * kPart * sizeof(double);
  // prefill with its key chunks split: at most the split of one KV head
  // (more KV heads give more workgroups, so no larger split) at the last
  // position a call of S rows may start at (S <= T for any valid call)
  const int ns = attention_prefill_split(B, S, NH, 1, T, std::max(0, T - S));
  return ns > 1 ? (size_t)B * NH * S * ns * kPart * sizeof(double) : 0;
}

bool attention_stats(int B, int S, int NH, int NKV, int T, int pmax) {
  return S > 1 && attention_prefill_supported(NH, NKV) &&
         attention_prefill_split(B, S, NH, NKV, T, pmax) == 1;
}

hipError_t launch_attention_merge(hipStream_t st, int B, int S, int NH, int nsplit,
                                  const double* part, void* out, bool bf16) {
  if (bf16)
    hipLaunchKernelGGL(k_attn_combine<true>, dim3(B * NH * S), dim3(128), 0, st, S, NH, nsplit, part,
                       (float*)out);
  else
    hipLaunchKernelGGL(k_attn_combine<false>, dim3(B * NH * S), dim3(128), 0, st, S, NH, nsplit, part,
                       (float*)out);
  return hipGetLastError();
}

hipError_t launch_attention(hipStream_t st, int B, int S, int NH, int NKV, int T, const float* q,
                            const float* k_cache, const float* v_cache, const float* k_delta,
                            const float* v_delta, const PosArgs& pos, float* out, void* ws,
                            const SeqStats* stats, const RopeIn* rope) {
  AttnParams P = {};
  P.B = B;
  P.S = S;
  P.NH = NH;
  P.NKV = NKV;
  P.G = NH / NKV;
  P.T = T;
  P.q = q;
  P.kc = k_cache;
  P.vc = v_cache;
  P.kd = k_delta;
  P.vd = v_delta;
  P.pos = pos;
  P.out = out;
  P.part = (double*)ws;
  if (rope && !(S == 1 && P.G <= 8)) return hipErrorInvalidValue;
  if (rope) P.rope = *rope;
  if (S == 1 && P.G <= 8) {
    P.nsplit = decode_split(T, B, pos);
    P.tsplit = ad::DK;
    hipLaunchKernelGGL(k_attn_dec<false>, dim3(P.nsplit, B * NKV), dim3(256), 0, st, P);
    hipLaunchKernelGGL(k_attn_combine<false>, dim3(B * NH), dim3(128), 0, st, 1, NH, P.nsplit, P.part,
                       out);
  } else if (attention_prefill_supported(NH, NKV)) {
    return launch_attention_prefill(st, B, S, NH, NKV, T, q, k_cache, v_cache, k_delta, v_delta,
                                    pos, out, stats, ws);
  } else {
    P.nsplit = 1;
    P.tsplit = T;
    hipLaunchKernelGGL((k_attn<8, 16>), dim3((S + 7) / 8, B * NKV), dim3(256), 0, st, P);
  }
  return hipGetLastError();
}

hipError_t launch_attention_dec_bf16(hipStream_t st, const AttnBf16Params& Q, void* part) {
  if (Q.S != 1 || Q.NKV < 1 || Q.NH % Q.NKV != 0 || Q.NH / Q.NKV > 8 || !part)
    return hipErrorInvalidValue;
  AttnParams P = {};
  P.B = Q.B;
  P.S = 1;
  P.NH = Q.NH;
  P.NKV = Q.NKV;
  P.G = Q.NH / Q.NKV;
  P.T = Q.T;
  P.q = (const float*)Q.q;  // bf16 storage, read as such
  P.kc = (const float*)Q.kc;
  P.vc = (const float*)Q.vc;
  P.kd = (const float*)Q.kd;
  P.vd = (const float*)Q.vd;
  P.pos = Q.pos;
  P.out = (float*)Q.out;
  P.part = (double*)part;
  P.nsplit = decode_split(Q.T, Q.B, Q.pos);
  P.tsplit = ad::DK;
  hipLaunchKernelGGL(k_attn_dec<true>, dim3(P.nsplit, Q.B * Q.NKV), dim3(256), 0, st, P);
  hipLaunchKernelGGL(k_attn_combine<true>, dim3(Q.B * Q.NH), dim3(128), 0, st, 1, Q.NH, P.nsplit,
                     P.part, P.out);
  return hipGetLastError();
}

}  // namespace ark
