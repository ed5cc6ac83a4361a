// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ark {

// One int8 projection with its output: rows of the projection go to
// out[r * ldo + n] (n < m.n).
struct Seg {
  const int8_t* w;
  const float* sw;
  const int32_t* cs;
  const float* bias;
  int n;
  float* out;
  int ldo;
};

enum Epi { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2 };

// Optional record of one dynamic quantisation for the re-anchored parity
// tests: the fp32 tensor the quantiser saw (h: only where the quantiser
// itself computes it, i.e. behind an RMSNorm), the shifted codes it produced
// and its (s, z) per sequence.  Null members are not written.
struct QDump {
  float* h;
  int8_t* codes;
  float* s;
  int* z;
};

// Global-memory pointers: accesses through them compile to global (not
// flat) instructions, whose completion the compiler can count exactly.
template <typename T>
using gptr = T __attribute__((address_space(1)))*;

// a wave-uniform pointer taken through scalar registers (readfirstlane), as
// a global pointer
template <typename T>
__device__ __forceinline__ gptr<T> uniform_ptr(T* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (gptr<T>)(((uint64_t)hi << 32) | lo);
}

// 16-byte load through a global pointer (element i of float4s at p)
__device__ __forceinline__ float4 ld4(gptr<const float> p, int i) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  const f4 v = ((const f4 __attribute__((address_space(1)))*)p)[i];
  return make_float4(v.x, v.y, v.z, v.w);
}

// ---- prep / misc (k_misc.hip)
hipError_t launch_prep_weight(hipStream_t st, const float* w, int n, int k, int8_t* codes,
                              float* scale, int32_t* colsum);
hipError_t launch_rope_table(hipStream_t st, int T, int D, double theta, double* c, double* s);
hipError_t launch_embed(hipStream_t st, int B, int S, int H, int V, const int32_t* ids,
                        const uint16_t* table, const float* audio, int a0, int N, float* out);
// Weight-only int4 LM tier (k_lm4.hip): block quantisation of an fp32
// weight into packed uint4 codes [n][k/2], fp32 scales [n][k/128] and
// packed uint4 zero points [n][k/256]; the head over B fp32 rows.
hipError_t launch_prep_w4(hipStream_t st, const float* w, int n, int k, uint8_t* codes,
                          float* scale, uint8_t* zp);
bool lm4_supported(int K);
hipError_t launch_lm4(hipStream_t st, int B, int K, int N, const float* h, int ldh,
                      const uint8_t* w, const float* sc, const uint8_t* zp, float* logits,
                      int ldl);
hipError_t launch_masked_argmax(hipStream_t st, int B, int V, const float* logits,
                                const uint8_t* mask, int32_t* out_ids);
hipError_t launch_test_codes(hipStream_t st, int rows, int K, int R, const uint8_t* in,
                             int8_t* out, const float* s_in, const uint8_t* z_in, float* s_row,
                             int* z_row);
constexpr int kMaxLayers = 64;
hipError_t launch_cache_write(hipStream_t st, int L, int B, int S, int T, int row_floats,
                              const int32_t* pos_host, float* const* k_cache,
                              float* const* v_cache, const float* k_delta, const float* v_delta);
// Greedy-loop bookkeeping: tokens of finished sequences become end_id, the
// step's ids are copied to out_row, and done flags are updated.
hipError_t launch_greedy_post(hipStream_t st, int B, int32_t* tokens, int32_t* out_row,
                              int32_t end_id, int32_t* done);

// ---- quantisation (k_quant.hip)
// Per-sequence running min / max of an activation tensor, kept as ordered
// ints (float_to_ordered) so that producers combine partial results with
// integer atomics.  Atomics on one cache line serialise, so a set holds
// kStatsRep replicas, each a 512-byte block of lo[kMaxBatch], hi[kMaxBatch];
// a producer spreads its atomics over the replicas and a consumer folds
// them.  A producer accumulates into `cur` and resets `clr` (the other set)
// for the next producer: two sets used in turn, each cleared by the producer
// before the one that fills it.
constexpr int kMaxBatch = 64;
constexpr int kStatsRep = 64;
constexpr int kStatsSetInts = kStatsRep * 2 * kMaxBatch;
struct SeqStats {
  int* cur;  // [kStatsRep][2][kMaxBatch]
  int* clr;  // same shape
  int nseq;  // <= kMaxBatch
};
// Producer side (callers include common.hpp first): fold a wave's (lo, hi)
// of sequence b into replica rep; reset the other set (one workgroup).
__device__ __forceinline__ void stats_fold(const SeqStats& S, int rep, int b, float lo, float hi) {
  int* blk = S.cur + (rep % kStatsRep) * 2 * kMaxBatch;
  atomicMin(blk + b, float_to_ordered(lo));
  atomicMax(blk + kMaxBatch + b, float_to_ordered(hi));
}
__device__ __forceinline__ void stats_clear_other(const SeqStats& S) {
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int t = threadIdx.x; t < kStatsSetInts; t += blockDim.x)
      S.clr[t] = (t % (2 * kMaxBatch)) < kMaxBatch ? kOrdPosInf : kOrdNegInf;
}
// Consumer side: the range of sequence b, folded over the replicas by one
// wave (every lane gets it).
__device__ __forceinline__ void stats_range(const int* set, int b, float& lo, float& hi) {
  const int l = threadIdx.x & 63;
  float a = INFINITY, z = -INFINITY;
  for (int r = l; r < kStatsRep; r += 64) {
    a = fminf(a, ordered_to_float(set[r * 2 * kMaxBatch + b]));
    z = fmaxf(z, ordered_to_float(set[r * 2 * kMaxBatch + kMaxBatch + b]));
  }
  lo = wave_min(a);
  hi = wave_max(z);
}
// Constants of swiglu_f64: 1/k! for k = 12 down to 3 (each rounded to
// nearest), ln2_hi (ln2 with its low 21 mantissa bits cleared), ln2_lo =
// ln2 - ln2_hi, 1/ln2, and the clamp of the exponent's argument.
#define ARK_SWIGLU_CONSTS                                                                   \
  0x1.1eed8eff8d898p-29, 0x1.ae64567f544e4p-26, 0x1.27e4fb7789f5cp-22, 0x1.71de3a556c734p-19, \
      0x1.a01a01a01a01ap-16, 0x1.a01a01a01a01ap-13, 0x1.6c16c16c16c17p-10,                    \
      0x1.1111111111111p-7, 0x1.5555555555555p-5, 0x1.5555555555555p-3,                       \
      0x1.62e42fee00000p-1, 0x1.a39ef35793c76p-33, 0x1.71547652b82fep+0, -746.0
static __constant__ double kSwigluTab[14] = {ARK_SWIGLU_CONSTS};
struct SwigluK {
  double c[14];
};
// The table loaded once (a caller does it outside its loops) into scalar
// registers, from where the VALU instructions take the constants as scalar
// operands; as literals every use would first be copied into vector
// registers.  The table's address is made opaque so its values are not
// folded back into literals, and kept in the constant address space so
// the loads are scalar.
__device__ __forceinline__ SwigluK swiglu_consts() {
  typedef const double __attribute__((address_space(4))) * cptr;
  cptr c = (cptr)kSwigluTab;
  asm("" : "+s"(c));
  SwigluK K;
#pragma unroll
  for (int i = 0; i < 14; ++i) K.c[i] = c[i];
  return K;
}

// The same constants as literals, for code whose scalar registers are taken.
__device__ __forceinline__ SwigluK swiglu_consts_literal() {
  return SwigluK{{ARK_SWIGLU_CONSTS}};
}

// Qwen2 MLP gate, silu(g) * u = g / (1 + e^-g) * u, in fp64 and rounded
// once to fp32 (fp32 g and u).  Written as (g >= 0 ? g u : g u t) / (1 + t)
// with t = e^-|g| in [0, 1]: the denominator lies in [1, 2], so its
// reciprocal estimate needs two Newton steps and none of a general
// division's scaling or special cases.  g u is exact in fp64.
// e^-|g| by exp_nonpos_core (NaN in g or u propagates through g u).  A few
// fp64 ulp from the exact value.
// e^x for x <= 0 (x = -inf gives 0; NaN is not handled), fp64: x = k ln2 +
// r with |r| <= ln2 / 2 (ln2 in two parts, k ln2_hi exact), e^r by its
// Taylor series to degree 12 (first dropped term below 2e-16), times 2^k;
// below -746 the argument is clamped (the result underflows to 0).  A few
// fp64 ulp from the exact value.
__device__ __forceinline__ double exp_nonpos_core(double x, const SwigluK& K) {
  const double* c = K.c;
  const double xc = fmax(x, c[13]);
  const double k = rint(xc * c[12]);
  const double r = fma(-k, c[11], fma(-k, c[10], xc));
  double p = c[0];
#pragma unroll
  for (int i = 1; i < 10; ++i) p = fma(p, r, c[i]);
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  return ldexp(p, (int)k);
}
// The same with NaN passed through.
__device__ __forceinline__ double exp_nonpos_f64(double x, const SwigluK& K) {
  const double t = exp_nonpos_core(x, K);
  return x != x ? x : t;
}

__device__ __forceinline__ float swiglu_f64(float g, float u, const SwigluK& K) {
  const double gd = g;
  const double t = exp_nonpos_core(-fabs(gd), K);
  const double n = gd * (double)u;
  const double num = gd >= 0.0 ? n : n * t;
  const double d = 1.0 + t;
  double q = __builtin_amdgcn_rcp(d);
  q = fma(q, fma(-d, q, 1.0), q);
  q = fma(q, fma(-d, q, 1.0), q);
  return (float)(num * q);
}

// set = (+inf, -inf) everywhere
hipError_t launch_seq_stats_init(hipStream_t st, int* set);
// folded range of sequences 0..n-1 as fp32 (tests)
hipError_t launch_seq_stats_read(hipStream_t st, const int* set, int n, float* flo, float* fhi);
// Stats producer for R rows of K floats (row stride ldx), rows r of sequence
// r / rows_per_seq.  With gain: RMSNorm statistics (fp64 inside): rs_out[r] =
// 1 / sqrt(mean(x^2) + eps) and the min/max of h = fp32((x * rs) * gain);
// h itself is not written.  Without gain: the min/max of x.
hipError_t launch_row_stats(hipStream_t st, int R, int K, int rows_per_seq, const float* x,
                            int ldx, const float* gain, double eps, double* rs_out,
                            const SeqStats& stats);
// GELU (k_adapter.hip): y <- GELU(y) in place over R rows of N values (row
// stride ldy), plus row r % rows_per_seq of `add` when add != nullptr; the
// per-sequence range of the result folded into S (rows r of sequence
// r / rows_per_seq; clears S.clr) when S.cur != nullptr.
hipError_t launch_gelu_stats(hipStream_t st, int R, int N, int rows_per_seq, float* y, int ldy,
                             const SeqStats& S, const float* add = nullptr, int ldadd = 0);

// Audio encoder (k_encoder.hip).
// im2col of a width-3, padding-1 convolution: x [B][T][C] -> rows
// [B][To][3 C] with element (j, c) of row t = x[b][t * stride - 1 + j][c]
// (0 outside); C % 4 == 0.
hipError_t launch_im2col(hipStream_t st, int B, int T, int C, int stride, const float* x,
                         float* rows);
// LayerNorm of R rows of D values (fp64 inside, one rounding):
// y = fp32(((x - mean) / sqrt(var + eps)) * g + b); per-sequence range of y
// into S when S.cur != nullptr.
hipError_t launch_layernorm(hipStream_t st, int R, int D, int rows_per_seq, const float* x,
                            const float* g, const float* b, double eps, float* y,
                            const SeqStats& S);
// Bidirectional self-attention of B clips of F frames, H heads of 64: qkv
// rows [B][F][3 H 64] (q | k | v), q and k rotated (fp64 tables
// [>= F][32]) and rounded to fp32 before use, softmax(q.k / 8) v in fp64;
// out [B][F][H 64] and its per-sequence range into S (S.cur != nullptr).
// part (optional): enc_attention_ws_bytes(B, F, H) bytes; with it a launch
// of few workgroups (a short clip) splits the key chunks and merges.
size_t enc_attention_ws_bytes(int B, int F, int H);
hipError_t launch_enc_attention(hipStream_t st, int B, int F, int H, const float* qkv,
                                const double* cos, const double* sin, float* out,
                                const SeqStats& S, void* part = nullptr);

// Dynamic uint8 quantisation with one (s, z) per sequence from the range in
// `set`: codes of x (or of h recomputed from x, rs and gain when rs !=
// nullptr), shifted codes (code - 128) [R][K] and/or plain codes; s_out /
// z_out [nseq].
// h_out (optional, [R][K]): the values quantised (h where it is recomputed).
hipError_t launch_quant_seq(hipStream_t st, int R, int K, int rows_per_seq, const float* x,
                            int ldx, const double* rs, const float* gain, const int* set,
                            int8_t* codes, uint8_t* codes_u8, float* s_out, int* z_out,
                            float* h_out = nullptr);

// One row per sequence (decode): optional RMSNorm (gain != nullptr) and the
// row's dynamic quantisation in one kernel; shifted codes [B][K], s/z [B].
bool norm_quant_row_supported(int K);
// h_out (optional, [B][K]): the values quantised (the normed row with a gain).
hipError_t launch_norm_quant_row(hipStream_t st, int B, int K, const float* x, int ldx,
                                 const float* gain, double eps, int8_t* codes, float* s_out,
                                 int* z_out, float* h_out = nullptr);

// ---- int8 projections
// Decode GEMV (k_gemv.hip): B <= 4 rows of input x (row stride ldx), fused
// prologue (RMSNorm when gain != nullptr, then per-row quantisation), segments
// concatenated along the output dimension (EPI_SWIGLU: seg[0] gate, seg[1] up,
// result to seg[0].out).  acc_out (optional) receives raw int32 accumulators.
// qd (optional): workgroup 0 records its prologue's quantisation ([B][K]).
hipError_t launch_gemv(hipStream_t st, int B, int K, const float* x, int ldx, const float* gain,
                       double eps, const Seg* segs, int nseg, Epi epi, const QDump* qd = nullptr);
// Same GEMV on precomputed shifted codes [B][K] with per-row (s, z).
hipError_t launch_gemv_codes(hipStream_t st, int B, int K, const int8_t* codes, const float* s,
                             const int* z, const Seg* segs, int nseg, Epi epi, int32_t* acc_out);
// MFMA GEMM (k_gemm.hip): shifted codes [M][K]; row r uses (s[r / rows_per_seq],
// z[r / rows_per_seq]).
// Large-M GEMM (prefill): same contract as launch_gemm; requires
// gemm_big_supported(M, K).  split_ws (optional): gemm_big_split_ws_bytes()
// bytes, zero before the first launch (they stay zero between launches);
// with it a launch of few tiles splits K over several workgroups per tile.
bool gemm_big_supported(int M, int K);
size_t gemm_big_split_ws_bytes();
hipError_t launch_gemm_big(hipStream_t st, int M, int K, const int8_t* codes, const float* s,
                           const int* z, int rows_per_seq, const Seg* segs, int nseg, Epi epi,
                           int32_t* acc_out, const SeqStats* stats = nullptr,
                           void* split_ws = nullptr);
// Few-row GEMM (k_gemm_sk.hip, M < 128: batched decode, LM head of a
// batch, short prompts; one pass per 64 rows): same contract; scratch =
// gemm_skinny_ws_bytes() bytes whose counter words are zero
// (gemm_skinny_reset) and stay zero between launches.
bool gemm_skinny_supported(int M, int K);
size_t gemm_skinny_ws_bytes();
hipError_t gemm_skinny_reset(hipStream_t st, void* scratch);
// The scratch launch_gemm takes for calls of up to max_rows rows: the
// few-row GEMM's, then (max_rows >= 128) the large-tile GEMM's split-K
// blocks; gemm_scratch_reset zeroes all of it (once per forward call).
size_t gemm_ws_bytes(size_t max_rows);
hipError_t gemm_scratch_reset(hipStream_t st, void* scratch, size_t max_rows);
// p[0..n) = 0 with a small kernel (no memset node, so it may be captured)
hipError_t launch_zero_u32(hipStream_t st, uint32_t* p, int n);
hipError_t launch_gemm_skinny(hipStream_t st, int M, int K, const int8_t* codes, const float* s,
                              const int* z, int rows_per_seq, const Seg* segs, int nseg, Epi epi,
                              int32_t* acc_out, void* scratch);
// Dispatch: few-row GEMM when scratch is given and the shape allows it, the
// large-tile GEMM for M >= 128 (splitting K over the scratch's split-K
// blocks when given: scratch must then hold gemm_ws_bytes(M) bytes), else
// the tiled GEMM; tiled_only forces the latter (tests).  stats (EPI_SWIGLU only): the large-tile GEMM also
// produces the per-sequence min / max of its output into *stats;
// gemm_swiglu_stats(M, K, scratch) tells whether this call's dispatch does.
bool gemm_swiglu_stats(int M, int K, const void* scratch);
// y[i] = swiglu_f64(g[i], u[i]) for i < n (tests of the GEMM epilogues' gate)
hipError_t launch_swiglu(hipStream_t st, int64_t n, const float* g, const float* u, float* y);
hipError_t launch_gemm(hipStream_t st, int M, int K, const int8_t* codes, const float* s,
                       const int* z, int rows_per_seq, const Seg* segs, int nseg, Epi epi,
                       int32_t* acc_out, void* scratch = nullptr, bool tiled_only = false,
                       const SeqStats* stats = nullptr);

// Few-row GEMM in two launches (M <= 64 rows, one per sequence; store or
// residual epilogue): the split-K launch stores each split's int32 sums
// (part: gemm_rows_part_bytes(M, ncols) bytes), then a row kernel adds them
// and runs the same epilogue, and with `norm` (residual, one segment) also
// RMSNorm and the dynamic quantiser of each output row as
// launch_norm_quant_row does.  Results are those of launch_gemm followed by
// launch_norm_quant_row.
struct RowNorm {
  const float* g;
  double eps;
  int8_t* codes;
  float* s;
  int* z;
  float* h_out;
};
bool row_epi_supported(int ncols);
bool gemm_rows_supported(int M, int K, Epi epi, int ncols);
size_t gemm_rows_part_bytes(int M, int ncols);
hipError_t launch_gemm_rows(hipStream_t st, int M, int K, const int8_t* codes, const float* s,
                            const int* z, const Seg* segs, int nseg, Epi epi, int32_t* part,
                            const RowNorm* norm);
hipError_t launch_row_epi(hipStream_t st, int M, int ks, const int32_t* part, const float* s,
                          const int* z, const Seg* segs, int nseg, Epi epi, const RowNorm* norm);

// ---- rotary + attention (k_attn.hip)
// qkv_raw [R][q_dim + 2*kv_dim] (bias added) -> q_rot [R][q_dim], k_delta /
// v_delta [R][kv_dim]; row r of sequence r / S sits at pos[r / S] + r % S.
struct PosArgs {
  int32_t p[64];
};

// Prefill attention (S > 1) on fp64 matrix cores; G = NH / NKV <= 8.
bool attention_prefill_supported(int NH, int NKV);
// Key-chunk split of a prefill launch of few workgroups (a single prompt):
// the number of workgroups each query tile's chunks are dealt over (1: no
// split), given the largest start position pmax.
int attention_prefill_split(int B, int S, int NH, int NKV, int T, int pmax);
// stats (optional): per-sequence min / max of out, as a stats producer (not
// when the launch splits; attention_stats tells).  part (optional):
// attention_ws_bytes(B, S, NH, T) bytes for the split partial states; with
// it a launch of few workgroups splits its key chunks and merges the states.
hipError_t launch_attention_prefill(hipStream_t st, int B, int S, int NH, int NKV, int T,
                                    const float* q, const float* k_cache, const float* v_cache,
                                    const float* k_delta, const float* v_delta,
                                    const PosArgs& pos, float* out,
                                    const SeqStats* stats = nullptr, void* part = nullptr);
// Merge of split partial softmax states part [B][NH][S][nsplit][2 + 128]
// into out [B][S][NH][128] (fp32, or bf16 when bf16).
hipError_t launch_attention_merge(hipStream_t st, int B, int S, int NH, int nsplit,
                                  const double* part, void* out, bool bf16);
hipError_t launch_rope(hipStream_t st, int B, int S, int NH, int NKV, const float* qkv,
                       const double* cosT, const double* sinT, const PosArgs& pos, float* q,
                       float* k_delta, float* v_delta);
// Full-cache GQA attention.  out [B*S][NH*128] fp32.  ws: scratch for split
// partials (decode, and a split prefill); attention_ws_bytes gives its
// size.  stats: as for launch_attention_prefill, honoured when
// attention_stats(B, S, NH, NKV, T, pmax) with pmax the largest position.
size_t attention_ws_bytes(int B, int S, int NH, int T);
// Decode (S = 1, NH / NKV <= 8) with the rotary step folded in: q, k and v
// are read unrotated from the q|k|v projection rows (stride ld) and the
// rotated key and the value of each sequence are written to kd_out / vd_out
// ([B][NKV][128]), as launch_rope would (same arithmetic).
struct RopeIn {
  const float* qkv;
  int ld;
  const double* cosT;
  const double* sinT;
  float* kd_out;
  float* vd_out;
};
bool attention_stats(int B, int S, int NH, int NKV, int T, int pmax);
hipError_t launch_attention(hipStream_t st, int B, int S, int NH, int NKV, int T, const float* q,
                            const float* k_cache, const float* v_cache, const float* k_delta,
                            const float* v_delta, const PosArgs& pos, float* out, void* ws,
                            const SeqStats* stats = nullptr, const RopeIn* rope = nullptr);

// ---- persistent batch-1 decode step for the ARK geometry (k_decode.hip)
// Re-anchored parity record (layout of ark_dump_layout in ark.h): layer l
// with bit l of mask set has its record at base + (index among the recorded
// layers) * rec; f[] are the field offsets inside a record and head[] the
// offsets of the LM-head fields from base.  base == nullptr: none.
struct DumpRec {
  char* base;
  uint64_t mask;
  size_t rec;
  size_t f[13];
  size_t head[4];
};
struct MegaLayer {
  const int8_t* w[7];  // q, k, v, o, gate, up, down
  const float* sw[7];
  const int32_t* cs[7];
  const float* bias[3];
  const float* ln1;
  const float* ln2;
  const float* kc;
  const float* vc;
};
struct MegaStep {
  int L, T, V, pos;
  double eps;
  const int32_t* token;
  const uint16_t* table;
  const float* final_norm;
  const int8_t* lm_w;
  const float* lm_sw;
  const int32_t* lm_cs;
  // the int4 LM tier (lm4_w != nullptr, lm_w == nullptr): packed codes
  // [V][H/2], scales [V][H/128], packed zero points [V][H/256]
  const uint8_t* lm4_w;
  const float* lm4_s;
  const uint8_t* lm4_z;
  const double* rcos;
  const double* rsin;
  float* kdelta;
  float* vdelta;
  float* logits;
  float* hidden_out;
  const uint8_t* mask;
  int32_t* out_token;
  DumpRec dump;         // base == nullptr: the production kernel, no record
  int64_t spin_limit;   // rounds per bounded wait; < 0: the default bound
};
bool decode_mega_supported(int H, int NH, int NKV, int D, int I, int T, int L);
size_t decode_mega_ws_bytes(int L, int T);
size_t decode_mega_trace_offset(int L, int T);
hipError_t decode_mega_init();
// ARK_DECODE_LAUNCH=cooperative: launch the persistent step cooperatively
bool decode_mega_cooperative();
hipError_t decode_mega_upload(hipStream_t st, void* ws, int L, int T, const MegaLayer* layers);
// ev_begin / ev_end (nullable) are recorded around the persistent kernel
// alone (not its preparation kernel).  prep = false: the launch was
// prepared already (by decode_mega_between of the previous token).
hipError_t decode_mega_launch(hipStream_t st, void* ws, const MegaStep& S, hipEvent_t ev_begin,
                              hipEvent_t ev_end, bool prep = true);
// After a step of the greedy loop (S as launched): its deltas into the
// caches at row S.pos, the stop rule on *S.token (out_row, done, end_id as
// for launch_greedy_post), and with prep the preparation of the next
// step's launch for the resulting id.
hipError_t decode_mega_between(hipStream_t st, void* ws, const MegaStep& S, float* const* k_cache,
                               float* const* v_cache, int32_t* out_row, int32_t end_id,
                               int32_t* done, bool prep);
// Error word of the last persistent launch on this workspace (0: every
// bounded wait was met; read after the stream has completed that launch).
const uint32_t* decode_mega_err_word(const void* ws, int L, int T);
// The word that marks the workspace's exchange area as initialised for this
// layout; zeroing it makes the next launch clear the area and restart its
// tags.
uint64_t* decode_mega_marker(void* ws, int L, int T);

// bf16 serving variant (k_bf16.hip).  A segment of output columns: bf16
// weight rows [n][K], optional bf16 bias, output (bf16, or fp32 for
// BE_F32) with row stride ldo.
enum { BE_STORE = 0, BE_RESID = 1, BE_SWIGLU = 2, BE_F32 = 3 };
struct BSeg {
  const uint16_t* w;
  const uint16_t* bias;
  void* out;
  int n, ldo;
};
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
// nearest even; NaN stays a (quiet) NaN
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((b >> 16) | 0x40u);
  b += 0x7fffu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}
__device__ __forceinline__ float rbf(float f) { return bf2f(f2bf(f)); }

// four values of a row from fp32 (BF false) or bf16 (BF true) storage; off
// counts elements of the storage type
template <bool BF>
__device__ __forceinline__ float4 ld4e(gptr<const float> base, size_t off, int d4) {
  if constexpr (BF) {
    typedef unsigned int u2 __attribute__((ext_vector_type(2)));
    const u2 u = ((const u2 __attribute__((address_space(1)))*)((gptr<const uint16_t>)base + off))[d4];
    return make_float4(bf2f((uint16_t)u.x), bf2f((uint16_t)(u.x >> 16)), bf2f((uint16_t)u.y),
                       bf2f((uint16_t)(u.y >> 16)));
  } else {
    return ld4(base + off, d4);
  }
}

// ---- the epilogue of one output value
// BE_STORE: bf16(acc + bias); BE_RESID: bf16(old + bf16(acc + bias));
// BE_F32: fp32 acc (the logits); the SwiGLU pair is handled by the callers.
__device__ __forceinline__ void bf_out(int epi, const BSeg& S, int row, int n, float acc) {
  float y = acc;
  if (epi == BE_F32) {
    ((float*)S.out)[(size_t)row * S.ldo + n] = y;
    return;
  }
  if (S.bias) y = y + bf2f(S.bias[n]);
  uint16_t* o = (uint16_t*)S.out + (size_t)row * S.ldo + n;
  if (epi == BE_RESID)
    *o = f2bf(bf2f(*o) + rbf(y));
  else
    *o = f2bf(y);
}
// a = bf16(bf16(silu(bf16(g))) * bf16(u))
__device__ __forceinline__ uint16_t bf_swiglu(float g, float u) {
  const float gb = rbf(g), ub = rbf(u);
  const float sg = rbf(gb / (1.0f + expf(-gb)));
  return f2bf(sg * ub);
}

struct GemvBf16Params {
  int M, K, ldx, nseg, epi, ncols;
  const uint16_t* x;
  BSeg seg[3];
  int seg_start[4];
};
hipError_t launch_to_bf16(hipStream_t st, int64_t n, const float* x, uint16_t* y);
bool gemm_bf16_supported(int K);
// y = x W^T over M rows of x (row stride ldx); epilogue epi (BE_SWIGLU: seg
// 0 gate, seg 1 up, result to seg 0's output)
hipError_t launch_gemm_bf16(hipStream_t st, int M, int K, const uint16_t* x, int ldx,
                            const BSeg* segs, int nseg, int epi);
// the same at M >= 128 rows on the large LDS-DMA tiles (x row stride K)
hipError_t launch_gemm_big_bf16(hipStream_t st, int M, int K, const uint16_t* x, const BSeg* segs,
                                int nseg, int epi);
hipError_t launch_rmsnorm_bf16(hipStream_t st, int R, int H, const uint16_t* x, int ldx,
                               const uint16_t* g, double eps, uint16_t* y);
hipError_t launch_rope_bf16(hipStream_t st, int B, int S, int NH, int NKV, const uint16_t* qkv,
                            const double* cosT, const double* sinT, const PosArgs& pos,
                            uint16_t* q_out, uint16_t* kd, uint16_t* vd);
struct AttnBf16Params {
  int B, S, NH, NKV, T;
  const uint16_t* q;   // [B][S][NH][128] rotated
  const uint16_t* kc;  // [B][T][NKV][128]
  const uint16_t* vc;
  const uint16_t* kd;  // [B][S][NKV][128]
  const uint16_t* vd;
  PosArgs pos;
  uint16_t* out;       // [B][S][NH * 128]
};
// query heads per KV head at most 8; part: attention_ws_bytes(B, S, NH, T)
// bytes (decode partial states; unused for S > 1)
bool attn_bf16_supported(int NH, int NKV);
hipError_t launch_attn_bf16(hipStream_t st, const AttnBf16Params& P, void* part);
// the prefill attention of k_attn2.hip on bf16 storage (S >= 1,
// attention_prefill_supported(NH, NKV)); out rounded to bf16
hipError_t launch_attention_prefill_bf16(hipStream_t st, const AttnBf16Params& P,
                                         void* part = nullptr);
// the split decode attention of k_attn.hip on bf16 storage (S == 1,
// NH / NKV <= 8); part: attention_ws_bytes(B, 1, NH, T) bytes of partial
// states; out rounded to bf16
hipError_t launch_attention_dec_bf16(hipStream_t st, const AttnBf16Params& P, void* part);
hipError_t launch_embed_bf16(hipStream_t st, int R, int H, int V, const int32_t* ids,
                             const uint16_t* table, uint16_t* x);
struct CacheBf16Args {
  uint16_t* k[kMaxLayers];
  uint16_t* v[kMaxLayers];
};
hipError_t launch_cache_write_bf16(hipStream_t st, int L, int B, int S, int T, int KVW,
                                   const PosArgs& pos, const CacheBf16Args& A, const uint16_t* kd,
                                   const uint16_t* vd);

}  // namespace ark
