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

// ---- prep / misc (k_misc.hip)
hipError_t launch_prep_weight(hipStream_t st, const float* w, int n, int k, int8_t* codes,
                              float* scale, int32_t* colsum);
hipError_t launch_rope_table(hipStream_t st, int T, int D, double theta, double* c, double* s);
hipError_t launch_embed(hipStream_t st, int B, int S, int H, int V, const int32_t* ids,
                        const uint16_t* table, const float* audio, int a0, int N, float* out);
hipError_t launch_masked_argmax(hipStream_t st, int B, int V, const float* logits,
                                const uint8_t* mask, int32_t* out_ids);
hipError_t launch_test_codes(hipStream_t st, int rows, int K, int R, const uint8_t* in,
                             int8_t* out, const float* s_in, const uint8_t* z_in, float* s_row,
                             int* z_row);
constexpr int kMaxLayers = 64;
constexpr int kMaxBatch = 64;
hipError_t launch_cache_write(hipStream_t st, int L, int B, int S, int T, int row_floats,
                              const int32_t* pos_host, float* const* k_cache,
                              float* const* v_cache, const float* k_delta, const float* v_delta);
// Greedy-loop bookkeeping: tokens of finished sequences become end_id, the
// step's ids are copied to out_row, and done flags are updated.
hipError_t launch_greedy_post(hipStream_t st, int B, int32_t* tokens, int32_t* out_row,
                              int32_t end_id, int32_t* done);

// ---- quantisation (k_quant.hip)
// h[r] = rmsnorm(x[r]) (fp64 inside), plus per-row min/max of h.
hipError_t launch_rmsnorm_rows(hipStream_t st, int R, int H, const float* x, int ldx,
                               const float* gain, double eps, float* h, float* rmin, float* rmax);
hipError_t launch_rowminmax(hipStream_t st, int R, int K, const float* x, float* rmin, float* rmax);
// Rows r of sequence b = r / S share one (s, z) from the min/max of all their
// rows; writes shifted codes (code - 128) and, if non-null, plain uint8 codes.
hipError_t launch_quant_rows(hipStream_t st, int B, int S, int K, const float* x,
                             const float* rmin, const float* rmax, int8_t* codes,
                             uint8_t* codes_u8, float* s_out, int* z_out);

// One row per sequence (decode): optional RMSNorm (gain != nullptr) and the
// row's dynamic quantisation in one kernel; shifted codes [B][K], s/z [B].
bool norm_quant_row_supported(int K);
hipError_t launch_norm_quant_row(hipStream_t st, int B, int K, const float* x, int ldx,
                                 const float* gain, double eps, int8_t* codes, float* s_out,
                                 int* z_out);

// ---- int8 projections
// Decode GEMV (k_gemv.hip): B <= 4 rows of input x (row stride ldx), fused
// prologue (RMSNorm when gain != nullptr, then per-row quantisation), segments
// concatenated along the output dimension (EPI_SWIGLU: seg[0] gate, seg[1] up,
// result to seg[0].out).  acc_out (optional) receives raw int32 accumulators.
hipError_t launch_gemv(hipStream_t st, int B, int K, const float* x, int ldx, const float* gain,
                       double eps, const Seg* segs, int nseg, Epi epi);
// Same GEMV on precomputed shifted codes [B][K] with per-row (s, z).
hipError_t launch_gemv_codes(hipStream_t st, int B, int K, const int8_t* codes, const float* s,
                             const int* z, const Seg* segs, int nseg, Epi epi, int32_t* acc_out);
// MFMA GEMM (k_gemm.hip): shifted codes [M][K]; row r uses (s[r / rows_per_seq],
// z[r / rows_per_seq]).
// Large-M GEMM (prefill): same contract as launch_gemm; requires
// gemm_big_supported(M, K).
bool gemm_big_supported(int M, int K);
hipError_t launch_gemm_big(hipStream_t st, int M, int K, const int8_t* codes, const float* s,
                           const int* z, int rows_per_seq, const Seg* segs, int nseg, Epi epi,
                           int32_t* acc_out);
// Few-row GEMM (k_gemm_sk.hip, M <= 32: batched decode, LM head of a
// batch): same contract; scratch = gemm_skinny_ws_bytes() bytes whose
// counter words are zero (gemm_skinny_reset) and stay zero between launches.
bool gemm_skinny_supported(int M, int K);
size_t gemm_skinny_ws_bytes();
hipError_t gemm_skinny_reset(hipStream_t st, void* scratch);
hipError_t launch_gemm_skinny(hipStream_t st, int M, int K, const int8_t* codes, const float* s,
                              const int* z, int rows_per_seq, const Seg* segs, int nseg, Epi epi,
                              int32_t* acc_out, void* scratch);
// Dispatch: few-row GEMM when scratch is given and the shape allows it, the
// large-tile GEMM for M >= 128, else the tiled GEMM; tiled_only forces the
// latter (tests).
hipError_t launch_gemm(hipStream_t st, int M, int K, const int8_t* codes, const float* s,
                       const int* z, int rows_per_seq, const Seg* segs, int nseg, Epi epi,
                       int32_t* acc_out, void* scratch = nullptr, bool tiled_only = false);

// ---- rotary + attention (k_attn.hip)
// qkv_raw [R][q_dim + 2*kv_dim] (bias added) -> q_rot [R][q_dim], k_delta /
// v_delta [R][kv_dim]; row r of sequence r / S sits at pos[r / S] + r % S.
struct PosArgs {
  int32_t p[64];
};

// Prefill attention (S > 1) on fp64 matrix cores; G = NH / NKV <= 8.
bool attention_prefill_supported(int NH, int NKV);
hipError_t launch_attention_prefill(hipStream_t st, int B, int S, int NH, int NKV, int T,
                                    const float* q, const float* k_cache, const float* v_cache,
                                    const float* k_delta, const float* v_delta,
                                    const PosArgs& pos, float* out);
hipError_t launch_rope(hipStream_t st, int B, int S, int NH, int NKV, const float* qkv,
                       const double* cosT, const double* sinT, const PosArgs& pos, float* q,
                       float* k_delta, float* v_delta);
// Full-cache GQA attention.  out [B*S][NH*128] fp32.  ws: scratch for split
// partials (decode); attention_ws_bytes gives its size.
size_t attention_ws_bytes(int B, int S, int NH, int T);
hipError_t launch_attention(hipStream_t st, int B, int S, int NH, int NKV, int T, const float* q,
                            const float* k_cache, const float* v_cache, const float* k_delta,
                            const float* v_delta, const PosArgs& pos, float* out, void* ws);

// ---- persistent batch-1 decode step for the ARK geometry (k_decode.hip)
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
  const double* rcos;
  const double* rsin;
  float* kdelta;
  float* vdelta;
  float* logits;
  float* hidden_out;
  const uint8_t* mask;
  int32_t* out_token;
};
bool decode_mega_supported(int H, int NH, int NKV, int D, int I, int T, int L);
size_t decode_mega_ws_bytes(int L, int T);
size_t decode_mega_trace_offset(int L, int T);
hipError_t decode_mega_init();
hipError_t decode_mega_upload(hipStream_t st, void* ws, int L, int T, const MegaLayer* layers);
// ev_begin / ev_end (nullable) are recorded around the persistent kernel
// alone (not its preparation kernel).
hipError_t decode_mega_launch(hipStream_t st, void* ws, const MegaStep& S, hipEvent_t ev_begin,
                              hipEvent_t ev_end);

}  // namespace ark
