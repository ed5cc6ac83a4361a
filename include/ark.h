/*
 * ark.h -- C ABI of the ARK-ASR-3B int8 decoder step on MI355X (gfx950).
 *
 * What the library computes is the decoder of the model card
 * "ark-asr-3b-onnx" (Audio8/ARK-ASR-3B, INT8 ONNX export):
 *   - section "Shapes": 36 layers, hidden 2048, 16 query heads sharing 2 KV
 *     heads of dimension 128; a static, sequence-major KV cache
 *     [1, max_total_len, 2, 128] per layer that is attended over ALL
 *     max_total_len positions on every token; each call returns only the
 *     key/value rows it wrote ("deltas"), which the host copies into its cache
 *     at cache_position;
 *   - section "Files": MatMuls are dynamically quantised int8 with
 *     per-channel weights;
 *   - section "Inference": prompt embeddings with the audio slots overwritten,
 *     prefill, then greedy decoding with every added-vocab <...> token masked
 *     except <|im_end|>;
 *   - section "Revision history": fp16 embedding table, int8 LM head.
 * The block structure is the dense Qwen2 decoder named by the sglang-omni
 * cookbook page "ARK-ASR-3B" (introduction): RMSNorm -> q/k/v (with bias) ->
 * rotary embedding -> grouped-query attention -> o -> residual; RMSNorm ->
 * SwiGLU MLP -> residual.
 *
 * Numeric contract (identical to the CPU oracle the tests compare against):
 *   weights   int8 codes, symmetric per output channel: scale[n] =
 *             max|W[n,:]| / 127 (fp32), code = clamp(rne(W / scale), -127, 127)
 *   activations  one uint8 quantisation per sequence and per quantisation
 *             point (h1 -> q,k,v; attention -> o; h2 -> gate,up; a -> down;
 *             last row -> LM head): range widened to include 0,
 *             s = (max - min) / 255, z = sat(rne(-min / s)),
 *             q = sat(rne(x / s) + z), fp32 with correctly rounded division
 *   MatMul    acc = sum_k (q - z) * w exact in int32;
 *             y = fp32(fp32(acc) * fp32(s * scale[n])) (+ bias[n]), no FMA
 *   tensors between operations are fp32; RMSNorm, rotary embedding,
 *   attention softmax and SwiGLU compute in fp64 inside and round to fp32.
 *
 * Conventions for every entry point:
 *   - Pointers are device memory unless marked [host].  The caller owns all
 *     memory; the library allocates nothing and keeps no state between calls.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work on it; results are valid once the caller has
 *     synchronised the stream.  The host arrays passed in are read before
 *     the call returns.
 *   - Every argument is validated on the host before the first launch; a
 *     call that returns an error has enqueued nothing.  ARK_E_HIP reports a
 *     launch failure after work may already be queued.
 *   - Calls are thread-safe as long as concurrent calls use distinct
 *     workspaces and outputs.
 *   - Layouts are row-major, last index contiguous.
 */
#ifndef ARK_H
#define ARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum ark_status {
  ARK_OK = 0,
  ARK_E_NULL = -1,        /* a required pointer is NULL */
  ARK_E_SHAPE = -2,       /* a size is < 1, inconsistent, or unsupported */
  ARK_E_RANGE = -3,       /* cache_position < 0 or cache_position + S > T */
  ARK_E_WORKSPACE = -4,   /* workspace smaller than ark_workspace_bytes() */
  ARK_E_HIP = -5,         /* a HIP launch failed */
  ARK_E_ALIGN = -6        /* a pointer is not aligned as documented */
};

/* Model geometry.  Supported: 1 <= n_layers <= 64, head_dim == 128,
 * n_heads % n_kv_heads == 0, n_heads / n_kv_heads <= 8, hidden % 256 == 0,
 * intermediate % 64 == 0, max_total_len % 32 == 0 and <= 8192, vocab >= 1.
 * Batch sizes B are 1..64.  The ARK-ASR-3B decoder is
 * {36, 2048, 16, 2, 128, 11008, 151936, 512, 1e-6, 1e6}. */
typedef struct {
  int32_t n_layers, hidden, n_heads, n_kv_heads, head_dim, intermediate;
  int32_t vocab;          /* rows of embed_f16 (and of the LM head, if any) */
  int32_t max_total_len;  /* T: cache rows per sequence */
  double rms_eps;         /* RMSNorm epsilon */
  double rope_theta;      /* rotary base */
} ark_dims;

/* One int8 projection W[n][k] (k contiguous), prepared by ark_prep_weight.
 * All arrays 16-byte aligned; k % 16 == 0. */
typedef struct {
  const int8_t* w;        /* [n][k] codes in [-127, 127] */
  const float* scale;     /* [n] per-channel scale */
  const int32_t* colsum;  /* [n] sum_k w[n][k] */
  const float* bias;      /* [n] fp32 or NULL (only q, k, v carry one) */
  int32_t n, k;
} ark_qlinear;

/* One decoder layer.  q: n = n_heads*head_dim (head h owns rows
 * [h*head_dim, (h+1)*head_dim)), k and v: n = n_kv_heads*head_dim, all with
 * bias; o: [hidden][n_heads*head_dim]; gate, up: [intermediate][hidden];
 * down: [hidden][intermediate]; ln1, ln2: [hidden] RMSNorm gains. */
typedef struct {
  const float* ln1;
  const float* ln2;
  ark_qlinear q, k, v, o, gate, up, down;
} ark_layer;

typedef struct {
  ark_dims d;
  const ark_layer* layers;    /* [host] d.n_layers entries */
  const float* final_norm;    /* [hidden] gain of the last RMSNorm (LM head only) */
  ark_qlinear lm_head;        /* [vocab][hidden], no bias; w == NULL: none */
  const uint16_t* embed_f16;  /* [vocab][hidden] IEEE fp16 bits (decode gather) */
  const double* rope_cos;     /* [max_total_len][head_dim/2] from ark_rope_table */
  const double* rope_sin;     /* [max_total_len][head_dim/2] */
} ark_model;

/* Workspace bytes needed by ark_prefill / ark_decode_step for B sequences
 * of S rows (S = 1 for decode).  0 if the dims are invalid. */
size_t ark_workspace_bytes(const ark_dims* d, int32_t B, int32_t S);

/* Text of a status code (static storage, never NULL). */
const char* ark_status_string(int status);

/* ---------------------------------------------------------------- prep -- */

/* Quantise an fp32 weight W[n][k] (device) into int8 codes, per-channel
 * scales and per-row code sums (model card "Files": per-channel int8
 * MatMul weights).  A zero row gets scale 0 and codes 0.  codes: [n][k],
 * scale: [n], colsum: [n]; k % 16 == 0.  Errors: ARK_E_NULL, ARK_E_SHAPE. */
int ark_prep_weight(const float* w, int32_t n, int32_t k, int8_t* codes,
                    float* scale, int32_t* colsum, void* stream);

/* Rotary tables: cos/sin[pos][j] of pos * theta^(-2j/head_dim), fp64, for
 * pos < T and j < head_dim/2.  Errors: ARK_E_NULL, ARK_E_SHAPE. */
int ark_rope_table(int32_t T, int32_t head_dim, double theta, double* cos_out,
                   double* sin_out, void* stream);

/* --------------------------------------------------------------- a1 ---- */

/* Prompt embeddings with audio rows spliced in (model card "Inference",
 * steps 4-5): out[b][i] = fp32(embed_f16[ids[b][i]]) for i outside
 * [a0, a0 + N), and audio[b][i - a0] inside it.  ids: [B][S] int32 in
 * [0, vocab); audio: [B][N][hidden] fp32 (NULL iff N == 0); out:
 * [B][S][hidden].  Errors: ARK_E_NULL, ARK_E_SHAPE (a0 < 0, a0 + N > S). */
int ark_embed_splice(const ark_dims* d, int32_t B, int32_t S, const int32_t* ids,
                     const uint16_t* embed_f16, const float* audio, int32_t a0,
                     int32_t N, float* out, void* stream);

/* ------------------------------------------------------------ a2-a11 --- */

/* Prefill of B sequences of S rows each (model card "Inference" step 6).
 *   embeds          [B][S][hidden] fp32 input rows
 *   cache_position  [host][B]: row index of each sequence's first row
 *   k_cache,v_cache [host][n_layers] device pointers, each [B][T][n_kv][128]
 *                   fp32; READ ONLY here (ark_cache_write is the writer).
 *                   Rows >= cache_position[b] + S may hold any value: they
 *                   are masked by selection, never read into a result.
 *   k_delta,v_delta [n_layers][B][S][n_kv][128] fp32 out: rotated keys and
 *                   values of this call's rows (model card "Shapes")
 *   logits          [B][vocab] fp32 out for each sequence's last row, or
 *                   NULL (required NULL when the model has no LM head)
 *   hidden_out      [B][S][hidden] fp32 out (residual stream after the last
 *                   layer, before the final norm), or NULL
 *   workspace       >= ark_workspace_bytes(&m->d, B, S) bytes, 256-aligned
 * Row i of sequence b sits at position cache_position[b] + i and attends to
 * every cache row j <= cache_position[b] + i, with rows [p, p + S) taken
 * from this call's deltas.
 * Errors: ARK_E_NULL, ARK_E_SHAPE, ARK_E_RANGE (p < 0 or p + S > T),
 * ARK_E_WORKSPACE, ARK_E_ALIGN, ARK_E_HIP. */
int ark_prefill(const ark_model* m, int32_t B, int32_t S, const float* embeds,
                const int32_t* cache_position, const float* const* k_cache,
                const float* const* v_cache, float* k_delta, float* v_delta,
                float* logits, float* hidden_out, void* workspace,
                size_t workspace_bytes, void* stream);

/* One decode step (S = 1) for B sequences: token_ids [B] int32 (device) are
 * gathered from m->embed_f16, then the same computation as ark_prefill.
 * k_delta, v_delta: [n_layers][B][1][n_kv][128].  Other arguments and
 * errors as ark_prefill with S = 1. */
int ark_decode_step(const ark_model* m, int32_t B, const int32_t* token_ids,
                    const int32_t* cache_position, const float* const* k_cache,
                    const float* const* v_cache, float* k_delta, float* v_delta,
                    float* logits, float* hidden_out, void* workspace,
                    size_t workspace_bytes, void* stream);

/* ----------------------------------------------------------------- a12 -- */

/* Masked greedy argmax (model card "Inference" step 6; cookbook "Marker-
 * Token Suppression"): out_ids[b] = the lowest id v with mask[v] == 0 whose
 * logit is the maximum over unmasked ids; NaN logits are never chosen; -1 if
 * no id qualifies.  logits [B][V] fp32, mask [V] uint8 (1 = masked),
 * out_ids [B] int32.  Errors: ARK_E_NULL, ARK_E_SHAPE. */
int ark_masked_argmax(int32_t B, int32_t V, const float* logits, const uint8_t* mask,
                      int32_t* out_ids, void* stream);

/* ----------------------------------------------------------------- a13 -- */

/* Host write-back of the deltas (model card "Shapes"): for every layer l and
 * sequence b, cache[l][b][cache_position[b] + i] = delta[l][b][i], i < S, for
 * keys and values; no other row changes.  k_cache, v_cache: [host][L]
 * device pointers [B][T][n_kv][128]; deltas as returned by ark_prefill /
 * ark_decode_step.  Errors: ARK_E_NULL, ARK_E_SHAPE, ARK_E_RANGE. */
int ark_cache_write(const ark_dims* d, int32_t B, int32_t S, const int32_t* cache_position,
                    float* const* k_cache, float* const* v_cache, const float* k_delta,
                    const float* v_delta, void* stream);

/* ----------------------------------------------------------------- a14 -- */

/* Greedy decode loop (model card "Inference" step 6; the README's vLLM
 * section names <|im_end|> as the stop token): starting from token_ids [B]
 * (device) at positions cache_position [host][B] (updated in place), run up
 * to max_steps steps of ark_decode_step -> ark_masked_argmax ->
 * ark_cache_write, all sequences in lockstep (every position advances by
 * one per step).  Step t writes its B chosen ids to out_tokens[t][B]
 * (device).  A sequence finishes when it emits end_id; from then on its ids
 * are reported (and fed back) as end_id.  The loop stops when every
 * sequence has finished, when the next step would pass the end of the
 * cache, or after max_steps.  Returns the number of steps run (>= 0) or an
 * error code.  token_ids ends holding the last step's ids.  logits:
 * [B][vocab] (last step's logits on return).  mask: [vocab] uint8.
 * check_every (>= 1): the host reads the finished flags every this many
 * steps; larger values avoid a host round trip per step but may run up to
 * check_every - 1 steps after the last sequence finished. */
int ark_greedy_decode(const ark_model* m, int32_t B, int32_t* token_ids,
                      int32_t* cache_position, float* const* k_cache,
                      float* const* v_cache, float* k_delta, float* v_delta,
                      float* logits, const uint8_t* mask, int32_t end_id,
                      int32_t max_steps, int32_t check_every, int32_t* out_tokens,
                      void* workspace, size_t workspace_bytes, void* stream);

/* --------------------------------------------------------- test access -- */

/* Dynamic quantisation of B tensors x[b] of R*K fp32 values each (one
 * (s, z) per tensor; model card "Files": activations quantised at run
 * time), with the kernels of the prefill path.  codes [B][R][K] uint8,
 * scale [B] fp32, zp [B] int32.  B <= 64.  workspace >=
 * ark_test_dynquant_workspace_bytes() bytes.  Errors: ARK_E_NULL,
 * ARK_E_SHAPE, ARK_E_WORKSPACE. */
size_t ark_test_dynquant_workspace_bytes(void);
int ark_test_dynquant(int32_t B, int32_t R, int32_t K, const float* x, uint8_t* codes,
                      float* scale, int32_t* zp, void* workspace, size_t workspace_bytes,
                      void* stream);

/* One int8 MatMul on given codes: rows r of sequence b = r / R use (scale[b],
 * zp[b]).  codes [B*R][W->k] uint8; acc [B*R][W->n] int32 (or NULL): the
 * exact sum_k (code - zp) * w; y [B*R][W->n] fp32 dequantised output with
 * bias.  use_gemm selects the kernel: 0 the decode GEMV (requires B*R <= 4);
 * 1 the matrix-core GEMM as the decoder dispatches it (few-row kernel, one
 * pass per 64 rows, for B*R < 128 and W->k % 128 == 0, large-tile kernel for
 * B*R >= 128, tiled kernel otherwise); 2 the tiled kernel for any B*R.  workspace >=
 * ark_test_qlinear_workspace_bytes(B*R, W->k, use_gemm).  Errors: ARK_E_NULL,
 * ARK_E_SHAPE, ARK_E_WORKSPACE. */
size_t ark_test_qlinear_workspace_bytes(int32_t rows, int32_t k, int32_t use_gemm);
int ark_test_qlinear(int32_t B, int32_t R, const uint8_t* codes, const float* scale,
                     const uint8_t* zp, const ark_qlinear* W, int32_t* acc, float* y,
                     int32_t use_gemm, void* workspace, size_t workspace_bytes,
                     void* stream);

/* The MLP gate's elementwise part as the GEMM epilogues compute it (cookbook
 * "ARK-ASR-3B" introduction: Qwen2 MLP, silu(g) * u = g / (1 + e^-g) * u),
 * in fp64 and rounded once to fp32: y[i] for g[i], u[i], i < n, all three
 * fp32 device arrays of n elements (n == 0: nothing is read or written).
 * Errors: ARK_E_SHAPE (n < 0), ARK_E_NULL. */
int ark_test_swiglu(int64_t n, const float* g, const float* u, float* y, void* stream);

/* SwiGLU half of the MLP on given codes, as the prefill runs it (cookbook
 * "ARK-ASR-3B" introduction: Qwen2 MLP; model card "Files": int8 MatMuls on
 * dynamically quantised activations): y = silu(gate(x)) * up(x) with rows r
 * of sequence b = r / R using (scale[b], zp[b]) for both products, plus the
 * per-sequence min / max of y that the next dynamic quantisation takes
 * (produced inside the GEMM where the dispatch allows it).  codes
 * [B*R][k] uint8; gate, up: [n][k] with equal shapes, k % 64 == 0; y
 * [B*R][n] fp32; seq_min, seq_max [B] fp32.  B <= 64.  workspace >=
 * ark_test_gate_up_workspace_bytes(B, R, k).  Errors: ARK_E_NULL,
 * ARK_E_SHAPE, ARK_E_WORKSPACE. */
size_t ark_test_gate_up_workspace_bytes(int32_t B, int32_t R, int32_t k);
int ark_test_gate_up(int32_t B, int32_t R, const uint8_t* codes, const float* scale,
                     const uint8_t* zp, const ark_qlinear* gate, const ark_qlinear* up, float* y,
                     float* seq_min, float* seq_max, void* workspace, size_t workspace_bytes,
                     void* stream);

/* Full-cache GQA attention of B sequences of S rows, as the decoder runs it
 * (model card "ark-asr-3b-onnx", section "Shapes": row i of sequence b
 * sits at cache_position[b] + i and sees every cache row up to its own,
 * rows [p, p + S) taken from this call's deltas), plus the per-sequence
 * min / max of the output.  head_dim 128, n_heads / n_kv_heads <= 8, T a
 * multiple of 32 up to 8192; q [B*S][n_heads*128]; k_cache,
 * v_cache [B][T][n_kv_heads][128]; k_delta, v_delta [B*S][n_kv_heads][128];
 * out [B*S][n_heads*128] fp32; seq_min, seq_max [B].  cache_position is
 * host memory.  workspace >= ark_test_attention_workspace_bytes(B, S,
 * n_heads, T).  Errors: ARK_E_NULL, ARK_E_SHAPE, ARK_E_RANGE (a sequence
 * that does not fit in T), ARK_E_WORKSPACE. */
size_t ark_test_attention_workspace_bytes(int32_t B, int32_t S, int32_t n_heads, int32_t T);
int ark_test_attention(int32_t B, int32_t S, int32_t n_heads, int32_t n_kv_heads, int32_t T,
                       const int32_t* cache_position, const float* q, const float* k_cache,
                       const float* v_cache, const float* k_delta, const float* v_delta,
                       float* out, float* seq_min, float* seq_max, void* workspace,
                       size_t workspace_bytes, void* stream);

/* ------------------------------------------------- instrumentation ---- */

/* Benchmark instrumentation of the decode step's dominant kernel (the
 * kernel that moves most of a bs1 decode token's bytes; its name is
 * returned by ark_dominant_kernel()).  While armed, the library records
 * events[2i] / events[2i+1] (caller-created hipEvent_t, passed as void*)
 * on the launch stream immediately before / after the i-th launch of that
 * kernel, for i < n_pairs; ark_profile_arm(NULL, 0) disarms (the count of
 * recorded launches is kept until the next arming).  Process-wide state, not
 * thread-safe: for benchmarks only.  Errors: ARK_E_SHAPE. */
int ark_profile_arm(void* const* events, int32_t n_pairs);
/* Launches recorded since the last arming. */
int32_t ark_profile_count(void);
/* Name of the instrumented kernel (static storage). */
const char* ark_dominant_kernel(void);

/* Diagnostics of the persistent batch-1 decode kernel: when the environment
 * variable ARK_MEGA_TRACE is "1", each decode step records 100 MHz
 * real-time-counter stamps at its phase boundaries (workgroups 0, 1 and 255;
 * uint64 [3][n_layers + 1][16]) at this byte offset of the workspace.
 * 0 if the dims are invalid. */
size_t ark_decode_trace_offset(const ark_dims* d);

#ifdef __cplusplus
}
#endif

#endif /* ARK_H */
