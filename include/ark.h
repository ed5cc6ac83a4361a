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
 *   - section "Revision history": fp16 embedding table, int8 LM head, and a
 *     weight-only int4 LM tier (ark_qlinear4; its format is a reading, stated
 *     at ark_prep_weight_int4).
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
 *     memory; the library allocates no device memory.  State kept between
 *     calls lives in the caller's workspace (the persistent decode kernel's
 *     exchange area, its launch counter and error word), except for
 *     process-wide one-time kernel set-up (guarded, thread-safe) and the
 *     benchmark instrumentation of ark_profile_arm (not thread-safe).
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
  ARK_E_ALIGN = -6,       /* a pointer is not aligned as documented */
  ARK_E_TIMEOUT = -7,     /* a bounded wait of the persistent batch-1 decode
                             kernel gave up: the outputs of that step (and of
                             every greedy step fed from it) are invalid */
  ARK_E_NOALLOC = -8      /* ark_decode_step_noalloc: the call needs more
                             scratch than ark_noalloc_max_bytes() */
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

/* The weight-only int4 LM head W[n][k] (model card "ark-asr-3b-onnx",
 * "Revision history": the int4 LM tier), prepared by ark_prep_weight_int4.
 * Blocks of 128 consecutive weights along k; k % 256 == 0.  All arrays
 * 16-byte aligned. */
typedef struct {
  const uint8_t* w;       /* [n][k/2] uint4 codes, two per byte: byte i of a
                             row holds k = 2i (low nibble) and 2i + 1 (high) */
  const float* scale;     /* [n][k/128] fp32 scale per block */
  const uint8_t* zp;      /* [n][k/256] uint4 zero points, two per byte:
                             byte j holds block 2j (low nibble) and 2j + 1 */
  int32_t n, k;
} ark_qlinear4;

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
  ark_qlinear4 lm_head4;      /* [vocab][hidden] int4 tier; w == NULL: none.
                                 At most one of lm_head and lm_head4 is set;
                                 with lm_head4 the LM head multiplies the
                                 final-normed fp32 rows (not quantised) by
                                 the dequantised int4 weights */
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

/* Quantise an fp32 weight W[n][k] (device) into the int4 LM tier's blocks
 * (model card "ark-asr-3b-onnx", "Revision history"; the page names the
 * tier, not its format).  Reading: each block of 128 weights along k is
 * quantised like an activation tensor with 15 levels -- range widened to
 * include 0, s = (max - min) / 15, z = sat(rne(-min / s)) in [0, 15],
 * q = sat(rne(w / s) + z) in [0, 15], fp32 with correctly rounded division;
 * a block of zeros gets s = 0, z = 0, codes 0.  The weights multiplied are
 * w' = fp32((q - z) * s).  Outputs as ark_qlinear4 describes (codes
 * [n][k/2], scale [n][k/128], zp [n][k/256]); k % 256 == 0, all pointers
 * 16-byte aligned.  Errors: ARK_E_NULL, ARK_E_SHAPE, ARK_E_ALIGN. */
int ark_prep_weight_int4(const float* w, int32_t n, int32_t k, uint8_t* codes, float* scale,
                         uint8_t* zp, void* stream);

/* The weight-only int4 LM head on B given rows: logits[b][j] =
 * sum_i h[b][i] w'[j][i] in fp32 arithmetic.  The order of the sums, and at
 * k == 2048 the form s (sum h q - z sum h) per 32-weight chunk, are the
 * kernel's; the result lies within (32 ceil(k / 2048) + 12) u
 * sum_i s_i |h[b][i]| (q_i + z_i) of the exact sum (u = 2^-24; s, q, z of
 * weight i's block).  h:
 * [B][ldh] fp32 (the final-normed last rows; the decoder calls this after
 * its final RMSNorm); logits: [B][ldl].  1 <= B <= 64, ldh >= k, ldl >= n,
 * h 16-byte aligned.  Errors: ARK_E_NULL, ARK_E_SHAPE, ARK_E_ALIGN,
 * ARK_E_HIP. */
int ark_lm_head_int4(int32_t B, const float* h, int32_t ldh, const ark_qlinear4* W,
                     float* logits, int32_t ldl, void* stream);

/* Rotary tables: cos/sin[pos][j] of pos * theta^(-2j/head_dim), fp64, for
 * pos < T and j < head_dim/2.  Errors: ARK_E_NULL, ARK_E_SHAPE. */
int ark_rope_table(int32_t T, int32_t head_dim, double theta, double* cos_out,
                   double* sin_out, void* stream);

/* ------------------------------------------------------ audio adapter -- */

/* The frame-merging int8 MLP adapter in front of the decoder (model card
 * "ark-asr-3b-onnx", "Inference" steps 2-3: the encoder output cut to a
 * multiple of `merge` frames, every `merge` consecutive frames side by side
 * in one row, the adapter mapping the rows to the decoder's width; "Files":
 * its MatMuls are int8 with dynamic activations; Audio8 article, "What
 * arkasr actually is": two linear layers with biases).  Readings (the
 * pages give no 3B widths and no activation): up is [inner][merge *
 * frame_dim] with inner = 4096 for the ARK geometry, then the erf GELU
 * x Phi(x) computed in fp64 and rounded once to fp32, then down
 * [hidden][inner]; each of the two quantisation points takes one (s, z)
 * per sequence, as in the decoder.  Both projections carry a bias. */
typedef struct {
  ark_qlinear up;       /* [inner][merge * frame_dim], bias [inner] */
  ark_qlinear down;     /* [hidden][inner], bias [hidden] */
  int32_t frame_dim;    /* encoder output width (1280) */
  int32_t merge;        /* frames per merged row (4) */
} ark_adapter;

/* Workspace bytes of ark_audio_adapter for B sequences of `frames` encoder
 * frames each; 0 if the arguments are invalid. */
size_t ark_adapter_workspace_bytes(const ark_adapter* A, int32_t B, int32_t frames);

/* Adapter rows of B sequences: enc [B][frames][frame_dim] fp32 (sequence b
 * at enc + b * frames * frame_dim); n = frames / merge rows per sequence
 * (trailing frames dropped, n >= 1); out [B][n][hidden] fp32, the rows
 * ark_embed_splice writes into the <|audio|> slots; mid (optional, NULL:
 * not written) [B][n][inner] fp32, the GELU output that the second
 * quantisation sees.  1 <= B <= 64; up.k == merge * frame_dim, up.n ==
 * down.k, both with a bias, k % 64 == 0; pointers 16-byte aligned,
 * workspace 256-byte aligned.  Errors: ARK_E_NULL, ARK_E_SHAPE,
 * ARK_E_WORKSPACE, ARK_E_ALIGN, ARK_E_HIP. */
int ark_audio_adapter(const ark_adapter* A, int32_t B, int32_t frames, const float* enc,
                      float* out, float* mid, void* workspace, size_t workspace_bytes,
                      void* stream);

/* ------------------------------------------------------ audio encoder -- */

/* The Whisper-style audio encoder in front of the adapter (model card
 * "ark-asr-3b-onnx", "Inference" step 1: log-mel features to [1, seq, 1280];
 * "Files": dynamically quantised int8 with per-channel MatMul weights;
 * cookbook "ARK-ASR-3B" introduction: a Whisper-style tower with rotary
 * self-attention; Audio8 article, "What arkasr actually is": 636,968,960
 * parameters, the Whisper large encoder's count).  Per clip:
 *   a = GELU(conv1(mel))            width 3, stride 1, padding 1, + bias
 *   x = GELU(conv2(a)) + pos[t]     width 3, stride 2, padding 1, + bias
 *   32 x: x += o(attn(rope(q), rope(k), v))   of LayerNorm1(x)
 *         x += fc2(GELU(fc1(LayerNorm2(x))))
 *   out = LayerNorm_f(x)
 * Readings (the pages fix the structure by its parameter count, not these):
 * 20 heads of 64; q, v, o, fc1, fc2 and the convolutions carry biases, k
 * does not; rotary embedding (rotate-half, pairs (d, d + 32), the tables
 * of ark_rope_table(max_pos, 64, theta)) on q and k at positions 0..F-1 in
 * every layer, in addition to the positional rows; attention is
 * bidirectional with scores q.k / 8; every MatMul and both convolutions
 * are int8 with one (s, z) per clip and quantisation point (the
 * convolutions as GEMMs over tap-major im2col rows); LayerNorm, rotary
 * embedding, softmax and GELU (erf form) compute in fp64 and round once to
 * fp32.  Convolution weights are stored tap-major: conv1 is [d][3 n_mels]
 * with element (j, c) = tap j of input channel c (a transpose of the usual
 * [d][n_mels][3]), conv2 [d][3 d] likewise. */
typedef struct {
  const float* ln1_g;
  const float* ln1_b;
  const float* ln2_g;
  const float* ln2_b;
  ark_qlinear q, k, v, o;   /* [d][d]; k without bias */
  ark_qlinear fc1;          /* [ffn][d] */
  ark_qlinear fc2;          /* [d][ffn] */
} ark_enc_layer;

typedef struct {
  int32_t n_mels, d_model, n_heads, ffn, n_layers, max_pos;
  double ln_eps;               /* LayerNorm epsilon (1e-5) */
  ark_qlinear conv1;           /* [d][3 n_mels], bias [d] */
  ark_qlinear conv2;           /* [d][3 d], bias [d] */
  const float* pos;            /* [max_pos][d] positional rows */
  const ark_enc_layer* layers; /* [host] n_layers entries */
  const float* lnf_g;          /* [d] final LayerNorm */
  const float* lnf_b;
  const double* rope_cos;      /* [max_pos][32] from ark_rope_table(max_pos, 64, theta) */
  const double* rope_sin;
} ark_encoder;

/* Workspace bytes of ark_audio_encoder for B clips of M mel frames each; 0
 * if the arguments are invalid. */
size_t ark_encoder_workspace_bytes(const ark_encoder* E, int32_t B, int32_t mel_frames);

/* Encoder frames of B clips: mel [B][M][n_mels] fp32 (time-major log-mel
 * features); out [B][F][d_model] fp32 with F = (M - 1) / 2 + 1 <= max_pos
 * (the adapter's input).  Supported: d_model == 64 n_heads, n_mels % 64 ==
 * 0, ffn % 64 == 0, 1 <= B <= 64, B * M <= 2^24;
 * pointers 16-byte aligned, workspace 256-byte aligned.  Errors:
 * ARK_E_NULL, ARK_E_SHAPE, ARK_E_WORKSPACE, ARK_E_ALIGN, ARK_E_HIP. */
int ark_audio_encoder(const ark_encoder* E, int32_t B, int32_t mel_frames, const float* mel,
                      float* out, void* workspace, size_t workspace_bytes, void* stream);

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
 * errors as ark_prefill with S = 1.  At B = 1 with the ARK geometry the
 * step is one persistent kernel (ark_decode_path) whose 256 workgroups, one
 * per CU, exchange data through bounded waits; the return value reports
 * only the launch, so a caller that needs to know that every wait was met
 * calls ark_decode_check afterwards.  The kernel is launched as an ordinary
 * kernel: its workgroups are all resident at once when no kernel on
 * another stream holds CUs, and one held longer than the wait bound ends
 * the step with ARK_E_TIMEOUT.  The environment variable ARK_DECODE_LAUNCH
 * set to "cooperative" selects a cooperative launch, which guarantees
 * residency at a cost of about 20 us per step. */
int ark_decode_step(const ark_model* m, int32_t B, const int32_t* token_ids,
                    const int32_t* cache_position, const float* const* k_cache,
                    const float* const* v_cache, float* k_delta, float* v_delta,
                    float* logits, float* hidden_out, void* workspace,
                    size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * step as ark_decode_step, with the library's own scratch in place of the
 * workspace.  The scratch is one static device array per GPU of
 * ark_noalloc_max_bytes() bytes (64 MiB), held until the process ends; its
 * address is resolved on the first call on each device.  The call
 * allocates nothing.  A call whose ark_workspace_bytes(&m->d, B, 1) exceeds
 * that size returns ARK_E_NOALLOC (the ARK geometry at T = 512 needs at
 * most about 36 MiB: 34.6 MiB at B = 1, 9-36 MiB at 2 <= B <= 64).  Every call on a GPU shares
 * that GPU's array and it keeps the last call's contents (the step clears
 * what must start at zero): calls that overlap on one GPU - concurrent
 * streams or threads - race and give undefined results.  Status of a
 * persistent-kernel step: ark_decode_check is not available (no workspace);
 * use ark_decode_step when the time-out status is needed.  Other arguments
 * and errors as ark_decode_step. */
size_t ark_noalloc_max_bytes(void);
int ark_decode_step_noalloc(const ark_model* m, int32_t B, const int32_t* token_ids,
                            const int32_t* cache_position, const float* const* k_cache,
                            const float* const* v_cache, float* k_delta, float* v_delta,
                            float* logits, float* hidden_out, void* stream);

/* Status of the last decode step enqueued on this workspace for B
 * sequences: synchronises `stream`, then returns ARK_E_TIMEOUT if the
 * persistent kernel (ark_decode_path(m, B) == 1) had a wait give up, else
 * ARK_OK (the multi-kernel path has no bounded waits).  Errors: ARK_E_NULL,
 * ARK_E_SHAPE, ARK_E_WORKSPACE, ARK_E_HIP. */
int ark_decode_check(const ark_model* m, int32_t B, const void* workspace,
                     size_t workspace_bytes, void* stream);

/* Which decode path ark_decode_step / ark_greedy_decode take for B
 * sequences: 1 = the persistent batch-1 kernel, 0 = the multi-kernel path;
 * negative: ARK_E_NULL / ARK_E_SHAPE.  (The environment variable
 * ARK_DECODE_PATH=multi forces the multi-kernel path.) */
int ark_decode_path(const ark_model* m, int32_t B);

/* ----------------------------------------------------------------- a12 -- */

/* Masked greedy argmax (model card "Inference" step 6; cookbook "Marker-
 * Token Suppression"): out_ids[b] = the lowest id v with mask[v] == 0 whose
 * logit is the maximum over unmasked ids; NaN logits are never chosen; -1 if
 * no id qualifies.  logits [B][V] fp32, mask [V] uint8 (1 = masked),
 * out_ids [B] int32.  Errors: ARK_E_NULL, ARK_E_SHAPE. */
int ark_masked_argmax(int32_t B, int32_t V, const float* logits, const uint8_t* mask,
                      int32_t* out_ids, void* stream);

/* ----------------------------------------------- bf16 serving variant -- */

/* The decoder in bf16 (cookbook "ARK-ASR-3B", "dtype": bfloat16 is the
 * default serving dtype): the checkpoint's weights, every activation and
 * the KV cache in bf16 (IEEE bfloat16 bits in uint16_t), half the cache
 * bytes of the fp32 path.  Each operation rounds its output once to bf16
 * (nearest even): RMSNorm bf16(g * bf16(x / rms)), linear bf16(x W^T + b),
 * the rotated q and k, attention bf16(softmax(q.k / sqrt(128)) v),
 * residual adds, the MLP gate bf16(bf16(silu(g)) * u); the logits are the
 * fp32 sums of the final-normed row with the head's rows.  Sums run in fp32
 * (matrix cores, attention) or fp64 (norm statistics, rotary step), so
 * results match a reference that rounds at the same points within bf16
 * rounding (2e-2 relative, the serving dtype's tolerance).  Same geometry,
 * cache contract and workspace rules as the int8 path. */
typedef struct {
  const uint16_t* w;     /* [n][k] bf16 */
  const uint16_t* bias;  /* [n] bf16 or NULL (q, k, v only) */
  int32_t n, k;
} ark_linear_bf16;

typedef struct {
  const uint16_t* ln1;   /* [hidden] bf16 gains */
  const uint16_t* ln2;
  ark_linear_bf16 q, k, v, o, gate, up, down;
} ark_layer_bf16;

typedef struct {
  ark_dims d;
  const ark_layer_bf16* layers;  /* [host] d.n_layers entries */
  const uint16_t* final_norm;    /* [hidden] bf16 */
  ark_linear_bf16 lm_head;       /* [vocab][hidden]; w == NULL: none */
  const uint16_t* embed;         /* [vocab][hidden] bf16 */
  const double* rope_cos;        /* as ark_model */
  const double* rope_sin;
} ark_model_bf16;

/* fp32 -> bf16 (nearest even; NaN stays NaN) of n values (weights, inputs).
 * Errors: ARK_E_NULL, ARK_E_SHAPE (n < 0), ARK_E_HIP. */
int ark_to_bf16(const float* x, int64_t n, uint16_t* out, void* stream);

/* Workspace bytes of ark_prefill_bf16 / ark_decode_step_bf16 for B
 * sequences of S rows; 0 if the dims are invalid. */
size_t ark_workspace_bytes_bf16(const ark_dims* d, int32_t B, int32_t S);

/* Prefill of B sequences of S bf16 rows, the bf16 counterpart of
 * ark_prefill: embeds [B][S][hidden] bf16; k_cache, v_cache [host][L] of
 * [B][T][n_kv][128] bf16 (read only); k_delta, v_delta
 * [L][B][S][n_kv][128] bf16 out; logits [B][vocab] fp32 or NULL;
 * hidden_out [B][S][hidden] bf16 or NULL.  1 <= B <= 64.  Errors as
 * ark_prefill. */
int ark_prefill_bf16(const ark_model_bf16* m, int32_t B, int32_t S, const uint16_t* embeds,
                     const int32_t* cache_position, const uint16_t* const* k_cache,
                     const uint16_t* const* v_cache, uint16_t* k_delta, uint16_t* v_delta,
                     float* logits, uint16_t* hidden_out, void* workspace,
                     size_t workspace_bytes, void* stream);

/* One decode step of the bf16 variant: token_ids [B] gathered from
 * m->embed, then as ark_prefill_bf16 with S = 1. */
int ark_decode_step_bf16(const ark_model_bf16* m, int32_t B, const int32_t* token_ids,
                         const int32_t* cache_position, const uint16_t* const* k_cache,
                         const uint16_t* const* v_cache, uint16_t* k_delta, uint16_t* v_delta,
                         float* logits, uint16_t* hidden_out, void* workspace,
                         size_t workspace_bytes, void* stream);

/* ark_cache_write for the bf16 caches and deltas. */
int ark_cache_write_bf16(const ark_dims* d, int32_t B, int32_t S, const int32_t* cache_position,
                         uint16_t* const* k_cache, uint16_t* const* v_cache,
                         const uint16_t* k_delta, const uint16_t* v_delta, void* stream);

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
 * check_every - 1 steps after the last sequence finished.  On the
 * persistent path the kernel's error word is cleared once per call and read
 * at the same points and at the end: a wait that timed out in any step
 * returns ARK_E_TIMEOUT instead of a count.  On that path the write-back,
 * the stop rule and the next step's preparation run as one small kernel
 * between two persistent launches. */
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
/* The audio encoder's LayerNorm on B sequences of S rows of D values
 * (fp64 inside, one rounding): y [B][S][D] and each sequence's (min, max)
 * of y in lo[B], hi[B] (the range its dynamic quantisation takes).
 * workspace >= ark_test_dynquant_workspace_bytes().  Errors: ARK_E_NULL,
 * ARK_E_SHAPE, ARK_E_WORKSPACE, ARK_E_HIP. */
int ark_test_layernorm(int32_t B, int32_t S, int32_t D, const float* x, const float* g,
                       const float* b, double eps, float* y, float* lo, float* hi,
                       void* workspace, size_t workspace_bytes, void* stream);

/* The audio encoder's rotary bidirectional self-attention on B clips of F
 * frames and H heads of 64: qkv [B][F][3 H 64] (q | k | v rows as the
 * projections write them), rotary tables [>= F][32] fp64; out [B][F][H 64]
 * and each clip's (min, max) of out in lo[B], hi[B].  workspace >=
 * ark_test_dynquant_workspace_bytes(); with
 * ark_test_enc_attention_workspace_bytes(B, F, H) bytes a launch of few
 * workgroups takes the split form ark_audio_encoder uses (key chunks over
 * several workgroups, then a merge).  Errors: ARK_E_NULL, ARK_E_SHAPE,
 * ARK_E_WORKSPACE, ARK_E_HIP. */
size_t ark_test_enc_attention_workspace_bytes(int32_t B, int32_t F, int32_t H);
int ark_test_enc_attention(int32_t B, int32_t F, int32_t H, const float* qkv,
                           const double* rope_cos, const double* rope_sin, float* out, float* lo,
                           float* hi, void* workspace, size_t workspace_bytes, void* stream);

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
 * real-time-counter stamps at this byte offset of the workspace: uint64
 * [3][n_layers + 1][32] (workgroups 0, 1 and 255: events 0..15 at the
 * phase boundaries of every layer, 16..31 inside phases), then uint64
 * [256][16] (every workgroup, for layer 2 only).  0 if the dims are
 * invalid.  The test-only environment variable ARK_TEST_SPIN_LIMIT (rounds,
 * >= 0) replaces the bound of the kernel's waits; 0 makes every wait give
 * up at once (the kernel still runs to completion, and the step reports
 * ARK_E_TIMEOUT through ark_decode_check / ark_greedy_decode). */
size_t ark_decode_trace_offset(const ark_dims* d);

/* ------------------------------------------- re-anchored parity record --
 * Test access (the parity protocol "bit-exact codes on the GPU's own
 * tensors"): the dump variants of prefill and decode run the same kernels
 * as ark_prefill / ark_decode_step (the persistent decode kernel as an
 * instantiation that also stores its record) and also write, for every
 * layer l whose bit is set in layer_mask, one record of the tensors each
 * of the layer's four dynamic quantisations saw and produced (model card
 * "Files": int8 MatMuls on activations quantised at run time), and, when
 * logits are requested, one record of the LM head's input quantisation.
 * Layer records follow each other in increasing l, then the head record;
 * every field starts 256-byte aligned at the offsets ark_dump_layout
 * gives.  R = B * S rows, row r of sequence r / S.  Codes are stored as
 * int8 (code - 128).  s / z: [4][B], point order h1, attention, h2, SwiGLU. */
enum ark_dump_field {
  ARK_DUMP_H1 = 0,    /* f32 [R][hidden]  RMSNorm 1 output (quantised for q|k|v) */
  ARK_DUMP_QKV = 1,   /* f32 [R][q+2kv]   q|k|v projections with bias, before rotary */
  ARK_DUMP_ATTN = 2,  /* f32 [R][q]       attention output (quantised for o) */
  ARK_DUMP_X1 = 3,    /* f32 [R][hidden]  x + o */
  ARK_DUMP_H2 = 4,    /* f32 [R][hidden]  RMSNorm 2 output (quantised for gate|up) */
  ARK_DUMP_A = 5,     /* f32 [R][inter]   SwiGLU output (quantised for down) */
  ARK_DUMP_X2 = 6,    /* f32 [R][hidden]  x1 + down: the layer's output */
  ARK_DUMP_C1 = 7,    /* i8  [R][hidden]  codes of h1 */
  ARK_DUMP_C2 = 8,    /* i8  [R][q]       codes of the attention output */
  ARK_DUMP_C3 = 9,    /* i8  [R][hidden]  codes of h2 */
  ARK_DUMP_C4 = 10,   /* i8  [R][inter]   codes of the SwiGLU output */
  ARK_DUMP_S = 11,    /* f32 [4][B]       scales */
  ARK_DUMP_Z = 12,    /* i32 [4][B]       zero points */
  ARK_DUMP_NFIELDS = 13
};
/* Head record: f32 [B][hidden] final-norm output of each last row, i8
 * [B][hidden] its codes, f32 [B] scales, i32 [B] zero points. */

/* Bytes of the record for B sequences of S rows with the layers of
 * layer_mask (bits >= n_layers ignored); fills field_off[ARK_DUMP_NFIELDS]
 * (offsets inside a layer record), *record_bytes (one layer record) and
 * head_off[4] (absolute offsets of the head fields) when not NULL.  0 if the
 * dims or sizes are invalid. */
size_t ark_dump_layout(const ark_dims* d, int32_t B, int32_t S, uint64_t layer_mask,
                       size_t* field_off, size_t* record_bytes, size_t* head_off);

/* ark_prefill / ark_decode_step plus the record described above, written to
 * dump (device, 256-byte aligned, >= ark_dump_layout(...) bytes).  Errors
 * as the plain calls, plus ARK_E_WORKSPACE when dump_bytes is too small. */
int ark_prefill_dump(const ark_model* m, int32_t B, int32_t S, const float* embeds,
                     const int32_t* cache_position, const float* const* k_cache,
                     const float* const* v_cache, float* k_delta, float* v_delta,
                     float* logits, float* hidden_out, void* workspace,
                     size_t workspace_bytes, void* stream, void* dump, size_t dump_bytes,
                     uint64_t layer_mask);
int ark_decode_step_dump(const ark_model* m, int32_t B, const int32_t* token_ids,
                         const int32_t* cache_position, const float* const* k_cache,
                         const float* const* v_cache, float* k_delta, float* v_delta,
                         float* logits, float* hidden_out, void* workspace,
                         size_t workspace_bytes, void* stream, void* dump,
                         size_t dump_bytes, uint64_t layer_mask);

#ifdef __cplusplus
}
#endif

#endif /* ARK_H */
