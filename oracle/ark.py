"""Plain, slow CPU oracle of the ARK-ASR-3B int8 decoder step (numpy only).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages cited (by title and section):
  [card]   model card "ark-asr-3b-onnx": sections "Files" (int8 dynamic
           quantisation, per-channel MatMul weights), "Shapes" (geometry,
           static cache, deltas), "Inference" (prompt, slot count, masked
           greedy loop), "Revision history" (fp16 table, int8 LM head, the
           weight-only int4 LM tier).
  [cook]   sglang-omni cookbook "ARK-ASR-3B": intro (Qwen2 decoder), "Audio
           Handling" (token count), "Marker-Token Suppression" (mask set).
  [readme] "ARK-ASR-3B" README: "vLLM" section (<|im_end|> is the stop token).
  [audio8] article "Audio8: eight checkpoints, one broken link, and a 3B
           model with nowhere to ship": "What arkasr actually is" (the
           frame-merging MLP adapter, the Whisper-style encoder with
           RoPE-augmented layers, their parameter counts at 0.6B).
  [clover] article "Inside ARK-ASR-3B's Whisper and Qwen architecture"
           (a Whisper-style audio encoder with rotary position embeddings).
  [cook]   also "dtype": the default serving dtype is bfloat16 (the
           bf16-activation decoder variant at the end of this file).

Numeric conventions of this oracle (readings of what the pages leave open):
  * Tensors between operations are fp32, as in the card's fp32 ONNX graph.
  * Integer contractions are exact: int8 operands are widened to float64 and
    multiplied with BLAS; |acc| <= 255*127*11008 < 2**53, so every partial
    sum is an exactly representable integer whatever the summation order.
  * Dynamic quantisation and dequantisation use fp32 arithmetic exactly as
    written (correctly rounded division, round-half-to-even).
  * Normalisation, RoPE, attention and SwiGLU compute in float64 and round
    their outputs to fp32 once.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "n_audio_slots", "n_audio_slots_from_mel", "prep_weight", "dynquant",
    "matmul_integer", "dequant", "qlinear", "rmsnorm", "rope_tables",
    "apply_rope", "attention", "swiglu", "masked_argmax", "cache_write",
    "embed_splice", "embed_ids", "OracleLayer", "OracleModel", "build_model",
    "layer_forward", "forward", "prefill", "decode_step", "layer_param_count",
    "INT4_BLOCK", "prep_weight_int4", "dequant_weight_int4", "lm_head_int4",
    "int4_size_ratio", "MERGE", "n_encoder_frames", "frame_merge", "gelu",
    "OracleAdapter", "build_adapter", "adapter", "adapter_param_count",
    "ENC_LN_EPS", "ENC_ROPE_THETA", "encoder_param_count", "layernorm", "conv_out_len",
    "im2col", "enc_attention", "OracleEncLayer", "OracleEncoder", "build_encoder",
    "encoder_forward", "bf16_round", "Bf16Layer", "Bf16Model", "build_bf16_model",
    "bf16_rmsnorm", "bf16_linear", "bf16_layer_forward", "bf16_forward", "bf16_prefill",
    "bf16_decode_step",
]

F32 = np.float32
F64 = np.float64


# ----------------------------------------------------------- audio slots --
def n_audio_slots(samples: int) -> int:
    """Number of <|audio|> slots for a clip of `samples` 16 kHz samples.

    [card] "Inference", step 4: N = max(((samples // 160) + 1) // 2 // 4, 1).
    """
    return max(((int(samples) // 160) + 1) // 2 // 4, 1)


def n_audio_slots_from_mel(mel_frames: int, merge_factor: int = 4) -> int:
    """[cook] "Audio Handling": (mel_frames + 1) // 2 // merge_factor."""
    return (int(mel_frames) + 1) // 2 // int(merge_factor)


# ------------------------------------------------------- weight quantiser --
def prep_weight(w: np.ndarray):
    """Symmetric int8 quantisation per output channel of a weight [n][k].

    [card] "Files": MatMul weights are int8 per channel.  Reading: scale
    s[n] = fp32(max_k |W[n,k]| / 127); code = clamp(rne(fp32(W / s)), -127,
    127); a zero row has s = 0 and codes 0.
    Returns (codes int8 [n][k], scale fp32 [n]).
    """
    w = np.asarray(w, F32)
    amax = np.max(np.abs(w), axis=1)
    s = (amax / F32(127.0)).astype(F32)
    safe = np.where(s > 0, s, F32(1.0)).astype(F32)
    q = np.rint((w / safe[:, None]).astype(F32))
    q = np.clip(q, -127, 127).astype(np.int8)
    q[s == 0] = 0
    return q, s


# ------------------------------------------------ weight-only int4 tier --
# [card] "Revision history": v2 added a weight-only int4 LM tier.  Reading
# (the page names the tier, not its format): the LM head's weights are
# stored as uint4 codes in blocks of INT4_BLOCK consecutive weights along K,
# each block with an fp32 scale and a uint4 zero point (the asymmetric block
# format of an ONNX 4-bit MatMul); "weight-only" means the activation stays
# fp32: logits = h . dequant(W4)^T with no activation quantisation.  The
# block is quantised like a dynamic activation tensor with 15 levels: range
# widened to include 0, s = (max - min) / 15, z = sat(rne(-min / s)),
# q = sat(rne(w / s) + z); a block of zeros has s = 0, z = 0, q = 0.
INT4_BLOCK = 128


def int4_size_ratio(block: int, zero_point: bool = True) -> float:
    """fp32 bytes over int4-tier bytes per weight: 4 bits per code plus one
    fp32 scale (and a 4-bit zero point) per block."""
    per = 0.5 + 4.0 / block + (0.5 / block if zero_point else 0.0)
    return 4.0 / per


def prep_weight_int4(w: np.ndarray, block: int = INT4_BLOCK):
    """uint4 codes [n][k] (one per byte here, values 0..15), scales
    fp32 [n][k / block], zero points uint8 [n][k / block] of W [n][k]."""
    w = np.asarray(w, F32)
    n, k = w.shape
    assert k % block == 0
    wb = w.reshape(n, k // block, block)
    lo = np.minimum(wb.min(axis=2), F32(0.0)).astype(F32)
    hi = np.maximum(wb.max(axis=2), F32(0.0)).astype(F32)
    s = ((hi - lo).astype(F32) / F32(15.0)).astype(F32)
    safe = np.where(s > 0, s, F32(1.0)).astype(F32)
    z = np.clip(np.rint((-lo / safe).astype(F32)), 0, 15)
    q = np.rint((wb / safe[:, :, None]).astype(F32)) + z[:, :, None].astype(F32)
    q = np.clip(q, 0, 15)
    q[s == 0] = 0
    z[s == 0] = 0
    return q.reshape(n, k).astype(np.uint8), s, z.astype(np.uint8)


def dequant_weight_int4(codes, scale, zp, block: int = INT4_BLOCK) -> np.ndarray:
    """w' = fp32((q - z) * s) per element (the weights the int4 tier
    multiplies)."""
    n, k = codes.shape
    qz = codes.reshape(n, k // block, block).astype(F32) - zp[:, :, None].astype(F32)
    return (qz * scale[:, :, None].astype(F32)).astype(F32).reshape(n, k)


def lm_head_int4(h: np.ndarray, codes, scale, zp, block: int = INT4_BLOCK) -> np.ndarray:
    """Weight-only int4 LM head: logits[b, n] = fp32(sum_k h[b, k] w'[n, k])
    with the products summed in float64 (one rounding to fp32).  h [B, K]
    fp32 (the final-normed last rows, not quantised)."""
    wd = dequant_weight_int4(codes, scale, zp, block).astype(F64)
    return (np.asarray(h, F32).astype(F64) @ wd.T).astype(F32)


# --------------------------------------------------- activation quantiser --
def dynquant(x: np.ndarray):
    """Dynamic per-tensor uint8 quantisation of one activation tensor.

    [card] "Files": activations are quantised at run time ("dynamically
    quantized" ONNX export).  Reading: ONNX DynamicQuantizeLinear in fp32 --
    the range is widened to include 0, s = (max - min) / 255,
    z = sat(rne(-min / s)), q = sat(rne(x / s) + z); an all-zero tensor has
    s = 0, z = 0 and codes 0.
    Returns (codes uint8 (shape of x), s fp32 scalar, z uint8 scalar).
    """
    x = np.asarray(x, F32)
    lo = min(F32(0.0), F32(x.min())) if x.size else F32(0.0)
    hi = max(F32(0.0), F32(x.max())) if x.size else F32(0.0)
    s = F32(F32(hi - lo) / F32(255.0))
    if s == 0:
        return np.zeros(x.shape, np.uint8), F32(0.0), np.uint8(0)
    z = np.clip(np.rint(F32(-lo) / s), 0, 255)
    q = np.rint((x / s).astype(F32)) + F32(z)
    q = np.clip(q, 0, 255).astype(np.uint8)
    return q, s, np.uint8(z)


# ------------------------------------------------------------ int8 linear --
def matmul_integer(codes: np.ndarray, z, wq: np.ndarray) -> np.ndarray:
    """acc[r, n] = sum_k (codes[r, k] - z) * wq[n, k], exact (int64).

    [card] "Files": int8 MatMuls.  Reading: ONNX MatMulInteger with the
    activation zero point subtracted and weight zero point 0.  Float64 BLAS
    on integer-valued operands is exact here (|acc| < 2**53).
    """
    a = codes.astype(F64) - F64(z)
    return (a @ wq.astype(F64).T).astype(np.int64)


def dequant(acc: np.ndarray, s, sw: np.ndarray, bias=None) -> np.ndarray:
    """y = fp32(fp32(acc) * fp32(s * sw[n])) (+ bias[n] in fp32).

    Reading of the int8 MatMul's float output: one fp32 multiplier per output
    channel (activation scale times weight scale), applied to the rounded
    accumulator, then the bias added in fp32.  No fused multiply-add.
    """
    facc = acc.astype(F64).astype(F32)            # exact int -> nearest fp32
    mult = (F32(s) * np.asarray(sw, F32)).astype(F32)
    y = (facc * mult).astype(F32)
    if bias is not None:
        y = (y + np.asarray(bias, F32)).astype(F32)
    return y


def qlinear(codes, s, z, wq, sw, bias=None) -> np.ndarray:
    """Dequantised output of one int8 MatMul (matmul_integer then dequant)."""
    return dequant(matmul_integer(codes, z, wq), s, sw, bias)


# ------------------------------------------------------------ float ops --
def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """Qwen2 RMSNorm over the last axis ([cook] intro: dense Qwen2 LM).

    y = x / sqrt(mean(x^2) + eps) * g, float64 inside, fp32 out.
    """
    x64 = np.asarray(x, F32).astype(F64)
    ms = np.mean(x64 * x64, axis=-1, keepdims=True)
    r = 1.0 / np.sqrt(ms + F64(eps))
    return ((x64 * r) * np.asarray(g, F32).astype(F64)).astype(F32)


def rope_tables(T: int, D: int, theta: float):
    """cos, sin of angle pos * theta^(-2j/D) for pos < T, j < D/2 (float64)."""
    j = np.arange(D // 2, dtype=F64)
    inv = np.power(F64(theta), -(2.0 * j) / F64(D))
    ang = np.arange(T, dtype=F64)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def apply_rope(x: np.ndarray, pos: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate-half rotary embedding (Qwen2 reading) on the last axis.

    x [..., D] fp32, pos broadcastable to x.shape[:-1].  Pairs (j, j + D/2)
    rotate by the angle of position pos:
      out[j]       = x[j] cos - x[j+D/2] sin
      out[j+D/2]   = x[j+D/2] cos + x[j] sin       (float64, fp32 out)
    """
    x64 = np.asarray(x, F32).astype(F64)
    h = x64.shape[-1] // 2
    c = cos[pos][..., None, :] if x64.ndim == pos.ndim + 2 else cos[pos]
    s = sin[pos][..., None, :] if x64.ndim == pos.ndim + 2 else sin[pos]
    a, b = x64[..., :h], x64[..., h:]
    out = np.concatenate([a * c - b * s, b * c + a * s], axis=-1)
    return out.astype(F32)


def attention(q: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray, p: int) -> np.ndarray:
    """GQA attention of one sequence over the whole static cache.

    [card] "Shapes": the decoder attends over ALL max_total_len positions on
    every token, however few are valid.  Query row i sits at position p + i
    and sees cache rows j <= p + i; every other row is masked (selected out,
    never multiplied, so its contents cannot leak).  q head h reads KV head
    h // (NH / NKV).  Scores are q.k / sqrt(D); softmax and the weighted sum
    in float64; fp32 out.

    q [S, NH, D]; k_hat, v_hat [T, NKV, D] (cache with this call's rows
    already replaced by the deltas).  Returns [S, NH * D] fp32.
    """
    S, NH, D = q.shape
    T, NKV, _ = k_hat.shape
    G = NH // NKV
    rows = p + np.arange(S)
    valid = np.arange(T)[None, :] <= rows[:, None]                 # [S, T]
    live = np.arange(T) < p + S                                    # rows any query may see
    out = np.empty((S, NH, D), F64)
    scale = 1.0 / np.sqrt(F64(D))
    for g in range(NKV):
        kg = np.where(live[:, None], k_hat[:, g, :].astype(F64), 0.0)   # [T, D]
        vg = np.where(live[:, None], v_hat[:, g, :].astype(F64), 0.0)
        for hh in range(G):
            h = g * G + hh
            sc = (q[:, h, :].astype(F64) @ kg.T) * scale               # [S, T]
            sc = np.where(valid, sc, -np.inf)
            m = np.max(sc, axis=1, keepdims=True)
            e = np.where(valid, np.exp(sc - m), 0.0)
            out[:, h, :] = (e @ vg) / np.sum(e, axis=1, keepdims=True)
    return out.reshape(S, NH * D).astype(F32)


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """Qwen2 MLP gate: silu(g) * u = g / (1 + exp(-g)) * u (float64, fp32 out)."""
    g64 = np.asarray(g, F32).astype(F64)
    return (g64 / (1.0 + np.exp(-g64)) * np.asarray(u, F32).astype(F64)).astype(F32)


# ---------------------------------------------------------- host-side ops --
def masked_argmax(logits: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """Greedy token per row with added-vocab ids masked.

    [card] "Inference" step 6: decode greedily, masking every <...> added
    token except <|im_end|>; [cook] "Marker-Token Suppression": masked ids
    can never be sampled.  Masked ids and NaN logits are never chosen; ties
    go to the lowest id; a row with no candidate returns -1.
    logits [B, V] fp32, mask [V] uint8 (1 = masked) -> int32 [B].
    """
    lg = np.asarray(logits, F32)
    out = np.empty(lg.shape[0], np.int32)
    ok = (np.asarray(mask) == 0)[None, :] & ~np.isnan(lg)
    for b in range(lg.shape[0]):
        cand = np.nonzero(ok[b])[0]
        if cand.size == 0:
            out[b] = -1
            continue
        vals = lg[b, cand]
        out[b] = cand[np.argmax(vals)]       # first (lowest-id) maximum
    return out


def cache_write(cache: np.ndarray, delta: np.ndarray, p) -> np.ndarray:
    """Host write-back of one layer's deltas ([card] "Shapes": the decoder
    returns only the positions this call wrote; the host copies them into its
    cache at cache_position).  cache [B, T, NKV, D], delta [B, S, NKV, D],
    p [B].  Returns a new array; rows outside [p_b, p_b + S) are untouched."""
    out = np.array(cache, copy=True)
    S = delta.shape[1]
    for b in range(cache.shape[0]):
        out[b, int(p[b]):int(p[b]) + S] = delta[b]
    return out


def embed_ids(table_f16: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Embedding rows of `ids`, fp16 table upcast exactly to fp32
    ([card] "Revision history": the table is stored as fp16)."""
    return np.asarray(table_f16, np.float16)[np.asarray(ids)].astype(F32)


def embed_splice(table_f16, ids, audio, a0: int) -> np.ndarray:
    """Prompt embeddings with the audio slots overwritten ([card]
    "Inference" step 5).  ids [B, S]; audio [B, N, H] replaces rows
    [a0, a0 + N) of every sequence.  Returns [B, S, H] fp32."""
    x = embed_ids(table_f16, ids)
    n = 0 if audio is None else audio.shape[1]
    if n:
        x[:, a0:a0 + n] = np.asarray(audio, F32)
    return x


# ----------------------------------------------------------------- model --
@dataclass
class OracleLayer:
    ln1: np.ndarray
    ln2: np.ndarray
    mats: dict            # name -> (codes int8 [n][k], scale fp32 [n])
    bq: np.ndarray
    bk: np.ndarray
    bv: np.ndarray
    fp32: dict = field(default_factory=dict)   # float weights (float-linear mode)


@dataclass
class OracleModel:
    cfg: object
    layers: list
    final_norm: np.ndarray | None = None
    lm_head: tuple | None = None              # (codes, scale) or None
    lm_head4: tuple | None = None             # int4 tier (codes, scale, zp) or None
    embed: np.ndarray | None = None           # fp16 table
    cos: np.ndarray | None = None
    sin: np.ndarray | None = None
    linear: str = "int8"                      # "int8" or "float" (test mode)


def build_model(cfg, synth, layers=None, with_embed=True, linear="int8",
                keep_fp32=False, lm_head4=False) -> OracleModel:
    """Quantise the seeded fp32 weights of `cfg` into an oracle model.
    `layers` (iterable of layer indices) restricts the layers built;
    `lm_head4` selects the weight-only int4 tier for the LM head."""
    idx = range(cfg.n_layers) if layers is None else layers
    out = []
    for l in idx:
        w = synth.layer_weights(cfg, l)
        mats = {n: prep_weight(w[n]) for n in ("wq", "wk", "wv", "wo", "wg", "wu", "wd")}
        fp = {n: w[n] for n in ("wq", "wk", "wv", "wo", "wg", "wu", "wd")} if (keep_fp32 or linear == "float") else {}
        out.append(OracleLayer(w["ln1"], w["ln2"], mats, w["bq"], w["bk"], w["bv"], fp))
        del w
    m = OracleModel(cfg=cfg, layers=out, linear=linear)
    if cfg.lm_head:
        m.final_norm = synth.final_norm(cfg)
        w = synth.lm_head(cfg)
        m.lm_head = prep_weight(w)
        if lm_head4:
            m.lm_head4 = prep_weight_int4(w)
        del w
    if with_embed:
        m.embed = synth.embed_table_f16(cfg)
    m.cos, m.sin = rope_tables(cfg.max_total_len, cfg.head_dim, cfg.rope_theta)
    return m


def _linear(model: OracleModel, lay: OracleLayer, name: str, x_seq: list, quant: list, bias=None):
    """Apply projection `name` to each sequence's rows.  `quant[b]` is the
    shared (codes, s, z) of that sequence's input; float mode ignores it."""
    if model.linear == "float":
        w = lay.fp32[name].astype(F64)
        ys = []
        for x in x_seq:
            y = x.astype(F64) @ w.T
            if bias is not None:
                y = y + bias.astype(F64)
            ys.append(y.astype(F32))
        return ys
    codes_w, sw = lay.mats[name]
    # one exact integer GEMM over all rows of all sequences
    a = np.concatenate([q[0].astype(F64) - F64(q[2]) for q in quant], axis=0)
    acc = (a @ codes_w.astype(F64).T).astype(np.int64)
    ys, r = [], 0
    for (codes, s, z) in quant:
        n = codes.shape[0]
        ys.append(dequant(acc[r:r + n], s, sw, bias))
        r += n
    return ys


def _quant_each(model, xs):
    if model.linear == "float":
        return [None] * len(xs)
    return [dynquant(x) for x in xs]


def layer_forward(model: OracleModel, l: int, x: np.ndarray, p: np.ndarray,
                  k_cache: np.ndarray, v_cache: np.ndarray, trace: dict | None = None):
    """One Qwen2 decoder layer over B sequences of S rows ([card] "Shapes";
    [cook] intro).

    x [B, S, H] fp32, p [B] cache positions, k_cache / v_cache [B, T, NKV, D]
    (read only).  Every dynamic quantisation covers one sequence's whole
    [S, K] input; q/k/v share one quantisation of h1 and gate/up share one of
    h2.  Returns (x_out [B, S, H], k_delta, v_delta [B, S, NKV, D]).
    """
    cfg = model.cfg
    lay = model.layers[l]
    B, S, H = x.shape
    NH, NKV, D = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    h1 = rmsnorm(x, lay.ln1, cfg.rms_eps)
    qh1 = _quant_each(model, [h1[b] for b in range(B)])
    hs = [h1[b] for b in range(B)]
    q = np.stack(_linear(model, lay, "wq", hs, qh1, lay.bq)).reshape(B, S, NH, D)
    k = np.stack(_linear(model, lay, "wk", hs, qh1, lay.bk)).reshape(B, S, NKV, D)
    v = np.stack(_linear(model, lay, "wv", hs, qh1, lay.bv)).reshape(B, S, NKV, D)
    pos = (np.asarray(p)[:, None] + np.arange(S)[None, :]).astype(np.int64)   # [B, S]
    q = apply_rope(q, pos, model.cos, model.sin)
    k = apply_rope(k, pos, model.cos, model.sin)
    k_delta, v_delta = k, v
    attn = np.empty((B, S, NH * D), F32)
    for b in range(B):
        kh = cache_write(k_cache[b:b + 1], k_delta[b:b + 1], p[b:b + 1])[0]
        vh = cache_write(v_cache[b:b + 1], v_delta[b:b + 1], p[b:b + 1])[0]
        attn[b] = attention(q[b], kh, vh, int(p[b]))
    qa = _quant_each(model, [attn[b] for b in range(B)])
    o = np.stack(_linear(model, lay, "wo", [attn[b] for b in range(B)], qa))
    x1 = (x + o).astype(F32)
    h2 = rmsnorm(x1, lay.ln2, cfg.rms_eps)
    qh2 = _quant_each(model, [h2[b] for b in range(B)])
    h2s = [h2[b] for b in range(B)]
    g = np.stack(_linear(model, lay, "wg", h2s, qh2))
    u = np.stack(_linear(model, lay, "wu", h2s, qh2))
    a = swiglu(g, u)
    qa2 = _quant_each(model, [a[b] for b in range(B)])
    d = np.stack(_linear(model, lay, "wd", [a[b] for b in range(B)], qa2))
    x2 = (x1 + d).astype(F32)
    if trace is not None:
        trace[l] = dict(h1=h1, q=q, k=k_delta, v=v_delta, attn=attn, x1=x1, h2=h2,
                        g=g, u=u, a=a, x2=x2, quant=dict(h1=qh1, attn=qa, h2=qh2, a=qa2))
    return x2, k_delta, v_delta


def forward(model: OracleModel, x: np.ndarray, p, k_caches, v_caches, trace=None):
    """All layers, then the LM head on each sequence's last row.

    [card] "Shapes"/"Inference": returns (logits [B, V] or None,
    k_deltas, v_deltas [L][B, S, NKV, D], hidden [B, S, H] after the last
    layer).  [card] "Revision history": the LM head is int8 (per-channel
    weights, per-sequence dynamic activation scale, no bias).
    """
    p = np.asarray(p, np.int64)
    kd, vd = [], []
    for l in range(len(model.layers)):
        x, k, v = layer_forward(model, l, x, p, k_caches[l], v_caches[l], trace)
        kd.append(k)
        vd.append(v)
    logits = None
    if model.lm_head4 is not None:
        # the weight-only int4 tier: fp32 rows, no activation quantisation
        hn = rmsnorm(x[:, -1, :], model.final_norm, model.cfg.rms_eps)
        logits = lm_head_int4(hn, *model.lm_head4)
    elif model.lm_head is not None:
        last = x[:, -1, :]                                      # [B, H]
        hn = rmsnorm(last, model.final_norm, model.cfg.rms_eps)
        codes_w, sw = model.lm_head
        rows = []
        for b in range(hn.shape[0]):
            c, s, z = dynquant(hn[b:b + 1])
            rows.append(dequant(matmul_integer(c, z, codes_w), s, sw)[0])
        logits = np.stack(rows).astype(F32)
    return logits, kd, vd, x


def prefill(model: OracleModel, embeds: np.ndarray, p, k_caches, v_caches, trace=None):
    """Prefill of B sequences of S rows at positions p ([card] "Inference"
    step 6); the caches are read only, the deltas are returned."""
    return forward(model, np.asarray(embeds, F32), p, k_caches, v_caches, trace)


def decode_step(model: OracleModel, ids, p, k_caches, v_caches, trace=None):
    """One greedy decode step: embed the B token ids (fp16 table), run the
    decoder with S = 1 at positions p."""
    x = embed_ids(model.embed, np.asarray(ids).reshape(-1, 1))
    return forward(model, x, p, k_caches, v_caches, trace)


# ------------------------------------------------------------- structure --
def layer_param_count(hidden: int, kv_dim: int, intermediate: int, q_dim=None) -> int:
    """Parameters of one Qwen2 block as this oracle builds it: q/k/v with
    bias, o without, gate/up/down without, two RMSNorm gains."""
    q_dim = hidden if q_dim is None else q_dim
    return (q_dim * hidden + q_dim) + 2 * (kv_dim * hidden + kv_dim) + hidden * q_dim \
        + 3 * intermediate * hidden + 2 * hidden


# ----------------------------------------------- frame merge and adapter --
# [card] "Inference", steps 2-3: the encoder output [1, seq, 1280] is cut to
# a multiple of 4 frames, every 4 consecutive frames become one 5120-wide
# row, and the adapter maps the rows to the decoder's width (2048); their
# outputs overwrite the <|audio|> slots (step 5, embed_splice).  [card]
# "Files": the adapter's MatMuls are int8 with dynamic activations, like
# the decoder's.  [audio8] "What arkasr actually is": an MLP adapter that
# merges merge_factor consecutive frames; the 0.6B model's adapter holds
# 10,783,360 parameters, which is 5120 x 1792 + 1792 + 1792 x 896 + 896: two
# linear layers with biases whose inner width is twice the decoder's hidden
# width.  Readings for the 3B adapter (the pages give no widths or
# activation): inner width 2 x 2048 = 4096; between the two layers the erf
# GELU of the Whisper encoder the frames come from, in float64 rounded once
# to fp32 (as the decoder's float operations); one (s, z) per sequence and
# quantisation point (merged rows; GELU output).
MERGE = 4


def n_encoder_frames(samples: int) -> int:
    """Encoder frames of a clip: [card] "Inference" step 4's count before its
    division by the merge factor, ((samples // 160) + 1) // 2."""
    return ((int(samples) // 160) + 1) // 2


def frame_merge(frames: np.ndarray, merge: int = MERGE) -> np.ndarray:
    """[seq][D] frames -> [seq // merge][merge * D]: row r is frames
    merge*r .. merge*r + merge - 1 side by side; trailing frames dropped."""
    frames = np.asarray(frames, F32)
    seq, D = frames.shape
    n = seq // merge
    return frames[:n * merge].reshape(n, merge * D).copy()


def gelu(x: np.ndarray) -> np.ndarray:
    """x Phi(x) = 0.5 x (1 + erf(x / sqrt 2)) in float64, rounded to fp32."""
    from scipy.special import erf
    xd = np.asarray(x, F32).astype(F64)
    return (0.5 * xd * (1.0 + erf(xd / np.sqrt(2.0)))).astype(F32)


@dataclass
class OracleAdapter:
    up: tuple            # (int8 codes [inner][merge*D], fp32 scales [inner])
    up_bias: np.ndarray  # [inner]
    down: tuple          # (int8 codes [hidden][inner], fp32 scales [hidden])
    down_bias: np.ndarray
    merge: int = MERGE


def build_adapter(cfg, synth) -> OracleAdapter:
    """The seeded fp32 adapter weights of `cfg`, quantised per channel."""
    w = synth.adapter_weights(cfg)
    return OracleAdapter(prep_weight(w["w1"]), w["b1"], prep_weight(w["w2"]), w["b2"])


def adapter(ad: OracleAdapter, frames: np.ndarray) -> np.ndarray:
    """Merged rows -> int8 linear (+ bias) -> GELU -> int8 linear (+ bias),
    per sequence.  frames [B][seq][D] fp32 -> [B][seq // merge][hidden]."""
    frames = np.asarray(frames, F32)
    out = []
    for b in range(frames.shape[0]):
        m = frame_merge(frames[b], ad.merge)
        c, s, z = dynquant(m)
        y = qlinear(c, s, z, ad.up[0], ad.up[1], ad.up_bias)
        a = gelu(y)
        c2, s2, z2 = dynquant(a)
        out.append(qlinear(c2, s2, z2, ad.down[0], ad.down[1], ad.down_bias))
    return np.stack(out)


def adapter_param_count(frame_dim: int, merge: int, inner: int, hidden: int) -> int:
    """Parameters of the two-layer adapter with biases."""
    return merge * frame_dim * inner + inner + inner * hidden + hidden


# ---------------------------------------------------------- audio encoder --
# [card] "Inference" step 1: the encoder maps log-mel features (128 bins,
# hop 160, the unpadded clip) to [1, seq, 1280]; "Files": the audio encoder
# is dynamically quantised int8 with per-channel MatMul weights.  [cook]
# introduction and [clover]: a Whisper-style audio tower with rotary
# self-attention.  [audio8] "What arkasr actually is": Whisper-style layers
# with RoPE, and the audio_encoder.whisper.* tensors hold 636,968,960
# parameters -- exactly the Whisper large encoder: two width-3 convolutions
# with biases (128 -> 1280, stride 1; 1280 -> 1280, stride 2), a
# 1500 x 1280 positional table, 32 pre-LayerNorm layers of self-attention
# (q, v, o with bias, k without) and a 5120-wide GELU MLP, and a final
# LayerNorm (encoder_param_count pins it).  Readings: 20 heads of 64; the
# positional rows are added after the convolutions and rotary embedding
# (rotate-half, theta 10000, positions 0..F-1) is applied to q and k in
# every layer; attention is bidirectional (a clip attends to all its
# frames); scores are q.k / sqrt(64); LayerNorm eps 1e-5; the convolutions
# are int8 too (the dynamic quantiser's integer convolution: one (s, z) over
# the layer input, per-output-channel weights, zero padding contributing 0);
# GELU is the erf form; LayerNorm, rotary embedding, softmax and GELU in
# float64 rounded once to fp32 (as the decoder's float steps); one (s, z)
# per sequence at every quantisation point.
ENC_LN_EPS = 1e-5
ENC_ROPE_THETA = 10000.0


def encoder_param_count(n_mels: int, d: int, layers: int, ffn: int, max_pos: int) -> int:
    """Parameters of the encoder as built here."""
    attn = 4 * d * d + 3 * d                  # q, k, v, o; q, v, o biases
    layer = attn + 2 * 2 * d + (d * ffn + ffn) + (ffn * d + d)
    convs = (3 * n_mels * d + d) + (3 * d * d + d)
    return layers * layer + convs + max_pos * d + 2 * d


def layernorm(x: np.ndarray, g: np.ndarray, b: np.ndarray, eps: float = ENC_LN_EPS) -> np.ndarray:
    """(x - mean) / sqrt(var + eps) * g + b over the last axis (population
    variance), float64 inside, fp32 out."""
    x64 = np.asarray(x, F32).astype(F64)
    mu = np.mean(x64, axis=-1, keepdims=True)
    xc = x64 - mu
    var = np.mean(xc * xc, axis=-1, keepdims=True)
    r = 1.0 / np.sqrt(var + F64(eps))
    return ((xc * r) * np.asarray(g, F32).astype(F64) + np.asarray(b, F32).astype(F64)).astype(F32)


def conv_out_len(T: int, stride: int) -> int:
    """Output length of a width-3 convolution with padding 1."""
    return (int(T) + 2 - 3) // int(stride) + 1


def im2col(x: np.ndarray, stride: int) -> np.ndarray:
    """Rows of a width-3, padding-1 convolution: x [T][C] -> [T_out][3 C]
    with element (j, c) of row t = x[t * stride - 1 + j][c] (0 outside)."""
    x = np.asarray(x, F32)
    T, C = x.shape
    To = conv_out_len(T, stride)
    xp = np.zeros((T + 2, C), F32)
    xp[1:T + 1] = x
    rows = np.empty((To, 3 * C), F32)
    for j in range(3):
        rows[:, j * C:(j + 1) * C] = xp[j:j + stride * (To - 1) + 1:stride]
    return rows


def enc_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Bidirectional attention of one clip: q, k, v [F, H, Dh] fp32 (q and k
    rotated) -> [F, H * Dh]: softmax(q.k / sqrt(Dh)) v over all F frames,
    float64 inside."""
    F_, H, Dh = q.shape
    out = np.empty((F_, H, Dh), F64)
    scale = 1.0 / np.sqrt(F64(Dh))
    for h in range(H):
        sc = (q[:, h, :].astype(F64) @ k[:, h, :].astype(F64).T) * scale
        m = np.max(sc, axis=1, keepdims=True)
        e = np.exp(sc - m)
        out[:, h, :] = (e @ v[:, h, :].astype(F64)) / np.sum(e, axis=1, keepdims=True)
    return out.reshape(F_, H * Dh).astype(F32)


@dataclass
class OracleEncLayer:
    ln1: tuple
    ln2: tuple
    mats: dict           # name -> (int8 codes, fp32 scales): wq wk wv wo w1 w2
    bias: dict           # bq bv bo b1 b2


@dataclass
class OracleEncoder:
    cfg: object
    conv1: tuple
    conv1_b: np.ndarray
    conv2: tuple
    conv2_b: np.ndarray
    pos: np.ndarray
    layers: list
    lnf: tuple
    cos: np.ndarray
    sin: np.ndarray


def build_encoder(cfg, synth, layers=None) -> OracleEncoder:
    """The seeded encoder of `cfg` with int8 per-channel weights; `layers`
    (optional) limits the stack to those layer indices, in order."""
    fr = synth.encoder_front(cfg)
    idx = range(cfg.enc_layers) if layers is None else layers
    ls = []
    for l in idx:
        w = synth.encoder_layer_weights(cfg, l)
        ls.append(OracleEncLayer((w["ln1_g"], w["ln1_b"]), (w["ln2_g"], w["ln2_b"]),
                                 {n: prep_weight(w[n]) for n in ("wq", "wk", "wv", "wo", "w1", "w2")},
                                 {n: w[n] for n in ("bq", "bv", "bo", "b1", "b2")}))
    cos, sin = rope_tables(cfg.enc_max_pos, cfg.enc_dim // cfg.enc_heads, ENC_ROPE_THETA)
    return OracleEncoder(cfg, prep_weight(fr["conv1"]), fr["conv1_b"], prep_weight(fr["conv2"]),
                         fr["conv2_b"], fr["pos"], ls, (fr["lnf_g"], fr["lnf_b"]), cos, sin)


def _enc_linear(x, mat, bias=None):
    c, s, z = dynquant(x)
    return qlinear(c, s, z, mat[0], mat[1], bias)


def encoder_forward(enc: OracleEncoder, mel: np.ndarray, trace=None) -> np.ndarray:
    """mel [B][M][n_mels] fp32 -> [B][F][d], F = conv_out_len(M, 2), one clip
    at a time (one (s, z) per clip and quantisation point)."""
    cfg = enc.cfg
    H = cfg.enc_heads
    Dh = cfg.enc_dim // H
    out = []
    for b in range(mel.shape[0]):
        a = gelu(_enc_linear(im2col(mel[b], 1), enc.conv1, enc.conv1_b))
        x = gelu(_enc_linear(im2col(a, 2), enc.conv2, enc.conv2_b))
        F_ = x.shape[0]
        assert F_ <= enc.pos.shape[0]
        x = (x + enc.pos[:F_]).astype(F32)
        pos = np.arange(F_)
        for li, L in enumerate(enc.layers):
            h = layernorm(x, *L.ln1)
            c, s, z = dynquant(h)
            q = qlinear(c, s, z, *L.mats["wq"], L.bias["bq"]).reshape(F_, H, Dh)
            k = qlinear(c, s, z, *L.mats["wk"]).reshape(F_, H, Dh)
            v = qlinear(c, s, z, *L.mats["wv"], L.bias["bv"]).reshape(F_, H, Dh)
            qr = apply_rope(q, pos, enc.cos, enc.sin)
            kr = apply_rope(k, pos, enc.cos, enc.sin)
            att = enc_attention(qr, kr, v)
            x = (x + _enc_linear(att, L.mats["wo"], L.bias["bo"])).astype(F32)
            h2 = layernorm(x, *L.ln2)
            f = gelu(_enc_linear(h2, L.mats["w1"], L.bias["b1"]))
            x = (x + _enc_linear(f, L.mats["w2"], L.bias["b2"])).astype(F32)
            if trace is not None:
                trace.append({"seq": b, "layer": li, "h1": h, "q": qr, "k": kr, "v": v,
                              "attn": att, "h2": h2, "f": f, "x": x})
        out.append(layernorm(x, *enc.lnf))
    return np.stack(out)


# ------------------------------------------------ bf16 serving variant --
# [cook] "dtype": the model is served in bfloat16 by default (the validated
# path); [clover] runs it the same way.  This variant is the decoder of the
# functions above with the checkpoint's weights and every activation in
# bf16 instead of int8 MatMuls over fp32 tensors: weights, biases, gains and
# the embedding table rounded to bf16, the KV cache in bf16 (half the bytes
# of the fp32 cache).  Reading of where values are rounded (each operation
# of the bf16 model rounds its output to bf16 once; the operations compute
# in float64 inside, with exact bf16 x bf16 products):
#   RMSNorm      bf16(g * bf16(x / sqrt(mean(x^2) + eps)))
#   linear       bf16(sum_k x w + b)
#   rotary step  bf16 of the rotated pair (the fp64 tables of rope_tables)
#   attention    bf16(softmax(q.k / sqrt(D)) v)
#   residual add bf16(x + y)
#   MLP gate     bf16(bf16(silu(g)) * u)
#   LM head      fp32(sum_k h w) (the logits stay fp32: rounding them to bf16
#                would make the greedy choice a tie far more often)
BF16_MASK = np.uint32(0xFFFF0000)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 of fp32 values (ties to even), returned as fp32
    holding the bf16 value; NaN stays NaN, +-inf stays +-inf."""
    x = np.asarray(x, F32)
    b = x.view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    r = ((b + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)).astype(np.uint32)
    out = r.view(F32).copy()
    nan = np.isnan(x)
    out[nan] = x[nan]
    return out.reshape(x.shape)


@dataclass
class Bf16Layer:
    ln1: np.ndarray
    ln2: np.ndarray
    w: dict              # name -> bf16-valued fp32 [n][k]: wq wk wv wo wg wu wd
    bq: np.ndarray
    bk: np.ndarray
    bv: np.ndarray


@dataclass
class Bf16Model:
    cfg: object
    layers: list
    final_norm: np.ndarray | None = None
    lm_head: np.ndarray | None = None
    embed: np.ndarray | None = None      # bf16-valued fp32 [V][H]
    cos: np.ndarray | None = None
    sin: np.ndarray | None = None
    round: object = None                 # the rounding function (bf16_round; identity in tests)


def build_bf16_model(cfg, synth, layers=None, with_embed=True, rounding=None) -> Bf16Model:
    """The seeded fp32 weights of `cfg` rounded to bf16 (`rounding` replaces
    bf16_round everywhere, for tests)."""
    rnd = bf16_round if rounding is None else rounding
    idx = range(cfg.n_layers) if layers is None else layers
    out = []
    for l in idx:
        w = synth.layer_weights(cfg, l)
        out.append(Bf16Layer(rnd(w["ln1"]), rnd(w["ln2"]),
                             {n: rnd(w[n]) for n in ("wq", "wk", "wv", "wo", "wg", "wu", "wd")},
                             rnd(w["bq"]), rnd(w["bk"]), rnd(w["bv"])))
    m = Bf16Model(cfg=cfg, layers=out, round=rnd)
    if cfg.lm_head:
        m.final_norm = rnd(synth.final_norm(cfg))
        m.lm_head = rnd(synth.lm_head(cfg))
    if with_embed:
        m.embed = rnd(synth.embed_table_f16(cfg).astype(F32))
    m.cos, m.sin = rope_tables(cfg.max_total_len, cfg.head_dim, cfg.rope_theta)
    return m


def bf16_rmsnorm(m: Bf16Model, x: np.ndarray, g: np.ndarray) -> np.ndarray:
    x64 = np.asarray(x, F32).astype(F64)
    r = 1.0 / np.sqrt(np.mean(x64 * x64, axis=-1, keepdims=True) + F64(m.cfg.rms_eps))
    y = m.round((x64 * r).astype(F32))
    return m.round((y.astype(F64) * np.asarray(g, F32).astype(F64)).astype(F32))


def bf16_linear(m: Bf16Model, x: np.ndarray, w: np.ndarray, bias=None) -> np.ndarray:
    y = np.asarray(x, F32).astype(F64) @ np.asarray(w, F32).astype(F64).T
    if bias is not None:
        y = y + np.asarray(bias, F32).astype(F64)
    return m.round(y.astype(F32))


def bf16_layer_forward(m: Bf16Model, l: int, x: np.ndarray, p: np.ndarray,
                       k_cache: np.ndarray, v_cache: np.ndarray, trace: dict | None = None):
    """One layer over B sequences of S rows (the wiring of layer_forward):
    x [B, S, H] bf16-valued, caches [B, T, NKV, D] bf16-valued (read only).
    Returns (x_out, k_delta, v_delta)."""
    cfg = m.cfg
    lay = m.layers[l]
    B, S, H = x.shape
    NH, NKV, D = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    h1 = bf16_rmsnorm(m, x, lay.ln1)
    q = bf16_linear(m, h1, lay.w["wq"], lay.bq).reshape(B, S, NH, D)
    k = bf16_linear(m, h1, lay.w["wk"], lay.bk).reshape(B, S, NKV, D)
    v = bf16_linear(m, h1, lay.w["wv"], lay.bv).reshape(B, S, NKV, D)
    pos = (np.asarray(p)[:, None] + np.arange(S)[None, :]).astype(np.int64)
    q = m.round(apply_rope(q, pos, m.cos, m.sin))
    k = m.round(apply_rope(k, pos, m.cos, m.sin))
    attn = np.empty((B, S, NH * D), F32)
    for b in range(B):
        kh = cache_write(k_cache[b:b + 1], k[b:b + 1], p[b:b + 1])[0]
        vh = cache_write(v_cache[b:b + 1], v[b:b + 1], p[b:b + 1])[0]
        attn[b] = m.round(attention(q[b], kh, vh, int(p[b])))
    o = bf16_linear(m, attn, lay.w["wo"])
    x1 = m.round((x.astype(F64) + o.astype(F64)).astype(F32))
    h2 = bf16_rmsnorm(m, x1, lay.ln2)
    g = bf16_linear(m, h2, lay.w["wg"])
    u = bf16_linear(m, h2, lay.w["wu"])
    g64 = g.astype(F64)
    sg = m.round((g64 / (1.0 + np.exp(-g64))).astype(F32))
    a = m.round((sg.astype(F64) * u.astype(F64)).astype(F32))
    d = bf16_linear(m, a, lay.w["wd"])
    x2 = m.round((x1.astype(F64) + d.astype(F64)).astype(F32))
    if trace is not None:
        trace.update(h1=h1, q=q, k=k, v=v, attn=attn, x1=x1, h2=h2, g=g, u=u, a=a, x2=x2)
    return x2, k, v


def bf16_forward(m: Bf16Model, x: np.ndarray, p, k_caches, v_caches):
    """All layers, then the LM head on each sequence's last row: (logits
    [B, V] fp32 or None, k_deltas, v_deltas, hidden)."""
    p = np.asarray(p, np.int64)
    x = np.asarray(x, F32)
    kd, vd = [], []
    for l in range(len(m.layers)):
        x, k, v = bf16_layer_forward(m, l, x, p, k_caches[l], v_caches[l])
        kd.append(k)
        vd.append(v)
    logits = None
    if m.lm_head is not None:
        hn = bf16_rmsnorm(m, x[:, -1, :], m.final_norm)
        logits = (hn.astype(F64) @ m.lm_head.astype(F64).T).astype(F32)
    return logits, kd, vd, x


def bf16_prefill(m: Bf16Model, embeds: np.ndarray, p, k_caches, v_caches):
    """Prefill from bf16 rows (the caller's embeddings rounded to bf16)."""
    return bf16_forward(m, m.round(np.asarray(embeds, F32)), p, k_caches, v_caches)


def bf16_decode_step(m: Bf16Model, ids, p, k_caches, v_caches):
    x = m.embed[np.asarray(ids).reshape(-1)][:, None, :]
    return bf16_forward(m, x, p, k_caches, v_caches)
