"""Plain, slow CPU oracle of the ARK-ASR-3B int8 decoder step (numpy only).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages cited (by title and section):
  [card]   model card "ark-asr-3b-onnx": sections "Files" (int8 dynamic
           quantisation, per-channel MatMul weights), "Shapes" (geometry,
           static cache, deltas), "Inference" (prompt, slot count, masked
           greedy loop), "Revision history" (fp16 table, int8 LM head).
  [cook]   sglang-omni cookbook "ARK-ASR-3B": intro (Qwen2 decoder), "Audio
           Handling" (token count), "Marker-Token Suppression" (mask set).
  [readme] "ARK-ASR-3B" README: "vLLM" section (<|im_end|> is the stop token).

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
    embed: np.ndarray | None = None           # fp16 table
    cos: np.ndarray | None = None
    sin: np.ndarray | None = None
    linear: str = "int8"                      # "int8" or "float" (test mode)


def build_model(cfg, synth, layers=None, with_embed=True, linear="int8",
                keep_fp32=False) -> OracleModel:
    """Quantise the seeded fp32 weights of `cfg` into an oracle model.
    `layers` (iterable of layer indices) restricts the layers built."""
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
        m.lm_head = prep_weight(synth.lm_head(cfg))
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
    if model.lm_head is not None:
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
