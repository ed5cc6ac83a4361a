"""Seeded synthetic inputs for the ARK-ASR-3B int8 decoder step.

This module is shared by the CPU oracle, the tests and the benchmark.  It
draws random numbers and nothing else: it holds none of the method's
arithmetic (no quantisation, no normalisation, no RoPE, no attention).  Every
array is a pure function of (config seed, tag, layer, chunk), so any process
that imports it regenerates bit-identical inputs.

Workload shapes follow the model card "ark-asr-3b-onnx" (section "Shapes":
36 layers, hidden 2048, 16 heads, 2 KV heads, head dim 128, a static
[1, 512, 2, 128] cache; section "Inference": the prompt layout and the
audio-slot count; section "Revision history": fp16 embedding table, 512 vs
1024 cache length).  The FFN width (11008), RMSNorm eps (1e-6), RoPE theta
(1e6) and vocabulary (151936) are not on the pages; they are fixed here.

Distributions:
  * projection weights          N(0, 0.02) fp32, [out][in] row-major
  * q/k/v biases                N(0, 0.02) fp32
  * RMSNorm gains               1 + N(0, 0.02) fp32
  * embedding table             N(0, 1) rounded to fp16 (stored as uint16 bits)
  * audio stand-ins, embeddings N(0, 1) fp32
  * pre-filled caches           rows < valid length N(0, 1) fp32, other rows 0
  * token ids                   uniform over the unmasked vocabulary
  * adapter weights, biases     N(0, 0.02) fp32 ([out][in] row-major)
  * encoder frames              N(0, 1) fp32 [B][frames][frame_dim]
  * audio encoder weights       N(0, 0.02) fp32 (LayerNorm gains 1 + N(0, 0.02),
                                LayerNorm biases and positional rows N(0, 0.02))
  * log-mel features            N(0, 1) fp32 [B][mel_frames][n_mels]

Adapter geometry: frames of width 1280 (the encoder output of the model
card's "Inference" step 1), 4 frames per merged row (step 2), an inner width
of 4096; encoder frame counts 150 and 1500 for the 3 s and 30 s clips.
Audio encoder geometry: 128 mel bins, width 1280, 20 heads, FFN 5120, 32
layers, 1500 positions; 300 and 3000 mel frames for the 3 s and 30 s clips.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

# Tags naming each random stream.
TAG_WQ, TAG_WK, TAG_WV = 1, 2, 3
TAG_BQ, TAG_BK, TAG_BV = 4, 5, 6
TAG_WO, TAG_WG, TAG_WU, TAG_WD = 7, 8, 9, 10
TAG_LN1, TAG_LN2, TAG_FINAL_NORM = 11, 12, 13
TAG_LM_HEAD, TAG_EMBED = 14, 15
TAG_PROMPT_IDS, TAG_AUDIO, TAG_PREFILL_EMBEDS = 16, 17, 18
TAG_DECODE_IDS, TAG_CACHE_LEN, TAG_CACHE_K, TAG_CACHE_V = 19, 20, 21, 22
TAG_START_IDS = 23
TAG_AD_W1, TAG_AD_B1, TAG_AD_W2, TAG_AD_B2, TAG_FRAMES = 24, 25, 26, 27, 28
TAG_ENC_W = 40            # + index of the tensor within a layer (see ENC_LAYER_TENSORS)
TAG_ENC_FRONT = 60        # + index within ENC_FRONT_TENSORS
TAG_MEL = 70

ROW_CHUNK = 2048          # rows per independent random stream of a big matrix
WEIGHT_STD = 0.02


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


@dataclass(frozen=True)
class ArkConfig:
    """One workload: model geometry plus the run it describes."""
    name: str
    seed: int
    n_layers: int = 36
    hidden: int = 2048
    n_heads: int = 16
    n_kv_heads: int = 2
    head_dim: int = 128
    intermediate: int = 11008
    vocab: int = 151936          # rows of the embedding table (and LM head)
    max_total_len: int = 512
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    batch: int = 1
    prefill_len: int = 0         # S of the prefill call (0: no prefill)
    n_decode: int = 0            # decode steps after the prefill
    lm_head: bool = True
    audio_slots: int = 0         # N audio rows spliced into the prompt
    audio_offset: int = 2        # <|user|><|begin_of_audio|> precede the slots
    prefill_from_embeds: bool = False   # prefill input is N(0,1) rows, not ids
    n_added: int = 64            # added-vocab ids at the top of the vocabulary
    cache_fill: tuple = ()       # (lo, hi): pre-filled valid length per sequence
    decode_ids_fixed: bool = False      # decode ids are drawn, not greedy
    frame_dim: int = 1280        # encoder output width
    merge: int = 4               # frames per merged adapter row
    adapter_inner: int = 4096    # adapter's inner width
    enc_frames: int = 0          # encoder frames per sequence (0: no adapter input)
    n_mels: int = 128            # audio encoder input bins
    enc_dim: int = 1280          # audio encoder width
    enc_heads: int = 20
    enc_ffn: int = 5120
    enc_layers: int = 32
    enc_max_pos: int = 1500      # rows of the encoder's positional table
    mel_frames: int = 0          # log-mel frames per sequence (0: no encoder input)
    enc_ln_eps: float = 1e-5     # encoder LayerNorm epsilon
    enc_rope_theta: float = 1e4  # encoder rotary base

    # Added-vocab convention: ids [vocab - n_added, vocab) are the "<...>"
    # added tokens; the first of them is the end token, which stays unmasked.
    @property
    def end_id(self) -> int:
        return self.vocab - self.n_added

    def mask(self) -> np.ndarray:
        """uint8 [vocab], 1 = masked (every added id except the end id)."""
        m = np.zeros(self.vocab, np.uint8)
        if self.n_added > 0:
            m[self.vocab - self.n_added + 1:] = 1
        return m

    @property
    def group(self) -> int:
        return self.n_heads // self.n_kv_heads

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def with_(self, **kw) -> "ArkConfig":
        return replace(self, **kw)


# Audio-slot counts of a 3 s and a 30 s clip at 16 kHz (48000 and 480000
# samples) and their encoder frame counts.  The oracle owns the formulas of
# the model card's "Inference" steps 2-4; its tests check that they give
# these numbers.
_N3S = 37
_N30S = 375
_F3S = 150
_F30S = 1500

CONFIGS = {
    # Single layer at real shape, one sequence: 64-row prefill of N(0,1)
    # embeddings, then 16 decode steps whose ids index a 1024-row fp16 table.
    "c0": ArkConfig(name="c0", seed=1000, n_layers=1, vocab=1024, lm_head=False,
                    prefill_len=64, n_decode=16, prefill_from_embeds=True,
                    n_added=0, decode_ids_fixed=True),
    # 3 s clip: 2 + 37 + 10 prompt rows, 32 greedy steps.
    "c1": ArkConfig(name="c1", seed=1001, prefill_len=2 + _N3S + 10, n_decode=32,
                    audio_slots=_N3S, enc_frames=_F3S, mel_frames=2 * _F3S),
    # 30 s clip: 2 + 375 + 10 prompt rows, greedy until the 512 cache is full.
    "c2": ArkConfig(name="c2", seed=1002, prefill_len=2 + _N30S + 10,
                    n_decode=512 - (2 + _N30S + 10), audio_slots=_N30S, enc_frames=_F30S,
                    mel_frames=2 * _F30S),
    # 32 independent sequences with pre-filled caches, 64 lockstep steps.
    "c3": ArkConfig(name="c3", seed=1003, batch=32, prefill_len=0, n_decode=64,
                    cache_fill=(50, 400)),
    # Coalesced prefill of 16 x 387 N(0,1) rows, then 16 decode steps.
    "c4": ArkConfig(name="c4", seed=1004, batch=16, prefill_len=2 + _N30S + 10,
                    n_decode=16, prefill_from_embeds=True, enc_frames=_F30S,
                    mel_frames=2 * _F30S),
    "c4_t1024": ArkConfig(name="c4_t1024", seed=1004, batch=16,
                          prefill_len=2 + _N30S + 10, n_decode=16,
                          prefill_from_embeds=True, max_total_len=1024),
}

# Small geometries for fast tests.  "tiny" is for pure-Python brute force;
# "small" keeps the real head_dim (128) and spans several kernel tiles with a
# ragged tail while the oracle still finishes in seconds.
TINY = ArkConfig(name="tiny", seed=7, n_layers=2, hidden=64, n_heads=4, n_kv_heads=2,
                 head_dim=16, intermediate=96, vocab=50, max_total_len=16,
                 prefill_len=5, n_decode=4, n_added=8, audio_slots=2,
                 frame_dim=8, adapter_inner=24, enc_frames=10,
                 n_mels=4, enc_dim=8, enc_heads=2, enc_ffn=16, enc_layers=2, enc_max_pos=16,
                 mel_frames=19)
SMALL = ArkConfig(name="small", seed=11, n_layers=2, hidden=512, n_heads=4,
                  n_kv_heads=2, head_dim=128, intermediate=1344, vocab=3000,
                  max_total_len=64, prefill_len=21, n_decode=6, n_added=64,
                  audio_slots=9, frame_dim=320, adapter_inner=1024, enc_frames=39,
                  n_mels=64, enc_dim=320, enc_heads=5, enc_ffn=640, enc_layers=2,
                  enc_max_pos=128, mel_frames=77)


# ---------------------------------------------------------------- weights --
def _normal_rows(cfg: ArkConfig, tag: int, layer: int, rows: int, cols: int,
                 std: float, mean: float = 0.0) -> np.ndarray:
    out = np.empty((rows, cols), np.float32)

    def fill(c: int) -> None:
        r0 = c * ROW_CHUNK
        r1 = min(rows, r0 + ROW_CHUNK)
        blk = _rng(cfg.seed, tag, layer, c).standard_normal((r1 - r0, cols), dtype=np.float32)
        blk *= np.float32(std)
        if mean:
            blk += np.float32(mean)
        out[r0:r1] = blk

    n_chunks = (rows + ROW_CHUNK - 1) // ROW_CHUNK
    if n_chunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out


def _normal_vec(cfg: ArkConfig, tag: int, layer: int, n: int, std: float,
                mean: float = 0.0) -> np.ndarray:
    v = _rng(cfg.seed, tag, layer, 0).standard_normal(n, dtype=np.float32)
    v *= np.float32(std)
    if mean:
        v += np.float32(mean)
    return v


def layer_weights(cfg: ArkConfig, layer: int) -> dict:
    """fp32 weights of one decoder layer (projection matrices [out][in])."""
    H, I, Q, KV = cfg.hidden, cfg.intermediate, cfg.q_dim, cfg.kv_dim
    s = WEIGHT_STD
    return {
        "ln1": _normal_vec(cfg, TAG_LN1, layer, H, s, 1.0),
        "ln2": _normal_vec(cfg, TAG_LN2, layer, H, s, 1.0),
        "wq": _normal_rows(cfg, TAG_WQ, layer, Q, H, s),
        "wk": _normal_rows(cfg, TAG_WK, layer, KV, H, s),
        "wv": _normal_rows(cfg, TAG_WV, layer, KV, H, s),
        "bq": _normal_vec(cfg, TAG_BQ, layer, Q, s),
        "bk": _normal_vec(cfg, TAG_BK, layer, KV, s),
        "bv": _normal_vec(cfg, TAG_BV, layer, KV, s),
        "wo": _normal_rows(cfg, TAG_WO, layer, H, Q, s),
        "wg": _normal_rows(cfg, TAG_WG, layer, I, H, s),
        "wu": _normal_rows(cfg, TAG_WU, layer, I, H, s),
        "wd": _normal_rows(cfg, TAG_WD, layer, H, I, s),
    }


def final_norm(cfg: ArkConfig) -> np.ndarray:
    return _normal_vec(cfg, TAG_FINAL_NORM, 0, cfg.hidden, WEIGHT_STD, 1.0)


def lm_head_rows(cfg: ArkConfig, r0: int, r1: int) -> np.ndarray:
    """fp32 LM-head rows [r0, r1); r0 and r1 must be multiples of ROW_CHUNK
    (r1 may also be the vocabulary size)."""
    assert r0 % ROW_CHUNK == 0 and (r1 % ROW_CHUNK == 0 or r1 == cfg.vocab)
    out = np.empty((r1 - r0, cfg.hidden), np.float32)

    def fill(c: int) -> None:
        a = c * ROW_CHUNK
        b = min(cfg.vocab, a + ROW_CHUNK)
        blk = _rng(cfg.seed, TAG_LM_HEAD, 0, c).standard_normal((b - a, cfg.hidden), dtype=np.float32)
        blk *= np.float32(WEIGHT_STD)
        out[a - r0:b - r0] = blk

    chunks = range(r0 // ROW_CHUNK, (r1 + ROW_CHUNK - 1) // ROW_CHUNK)
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, chunks))
    return out


def lm_head(cfg: ArkConfig) -> np.ndarray:
    return lm_head_rows(cfg, 0, cfg.vocab)


def embed_table_f16(cfg: ArkConfig) -> np.ndarray:
    """[vocab, hidden] float16 table (N(0,1) rounded to fp16)."""
    t = _normal_rows(cfg, TAG_EMBED, 0, cfg.vocab, cfg.hidden, 1.0)
    return t.astype(np.float16)


def adapter_weights(cfg: ArkConfig) -> dict:
    """fp32 adapter weights: w1 [inner][merge * frame_dim], b1 [inner],
    w2 [hidden][inner], b2 [hidden]."""
    K1, I, H = cfg.merge * cfg.frame_dim, cfg.adapter_inner, cfg.hidden
    s = WEIGHT_STD
    return {
        "w1": _normal_rows(cfg, TAG_AD_W1, 0, I, K1, s),
        "b1": _normal_vec(cfg, TAG_AD_B1, 0, I, s),
        "w2": _normal_rows(cfg, TAG_AD_W2, 0, H, I, s),
        "b2": _normal_vec(cfg, TAG_AD_B2, 0, H, s),
    }


ENC_LAYER_TENSORS = ("ln1_g", "ln1_b", "wq", "bq", "wk", "wv", "bv", "wo", "bo",
                     "ln2_g", "ln2_b", "w1", "b1", "w2", "b2")
ENC_FRONT_TENSORS = ("conv1", "conv1_b", "conv2", "conv2_b", "pos", "lnf_g", "lnf_b")


def encoder_layer_weights(cfg: ArkConfig, layer: int) -> dict:
    """fp32 weights of one audio encoder layer ([out][in] row-major; the
    key projection has no bias)."""
    D, F = cfg.enc_dim, cfg.enc_ffn
    s = WEIGHT_STD
    shapes = {"wq": (D, D), "wk": (D, D), "wv": (D, D), "wo": (D, D), "w1": (F, D), "w2": (D, F)}
    out = {}
    for i, name in enumerate(ENC_LAYER_TENSORS):
        tag = TAG_ENC_W + i
        if name in shapes:
            out[name] = _normal_rows(cfg, tag, layer, *shapes[name], s)
        elif name.endswith("_g"):
            out[name] = _normal_vec(cfg, tag, layer, D, s, 1.0)
        else:
            out[name] = _normal_vec(cfg, tag, layer, F if name == "b1" else D, s)
    return out


def encoder_front(cfg: ArkConfig) -> dict:
    """fp32 convolution weights [out][3][in] (tap-major: element (j, c) of an
    output row is tap j of input channel c), their biases, the positional
    table [max_pos][D] and the final LayerNorm."""
    D, M = cfg.enc_dim, cfg.n_mels
    s = WEIGHT_STD
    t = {n: TAG_ENC_FRONT + i for i, n in enumerate(ENC_FRONT_TENSORS)}
    return {
        "conv1": _normal_rows(cfg, t["conv1"], 0, D, 3 * M, s),
        "conv1_b": _normal_vec(cfg, t["conv1_b"], 0, D, s),
        "conv2": _normal_rows(cfg, t["conv2"], 0, D, 3 * D, s),
        "conv2_b": _normal_vec(cfg, t["conv2_b"], 0, D, s),
        "pos": _normal_rows(cfg, t["pos"], 0, cfg.enc_max_pos, D, s),
        "lnf_g": _normal_vec(cfg, t["lnf_g"], 0, D, s, 1.0),
        "lnf_b": _normal_vec(cfg, t["lnf_b"], 0, D, s),
    }


# ------------------------------------------------------------------ inputs --
def mel_features(cfg: ArkConfig, frames: int | None = None) -> np.ndarray:
    """[B, mel_frames, n_mels] fp32 N(0, 1) stand-ins for log-mel features."""
    n = cfg.mel_frames if frames is None else int(frames)
    return _rng(cfg.seed, TAG_MEL, n, 0).standard_normal((cfg.batch, n, cfg.n_mels), dtype=np.float32)


def encoder_frames(cfg: ArkConfig, frames: int | None = None) -> np.ndarray:
    """[B, frames, frame_dim] fp32 N(0, 1) stand-ins for the encoder output."""
    n = cfg.enc_frames if frames is None else int(frames)
    return _rng(cfg.seed, TAG_FRAMES, n, 0).standard_normal(
        (cfg.batch, n, cfg.frame_dim), dtype=np.float32)


def unmasked_ids(cfg: ArkConfig, rng: np.random.Generator, shape) -> np.ndarray:
    """Token ids drawn uniformly from the ids that are neither masked nor the
    end token (so a drawn prompt never contains a stop token)."""
    hi = cfg.vocab - cfg.n_added
    return rng.integers(0, hi, size=shape, dtype=np.int64).astype(np.int32)


def prompt_ids(cfg: ArkConfig) -> np.ndarray:
    """[B, S] int32 prompt ids; audio slots hold placeholder ids (overwritten)."""
    ids = unmasked_ids(cfg, _rng(cfg.seed, TAG_PROMPT_IDS, 0, 0), (cfg.batch, cfg.prefill_len))
    return ids


def audio_rows(cfg: ArkConfig) -> np.ndarray:
    """[B, N, H] fp32 stand-ins for the adapter output."""
    return _rng(cfg.seed, TAG_AUDIO, 0, 0).standard_normal(
        (cfg.batch, cfg.audio_slots, cfg.hidden), dtype=np.float32)


def prefill_embeds(cfg: ArkConfig) -> np.ndarray:
    """[B, S, H] fp32 N(0,1) prefill rows (configs that prefill from embeddings)."""
    return _rng(cfg.seed, TAG_PREFILL_EMBEDS, 0, 0).standard_normal(
        (cfg.batch, cfg.prefill_len, cfg.hidden), dtype=np.float32)


def decode_ids(cfg: ArkConfig) -> np.ndarray:
    """[n_decode, B] int32 ids for configs whose decode ids are drawn."""
    return _rng(cfg.seed, TAG_DECODE_IDS, 0, 0).integers(
        0, cfg.vocab, size=(cfg.n_decode, cfg.batch), dtype=np.int64).astype(np.int32)


def start_ids(cfg: ArkConfig) -> np.ndarray:
    """[B] int32 first decode ids for configs without a prefill."""
    return unmasked_ids(cfg, _rng(cfg.seed, TAG_START_IDS, 0, 0), (cfg.batch,))


def cache_lengths(cfg: ArkConfig) -> np.ndarray:
    """[B] int32 valid lengths of pre-filled caches (uniform in [lo, hi])."""
    lo, hi = cfg.cache_fill
    return _rng(cfg.seed, TAG_CACHE_LEN, 0, 0).integers(
        lo, hi + 1, size=cfg.batch, dtype=np.int64).astype(np.int32)


def prefilled_cache(cfg: ArkConfig, layer: int, which: str, lengths: np.ndarray,
                    garbage: float = 0.0) -> np.ndarray:
    """[B, T, NKV, D] fp32 cache of one layer: N(0,1) rows below each
    sequence's valid length; the other rows are 0 (or `garbage`)."""
    tag = TAG_CACHE_K if which == "k" else TAG_CACHE_V
    B, T = cfg.batch, cfg.max_total_len
    c = _rng(cfg.seed, tag, layer, 0).standard_normal(
        (B, T, cfg.n_kv_heads, cfg.head_dim), dtype=np.float32)
    for b in range(B):
        c[b, int(lengths[b]):] = np.float32(garbage)
    return c
