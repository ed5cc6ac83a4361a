"""The audio encoder on the GPU against the oracle (model card
"ark-asr-3b-onnx", "Inference" step 1 and "Files"; cookbook "ARK-ASR-3B"
introduction: rotary self-attention; Audio8 article, "What arkasr actually
is": the encoder's parameter count).

  * the new float kernels alone: LayerNorm within 1e-6 of the oracle's
    (fp64 inside on both sides, one rounding) with the per-sequence range
    exactly the min / max of the values written; the rotary bidirectional
    attention within 1e-5 (the decoder attention's bound: fp64 sums in
    another order), its range likewise, at 1..300 frames, 1..20 heads, with
    the GPU's own rotary tables against the oracle's;
  * the whole encoder (int8 convolutions and projections, which the kernel
    tests pin bit for bit, between those float steps) against
    oracle.encoder_forward within 1e-3 per clip (a quantisation code that
    flips on a last-bit difference upstream moves later values by
    quantisation noise), at the small geometry over ragged and minimal
    frame counts and several clips, and at full size for the 3 s clip and a
    30 s clip;
  * mel -> encoder -> adapter -> splice -> prefill -> token against the
    oracle's chain at the small geometry.
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
from speech_decoder_int8_amd import ark  # noqa: E402

from gpu_util import GpuState, assert_close, check_tokens, host, t  # noqa: E402

pytestmark = pytest.mark.gpu
F32 = np.float32


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


@pytest.mark.parametrize("B,S,D", [(1, 1, 64), (2, 37, 1280), (3, 150, 320), (1, 5, 1000)])
def test_layernorm_kernel(B, S, D):
    rng = np.random.default_rng(B * 100 + S + D)
    x = (rng.standard_normal((B, S, D)) * 2 + 0.7).astype(F32)
    x[-1] *= 9.0
    g = (1 + 0.05 * rng.standard_normal(D)).astype(F32)
    b = (0.05 * rng.standard_normal(D)).astype(F32)
    y, lo, hi = ark.test_layernorm(t(x), t(g), t(b), 1e-5)
    y, lo, hi = host(y), host(lo), host(hi)
    want = oracle.layernorm(x, g, b, 1e-5)
    assert rel(y, want) <= 1e-6
    assert np.count_nonzero(y.view(np.uint32) != want.view(np.uint32)) <= max(2, want.size // 10000)
    for i in range(B):
        assert lo[i] == y[i].min() and hi[i] == y[i].max()


@pytest.mark.parametrize("B,F,H", [(1, 1, 1), (1, 5, 2), (2, 16, 5), (1, 64, 3), (2, 65, 5),
                                   (1, 150, 20), (2, 300, 4)])
def test_enc_attention_kernel(B, F, H):
    rng = np.random.default_rng(B * 1000 + F * 10 + H)
    qkv = rng.standard_normal((B, F, 3 * H * 64)).astype(F32)
    qkv[:, :, :H * 64] *= 1.5                     # sharper scores
    cos, sin = ark.rope_table(max(F, 8), 64, 1e4)
    out, lo, hi = ark.test_enc_attention(t(qkv), H, cos, sin)
    out, lo, hi = host(out), host(lo), host(hi)
    oc, os_ = oracle.rope_tables(max(F, 8), 64, 1e4)
    pos = np.arange(F)
    for b in range(B):
        q = qkv[b, :, :H * 64].reshape(F, H, 64)
        k = qkv[b, :, H * 64:2 * H * 64].reshape(F, H, 64)
        v = qkv[b, :, 2 * H * 64:].reshape(F, H, 64)
        want = oracle.enc_attention(oracle.apply_rope(q, pos, oc, os_),
                                    oracle.apply_rope(k, pos, oc, os_), v)
        assert rel(out[b], want) <= 1e-5, (b, rel(out[b], want))
        assert lo[b] == out[b].min() and hi[b] == out[b].max()


SMALL = synth.SMALL


@pytest.fixture(scope="module")
def small_enc():
    return oracle.build_encoder(SMALL, synth), ark.load_encoder(SMALL, synth)


def _run(enc, mel):
    B, M = mel.shape[0], mel.shape[1]
    F = (M - 1) // 2 + 1
    out = torch.full((B, F, enc.cfg.enc_dim), float("nan"), device="cuda")
    ark.audio_encoder(enc, t(mel), out)
    return host(out)


@pytest.mark.parametrize("B,M", [(1, 77), (2, 77), (1, 1), (2, 2), (3, 20), (1, 255)])
def test_encoder_small(small_enc, B, M):
    eo, eg = small_enc
    mel = synth.mel_features(SMALL.with_(batch=B), M)
    mel[-1] *= 2.5
    got = _run(eg, mel)
    want = oracle.encoder_forward(eo, mel)
    assert got.shape == want.shape
    for b in range(B):
        assert np.all(np.isfinite(got[b]))
        assert rel(got[b], want[b]) <= 1e-3, (b, rel(got[b], want[b]))


def test_mel_encoder_adapter_prefill_pipeline(small_enc):
    """mel -> encoder -> adapter -> splice -> prefill -> token at the small
    geometry, against the oracle's chain."""
    cfg = SMALL
    eo, eg = small_enc
    ad_o, ad = oracle.build_adapter(cfg, synth), ark.load_adapter(cfg, synth)
    om, gm = oracle.build_model(cfg, synth), ark.load_model(cfg, synth)
    mel = synth.mel_features(cfg)
    F = cfg.enc_frames
    frames = torch.empty((1, F, cfg.enc_dim), device="cuda")
    ark.audio_encoder(eg, t(mel), frames)
    n = F // cfg.merge
    rows = torch.empty((1, n, cfg.hidden), device="cuda")
    ark.audio_adapter(ad, frames, rows)
    ids = synth.prompt_ids(cfg)
    x = torch.empty((1, cfg.prefill_len, cfg.hidden), device="cuda")
    ark.embed_splice(gm.dims, t(ids), gm.embed_f16, rows, cfg.audio_offset, x)
    gs = GpuState(gm, 1, cfg.prefill_len)
    kd, vd = gs.deltas(cfg.prefill_len)
    ark.prefill(gm, x, [0], gs.kc, gs.vc, kd, vd, gs.logits, ws=gs.ws)
    tok = torch.empty(1, dtype=torch.int32, device="cuda")
    ark.masked_argmax(gs.logits, t(cfg.mask()), tok)
    fr_o = oracle.encoder_forward(eo, mel)
    assert rel(host(frames), fr_o) <= 1e-3
    rows_o = oracle.adapter(ad_o, fr_o)
    x_o = oracle.embed_splice(om.embed, ids, rows_o, cfg.audio_offset)
    zero = np.zeros((1, cfg.max_total_len, cfg.n_kv_heads, cfg.head_dim), F32)
    lo, _, _, _ = oracle.prefill(om, x_o, np.array([0]), [zero] * cfg.n_layers, [zero] * cfg.n_layers)
    err = assert_close(host(gs.logits), lo, "pipeline logits")
    check_tokens(host(tok), oracle.masked_argmax(lo, cfg.mask()), lo, cfg.mask(),
                 err * np.max(np.abs(lo)), "pipeline token")


# ------------------------------------------------------------- full size --
FULL = synth.CONFIGS["c1"]


@pytest.fixture(scope="module")
def full_enc():
    eg = ark.load_encoder(FULL, synth)
    eo = oracle.build_encoder(FULL, synth)
    yield eo, eg
    del eg
    torch.cuda.empty_cache()


def test_encoder_full_c1(full_enc):
    """The 3 s clip: 300 mel frames -> 150 encoder frames of 1280."""
    eo, eg = full_enc
    mel = synth.mel_features(FULL)
    got = _run(eg, mel)
    assert got.shape == (1, 150, 1280)
    assert rel(got[0], oracle.encoder_forward(eo, mel)[0]) <= 1e-3


def test_encoder_full_30s_clip(full_enc):
    """Two 30 s clips in one call (3000 mel frames -> 1500 frames each, the
    positional table's full length); the second checked against the oracle."""
    eo, eg = full_enc
    c4 = synth.CONFIGS["c4"]
    mel = synth.mel_features(c4.with_(batch=2))
    got = _run(eg, mel)
    assert got.shape == (2, 1500, 1280) and np.all(np.isfinite(got))
    assert rel(got[1], oracle.encoder_forward(eo, mel[1:2])[0]) <= 1e-3
