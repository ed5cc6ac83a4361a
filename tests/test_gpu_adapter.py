"""The frame merge and int8 MLP adapter on the GPU against the oracle (model
card "ark-asr-3b-onnx", "Inference" steps 2-3 and 5, "Files").

Every case checks, per sequence:
  * the GELU output the second quantisation sees (`mid`) against the
    oracle's GELU of the oracle's first projection, which is exact given
    the merged rows (codes, int32 accumulators and dequantisation are
    bit-exact by construction): within 1e-6 relative, and nearly all
    elements bit for bit (the two sides' fp64 erf may differ in its last
    bit, which moves an fp32 result only at a rounding boundary);
  * re-anchored on the GPU's own `mid`: the oracle's quantisation of it and
    its second projection (+ bias) equal the GPU's rows bit for bit;
  * end to end against oracle.adapter: bit for bit whenever the two mids
    quantise to the same codes.
Shapes: the small geometry (frame width 320, inner 1024, hidden 512) with
ragged frame counts (a compacted copy when several sequences are cut), one
row, the few-row GEMM and the large-tile GEMM; the full geometry for the
3 s clip (150 frames) and sampled sequences of sixteen 30 s clips (1500
frames each).  A pipeline case runs frames -> adapter -> splice -> prefill
-> greedy token against the oracle's chain.
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


def _check(ad_o, frames_np, out, mid, seqs, what):
    """The checks of the module docstring for sequences `seqs`."""
    for b in seqs:
        m = oracle.frame_merge(frames_np[b], ad_o.merge)
        c, s, z = oracle.dynquant(m)
        y = oracle.qlinear(c, s, z, ad_o.up[0], ad_o.up[1], ad_o.up_bias)
        a_o = oracle.gelu(y)
        a_g = mid[b]
        assert np.all(np.isfinite(a_g)), f"{what} seq {b}: non-finite mid"
        r = float(np.max(np.abs(a_g.astype(np.float64) - a_o)) / np.max(np.abs(a_o)))
        assert r <= 1e-6, f"{what} seq {b}: GELU output relative error {r:.3g}"
        diff = int(np.count_nonzero(a_g.view(np.uint32) != a_o.view(np.uint32)))
        assert diff <= max(2, a_o.size // 100000), f"{what} seq {b}: {diff} GELU values differ"
        c2, s2, z2 = oracle.dynquant(a_g)
        want = oracle.qlinear(c2, s2, z2, ad_o.down[0], ad_o.down[1], ad_o.down_bias)
        bad = np.argwhere(out[b].view(np.uint32) != want.view(np.uint32))
        assert bad.size == 0, f"{what} seq {b}: {len(bad)} rows x cols differ from the re-anchored oracle, first {bad[:4]}"
        c2o, _, _ = oracle.dynquant(a_o)
        if np.array_equal(c2o, c2):
            full = oracle.qlinear(c2o, s2, z2, ad_o.down[0], ad_o.down[1], ad_o.down_bias)
            assert np.array_equal(out[b].view(np.uint32), full.view(np.uint32))


def _run(ad, frames_np):
    B, F = frames_np.shape[0], frames_np.shape[1]
    n = F // ad.merge
    out = torch.full((B, n, ad.down.codes.shape[0]), float("nan"), device="cuda")
    mid = torch.full((B, n, ad.up.codes.shape[0]), float("nan"), device="cuda")
    ark.audio_adapter(ad, t(frames_np), out, mid)
    return host(out), host(mid)


SMALL = synth.SMALL


@pytest.fixture(scope="module")
def small_ad():
    return oracle.build_adapter(SMALL, synth), ark.load_adapter(SMALL, synth)


@pytest.mark.parametrize("B,frames", [(1, 39), (3, 39), (2, 40), (1, 4), (2, 7), (3, 200),
                                      (1, 700), (3, 700)])
def test_adapter_small(small_ad, B, frames):
    ad_o, ad = small_ad
    f = synth.encoder_frames(SMALL.with_(batch=B), frames)
    f[-1] *= 3.0                                      # sequences of different range
    out, mid = _run(ad, f)
    _check(ad_o, f, out, mid, range(B), f"B={B} frames={frames}")


def test_adapter_without_mid_output(small_ad):
    """The same rows when the GELU output is not requested."""
    _, ad = small_ad
    f = synth.encoder_frames(SMALL.with_(batch=2), 41)
    out1, _ = _run(ad, f)
    out2 = torch.empty((2, 10, SMALL.hidden), device="cuda")
    ark.audio_adapter(ad, t(f), out2)
    assert np.array_equal(host(out2), out1)


def test_adapter_zero_frames_give_bias_rows(small_ad):
    """All-zero input: the quantiser's s = 0 case (codes 0, output = bias
    through GELU of the first bias)."""
    ad_o, ad = small_ad
    f = np.zeros((1, 8, SMALL.frame_dim), F32)
    out, mid = _run(ad, f)
    _check(ad_o, f, out, mid, [0], "zeros")


def test_frames_adapter_splice_prefill_pipeline():
    """frames -> adapter -> audio-slot splice -> prefill -> greedy token, at
    the small geometry, against the oracle's chain."""
    cfg = SMALL
    ad_o, ad = oracle.build_adapter(cfg, synth), ark.load_adapter(cfg, synth)
    om, gm = oracle.build_model(cfg, synth), ark.load_model(cfg, synth)
    f = synth.encoder_frames(cfg)
    n = cfg.enc_frames // cfg.merge
    assert n == cfg.audio_slots
    rows = torch.empty((1, n, cfg.hidden), device="cuda")
    ark.audio_adapter(ad, t(f), rows)
    ids = synth.prompt_ids(cfg)
    x = torch.empty((1, cfg.prefill_len, cfg.hidden), device="cuda")
    ark.embed_splice(gm.dims, t(ids), gm.embed_f16, rows, cfg.audio_offset, x)
    gs = GpuState(gm, 1, cfg.prefill_len)
    kd, vd = gs.deltas(cfg.prefill_len)
    ark.prefill(gm, x, [0], gs.kc, gs.vc, kd, vd, gs.logits, ws=gs.ws)
    tok = torch.empty(1, dtype=torch.int32, device="cuda")
    ark.masked_argmax(gs.logits, t(cfg.mask()), tok)
    rows_o = oracle.adapter(ad_o, f)
    assert_close(host(rows), rows_o, "adapter rows", 1e-4)
    x_o = oracle.embed_splice(om.embed, ids, rows_o, cfg.audio_offset)
    assert_close(host(x), x_o, "spliced prompt", 1e-4)
    zero = np.zeros((1, cfg.max_total_len, cfg.n_kv_heads, cfg.head_dim), F32)
    lo, _, _, _ = oracle.prefill(om, x_o, np.array([0]), [zero] * cfg.n_layers, [zero] * cfg.n_layers)
    err = assert_close(host(gs.logits), lo, "pipeline logits")
    check_tokens(host(tok), oracle.masked_argmax(lo, cfg.mask()), lo, cfg.mask(),
                 err * np.max(np.abs(lo)), "pipeline token")


# ------------------------------------------------------------- full size --
FULL1 = synth.CONFIGS["c1"]


@pytest.fixture(scope="module")
def full_ad():
    return oracle.build_adapter(FULL1, synth), ark.load_adapter(FULL1, synth)


def test_adapter_full_c1(full_ad):
    """The 3 s clip: 150 frames -> 37 rows of 2048 (two frames dropped)."""
    ad_o, ad = full_ad
    f = synth.encoder_frames(FULL1)
    out, mid = _run(ad, f)
    assert out.shape == (1, 37, 2048)
    _check(ad_o, f, out, mid, [0], "c1")


def test_adapter_full_c4_sampled(full_ad):
    """Sixteen 30 s clips (1500 frames each, 6000 merged rows through the
    large-tile GEMM); sequences 0, 7 and 15 checked in full."""
    ad_o, ad = full_ad
    c4 = synth.CONFIGS["c4"]
    f = synth.encoder_frames(c4)
    assert f.shape == (16, 1500, 1280)
    out, mid = _run(ad, f)
    _check(ad_o, f, out, mid, [0, 7, 15], "c4")
    assert np.all(np.isfinite(out))
