"""Pins of the oracle's frame merge and int8 MLP adapter (model card
"ark-asr-3b-onnx", "Inference" steps 2-3 and "Files"; Audio8 article, "What
arkasr actually is").

  * the adapter's structure by the parameter count the Audio8 article
    prints for the 0.6B model (two linear layers with biases, inner width
    twice the hidden width);
  * the frame merge by brute-force index mapping and by the card's slot
    count (merged rows of a clip == its <|audio|> slots);
  * GELU by x Phi(x) with Phi integrated numerically (no erf), its odd-part
    identity and its limits;
  * the whole adapter by a pure-Python brute force at a tiny geometry
    (integer loops, binary32 rounding emulated with struct, binary64 GELU
    from the same numerical Phi).
"""
import math
import struct

import numpy as np
import pytest

import oracle
import synth


def f32(x: float) -> float:
    return struct.unpack("f", struct.pack("f", x))[0]


def test_adapter_structure_from_the_printed_parameter_count():
    # Audio8 article: the 0.6B model's audio_encoder.adapting.* tensors hold
    # 10,783,360 parameters; its decoder is 896 wide and merges 4 frames of
    # the 1280-wide encoder output (card "Inference" step 2).
    assert oracle.adapter_param_count(1280, 4, 2 * 896, 896) == 10_783_360
    # no other inner width of two biased layers gives the printed count
    hits = [i for i in range(1, 8192) if oracle.adapter_param_count(1280, 4, i, 896) == 10_783_360]
    assert hits == [1792]
    # the reading for the 3B adapter: inner width twice its hidden width
    assert synth.CONFIGS["c1"].adapter_inner == 2 * synth.CONFIGS["c1"].hidden


def test_frame_merge_brute_force():
    rng = np.random.default_rng(3)
    for seq, D in ((9, 3), (8, 5), (3, 4), (0, 2), (17, 1)):
        f = rng.standard_normal((seq, D)).astype(np.float32)
        m = oracle.frame_merge(f, 4)
        n = seq // 4
        assert m.shape == (n, 4 * D)
        for r in range(n):
            for j in range(4):
                for d in range(D):
                    assert m[r, j * D + d] == f[4 * r + j, d]


def test_merged_rows_fill_the_audio_slots():
    # card "Inference": N = max(((samples // 160) + 1) // 2 // 4, 1) slots;
    # the encoder frames before the merge are ((samples // 160) + 1) // 2
    assert oracle.n_encoder_frames(48000) == 150       # the 3 s clip
    assert oracle.n_encoder_frames(480000) == 1500     # the 30 s clip
    for samples in list(range(0, 20000, 37)) + [48000, 480000, 479999]:
        frames = oracle.n_encoder_frames(samples)
        rows = oracle.frame_merge(np.zeros((frames, 1), np.float32)).shape[0]
        assert max(rows, 1) == oracle.n_audio_slots(samples)
    for name in ("c1", "c2"):
        cfg = synth.CONFIGS[name]
        assert cfg.enc_frames // cfg.merge == cfg.audio_slots


def _simpson(f, a: float, b: float, n: int) -> float:
    h = (b - a) / n
    s = f(a) + f(b)
    for i in range(1, n):
        s += (4.0 if i % 2 else 2.0) * f(a + i * h)
    return s * h / 3.0


def phi(x: float, n: int = 4000) -> float:
    """Standard normal CDF by composite Simpson integration of the density
    (binary64, no erf): 0.5 plus the integral over [0, x] for x >= 0, the
    left tail over [x - 12, x] for x < 0 (no cancellation for small
    values; the density beyond 12 more is below 1e-31 of it)."""
    f = lambda t: math.exp(-0.5 * t * t) / math.sqrt(2.0 * math.pi)  # noqa: E731
    if x >= 0.0:
        return 0.5 + (_simpson(f, 0.0, x, n) if x > 0.0 else 0.0)
    return _simpson(f, x - 12.0, x, n)


def test_gelu_against_integrated_phi():
    xs = [-6.0, -3.0, -2.5, -1.0, -0.5, -1e-3, 0.0, 1e-3, 0.25, 0.5, 1.0, 1.7, 2.0, 3.0, 4.5, 6.0]
    got = oracle.gelu(np.array(xs, np.float32))
    for x, g in zip(xs, got):
        want = f32(x * phi(x))
        if want == 0.0:
            assert g == 0.0
        else:
            assert abs(float(g) - want) <= abs(want) * 2.0 ** -23, (x, g, want)
    # textbook value: Phi(1) = 0.841344746...
    assert abs(float(oracle.gelu(np.array([1.0], np.float32))[0]) - 0.8413447460685429) < 1e-7


def test_gelu_identities():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(5000) * 3).astype(np.float32)
    g = oracle.gelu(x).astype(np.float64)
    gn = oracle.gelu(-x).astype(np.float64)
    # x Phi(x) - (-x) Phi(-x) = x: each side rounded once to fp32
    ulp = np.spacing(np.abs(g).astype(np.float32)).astype(np.float64) + \
        np.spacing(np.abs(gn).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(g - gn - x) <= ulp)
    big = np.array([8.0, 20.0, 1e4], np.float32)
    assert np.array_equal(oracle.gelu(big), big)               # Phi == 1 in binary64
    assert np.all(oracle.gelu(-big) <= 0) and np.all(oracle.gelu(-big) > -1e-13)
    assert oracle.gelu(np.array([0.0], np.float32))[0] == 0.0


# ------------------------------------------------------- brute force --
def bf_prep(rows):
    codes, scales = [], []
    for r in rows:
        s = f32(max(abs(v) for v in r) / 127.0)
        scales.append(s)
        codes.append([0] * len(r) if s == 0.0 else
                     [max(-127, min(127, round(f32(v / s)))) for v in r])
    return codes, scales


def bf_quant(vals):
    lo = min(0.0, min(vals))
    hi = max(0.0, max(vals))
    s = f32(f32(hi - lo) / 255.0)
    if s == 0.0:
        return [0] * len(vals), 0.0, 0
    z = max(0, min(255, round(f32(-lo / s))))
    return [max(0, min(255, round(f32(v / s)) + z)) for v in vals], s, z


def bf_linear(rows, s, z, W, bias):
    codes, ws = W
    out = []
    for r in rows:
        y = []
        for n in range(len(codes)):
            acc = sum((c - z) * w for c, w in zip(r, codes[n]))
            y.append(f32(f32(f32(float(acc)) * f32(s * ws[n])) + bias[n]))
        out.append(y)
    return out


def bf_adapter(w, frames, merge, D):
    """frames: list of [seq][D] lists for one sequence."""
    n = len(frames) // merge
    rows = [[frames[merge * r + j][d] for j in range(merge) for d in range(D)] for r in range(n)]
    flat = [v for r in rows for v in r]
    c, s, z = bf_quant(flat)
    K1 = merge * D
    crow = [c[i * K1:(i + 1) * K1] for i in range(n)]
    y = bf_linear(crow, s, z, bf_prep(w["w1"].tolist()), w["b1"].tolist())
    a = [[f32(v * phi(v, 2000)) for v in r] for r in y]
    flat = [v for r in a for v in r]
    c2, s2, z2 = bf_quant(flat)
    I = len(a[0])
    crow = [c2[i * I:(i + 1) * I] for i in range(n)]
    return bf_linear(crow, s2, z2, bf_prep(w["w2"].tolist()), w["b2"].tolist()), (c, s, z), (c2, s2, z2)


@pytest.mark.parametrize("frames", [10, 13, 4])
def test_adapter_matches_brute_force(frames):
    cfg = synth.TINY.with_(batch=2)
    w = synth.adapter_weights(cfg)
    ad = oracle.build_adapter(cfg, synth)
    f = synth.encoder_frames(cfg, frames)
    got = oracle.adapter(ad, f)
    assert got.shape == (2, frames // 4, cfg.hidden)
    for b in range(2):
        want, q1, q2 = bf_adapter(w, f[b].tolist(), cfg.merge, cfg.frame_dim)
        # the first quantisation is exact; GELU (erf vs integrated Phi) may
        # move a value by an ulp, so the rest is checked to 1e-6
        c, s, z = oracle.dynquant(oracle.frame_merge(f[b]))
        assert list(c.reshape(-1)) == q1[0] and float(s) == q1[1] and int(z) == q1[2]
        np.testing.assert_allclose(got[b], np.array(want, np.float32), rtol=0, atol=1e-6 * np.max(np.abs(want)))


def test_adapter_per_sequence_quantisation():
    # one (s, z) per sequence: a batch gives the rows of each sequence alone
    cfg = synth.TINY.with_(batch=3)
    ad = oracle.build_adapter(cfg, synth)
    f = synth.encoder_frames(cfg, 14)
    f[1] *= 7.0
    both = oracle.adapter(ad, f)
    for b in range(3):
        assert np.array_equal(both[b], oracle.adapter(ad, f[b:b + 1])[0])
