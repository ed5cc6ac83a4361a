"""Pins of the oracle's weight-only int4 LM tier (model card "ark-asr-3b-onnx",
"Revision history": v2 added a weight-only int4 LM tier; the Audio8 article,
"What INT8 and INT4 actually buy": measured fp32 / INT4 size ratios of an
ONNX decoder).

The pages name the tier, not its format; the block format and the block
size are readings, and these tests pin them to what the pages print and to
the arithmetic of the format itself."""
import math
import struct

import numpy as np
import pytest

import oracle
import synth


def f32(x: float) -> float:
    return struct.unpack("f", struct.pack("f", x))[0]


def test_block_size_from_the_printed_size_ratios():
    # Audio8 article: the 0.1B decoder graphs are 395.0 MB in fp32 and 53.1 MB
    # as INT4 (7.45x prefill, 7.44x decode), "mostly quantization overhead
    # (scale/zero-point tensors, a handful of ops left at higher precision)".
    # 4-bit codes with an fp32 scale and a 4-bit zero point per block: only a
    # block of 128 lands within 0.05 of the printed ratio, and just above it
    # (the ops left at higher precision lower the real ratio further).
    printed = 395.0 / 53.1
    assert round(printed, 2) == 7.44 or round(printed, 2) == 7.45
    near = {b: oracle.int4_size_ratio(b) for b in (32, 64, 128, 256, 512)}
    best = min(near, key=lambda b: abs(near[b] - printed))
    assert best == oracle.INT4_BLOCK == 128
    assert abs(near[128] - printed) < 0.05 and near[128] >= printed
    # the INT8 ratio of the same table (3.95x) is the per-channel int8 format
    assert abs(4.0 / (1.0 + 4.0 / 1024) - 3.95) < 0.05


def _bf_block(vals):
    lo = min(0.0, min(vals))
    hi = max(0.0, max(vals))
    s = f32(f32(hi - lo) / 15.0)
    if s == 0.0:
        return [0] * len(vals), 0.0, 0
    z = max(0, min(15, round(f32(-lo / s))))
    return [max(0, min(15, round(f32(v / s)) + z)) for v in vals], s, z


def test_int4_prep_brute_force():
    rng = np.random.default_rng(5)
    for trial in range(12):
        n = int(rng.integers(1, 5))
        blocks = int(rng.integers(1, 4))
        w = (rng.standard_normal((n, 128 * blocks)) * 0.02).astype(np.float32)
        if trial % 4 == 1:
            w = np.abs(w)                    # all >= 0: range widened down to 0
        if trial % 4 == 2:
            w[0, :128] = 0.0                 # a zero block
        q, s, z = oracle.prep_weight_int4(w)
        assert q.dtype == np.uint8 and s.dtype == np.float32 and z.dtype == np.uint8
        for r in range(n):
            for j in range(blocks):
                bq, bs, bz = _bf_block([float(v) for v in w[r, 128 * j:128 * (j + 1)]])
                assert float(s[r, j]) == bs and int(z[r, j]) == bz
                assert [int(v) for v in q[r, 128 * j:128 * (j + 1)]] == bq


def test_int4_prep_invariants():
    rng = np.random.default_rng(6)
    w = (rng.standard_normal((40, 512)) * 0.02).astype(np.float32)
    q, s, z = oracle.prep_weight_int4(w)
    assert q.max() <= 15 and z.max() <= 15
    wd = oracle.dequant_weight_int4(q, s, z)
    err = np.abs(wd.astype(np.float64) - w.astype(np.float64))
    bound = np.repeat(s.astype(np.float64), 128, axis=1) * 0.5 * (1 + 1e-5)
    assert np.all(err <= bound)
    # each block's extremes sit on the ends of the code range (up to the
    # rounding of the zero point)
    wb = w.reshape(40, 4, 128)
    qb = q.reshape(40, 4, 128)
    ia, ib = np.argmin(wb, axis=2), np.argmax(wb, axis=2)
    lo = np.take_along_axis(qb, ia[..., None], 2)[..., 0]
    hi = np.take_along_axis(qb, ib[..., None], 2)[..., 0]
    assert np.all(lo <= 1) and np.all(hi >= 14)
    # the exact zero is representable: code z dequantises to 0
    assert np.all(oracle.dequant_weight_int4(z.repeat(128, axis=1), s, z) == 0)


def test_int4_lm_head_closed_form_and_tracks_float():
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((30, 256)) * 0.02).astype(np.float32)
    h = rng.standard_normal((3, 256)).astype(np.float32)
    q, s, z = oracle.prep_weight_int4(w)
    lg = oracle.lm_head_int4(h, q, s, z)
    wd = oracle.dequant_weight_int4(q, s, z)
    for b in range(3):
        for n in range(30):
            exact = math.fsum(float(h[b, k]) * float(wd[n, k]) for k in range(256))
            assert abs(float(lg[b, n]) - exact) <= abs(exact) * 2 ** -23 + 1e-30
    ref = h.astype(np.float64) @ w.astype(np.float64).T
    assert np.corrcoef(lg.ravel(), ref.ravel())[0, 1] > 0.98


def test_int4_tier_in_the_model_uses_the_unquantised_final_norm():
    cfg = synth.TINY.with_(hidden=128, n_heads=4, head_dim=32, n_kv_heads=2, intermediate=96)
    om = oracle.build_model(cfg, synth, lm_head4=True)
    x = np.random.default_rng(8).standard_normal((2, 3, cfg.hidden)).astype(np.float32)
    zero = np.zeros((2, cfg.max_total_len, cfg.n_kv_heads, cfg.head_dim), np.float32)
    lg, _, _, h = oracle.forward(om, x, np.array([0, 0]), [zero] * 2, [zero] * 2)
    hn = oracle.rmsnorm(h[:, -1], om.final_norm, cfg.rms_eps)
    assert np.array_equal(lg, oracle.lm_head_int4(hn, *om.lm_head4))
    # and not the int8 head's quantised input
    om8 = oracle.OracleModel(**{**om.__dict__, "lm_head4": None})
    lg8, _, _, _ = oracle.forward(om8, x, np.array([0, 0]), [zero] * 2, [zero] * 2)
    assert not np.array_equal(lg, lg8)
    assert np.corrcoef(lg.ravel(), lg8.ravel())[0, 1] > 0.97
