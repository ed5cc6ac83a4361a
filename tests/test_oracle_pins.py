"""Pins of the CPU oracle against facts other than the oracle itself.

Each test checks one oracle function against the pages' printed numbers, a
closed form, an invariant of the operation, a special case that reduces to a
textbook result, or brute force on a tiny input.  The set is chosen so that a
plausible slip (a dropped term, a wrong sign or index, a transposed operand,
a wrong rounding mode) fails at least one of them.
"""
import math
import struct

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def f32(x: float) -> float:
    """Round a Python float (binary64) to the nearest binary32 (ties to even)."""
    return struct.unpack("f", struct.pack("f", x))[0]


# ------------------------------------------------------------ audio slots --
def test_audio_slots_printed_formula_values():
    # model card "Inference" step 4 applied to a 3 s and a 30 s 16 kHz clip
    assert oracle.n_audio_slots(48000) == 37
    assert oracle.n_audio_slots(480000) == 375
    # the clamp to at least one slot
    assert oracle.n_audio_slots(0) == 1
    assert oracle.n_audio_slots(1119) == 1
    assert oracle.n_audio_slots(1120) == 1
    assert oracle.n_audio_slots(2399) == 1
    assert oracle.n_audio_slots(2400) == 2


def test_audio_slots_agree_with_cookbook_mel_formula():
    # cookbook "Audio Handling": (mel_frames + 1) // 2 // merge_factor with the
    # mel length of an unpadded clip at hop 160; the two pages agree above the clamp
    for samples in list(range(0, 20000, 37)) + [48000, 160000, 480000]:
        mel = samples // 160
        assert oracle.n_audio_slots(samples) == max(oracle.n_audio_slots_from_mel(mel, 4), 1)


def test_synthetic_prompt_lengths_match_slot_formula():
    assert synth.CONFIGS["c1"].prefill_len == 2 + oracle.n_audio_slots(48000) + 10 == 49
    assert synth.CONFIGS["c2"].prefill_len == 2 + oracle.n_audio_slots(480000) + 10 == 387


def test_vocab_matches_embedding_bytes():
    # model card "Revision history": the fp32 table is 1.24 GB and the fp16 one
    # 622 MB at hidden 2048; the chosen vocabulary reproduces both figures
    V, H = synth.CONFIGS["c1"].vocab, synth.CONFIGS["c1"].hidden
    assert round(V * H * 2 / 1e6) == 622
    assert round(V * H * 4 / 1e9, 2) == 1.24


def test_block_parameter_count_of_the_06b_sibling():
    # Audio8 article, table of tensor counts: the 0.6B decoder stack plus final
    # norm holds 357,898,112 parameters at hidden 896.  With 24 layers, a
    # 2 x 64 KV width and FFN 4864 this is reproduced only with q/k/v biases.
    per_layer = oracle.layer_param_count(896, 128, 4864)
    assert 24 * per_layer + 896 == 357_898_112
    no_bias = per_layer - (896 + 2 * 128)
    assert 24 * no_bias + 896 != 357_898_112


# -------------------------------------------------------- weight quantiser --
def test_prep_weight_invariants():
    rng = np.random.default_rng(0)
    w = (rng.standard_normal((37, 300)) * 0.02).astype(np.float32)
    w[5] = 0.0
    q, s = oracle.prep_weight(w)
    assert q.dtype == np.int8 and s.dtype == np.float32
    assert np.all(np.abs(q.astype(int)) <= 127)
    assert s[5] == 0 and np.all(q[5] == 0)
    for n in range(37):
        if n == 5:
            continue
        j = int(np.argmax(np.abs(w[n])))
        assert abs(int(q[n, j])) == 127 and np.sign(q[n, j]) == np.sign(w[n, j])
        err = np.abs(q[n].astype(np.float64) * float(s[n]) - w[n].astype(np.float64))
        assert np.all(err <= 0.5 * float(s[n]) * (1 + 1e-5))
    # exact power-of-two scaling leaves codes unchanged and doubles scales
    q2, s2 = oracle.prep_weight(w * np.float32(2))
    assert np.array_equal(q, q2) and np.array_equal(s2, s * np.float32(2))


def test_prep_weight_brute_force():
    rng = np.random.default_rng(1)
    w = (rng.standard_normal((4, 9)) * 0.02).astype(np.float32)
    q, s = oracle.prep_weight(w)
    for n in range(4):
        amax = max(abs(float(v)) for v in w[n])
        sn = f32(amax / 127.0)
        assert sn == float(s[n])
        for k in range(9):
            c = round(f32(float(w[n, k]) / sn))     # round() is half-to-even
            assert int(q[n, k]) == max(-127, min(127, c))


# ---------------------------------------------------- activation quantiser --
def _bf_dynquant(xs):
    lo = min(0.0, min(xs))
    hi = max(0.0, max(xs))
    s = f32(f32(hi - lo) / 255.0)
    if s == 0.0:
        return [0] * len(xs), 0.0, 0
    z = max(0, min(255, round(f32(-lo / s))))
    return [max(0, min(255, round(f32(x / s)) + z)) for x in xs], s, z


def test_dynquant_brute_force():
    rng = np.random.default_rng(2)
    for trial in range(40):
        n = int(rng.integers(1, 50))
        x = (rng.standard_normal(n) * rng.uniform(0.01, 10)).astype(np.float32)
        if trial % 5 == 1:
            x = np.abs(x)            # all >= 0: range widened down to 0
        if trial % 5 == 2:
            x = -np.abs(x)           # all <= 0
        q, s, z = oracle.dynquant(x)
        bq, bs, bz = _bf_dynquant([float(v) for v in x])
        assert float(s) == bs and int(z) == bz
        assert [int(v) for v in q] == bq


def test_dynquant_hand_example():
    # x = [-1, 0, 3]: s = 4/255, z = rne(63.75) = 64, codes 0, 64, rne(191.25)+64 = 255
    q, s, z = oracle.dynquant(np.array([-1.0, 0.0, 3.0], np.float32))
    assert float(s) == f32(4.0 / 255.0) and int(z) == 64
    assert q.tolist() == [0, 64, 255]


def test_dynquant_invariants():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((7, 513)) * 3).astype(np.float32)
    x[2, 7] = 0.0
    q, s, z = oracle.dynquant(x)
    s, z = float(s), int(z)
    assert q[2, 7] == z                                        # zero is exact
    assert q.flat[np.argmin(x)] == 0                           # the minimum maps to 0
    assert q.flat[np.argmax(x)] in (254, 255)                  # the maximum to the top
    rec = s * (q.astype(np.float64) - z)
    err = np.abs(rec - x.astype(np.float64))
    inner = (q > 0) & (q < 255)
    assert np.all(err[inner] <= 0.5 * s * (1 + 1e-5))
    assert np.all(err <= 1.5 * s)
    # one (s, z) per tensor: quantising the flattened tensor is the same
    q2, s2, z2 = oracle.dynquant(x.reshape(-1))
    assert np.array_equal(q.reshape(-1), q2) and float(s2) == s and int(z2) == z
    # exact power-of-two scaling: same codes and zero point, doubled scale
    q3, s3, z3 = oracle.dynquant(x * np.float32(2))
    assert np.array_equal(q, q3) and int(z3) == z and float(s3) == 2 * s


def test_dynquant_all_zero():
    q, s, z = oracle.dynquant(np.zeros(10, np.float32))
    assert float(s) == 0.0 and int(z) == 0 and not q.any()


# ------------------------------------------------------------ int8 linear --
def test_matmul_integer_brute_force():
    rng = np.random.default_rng(4)
    a = rng.integers(0, 256, (3, 11)).astype(np.uint8)
    w = rng.integers(-127, 128, (5, 11)).astype(np.int8)
    z = 131
    acc = oracle.matmul_integer(a, z, w)
    for r in range(3):
        for n in range(5):
            assert acc[r, n] == sum((int(a[r, k]) - z) * int(w[n, k]) for k in range(11))


def test_matmul_integer_extreme_is_exact():
    # the largest accumulator of the real shape: K = 11008, all (255 - 0) * 127
    a = np.full((1, 11008), 255, np.uint8)
    w = np.full((2, 11008), 127, np.int8)
    w[1] = -127
    acc = oracle.matmul_integer(a, 0, w)
    assert acc[0, 0] == 255 * 127 * 11008 and acc[0, 1] == -255 * 127 * 11008


def test_dequant_closed_form():
    rng = np.random.default_rng(5)
    acc = rng.integers(-2**28, 2**28, (2, 6))
    sw = (rng.uniform(1e-4, 1e-3, 6)).astype(np.float32)
    b = (rng.standard_normal(6) * 0.02).astype(np.float32)
    s = np.float32(0.0123)
    y = oracle.dequant(acc, s, sw, b)
    for r in range(2):
        for n in range(6):
            m = f32(float(s) * float(sw[n]))
            want = f32(f32(f32(float(acc[r, n])) * m) + float(b[n]))
            assert float(y[r, n]) == want


def test_qlinear_approximates_float_linear_within_quantisation_bound():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((4, 256)).astype(np.float32)
    w = (rng.standard_normal((96, 256)) * 0.02).astype(np.float32)
    b = (rng.standard_normal(96) * 0.02).astype(np.float32)
    wq, sw = oracle.prep_weight(w)
    codes, s, z = oracle.dynquant(x)
    y = oracle.qlinear(codes, s, z, wq, sw, b)
    ref = x.astype(np.float64) @ w.astype(np.float64).T + b
    # |x_hat w_hat - x w| <= sum_k |x_hat||dw| + |dx||w| with |dx| <= s/2, |dw| <= sw/2
    xh = float(s) * (codes.astype(np.float64) - int(z))
    bound = (np.abs(xh) @ np.broadcast_to(sw.astype(np.float64)[:, None] / 2, (96, 256)).T
             + float(s) / 2 * np.abs(w.astype(np.float64)).sum(1)[None, :]) * (1 + 1e-4) + 1e-6
    assert np.all(np.abs(y - ref) <= bound)
    # and it is close in the plain sense too (rules out a transposed operand)
    assert np.max(np.abs(y - ref)) / np.max(np.abs(ref)) < 0.03


# ------------------------------------------------------------- float ops --
def test_rmsnorm_closed_forms():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((5, 2048)) * rng.uniform(0.1, 10, (5, 1))).astype(np.float32)
    g = np.ones(2048, np.float32)
    y = oracle.rmsnorm(x, g, 0.0).astype(np.float64)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-6)
    eps = 0.5
    y = oracle.rmsnorm(x, g, eps).astype(np.float64)
    ms = np.mean(x.astype(np.float64) ** 2, axis=1)
    assert np.allclose(np.mean(y * y, axis=1), ms / (ms + eps), rtol=1e-6)
    # scale invariance without eps, and the gain multiplies elementwise
    gg = (1 + 0.02 * rng.standard_normal(2048)).astype(np.float32)
    a = oracle.rmsnorm(x, gg, 0.0).astype(np.float64)
    c = oracle.rmsnorm(x * np.float32(4), gg, 0.0).astype(np.float64)
    assert np.allclose(a, c, rtol=1e-6, atol=0)
    assert np.allclose(a / gg, oracle.rmsnorm(x, g, 0.0), rtol=1e-6)


def test_rope_complex_rotation_and_invariants():
    T, D, theta = 64, 128, 1e6
    cos, sin = oracle.rope_tables(T, D, theta)
    # frequencies: pair 0 turns one radian per position; pair j by theta^(-2j/D)
    assert cos[1, 0] == math.cos(1.0) and sin[1, 0] == math.sin(1.0)
    assert abs(math.atan2(sin[1, 63], cos[1, 63]) - theta ** (-126 / 128)) < 1e-18
    rng = np.random.default_rng(8)
    x = rng.standard_normal((6, D)).astype(np.float32)
    pos = np.array([0, 1, 5, 17, 40, 63])
    y = oracle.apply_rope(x, pos, cos, sin)
    assert np.array_equal(y[0], x[0])                          # position 0: identity
    for r, p in enumerate(pos):
        zc = x[r, :64].astype(np.float64) + 1j * x[r, 64:].astype(np.float64)
        inv = theta ** (-(2.0 * np.arange(64)) / D)
        rot = zc * np.exp(1j * p * inv)                        # textbook complex form
        assert np.allclose(y[r, :64], rot.real, rtol=0, atol=1e-6)
        assert np.allclose(y[r, 64:], rot.imag, rtol=0, atol=1e-6)
        n0 = x[r, :64].astype(np.float64) ** 2 + x[r, 64:].astype(np.float64) ** 2
        n1 = y[r, :64].astype(np.float64) ** 2 + y[r, 64:].astype(np.float64) ** 2
        assert np.allclose(n0, n1, rtol=1e-6)
    # <rope(q, m), rope(k, n)> depends on m - n only
    q, k = x[1:2], x[2:3]
    dots = []
    for m, n in [(10, 3), (20, 13), (63, 56)]:
        a = oracle.apply_rope(q, np.array([m]), cos, sin).astype(np.float64)
        b = oracle.apply_rope(k, np.array([n]), cos, sin).astype(np.float64)
        dots.append(float((a @ b.T)[0, 0]))
    assert np.allclose(dots, dots[0], rtol=1e-5)


def _bf_attention(q, k, v, p):
    # pure-Python softmax attention over the valid prefix only
    S, NH, D = q.shape
    G = NH // k.shape[1]
    out = np.zeros((S, NH, D))
    for i in range(S):
        for h in range(NH):
            g = h // G
            sc = [sum(float(q[i, h, d]) * float(k[j, g, d]) for d in range(D)) / math.sqrt(D)
                  for j in range(p + i + 1)]
            m = max(sc)
            e = [math.exp(t - m) for t in sc]
            tot = sum(e)
            for d in range(D):
                out[i, h, d] = sum(e[j] * float(v[j, g, d]) for j in range(p + i + 1)) / tot
    return out.reshape(S, NH * D)


def test_attention_brute_force_and_masking():
    rng = np.random.default_rng(9)
    T, NH, NKV, D, S, p = 12, 4, 2, 8, 3, 4
    q = rng.standard_normal((S, NH, D)).astype(np.float32)
    k = rng.standard_normal((T, NKV, D)).astype(np.float32)
    v = rng.standard_normal((T, NKV, D)).astype(np.float32)
    o = oracle.attention(q, k, v, p)
    assert np.allclose(o, _bf_attention(q, k, v, p), rtol=1e-6, atol=1e-7)
    # rows past p + S are masked for every query: garbage there has no effect
    k2, v2 = k.copy(), v.copy()
    k2[p + S:] = np.nan
    v2[p + S:] = np.inf
    assert np.array_equal(oracle.attention(q, k2, v2, p), o)
    # full-T with masking equals attention over the valid prefix only
    assert np.array_equal(oracle.attention(q, k[:p + S], v[:p + S], p), o)


def test_attention_single_valid_row_returns_it():
    rng = np.random.default_rng(10)
    q = rng.standard_normal((1, 4, 16)).astype(np.float32)
    k = rng.standard_normal((9, 2, 16)).astype(np.float32)
    v = rng.standard_normal((9, 2, 16)).astype(np.float32)
    o = oracle.attention(q, k, v, 0).reshape(4, 16)
    assert np.array_equal(o[:2], np.broadcast_to(v[0, 0], (2, 16)))
    assert np.array_equal(o[2:], np.broadcast_to(v[0, 1], (2, 16)))


def test_attention_uniform_scores_average_values():
    rng = np.random.default_rng(11)
    q = np.zeros((2, 2, 8), np.float32)
    k = rng.standard_normal((6, 1, 8)).astype(np.float32)
    v = rng.standard_normal((6, 1, 8)).astype(np.float32)
    o = oracle.attention(q, k, v, 2).reshape(2, 2, 8)
    assert np.allclose(o[0, 0], v[:3, 0].astype(np.float64).mean(0), rtol=1e-6)
    assert np.allclose(o[1, 1], v[:4, 0].astype(np.float64).mean(0), rtol=1e-6)


def test_gqa_equals_mha_with_replicated_kv():
    rng = np.random.default_rng(12)
    T, NH, NKV, D, S, p = 10, 16, 2, 16, 2, 5
    q = rng.standard_normal((S, NH, D)).astype(np.float32)
    k = rng.standard_normal((T, NKV, D)).astype(np.float32)
    v = rng.standard_normal((T, NKV, D)).astype(np.float32)
    o = oracle.attention(q, k, v, p)
    km = np.repeat(k, NH // NKV, axis=1)
    vm = np.repeat(v, NH // NKV, axis=1)
    assert np.array_equal(oracle.attention(q, km, vm, p), o)


def test_swiglu_closed_form():
    g = np.array([0.0, 1.0, -1.0, 30.0, -30.0, 0.5], np.float32)
    u = np.array([2.0, 3.0, 3.0, 1.0, 1.0, -4.0], np.float32)
    y = oracle.swiglu(g, u)
    for i in range(6):
        want = f32(float(g[i]) / (1 + math.exp(-float(g[i]))) * float(u[i]))
        assert float(y[i]) == want
    assert y[0] == 0.0 and abs(float(y[3]) - 30.0) < 1e-6 and abs(float(y[4])) < 1e-10


# ---------------------------------------------------------- host-side ops --
def test_masked_argmax_forced_cases():
    V = 20
    mask = np.zeros(V, np.uint8)
    mask[13:] = 1                        # added ids 12..19, end id 12 unmasked
    lg = np.zeros((5, V), np.float32)
    lg[0, 15] = 9.0
    lg[0, 3] = 5.0                       # masked raw max loses to id 3
    lg[1, 12] = 4.0                      # the end id can win
    lg[2, :] = -1.0
    lg[2, 7] = lg[2, 2] = 0.5            # tie -> lowest id
    lg[3, :] = np.nan
    lg[3, 6] = -3.0                      # NaN never chosen
    lg[4, :13] = np.nan                  # nothing but masked ids left
    out = oracle.masked_argmax(lg, mask)
    assert out.tolist() == [3, 12, 2, 6, -1]
    assert out.tolist()[:3] == [int(np.argmax(np.where(mask == 1, -np.inf, lg[b]))) for b in range(3)]


def test_cache_write_touches_only_delta_rows():
    rng = np.random.default_rng(13)
    c = rng.standard_normal((3, 10, 2, 4)).astype(np.float32)
    d = rng.standard_normal((3, 2, 2, 4)).astype(np.float32)
    p = np.array([0, 4, 8])
    out = oracle.cache_write(c, d, p)
    for b in range(3):
        assert np.array_equal(out[b, p[b]:p[b] + 2], d[b])
        keep = np.ones(10, bool)
        keep[p[b]:p[b] + 2] = False
        assert np.array_equal(out[b, keep], c[b, keep])


def test_embed_splice():
    rng = np.random.default_rng(14)
    table = rng.standard_normal((30, 8)).astype(np.float16)
    ids = rng.integers(0, 30, (2, 7))
    audio = rng.standard_normal((2, 3, 8)).astype(np.float32)
    x = oracle.embed_splice(table, ids, audio, 2)
    assert x.dtype == np.float32
    assert np.array_equal(x[:, :2], table[ids[:, :2]].astype(np.float32))
    assert np.array_equal(x[:, 2:5], audio)
    assert np.array_equal(x[:, 5:], table[ids[:, 5:]].astype(np.float32))
