"""Pins of the oracle's audio encoder (model card "ark-asr-3b-onnx",
"Inference" step 1 and "Files"; cookbook "ARK-ASR-3B" introduction and
clover "Inside ARK-ASR-3B's Whisper and Qwen architecture": a Whisper-style
tower with rotary self-attention; Audio8 article, "What arkasr actually is":
the encoder's printed parameter count).

  * the structure by the printed count 636,968,960, which among the nearby
    variants only this one reaches;
  * the frame counts by the card's slot formula (300 / 3000 mel frames ->
    150 / 1500 encoder frames, the table's 1500 rows at 30 s);
  * im2col against a direct convolution written as loops;
  * LayerNorm by brute force and its invariants;
  * bidirectional attention against a pure-Python softmax and its
    identities;
  * the whole encoder at a tiny geometry against a pure-Python brute force
    (integer loops, binary32 emulated with struct, binary64 for the float
    steps, GELU from a numerically integrated normal CDF).
"""
import itertools
import math
import struct

import numpy as np
import pytest

import oracle
import synth


def f32(x: float) -> float:
    return struct.unpack("f", struct.pack("f", x))[0]


def test_structure_from_the_printed_parameter_count():
    # Audio8 article: audio_encoder.whisper.* = 636,968,960 parameters
    assert oracle.encoder_param_count(128, 1280, 32, 5120, 1500) == 636_968_960
    hits = []
    for layers, ffn, kbias, table, convbias in itertools.product(
            range(24, 41), (4096, 5120, 6144), (False, True), (False, True), (False, True)):
        n = oracle.encoder_param_count(128, 1280, layers, ffn, 1500 if table else 0)
        n += layers * 1280 if kbias else 0
        n -= 0 if convbias else 2 * 1280
        if n == 636_968_960:
            hits.append((layers, ffn, kbias, table, convbias))
    assert hits == [(32, 5120, False, True, True)]


def test_workload_settings_match_the_oracle_readings():
    for cfg in (synth.CONFIGS["c1"], synth.TINY, synth.SMALL):
        assert cfg.enc_ln_eps == oracle.ENC_LN_EPS and cfg.enc_rope_theta == oracle.ENC_ROPE_THETA


def test_frame_counts():
    # 3 s and 30 s clips: samples // 160 mel frames, stride-2 second conv
    for samples, frames in ((48000, 150), (480000, 1500)):
        mel = samples // 160
        assert oracle.conv_out_len(oracle.conv_out_len(mel, 1), 2) == frames
        assert frames == oracle.n_encoder_frames(samples)
    assert oracle.conv_out_len(3000, 2) == synth.CONFIGS["c4"].enc_max_pos
    for name in ("c1", "c2", "c4"):
        cfg = synth.CONFIGS[name]
        assert oracle.conv_out_len(cfg.mel_frames, 2) == cfg.enc_frames
    for cfg in (synth.TINY, synth.SMALL):
        assert oracle.conv_out_len(cfg.mel_frames, 2) == cfg.enc_frames
        assert cfg.frame_dim == cfg.enc_dim


@pytest.mark.parametrize("T,C,stride", [(7, 3, 1), (7, 3, 2), (8, 2, 2), (1, 4, 1), (2, 1, 2)])
def test_im2col_is_a_convolution(T, C, stride):
    rng = np.random.default_rng(T * 10 + C + stride)
    x = rng.standard_normal((T, C)).astype(np.float32)
    O = 5
    w = rng.standard_normal((O, 3, C))
    rows = oracle.im2col(x, stride)
    assert rows.shape == (oracle.conv_out_len(T, stride), 3 * C)
    got = rows.astype(np.float64) @ w.reshape(O, 3 * C).T
    for t in range(rows.shape[0]):
        for o in range(O):
            acc = 0.0
            for j in range(3):
                src = t * stride - 1 + j
                if 0 <= src < T:
                    for c in range(C):
                        acc += w[o, j, c] * float(x[src, c])
            assert abs(acc - got[t, o]) <= 1e-12 * (1 + abs(acc))


def test_layernorm():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((6, 40)) * 3 + 1.5).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(40)).astype(np.float32)
    b = (0.1 * rng.standard_normal(40)).astype(np.float32)
    y = oracle.layernorm(x, g, b, 1e-5)
    for r in range(6):
        xs = [float(v) for v in x[r]]
        mu = math.fsum(xs) / 40
        var = math.fsum((v - mu) ** 2 for v in xs) / 40
        for i in range(40):
            want = f32((xs[i] - mu) / math.sqrt(var + 1e-5) * float(g[i]) + float(b[i]))
            assert abs(float(y[r, i]) - want) <= 2 * abs(want) * 2.0 ** -24 + 1e-30
    unit = oracle.layernorm(x, np.ones(40, np.float32), np.zeros(40, np.float32), 0.0).astype(np.float64)
    assert np.allclose(unit.mean(axis=1), 0, atol=1e-6) and np.allclose(unit.var(axis=1), 1, atol=1e-5)
    # invariant to a shift and a positive scale of the input (eps 0)
    y2 = oracle.layernorm(x * 4 + 7, g, b, 0.0)
    assert np.allclose(y2, oracle.layernorm(x, g, b, 0.0), atol=2e-6)


def bf_softmax_attn(q, k, v):
    F_, H, D = q.shape
    out = np.zeros((F_, H * D))
    for h in range(H):
        for i in range(F_):
            sc = [sum(float(q[i, h, d]) * float(k[j, h, d]) for d in range(D)) / math.sqrt(D)
                  for j in range(F_)]
            m = max(sc)
            e = [math.exp(s - m) for s in sc]
            tot = math.fsum(e)
            for d in range(D):
                out[i, h * D + d] = math.fsum(e[j] * float(v[j, h, d]) for j in range(F_)) / tot
    return out


def test_enc_attention():
    rng = np.random.default_rng(4)
    F_, H, D = 6, 2, 4
    q, k, v = (rng.standard_normal((F_, H, D)).astype(np.float32) for _ in range(3))
    got = oracle.enc_attention(q, k, v)
    assert np.allclose(got, bf_softmax_attn(q, k, v), rtol=1e-6, atol=1e-7)
    # zero queries: the plain mean of the values; one frame: the value itself
    z = oracle.enc_attention(np.zeros_like(q), k, v).reshape(F_, H, D)
    assert np.allclose(z, np.broadcast_to(v.astype(np.float64).mean(axis=0), z.shape), atol=1e-7)
    one = oracle.enc_attention(q[:1], k[:1], v[:1])
    assert np.array_equal(one, v[:1].reshape(1, -1))
    # no mask: permuting the frames permutes the rows
    p = rng.permutation(F_)
    assert np.allclose(oracle.enc_attention(q[p], k[p], v[p]), got[p], atol=1e-7)


# ------------------------------------------------------------ brute force --
def _simpson(f, a, b, n):
    h = (b - a) / n
    s = f(a) + f(b)
    for i in range(1, n):
        s += (4.0 if i % 2 else 2.0) * f(a + i * h)
    return s * h / 3.0


def phi(x):
    f = lambda t: math.exp(-0.5 * t * t) / math.sqrt(2.0 * math.pi)  # noqa: E731
    if x >= 0.0:
        return 0.5 + (_simpson(f, 0.0, x, 400) if x > 0.0 else 0.0)
    return _simpson(f, x - 12.0, x, 1200)


def bf_prep(rows):
    codes, scales = [], []
    for r in rows:
        s = f32(max(abs(v) for v in r) / 127.0)
        scales.append(s)
        codes.append([0] * len(r) if s == 0.0 else [max(-127, min(127, round(f32(v / s)))) for v in r])
    return codes, scales


def bf_quant(rows):
    flat = [v for r in rows for v in r]
    lo, hi = min(0.0, min(flat)), max(0.0, max(flat))
    s = f32(f32(hi - lo) / 255.0)
    if s == 0.0:
        return [[0] * len(r) for r in rows], 0.0, 0
    z = max(0, min(255, round(f32(-lo / s))))
    return [[max(0, min(255, round(f32(v / s)) + z)) for v in r] for r in rows], s, z


def bf_linear(rows, W, bias=None):
    codes, s, z = bf_quant(rows)
    wc, ws = W
    out = []
    for r in codes:
        y = []
        for n in range(len(wc)):
            acc = sum((c - z) * w for c, w in zip(r, wc[n]))
            v = f32(f32(float(acc)) * f32(s * ws[n]))
            y.append(f32(v + bias[n]) if bias is not None else v)
        out.append(y)
    return out


def bf_im2col(x, stride):
    T = len(x)
    C = len(x[0])
    To = (T - 1) // stride + 1
    return [[(x[t * stride - 1 + j][c] if 0 <= t * stride - 1 + j < T else 0.0)
             for j in range(3) for c in range(C)] for t in range(To)]


def bf_ln(x, g, b, eps):
    out = []
    for r in x:
        mu = math.fsum(r) / len(r)
        var = math.fsum((v - mu) ** 2 for v in r) / len(r)
        rs = 1.0 / math.sqrt(var + eps)
        out.append([f32((v - mu) * rs * gi + bi) for v, gi, bi in zip(r, g, b)])
    return out


def bf_rope(vec, pos, theta):
    D = len(vec)
    h = D // 2
    out = [0.0] * D
    for j in range(h):
        ang = pos * theta ** (-(2.0 * j) / D)
        c, s = math.cos(ang), math.sin(ang)
        out[j] = f32(vec[j] * c - vec[j + h] * s)
        out[j + h] = f32(vec[j + h] * c + vec[j] * s)
    return out


def bf_encoder(cfg, mel):
    fr = synth.encoder_front(cfg)
    H, D = cfg.enc_heads, cfg.enc_dim
    Dh = D // H
    gelu = lambda v: f32(v * phi(v))  # noqa: E731
    a = [[gelu(v) for v in r] for r in bf_linear(bf_im2col(mel, 1), bf_prep(fr["conv1"].tolist()),
                                                  fr["conv1_b"].tolist())]
    x = [[gelu(v) for v in r] for r in bf_linear(bf_im2col(a, 2), bf_prep(fr["conv2"].tolist()),
                                                  fr["conv2_b"].tolist())]
    F_ = len(x)
    x = [[f32(v + float(fr["pos"][t][i])) for i, v in enumerate(r)] for t, r in enumerate(x)]
    for l in range(cfg.enc_layers):
        w = synth.encoder_layer_weights(cfg, l)
        P = {n: bf_prep(w[n].tolist()) for n in ("wq", "wk", "wv", "wo", "w1", "w2")}
        h = bf_ln(x, w["ln1_g"].tolist(), w["ln1_b"].tolist(), oracle.ENC_LN_EPS)
        q = bf_linear(h, P["wq"], w["bq"].tolist())
        k = bf_linear(h, P["wk"])
        v = bf_linear(h, P["wv"], w["bv"].tolist())
        att = []
        for i in range(F_):
            row = []
            for hd in range(H):
                qi = bf_rope(q[i][hd * Dh:(hd + 1) * Dh], i, oracle.ENC_ROPE_THETA)
                sc = []
                for j in range(F_):
                    kj = bf_rope(k[j][hd * Dh:(hd + 1) * Dh], j, oracle.ENC_ROPE_THETA)
                    sc.append(sum(a_ * b_ for a_, b_ in zip(qi, kj)) / math.sqrt(Dh))
                m = max(sc)
                e = [math.exp(s - m) for s in sc]
                tot = math.fsum(e)
                for d in range(Dh):
                    row.append(f32(math.fsum(e[j] * v[j][hd * Dh + d] for j in range(F_)) / tot))
            att.append(row)
        o = bf_linear(att, P["wo"], w["bo"].tolist())
        x = [[f32(a_ + b_) for a_, b_ in zip(r, ro)] for r, ro in zip(x, o)]
        h2 = bf_ln(x, w["ln2_g"].tolist(), w["ln2_b"].tolist(), oracle.ENC_LN_EPS)
        f = [[gelu(v) for v in r] for r in bf_linear(h2, P["w1"], w["b1"].tolist())]
        o2 = bf_linear(f, P["w2"], w["b2"].tolist())
        x = [[f32(a_ + b_) for a_, b_ in zip(r, ro)] for r, ro in zip(x, o2)]
    return bf_ln(x, fr["lnf_g"].tolist(), fr["lnf_b"].tolist(), oracle.ENC_LN_EPS)


def test_encoder_matches_brute_force():
    cfg = synth.TINY.with_(batch=2)
    enc = oracle.build_encoder(cfg, synth)
    mel = synth.mel_features(cfg)
    mel[1] *= 2.0
    got = oracle.encoder_forward(enc, mel)
    assert got.shape == (2, cfg.enc_frames, cfg.enc_dim)
    for b in range(2):
        want = np.array(bf_encoder(cfg, mel[b].tolist()), np.float32)
        err = float(np.max(np.abs(got[b].astype(np.float64) - want)) / np.max(np.abs(want)))
        assert err <= 1e-5, (b, err)


def test_encoder_per_clip_quantisation():
    cfg = synth.TINY.with_(batch=3)
    enc = oracle.build_encoder(cfg, synth)
    mel = synth.mel_features(cfg)
    mel[2] *= 5.0
    both = oracle.encoder_forward(enc, mel)
    for b in range(3):
        assert np.array_equal(both[b], oracle.encoder_forward(enc, mel[b:b + 1])[0])


def _gelu_tanh(x):
    x64 = np.asarray(x, np.float32).astype(np.float64)
    return (0.5 * x64 * (1 + np.tanh(math.sqrt(2 / math.pi) * (x64 + 0.044715 * x64 ** 3)))).astype(np.float32)


def _rmsnorm_as_ln(x, g, b, eps=oracle.ENC_LN_EPS):
    x64 = np.asarray(x, np.float32).astype(np.float64)
    r = 1.0 / np.sqrt(np.mean(x64 * x64, axis=-1, keepdims=True) + eps)
    return (x64 * r * g.astype(np.float64) + b.astype(np.float64)).astype(np.float32)


def _interleaved_rope(x, pos, cos, sin):
    # pairs (2j, 2j + 1) instead of (j, j + D/2)
    D = x.shape[-1]
    perm = np.concatenate([np.arange(0, D, 2), np.arange(1, D, 2)])
    inv = np.argsort(perm)
    return _ORIG["apply_rope"](x[..., perm], pos, cos, sin)[..., inv]


def _per_row_dynquant(x):
    x = np.asarray(x, np.float32)
    rows = [_ORIG["dynquant"](x[i:i + 1]) for i in range(x.shape[0])]
    return (np.concatenate([r[0] for r in rows]), np.array([r[1] for r in rows], np.float32)[:, None],
            np.array([r[2] for r in rows], np.int32)[:, None])


_ORIG = {}


def _plants():
    """Plausible slips in the oracle's encoder, each planted on the CPU by
    replacing one function of oracle.ark (the encoder looks them up there)."""
    import oracle.ark as oa

    calls = {"n": 0}

    def rope_q_only(x, pos, cos, sin):
        calls["n"] += 1
        return _ORIG["apply_rope"](x, pos, cos, sin) if calls["n"] % 2 else x

    def attn_scale_1_over_d(q, k, v):
        return _ORIG["enc_attention"](q / np.float32(np.sqrt(q.shape[-1])), k, v)

    return {
        "k not rotated": ("apply_rope", rope_q_only),
        "rotary pairs interleaved": ("apply_rope", _interleaved_rope),
        "scores scaled by 1/D": ("enc_attention", attn_scale_1_over_d),
        "tanh GELU": ("gelu", _gelu_tanh),
        "RMSNorm in place of LayerNorm": ("layernorm", _rmsnorm_as_ln),
        "one (s, z) per frame": ("dynquant", _per_row_dynquant),
    }, oa


def test_brute_force_catches_planted_slips():
    """Every slip above moves the oracle's encoder output past the 1e-5 bar
    of the brute-force comparison, and the positional rows matter too.  The
    features are scaled up so that the first GELU sees inputs of order one
    (with the seeded 0.02 weights its inputs are otherwise near zero, where
    the erf and tanh forms agree to 1e-7)."""
    cfg = synth.TINY.with_(batch=1)
    mel = synth.mel_features(cfg) * np.float32(30.0)
    want = np.array(bf_encoder(cfg, mel[0].tolist()), np.float32)

    def err(enc):
        got = oracle.encoder_forward(enc, mel)[0]
        return float(np.max(np.abs(got.astype(np.float64) - want)) / np.max(np.abs(want)))

    enc = oracle.build_encoder(cfg, synth)
    assert err(enc) <= 1e-5
    plants, oa = _plants()
    for name, (fn, repl) in plants.items():
        _ORIG[fn] = getattr(oa, fn)
        setattr(oa, fn, repl)
        try:
            e = err(enc)
        finally:
            setattr(oa, fn, _ORIG[fn])
        assert e > 1e-4, (name, e)
    nopos = oracle.build_encoder(cfg, synth)
    nopos.pos = np.zeros_like(nopos.pos)
    assert err(nopos) > 1e-4
