"""Pins of the oracle's bf16 serving variant (cookbook "ARK-ASR-3B",
"dtype": bfloat16 is the default serving dtype).

  * bf16_round against torch's own float32 -> bfloat16 conversion (a library
    routine, round to nearest even) and against the exact nearest point of
    the bf16 grid computed with rationals;
  * the variant's wiring: with the rounding replaced by the identity it is
    the oracle's float model (whose wiring the int8 brute force pins);
  * the rounding points: one layer written out again in pure Python with
    bf16 rounding at each operation's output;
  * its outputs are bf16 values and stay within bf16 noise of the float
    model.
"""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(1e3),
        (rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32)).view(np.float32),
        np.array([0.0, -0.0, 1.0, np.inf, -np.inf, 3.4028235e38, -3.4028235e38, 1e-45, 1.17549435e-38],
                 np.float32)])
    # exact ties: the 16 dropped bits are 0x8000
    ties = (rng.integers(0, 2 ** 15, 2000, dtype=np.uint32) << np.uint32(17)) | np.uint32(0x8000)
    x = np.concatenate([x, ties.view(np.float32), (ties | np.uint32(0x10000)).view(np.float32)])
    got = oracle.bf16_round(x)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    nan = np.isnan(x)
    assert np.all(np.isnan(got[nan]))
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def test_bf16_round_is_nearest_even_on_the_grid():
    rng = np.random.default_rng(2)
    for v in rng.standard_normal(300).astype(np.float32) * np.float32(7.3):
        v = float(v)
        r = float(oracle.bf16_round(np.array([v], np.float32))[0])
        if v == 0.0:
            assert r == 0.0
            continue
        e = math.frexp(abs(v))[1]               # |v| in [2^(e-1), 2^e)
        ulp = Fraction(2) ** (e - 8)             # 8 significant bits
        q = Fraction(abs(v)) / ulp
        lo = math.floor(q)
        frac = q - lo
        n = lo + (1 if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and lo % 2 == 1) else 0)
        assert Fraction(abs(r)) == n * ulp and math.copysign(1.0, r) == math.copysign(1.0, v)


def _zeros(cfg, B=1):
    return [np.zeros((B, cfg.max_total_len, cfg.n_kv_heads, cfg.head_dim), np.float32)] * cfg.n_layers


def test_wiring_equals_the_float_model_without_rounding():
    cfg = synth.TINY
    ident = lambda a: np.asarray(a, np.float32)  # noqa: E731
    mb = oracle.build_bf16_model(cfg, synth, rounding=ident)
    mf = oracle.build_model(cfg, synth, linear="float")
    x = synth.prefill_embeds(cfg.with_(prefill_from_embeds=True))
    lb, kdb, vdb, hb = oracle.bf16_prefill(mb, x, [0], _zeros(cfg), _zeros(cfg))
    lf, kdf, vdf, hf = oracle.prefill(mf, x, np.array([0]), _zeros(cfg), _zeros(cfg))
    assert np.allclose(hb, hf, rtol=0, atol=1e-5 * np.max(np.abs(hf)))
    for l in range(cfg.n_layers):
        assert np.allclose(kdb[l], kdf[l], atol=1e-5 * np.max(np.abs(kdf[l])))
        assert np.allclose(vdb[l], vdf[l], atol=1e-5 * np.max(np.abs(vdf[l])))
    # the float model's head is int8; compare with its fp32 weights instead
    hn = oracle.rmsnorm(hf[:, -1], mf.final_norm, cfg.rms_eps)
    lf32 = (hn.astype(np.float64) @ synth.lm_head(cfg).astype(np.float64).T)
    assert np.allclose(lb, lf32, atol=1e-5 * np.max(np.abs(lf32)))


def bf(v: float) -> float:
    """bf16 of a Python float: through binary32, then nearest even of the
    top 16 bits (NaN and overflow not needed here)."""
    b = struct.unpack("I", struct.pack("f", v))[0]
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return struct.unpack("f", struct.pack("I", b))[0]


def bf_layer(cfg, lay, x, cos, sin):
    """One bf16 layer, prefill of the rows x (lists) at positions 0..S-1
    from an empty cache, in plain Python."""
    S, H = len(x), cfg.hidden
    NH, NKV, D = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim

    def norm(rows, g):
        out = []
        for r in rows:
            rs = 1.0 / math.sqrt(math.fsum(v * v for v in r) / H + cfg.rms_eps)
            out.append([bf(float(gi) * bf(v * rs)) for v, gi in zip(r, g)])
        return out

    def lin(rows, w, b=None):
        return [[bf(math.fsum(a * float(c) for a, c in zip(r, wr)) + (float(b[n]) if b is not None else 0.0))
                 for n, wr in enumerate(w)] for r in rows]

    def rope(vec, pos):
        h = D // 2
        o = [0.0] * D
        for j in range(h):
            c, s = cos[pos][j], sin[pos][j]
            o[j] = bf(vec[j] * c - vec[j + h] * s)
            o[j + h] = bf(vec[j + h] * c + vec[j] * s)
        return o

    tr = {}
    h1 = tr["h1"] = norm(x, lay.ln1)
    q = lin(h1, lay.w["wq"], lay.bq)
    k = lin(h1, lay.w["wk"], lay.bk)
    v = lin(h1, lay.w["wv"], lay.bv)
    G = NH // NKV
    tr["q"] = [sum((rope(q[i][hd * D:(hd + 1) * D], i) for hd in range(NH)), []) for i in range(S)]
    tr["v"] = v
    att = []
    for i in range(S):
        row = []
        for hd in range(NH):
            g = hd // G
            qi = rope(q[i][hd * D:(hd + 1) * D], i)
            ks = [rope(k[j][g * D:(g + 1) * D], j) for j in range(i + 1)]
            sc = [math.fsum(a * b for a, b in zip(qi, kj)) / math.sqrt(D) for kj in ks]
            mx = max(sc)
            e = [math.exp(s - mx) for s in sc]
            tot = math.fsum(e)
            for d in range(D):
                row.append(bf(math.fsum(e[j] * v[j][g * D + d] for j in range(i + 1)) / tot))
        att.append(row)
    tr["attn"] = att
    o = lin(att, lay.w["wo"])
    x1 = tr["x1"] = [[bf(a + b) for a, b in zip(r, ro)] for r, ro in zip(x, o)]
    h2 = tr["h2"] = norm(x1, lay.ln2)
    gg = lin(h2, lay.w["wg"])
    uu = lin(h2, lay.w["wu"])
    a = tr["a"] = [[bf(bf(gv / (1.0 + math.exp(-gv))) * uv) for gv, uv in zip(gr, ur)]
                   for gr, ur in zip(gg, uu)]
    d = lin(a, lay.w["wd"])
    tr["x2"] = [[bf(p + q_) for p, q_ in zip(r, rd)] for r, rd in zip(x1, d)]
    return tr


def _layer_case():
    cfg = synth.TINY.with_(n_layers=1)
    m = oracle.build_bf16_model(cfg, synth)
    x = oracle.bf16_round(synth.prefill_embeds(cfg.with_(prefill_from_embeds=True, prefill_len=4)))
    bft = bf_layer(cfg, m.layers[0], x[0].astype(np.float64).tolist(), m.cos, m.sin)
    return cfg, m, x, bft


def _layer_mismatches(cfg, m, x, bft):
    """Names of the intermediates where the oracle's layer leaves the brute
    force: both sides round at the same points; the fp64 sums differ in
    order, which moves a bf16 result by one step only at a rounding
    boundary (at most 1% of the values, each by at most one step)."""
    tr = {}
    oracle.bf16_layer_forward(m, 0, x, np.array([0]), _zeros(cfg)[0], _zeros(cfg)[0], tr)
    bad = []
    for name in ("h1", "q", "v", "attn", "x1", "h2", "a", "x2"):
        got = tr[name][0].reshape(len(bft[name]), -1).astype(np.float64)
        want = np.array(bft[name], np.float64)
        diff = np.abs(got - want)
        if not (np.all(diff <= np.abs(want) * 2.0 ** -7 + 1e-30)
                and np.count_nonzero(diff) <= max(1, want.size // 100)):
            bad.append(name)
    return bad


def test_one_layer_matches_brute_force():
    assert _layer_mismatches(*_layer_case()) == []


def test_brute_force_catches_planted_slips():
    """Slips planted in the oracle on the CPU (one function of oracle.ark
    replaced at a time; the layer looks them up there) that the pure-Python
    layer must catch."""
    import oracle.ark as oa
    F64 = np.float64
    orig = {n: getattr(oa, n) for n in ("bf16_rmsnorm", "bf16_linear", "apply_rope")}

    def norm_one_rounding(m, x, g):
        x64 = np.asarray(x, np.float32).astype(F64)
        r = 1.0 / np.sqrt(np.mean(x64 * x64, axis=-1, keepdims=True) + m.cfg.rms_eps)
        return m.round((x64 * r * np.asarray(g, np.float32).astype(F64)).astype(np.float32))

    def linear_unrounded(m, x, w, bias=None):
        y = np.asarray(x, np.float32).astype(F64) @ np.asarray(w, np.float32).astype(F64).T
        return (y + (0 if bias is None else np.asarray(bias, np.float32).astype(F64))).astype(np.float32)

    def linear_bias_after_rounding(m, x, w, bias=None):
        y = orig["bf16_linear"](m, x, w)
        return y if bias is None else m.round((y.astype(F64) + bias.astype(F64)).astype(np.float32))

    def rope_interleaved(x, pos, cos, sin):
        D = x.shape[-1]
        perm = np.concatenate([np.arange(0, D, 2), np.arange(1, D, 2)])
        return orig["apply_rope"](x[..., perm], pos, cos, sin)[..., np.argsort(perm)]

    case = _layer_case()
    plants = {
        "norm rounded once": ("bf16_rmsnorm", norm_one_rounding, "h1"),
        "linear not rounded": ("bf16_linear", linear_unrounded, "q"),
        "bias added after rounding": ("bf16_linear", linear_bias_after_rounding, "q"),
        "rotary pairs interleaved": ("apply_rope", rope_interleaved, "q"),
    }
    for name, (fn, repl, first) in plants.items():
        setattr(oa, fn, repl)
        try:
            bad = _layer_mismatches(*case)
        finally:
            setattr(oa, fn, orig[fn])
        assert first in bad, (name, bad)


def test_outputs_are_bf16_and_near_the_float_model():
    cfg = synth.TINY
    mb = oracle.build_bf16_model(cfg, synth)
    mf = oracle.build_model(cfg, synth, linear="float")
    x = synth.prefill_embeds(cfg.with_(prefill_from_embeds=True))
    lb, kdb, vdb, hb = oracle.bf16_prefill(mb, x, [0], _zeros(cfg), _zeros(cfg))
    _, _, _, hf = oracle.prefill(mf, x, np.array([0]), _zeros(cfg), _zeros(cfg))
    assert np.array_equal(oracle.bf16_round(hb), hb)
    for a in kdb + vdb:
        assert np.array_equal(oracle.bf16_round(a), a)
    assert float(np.max(np.abs(hb - hf)) / np.max(np.abs(hf))) < 5e-2
