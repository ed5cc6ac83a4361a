"""The bf16 serving variant on the GPU against the oracle (cookbook
"ARK-ASR-3B", "dtype": bfloat16 is the default serving dtype).

  * fp32 -> bf16 conversion bit for bit with oracle.bf16_round (ties,
    subnormals, infinities, NaN);
  * the bf16 cache write bit for bit;
  * prefill and decode steps of the bf16 decoder against
    oracle.bf16_prefill / bf16_decode_step: every step rounds at the same
    points on both sides, the GPU sums in fp32 and the oracle in fp64, so a
    bf16 result may move by one rounding step and the difference propagates
    through the layers; the bar is the serving dtype's 2e-2 relative
    (per tensor, max |gpu - oracle| / max |oracle|) on logits, deltas and
    the hidden rows, every delta and hidden value a bf16 value, and the
    greedy id equal unless the oracle's top two are within twice the
    logit error.  Cases cover the row kernel (1..8 rows), both matrix-core
    tile heights, prefill at several positions, and the real LM head shape.
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
from speech_decoder_int8_amd import ark  # noqa: E402

from gpu_util import check_tokens, host, t  # noqa: E402

pytestmark = pytest.mark.gpu
F32 = np.float32
TOL = 2e-2


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


def f32(x):
    return host(x.float())


def test_to_bf16_bit_exact():
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(100000).astype(F32) * F32(50),
        rng.integers(0, 2 ** 32, 100000, dtype=np.uint64).astype(np.uint32).view(F32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.4028235e38, 1e-45, -1e-40], F32)])
    ties = (rng.integers(0, 2 ** 15, 5000, dtype=np.uint32) << np.uint32(17)) | np.uint32(0x8000)
    x = np.concatenate([x, ties.view(F32), (ties | np.uint32(0x10000)).view(F32)])
    got = f32(ark.to_bf16(t(x)))
    want = oracle.bf16_round(x)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


class State:
    def __init__(self, gm, B, S_max):
        cfg = gm.cfg
        shape = (B, cfg.max_total_len, cfg.n_kv_heads, cfg.head_dim)
        self.kc = [torch.zeros(shape, dtype=torch.bfloat16, device="cuda") for _ in range(cfg.n_layers)]
        self.vc = [torch.zeros(shape, dtype=torch.bfloat16, device="cuda") for _ in range(cfg.n_layers)]
        self.kd = torch.empty((cfg.n_layers, B, S_max, cfg.n_kv_heads, cfg.head_dim),
                              dtype=torch.bfloat16, device="cuda")
        self.vd = torch.empty_like(self.kd)
        self.logits = torch.empty((B, cfg.vocab), device="cuda")
        self.ws = gm.workspace(B, S_max)
        self.B = B

    def deltas(self, S):
        n = self.kd[:, :, :S].numel()
        shp = (self.kd.shape[0], self.B, S, *self.kd.shape[3:])
        return self.kd.view(-1)[:n].view(shp), self.vd.view(-1)[:n].view(shp)

    def load(self, kc, vc):
        for l in range(len(self.kc)):
            self.kc[l].copy_(t(kc[l]).to(torch.bfloat16))
            self.vc[l].copy_(t(vc[l]).to(torch.bfloat16))


def _caches(cfg, B, lengths, rng):
    """bf16-valued caches with N(0,1) rows below each length and garbage above."""
    shape = (B, cfg.max_total_len, cfg.n_kv_heads, cfg.head_dim)
    kc, vc = [], []
    for _ in range(cfg.n_layers):
        k = np.zeros(shape, F32)
        v = np.zeros(shape, F32)
        for b in range(B):
            n = int(lengths[b])
            k[b, :n] = rng.standard_normal((n, cfg.n_kv_heads, cfg.head_dim))
            v[b, :n] = rng.standard_normal((n, cfg.n_kv_heads, cfg.head_dim))
            k[b, n:] = 3.0e4
            v[b, n:] = -7.0
        kc.append(oracle.bf16_round(k))
        vc.append(oracle.bf16_round(v))
    return kc, vc


def _check(what, lg, lo, kd, kdo, vd, vdo, hid, hido, mask):
    for name, g, o in (("hidden", hid, hido),) + tuple(
            (f"k delta {l}", kd[l], kdo[l]) for l in range(len(kdo))) + tuple(
            (f"v delta {l}", vd[l], vdo[l]) for l in range(len(vdo))):
        g = np.asarray(g, F32).reshape(np.asarray(o).shape)
        assert np.array_equal(oracle.bf16_round(g), g), f"{what} {name}: not bf16 values"
        r = rel(g, o)
        assert r <= TOL, f"{what} {name}: relative error {r:.3g}"
    if lo is not None:
        err = rel(lg, lo)
        assert err <= TOL, f"{what} logits: relative error {err:.3g}"
        tok = oracle.masked_argmax(lg, mask)
        check_tokens(tok, oracle.masked_argmax(lo, mask), lo, mask, err * np.max(np.abs(lo)), what)


CFG = synth.CONFIGS["c1"].with_(name="real2", n_layers=2, vocab=4096, seed=78)


@pytest.fixture(scope="module")
def small():
    return oracle.build_bf16_model(CFG, synth), ark.load_model_bf16(CFG, synth)


@pytest.mark.parametrize("B,S,p", [(1, 21, [0]), (3, 70, [5, 0, 100]), (2, 130, [0, 200]),
                                   (1, 387, [0])])
def test_prefill_bf16(small, B, S, p):
    om, gm = small
    rng = np.random.default_rng(500 + B * S)
    kc, vc = _caches(CFG, B, p, rng)
    st = State(gm, B, S)
    st.load(kc, vc)
    x = oracle.bf16_round(rng.standard_normal((B, S, CFG.hidden)).astype(F32))
    kd, vd = st.deltas(S)
    hid = torch.empty((B, S, CFG.hidden), dtype=torch.bfloat16, device="cuda")
    ark.prefill_bf16(gm, t(x).to(torch.bfloat16), p, st.kc, st.vc, kd, vd, st.logits, hid, st.ws)
    lo, kdo, vdo, ho = oracle.bf16_prefill(om, x, np.array(p), kc, vc)
    _check(f"prefill {B}x{S}", f32(st.logits), lo, f32(kd), kdo, f32(vd), vdo, f32(hid), ho, CFG.mask())


@pytest.mark.parametrize("B", [1, 3, 6, 8, 12, 40])
def test_decode_bf16(small, B):
    om, gm = small
    rng = np.random.default_rng(600 + B)
    lengths = rng.integers(0, CFG.max_total_len - 1, size=B)
    lengths[0] = 130
    kc, vc = _caches(CFG, B, lengths, rng)
    st = State(gm, B, 1)
    st.load(kc, vc)
    ids = rng.integers(0, CFG.vocab - 64, size=B).astype(np.int32)
    kd, vd = st.deltas(1)
    hid = torch.empty((B, 1, CFG.hidden), dtype=torch.bfloat16, device="cuda")
    ark.decode_step_bf16(gm, t(ids), lengths, st.kc, st.vc, kd, vd, st.logits, hid, st.ws)
    lo, kdo, vdo, ho = oracle.bf16_decode_step(om, ids, lengths, kc, vc)
    _check(f"decode B={B}", f32(st.logits), lo, f32(kd), kdo, f32(vd), vdo, f32(hid), ho, CFG.mask())


def test_cache_write_bf16(small):
    om, gm = small
    rng = np.random.default_rng(9)
    B, S = 3, 5
    st = State(gm, B, S)
    kd, vd = st.deltas(S)
    kd.copy_(t(rng.standard_normal(kd.shape).astype(F32)).to(torch.bfloat16))
    vd.copy_(t(rng.standard_normal(vd.shape).astype(F32)).to(torch.bfloat16))
    pos = [0, 17, CFG.max_total_len - S]
    ark.cache_write_bf16(gm.dims, pos, st.kc, st.vc, kd, vd)
    kdh, vdh = host(kd.view(torch.int16)), host(vd.view(torch.int16))
    for l in range(CFG.n_layers):
        kcl, vcl = host(st.kc[l].view(torch.int16)), host(st.vc[l].view(torch.int16))
        want_k = np.zeros_like(kcl)
        want_v = np.zeros_like(vcl)
        for b in range(B):
            want_k[b, pos[b]:pos[b] + S] = kdh[l, b]
            want_v[b, pos[b]:pos[b] + S] = vdh[l, b]
        assert np.array_equal(kcl, want_k) and np.array_equal(vcl, want_v)


def test_greedy_steps_bf16(small):
    """A prompt prefill, then greedy steps through the cache write, against
    the oracle run the same way."""
    om, gm = small
    rng = np.random.default_rng(11)
    S = 20
    st = State(gm, 1, S)
    zero = [np.zeros((1, CFG.max_total_len, CFG.n_kv_heads, CFG.head_dim), F32)] * CFG.n_layers
    x = oracle.bf16_round(rng.standard_normal((1, S, CFG.hidden)).astype(F32))
    kd, vd = st.deltas(S)
    ark.prefill_bf16(gm, t(x).to(torch.bfloat16), [0], st.kc, st.vc, kd, vd, st.logits, None, st.ws)
    ark.cache_write_bf16(gm.dims, [0], st.kc, st.vc, kd, vd)
    lo, kdo, vdo, _ = oracle.bf16_prefill(om, x, np.array([0]), zero, zero)
    kco = [oracle.cache_write(zero[l], kdo[l], [0]) for l in range(CFG.n_layers)]
    vco = [oracle.cache_write(zero[l], vdo[l], [0]) for l in range(CFG.n_layers)]
    mask = CFG.mask()
    lg = f32(st.logits)
    tok = oracle.masked_argmax(lg, mask)
    p = S
    for step in range(3):
        to = oracle.masked_argmax(lo, mask)
        if int(tok[0]) != int(to[0]):
            check_tokens(tok, to, lo, mask, rel(lg, lo) * np.max(np.abs(lo)), f"step {step}")
            break
        kd1, vd1 = st.deltas(1)
        ark.decode_step_bf16(gm, t(tok.astype(np.int32)), [p], st.kc, st.vc, kd1, vd1, st.logits, None,
                             st.ws)
        ark.cache_write_bf16(gm.dims, [p], st.kc, st.vc, kd1, vd1)
        lo, kdo, vdo, _ = oracle.bf16_decode_step(om, to, np.array([p]), kco, vco)
        kco = [oracle.cache_write(kco[l], kdo[l], [p]) for l in range(CFG.n_layers)]
        vco = [oracle.cache_write(vco[l], vdo[l], [p]) for l in range(CFG.n_layers)]
        lg = f32(st.logits)
        assert rel(lg, lo) <= TOL, f"step {step}: {rel(lg, lo):.3g}"
        tok = oracle.masked_argmax(lg, mask)
        p += 1


def test_real_lm_head_shape():
    """The real vocabulary (151936 rows of the head) with two layers: the 3 s
    clip's prompt length, then one decode step."""
    cfg = synth.CONFIGS["c1"].with_(name="real2v", n_layers=2)
    om, gm = oracle.build_bf16_model(cfg, synth), ark.load_model_bf16(cfg, synth)
    rng = np.random.default_rng(12)
    S = cfg.prefill_len
    st = State(gm, 1, S)
    zero = [np.zeros((1, cfg.max_total_len, cfg.n_kv_heads, cfg.head_dim), F32)] * cfg.n_layers
    x = oracle.bf16_round(rng.standard_normal((1, S, cfg.hidden)).astype(F32))
    kd, vd = st.deltas(S)
    hid = torch.empty((1, S, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    ark.prefill_bf16(gm, t(x).to(torch.bfloat16), [0], st.kc, st.vc, kd, vd, st.logits, hid, st.ws)
    lo, kdo, vdo, ho = oracle.bf16_prefill(om, x, np.array([0]), zero, zero)
    _check("real head prefill", f32(st.logits), lo, f32(kd), kdo, f32(vd), vdo, f32(hid), ho, cfg.mask())
