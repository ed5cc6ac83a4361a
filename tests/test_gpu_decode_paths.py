"""Decode at the real ARK geometry (hidden 2048, 16/2 heads, FFN 11008) on
both decode paths of the library: the persistent single-kernel step
(batch 1) and the multi-kernel path, against the CPU oracle.  Two layers and a
4096-id LM head keep the oracle fast."""
import os

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
from speech_decoder_int8_amd import ark  # noqa: E402

from gpu_util import GpuState, assert_close, check_tokens, host, t  # noqa: E402

pytestmark = pytest.mark.gpu

CFG = synth.CONFIGS["c1"].with_(name="real2", n_layers=2, vocab=4096, seed=77)


@pytest.fixture(scope="module")
def models():
    return oracle.build_model(CFG, synth), ark.load_model(CFG, synth)


@pytest.fixture(params=["mega", "multi"])
def path(request, monkeypatch):
    if request.param == "multi":
        monkeypatch.setenv("ARK_DECODE_PATH", "multi")
    else:
        monkeypatch.delenv("ARK_DECODE_PATH", raising=False)
    return request.param


def _caches(cfg, lengths, rng):
    shape = (1, cfg.max_total_len, cfg.n_kv_heads, cfg.head_dim)
    kc, vc = [], []
    for _ in range(cfg.n_layers):
        k = np.zeros(shape, np.float32)
        v = np.zeros(shape, np.float32)
        n = int(lengths[0])
        k[0, :n] = rng.standard_normal((n, 2, 128))
        v[0, :n] = rng.standard_normal((n, 2, 128))
        k[0, n:] = np.nan                     # unwritten rows: garbage the mask must drop
        v[0, n:] = np.inf
        kc.append(k)
        vc.append(v)
    return kc, vc


# live 64-key chunks 1, 2 (one item folding two), 3 (two items, uneven),
# 5 (three items) and 8 (four items, cache full after the second step)
@pytest.mark.parametrize("p0", [0, 100, 150, 300, 510])
def test_decode_steps_match_oracle(models, path, p0):
    om, gm = models
    rng = np.random.default_rng(p0 + 5)
    kc, vc = _caches(CFG, [p0], rng)
    gs = GpuState(gm, 1, 1)
    gs.load_caches(kc, vc)
    mask = CFG.mask()
    tok = np.array([int(rng.integers(0, CFG.vocab - 64))], np.int32)
    p = np.array([p0])
    for step in range(min(2, CFG.max_total_len - p0)):
        kd, vd, hid = gs.decode(t(tok), p)
        lo, kdo, vdo, hido = oracle.decode_step(om, tok, p, kc, vc)
        for l in range(CFG.n_layers):
            assert_close(host(kd[l]), kdo[l], f"{path} step {step} k_delta {l}")
            assert_close(host(vd[l]), vdo[l], f"{path} step {step} v_delta {l}")
        assert_close(host(hid), hido, f"{path} step {step} hidden")
        lg = host(gs.logits)
        err = assert_close(lg, lo, f"{path} step {step} logits") * np.max(np.abs(lo))
        check_tokens(oracle.masked_argmax(lg, mask), oracle.masked_argmax(lo, mask), lo, mask, err,
                     f"{path} step {step}")
        gs.write_back(p, kd, vd)
        kc = [oracle.cache_write(kc[l], kdo[l], p) for l in range(CFG.n_layers)]
        vc = [oracle.cache_write(vc[l], vdo[l], p) for l in range(CFG.n_layers)]
        tok = oracle.masked_argmax(lo, mask)
        p = p + 1


def test_greedy_loop_matches_oracle(models, path):
    om, gm = models
    rng = np.random.default_rng(9)
    kc, vc = _caches(CFG, [60], rng)
    mask = CFG.mask()
    gs = GpuState(gm, 1, 1)
    gs.load_caches(kc, vc)
    tok = np.array([123], np.int32)
    steps = 6
    want, cur, p = [], tok, np.array([60])
    for _ in range(steps):
        lg, kdo, vdo, _ = oracle.decode_step(om, cur, p, kc, vc)
        kc = [oracle.cache_write(kc[l], kdo[l], p) for l in range(CFG.n_layers)]
        vc = [oracle.cache_write(vc[l], vdo[l], p) for l in range(CFG.n_layers)]
        cur = oracle.masked_argmax(lg, mask)
        want.append(cur)
        p = p + 1
    out = torch.empty((steps, 1), dtype=torch.int32, device="cuda")
    kd1, vd1 = gs.deltas(1)
    n, newpos = ark.greedy_decode(gm, t(tok), [60], gs.kc, gs.vc, kd1, vd1, gs.logits, t(mask),
                                  CFG.end_id, steps, out, ws=gs.ws, check_every=3)
    assert n == steps and newpos.tolist() == [60 + steps]
    assert np.array_equal(host(out), np.stack(want))
    for l in range(CFG.n_layers):
        assert_close(host(gs.kc[l])[0, :60 + steps], kc[l][0, :60 + steps], f"{path} k cache {l}")


CFG_LONG = CFG.with_(name="real2_t1024", max_total_len=1024)


@pytest.fixture(scope="module")
def models_long():
    return oracle.build_model(CFG_LONG, synth), ark.load_model(CFG_LONG, synth)


@pytest.mark.parametrize("p0", [511, 700, 1022])
def test_long_cache_decode_matches_oracle(models_long, path, p0):
    # more than 8 live 64-key chunks per KV head: each attention item of the
    # single-kernel step folds several chunks
    om, gm = models_long
    rng = np.random.default_rng(p0 + 7)
    kc, vc = _caches(CFG_LONG, [p0], rng)
    gs = GpuState(gm, 1, 1)
    gs.load_caches(kc, vc)
    mask = CFG_LONG.mask()
    tok = np.array([int(rng.integers(0, CFG_LONG.vocab - 64))], np.int32)
    p = np.array([p0])
    for step in range(min(2, CFG_LONG.max_total_len - p0)):
        kd, vd, hid = gs.decode(t(tok), p)
        lo, kdo, vdo, hido = oracle.decode_step(om, tok, p, kc, vc)
        for l in range(CFG_LONG.n_layers):
            assert_close(host(kd[l]), kdo[l], f"{path} step {step} k_delta {l}")
            assert_close(host(vd[l]), vdo[l], f"{path} step {step} v_delta {l}")
        assert_close(host(hid), hido, f"{path} step {step} hidden")
        lg = host(gs.logits)
        err = assert_close(lg, lo, f"{path} step {step} logits") * np.max(np.abs(lo))
        check_tokens(oracle.masked_argmax(lg, mask), oracle.masked_argmax(lo, mask), lo, mask, err,
                     f"{path} step {step}")
        gs.write_back(p, kd, vd)
        kc = [oracle.cache_write(kc[l], kdo[l], p) for l in range(CFG_LONG.n_layers)]
        vc = [oracle.cache_write(vc[l], vdo[l], p) for l in range(CFG_LONG.n_layers)]
        tok = oracle.masked_argmax(lo, mask)
        p = p + 1
