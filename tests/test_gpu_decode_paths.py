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


# "mega": the persistent kernel as an ordinary launch (the default);
# "mega_coop": the same kernel launched cooperatively (ARK_DECODE_LAUNCH)
@pytest.fixture(params=["mega", "mega_coop", "multi"])
def path(request, monkeypatch):
    if request.param == "multi":
        monkeypatch.setenv("ARK_DECODE_PATH", "multi")
    else:
        monkeypatch.delenv("ARK_DECODE_PATH", raising=False)
    if request.param == "mega_coop":
        monkeypatch.setenv("ARK_DECODE_LAUNCH", "cooperative")
    else:
        monkeypatch.delenv("ARK_DECODE_LAUNCH", raising=False)
    return "mega" if request.param.startswith("mega") else "multi"


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
    assert ark.decode_path(gm, 1) == (1 if path == "mega" else 0)
    rng = np.random.default_rng(p0 + 5)
    kc, vc = _caches(CFG, [p0], rng)
    gs = GpuState(gm, 1, 1)
    gs.load_caches(kc, vc)
    mask = CFG.mask()
    tok = np.array([int(rng.integers(0, CFG.vocab - 64))], np.int32)
    p = np.array([p0])
    for step in range(min(2, CFG.max_total_len - p0)):
        kd, vd, hid = gs.decode(t(tok), p)
        assert ark.decode_check(gm, 1, gs.ws) == ark.ARK_OK
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


@pytest.mark.parametrize("B", [6, 40])
def test_batched_decode_matches_oracle(models, B):
    """The multi-kernel path at more than 4 sequences on the real geometry:
    the q|k|v, o and down GEMMs store their split sums and a row kernel per
    sequence runs the epilogue and, behind o and down, the RMSNorm and
    quantiser that follow (B = 40: two 32-row blocks per weight fragment).
    Each sequence at its own position, two steps against the oracle."""
    om, gm = models
    assert ark.decode_path(gm, B) == 0
    rng = np.random.default_rng(B)
    T = CFG.max_total_len
    pos = rng.integers(1, T - 2, size=B)
    shape = (B, T, CFG.n_kv_heads, CFG.head_dim)
    kc, vc = [], []
    for _ in range(CFG.n_layers):
        k = rng.standard_normal(shape).astype(np.float32)
        v = rng.standard_normal(shape).astype(np.float32)
        for b in range(B):
            k[b, pos[b]:] = np.nan  # unwritten rows: garbage the mask must drop
            v[b, pos[b]:] = np.inf
        kc.append(k)
        vc.append(v)
    gs = GpuState(gm, B, 1)
    gs.load_caches(kc, vc)
    mask = CFG.mask()
    tok = rng.integers(0, CFG.vocab - 64, size=B).astype(np.int32)
    p = pos.astype(np.int64)
    for step in range(2):
        kd, vd, hid = gs.decode(t(tok), p)
        assert ark.decode_check(gm, B, gs.ws) == ark.ARK_OK
        lo, kdo, vdo, hido = oracle.decode_step(om, tok, p, kc, vc)
        for l in range(CFG.n_layers):
            assert_close(host(kd[l]), kdo[l], f"B={B} step {step} k_delta {l}")
            assert_close(host(vd[l]), vdo[l], f"B={B} step {step} v_delta {l}")
        assert_close(host(hid), hido, f"B={B} step {step} hidden")
        lg = host(gs.logits)
        err = assert_close(lg, lo, f"B={B} step {step} logits") * np.max(np.abs(lo))
        check_tokens(oracle.masked_argmax(lg, mask), oracle.masked_argmax(lo, mask), lo, mask, err,
                     f"B={B} step {step}")
        gs.write_back(p, kd, vd)
        kc = [oracle.cache_write(kc[l], kdo[l], p) for l in range(CFG.n_layers)]
        vc = [oracle.cache_write(vc[l], vdo[l], p) for l in range(CFG.n_layers)]
        tok = oracle.masked_argmax(lo, mask)
        p = p + 1


def test_greedy_loop_matches_oracle(models, path):
    om, gm = models
    assert ark.decode_path(gm, 1) == (1 if path == "mega" else 0)
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


def test_persistent_wait_timeout_is_reported(models, monkeypatch):
    """A bounded wait of the persistent kernel that gives up is reported:
    the test-only spin limit 0 makes the waits give up at their first
    unmet check (every workgroup still runs to its end), ark_decode_check
    returns ARK_E_TIMEOUT and the greedy loop fails with it; the next
    ordinary step reports ARK_OK again."""
    om, gm = models
    monkeypatch.delenv("ARK_DECODE_PATH", raising=False)
    assert ark.decode_path(gm, 1) == 1
    rng = np.random.default_rng(3)
    kc, vc = _caches(CFG, [200], rng)
    gs = GpuState(gm, 1, 1)
    gs.load_caches(kc, vc)
    tok = t(np.array([17], np.int32))
    gs.decode(tok, [200])
    assert ark.decode_check(gm, 1, gs.ws) == ark.ARK_OK
    monkeypatch.setenv("ARK_TEST_SPIN_LIMIT", "0")
    gs.decode(tok, [200])
    assert ark.decode_check(gm, 1, gs.ws) == ark.ARK_E_TIMEOUT
    out = torch.empty((3, 1), dtype=torch.int32, device="cuda")
    kd1, vd1 = gs.deltas(1)
    with pytest.raises(ark.ArkError) as err:
        ark.greedy_decode(gm, tok, [200], gs.kc, gs.vc, kd1, vd1, gs.logits, t(CFG.mask()),
                          CFG.end_id, 3, out, ws=gs.ws, check_every=2)
    assert err.value.status == ark.ARK_E_TIMEOUT
    monkeypatch.delenv("ARK_TEST_SPIN_LIMIT")
    gs.load_caches(kc, vc)
    gs.decode(t(np.array([17], np.int32)), [200])
    assert ark.decode_check(gm, 1, gs.ws) == ark.ARK_OK


def test_greedy_loop_stop_rules_persistent(models, path):
    """The stop rule of the native loop on both paths at the real geometry:
    an end id emitted at step 3 with the host checking every 4 steps (the
    loop runs on to the check and reports end_id after it), and a cache
    that fills up.  On the persistent path the write-back, the stop rule and
    the next launch's preparation run in one kernel between launches."""
    om, gm = models
    rng = np.random.default_rng(31)
    kc, vc = _caches(CFG, [60], rng)
    mask = CFG.mask()
    tok = np.array([123], np.int32)
    want, cur, p = [], tok, np.array([60])
    kco, vco = kc, vc
    for _ in range(3):
        lg, kdo, vdo, _ = oracle.decode_step(om, cur, p, kco, vco)
        kco = [oracle.cache_write(kco[l], kdo[l], p) for l in range(CFG.n_layers)]
        vco = [oracle.cache_write(vco[l], vdo[l], p) for l in range(CFG.n_layers)]
        cur = oracle.masked_argmax(lg, mask)
        want.append(int(cur[0]))
        p = p + 1
    end = want[2]                     # the third greedy id ends the sequence
    if end in want[:2]:
        pytest.skip("the seeded run repeats its third id earlier")
    gs = GpuState(gm, 1, 1)
    gs.load_caches(kc, vc)
    out = torch.full((8, 1), -5, dtype=torch.int32, device="cuda")
    kd1, vd1 = gs.deltas(1)
    n, newpos = ark.greedy_decode(gm, t(tok), [60], gs.kc, gs.vc, kd1, vd1, gs.logits, t(mask),
                                  end, 8, out, ws=gs.ws, check_every=4)
    got = host(out)[:, 0].tolist()
    assert n == 4 and newpos.tolist() == [64]
    assert got[:4] == want[:3] + [end] and got[4:] == [-5] * 4
    # a full cache: two rows left, two steps
    T = CFG.max_total_len
    n, newpos = ark.greedy_decode(gm, t(tok), [T - 2], gs.kc, gs.vc, kd1, vd1, gs.logits,
                                  t(mask), -1, 8, out, ws=gs.ws, check_every=8)
    assert n == 2 and newpos.tolist() == [T]
