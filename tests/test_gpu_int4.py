"""The weight-only int4 LM tier on the GPU (model card "ark-asr-3b-onnx",
"Revision history": the int4 LM tier; the block format is the reading the
oracle's int4 functions state and pin).

  * ark_prep_weight_int4: codes, scales and zero points bit for bit equal to
    oracle.prep_weight_int4 (after the layout packing: two uint4 per byte);
  * ark_lm_head_int4: logits within the bound of fp32 summation, on
    weights the oracle prepared:
        |gpu - oracle| <= (32 ceil(K / 2048) + 12) u sum_k s_k |h_k| (q_k + z_k) + u |oracle|
    (u = 2^-24.  A lane sums 32 ceil(K / 2048) terms in sequence and the
    wave then adds 64 partial sums in 6 levels.  At K = 2048 the lane forms
    s (sum h q - z sum h), whose terms are bounded by s |h| (q + z) rather
    than |h w'|; the other kernel sums h w' directly, which the same bound
    covers since |w'| <= s |q - z| (1 + u).  The oracle's fp64 sum is
    rounded once);
  * the decoder with the int4 head on every dispatch path (persistent
    batch-1 kernel, GEMV, row quantiser, prefill): the final norm of the
    GPU's own last hidden row within 1e-6, the logits from the GPU's normed
    row within the bound above, the greedy id the masked argmax of those
    logits; the whole step against the oracle's own forward within the
    decoder tests' 1e-3;
  * at full size (the 3 s clip's prompt and persistent decode steps) on
    sampled vocabulary rows, and the greedy loop against single steps.
"""
import math

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
from speech_decoder_int8_amd import ark  # noqa: E402

import mode_r  # noqa: E402
from gpu_util import GpuState, assert_close, check_tokens, host, t  # noqa: E402

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
F32 = np.float32


def pack_nibbles(q):
    """[n][2m] values 0..15 -> [n][m] bytes, element 2i in the low nibble."""
    q = np.asarray(q, np.uint8)
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(pk):
    pk = np.asarray(pk, np.uint8)
    out = np.empty((pk.shape[0], 2 * pk.shape[1]), np.uint8)
    out[:, 0::2] = pk & 15
    out[:, 1::2] = pk >> 4
    return out


def to_device4(codes, scale, zp):
    """The oracle's int4 weight in the library's layout, on the GPU."""
    return ark.QLinear4(t(pack_nibbles(codes)), t(np.ascontiguousarray(scale, F32)), t(pack_nibbles(zp)))


def bound(h, codes, scale, zp, want):
    """Per-element bound of the kernels' fp32 summation (module docstring)."""
    K = h.shape[1]
    n = codes.shape[0]
    nb = K // oracle.INT4_BLOCK
    qz = codes.reshape(n, nb, -1).astype(np.float64) + zp[:, :, None].astype(np.float64)
    mag = (qz * scale[:, :, None].astype(np.float64)).reshape(n, K)     # s (q + z) per weight
    absum = np.abs(np.asarray(h, np.float64)) @ mag.T
    depth = 32 * math.ceil(K / 2048) + 12
    return depth * U * absum + U * np.abs(np.asarray(want, np.float64))


def check_logits(got, want, bnd, what):
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite logits"
    err = np.abs(got - np.asarray(want, np.float64))
    bad = np.argwhere(err > bnd)
    assert bad.size == 0, f"{what}: {len(bad)} logits outside the bound, first {bad[:4]} " \
                          f"(err {err[tuple(bad[0])]:.3g} > {bnd[tuple(bad[0])]:.3g})"
    return float(np.max(err / np.maximum(bnd, 1e-300)))


def special_weights(rng, n, k):
    """Seeded weights with the degenerate blocks of the format: a block of
    zeros, all positive, all negative, a constant block, one outlier, a
    block whose minimum sits exactly at a level."""
    w = (rng.standard_normal((n, k)) * 0.02).astype(F32)
    B = oracle.INT4_BLOCK
    w[0, :B] = 0.0
    w[1, B:2 * B] = np.abs(w[1, B:2 * B]) + 0.01
    w[2, :B] = -np.abs(w[2, :B]) - 0.01
    w[3, :B] = 0.0371
    w[4, 5] = 3.0
    w[5, :B] = np.linspace(-0.15, 0.6, B).astype(F32)
    w[6, :] = 0.0                               # a whole row of zeros
    return w


@pytest.mark.parametrize("n,k", [(64, 256), (300, 2048), (37, 768), (9, 4096)])
def test_prep_weight_int4_bit_exact(n, k):
    rng = np.random.default_rng(n * 7 + k)
    w = special_weights(rng, n, k)
    codes, scale, zp = ark.prep_weight_int4(t(w))
    q, s, z = oracle.prep_weight_int4(w)
    assert np.array_equal(unpack_nibbles(host(codes)), q)
    gs = host(scale)
    assert np.array_equal(gs.view(np.uint32), s.astype(F32).view(np.uint32))
    assert np.array_equal(unpack_nibbles(host(zp)), z)


def head_rows(cfg, r0, n):
    """Seeded fp32 LM-head rows [r0, r0 + n) (within one generator chunk)."""
    c0 = r0 // synth.ROW_CHUNK * synth.ROW_CHUNK
    c1 = min(cfg.vocab, c0 + synth.ROW_CHUNK)
    assert r0 + n <= c1
    return np.ascontiguousarray(synth.lm_head_rows(cfg, c0, c1)[r0 - c0:r0 - c0 + n])


def test_prep_weight_int4_lm_head_rows():
    """The seeded LM-head rows of the real geometry (several row slices)."""
    cfg = synth.CONFIGS["c1"]
    for r0 in (0, 73828, cfg.vocab - 300):
        w = head_rows(cfg, r0, 300)
        codes, scale, zp = ark.prep_weight_int4(t(w))
        q, s, z = oracle.prep_weight_int4(w)
        assert np.array_equal(unpack_nibbles(host(codes)), q), r0
        assert np.array_equal(host(scale).view(np.uint32), s.view(np.uint32)), r0
        assert np.array_equal(unpack_nibbles(host(zp)), z), r0


HEAD_CASES = [(1, 2048, 1000), (1, 2048, 4099), (1, 2048, 1), (2, 2048, 777), (3, 2048, 513),
              (4, 2048, 1000), (5, 2048, 1000), (7, 2048, 129), (16, 2048, 300), (33, 2048, 200),
              (64, 2048, 64), (1, 256, 37), (3, 768, 100), (17, 4096, 64), (2, 512, 1)]


@pytest.mark.parametrize("B,K,N", HEAD_CASES)
def test_lm_head_int4_kernel(B, K, N):
    rng = np.random.default_rng(B * 1000 + K + N)
    w = special_weights(rng, max(N, 8), K)[:N]
    codes, scale, zp = oracle.prep_weight_int4(w)
    h = rng.standard_normal((B, K)).astype(F32)
    h[0, :3] = [40.0, -35.0, 0.0]
    W = to_device4(codes, scale, zp)
    logits = torch.full((B, N), float("nan"), dtype=torch.float32, device="cuda")
    ark.lm_head_int4(t(h), W, logits)
    want = oracle.lm_head_int4(h, codes, scale, zp)
    check_logits(host(logits), want, bound(h, codes, scale, zp, want), f"B={B} K={K} N={N}")


def test_lm_head_int4_strided_rows():
    """Rows with a stride that is not a multiple of 4 floats (the LDS kernel
    at K = 2048) and an output stride wider than N."""
    rng = np.random.default_rng(9)
    B, K, N = 3, 2048, 500
    w = special_weights(rng, N, K)
    codes, scale, zp = oracle.prep_weight_int4(w)
    hbuf = rng.standard_normal((B, K + 3)).astype(F32)
    h = hbuf[:, :K]
    W = to_device4(codes, scale, zp)
    out = torch.full((B, N + 11), -5.0, dtype=torch.float32, device="cuda")
    hd = t(hbuf)[:, :K]
    ark.lm_head_int4(hd, W, out)
    got = host(out)
    want = oracle.lm_head_int4(h, codes, scale, zp)
    check_logits(got[:, :N], want, bound(h, codes, scale, zp, want), "strided")
    assert np.all(got[:, N:] == -5.0)


# ---------------------------------------------------------- in the decoder --
CFG = synth.CONFIGS["c1"].with_(name="real2", n_layers=2, vocab=4096, seed=78)


@pytest.fixture(scope="module")
def small4():
    om = oracle.build_model(CFG, synth, lm_head4=True)
    gm = ark.load_model(CFG, synth, lm_head4=True)
    assert gm.lm_head is None and gm.lm_head4 is not None
    return om, gm


def _head4_check(om, head, x_last, logits, mask, what):
    """The int4 head's record: final norm of the GPU's last row, then the
    logits from the GPU's normed rows within the summation bound; returns
    the masked argmax of the GPU's logits."""
    cfg = om.cfg
    hn = head["hn"]
    mode_r.check_close(hn, oracle.rmsnorm(x_last, om.final_norm, cfg.rms_eps), 1e-6, f"{what} final norm")
    want = oracle.lm_head_int4(hn, *om.lm_head4)
    check_logits(logits, want, bound(hn, *om.lm_head4, want), f"{what} logits")
    return oracle.masked_argmax(logits, mask)


def _caches(cfg, B, lengths, rng):
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
        kc.append(k)
        vc.append(v)
    return kc, vc


@pytest.mark.parametrize("case", ["mega_b1", "gemv_b1", "gemv_b3", "rows_b6"])
def test_decode_with_int4_head(small4, case, monkeypatch):
    om, gm = small4
    if case == "mega_b1":
        monkeypatch.delenv("ARK_DECODE_PATH", raising=False)
    else:
        monkeypatch.setenv("ARK_DECODE_PATH", "multi")
    B = {"mega_b1": 1, "gemv_b1": 1, "gemv_b3": 3, "rows_b6": 6}[case]
    assert ark.decode_path(gm, B) == (1 if case == "mega_b1" else 0)
    rng = np.random.default_rng(300 + B)
    lengths = rng.integers(0, CFG.max_total_len - 1, size=B)
    kc, vc = _caches(CFG, B, lengths, rng)
    gs = GpuState(gm, B, 1)
    gs.load_caches(kc, vc)
    ids = rng.integers(0, CFG.vocab - 64, size=B).astype(np.int32)
    rec = ark.DumpRecord(gm, B, 1, range(CFG.n_layers))
    kd, vd = gs.deltas(1)
    hid = torch.empty((B, 1, CFG.hidden), dtype=torch.float32, device="cuda")
    ark.decode_step_dump(gm, t(ids), lengths, gs.kc, gs.vc, kd, vd, rec, gs.logits, hid, gs.ws)
    assert ark.decode_check(gm, B, gs.ws) == ark.ARK_OK
    _, head = rec.read()
    lg = host(gs.logits)
    mask = CFG.mask()
    tok = _head4_check(om, head, host(hid).reshape(B, -1), lg, mask, case)
    out = torch.empty(B, dtype=torch.int32, device="cuda")
    ark.masked_argmax(gs.logits, t(mask), out)
    assert np.array_equal(host(out), tok)
    # the whole step against the oracle's own forward
    lo, _, _, _ = oracle.decode_step(om, ids, lengths, kc, vc)
    err = assert_close(lg, lo, f"{case} logits vs oracle forward")
    check_tokens(tok, oracle.masked_argmax(lo, mask), lo, mask, err * np.max(np.abs(lo)), case)


@pytest.mark.parametrize("B,S,p", [(1, 21, [0]), (3, 70, [5, 0, 100])])
def test_prefill_with_int4_head(small4, B, S, p):
    om, gm = small4
    rng = np.random.default_rng(400 + B * S)
    kc, vc = _caches(CFG, B, p, rng)
    gs = GpuState(gm, B, S)
    gs.load_caches(kc, vc)
    x = rng.standard_normal((B, S, CFG.hidden)).astype(F32)
    rec = ark.DumpRecord(gm, B, S, range(CFG.n_layers))
    kd, vd = gs.deltas(S)
    hid = torch.empty((B, S, CFG.hidden), dtype=torch.float32, device="cuda")
    ark.prefill_dump(gm, t(x), p, gs.kc, gs.vc, kd, vd, rec, gs.logits, hid, gs.ws)
    _, head = rec.read()
    lg = host(gs.logits)
    _head4_check(om, head, host(hid)[:, -1], lg, CFG.mask(), f"prefill {B}x{S}")
    lo, _, _, _ = oracle.prefill(om, x, np.array(p), kc, vc)
    assert_close(lg, lo, f"prefill {B}x{S} logits vs oracle forward")


def test_greedy_loop_with_int4_head(small4):
    """ark_greedy_decode with the int4 head (persistent kernel, then the
    head and the argmax) gives the tokens of single steps, and those the
    oracle's."""
    om, gm = small4
    rng = np.random.default_rng(21)
    mask = CFG.mask()
    steps = 4
    kc, vc = _caches(CFG, 1, [40], rng)
    start = np.array([17], np.int32)
    gs = GpuState(gm, 1, 1)
    gs.load_caches(kc, vc)
    ids = t(start)
    out = torch.full((steps, 1), -1, dtype=torch.int32, device="cuda")
    pos = np.array([40], np.int32)
    kd, vd = gs.deltas(1)
    n, newpos = ark.greedy_decode(gm, ids, pos, gs.kc, gs.vc, kd, vd, gs.logits, t(mask), -1, steps,
                                  out, gs.ws, check_every=2)
    assert n == steps and int(newpos[0]) == 40 + steps
    got = host(out)[:, 0]
    # the oracle, step by step from the same caches
    kco, vco = [k.copy() for k in kc], [v.copy() for v in vc]
    tok = start.copy()
    p = 40
    for s in range(steps):
        lo, kdo, vdo, _ = oracle.decode_step(om, tok, np.array([p]), kco, vco)
        nxt = oracle.masked_argmax(lo, mask)
        if int(got[s]) != int(nxt[0]):
            # allowed only at a near tie of the oracle's top two; the sequences part here
            check_tokens(got[s:s + 1], nxt, lo, mask, 1e-3 * np.max(np.abs(lo)), f"step {s}")
            break
        for l in range(CFG.n_layers):
            kco[l] = oracle.cache_write(kco[l], kdo[l], [p])
            vco[l] = oracle.cache_write(vco[l], vdo[l], [p])
        tok = nxt.astype(np.int32)
        p += 1


# ------------------------------------------------------------- full size --
FULL = synth.CONFIGS["c1"]
SAMPLE_ROWS = [(0, 256), (75000, 75256), (FULL.vocab - 256, FULL.vocab)]     # each in one chunk


@pytest.fixture(scope="module")
def full4():
    gm = ark.load_model(FULL, synth, lm_head4=True)
    fn = synth.final_norm(FULL)
    yield gm, fn
    del gm
    torch.cuda.empty_cache()


def test_full_c1_int4_head_persistent_decode(full4):
    """The 3 s clip's prompt, then three persistent decode steps with the
    int4 head: the GPU's prepared weights and its logits on sampled
    vocabulary rows against the oracle, the greedy ids the masked argmax of
    the GPU's logits."""
    gm, fn = full4
    cfg = FULL
    mask = cfg.mask()
    # the GPU's own prepared head on the sampled rows, bit for bit
    ora = {}
    for r0, r1 in SAMPLE_ROWS:
        q, s, z = oracle.prep_weight_int4(head_rows(cfg, r0, r1 - r0))
        ora[r0] = (q, s, z)
        assert np.array_equal(unpack_nibbles(host(gm.lm_head4.codes[r0:r1])), q), r0
        assert np.array_equal(host(gm.lm_head4.scale[r0:r1]).view(np.uint32), s.view(np.uint32)), r0
        assert np.array_equal(unpack_nibbles(host(gm.lm_head4.zp[r0:r1])), z), r0
    S = cfg.prefill_len
    gs = GpuState(gm, 1, S)
    x = torch.empty((1, S, cfg.hidden), dtype=torch.float32, device="cuda")
    ark.embed_splice(gm.dims, t(synth.prompt_ids(cfg)), gm.embed_f16, t(synth.audio_rows(cfg)),
                     cfg.audio_offset, x)
    kd, vd = gs.deltas(S)
    ark.prefill(gm, x, [0], gs.kc, gs.vc, kd, vd, gs.logits, ws=gs.ws)
    gs.write_back([0], kd, vd)
    ids = torch.empty(1, dtype=torch.int32, device="cuda")
    ark.masked_argmax(gs.logits, t(mask), ids)
    p = S
    for step in range(3):
        assert ark.decode_path(gm, 1) == 1
        rec = ark.DumpRecord(gm, 1, 1, [])
        kd, vd = gs.deltas(1)
        hid = torch.empty((1, 1, cfg.hidden), dtype=torch.float32, device="cuda")
        ark.decode_step_dump(gm, ids, [p], gs.kc, gs.vc, kd, vd, rec, gs.logits, hid, gs.ws)
        assert ark.decode_check(gm, 1, gs.ws) == ark.ARK_OK
        _, head = rec.read()
        hn = head["hn"]
        mode_r.check_close(hn, oracle.rmsnorm(host(hid).reshape(1, -1), fn, cfg.rms_eps), 1e-6,
                           f"step {step} final norm")
        lg = host(gs.logits)
        for (r0, r1) in SAMPLE_ROWS:
            q, s, z = ora[r0]
            want = oracle.lm_head_int4(hn, q, s, z)
            check_logits(lg[:, r0:r1], want, bound(hn, q, s, z, want), f"step {step} rows {r0}")
        tok = oracle.masked_argmax(lg, mask)
        gs.write_back([p], kd, vd)
        ark.masked_argmax(gs.logits, t(mask), ids)
        assert int(host(ids)[0]) == int(tok[0])
        p += 1
