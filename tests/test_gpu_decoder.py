"""End-to-end parity of the decoder step (GPU vs CPU oracle, same seeded
inputs).  Hidden states, deltas and logits must agree within 1e-3 relative
(max-norm); greedy ids must match exactly except at a near tie of the
oracle's top-2 logits.  The GPU is fed the oracle's tokens (teacher forcing)
so both follow one trajectory."""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
from speech_decoder_int8_amd import ark  # noqa: E402

from gpu_util import GpuState, assert_close, check_tokens, host, rel, t  # noqa: E402

pytestmark = pytest.mark.gpu


def _empty(cfg, B):
    shape = (B, cfg.max_total_len, cfg.n_kv_heads, cfg.head_dim)
    return ([np.zeros(shape, np.float32) for _ in range(cfg.n_layers)],
            [np.zeros(shape, np.float32) for _ in range(cfg.n_layers)])


def _compare_step(cfg, what, gs, kd, vd, hid, lo, kdo, vdo, hido, mask):
    S = kdo[0].shape[1]
    for l in range(cfg.n_layers):
        assert_close(host(kd[l]), kdo[l], f"{what} k_delta layer {l}")
        assert_close(host(vd[l]), vdo[l], f"{what} v_delta layer {l}")
    assert_close(host(hid), hido, f"{what} hidden")
    if lo is not None:
        lg = host(gs.logits)
        err = assert_close(lg, lo, f"{what} logits") * np.max(np.abs(lo))
        tok = oracle.masked_argmax(lg, mask)
        check_tokens(tok, oracle.masked_argmax(lo, mask), lo, mask, err, what)
    return S


def run_parity(cfg, om, gm, x, pos0, kc0, vc0, n_decode, ids=None):
    """Prefill (if x is not None) then n_decode steps, comparing every call.
    ids: [n_decode, B] drawn decode ids for a model without an LM head, or
    [1, B] start ids of a greedy run without a prefill."""
    B = cfg.batch
    mask = cfg.mask()
    fixed = ids is not None and om.lm_head is None
    gs = GpuState(gm, B, max(1, 0 if x is None else x.shape[1]))
    gs.load_caches(kc0, vc0)
    kc, vc = kc0, vc0
    p = np.asarray(pos0, np.int64)
    tok = None if ids is None else ids[0]
    if x is not None:
        S = x.shape[1]
        kd, vd, hid = gs.prefill(t(x), p)
        lo, kdo, vdo, hido = oracle.prefill(om, x, p, kc, vc)
        _compare_step(cfg, "prefill", gs, kd, vd, hid, lo, kdo, vdo, hido, mask)
        gs.write_back(p, kd, vd)
        kc = [oracle.cache_write(kc[l], kdo[l], p) for l in range(cfg.n_layers)]
        vc = [oracle.cache_write(vc[l], vdo[l], p) for l in range(cfg.n_layers)]
        p = p + S
        if lo is not None:
            tok = oracle.masked_argmax(lo, mask)
    for step in range(n_decode):
        if fixed:
            tok = ids[step]
        kd, vd, hid = gs.decode(t(np.asarray(tok, np.int32)), p)
        lo, kdo, vdo, hido = oracle.decode_step(om, tok, p, kc, vc)
        _compare_step(cfg, f"decode step {step}", gs, kd, vd, hid, lo, kdo, vdo, hido, mask)
        gs.write_back(p, kd, vd)
        kc = [oracle.cache_write(kc[l], kdo[l], p) for l in range(cfg.n_layers)]
        vc = [oracle.cache_write(vc[l], vdo[l], p) for l in range(cfg.n_layers)]
        p = p + 1
        if lo is not None:
            tok = oracle.masked_argmax(lo, mask)
    # the caches written back on the GPU equal the oracle's (garbage rows
    # that were never written stay bit-identical)
    for l in range(cfg.n_layers):
        for g, o, nm in ((gs.kc[l], kc[l], "k"), (gs.vc[l], vc[l], "v")):
            g = host(g)
            bad = ~np.isfinite(o)
            assert np.array_equal(g[bad], o[bad], equal_nan=True), f"{nm} cache garbage rows, layer {l}"
            assert_close(g[~bad], o[~bad], f"{nm} cache layer {l}")
    return gs


@pytest.fixture(scope="module")
def small():
    cfg = synth.SMALL.with_(batch=3)
    return cfg, oracle.build_model(cfg, synth), ark.load_model(cfg, synth)


def test_small_prompt_prefill_then_decode(small):
    cfg, om, gm = small
    ids = synth.prompt_ids(cfg)
    audio = synth.audio_rows(cfg)
    out = torch.empty((cfg.batch, cfg.prefill_len, cfg.hidden), dtype=torch.float32, device="cuda")
    ark.embed_splice(gm.dims, t(ids), gm.embed_f16, t(audio), cfg.audio_offset, out)
    x = oracle.embed_splice(om.embed, ids, audio, cfg.audio_offset)
    assert np.array_equal(host(out), x)
    kc, vc = _empty(cfg, cfg.batch)
    run_parity(cfg, om, gm, x, [0, 0, 0], kc, vc, cfg.n_decode)


def test_small_prefill_at_positions_with_garbage_rows(small):
    # sequences start at different cache positions; rows past each valid
    # prefix hold NaN/inf garbage that the masking must select away
    cfg, om, gm = small
    rng = np.random.default_rng(31)
    B, T = cfg.batch, cfg.max_total_len
    pos = np.array([0, 9, T - cfg.prefill_len - 3])
    kc, vc = _empty(cfg, B)
    for l in range(cfg.n_layers):
        for b in range(B):
            kc[l][b, :pos[b]] = rng.standard_normal((pos[b], 2, 128))
            vc[l][b, :pos[b]] = rng.standard_normal((pos[b], 2, 128))
            kc[l][b, pos[b]:] = np.nan
            vc[l][b, pos[b]:] = np.inf
    x = rng.standard_normal((B, cfg.prefill_len, cfg.hidden)).astype(np.float32)
    run_parity(cfg, om, gm, x, pos, kc, vc, 3)


@pytest.mark.parametrize("B", [1, 2, 6, 40])
def test_small_decode_from_prefilled_caches(small, B):
    # B <= 4 runs the fused decode GEMV, B > 4 the MFMA GEMM path (33..64
    # rows: two 32-row blocks per weight fragment, split sums through the
    # row kernel)
    cfg, om, gm = small
    cfg = cfg.with_(batch=B, cache_fill=(5, 40))
    lengths = synth.cache_lengths(cfg)
    kc = [synth.prefilled_cache(cfg, l, "k", lengths) for l in range(cfg.n_layers)]
    vc = [synth.prefilled_cache(cfg, l, "v", lengths) for l in range(cfg.n_layers)]
    ids = synth.start_ids(cfg)[None, :]
    run_parity(cfg, om, gm, None, lengths, kc, vc, 4, ids=ids)


def test_small_long_prefill_large_tile_gemm(small):
    # 2 x 150 rows: every projection of the prefill runs the large-tile GEMM
    # (store + bias, residual and SwiGLU epilogues, ragged last tiles)
    cfg, om, _ = small
    cfg = cfg.with_(batch=2, prefill_len=150, max_total_len=192)
    om = oracle.build_model(cfg, synth)
    gm = ark.load_model(cfg, synth)
    rng = np.random.default_rng(33)
    x = rng.standard_normal((2, 150, cfg.hidden)).astype(np.float32)
    kc, vc = _empty(cfg, 2)
    run_parity(cfg, om, gm, x, [0, 20], kc, vc, 2)


def test_small_native_greedy_loop_matches_oracle(small):
    cfg, om, gm = small
    B = cfg.batch
    mask = cfg.mask()
    rng = np.random.default_rng(32)
    x = rng.standard_normal((B, 8, cfg.hidden)).astype(np.float32)
    kc, vc = _empty(cfg, B)
    lo, kdo, vdo, _ = oracle.prefill(om, x, np.zeros(B, np.int64), kc, vc)
    gs = GpuState(gm, B, 8)
    kd, vd, _ = gs.prefill(t(x), [0] * B)
    gs.write_back([0] * B, kd, vd)
    kc = [oracle.cache_write(kc[l], kdo[l], [0] * B) for l in range(cfg.n_layers)]
    vc = [oracle.cache_write(vc[l], vdo[l], [0] * B) for l in range(cfg.n_layers)]
    tok = oracle.masked_argmax(lo, mask)
    steps = 10
    p = np.full(B, 8, np.int64)
    want = []
    cur = tok
    for _ in range(steps):
        lg, kdo, vdo, _ = oracle.decode_step(om, cur, p, kc, vc)
        kc = [oracle.cache_write(kc[l], kdo[l], p) for l in range(cfg.n_layers)]
        vc = [oracle.cache_write(vc[l], vdo[l], p) for l in range(cfg.n_layers)]
        cur = oracle.masked_argmax(lg, mask)
        want.append(cur)
        p = p + 1
    ids = t(tok.astype(np.int32))
    out = torch.empty((steps, B), dtype=torch.int32, device="cuda")
    kd1, vd1 = gs.deltas(1)
    n, newpos = ark.greedy_decode(gm, ids, [8] * B, gs.kc, gs.vc, kd1, vd1, gs.logits, t(mask),
                                  cfg.end_id, steps, out, ws=ark.workspace(gm, B, 1), check_every=4)
    assert n == steps and newpos.tolist() == [8 + steps] * B
    got = host(out)
    assert np.array_equal(got, np.stack(want)), (got, np.stack(want))


def test_greedy_loop_stop_rules(small):
    cfg, om, gm = small
    B = cfg.batch
    gs = GpuState(gm, B, 1)
    kd1, vd1 = gs.deltas(1)
    out = torch.empty((8, B), dtype=torch.int32, device="cuda")
    only_end = np.ones(cfg.vocab, np.uint8)
    only_end[cfg.end_id] = 0                       # the end id is the only candidate
    ids = t(np.array([1, 2, 3], np.int32))
    n, pos = ark.greedy_decode(gm, ids, [0] * B, gs.kc, gs.vc, kd1, vd1, gs.logits, t(only_end),
                               cfg.end_id, 8, out, check_every=1)
    assert n == 1 and pos.tolist() == [1] * B and host(out)[0].tolist() == [cfg.end_id] * B
    # a full cache stops the loop: two rows left
    T = cfg.max_total_len
    n, pos = ark.greedy_decode(gm, ids, [T - 2] * B, gs.kc, gs.vc, kd1, vd1, gs.logits,
                               t(cfg.mask()), cfg.end_id, 8, out, check_every=1)
    assert n == 2 and pos.tolist() == [T] * B


def test_c0_single_layer_real_shape():
    # one decoder layer at the real shape: 64-row prefill, 16 decode steps fed
    # from a 1024-row fp16 table, no LM head
    cfg = synth.CONFIGS["c0"]
    om = oracle.build_model(cfg, synth)
    gm = ark.load_model(cfg, synth)
    kc, vc = _empty(cfg, 1)
    ids = synth.decode_ids(cfg)
    run_parity(cfg, om, gm, synth.prefill_embeds(cfg), [0], kc, vc, cfg.n_decode, ids=ids)
