"""Model-level pins of the oracle: cache logic, batching and the int8 path
against the float model it quantises."""
import numpy as np
import pytest

import oracle
import synth


def _empty_caches(cfg, B):
    shape = (B, cfg.max_total_len, cfg.n_kv_heads, cfg.head_dim)
    return ([np.zeros(shape, np.float32) for _ in range(cfg.n_layers)],
            [np.zeros(shape, np.float32) for _ in range(cfg.n_layers)])


@pytest.fixture(scope="module")
def tiny_float():
    return oracle.build_model(synth.TINY, synth, linear="float")


@pytest.fixture(scope="module")
def tiny_int8():
    return oracle.build_model(synth.TINY, synth, keep_fp32=True)


def _run_incremental(model, x, split):
    """Prefill rows [0, split), then one row at a time with write-back."""
    cfg = model.cfg
    kc, vc = _empty_caches(cfg, x.shape[0])
    p = np.zeros(x.shape[0], np.int64)
    outs = []
    chunks = [x[:, :split]] + [x[:, i:i + 1] for i in range(split, x.shape[1])]
    for xc in chunks:
        _, kd, vd, h = oracle.forward(model, xc, p, kc, vc)
        kc = [oracle.cache_write(kc[l], kd[l], p) for l in range(cfg.n_layers)]
        vc = [oracle.cache_write(vc[l], vd[l], p) for l in range(cfg.n_layers)]
        p = p + xc.shape[1]
        outs.append(h)
    return np.concatenate(outs, axis=1), kc, vc


def test_prefill_equals_prefill_then_decodes_without_quantisation(tiny_float):
    # the static-cache contract of the model card's "Shapes" section: deltas
    # written back at cache_position make later calls see exactly the rows a
    # longer prefill would have seen
    cfg = synth.TINY
    rng = np.random.default_rng(20)
    x = rng.standard_normal((2, 9, cfg.hidden)).astype(np.float32)
    full, kf, vf = _run_incremental(tiny_float, x, 9)
    for split in (1, 4, 8):
        inc, ki, vi = _run_incremental(tiny_float, x, split)
        assert np.allclose(inc, full, rtol=1e-5, atol=1e-5)
        for l in range(cfg.n_layers):
            assert np.allclose(ki[l], kf[l], rtol=1e-5, atol=1e-5)
            assert np.allclose(vi[l], vf[l], rtol=1e-5, atol=1e-5)


def test_batched_equals_individual_bit_exact(tiny_int8):
    # one dynamic quantisation per sequence: a sequence's result does not
    # depend on the other sequences of the batch
    cfg = synth.TINY
    rng = np.random.default_rng(21)
    B, S = 3, 5
    x = rng.standard_normal((B, S, cfg.hidden)).astype(np.float32) * np.float32([[[1.0]], [[5.0]], [[0.2]]])
    kc, vc = _empty_caches(cfg, B)
    for l in range(cfg.n_layers):
        kc[l][:, :4] = rng.standard_normal((B, 4, cfg.n_kv_heads, cfg.head_dim))
        vc[l][:, :4] = rng.standard_normal((B, 4, cfg.n_kv_heads, cfg.head_dim))
    p = np.array([4, 2, 0])
    lg, kd, vd, h = oracle.forward(tiny_int8, x, p, kc, vc)
    for b in range(B):
        lg1, kd1, vd1, h1 = oracle.forward(tiny_int8, x[b:b + 1], p[b:b + 1],
                                           [c[b:b + 1] for c in kc], [c[b:b + 1] for c in vc])
        assert np.array_equal(lg1[0], lg[b]) and np.array_equal(h1[0], h[b])
        for l in range(cfg.n_layers):
            assert np.array_equal(kd1[l][0], kd[l][b]) and np.array_equal(vd1[l][0], vd[l][b])


def test_int8_model_tracks_float_model(tiny_int8):
    # the int8 path computes the float model up to quantisation noise; a
    # transposed operand, a missing zero point or a wrong scale breaks this
    cfg = synth.TINY
    fmodel = oracle.OracleModel(**{**tiny_int8.__dict__, "linear": "float"})
    rng = np.random.default_rng(22)
    x = rng.standard_normal((1, 6, cfg.hidden)).astype(np.float32)
    kc, vc = _empty_caches(cfg, 1)
    lq, _, _, hq = oracle.forward(tiny_int8, x, np.array([0]), kc, vc)
    lf, _, _, hf = oracle.forward(fmodel, x, np.array([0]), kc, vc)
    assert np.max(np.abs(hq - hf)) / np.max(np.abs(hf)) < 0.05
    assert np.max(np.abs(lq - lf)) / np.max(np.abs(lf)) < 0.1
    assert np.corrcoef(lq.ravel(), lf.ravel())[0, 1] > 0.99


def test_delta_rows_are_the_rows_the_cache_receives(tiny_int8):
    cfg = synth.TINY
    rng = np.random.default_rng(23)
    x = rng.standard_normal((1, 3, cfg.hidden)).astype(np.float32)
    kc, vc = _empty_caches(cfg, 1)
    trace = {}
    _, kd, vd, _ = oracle.forward(tiny_int8, x, np.array([6]), kc, vc, trace)
    for l in range(cfg.n_layers):
        assert kd[l].shape == (1, 3, cfg.n_kv_heads, cfg.head_dim)
        assert np.array_equal(kd[l], trace[l]["k"]) and np.array_equal(vd[l], trace[l]["v"])
        w = oracle.cache_write(kc[l], kd[l], [6])
        assert np.array_equal(w[0, 6:9], kd[l][0]) and not w[0, :6].any() and not w[0, 9:].any()


def test_decode_step_is_forward_of_the_embedded_token(tiny_int8):
    cfg = synth.TINY
    kc, vc = _empty_caches(cfg, 2)
    ids = np.array([3, 41])
    a = oracle.decode_step(tiny_int8, ids, np.array([0, 0]), kc, vc)
    x = tiny_int8.embed[ids][:, None, :].astype(np.float32)
    b = oracle.forward(tiny_int8, x, np.array([0, 0]), kc, vc)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[3], b[3])


def test_masked_greedy_never_emits_masked_ids(tiny_int8):
    # with the mask applied the chosen id is never one of the masked added ids,
    # even when the raw maximum is one of them
    cfg = synth.TINY
    mask = cfg.mask()
    assert mask.sum() == cfg.n_added - 1 and mask[cfg.end_id] == 0
    rng = np.random.default_rng(24)
    lg = rng.standard_normal((64, cfg.vocab)).astype(np.float32)
    lg[:, cfg.vocab - 1] = 100.0
    t = oracle.masked_argmax(lg, mask)
    assert not mask[t].any()
