"""Re-anchored parity through the fused kernels (the parity protocol's
"bit-exact codes, accumulators and ids on the GPU's own tensors").

Each case runs one prefill or decode call through the dump variant of the
C ABI (ark_prefill_dump / ark_decode_step_dump), which records, per layer,
the fp32 tensor in front of each of the four dynamic quantisations, the
codes and (s, z) the kernels actually used, and the projection outputs.
tests/mode_r.py then applies the oracle to the GPU's own tensors: codes,
scales, zero points, q|k|v, both residual sums and the logits must agree
bit for bit, the float steps within their rounding.  Every dispatch path
of the library is covered:
  * batch-1 decode on the persistent kernel (quantisers fused into its
    polls, SwiGLU codes made by the producers) and on the multi-kernel
    path (GEMV prologue);
  * batched decode, B <= 4 (GEMV) and B > 4 (row quantiser + few-row GEMM);
  * prefill below 128 rows (few-row GEMM) and above (large-tile GEMM with
    producer-folded ranges and the matrix-core attention);
  * the full-size workloads: the 3 s clip's 49-row prefill and persistent
    decode steps (all 36 layers), 32 sequences decoding at their own cache
    lengths, and the 16 x 387 coalesced prefill.
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
from speech_decoder_int8_amd import ark  # noqa: E402

import mode_r  # noqa: E402
from gpu_util import GpuState, host, t  # noqa: E402

pytestmark = pytest.mark.gpu

CFG = synth.CONFIGS["c1"].with_(name="real2", n_layers=2, vocab=4096, seed=78)


@pytest.fixture(scope="module")
def small():
    return oracle.build_model(CFG, synth), ark.load_model(CFG, synth)


def _caches(cfg, B, lengths, rng):
    shape = (B, cfg.max_total_len, cfg.n_kv_heads, cfg.head_dim)
    kc, vc = [], []
    for _ in range(cfg.n_layers):
        k = np.zeros(shape, np.float32)
        v = np.zeros(shape, np.float32)
        for b in range(B):
            n = int(lengths[b])
            k[b, :n] = rng.standard_normal((n, cfg.n_kv_heads, cfg.head_dim))
            v[b, :n] = rng.standard_normal((n, cfg.n_kv_heads, cfg.head_dim))
            k[b, n:] = 3.0e4                   # stale rows: selected out, never read into a result
            v[b, n:] = -7.0
        kc.append(k)
        vc.append(v)
    return kc, vc


def _check_call(om, layers, rec, head, x0, B, S, pos, kc, vc, logits, mask, rows, what,
                hidden=None):
    """Check every recorded layer (layers: model layer ids in the record, in
    order; om.layers[i] holds model layer layers[i]) and the head."""
    cfg = om.cfg
    x_in = x0
    prev = None
    for i, l in enumerate(layers):
        d = rec[l]
        xi = x_in if (l == 0 or prev == l - 1) else None
        mode_r.check_layer(om.layers[i], cfg, d, xi, B, S, pos, kc[l], vc[l], om.cos, om.sin,
                           rows, f"{what} layer {l}")
        x_in = d["x2"]
        prev = l
    if logits is not None:
        last = (hidden if hidden is not None else x_in).reshape(B, S, -1)[:, -1]
        tok = mode_r.check_head(om, head, last, logits, mask, range(B), f"{what} head")
        return tok
    return None


def _rows(B, S, per_seq, rng):
    out = []
    for b in range(B):
        pick = {0, S - 1} | set(rng.integers(0, S, size=max(0, per_seq - 2)).tolist())
        out += [b * S + i for i in sorted(pick)]
    return out


@pytest.mark.parametrize("case", ["mega_b1", "gemv_b1", "gemv_b3", "rows_b6", "rows_b40"])
def test_decode_record_small(small, case, monkeypatch):
    om, gm = small
    if case == "mega_b1":
        monkeypatch.delenv("ARK_DECODE_PATH", raising=False)
    else:
        monkeypatch.setenv("ARK_DECODE_PATH", "multi")
    B = {"mega_b1": 1, "gemv_b1": 1, "gemv_b3": 3, "rows_b6": 6, "rows_b40": 40}[case]
    assert ark.decode_path(gm, B) == (1 if case == "mega_b1" else 0)
    rng = np.random.default_rng(100 + B)
    lengths = rng.integers(0, CFG.max_total_len - 1, size=B)
    lengths[0] = 130                           # three live 64-key chunks
    kc, vc = _caches(CFG, B, lengths, rng)
    gs = GpuState(gm, B, 1)
    gs.load_caches(kc, vc)
    ids = rng.integers(0, CFG.vocab - 64, size=B).astype(np.int32)
    rec = ark.DumpRecord(gm, B, 1, range(CFG.n_layers))
    kd, vd = gs.deltas(1)
    hid = torch.empty((B, 1, CFG.hidden), dtype=torch.float32, device="cuda")
    ark.decode_step_dump(gm, t(ids), lengths, gs.kc, gs.vc, kd, vd, rec, gs.logits, hid, gs.ws)
    assert ark.decode_check(gm, B, gs.ws) == ark.ARK_OK
    layers, head = rec.read()
    x0 = oracle.embed_ids(om.embed, ids)
    lg = host(gs.logits)
    _check_call(om, list(range(CFG.n_layers)), layers, head, x0, B, 1, lengths, kc, vc, lg,
                CFG.mask(), range(B), case, host(hid).reshape(B, -1))
    # the deltas are the rotated keys and the values the record implies
    for l in range(CFG.n_layers):
        d = layers[l]
        kr, v = mode_r.check_layer(om.layers[l], CFG, d, None, B, 1, lengths, kc[l], vc[l],
                                   om.cos, om.sin, [], f"{case} deltas {l}")
        mode_r.check_close(host(kd[l]).reshape(kr.shape), kr, 1e-6, f"{case} k delta {l}")
        assert np.array_equal(host(vd[l]).reshape(v.shape), v), f"{case} v delta {l}"


@pytest.mark.parametrize("B,S,p", [(1, 21, [0]), (2, 70, [0, 100]), (3, 130, [5, 0, 200])])
def test_prefill_record_small(small, B, S, p):
    om, gm = small
    rng = np.random.default_rng(200 + B * S)
    kc, vc = _caches(CFG, B, p, rng)
    gs = GpuState(gm, B, S)
    gs.load_caches(kc, vc)
    x = rng.standard_normal((B, S, CFG.hidden)).astype(np.float32)
    rec = ark.DumpRecord(gm, B, S, range(CFG.n_layers))
    kd, vd = gs.deltas(S)
    hid = torch.empty((B, S, CFG.hidden), dtype=torch.float32, device="cuda")
    ark.prefill_dump(gm, t(x), p, gs.kc, gs.vc, kd, vd, rec, gs.logits, hid, gs.ws)
    layers, head = rec.read()
    _check_call(om, list(range(CFG.n_layers)), layers, head, x.reshape(B * S, -1), B, S,
                np.array(p), kc, vc, host(gs.logits), CFG.mask(), _rows(B, S, 6, rng),
                f"prefill {B}x{S}", host(hid).reshape(B * S, -1))


# ------------------------------------------------------------- full size --
# The three full-size workloads share one set of seeded weights (the 3 s
# clip's); their inputs are each workload's own.
FULL = synth.CONFIGS["c1"]
REC_LAYERS = [0, 1, 35]


@pytest.fixture(scope="module")
def full():
    gm = ark.load_model(FULL, synth)
    om = oracle.build_model(FULL, synth, layers=REC_LAYERS, with_embed=True)
    yield om, gm
    del gm
    torch.cuda.empty_cache()


def _full_check(om, layers_rec, head, x0, B, S, pos, kc, vc, logits, mask, rows, what, hidden):
    """Recorded layers REC_LAYERS of a full-size call (om holds those three)."""
    return _check_call(om, REC_LAYERS, layers_rec, head, x0, B, S, pos, kc, vc, logits, mask,
                       rows, what, hidden)


def test_full_c1_prefill_then_persistent_decode(full):
    """The 3 s clip: the spliced 49-row prompt (few-row GEMM path), then
    three greedy steps on the persistent kernel with every layer recorded;
    the greedy ids are the masked argmax of the GPU's own logits."""
    om, gm = full
    cfg = FULL
    mask = cfg.mask()
    S = cfg.prefill_len
    gs = GpuState(gm, 1, S)
    x = torch.empty((1, S, cfg.hidden), dtype=torch.float32, device="cuda")
    ark.embed_splice(gm.dims, t(synth.prompt_ids(cfg)), gm.embed_f16, t(synth.audio_rows(cfg)),
                     cfg.audio_offset, x)
    zeros = [np.zeros((1, cfg.max_total_len, 2, 128), np.float32)] * 36
    rec = ark.DumpRecord(gm, 1, S, REC_LAYERS)
    kd, vd = gs.deltas(S)
    hid = torch.empty((1, S, cfg.hidden), dtype=torch.float32, device="cuda")
    ark.prefill_dump(gm, x, [0], gs.kc, gs.vc, kd, vd, rec, gs.logits, hid, gs.ws)
    layers, head = rec.read()
    rng = np.random.default_rng(5)
    tok = _full_check(om, layers, head, host(x).reshape(S, -1), 1, S, np.array([0]), zeros, zeros,
                      host(gs.logits), mask, _rows(1, S, 8, rng), "c1 prefill",
                      host(hid).reshape(S, -1))
    gs.write_back([0], kd, vd)
    ids = torch.empty(1, dtype=torch.int32, device="cuda")
    ark.masked_argmax(gs.logits, t(mask), ids)
    assert int(host(ids)[0]) == int(tok[0])
    p = S
    all_layers = list(range(36))
    for step in range(3):
        assert ark.decode_path(gm, 1) == 1
        rec = ark.DumpRecord(gm, 1, 1, all_layers)
        kd, vd = gs.deltas(1)
        hid = torch.empty((1, 1, cfg.hidden), dtype=torch.float32, device="cuda")
        kc_before = [host(gs.kc[l]) for l in REC_LAYERS]
        vc_before = [host(gs.vc[l]) for l in REC_LAYERS]
        ark.decode_step_dump(gm, ids, [p], gs.kc, gs.vc, kd, vd, rec, gs.logits, hid, gs.ws)
        assert ark.decode_check(gm, 1, gs.ws) == ark.ARK_OK
        layers, head = rec.read()
        # every layer: the quantisation points
        for l in all_layers:
            d = layers[l]
            for pt, (hv, cv) in enumerate(mode_r.POINTS):
                mode_r.check_quant(d[hv], d[cv], d["s"][pt], d["z"][pt], 1, 1, f"c1 step {step} layer {l} {hv}")
            assert d["x2"].shape == (1, cfg.hidden) and np.all(np.isfinite(d["x2"]))
        # the recorded layers in full, from the caches the step read
        kcs = {l: kc_before[i] for i, l in enumerate(REC_LAYERS)}
        vcs = {l: vc_before[i] for i, l in enumerate(REC_LAYERS)}
        x0 = oracle.embed_ids(om.embed, host(ids))
        sub = {l: layers[l] for l in REC_LAYERS}
        # layer 1's input is layer 0's x2, layer 35's is layer 34's (recorded here)
        for i, l in enumerate(REC_LAYERS):
            xi = x0 if l == 0 else layers[l - 1]["x2"]
            mode_r.check_layer(om.layers[i], cfg, sub[l], xi, 1, 1, np.array([p]), kcs[l], vcs[l],
                               om.cos, om.sin, [0], f"c1 step {step} layer {l}")
        lg = host(gs.logits)
        tok = mode_r.check_head(om, head, host(hid).reshape(1, -1), lg, mask, [0], f"c1 step {step} head")
        gs.write_back([p], kd, vd)
        ark.masked_argmax(gs.logits, t(mask), ids)
        assert int(host(ids)[0]) == int(tok[0])
        p += 1


def test_full_c3_batched_decode(full):
    """32 sequences at their own cache lengths (uniform in [50, 400]), one
    lockstep step on the multi-kernel path (row quantiser, few-row GEMM,
    split decode attention)."""
    om, gm = full
    cfg3 = synth.CONFIGS["c3"]
    B = cfg3.batch
    lengths = synth.cache_lengths(cfg3)
    gs = GpuState(gm, B, 1)
    kc, vc = {}, {}
    for l in range(36):
        k = synth.prefilled_cache(cfg3, l, "k", lengths)
        v = synth.prefilled_cache(cfg3, l, "v", lengths)
        gs.kc[l].copy_(t(k))
        gs.vc[l].copy_(t(v))
        if l in REC_LAYERS:
            kc[l], vc[l] = k, v
    ids = synth.start_ids(cfg3)
    assert ark.decode_path(gm, B) == 0
    rec = ark.DumpRecord(gm, B, 1, REC_LAYERS)
    kd, vd = gs.deltas(1)
    hid = torch.empty((B, 1, FULL.hidden), dtype=torch.float32, device="cuda")
    ark.decode_step_dump(gm, t(ids), lengths, gs.kc, gs.vc, kd, vd, rec, gs.logits, hid, gs.ws)
    layers, head = rec.read()
    x0 = oracle.embed_ids(om.embed, ids)
    for i, l in enumerate(REC_LAYERS):
        xi = x0 if l == 0 else (layers[l - 1]["x2"] if (l - 1) in layers else None)
        mode_r.check_layer(om.layers[i], FULL, layers[l], xi, B, 1, lengths, kc[l], vc[l], om.cos,
                           om.sin, list(range(0, B, 3)), f"c3 layer {l}")
    mode_r.check_head(om, head, host(hid).reshape(B, -1), host(gs.logits), FULL.mask(), range(B),
                      "c3 head")


def test_full_c4_coalesced_prefill(full):
    """16 x 387 rows through the large-tile GEMM, the producer-folded
    quantisation ranges and the matrix-core prefill attention."""
    om, gm = full
    cfg4 = synth.CONFIGS["c4"]
    B, S = cfg4.batch, cfg4.prefill_len
    x = synth.prefill_embeds(cfg4)
    gs = GpuState(gm, B, S)
    rec = ark.DumpRecord(gm, B, S, REC_LAYERS)
    kd, vd = gs.deltas(S)
    hid = torch.empty((B, S, FULL.hidden), dtype=torch.float32, device="cuda")
    ark.prefill_dump(gm, t(x), [0] * B, gs.kc, gs.vc, kd, vd, rec, gs.logits, hid, gs.ws)
    layers, head = rec.read()
    del rec
    zeros = np.zeros((B, FULL.max_total_len, 2, 128), np.float32)
    rng = np.random.default_rng(44)
    for i, l in enumerate(REC_LAYERS):
        xi = x.reshape(B * S, -1) if l == 0 else (layers[l - 1]["x2"] if (l - 1) in layers else None)
        mode_r.check_layer(om.layers[i], FULL, layers[l], xi, B, S, np.zeros(B, np.int64), zeros,
                           zeros, om.cos, om.sin, _rows(B, S, 3, rng), f"c4 layer {l}")
    mode_r.check_head(om, head, host(hid)[:, -1], host(gs.logits), FULL.mask(), range(B), "c4 head")
