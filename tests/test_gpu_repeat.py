"""Run-twice bit identity and snapshot / resume of the decode state (model
card "ark-asr-3b-onnx", "Shapes": the state carried between calls is the
caches and cache_position, nothing else).

The kernels fold activation ranges and split-K partial sums with integer
atomics and exchange values between workgroups through tagged words; none
of that may make a result depend on arrival order.  Every path is run twice
on the same inputs and its outputs compared bit for bit: the persistent
batch-1 step (int8 and int4 heads), the multi-kernel step of 32 sequences,
a prefill of 1200 rows (large-tile GEMMs, producer ranges, prefill
attention), the adapter, the encoder and the bf16 variant.  Snapshot /
resume: a greedy run split in two, the caches copied to the host between
the halves and restored into fresh buffers and a fresh workspace, ends with
the same ids and caches, bit for bit, as the run in one piece.
"""
import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
from speech_decoder_int8_amd import ark  # noqa: E402

from gpu_util import GpuState, host, t  # noqa: E402

pytestmark = pytest.mark.gpu

CFG = synth.CONFIGS["c1"].with_(name="real2", n_layers=2, vocab=4096, seed=77)


@pytest.fixture(scope="module")
def model():
    return ark.load_model(CFG, synth)


def _same(a, b, what):
    a, b = host(a), host(b)
    assert a.shape == b.shape, what
    assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"{what}: runs differ"


def _prefilled(gs, B, lengths, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    for l in range(len(gs.kc)):
        gs.kc[l].normal_(generator=g)
        gs.vc[l].normal_(generator=g)
        for b in range(B):
            gs.kc[l][b, lengths[b]:] = 0
            gs.vc[l][b, lengths[b]:] = 0


@pytest.mark.parametrize("B,path", [(1, "mega"), (1, "multi"), (32, "multi")])
def test_decode_step_twice(model, B, path, monkeypatch):
    if path == "multi":
        monkeypatch.setenv("ARK_DECODE_PATH", "multi")
    else:
        monkeypatch.delenv("ARK_DECODE_PATH", raising=False)
    assert ark.decode_path(model, B) == (1 if path == "mega" else 0)
    rng = np.random.default_rng(B)
    lengths = rng.integers(50, 400, B) if B > 1 else np.array([300])
    gs = GpuState(model, B, 1)
    _prefilled(gs, B, lengths, 11)
    ids = t(rng.integers(0, CFG.vocab - 64, B).astype(np.int32))
    outs = []
    for _ in range(2):
        kd, vd, hid = gs.decode(ids, lengths.tolist())
        outs.append((gs.logits.clone(), kd.clone(), vd.clone(), hid.clone()))
    for name, a, b in zip(("logits", "k deltas", "v deltas", "hidden"), outs[0], outs[1]):
        _same(a, b, f"B={B} {path}: {name}")


def test_int4_head_decode_twice(model):
    m4 = model.with_lm_head(lm_head4=ark.load_lm_head_int4(CFG, synth))
    gs = GpuState(m4, 1, 1)
    _prefilled(gs, 1, [120], 5)
    ids = t(np.array([77], np.int32))
    runs = []
    for _ in range(2):
        kd, vd, hid = gs.decode(ids, [120])
        runs.append((gs.logits.clone(), kd.clone(), hid.clone()))
    for name, a, b in zip(("logits", "k deltas", "hidden"), runs[0], runs[1]):
        _same(a, b, f"int4 head: {name}")


def test_prefill_twice(model):
    B, S = 4, 300            # 1200 rows: the large-tile GEMMs
    gs = GpuState(model, B, S)
    x = torch.randn((B, S, CFG.hidden), device="cuda", generator=torch.Generator(device="cuda").manual_seed(3))
    runs = []
    for _ in range(2):
        kd, vd, hid = gs.prefill(x, [0, 17, 60, 200])
        runs.append((gs.logits.clone(), kd.clone(), vd.clone(), hid.clone()))
    for name, a, b in zip(("logits", "k deltas", "v deltas", "hidden"), runs[0], runs[1]):
        _same(a, b, f"prefill 4x300: {name}")


def test_adapter_and_encoder_twice():
    cfg = synth.SMALL
    enc = ark.load_encoder(cfg, synth)
    ad = ark.load_adapter(cfg, synth)
    mel = t(synth.mel_features(cfg.with_(batch=3)))
    F = (mel.shape[1] - 1) // 2 + 1
    runs = []
    for _ in range(2):
        frames = torch.empty((3, F, cfg.enc_dim), device="cuda")
        ark.audio_encoder(enc, mel, frames)
        rows = torch.empty((3, F // cfg.merge, cfg.hidden), device="cuda")
        ark.audio_adapter(ad, frames, rows)
        runs.append((frames, rows))
    _same(runs[0][0], runs[1][0], "encoder frames")
    _same(runs[0][1], runs[1][1], "adapter rows")


def test_bf16_twice():
    cfg = CFG
    mb = ark.load_model_bf16(cfg, synth)
    B, S = 2, 150
    shape = (B, cfg.max_total_len, cfg.n_kv_heads, cfg.head_dim)
    kc = [torch.zeros(shape, dtype=torch.bfloat16, device="cuda") for _ in range(cfg.n_layers)]
    vc = [torch.zeros_like(kc[0]) for _ in range(cfg.n_layers)]
    kd = torch.empty((cfg.n_layers, B, S, cfg.n_kv_heads, cfg.head_dim), dtype=torch.bfloat16,
                     device="cuda")
    vd = torch.empty_like(kd)
    x = torch.randn((B, S, cfg.hidden), device="cuda",
                    generator=torch.Generator(device="cuda").manual_seed(9)).to(torch.bfloat16)
    runs = []
    for _ in range(2):
        lg = torch.empty((B, cfg.vocab), device="cuda")
        ark.prefill_bf16(mb, x, [0, 40], kc, vc, kd, vd, lg)
        runs.append((lg, kd.clone(), vd.clone()))
    for name, a, b in zip(("logits", "k deltas", "v deltas"), runs[0], runs[1]):
        _same(a.float() if a.dtype == torch.bfloat16 else a,
              b.float() if b.dtype == torch.bfloat16 else b, f"bf16 prefill: {name}")


@pytest.mark.parametrize("B,path", [(1, "mega"), (6, "multi")])
def test_snapshot_resume(model, B, path, monkeypatch):
    if path == "multi":
        monkeypatch.setenv("ARK_DECODE_PATH", "multi")
    else:
        monkeypatch.delenv("ARK_DECODE_PATH", raising=False)
    rng = np.random.default_rng(40 + B)
    lengths = rng.integers(50, 300, B) if B > 1 else np.array([90])
    mask = t(CFG.mask())
    start = rng.integers(0, CFG.vocab - 64, B).astype(np.int32)
    steps = 8

    def run(gs, tok, pos, n):
        out = torch.empty((n, B), dtype=torch.int32, device="cuda")
        kd1, vd1 = gs.deltas(1)
        got, newpos = ark.greedy_decode(model, tok, pos, gs.kc, gs.vc, kd1, vd1, gs.logits, mask,
                                        -1, n, out, ws=gs.ws, check_every=n)
        assert got == n
        return host(out), newpos.tolist()

    whole = GpuState(model, B, 1)
    _prefilled(whole, B, lengths, 21)
    ids_whole, pos_whole = run(whole, t(start), lengths.tolist(), steps)

    first = GpuState(model, B, 1)
    _prefilled(first, B, lengths, 21)
    tok = t(start)
    ids_a, pos_a = run(first, tok, lengths.tolist(), steps // 2)
    # the decode state: caches and cache_position (and the next input ids)
    snap_k = [host(c) for c in first.kc]
    snap_v = [host(c) for c in first.vc]
    snap_tok = host(tok)
    del first
    torch.cuda.empty_cache()
    second = GpuState(model, B, 1)
    second.load_caches(snap_k, snap_v)
    ids_b, pos_b = run(second, t(snap_tok), pos_a, steps - steps // 2)
    assert pos_b == pos_whole
    assert np.array_equal(np.concatenate([ids_a, ids_b]), ids_whole)
    for l in range(CFG.n_layers):
        _same(second.kc[l], whole.kc[l], f"k cache {l}")
        _same(second.vc[l], whole.vc[l], f"v cache {l}")
