"""The decode step for callers that cannot allocate (ark_decode_step_noalloc,
scratch in the library's static device array) against ark_decode_step with
a caller workspace: the same kernels, so the deltas, hidden states and
logits must agree bit for bit.  Two calls in a row, the second smaller:
six sequences on the multi-kernel path, then one on the persistent kernel
(whose exchange area shares the array the first call used); then the first
size again."""
import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
from speech_decoder_int8_amd import ark  # noqa: E402

from gpu_util import GpuState, host, t  # noqa: E402

pytestmark = pytest.mark.gpu

CFG = synth.CONFIGS["c1"].with_(name="real2", n_layers=2, vocab=4096, seed=81)


def _one(gm, B, rng, monkeypatch):
    monkeypatch.delenv("ARK_DECODE_PATH", raising=False)
    print(f"no-alloc decode: B={B}, path {ark.decode_path(gm, B)}", flush=True)
    lengths = rng.integers(1, CFG.max_total_len - 1, size=B)
    lengths[0] = 200
    shape = (B, CFG.max_total_len, CFG.n_kv_heads, CFG.head_dim)
    ids = t(rng.integers(0, CFG.vocab - 64, size=B).astype(np.int32))
    ref = GpuState(gm, B, 1)
    got = GpuState(gm, B, 1)
    for l in range(CFG.n_layers):
        k = torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).cuda()
        v = torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).cuda()
        ref.kc[l].copy_(k)
        ref.vc[l].copy_(v)
        got.kc[l].copy_(k)
        got.vc[l].copy_(v)
    kd0, vd0, h0 = ref.decode(ids, lengths)
    kd1, vd1 = got.deltas(1)
    h1 = torch.empty((B, 1, CFG.hidden), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    ark.decode_step_noalloc(gm, ids, lengths, got.kc, got.vc, kd1, vd1, got.logits, h1)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    for name, a, b in (("k delta", kd1, kd0), ("v delta", vd1, vd0), ("hidden", h1, h0),
                       ("logits", got.logits, ref.logits)):
        a, b = host(a), host(b)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"B={B}: {name} differs"


def test_noalloc_decode_matches_workspace_entry(monkeypatch):
    gm = ark.load_model(CFG, synth)
    rng = np.random.default_rng(12)
    _one(gm, 6, rng, monkeypatch)
    _one(gm, 1, rng, monkeypatch)
    _one(gm, 6, rng, monkeypatch)
    _one(gm, 1, rng, monkeypatch)
