"""Helpers shared by the GPU parity tests: run the HIP path through the C
ABI and compare it with the oracle on the same seeded inputs."""
import numpy as np
import torch

from speech_decoder_int8_amd import ark

DEV = "cuda"
TOL = 1e-3        # max |gpu - oracle| / max |oracle| per tensor (fp32 values)


def t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(x):
    torch.cuda.synchronize()
    return x.cpu().numpy()


def rel(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.max(np.abs(b)) if b.size else 0.0
    return float(np.max(np.abs(a - b)) / den) if den > 0 else float(np.max(np.abs(a - b), initial=0.0))


def assert_close(a, b, what, tol=TOL):
    assert np.all(np.isfinite(a)), f"{what}: non-finite GPU values"
    r = rel(a, b)
    assert r <= tol, f"{what}: relative error {r:.3g} > {tol}"
    return r


def check_tokens(gpu_tok, ora_tok, logits_o, mask, err_bound, what):
    """Token ids must match; a mismatch is tolerated only at a near tie of the
    oracle's top-2 unmasked logits (gap <= 2 * the measured logit error)."""
    gpu_tok = np.asarray(gpu_tok)
    ora_tok = np.asarray(ora_tok)
    bad = np.nonzero(gpu_tok != ora_tok)[0]
    for b in bad:
        lg = np.where(mask == 1, -np.inf, logits_o[b].astype(np.float64))
        top2 = np.sort(lg)[-2:]
        gap = top2[1] - top2[0]
        assert gap <= 2 * err_bound, f"{what}: token mismatch at row {b} (gap {gap:.3g})"
    return len(bad)


class GpuState:
    """Device caches, deltas and buffers for B sequences of a model."""

    def __init__(self, model, B, S_max):
        cfg = model.cfg
        self.model, self.B = model, B
        shape = (B, cfg.max_total_len, cfg.n_kv_heads, cfg.head_dim)
        self.kc = [torch.zeros(shape, dtype=torch.float32, device=DEV) for _ in range(cfg.n_layers)]
        self.vc = [torch.zeros(shape, dtype=torch.float32, device=DEV) for _ in range(cfg.n_layers)]
        self.S_max = S_max
        self.kd = torch.empty((cfg.n_layers, B, S_max, cfg.n_kv_heads, cfg.head_dim),
                              dtype=torch.float32, device=DEV)
        self.vd = torch.empty_like(self.kd)
        self.logits = torch.empty((B, cfg.vocab), dtype=torch.float32, device=DEV) \
            if (model.lm_head is not None or getattr(model, "lm_head4", None) is not None) else None
        self.ws = ark.workspace(model, B, S_max)

    def load_caches(self, kc, vc):
        for l in range(len(self.kc)):
            self.kc[l].copy_(t(kc[l]))
            self.vc[l].copy_(t(vc[l]))

    def deltas(self, S):
        kd = self.kd.view(-1)[: self.kd[:, :, :S].numel()].view(self.kd.shape[0], self.B, S,
                                                                 *self.kd.shape[3:])
        vd = self.vd.view(-1)[: kd.numel()].view(kd.shape)
        return kd, vd

    def prefill(self, x, pos):
        B, S = x.shape[0], x.shape[1]
        kd, vd = self.deltas(S)
        hid = torch.empty((B, S, self.model.cfg.hidden), dtype=torch.float32, device=DEV)
        ark.prefill(self.model, x, pos, self.kc, self.vc, kd, vd, self.logits, hid, self.ws)
        return kd, vd, hid

    def decode(self, ids, pos):
        kd, vd = self.deltas(1)
        hid = torch.empty((self.B, 1, self.model.cfg.hidden), dtype=torch.float32, device=DEV)
        ark.decode_step(self.model, ids, pos, self.kc, self.vc, kd, vd, self.logits, hid, self.ws)
        return kd, vd, hid

    def write_back(self, pos, kd, vd):
        ark.cache_write(self.model.dims, pos, self.kc, self.vc, kd, vd)
