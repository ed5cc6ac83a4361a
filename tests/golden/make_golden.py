"""Write the expected values of the full-size workloads with the CPU oracle.

Calls only oracle/ and synth/.  Usage (from the repository root):
    python tests/golden/make_golden.py c1 [c2 c3 c4 c4_t1024]
Each run writes tests/golden/<config>.npz with sampled outputs of the
oracle's free-running greedy loop (prefill, then decode steps fed with the
oracle's own tokens):
  tokens [n_steps + 1, B]  greedy ids (row 0 from the prefill logits)
  gap    [n_steps + 1, B]  top-2 gap of the unmasked logits at each step
  top_ids / top_vals       [n_steps + 1, B, 16] largest unmasked logits
  samp_idx [512]; samp_vals [n_steps + 1, B, 512]  logits at fixed indices
  hid_last [n_steps + 1, B', H]  residual stream of each sequence's last row
  kd_* / vd_*              deltas of layers (0, L/2, L-1) at sampled rows
  seqs [B']                the sequences hid_last and the deltas keep (all of
                           them up to 4, else first, middle and last)
`python tests/golden/make_golden.py --trim c3` applies that subsetting to a
file written before it existed.
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
SAMPLE_SEED = 4242


def top_unmasked(logits, mask, k=16):
    lg = np.where(mask[None, :] == 1, -np.inf, logits.astype(np.float64))
    idx = np.argsort(-lg, axis=1, kind="stable")[:, :k]
    vals = np.take_along_axis(lg, idx, axis=1)
    return idx.astype(np.int32), vals.astype(np.float32), (vals[:, 0] - vals[:, 1]).astype(np.float32)


def empty_caches(cfg):
    shape = (cfg.batch, cfg.max_total_len, cfg.n_kv_heads, cfg.head_dim)
    return ([np.zeros(shape, np.float32) for _ in range(cfg.n_layers)],
            [np.zeros(shape, np.float32) for _ in range(cfg.n_layers)])


def prefill_input(cfg, model):
    if cfg.prefill_from_embeds:
        return synth.prefill_embeds(cfg)
    return oracle.embed_splice(model.embed, synth.prompt_ids(cfg), synth.audio_rows(cfg),
                               cfg.audio_offset)


def run(name: str) -> None:
    cfg = synth.CONFIGS[name]
    t0 = time.time()
    model = oracle.build_model(cfg, synth)
    print(f"[{name}] model built in {time.time() - t0:.1f}s", flush=True)
    mask = cfg.mask()
    L, B = cfg.n_layers, cfg.batch
    rng = np.random.default_rng(SAMPLE_SEED)
    samp_idx = np.sort(rng.choice(cfg.vocab, 512, replace=False)).astype(np.int32)
    layers = sorted({0, L // 2, L - 1})
    rec = {k: [] for k in ("tokens", "gap", "top_ids", "top_vals", "samp_vals", "hid_last")}
    deltas = {}

    def record(step, logits, kd, vd, hid):
        ti, tv, gap = top_unmasked(logits, mask)
        tok = oracle.masked_argmax(logits, mask)
        rec["tokens"].append(tok)
        rec["gap"].append(gap)
        rec["top_ids"].append(ti)
        rec["top_vals"].append(tv)
        rec["samp_vals"].append(logits[:, samp_idx])
        rec["hid_last"].append(hid[:, -1, :])
        S = kd[0].shape[1]
        rows = sorted({0, S // 2, S - 1})
        for l in layers:
            deltas[f"kd_s{step}_l{l}"] = kd[l][:, rows]
            deltas[f"vd_s{step}_l{l}"] = vd[l][:, rows]
            deltas[f"rows_s{step}"] = np.array(rows, np.int32)
        return tok

    kc, vc = empty_caches(cfg)
    if cfg.prefill_len:
        p = np.zeros(B, np.int64)
        x = prefill_input(cfg, model)
        t1 = time.time()
        logits, kd, vd, hid = oracle.prefill(model, x, p, kc, vc)
        print(f"[{name}] prefill {time.time() - t1:.1f}s", flush=True)
        tok = record(0, logits, kd, vd, hid)
        kc = [oracle.cache_write(kc[l], kd[l], p) for l in range(L)]
        vc = [oracle.cache_write(vc[l], vd[l], p) for l in range(L)]
        p = p + cfg.prefill_len
    else:
        lengths = synth.cache_lengths(cfg)
        kc = [synth.prefilled_cache(cfg, l, "k", lengths) for l in range(L)]
        vc = [synth.prefilled_cache(cfg, l, "v", lengths) for l in range(L)]
        p = lengths.astype(np.int64)
        tok = synth.start_ids(cfg)
        rec["tokens"].append(tok)          # row 0: the given start ids
        for k in ("gap", "top_ids", "top_vals", "samp_vals", "hid_last"):
            rec[k].append(None)
    for step in range(1, cfg.n_decode + 1):
        t1 = time.time()
        logits, kd, vd, hid = oracle.decode_step(model, tok, p, kc, vc)
        tok = record(step, logits, kd, vd, hid)
        kc = [oracle.cache_write(kc[l], kd[l], p) for l in range(L)]
        vc = [oracle.cache_write(vc[l], vd[l], p) for l in range(L)]
        p = p + 1
        print(f"[{name}] step {step}/{cfg.n_decode} {time.time() - t1:.1f}s", flush=True)

    out = {"samp_idx": samp_idx, "layers": np.array(layers, np.int32)}
    for k, v in rec.items():
        if v and v[0] is None:
            v = v[1:]
            out[k + "_from"] = np.array(1)
        out[k] = np.stack(v)
    out.update(deltas)
    path = os.path.join(HERE, f"{name}.npz")
    np.savez_compressed(path, **trim(out, B))
    print(f"[{name}] wrote {path} ({os.path.getsize(path) / 1e3:.0f} kB) in {time.time() - t0:.0f}s",
          flush=True)


def trim(out: dict, B: int) -> dict:
    """Keep the per-sequence hidden states and deltas of a few sequences."""
    if "seqs" in out:
        return out
    seqs = np.arange(B) if B <= 4 else np.array(sorted({0, B // 2, B - 1}))
    res = {}
    for k, v in out.items():
        if k == "hid_last" or k.startswith(("kd_", "vd_")):
            v = v[:, seqs] if k == "hid_last" else v[seqs]
        res[k] = v
    res["seqs"] = seqs.astype(np.int32)
    return res


if __name__ == "__main__":
    args = sys.argv[1:]
    if args and args[0] == "--trim":
        for n in args[1:]:
            path = os.path.join(HERE, f"{n}.npz")
            g = dict(np.load(path))
            np.savez_compressed(path, **trim(g, g["tokens"].shape[1]))
            print(f"[{n}] trimmed to {os.path.getsize(path) / 1e3:.0f} kB")
    else:
        for n in args:
            run(n)
