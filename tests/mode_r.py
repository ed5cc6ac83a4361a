"""Re-anchored parity checks: the oracle applied to the GPU's own tensors.

A parity record (ark_prefill_dump / ark_decode_step_dump) holds, for each
recorded layer, every tensor the layer's four dynamic quantisations saw,
the codes and (s, z) they produced, and the projection outputs.  The model
card "ark-asr-3b-onnx" ("Files": int8 MatMuls with per-channel weights on
activations quantised at run time) makes every code, scale, zero point and
int32 accumulator a deterministic function of the fp32 tensor in front of
it, so given the GPU's tensor the oracle must reproduce them bit for bit:

  * codes, s, z of every quantisation point == oracle.dynquant(the GPU's
    tensor), per sequence;
  * the q|k|v outputs == oracle dequant(matmul_integer(the GPU's codes));
    x1 == fp32(x + o) and x2 == fp32(x1 + down) from the GPU's codes and
    inputs; the LM head's logits likewise (all bit for bit: the int32
    accumulator and one rounding per operation decide them);
  * the float steps in between (RMSNorm, rotary embedding, attention, the
    SwiGLU gate) agree within their rounding (fp64 inside on both sides):
    1e-6 relative, 1e-5 for the attention.

Only the oracle is called here; nothing of the HIP path is imported.
"""
import numpy as np

import oracle

F32 = np.float32
POINTS = (("h1", "c1"), ("attn", "c2"), ("h2", "c3"), ("a", "c4"))


def bits_equal(a, b) -> bool:
    return np.array_equal(np.asarray(a, F32).view(np.uint32), np.asarray(b, F32).view(np.uint32))


def rel_err(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = float(np.max(np.abs(b))) if b.size else 0.0
    num = float(np.max(np.abs(a - b))) if b.size else 0.0
    return num / den if den > 0 else num


def check_close(a, b, tol, what):
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    r = rel_err(a, b)
    assert r <= tol, f"{what}: relative error {r:.3g} > {tol}"
    return r


def check_quant(vals, codes, s, z, B, S, what):
    """Codes, scale and zero point of each sequence's rows equal the
    oracle's quantisation of the same fp32 values."""
    for b in range(B):
        rows = slice(b * S, (b + 1) * S)
        c, so, zo = oracle.dynquant(vals[rows])
        assert bits_equal(so, s[b]), f"{what} seq {b}: scale {s[b]!r} != {so!r}"
        assert int(zo) == int(z[b]), f"{what} seq {b}: zero point {z[b]} != {zo}"
        bad = int(np.count_nonzero(c != codes[rows]))
        assert bad == 0, f"{what} seq {b}: {bad} codes differ"


def _proj(codes, z, s, mat, bias=None):
    wq, sw = mat
    return oracle.dequant(oracle.matmul_integer(codes, int(z), wq), s, sw, bias)


def _proj_rows(codes, z, s, mat, bias=None):
    """Rows with their own (s, z): one oracle integer MatMul over all rows
    (each row's zero point taken off its codes first, so the sum is still
    sum_k (code - z_row) w exactly), then each row's dequantisation."""
    wq, sw = mat
    shifted = codes.astype(np.int64) - np.asarray(z, np.int64)[:, None]
    acc = oracle.matmul_integer(shifted, 0, wq)
    return np.stack([oracle.dequant(acc[i:i + 1], s[i], sw, bias)[0] for i in range(len(acc))])


def check_layer(lay, cfg, d, x_in, B, S, pos, kc, vc, cos, sin, rows, what):
    """One layer's record.  lay: the oracle's layer (weights); d: the record
    ({field: array}, codes as uint8); x_in [R][H]: the GPU's layer input, or
    None when it is not known (then x1 is checked from the other side only);
    pos [B]; kc, vc [B][T][NKV][D]: the caches the call read; rows: sampled
    row indices for the projection checks."""
    H, NH, NKV, D = cfg.hidden, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    Q, KV = NH * D, NKV * D
    eps = cfg.rms_eps
    # every quantisation point, every row
    for pt, (hv, cv) in enumerate(POINTS):
        check_quant(d[hv], d[cv], d["s"][pt], d["z"][pt], B, S, f"{what} {hv}")
    # the normalisations, from the GPU's inputs
    if x_in is not None:
        check_close(d["h1"], oracle.rmsnorm(x_in, lay.ln1, eps), 1e-6, f"{what} h1")
    check_close(d["h2"], oracle.rmsnorm(d["x1"], lay.ln2, eps), 1e-6, f"{what} h2")
    # projections on sampled rows, bit for bit
    rows = np.asarray(list(rows), np.int64)
    if rows.size:
        bs = rows // S
        sz = lambda pt: (d["s"][pt][bs], d["z"][pt][bs])  # noqa: E731
        s1, z1 = sz(0)
        c1 = d["c1"][rows]
        want = np.concatenate([_proj_rows(c1, z1, s1, lay.mats["wq"], lay.bq),
                               _proj_rows(c1, z1, s1, lay.mats["wk"], lay.bk),
                               _proj_rows(c1, z1, s1, lay.mats["wv"], lay.bv)], axis=1)
        got = d["qkv"][rows]
        assert bits_equal(got, want), \
            f"{what}: q|k|v differ at {np.argwhere(got.view(np.uint32) != want.view(np.uint32))[:8]}"
        s2, z2 = sz(1)
        o = _proj_rows(d["c2"][rows], z2, s2, lay.mats["wo"])
        if x_in is not None:
            want = (x_in[rows] + o).astype(F32)
            assert bits_equal(d["x1"][rows], want), \
                f"{what}: x1 differs at {np.argwhere(d['x1'][rows].view(np.uint32) != want.view(np.uint32))[:8]}"
        s3, z3 = sz(2)
        c3 = d["c3"][rows]
        g = _proj_rows(c3, z3, s3, lay.mats["wg"])
        u = _proj_rows(c3, z3, s3, lay.mats["wu"])
        check_close(d["a"][rows], oracle.swiglu(g, u), 1e-6, f"{what} SwiGLU")
        s4, z4 = sz(3)
        dn = _proj_rows(d["c4"][rows], z4, s4, lay.mats["wd"])
        want = (d["x1"][rows] + dn).astype(F32)
        assert bits_equal(d["x2"][rows], want), \
            f"{what}: x2 differs at {np.argwhere(d['x2'][rows].view(np.uint32) != want.view(np.uint32))[:8]}"
    # rotary embedding and attention, from the GPU's q|k|v and caches
    qkv = d["qkv"].reshape(B, S, Q + 2 * KV)
    q = qkv[..., :Q].reshape(B, S, NH, D)
    k = qkv[..., Q:Q + KV].reshape(B, S, NKV, D)
    v = qkv[..., Q + KV:].reshape(B, S, NKV, D)
    posm = (np.asarray(pos)[:, None] + np.arange(S)[None, :]).astype(np.int64)
    qr = oracle.apply_rope(q, posm, cos, sin)
    kr = oracle.apply_rope(k, posm, cos, sin)
    for b in range(B):
        kh = oracle.cache_write(kc[b:b + 1], kr[b:b + 1], [int(pos[b])])[0]
        vh = oracle.cache_write(vc[b:b + 1], v[b:b + 1], [int(pos[b])])[0]
        att = oracle.attention(qr[b], kh, vh, int(pos[b]))
        check_close(d["attn"][b * S:(b + 1) * S], att, 1e-5, f"{what} seq {b} attention")
    return kr, v


def check_head(model, head, x_last, logits, mask, seqs, what):
    """The LM head's record: final norm of each sequence's last row, its
    quantisation, and the logits from those codes, bit for bit; the greedy
    id is the masked argmax of the GPU's logits."""
    cfg = model.cfg
    check_close(head["hn"], oracle.rmsnorm(x_last, model.final_norm, cfg.rms_eps), 1e-6, f"{what} final norm")
    B = head["hn"].shape[0]
    check_quant(head["hn"], head["hc"], head["s"], head["z"], B, 1, f"{what} LM-head input")
    seqs = np.asarray(list(seqs), np.int64)
    want = _proj_rows(head["hc"][seqs], head["z"][seqs], head["s"][seqs], model.lm_head)
    got = np.asarray(logits, F32)[seqs]
    bad = np.argwhere(got.view(np.uint32) != want.view(np.uint32))
    assert bad.size == 0, f"{what}: {len(bad)} logits differ, first at {bad[:8]}"
    return oracle.masked_argmax(logits, mask)


def record_from_trace(trace_l, B, S, lay):
    """A record built from the oracle's own trace of a layer (for checking
    this module on the CPU): the same fields as the GPU writes."""
    q = trace_l
    R = B * S
    d = {}
    d["h1"] = q["h1"].reshape(R, -1)
    d["attn"] = q["attn"].reshape(R, -1)
    d["x1"] = q["x1"].reshape(R, -1)
    d["h2"] = q["h2"].reshape(R, -1)
    d["a"] = q["a"].reshape(R, -1)
    d["x2"] = q["x2"].reshape(R, -1)
    s = np.zeros((4, B), F32)
    z = np.zeros((4, B), np.int32)
    for pt, (name, cname) in enumerate((("h1", "c1"), ("attn", "c2"), ("h2", "c3"), ("a", "c4"))):
        codes = []
        for b in range(B):
            c, sb, zb = q["quant"][name][b]
            codes.append(c)
            s[pt, b] = sb
            z[pt, b] = zb
        d[cname] = np.concatenate(codes, axis=0)
    d["s"], d["z"] = s, z
    # q|k|v before the rotary step, from the codes
    rows = []
    for r in range(R):
        b = r // S
        c1 = d["c1"][r:r + 1]
        rows.append(np.concatenate([_proj(c1, z[0, b], s[0, b], lay.mats["wq"], lay.bq),
                                    _proj(c1, z[0, b], s[0, b], lay.mats["wk"], lay.bk),
                                    _proj(c1, z[0, b], s[0, b], lay.mats["wv"], lay.bv)], axis=1)[0])
    d["qkv"] = np.stack(rows)
    return d
