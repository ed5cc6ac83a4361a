"""Brute-force pin of the oracle's block and model wiring.

The decoder below is written out again in plain Python at the tiny test
geometry (hidden 64, 4 query heads sharing 2 KV heads of 16, FFN 96,
vocabulary 50, cache 16, 2 layers): integer loops for every int8 MatMul,
binary32 rounding emulated with `struct` at every quantisation and
dequantisation point, Python floats (binary64) for the normalisation, the
rotary embedding, the attention and the MLP gate.  It calls nothing from
the oracle and no numpy arithmetic, so it checks what the oracle's layer and
model functions wire together: which gain feeds which projection, the two
residual adds, the bias on q/k/v only, the rotary step on q and k but not v,
the cache rows taken from this call's deltas, one quantisation per sequence
shared by q/k/v and by gate/up, the final norm of the last row feeding the
int8 LM head, and the masked greedy choice.

What it follows (pages by title and section):
  * model card "ark-asr-3b-onnx", "Shapes": static sequence-major cache,
    every position attended with later rows masked, deltas returned and
    written back at cache_position; "Files": int8 MatMuls, per-channel
    weights, activations quantised at run time; "Inference": prompt rows
    with the audio slots overwritten, masked greedy decoding; "Revision
    history": fp16 embedding table, int8 LM head.
  * sglang-omni cookbook "ARK-ASR-3B", introduction: a dense Qwen2 decoder
    (pre-norm RMSNorm, q/k/v with bias, rotary embedding, grouped-query
    attention, o, residual; RMSNorm, SwiGLU MLP, residual).

Codes, scales, zero points, accumulators and token ids must agree bit for
bit; the float tensors within 1e-6 relative (the two sides sum in different
orders inside binary64 before rounding once to binary32).
"""
import math
import struct

import numpy as np
import pytest

import oracle
import synth

CFG = synth.TINY


def f32(x: float) -> float:
    """Nearest binary32 of a binary64 value (ties to even)."""
    return struct.unpack("f", struct.pack("f", x))[0]


# ------------------------------------------------------- plain arithmetic --
def bf_prep_weight(rows):
    """Per-output-channel symmetric int8 codes of fp32 rows (lists)."""
    codes, scales = [], []
    for r in rows:
        amax = max(abs(v) for v in r)
        s = f32(amax / 127.0)
        scales.append(s)
        if s == 0.0:
            codes.append([0] * len(r))
        else:
            codes.append([max(-127, min(127, round(f32(v / s)))) for v in r])
    return codes, scales


def bf_dynquant(vals):
    """One uint8 (codes, s, z) for a flat list of fp32 values."""
    lo = min(0.0, min(vals))
    hi = max(0.0, max(vals))
    s = f32(f32(hi - lo) / 255.0)
    if s == 0.0:
        return [0] * len(vals), 0.0, 0
    z = max(0, min(255, round(f32(-lo / s))))
    return [max(0, min(255, round(f32(v / s)) + z)) for v in vals], s, z


def bf_matmul_int(codes_row, z, wcodes):
    """acc[n] = sum_k (code_k - z) w[n][k], exact Python integers."""
    a = [c - z for c in codes_row]
    return [sum(x * w for x, w in zip(a, wr)) for wr in wcodes]


def bf_dequant(acc, s, ws, bias=None):
    out = []
    for n, a in enumerate(acc):
        y = f32(f32(float(a)) * f32(s * ws[n]))
        if bias is not None:
            y = f32(y + bias[n])
        out.append(y)
    return out


def bf_rmsnorm(x, g, eps):
    ss = 0.0
    for v in x:
        ss += v * v
    r = 1.0 / math.sqrt(ss / len(x) + eps)
    return [f32((v * r) * gv) for v, gv in zip(x, g)]


def bf_rope(vec, pos, theta):
    """Rotate-half pairs (j, j + D/2) by pos * theta^(-2j/D)."""
    D = len(vec)
    h = D // 2
    out = [0.0] * D
    for j in range(h):
        ang = pos * theta ** (-(2.0 * j) / D)
        c, s = math.cos(ang), math.sin(ang)
        a, b = vec[j], vec[j + h]
        out[j] = f32(a * c - b * s)
        out[j + h] = f32(b * c + a * s)
    return out


def bf_silu_mul(g, u):
    return f32(g / (1.0 + math.exp(-g)) * u)


def bf_argmax_masked(logits, mask):
    best, bi = None, -1
    for v, val in enumerate(logits):
        if mask[v] or val != val:
            continue
        if best is None or val > best:
            best, bi = val, v
    return bi


# ---------------------------------------------------------------- model --
class BruteModel:
    """The tiny decoder's weights as lists, quantised by bf_prep_weight."""

    def __init__(self, cfg):
        self.cfg = cfg
        self.layers = []
        for l in range(cfg.n_layers):
            w = synth.layer_weights(cfg, l)
            lay = {"ln1": [float(v) for v in w["ln1"]], "ln2": [float(v) for v in w["ln2"]]}
            for name in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"):
                lay[name] = bf_prep_weight(w[name].astype(np.float64).tolist())
            for name in ("bq", "bk", "bv"):
                lay[name] = [float(v) for v in w[name]]
            self.layers.append(lay)
        self.final_norm = [float(v) for v in synth.final_norm(cfg)]
        self.lm = bf_prep_weight(synth.lm_head(cfg).astype(np.float64).tolist())
        self.table = synth.embed_table_f16(cfg).astype(np.float64).tolist()


def bf_layer(m, l, xs, p, kcache, vcache, rec):
    """One layer over the S rows xs (lists of H floats) of one sequence at
    position p.  kcache/vcache: [T][NKV][D] lists (read only).  Returns
    (rows out, k delta rows, v delta rows) and fills rec with every
    intermediate (codes, s, z, accumulators, tensors)."""
    cfg = m.cfg
    lay = m.layers[l]
    NH, NKV, D = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    G = NH // NKV
    S = len(xs)
    # RMSNorm 1 over each row, one quantisation over the sequence's rows
    h1 = [bf_rmsnorm(x, lay["ln1"], cfg.rms_eps) for x in xs]
    c1, s1, z1 = bf_dynquant([v for r in h1 for v in r])
    H = cfg.hidden
    rows1 = [c1[i * H:(i + 1) * H] for i in range(S)]
    q, k, v, accq = [], [], [], []
    for i in range(S):
        aq = bf_matmul_int(rows1[i], z1, lay["wq"][0])
        ak = bf_matmul_int(rows1[i], z1, lay["wk"][0])
        av = bf_matmul_int(rows1[i], z1, lay["wv"][0])
        accq.append(aq + ak + av)
        q.append(bf_dequant(aq, s1, lay["wq"][1], lay["bq"]))
        k.append(bf_dequant(ak, s1, lay["wk"][1], lay["bk"]))
        v.append(bf_dequant(av, s1, lay["wv"][1], lay["bv"]))
    # rotary step on every q head and k head (not v), at position p + i
    qr = [[bf_rope(q[i][h * D:(h + 1) * D], p + i, cfg.rope_theta) for h in range(NH)]
          for i in range(S)]
    kr = [[bf_rope(k[i][g * D:(g + 1) * D], p + i, cfg.rope_theta) for g in range(NKV)]
          for i in range(S)]
    vr = [[v[i][g * D:(g + 1) * D] for g in range(NKV)] for i in range(S)]
    # the cache this call sees: rows [p, p + S) replaced by the deltas
    Kh = [[list(kcache[j][g]) for g in range(NKV)] for j in range(cfg.max_total_len)]
    Vh = [[list(vcache[j][g]) for g in range(NKV)] for j in range(cfg.max_total_len)]
    for i in range(S):
        Kh[p + i] = kr[i]
        Vh[p + i] = vr[i]
    attn = []
    for i in range(S):
        row = []
        for h in range(NH):
            g = h // G
            sc = []
            for j in range(p + i + 1):       # keys at or before the row's position
                dot = 0.0
                for d in range(D):
                    dot += qr[i][h][d] * Kh[j][g][d]
                sc.append(dot / math.sqrt(D))
            mx = max(sc)
            e = [math.exp(t - mx) for t in sc]
            den = sum(e)
            for d in range(D):
                num = 0.0
                for j in range(len(e)):
                    num += e[j] * Vh[j][g][d]
                row.append(f32(num / den))
        attn.append(row)
    c2, s2, z2 = bf_dynquant([x for r in attn for x in r])
    Qd = NH * D
    x1, acco = [], []
    for i in range(S):
        ao = bf_matmul_int(c2[i * Qd:(i + 1) * Qd], z2, lay["wo"][0])
        acco.append(ao)
        o = bf_dequant(ao, s2, lay["wo"][1])
        x1.append([f32(a + b) for a, b in zip(xs[i], o)])
    h2 = [bf_rmsnorm(x, lay["ln2"], cfg.rms_eps) for x in x1]
    c3, s3, z3 = bf_dynquant([x for r in h2 for x in r])
    a, accg, accu = [], [], []
    for i in range(S):
        ag = bf_matmul_int(c3[i * H:(i + 1) * H], z3, lay["wg"][0])
        au = bf_matmul_int(c3[i * H:(i + 1) * H], z3, lay["wu"][0])
        accg.append(ag)
        accu.append(au)
        gv = bf_dequant(ag, s3, lay["wg"][1])
        uv = bf_dequant(au, s3, lay["wu"][1])
        a.append([bf_silu_mul(gg, uu) for gg, uu in zip(gv, uv)])
    c4, s4, z4 = bf_dynquant([x for r in a for x in r])
    I = cfg.intermediate
    x2, accd = [], []
    for i in range(S):
        ad = bf_matmul_int(c4[i * I:(i + 1) * I], z4, lay["wd"][0])
        accd.append(ad)
        dv = bf_dequant(ad, s4, lay["wd"][1])
        x2.append([f32(p_ + q_) for p_, q_ in zip(x1[i], dv)])
    rec.update(h1=h1, q1=(c1, s1, z1), accqkv=accq, qrot=qr, k=kr, v=vr, attn=attn,
               q2=(c2, s2, z2), acco=acco, x1=x1, h2=h2, q3=(c3, s3, z3), accg=accg,
               accu=accu, a=a, q4=(c4, s4, z4), accd=accd, x2=x2)
    kd = [[kr[i][g] for g in range(NKV)] for i in range(S)]
    vd = [[vr[i][g] for g in range(NKV)] for i in range(S)]
    return x2, kd, vd


def bf_forward(m, xs, p, kc, vc, recs):
    """All layers, then the LM head on the last row.  kc/vc: per layer
    [T][NKV][D] lists.  Returns (logits, k deltas, v deltas, rows)."""
    kds, vds = [], []
    for l in range(m.cfg.n_layers):
        rec = {}
        xs, kd, vd = bf_layer(m, l, xs, p, kc[l], vc[l], rec)
        recs.append(rec)
        kds.append(kd)
        vds.append(vd)
    hn = bf_rmsnorm(xs[-1], m.final_norm, m.cfg.rms_eps)
    c, s, z = bf_dynquant(hn)
    acc = bf_matmul_int(c, z, m.lm[0])
    logits = bf_dequant(acc, s, m.lm[1])
    recs.append({"hn": hn, "q": (c, s, z), "acc": acc, "logits": logits})
    return logits, kds, vds, xs


# -------------------------------------------------------------- compare --
def _close(a, b, rtol=1e-6):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    scale = max(float(np.max(np.abs(b))), 1e-30)
    err = float(np.max(np.abs(a - b))) / scale
    assert err <= rtol, err


def _same_quant(bq, oq, shape):
    codes, s, z = bq
    oc, os_, oz = oq
    assert float(os_) == s and int(oz) == z
    assert np.array_equal(np.asarray(codes, np.int64).reshape(shape), oc.astype(np.int64))


def _check_layer(om, l, rec, tr, x_in, S):
    """Every intermediate of the oracle's layer against the brute force."""
    cfg = om.cfg
    lay = om.layers[l]
    NH, NKV, D, H = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.hidden
    _close(rec["h1"], tr["h1"][0])
    _same_quant(rec["q1"], tr["quant"]["h1"][0], (S, H))
    # the integer accumulators of q|k|v, from the oracle's own codes
    c, s, z = tr["quant"]["h1"][0]
    acc = np.concatenate([oracle.matmul_integer(c, z, lay.mats[n][0]) for n in ("wq", "wk", "wv")], 1)
    assert np.array_equal(np.asarray(rec["accqkv"], np.int64), acc)
    _close(rec["qrot"], tr["q"][0])
    _close(rec["k"], tr["k"][0])
    _close(rec["v"], tr["v"][0])
    _close(rec["attn"], tr["attn"][0])
    _same_quant(rec["q2"], tr["quant"]["attn"][0], (S, NH * D))
    c, s, z = tr["quant"]["attn"][0]
    assert np.array_equal(np.asarray(rec["acco"], np.int64), oracle.matmul_integer(c, z, lay.mats["wo"][0]))
    _close(rec["x1"], tr["x1"][0])
    _close(rec["h2"], tr["h2"][0])
    _same_quant(rec["q3"], tr["quant"]["h2"][0], (S, H))
    c, s, z = tr["quant"]["h2"][0]
    assert np.array_equal(np.asarray(rec["accg"], np.int64), oracle.matmul_integer(c, z, lay.mats["wg"][0]))
    assert np.array_equal(np.asarray(rec["accu"], np.int64), oracle.matmul_integer(c, z, lay.mats["wu"][0]))
    _close(rec["a"], tr["a"][0])
    _same_quant(rec["q4"], tr["quant"]["a"][0], (S, cfg.intermediate))
    c, s, z = tr["quant"]["a"][0]
    assert np.array_equal(np.asarray(rec["accd"], np.int64), oracle.matmul_integer(c, z, lay.mats["wd"][0]))
    _close(rec["x2"], tr["x2"][0])


@pytest.fixture(scope="module")
def models():
    return BruteModel(CFG), oracle.build_model(CFG, synth)


def test_weights_quantise_identically(models):
    bm, om = models
    for l in range(CFG.n_layers):
        for name in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"):
            codes, scales = bm.layers[l][name]
            assert np.array_equal(np.asarray(codes, np.int64), om.layers[l].mats[name][0].astype(np.int64))
            assert np.array_equal(np.asarray(scales, np.float32), om.layers[l].mats[name][1])
    assert np.array_equal(np.asarray(bm.lm[0], np.int64), om.lm_head[0].astype(np.int64))


def test_prompt_prefill_then_greedy_steps_match_brute_force(models):
    """The tiny prompt (2 ids, 2 audio rows, 1 id) prefilled at position 0,
    then 3 greedy steps with write-back: every layer's codes, scales, zero
    points and accumulators bit for bit, tensors within 1e-6, token ids
    equal."""
    bm, om = models
    cfg = CFG
    L, T, NKV, D = cfg.n_layers, cfg.max_total_len, cfg.n_kv_heads, cfg.head_dim
    ids = synth.prompt_ids(cfg)[0]
    audio = synth.audio_rows(cfg)[0]
    a0, N = cfg.audio_offset, cfg.audio_slots
    S = cfg.prefill_len
    # brute-force prompt rows: table rows, audio rows spliced over [a0, a0 + N)
    xs = [list(bm.table[int(t)]) for t in ids]
    for i in range(N):
        xs[a0 + i] = [float(v) for v in audio[i]]
    x_or = oracle.embed_splice(om.embed, ids[None, :], audio[None], a0)
    assert np.array_equal(np.asarray(xs, np.float32), x_or[0])

    bkc = [[[[0.0] * D for _ in range(NKV)] for _ in range(T)] for _ in range(L)]
    bvc = [[[[0.0] * D for _ in range(NKV)] for _ in range(T)] for _ in range(L)]
    okc = [np.zeros((1, T, NKV, D), np.float32) for _ in range(L)]
    ovc = [np.zeros((1, T, NKV, D), np.float32) for _ in range(L)]
    mask = cfg.mask()
    p = 0
    rows = xs
    for step in range(1 + 3):
        recs = []
        logits, kds, vds, out_rows = bf_forward(bm, rows, p, bkc, bvc, recs)
        trace = {}
        lo, okd, ovd, oh = oracle.forward(om, np.asarray(rows, np.float32)[None], np.array([p]),
                                          okc, ovc, trace)
        for l in range(L):
            _check_layer(om, l, recs[l], trace[l], rows, len(rows))
            _close(kds[l], okd[l][0])
            _close(vds[l], ovd[l][0])
        head = recs[-1]
        _close(head["hn"], oracle.rmsnorm(oh[0, -1:], om.final_norm, cfg.rms_eps)[0])
        c, s, z = oracle.dynquant(oracle.rmsnorm(oh[:, -1], om.final_norm, cfg.rms_eps))
        _same_quant(head["q"], (c, s, z), (1, cfg.hidden))
        assert np.array_equal(np.asarray(head["acc"], np.int64)[None],
                              oracle.matmul_integer(c, z, om.lm_head[0]))
        _close(logits, lo[0])
        _close(out_rows, oh[0])
        tok = bf_argmax_masked(logits, mask)
        assert tok == int(oracle.masked_argmax(lo, mask)[0])
        # write-back of the deltas at the call's position, then the next token
        for l in range(L):
            for i in range(len(rows)):
                bkc[l][p + i] = kds[l][i]
                bvc[l][p + i] = vds[l][i]
            okc[l] = oracle.cache_write(okc[l], okd[l], [p])
            ovc[l] = oracle.cache_write(ovc[l], ovd[l], [p])
        p += len(rows)
        rows = [list(bm.table[tok])]
    assert p == S + 3


def test_two_sequences_at_different_positions_match_brute_force(models):
    """Two sequences in one oracle call, each with its own pre-filled cache
    and position: each is computed alone by the brute force (one
    quantisation per sequence), and the oracle's batched results equal
    them."""
    bm, om = models
    cfg = CFG
    L, T, NKV, D, H = cfg.n_layers, cfg.max_total_len, cfg.n_kv_heads, cfg.head_dim, cfg.hidden
    rng = np.random.default_rng(31)
    B, S = 2, 3
    pos = [5, 0]
    x = (rng.standard_normal((B, S, H)) * np.float32([[[1.0]], [[3.0]]])).astype(np.float32)
    okc = [np.zeros((B, T, NKV, D), np.float32) for _ in range(L)]
    ovc = [np.zeros((B, T, NKV, D), np.float32) for _ in range(L)]
    for l in range(L):
        okc[l][0, :5] = rng.standard_normal((5, NKV, D))
        ovc[l][0, :5] = rng.standard_normal((5, NKV, D))
        # rows past each sequence's valid length hold garbage that is masked
        okc[l][0, 8:] = 7.0
        ovc[l][1, 3:] = -9.0
    lo, okd, ovd, oh = oracle.forward(om, x, np.array(pos), okc, ovc)
    for b in range(B):
        recs = []
        kcl = [okc[l][b].astype(np.float64).tolist() for l in range(L)]
        vcl = [ovc[l][b].astype(np.float64).tolist() for l in range(L)]
        logits, kds, vds, rows = bf_forward(bm, x[b].astype(np.float64).tolist(), pos[b], kcl, vcl, recs)
        _close(rows, oh[b])
        _close(logits, lo[b])
        for l in range(L):
            _close(kds[l], okd[l][b])
            _close(vds[l], ovd[l][b])
