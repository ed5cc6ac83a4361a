"""The re-anchored parity checker (tests/mode_r.py) on the CPU: records
built from the oracle's own trace pass, and a record with one planted slip
(a code, a zero point, an ulp of a residual, a swapped SwiGLU row) fails."""
import copy

import numpy as np
import pytest

import oracle
import synth

import mode_r

CFG = synth.TINY


@pytest.fixture(scope="module")
def run():
    om = oracle.build_model(CFG, synth)
    rng = np.random.default_rng(41)
    B, S = 2, 3
    pos = np.array([5, 0])
    shape = (B, CFG.max_total_len, CFG.n_kv_heads, CFG.head_dim)
    kc = [np.zeros(shape, np.float32) for _ in range(CFG.n_layers)]
    vc = [np.zeros(shape, np.float32) for _ in range(CFG.n_layers)]
    for l in range(CFG.n_layers):
        kc[l][0, :5] = rng.standard_normal((5, CFG.n_kv_heads, CFG.head_dim))
        vc[l][0, :5] = rng.standard_normal((5, CFG.n_kv_heads, CFG.head_dim))
        kc[l][1, 3:] = np.nan                   # masked rows: any content
    x = rng.standard_normal((B, S, CFG.hidden)).astype(np.float32)
    trace = {}
    logits, kd, vd, hid = oracle.forward(om, x, pos, kc, vc, trace)
    recs = [mode_r.record_from_trace(trace[l], B, S, om.layers[l]) for l in range(CFG.n_layers)]
    last = hid[:, -1]
    hn = oracle.rmsnorm(last, om.final_norm, CFG.rms_eps)
    head = {"hn": hn, "hc": np.zeros(hn.shape, np.uint8), "s": np.zeros(B, np.float32),
            "z": np.zeros(B, np.int32)}
    for b in range(B):
        c, s, z = oracle.dynquant(hn[b:b + 1])
        head["hc"][b], head["s"][b], head["z"][b] = c[0], s, z
    return om, x.reshape(B * S, -1), pos, kc, vc, recs, head, logits, kd, vd, B, S


def _check_all(om, x, pos, kc, vc, recs, B, S):
    xin = x
    for l in range(CFG.n_layers):
        kr, v = mode_r.check_layer(om.layers[l], CFG, recs[l], xin, B, S, pos, kc[l], vc[l],
                                   om.cos, om.sin, range(B * S), f"layer {l}")
        xin = recs[l]["x2"]
    return kr, v


def test_oracle_records_pass(run):
    om, x, pos, kc, vc, recs, head, logits, kd, vd, B, S = run
    kr, v = _check_all(om, x, pos, kc, vc, recs, B, S)
    # the deltas the checker derives from the record are the oracle's deltas
    assert np.array_equal(kr, kd[-1]) and np.array_equal(v, vd[-1])
    tok = mode_r.check_head(om, head, recs[-1]["x2"].reshape(B, S, -1)[:, -1], logits,
                            CFG.mask(), range(B), "head")
    assert np.array_equal(tok, oracle.masked_argmax(logits, CFG.mask()))


@pytest.mark.parametrize("slip", ["code", "zero_point", "scale", "x2_ulp", "x1_ulp", "qkv_ulp",
                                  "swiglu_rows", "attention", "h2"])
def test_planted_slips_fail(run, slip):
    om, x, pos, kc, vc, recs, head, logits, kd, vd, B, S = run
    recs = copy.deepcopy(recs)
    d = recs[1]
    if slip == "code":
        d["c3"][2, 7] ^= 1
    elif slip == "zero_point":
        d["z"][1, 0] += 1
    elif slip == "scale":
        d["s"][3, 1] = np.nextafter(d["s"][3, 1], np.float32(1))
    elif slip == "x2_ulp":
        d["x2"][4, 3] = np.nextafter(d["x2"][4, 3], np.float32(10))
    elif slip == "x1_ulp":
        d["x1"][1, 0] = np.nextafter(d["x1"][1, 0], np.float32(10))
    elif slip == "qkv_ulp":
        d["qkv"][0, 5] = np.nextafter(d["qkv"][0, 5], np.float32(10))
    elif slip == "swiglu_rows":
        d["a"][[0, 1]] = d["a"][[1, 0]]
    elif slip == "attention":
        d["attn"][3] *= np.float32(1.001)
    elif slip == "h2":
        d["h2"][2] *= np.float32(1.0001)
    with pytest.raises(AssertionError):
        _check_all(om, x, pos, kc, vc, recs, B, S)
