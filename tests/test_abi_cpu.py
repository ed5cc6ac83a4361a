"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
its host-side validation rejects bad arguments before touching the GPU."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ark.h")

from speech_decoder_int8_amd import ark  # noqa: E402

pytestmark = pytest.mark.skipif(not os.path.exists(ark.LIB_PATH), reason="libark.so not built")


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ark_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared()
    assert len(names) >= 12
    lib = ark.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert ark.status_string(s)
    assert ark.status_string(-99) == "unknown status"


FAKE = 0x100000          # an aligned, never-dereferenced stand-in device address


def real_dims(**kw):
    d = dict(n_layers=2, hidden=2048, n_heads=16, n_kv_heads=2, head_dim=128,
             intermediate=11008, vocab=151936, max_total_len=512, rms_eps=1e-6, rope_theta=1e6)
    d.update(kw)
    return ark.ArkDims(**d)


def test_workspace_bytes_validates_dims():
    lib = ark.lib()
    d = real_dims()
    assert lib.ark_workspace_bytes(C.byref(d), 1, 1) > 0
    assert lib.ark_workspace_bytes(C.byref(d), 16, 387) > lib.ark_workspace_bytes(C.byref(d), 1, 1)
    for bad in (dict(head_dim=64), dict(n_heads=15), dict(hidden=2000), dict(intermediate=100),
                dict(max_total_len=500), dict(n_layers=0), dict(n_layers=65),
                dict(n_heads=32, n_kv_heads=2)):
        assert lib.ark_workspace_bytes(C.byref(real_dims(**bad)), 1, 1) == 0, bad
    assert lib.ark_workspace_bytes(C.byref(d), 0, 1) == 0
    assert lib.ark_workspace_bytes(C.byref(d), 65, 1) == 0
    assert lib.ark_workspace_bytes(C.byref(d), 1, 0) == 0
    assert lib.ark_workspace_bytes(None, 1, 1) == 0


def fake_qlinear(n, k, bias=False):
    return ark.ArkQLinear(FAKE, FAKE, FAKE, FAKE if bias else None, n, k)


def fake_model(L=2, lm=True, **kw):
    d = real_dims(n_layers=L, **kw)
    H, Q, KV, I = d.hidden, d.n_heads * 128, d.n_kv_heads * 128, d.intermediate
    layers = (ark.ArkLayer * L)()
    for i in range(L):
        layers[i] = ark.ArkLayer(FAKE, FAKE, fake_qlinear(Q, H, True), fake_qlinear(KV, H, True),
                                 fake_qlinear(KV, H, True), fake_qlinear(H, Q), fake_qlinear(I, H),
                                 fake_qlinear(I, H), fake_qlinear(H, I))
    m = ark.ArkModel(d, layers, FAKE, fake_qlinear(d.vocab, H) if lm else ark.ArkQLinear(),
                     FAKE, FAKE, FAKE)
    m._keep = layers
    return m


def prefill_status(m, B=1, S=4, pos=None, ws_bytes=None, **over):
    lib = ark.lib()
    L = m.d.n_layers
    args = dict(embeds=FAKE, kc=[FAKE] * L, vc=[FAKE] * L, kd=FAKE, vd=FAKE, logits=None,
                hidden=None, ws=FAKE, stream=None)
    args.update(over)
    if ws_bytes is None:
        ws_bytes = lib.ark_workspace_bytes(C.byref(m.d), max(B, 1), max(S, 1))
    pos = [0] * max(B, 1) if pos is None else pos
    kc = None if args["kc"] is None else (C.c_void_p * L)(*args["kc"])
    vc = None if args["vc"] is None else (C.c_void_p * L)(*args["vc"])
    return lib.ark_prefill(C.byref(m), B, S, args["embeds"], (C.c_int32 * len(pos))(*pos), kc, vc,
                           args["kd"], args["vd"], args["logits"], args["hidden"], args["ws"],
                           ws_bytes, args["stream"])


def test_prefill_error_paths_enqueue_nothing():
    m = fake_model()
    assert prefill_status(m, embeds=None) == ark.ARK_E_NULL
    assert prefill_status(m, kd=None) == ark.ARK_E_NULL
    assert prefill_status(m, ws=None) == ark.ARK_E_NULL
    assert prefill_status(m, kc=[FAKE, None]) == ark.ARK_E_NULL
    assert prefill_status(m, B=0) == ark.ARK_E_SHAPE
    assert prefill_status(m, B=65, pos=[0] * 65) == ark.ARK_E_SHAPE
    assert prefill_status(m, S=0) == ark.ARK_E_SHAPE
    # the static cache cannot grow: p + S must stay within max_total_len
    assert prefill_status(m, S=4, pos=[509]) == ark.ARK_E_RANGE
    assert prefill_status(m, S=4, pos=[-1]) == ark.ARK_E_RANGE
    assert prefill_status(m, B=2, S=1, pos=[0, 512]) == ark.ARK_E_RANGE
    assert prefill_status(m, ws_bytes=1024) == ark.ARK_E_WORKSPACE
    assert prefill_status(m, ws=FAKE + 16) == ark.ARK_E_ALIGN
    assert prefill_status(m, kd=FAKE + 4) == ark.ARK_E_ALIGN
    # logits requested from a model without an LM head
    assert prefill_status(fake_model(lm=False), logits=FAKE) == ark.ARK_E_SHAPE
    # inconsistent projection shapes / unsupported geometry
    m2 = fake_model()
    m2._keep[1].o = fake_qlinear(2048, 1024)
    assert prefill_status(m2) == ark.ARK_E_SHAPE
    m3 = fake_model()
    m3._keep[0].gate = ark.ArkQLinear(None, FAKE, FAKE, None, 11008, 2048)
    assert prefill_status(m3) == ark.ARK_E_NULL
    m4 = fake_model()
    m4._keep[0].down = fake_qlinear(2048, 11008, bias=True)   # only q/k/v carry a bias
    assert prefill_status(m4) == ark.ARK_E_SHAPE
    m5 = fake_model()
    m5._keep[0].q = ark.ArkQLinear(FAKE + 8, FAKE, FAKE, FAKE, 2048, 2048)
    assert prefill_status(m5) == ark.ARK_E_ALIGN
    assert prefill_status(fake_model(head_dim=64)) == ark.ARK_E_SHAPE
    assert ark.lib().ark_prefill(None, 1, 1, FAKE, None, None, None, FAKE, FAKE, None, None,
                                 FAKE, 1 << 30, None) == ark.ARK_E_NULL


def test_decode_and_loop_error_paths():
    lib = ark.lib()
    m = fake_model()
    L = 2
    kc = (C.c_void_p * L)(FAKE, FAKE)
    pos = (C.c_int32 * 1)(3)
    ws = lib.ark_workspace_bytes(C.byref(m.d), 1, 1)
    assert lib.ark_decode_step(C.byref(m), 1, None, pos, kc, kc, FAKE, FAKE, None, None, FAKE, ws,
                               None) == ark.ARK_E_NULL
    full = (C.c_int32 * 1)(512)
    assert lib.ark_decode_step(C.byref(m), 1, FAKE, full, kc, kc, FAKE, FAKE, None, None, FAKE, ws,
                               None) == ark.ARK_E_RANGE
    m_noemb = fake_model()
    m_noemb.embed_f16 = None
    assert lib.ark_decode_step(C.byref(m_noemb), 1, FAKE, pos, kc, kc, FAKE, FAKE, None, None, FAKE,
                               ws, None) == ark.ARK_E_NULL
    assert lib.ark_greedy_decode(C.byref(m), 1, FAKE, pos, kc, kc, FAKE, FAKE, FAKE, FAKE, 7, 4, 0,
                                 FAKE, FAKE, ws, None) == ark.ARK_E_SHAPE
    assert lib.ark_greedy_decode(C.byref(m), 1, FAKE, pos, kc, kc, FAKE, FAKE, FAKE, None, 7, 4, 1,
                                 FAKE, FAKE, ws, None) == ark.ARK_E_NULL
    assert lib.ark_greedy_decode(C.byref(fake_model(lm=False)), 1, FAKE, pos, kc, kc, FAKE, FAKE,
                                 FAKE, FAKE, 7, 4, 1, FAKE, FAKE, ws, None) == ark.ARK_E_SHAPE


def test_small_call_error_paths():
    lib = ark.lib()
    d = real_dims()
    pos = (C.c_int32 * 2)(0, 510)
    kc = (C.c_void_p * 2)(FAKE, FAKE)
    assert lib.ark_cache_write(C.byref(d), 2, 4, pos, kc, kc, FAKE, FAKE, None) == ark.ARK_E_RANGE
    assert lib.ark_cache_write(C.byref(d), 2, 1, pos, kc, kc, None, FAKE, None) == ark.ARK_E_NULL
    assert lib.ark_cache_write(C.byref(d), 0, 1, pos, kc, kc, FAKE, FAKE, None) == ark.ARK_E_SHAPE
    assert lib.ark_masked_argmax(1, 10, None, FAKE, FAKE, None) == ark.ARK_E_NULL
    assert lib.ark_masked_argmax(0, 10, FAKE, FAKE, FAKE, None) == ark.ARK_E_SHAPE
    assert lib.ark_embed_splice(C.byref(d), 1, 8, FAKE, FAKE, None, 2, 3, FAKE, None) == ark.ARK_E_NULL
    assert lib.ark_embed_splice(C.byref(d), 1, 8, FAKE, FAKE, FAKE, 6, 3, FAKE, None) == ark.ARK_E_SHAPE
    assert lib.ark_embed_splice(C.byref(d), 1, 8, FAKE, FAKE, FAKE, 2, 0, FAKE, None) == ark.ARK_E_SHAPE
    assert lib.ark_prep_weight(FAKE, 4, 40, FAKE, FAKE, FAKE, None) == ark.ARK_E_SHAPE
    assert lib.ark_prep_weight(None, 4, 64, FAKE, FAKE, FAKE, None) == ark.ARK_E_NULL
    assert lib.ark_rope_table(512, 127, 1e6, FAKE, FAKE, None) == ark.ARK_E_SHAPE
    assert lib.ark_test_dynquant(1, 1, 8, FAKE, FAKE, FAKE, FAKE, FAKE, 8, None) == ark.ARK_E_WORKSPACE
    q = ark.ArkQLinear(FAKE, FAKE, FAKE, None, 64, 128)
    assert lib.ark_test_qlinear(1, 5, FAKE, FAKE, FAKE, C.byref(q), None, FAKE, 0, FAKE, 1 << 20,
                                None) == ark.ARK_E_SHAPE
    assert lib.ark_test_swiglu(-1, FAKE, FAKE, FAKE, None) == ark.ARK_E_SHAPE
    assert lib.ark_test_swiglu(4, FAKE, None, FAKE, None) == ark.ARK_E_NULL
    assert lib.ark_test_swiglu(0, None, None, None, None) == ark.ARK_OK   # nothing to do
    q2 = ark.ArkQLinear(FAKE, FAKE, FAKE, None, 64, 192)
    assert lib.ark_test_gate_up(1, 4, FAKE, FAKE, FAKE, C.byref(q), C.byref(q2), FAKE, FAKE, FAKE,
                                FAKE, 1 << 30, None) == ark.ARK_E_SHAPE
    assert lib.ark_test_gate_up(1, 4, FAKE, FAKE, FAKE, C.byref(q), C.byref(q), FAKE, None, FAKE,
                                FAKE, 1 << 30, None) == ark.ARK_E_NULL
    assert lib.ark_test_gate_up(1, 4, FAKE, FAKE, FAKE, C.byref(q), C.byref(q), FAKE, FAKE, FAKE,
                                FAKE, 16, None) == ark.ARK_E_WORKSPACE
    p1 = (C.c_int32 * 1)(500)
    assert lib.ark_test_attention(1, 20, 16, 2, 512, p1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  FAKE, FAKE, 1 << 30, None) == ark.ARK_E_RANGE
    assert lib.ark_test_attention(1, 2, 18, 2, 512, p1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  FAKE, FAKE, 1 << 30, None) == ark.ARK_E_SHAPE
    assert lib.ark_test_attention(1, 2, 16, 2, 500, p1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  FAKE, FAKE, 1 << 30, None) == ark.ARK_E_SHAPE
    assert lib.ark_test_attention_workspace_bytes(0, 1, 16, 512) == 0
