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
    for s in (0, -1, -2, -3, -4, -5, -6, -7, -8):
        assert ark.status_string(s) != "unknown status"
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


def test_dump_layout():
    """The parity record layout: 13 fields per recorded layer, 256-byte
    aligned, each large enough for its array, then the head record."""
    lib = ark.lib()
    d = real_dims(n_layers=36)
    B, S = 3, 5
    R = B * S
    f = (C.c_size_t * 13)()
    rec = C.c_size_t()
    head = (C.c_size_t * 4)()
    mask = (1 << 0) | (1 << 17) | (1 << 35) | (1 << 40)     # bit 40 is past n_layers: ignored
    total = lib.ark_dump_layout(C.byref(d), B, S, C.c_uint64(mask), f, C.byref(rec), head)
    H, Q, KV, I = 2048, 2048, 256, 11008
    sizes = [R * H * 4, R * (Q + 2 * KV) * 4, R * Q * 4, R * H * 4, R * H * 4, R * I * 4, R * H * 4,
             R * H, R * Q, R * H, R * I, 4 * B * 4, 4 * B * 4]
    offs = list(f)
    assert offs[0] == 0 and all(o % 256 == 0 for o in offs)
    for i in range(12):
        assert offs[i + 1] - offs[i] >= sizes[i]
    assert rec.value >= offs[12] + sizes[12] and rec.value % 256 == 0
    hs = [B * H * 4, B * H, B * 4, B * 4]
    h = list(head)
    assert h[0] == 3 * rec.value and all(o % 256 == 0 for o in h)
    for i in range(3):
        assert h[i + 1] - h[i] >= hs[i]
    assert total >= h[3] + hs[3]
    assert lib.ark_dump_layout(C.byref(d), B, S, C.c_uint64(0), None, None, None) == total - 3 * rec.value
    assert lib.ark_dump_layout(C.byref(d), 0, S, C.c_uint64(1), None, None, None) == 0
    assert lib.ark_dump_layout(None, 1, 1, C.c_uint64(1), None, None, None) == 0


def test_dump_and_status_error_paths():
    lib = ark.lib()
    m = fake_model()
    L = 2
    kc = (C.c_void_p * L)(FAKE, FAKE)
    pos = (C.c_int32 * 1)(3)
    ws = lib.ark_workspace_bytes(C.byref(m.d), 1, 4)
    need = lib.ark_dump_layout(C.byref(m.d), 1, 4, C.c_uint64(3), None, None, None)
    args = (C.byref(m), 1, 4, FAKE, pos, kc, kc, FAKE, FAKE, None, None, FAKE, ws, None)
    assert lib.ark_prefill_dump(*args, None, need, C.c_uint64(3)) == ark.ARK_E_NULL
    assert lib.ark_prefill_dump(*args, FAKE, need - 1, C.c_uint64(3)) == ark.ARK_E_WORKSPACE
    assert lib.ark_prefill_dump(*args, FAKE + 64, need, C.c_uint64(3)) == ark.ARK_E_ALIGN
    # the plain call's own validation still applies
    bad = (C.byref(m), 1, 4, None, pos, kc, kc, FAKE, FAKE, None, None, FAKE, ws, None)
    assert lib.ark_prefill_dump(*bad, FAKE, need, C.c_uint64(3)) == ark.ARK_E_NULL
    ws1 = lib.ark_workspace_bytes(C.byref(m.d), 1, 1)
    need1 = lib.ark_dump_layout(C.byref(m.d), 1, 1, C.c_uint64(1), None, None, None)
    full = (C.c_int32 * 1)(512)
    assert lib.ark_decode_step_dump(C.byref(m), 1, FAKE, full, kc, kc, FAKE, FAKE, None, None, FAKE,
                                    ws1, None, FAKE, need1, C.c_uint64(1)) == ark.ARK_E_RANGE
    assert lib.ark_decode_step_dump(C.byref(m), 1, FAKE, pos, kc, kc, FAKE, FAKE, None, None, FAKE,
                                    ws1, None, FAKE, 16, C.c_uint64(1)) == ark.ARK_E_WORKSPACE
    # status and path queries validate before any GPU call
    assert lib.ark_decode_check(None, 1, FAKE, ws1, None) == ark.ARK_E_NULL
    assert lib.ark_decode_check(C.byref(m), 1, None, ws1, None) == ark.ARK_E_NULL
    assert lib.ark_decode_check(C.byref(m), 0, FAKE, ws1, None) == ark.ARK_E_SHAPE
    assert lib.ark_decode_check(C.byref(m), 1, FAKE, 16, None) == ark.ARK_E_WORKSPACE
    assert lib.ark_decode_path(None, 1) == ark.ARK_E_NULL
    assert lib.ark_decode_path(C.byref(m), 65) == ark.ARK_E_SHAPE


def test_noalloc_limit_and_validation():
    """The no-allocation decode step rejects, before any GPU call, a call
    whose scratch would exceed the static array, and invalid arguments."""
    lib = ark.lib()
    cap = lib.ark_noalloc_max_bytes()
    assert cap == 64 << 20
    m = fake_model(L=36)
    assert lib.ark_workspace_bytes(C.byref(m.d), 1, 1) <= cap
    assert lib.ark_workspace_bytes(C.byref(m.d), 32, 1) <= cap
    kc = (C.c_void_p * 36)(*([FAKE] * 36))
    pos = (C.c_int32 * 64)(*([3] * 64))
    big = fake_model(L=64, max_total_len=8192)
    kc64 = (C.c_void_p * 64)(*([FAKE] * 64))
    assert lib.ark_workspace_bytes(C.byref(big.d), 64, 1) > cap
    assert lib.ark_decode_step_noalloc(C.byref(big), 64, FAKE, pos, kc64, kc64, FAKE, FAKE, None,
                                       None, None) == ark.ARK_E_NOALLOC
    assert lib.ark_decode_step_noalloc(None, 1, FAKE, pos, kc, kc, FAKE, FAKE, None, None,
                                       None) == ark.ARK_E_NULL
    assert lib.ark_decode_step_noalloc(C.byref(m), 0, FAKE, pos, kc, kc, FAKE, FAKE, None, None,
                                       None) == ark.ARK_E_SHAPE
    assert lib.ark_decode_step_noalloc(C.byref(m), 1, None, pos, kc, kc, FAKE, FAKE, None, None,
                                       None) == ark.ARK_E_NULL


def fake_qlinear4(n, k, **kw):
    a = dict(w=FAKE, scale=FAKE, zp=FAKE, n=n, k=k)
    a.update(kw)
    return ark.ArkQLinear4(**a)


def test_int4_tier_validation():
    # the int4 LM tier replaces the int8 head: logits allowed, both heads not
    m = fake_model(lm=False)
    m.lm_head4 = fake_qlinear4(m.d.vocab, m.d.hidden)
    hid = prefill_status(m, logits=FAKE, ws=None)
    assert hid == ark.ARK_E_NULL            # got past the model checks to the workspace check
    both = fake_model(lm=True)
    both.lm_head4 = fake_qlinear4(both.d.vocab, both.d.hidden)
    assert prefill_status(both) == ark.ARK_E_SHAPE
    for bad, want in ((dict(zp=None), ark.ARK_E_NULL), (dict(scale=None), ark.ARK_E_NULL),
                      (dict(n=1000), ark.ARK_E_SHAPE), (dict(k=1024), ark.ARK_E_SHAPE),
                      (dict(w=FAKE + 8), ark.ARK_E_ALIGN), (dict(scale=FAKE + 2), ark.ARK_E_ALIGN)):
        mb = fake_model(lm=False)
        a = dict(n=mb.d.vocab, k=mb.d.hidden)
        a.update(bad)
        mb.lm_head4 = fake_qlinear4(**a)
        assert prefill_status(mb) == want, bad
    mn = fake_model(lm=False)
    mn.lm_head4 = fake_qlinear4(mn.d.vocab, mn.d.hidden)
    mn.final_norm = None
    assert prefill_status(mn) == ark.ARK_E_NULL


def test_int4_entry_points_error_paths():
    lib = ark.lib()
    assert lib.ark_prep_weight_int4(None, 4, 256, FAKE, FAKE, FAKE, None) == ark.ARK_E_NULL
    assert lib.ark_prep_weight_int4(FAKE, 4, 384, FAKE, FAKE, FAKE, None) == ark.ARK_E_SHAPE
    assert lib.ark_prep_weight_int4(FAKE, 0, 256, FAKE, FAKE, FAKE, None) == ark.ARK_E_SHAPE
    assert lib.ark_prep_weight_int4(FAKE, 4, 256, FAKE + 4, FAKE, FAKE, None) == ark.ARK_E_ALIGN
    W = fake_qlinear4(1000, 2048)
    assert lib.ark_lm_head_int4(1, None, 2048, C.byref(W), FAKE, 1000, None) == ark.ARK_E_NULL
    assert lib.ark_lm_head_int4(0, FAKE, 2048, C.byref(W), FAKE, 1000, None) == ark.ARK_E_SHAPE
    assert lib.ark_lm_head_int4(65, FAKE, 2048, C.byref(W), FAKE, 1000, None) == ark.ARK_E_SHAPE
    assert lib.ark_lm_head_int4(2, FAKE, 2047, C.byref(W), FAKE, 1000, None) == ark.ARK_E_SHAPE
    assert lib.ark_lm_head_int4(2, FAKE, 2048, C.byref(W), FAKE, 999, None) == ark.ARK_E_SHAPE
    assert lib.ark_lm_head_int4(1, FAKE + 4, 2048, C.byref(W), FAKE, 1000, None) == ark.ARK_E_ALIGN
    Wk = fake_qlinear4(1000, 2000)
    assert lib.ark_lm_head_int4(1, FAKE, 2048, C.byref(Wk), FAKE, 1000, None) == ark.ARK_E_SHAPE


def fake_adapter(frame_dim=1280, merge=4, inner=4096, hidden=2048, **over):
    up = fake_qlinear(inner, merge * frame_dim, bias=True)
    down = fake_qlinear(hidden, inner, bias=True)
    a = dict(up=up, down=down, frame_dim=frame_dim, merge=merge)
    a.update(over)
    return ark.ArkAdapter(**a)


def test_adapter_validation():
    lib = ark.lib()
    A = fake_adapter()
    n16 = lib.ark_adapter_workspace_bytes(C.byref(A), 16, 1500)
    assert n16 > lib.ark_adapter_workspace_bytes(C.byref(A), 1, 150) > 0
    # ragged frame counts of several sequences need a compacted copy
    assert lib.ark_adapter_workspace_bytes(C.byref(A), 2, 150) > lib.ark_adapter_workspace_bytes(C.byref(A), 2, 148)
    for B, frames in ((0, 150), (65, 150), (1, 3), (64, 4100)):
        assert lib.ark_adapter_workspace_bytes(C.byref(A), B, frames) == 0, (B, frames)
    assert lib.ark_adapter_workspace_bytes(None, 1, 150) == 0

    def call(A, B=1, frames=150, enc=FAKE, out=FAKE, mid=None, ws=FAKE, nbytes=None):
        if nbytes is None:
            nbytes = lib.ark_adapter_workspace_bytes(C.byref(A), max(B, 1), max(frames, 4)) or (1 << 30)
        return lib.ark_audio_adapter(C.byref(A), B, frames, enc, out, mid, ws, nbytes, None)

    assert call(A, enc=None) == ark.ARK_E_NULL
    assert call(A, out=None) == ark.ARK_E_NULL
    assert call(A, ws=None) == ark.ARK_E_NULL
    assert call(A, enc=FAKE + 4) == ark.ARK_E_ALIGN
    assert call(A, mid=FAKE + 8) == ark.ARK_E_ALIGN
    assert call(A, ws=FAKE + 16) == ark.ARK_E_ALIGN
    assert call(A, nbytes=1024) == ark.ARK_E_WORKSPACE
    assert call(A, frames=3) == ark.ARK_E_SHAPE
    assert call(A, B=0) == ark.ARK_E_SHAPE
    assert call(fake_adapter(up=fake_qlinear(4096, 5120, bias=False))) == ark.ARK_E_NULL
    assert call(fake_adapter(up=fake_qlinear(4096, 5000, bias=True))) == ark.ARK_E_SHAPE
    assert call(fake_adapter(down=fake_qlinear(2048, 4000, bias=True))) == ark.ARK_E_SHAPE
    assert call(fake_adapter(merge=0)) == ark.ARK_E_SHAPE
    assert lib.ark_audio_adapter(None, 1, 150, FAKE, FAKE, None, FAKE, 1 << 30, None) == ark.ARK_E_NULL


def test_adapter_rejects_partial_k_steps():
    lib = ark.lib()
    A = fake_adapter(frame_dim=1288, up=fake_qlinear(4096, 5152, bias=True))
    assert lib.ark_adapter_workspace_bytes(C.byref(A), 1, 150) == 0
    A2 = fake_adapter(inner=4064)
    assert lib.ark_adapter_workspace_bytes(C.byref(A2), 1, 150) == 0


def fake_encoder(L=2, d=1280, heads=20, n_mels=128, ffn=5120, max_pos=1500, **over):
    layers = (ark.ArkEncLayer * L)()
    for i in range(L):
        layers[i] = ark.ArkEncLayer(FAKE, FAKE, FAKE, FAKE, fake_qlinear(d, d, True),
                                    fake_qlinear(d, d, False), fake_qlinear(d, d, True),
                                    fake_qlinear(d, d, True), fake_qlinear(ffn, d, True),
                                    fake_qlinear(d, ffn, True))
    a = dict(n_mels=n_mels, d_model=d, n_heads=heads, ffn=ffn, n_layers=L, max_pos=max_pos,
             ln_eps=1e-5, conv1=fake_qlinear(d, 3 * n_mels, True), conv2=fake_qlinear(d, 3 * d, True),
             pos=FAKE, layers=layers, lnf_g=FAKE, lnf_b=FAKE, rope_cos=FAKE, rope_sin=FAKE)
    a.update(over)
    E = ark.ArkEncoder(**a)
    E._keep = layers
    return E


def test_encoder_validation():
    lib = ark.lib()
    E = fake_encoder()
    assert lib.ark_encoder_workspace_bytes(C.byref(E), 16, 3000) > lib.ark_encoder_workspace_bytes(C.byref(E), 1, 300) > 0
    for B, M in ((0, 300), (65, 300), (1, 0), (1, 3001)):     # 3001 frames -> 1501 > max_pos
        assert lib.ark_encoder_workspace_bytes(C.byref(E), B, M) == 0, (B, M)
    bad = [dict(n_heads=16), dict(n_mels=96, conv1=fake_qlinear(1280, 288, True)),
           dict(ffn=5000), dict(conv2=fake_qlinear(1280, 3000, True))]
    for kw in bad:
        assert lib.ark_encoder_workspace_bytes(C.byref(fake_encoder(**kw)), 1, 300) == 0, kw
    assert lib.ark_encoder_workspace_bytes(C.byref(fake_encoder(pos=None)), 1, 300) == 0

    def call(E, B=1, M=300, mel=FAKE, out=FAKE, ws=FAKE, nbytes=None):
        if nbytes is None:
            nbytes = lib.ark_encoder_workspace_bytes(C.byref(E), max(B, 1), max(M, 1)) or (1 << 40)
        return lib.ark_audio_encoder(C.byref(E), B, M, mel, out, ws, nbytes, None)

    assert call(E, mel=None) == ark.ARK_E_NULL
    assert call(E, out=None) == ark.ARK_E_NULL
    assert call(E, mel=FAKE + 4) == ark.ARK_E_ALIGN
    assert call(E, ws=FAKE + 16) == ark.ARK_E_ALIGN
    assert call(E, nbytes=4096) == ark.ARK_E_WORKSPACE
    assert call(E, M=0) == ark.ARK_E_SHAPE
    E2 = fake_encoder()
    E2._keep[1].k = fake_qlinear(1280, 1280, True)                # the key projection has no bias
    assert call(E2) == ark.ARK_E_SHAPE
    E3 = fake_encoder()
    E3._keep[0].fc1 = fake_qlinear(5120, 1280, False)             # fc1 needs its bias
    assert call(E3) == ark.ARK_E_NULL
    E4 = fake_encoder()
    E4._keep[0].ln2_b = None
    assert call(E4) == ark.ARK_E_NULL
    assert lib.ark_audio_encoder(None, 1, 300, FAKE, FAKE, FAKE, 1 << 40, None) == ark.ARK_E_NULL


def fake_bf16_model(L=2, lm=True, **kw):
    d = real_dims(n_layers=L, **kw)
    H, Q, KV, I = d.hidden, d.n_heads * 128, d.n_kv_heads * 128, d.intermediate

    def lin(n, k, bias=False):
        return ark.ArkLinearBf16(FAKE, FAKE if bias else None, n, k)
    layers = (ark.ArkLayerBf16 * L)()
    for i in range(L):
        layers[i] = ark.ArkLayerBf16(FAKE, FAKE, lin(Q, H, True), lin(KV, H, True), lin(KV, H, True),
                                     lin(H, Q), lin(I, H), lin(I, H), lin(H, I))
    m = ark.ArkModelBf16(d, layers, FAKE, lin(d.vocab, H) if lm else ark.ArkLinearBf16(), FAKE, FAKE,
                         FAKE)
    m._keep = layers
    return m


def test_bf16_validation():
    lib = ark.lib()
    m = fake_bf16_model()
    L = 2
    ws = lib.ark_workspace_bytes_bf16(C.byref(m.d), 1, 4)
    assert ws > 0 and lib.ark_workspace_bytes_bf16(C.byref(m.d), 0, 4) == 0
    kc = (C.c_void_p * L)(FAKE, FAKE)

    def pre(m, B=1, S=4, pos=None, nbytes=None, logits=None, embeds=FAKE, kd=FAKE):
        pos = [0] * B if pos is None else pos
        nb = lib.ark_workspace_bytes_bf16(C.byref(m.d), max(B, 1), max(S, 1)) if nbytes is None else nbytes
        return lib.ark_prefill_bf16(C.byref(m), B, S, embeds, (C.c_int32 * len(pos))(*pos), kc, kc, kd,
                                    FAKE, logits, None, FAKE, nb, None)
    assert pre(m, embeds=None) == ark.ARK_E_NULL
    assert pre(m, B=0, pos=[0]) == ark.ARK_E_SHAPE
    assert pre(m, pos=[510]) == ark.ARK_E_RANGE
    assert pre(m, nbytes=1024) == ark.ARK_E_WORKSPACE
    assert pre(m, kd=FAKE + 2) == ark.ARK_E_ALIGN
    assert pre(fake_bf16_model(lm=False), logits=FAKE) == ark.ARK_E_SHAPE
    m2 = fake_bf16_model()
    m2._keep[0].o = ark.ArkLinearBf16(FAKE, FAKE, 2048, 2048)        # o carries no bias
    assert pre(m2) == ark.ARK_E_SHAPE
    m3 = fake_bf16_model()
    m3._keep[1].down = ark.ArkLinearBf16(FAKE, None, 2048, 11000)
    assert pre(m3) == ark.ARK_E_SHAPE
    m4 = fake_bf16_model()
    m4._keep[0].ln2 = None
    assert pre(m4) == ark.ARK_E_NULL
    assert pre(fake_bf16_model(n_heads=64, n_kv_heads=2)) == ark.ARK_E_SHAPE
    pos = (C.c_int32 * 1)(3)
    assert lib.ark_decode_step_bf16(C.byref(m), 1, None, pos, kc, kc, FAKE, FAKE, None, None, FAKE,
                                    ws, None) == ark.ARK_E_NULL
    assert lib.ark_to_bf16(None, 4, FAKE, None) == ark.ARK_E_NULL
    assert lib.ark_to_bf16(FAKE, -1, FAKE, None) == ark.ARK_E_SHAPE
    d = real_dims()
    assert lib.ark_cache_write_bf16(C.byref(d), 1, 1, (C.c_int32 * 1)(512), kc, kc, FAKE, FAKE,
                                    None) == ark.ARK_E_RANGE
    assert lib.ark_cache_write_bf16(C.byref(d), 1, 1, (C.c_int32 * 1)(0), kc, kc, FAKE + 2, FAKE,
                                    None) == ark.ARK_E_ALIGN
