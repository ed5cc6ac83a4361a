"""ctypes binding of libark.so (include/ark.h).

Argument marshalling only: every step of the decoder runs in the library's
HIP kernels.  PyTorch supplies device memory and the current HIP stream.
The functions mirror the C entry points by name and raise ArkError on a
non-zero status.  Loading fails loudly when libark.so has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# ARK_LIBRARY selects another build of the same library (one built with host
# sanitizers, for instance); by default the one built in-tree.
LIB_PATH = os.environ.get("ARK_LIBRARY") or os.path.join(HERE, "libark.so")

ARK_OK, ARK_E_NULL, ARK_E_SHAPE, ARK_E_RANGE, ARK_E_WORKSPACE, ARK_E_HIP, ARK_E_ALIGN = \
    0, -1, -2, -3, -4, -5, -6
ARK_E_TIMEOUT = -7
ARK_E_NOALLOC = -8

# fields of a layer record of the parity dump (enum ark_dump_field)
DUMP_FIELDS = ("h1", "qkv", "attn", "x1", "h2", "a", "x2", "c1", "c2", "c3", "c4", "s", "z")


class ArkError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: {text} (status {status})")
        self.status = status


class ArkDims(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("hidden", C.c_int32), ("n_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("intermediate", C.c_int32),
                ("vocab", C.c_int32), ("max_total_len", C.c_int32), ("rms_eps", C.c_double),
                ("rope_theta", C.c_double)]


class ArkQLinear(C.Structure):
    _fields_ = [("w", C.c_void_p), ("scale", C.c_void_p), ("colsum", C.c_void_p),
                ("bias", C.c_void_p), ("n", C.c_int32), ("k", C.c_int32)]


class ArkQLinear4(C.Structure):
    _fields_ = [("w", C.c_void_p), ("scale", C.c_void_p), ("zp", C.c_void_p),
                ("n", C.c_int32), ("k", C.c_int32)]


class ArkAdapter(C.Structure):
    _fields_ = [("up", ArkQLinear), ("down", ArkQLinear), ("frame_dim", C.c_int32),
                ("merge", C.c_int32)]


class ArkEncLayer(C.Structure):
    _fields_ = [("ln1_g", C.c_void_p), ("ln1_b", C.c_void_p), ("ln2_g", C.c_void_p),
                ("ln2_b", C.c_void_p), ("q", ArkQLinear), ("k", ArkQLinear), ("v", ArkQLinear),
                ("o", ArkQLinear), ("fc1", ArkQLinear), ("fc2", ArkQLinear)]


class ArkEncoder(C.Structure):
    _fields_ = [("n_mels", C.c_int32), ("d_model", C.c_int32), ("n_heads", C.c_int32),
                ("ffn", C.c_int32), ("n_layers", C.c_int32), ("max_pos", C.c_int32),
                ("ln_eps", C.c_double), ("conv1", ArkQLinear), ("conv2", ArkQLinear),
                ("pos", C.c_void_p), ("layers", C.POINTER(ArkEncLayer)), ("lnf_g", C.c_void_p),
                ("lnf_b", C.c_void_p), ("rope_cos", C.c_void_p), ("rope_sin", C.c_void_p)]


class ArkLinearBf16(C.Structure):
    _fields_ = [("w", C.c_void_p), ("bias", C.c_void_p), ("n", C.c_int32), ("k", C.c_int32)]


class ArkLayerBf16(C.Structure):
    _fields_ = [("ln1", C.c_void_p), ("ln2", C.c_void_p), ("q", ArkLinearBf16), ("k", ArkLinearBf16),
                ("v", ArkLinearBf16), ("o", ArkLinearBf16), ("gate", ArkLinearBf16),
                ("up", ArkLinearBf16), ("down", ArkLinearBf16)]


class ArkLayer(C.Structure):
    _fields_ = [("ln1", C.c_void_p), ("ln2", C.c_void_p), ("q", ArkQLinear), ("k", ArkQLinear),
                ("v", ArkQLinear), ("o", ArkQLinear), ("gate", ArkQLinear), ("up", ArkQLinear),
                ("down", ArkQLinear)]


class ArkModel(C.Structure):
    _fields_ = [("d", ArkDims), ("layers", C.POINTER(ArkLayer)), ("final_norm", C.c_void_p),
                ("lm_head", ArkQLinear), ("embed_f16", C.c_void_p), ("rope_cos", C.c_void_p),
                ("rope_sin", C.c_void_p), ("lm_head4", ArkQLinear4)]


class ArkModelBf16(C.Structure):
    _fields_ = [("d", ArkDims), ("layers", C.POINTER(ArkLayerBf16)), ("final_norm", C.c_void_p),
                ("lm_head", ArkLinearBf16), ("embed", C.c_void_p), ("rope_cos", C.c_void_p),
                ("rope_sin", C.c_void_p)]


P = C.c_void_p
I32 = C.c_int32
PP = C.POINTER(C.c_void_p)
PI32 = C.POINTER(C.c_int32)
PSZ = C.POINTER(C.c_size_t)

_SIGS = {
    "ark_workspace_bytes": (C.c_size_t, [C.POINTER(ArkDims), I32, I32]),
    "ark_status_string": (C.c_char_p, [C.c_int]),
    "ark_prep_weight": (C.c_int, [P, I32, I32, P, P, P, P]),
    "ark_rope_table": (C.c_int, [I32, I32, C.c_double, P, P, P]),
    "ark_prep_weight_int4": (C.c_int, [P, I32, I32, P, P, P, P]),
    "ark_to_bf16": (C.c_int, [P, C.c_int64, P, P]),
    "ark_workspace_bytes_bf16": (C.c_size_t, [C.POINTER(ArkDims), I32, I32]),
    "ark_prefill_bf16": (C.c_int, [C.POINTER(ArkModelBf16), I32, I32, P, PI32, PP, PP, P, P, P, P, P,
                                   C.c_size_t, P]),
    "ark_decode_step_bf16": (C.c_int, [C.POINTER(ArkModelBf16), I32, P, PI32, PP, PP, P, P, P, P, P,
                                       C.c_size_t, P]),
    "ark_cache_write_bf16": (C.c_int, [C.POINTER(ArkDims), I32, I32, PI32, PP, PP, P, P, P]),
    "ark_adapter_workspace_bytes": (C.c_size_t, [C.POINTER(ArkAdapter), I32, I32]),
    "ark_encoder_workspace_bytes": (C.c_size_t, [C.POINTER(ArkEncoder), I32, I32]),
    "ark_audio_encoder": (C.c_int, [C.POINTER(ArkEncoder), I32, I32, P, P, P, C.c_size_t, P]),
    "ark_audio_adapter": (C.c_int, [C.POINTER(ArkAdapter), I32, I32, P, P, P, P, C.c_size_t, P]),
    "ark_lm_head_int4": (C.c_int, [I32, P, I32, C.POINTER(ArkQLinear4), P, I32, P]),
    "ark_embed_splice": (C.c_int, [C.POINTER(ArkDims), I32, I32, P, P, P, I32, I32, P, P]),
    "ark_prefill": (C.c_int, [C.POINTER(ArkModel), I32, I32, P, PI32, PP, PP, P, P, P, P, P,
                              C.c_size_t, P]),
    "ark_decode_step": (C.c_int, [C.POINTER(ArkModel), I32, P, PI32, PP, PP, P, P, P, P, P,
                                  C.c_size_t, P]),
    "ark_masked_argmax": (C.c_int, [I32, I32, P, P, P, P]),
    "ark_cache_write": (C.c_int, [C.POINTER(ArkDims), I32, I32, PI32, PP, PP, P, P, P]),
    "ark_greedy_decode": (C.c_int, [C.POINTER(ArkModel), I32, P, PI32, PP, PP, P, P, P, P, I32,
                                    I32, I32, P, P, C.c_size_t, P]),
    "ark_test_dynquant": (C.c_int, [I32, I32, I32, P, P, P, P, P, C.c_size_t, P]),
    "ark_test_qlinear_workspace_bytes": (C.c_size_t, [I32, I32, I32]),
    "ark_test_qlinear": (C.c_int, [I32, I32, P, P, P, C.POINTER(ArkQLinear), P, P, I32, P,
                                   C.c_size_t, P]),
    "ark_test_dynquant_workspace_bytes": (C.c_size_t, []),
    "ark_test_layernorm": (C.c_int, [I32, I32, I32, P, P, P, C.c_double, P, P, P, P, C.c_size_t, P]),
    "ark_test_enc_attention": (C.c_int, [I32, I32, I32, P, P, P, P, P, P, P, C.c_size_t, P]),
    "ark_test_enc_attention_workspace_bytes": (C.c_size_t, [I32, I32, I32]),
    "ark_test_swiglu": (C.c_int, [C.c_int64, P, P, P, P]),
    "ark_test_gate_up_workspace_bytes": (C.c_size_t, [I32, I32, I32]),
    "ark_test_gate_up": (C.c_int, [I32, I32, P, P, P, C.POINTER(ArkQLinear), C.POINTER(ArkQLinear),
                                   P, P, P, P, C.c_size_t, P]),
    "ark_test_attention_workspace_bytes": (C.c_size_t, [I32, I32, I32, I32]),
    "ark_test_attention": (C.c_int, [I32, I32, I32, I32, I32, C.POINTER(C.c_int32), P, P, P, P, P,
                                     P, P, P, P, C.c_size_t, P]),
    "ark_profile_arm": (C.c_int, [PP, I32]),
    "ark_profile_count": (C.c_int32, []),
    "ark_dominant_kernel": (C.c_char_p, []),
    "ark_decode_trace_offset": (C.c_size_t, [C.POINTER(ArkDims)]),
    "ark_decode_check": (C.c_int, [C.POINTER(ArkModel), I32, P, C.c_size_t, P]),
    "ark_noalloc_max_bytes": (C.c_size_t, []),
    "ark_decode_step_noalloc": (C.c_int, [C.POINTER(ArkModel), I32, P, PI32, PP, PP, P, P, P, P, P]),
    "ark_decode_path": (C.c_int, [C.POINTER(ArkModel), I32]),
    "ark_dump_layout": (C.c_size_t, [C.POINTER(ArkDims), I32, I32, C.c_uint64, PSZ, PSZ, PSZ]),
    "ark_prefill_dump": (C.c_int, [C.POINTER(ArkModel), I32, I32, P, PI32, PP, PP, P, P, P, P, P,
                                   C.c_size_t, P, P, C.c_size_t, C.c_uint64]),
    "ark_decode_step_dump": (C.c_int, [C.POINTER(ArkModel), I32, P, PI32, PP, PP, P, P, P, P, P,
                                       C.c_size_t, P, P, C.c_size_t, C.c_uint64]),
}

_LIB = None


def lib() -> C.CDLL:
    """Load libark.so (built in-tree); raises if it is missing."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m speech_decoder_int8_amd.build`")
        lb = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(lb, name)
            f.restype = res
            f.argtypes = args
        _LIB = lb
    return _LIB


def status_string(status: int) -> str:
    return lib().ark_status_string(status).decode()


def _check(fn: str, status: int) -> int:
    if status < 0:
        raise ArkError(fn, status, status_string(status))
    return status


# ------------------------------------------------------------- marshalling --
def _ptr(t) -> int | None:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _ptr_array(ts) -> C.Array:
    arr = (C.c_void_p * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = t.data_ptr()
    return arr


def _pos_array(pos) -> C.Array:
    p = np.ascontiguousarray(np.asarray(pos, dtype=np.int32).reshape(-1))
    arr = (C.c_int32 * len(p))(*p.tolist())
    return arr


def dims_of(cfg) -> ArkDims:
    return ArkDims(cfg.n_layers, cfg.hidden, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim,
                   cfg.intermediate, cfg.vocab, cfg.max_total_len, cfg.rms_eps, cfg.rope_theta)


def workspace_bytes(dims: ArkDims, B: int, S: int) -> int:
    return lib().ark_workspace_bytes(C.byref(dims), B, S)


# ------------------------------------------------------------------- prep --
def prep_weight(w, stream=None):
    """fp32 [n][k] device tensor -> (codes int8 [n][k], scale fp32 [n], colsum int32 [n])."""
    import torch
    n, k = w.shape
    codes = torch.empty((n, k), dtype=torch.int8, device=w.device)
    scale = torch.empty(n, dtype=torch.float32, device=w.device)
    colsum = torch.empty(n, dtype=torch.int32, device=w.device)
    _check("ark_prep_weight", lib().ark_prep_weight(_ptr(w), n, k, _ptr(codes), _ptr(scale),
                                                     _ptr(colsum), _stream(stream)))
    return codes, scale, colsum


INT4_BLOCK = 128


def prep_weight_int4(w, stream=None):
    """fp32 [n][k] device tensor -> the int4 tier's (codes uint8 [n][k/2],
    two uint4 per byte; scale fp32 [n][k/128]; zero points uint8 [n][k/256],
    two uint4 per byte)."""
    import torch
    n, k = w.shape
    codes = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
    scale = torch.empty((n, k // INT4_BLOCK), dtype=torch.float32, device=w.device)
    zp = torch.empty((n, k // (2 * INT4_BLOCK)), dtype=torch.uint8, device=w.device)
    _check("ark_prep_weight_int4", lib().ark_prep_weight_int4(_ptr(w), n, k, _ptr(codes), _ptr(scale),
                                                               _ptr(zp), _stream(stream)))
    return codes, scale, zp


class QLinear4:
    """Device tensors of the int4 LM tier's weight and its ctypes view."""

    def __init__(self, codes, scale, zp):
        self.codes, self.scale, self.zp = codes, scale, zp

    def c(self) -> ArkQLinear4:
        n, k2 = self.codes.shape
        return ArkQLinear4(_ptr(self.codes), _ptr(self.scale), _ptr(self.zp), n, 2 * k2)


def lm_head_int4(h, W: QLinear4, logits, stream=None):
    """logits [B][n] = h [B][k] . dequant(W)^T (ark_lm_head_int4)."""
    B, k = h.shape
    c = W.c()
    _check("ark_lm_head_int4", lib().ark_lm_head_int4(B, _ptr(h), h.stride(0), C.byref(c), _ptr(logits),
                                                       logits.stride(0), _stream(stream)))


def rope_table(T: int, head_dim: int, theta: float, device="cuda", stream=None):
    import torch
    c = torch.empty((T, head_dim // 2), dtype=torch.float64, device=device)
    s = torch.empty((T, head_dim // 2), dtype=torch.float64, device=device)
    _check("ark_rope_table", lib().ark_rope_table(T, head_dim, theta, _ptr(c), _ptr(s), _stream(stream)))
    return c, s


class QLinear:
    """Device tensors of one prepared projection and its ctypes view."""

    def __init__(self, codes, scale, colsum, bias=None):
        self.codes, self.scale, self.colsum, self.bias = codes, scale, colsum, bias

    @classmethod
    def from_f32(cls, w_f32, bias=None, stream=None):
        return cls(*prep_weight(w_f32, stream), bias)

    def c(self) -> ArkQLinear:
        n, k = self.codes.shape
        return ArkQLinear(_ptr(self.codes), _ptr(self.scale), _ptr(self.colsum), _ptr(self.bias), n, k)


class DeviceModel:
    """A prepared decoder on the GPU: int8 weights, gains, rope tables,
    embedding table, plus the ark_model struct that points at them."""

    def __init__(self, cfg, layers, final_norm, lm_head, embed_f16, rope_cos, rope_sin,
                 lm_head4=None):
        self.cfg = cfg
        self.layers = layers              # list of dicts of QLinear / tensors
        self.final_norm = final_norm
        self.lm_head = lm_head            # QLinear or None
        self.lm_head4 = lm_head4          # QLinear4 or None (the int4 tier)
        self.embed_f16 = embed_f16        # int16 tensor (fp16 bits) or None
        self.rope_cos, self.rope_sin = rope_cos, rope_sin
        self.dims = dims_of(cfg)
        self._layer_arr = (ArkLayer * cfg.n_layers)()
        for i, L in enumerate(layers):
            self._layer_arr[i] = ArkLayer(_ptr(L["ln1"]), _ptr(L["ln2"]), L["q"].c(), L["k"].c(),
                                          L["v"].c(), L["o"].c(), L["gate"].c(), L["up"].c(),
                                          L["down"].c())
        self.c = ArkModel(self.dims, self._layer_arr, _ptr(final_norm),
                          lm_head.c() if lm_head is not None else ArkQLinear(),
                          _ptr(embed_f16), _ptr(rope_cos), _ptr(rope_sin),
                          lm_head4.c() if lm_head4 is not None else ArkQLinear4())

    def with_max_total_len(self, T: int) -> "DeviceModel":
        """The same weights with a static cache of T rows (new rotary tables)."""
        cfg = self.cfg.with_(max_total_len=T)
        rc, rs = rope_table(T, cfg.head_dim, cfg.rope_theta, self.rope_cos.device)
        return DeviceModel(cfg, self.layers, self.final_norm, self.lm_head, self.embed_f16, rc, rs,
                           self.lm_head4)

    def view(self, layers=None) -> "DeviceModel":
        """The same weights restricted to some layers (no LM head)."""
        idx = list(range(self.cfg.n_layers)) if layers is None else list(layers)
        sub = DeviceModel.__new__(DeviceModel)
        sub.__dict__.update(self.__dict__)
        sub.cfg = self.cfg.with_(n_layers=len(idx))
        sub.layers = [self.layers[i] for i in idx]
        sub.dims = dims_of(sub.cfg)
        sub._layer_arr = (ArkLayer * len(idx))(*[self._layer_arr[i] for i in idx])
        sub.c = ArkModel(sub.dims, sub._layer_arr, None, ArkQLinear(), _ptr(self.embed_f16),
                         _ptr(self.rope_cos), _ptr(self.rope_sin))
        sub.lm_head = None
        sub.lm_head4 = None
        return sub

    def with_lm_head(self, lm_head=None, lm_head4=None) -> "DeviceModel":
        """The same layers with another LM head (an int8 QLinear, an int4
        QLinear4, or neither)."""
        return DeviceModel(self.cfg, self.layers, self.final_norm, lm_head, self.embed_f16,
                           self.rope_cos, self.rope_sin, lm_head4)


def load_lm_head_int4(cfg, synth, device="cuda", stream=None) -> QLinear4:
    """The seeded fp32 LM-head rows prepared into the int4 tier on the GPU
    (ark_prep_weight_int4), a slice of rows at a time."""
    import torch
    H = cfg.hidden
    codes = torch.empty((cfg.vocab, H // 2), dtype=torch.uint8, device=device)
    scale = torch.empty((cfg.vocab, H // INT4_BLOCK), dtype=torch.float32, device=device)
    zp = torch.empty((cfg.vocab, H // (2 * INT4_BLOCK)), dtype=torch.uint8, device=device)
    step = 16 * synth.ROW_CHUNK
    for r0 in range(0, cfg.vocab, step):
        r1 = min(cfg.vocab, r0 + step)
        wt = torch.from_numpy(np.ascontiguousarray(synth.lm_head_rows(cfg, r0, r1))).to(device)
        c, s, z = prep_weight_int4(wt, stream)
        codes[r0:r1].copy_(c)
        scale[r0:r1].copy_(s)
        zp[r0:r1].copy_(z)
        del wt, c, s, z
    return QLinear4(codes, scale, zp)


def load_model(cfg, synth, device="cuda", stream=None, layers=None,
               lm_head4: bool = False) -> DeviceModel:
    """Upload the seeded fp32 weights of `cfg` layer by layer and prepare them
    on the GPU (ark_prep_weight); the fp32 copies are released as it goes.
    lm_head4: prepare the LM head as the weight-only int4 tier instead of
    int8."""
    import torch

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    out = []
    for l in (range(cfg.n_layers) if layers is None else layers):
        w = synth.layer_weights(cfg, l)
        L = {"ln1": up(w["ln1"]), "ln2": up(w["ln2"])}
        for name, key, bias in (("q", "wq", "bq"), ("k", "wk", "bk"), ("v", "wv", "bv"),
                                ("o", "wo", None), ("gate", "wg", None), ("up", "wu", None),
                                ("down", "wd", None)):
            wt = up(w[key])
            L[name] = QLinear.from_f32(wt, up(w[bias]) if bias else None, stream)
            del wt
        out.append(L)
        del w
    final_norm, lm, lm4 = None, None, None
    if cfg.lm_head and lm_head4:
        final_norm = up(synth.final_norm(cfg))
        lm4 = load_lm_head_int4(cfg, synth, device, stream)
    elif cfg.lm_head:
        final_norm = up(synth.final_norm(cfg))
        codes = torch.empty((cfg.vocab, cfg.hidden), dtype=torch.int8, device=device)
        scale = torch.empty(cfg.vocab, dtype=torch.float32, device=device)
        colsum = torch.empty(cfg.vocab, dtype=torch.int32, device=device)
        step = 16 * synth.ROW_CHUNK
        for r0 in range(0, cfg.vocab, step):
            r1 = min(cfg.vocab, r0 + step)
            wt = up(synth.lm_head_rows(cfg, r0, r1))
            c, s, cs = prep_weight(wt, stream)
            codes[r0:r1].copy_(c)
            scale[r0:r1].copy_(s)
            colsum[r0:r1].copy_(cs)
            del wt, c, s, cs
        lm = QLinear(codes, scale, colsum)
    emb = up(synth.embed_table_f16(cfg).view(np.int16))
    rc, rs = rope_table(cfg.max_total_len, cfg.head_dim, cfg.rope_theta, device, stream)
    torch.cuda.current_stream().synchronize()
    return DeviceModel(cfg, out, final_norm, lm, emb, rc, rs, lm4)


# ----------------------------------------------------------- the adapter --
class DeviceAdapter:
    """The prepared audio adapter on the GPU and its ark_adapter struct."""

    def __init__(self, up: QLinear, down: QLinear, frame_dim: int, merge: int):
        self.up, self.down, self.frame_dim, self.merge = up, down, frame_dim, merge
        self.c = ArkAdapter(up.c(), down.c(), frame_dim, merge)

    def workspace(self, B: int, frames: int):
        import torch
        n = lib().ark_adapter_workspace_bytes(C.byref(self.c), B, frames)
        if n == 0:
            raise ArkError("ark_adapter_workspace_bytes", ARK_E_SHAPE, "invalid adapter call")
        return torch.empty(n, dtype=torch.uint8, device="cuda")


def load_adapter(cfg, synth, device="cuda", stream=None) -> DeviceAdapter:
    """The seeded fp32 adapter weights of `cfg`, prepared on the GPU."""
    import torch
    w = synth.adapter_weights(cfg)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)
    ad = DeviceAdapter(QLinear.from_f32(up(w["w1"]), up(w["b1"]), stream),
                       QLinear.from_f32(up(w["w2"]), up(w["b2"]), stream), cfg.frame_dim, cfg.merge)
    torch.cuda.current_stream().synchronize()
    return ad


def audio_adapter(ad: DeviceAdapter, enc, out, mid=None, ws=None, stream=None):
    """enc [B][frames][frame_dim] -> out [B][frames // merge][hidden]
    (ark_audio_adapter); mid: optional [B][frames // merge][inner]."""
    B, frames = enc.shape[0], enc.shape[1]
    if ws is None:
        ws = ad.workspace(B, frames)
    _check("ark_audio_adapter", lib().ark_audio_adapter(
        C.byref(ad.c), B, frames, _ptr(enc), _ptr(out), _ptr(mid), _ptr(ws), ws.numel(),
        _stream(stream)))


# ------------------------------------------------------------ the encoder --
class DeviceEncoder:
    """The prepared audio encoder on the GPU and its ark_encoder struct."""

    def __init__(self, cfg, conv1, conv2, pos, layers, lnf, rope):
        self.cfg = cfg
        self.conv1, self.conv2, self.pos, self.layers, self.lnf = conv1, conv2, pos, layers, lnf
        self.rope_cos, self.rope_sin = rope
        self._arr = (ArkEncLayer * len(layers))()
        for i, L in enumerate(layers):
            self._arr[i] = ArkEncLayer(_ptr(L["ln1_g"]), _ptr(L["ln1_b"]), _ptr(L["ln2_g"]),
                                       _ptr(L["ln2_b"]), L["q"].c(), L["k"].c(), L["v"].c(),
                                       L["o"].c(), L["fc1"].c(), L["fc2"].c())
        self.c = ArkEncoder(cfg.n_mels, cfg.enc_dim, cfg.enc_heads, cfg.enc_ffn, len(layers),
                            cfg.enc_max_pos, cfg.enc_ln_eps, conv1.c(), conv2.c(), _ptr(pos), self._arr,
                            _ptr(lnf[0]), _ptr(lnf[1]), _ptr(self.rope_cos), _ptr(self.rope_sin))

    def workspace(self, B: int, mel_frames: int):
        import torch
        n = lib().ark_encoder_workspace_bytes(C.byref(self.c), B, mel_frames)
        if n == 0:
            raise ArkError("ark_encoder_workspace_bytes", ARK_E_SHAPE, "invalid encoder call")
        return torch.empty(n, dtype=torch.uint8, device="cuda")


def load_encoder(cfg, synth, device="cuda", stream=None, layers=None) -> DeviceEncoder:
    """The seeded fp32 encoder weights of `cfg` (convolutions tap-major),
    prepared on the GPU layer by layer; `layers` limits the stack."""
    import torch

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)
    fr = synth.encoder_front(cfg)
    conv1 = QLinear.from_f32(up(fr["conv1"]), up(fr["conv1_b"]), stream)
    conv2 = QLinear.from_f32(up(fr["conv2"]), up(fr["conv2_b"]), stream)
    out = []
    for l in (range(cfg.enc_layers) if layers is None else layers):
        w = synth.encoder_layer_weights(cfg, l)
        L = {n: up(w[n]) for n in ("ln1_g", "ln1_b", "ln2_g", "ln2_b")}
        for name, key, bias in (("q", "wq", "bq"), ("k", "wk", None), ("v", "wv", "bv"),
                                ("o", "wo", "bo"), ("fc1", "w1", "b1"), ("fc2", "w2", "b2")):
            L[name] = QLinear.from_f32(up(w[key]), up(w[bias]) if bias else None, stream)
        out.append(L)
        del w
    rope = rope_table(cfg.enc_max_pos, cfg.enc_dim // cfg.enc_heads, cfg.enc_rope_theta, device, stream)
    enc = DeviceEncoder(cfg, conv1, conv2, up(fr["pos"]), out, (up(fr["lnf_g"]), up(fr["lnf_b"])),
                        rope)
    torch.cuda.current_stream().synchronize()
    return enc


def audio_encoder(enc: DeviceEncoder, mel, out, ws=None, stream=None):
    """mel [B][M][n_mels] -> out [B][(M - 1) // 2 + 1][d] (ark_audio_encoder)."""
    B, M = mel.shape[0], mel.shape[1]
    if ws is None:
        ws = enc.workspace(B, M)
    _check("ark_audio_encoder", lib().ark_audio_encoder(
        C.byref(enc.c), B, M, _ptr(mel), _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))


# ------------------------------------------------------ the bf16 variant --
def to_bf16(x, stream=None):
    """fp32 device tensor -> torch.bfloat16 tensor of the same shape (ark_to_bf16)."""
    import torch
    out = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)
    _check("ark_to_bf16", lib().ark_to_bf16(_ptr(x), x.numel(), _ptr(out), _stream(stream)))
    return out


class DeviceModelBf16:
    """The decoder's weights in bf16 on the GPU and its ark_model_bf16 struct."""

    def __init__(self, cfg, layers, final_norm, lm_head, embed, rope_cos, rope_sin):
        self.cfg = cfg
        self.layers, self.final_norm, self.lm_head, self.embed = layers, final_norm, lm_head, embed
        self.rope_cos, self.rope_sin = rope_cos, rope_sin
        self.dims = dims_of(cfg)

        def lin(w, b=None):
            return ArkLinearBf16(_ptr(w), _ptr(b), w.shape[0], w.shape[1])
        self._arr = (ArkLayerBf16 * len(layers))()
        for i, L in enumerate(layers):
            self._arr[i] = ArkLayerBf16(_ptr(L["ln1"]), _ptr(L["ln2"]), lin(L["wq"], L["bq"]),
                                        lin(L["wk"], L["bk"]), lin(L["wv"], L["bv"]), lin(L["wo"]),
                                        lin(L["wg"]), lin(L["wu"]), lin(L["wd"]))
        self.c = ArkModelBf16(self.dims, self._arr, _ptr(final_norm),
                              lin(lm_head) if lm_head is not None else ArkLinearBf16(),
                              _ptr(embed), _ptr(rope_cos), _ptr(rope_sin))

    def workspace(self, B: int, S: int):
        import torch
        n = lib().ark_workspace_bytes_bf16(C.byref(self.dims), B, S)
        if n == 0:
            raise ArkError("ark_workspace_bytes_bf16", ARK_E_SHAPE, "invalid dims")
        return torch.empty(n, dtype=torch.uint8, device="cuda")


def load_model_bf16(cfg, synth, device="cuda", stream=None) -> DeviceModelBf16:
    """The seeded fp32 weights of `cfg` converted to bf16 on the GPU."""
    import torch

    def bf(a):
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
        return to_bf16(t, stream)
    layers = []
    for l in range(cfg.n_layers):
        w = synth.layer_weights(cfg, l)
        layers.append({k: bf(v) for k, v in w.items()})
        del w
    final_norm = lm = None
    if cfg.lm_head:
        final_norm = bf(synth.final_norm(cfg))
        lm = torch.empty((cfg.vocab, cfg.hidden), dtype=torch.bfloat16, device=device)
        step = 16 * synth.ROW_CHUNK
        for r0 in range(0, cfg.vocab, step):
            r1 = min(cfg.vocab, r0 + step)
            lm[r0:r1].copy_(bf(synth.lm_head_rows(cfg, r0, r1)))
    emb = bf(synth.embed_table_f16(cfg).astype(np.float32))
    rc, rs = rope_table(cfg.max_total_len, cfg.head_dim, cfg.rope_theta, device, stream)
    torch.cuda.current_stream().synchronize()
    return DeviceModelBf16(cfg, layers, final_norm, lm, emb, rc, rs)


def prefill_bf16(model: DeviceModelBf16, embeds, cache_position, k_cache, v_cache, k_delta,
                 v_delta, logits=None, hidden_out=None, ws=None, stream=None):
    B, S = embeds.shape[0], embeds.shape[1]
    if ws is None:
        ws = model.workspace(B, S)
    _check("ark_prefill_bf16", lib().ark_prefill_bf16(
        C.byref(model.c), B, S, _ptr(embeds), _pos_array(cache_position), _ptr_array(k_cache),
        _ptr_array(v_cache), _ptr(k_delta), _ptr(v_delta), _ptr(logits), _ptr(hidden_out),
        _ptr(ws), ws.numel(), _stream(stream)))


def decode_step_bf16(model: DeviceModelBf16, token_ids, cache_position, k_cache, v_cache, k_delta,
                     v_delta, logits=None, hidden_out=None, ws=None, stream=None):
    B = token_ids.shape[0]
    if ws is None:
        ws = model.workspace(B, 1)
    _check("ark_decode_step_bf16", lib().ark_decode_step_bf16(
        C.byref(model.c), B, _ptr(token_ids), _pos_array(cache_position), _ptr_array(k_cache),
        _ptr_array(v_cache), _ptr(k_delta), _ptr(v_delta), _ptr(logits), _ptr(hidden_out),
        _ptr(ws), ws.numel(), _stream(stream)))


def cache_write_bf16(dims: ArkDims, cache_position, k_cache, v_cache, k_delta, v_delta, stream=None):
    B, S = k_delta.shape[1], k_delta.shape[2]
    _check("ark_cache_write_bf16", lib().ark_cache_write_bf16(
        C.byref(dims), B, S, _pos_array(cache_position), _ptr_array(k_cache), _ptr_array(v_cache),
        _ptr(k_delta), _ptr(v_delta), _stream(stream)))


# ------------------------------------------------------------- the path --
def workspace(model: DeviceModel, B: int, S: int):
    import torch
    n = workspace_bytes(model.dims, B, S)
    if n == 0:
        raise ArkError("ark_workspace_bytes", ARK_E_SHAPE, "invalid dims")
    return torch.empty(n, dtype=torch.uint8, device="cuda")


def embed_splice(dims: ArkDims, ids, table_f16, audio, a0: int, out, stream=None):
    B, S = ids.shape
    N = 0 if audio is None else audio.shape[1]
    _check("ark_embed_splice", lib().ark_embed_splice(C.byref(dims), B, S, _ptr(ids), _ptr(table_f16),
                                                       _ptr(audio), a0, N, _ptr(out), _stream(stream)))
    return out


def prefill(model: DeviceModel, embeds, cache_position, k_cache, v_cache, k_delta, v_delta,
            logits=None, hidden_out=None, ws=None, stream=None):
    B, S = embeds.shape[0], embeds.shape[1]
    if ws is None:
        ws = workspace(model, B, S)
    _check("ark_prefill", lib().ark_prefill(
        C.byref(model.c), B, S, _ptr(embeds), _pos_array(cache_position), _ptr_array(k_cache),
        _ptr_array(v_cache), _ptr(k_delta), _ptr(v_delta), _ptr(logits), _ptr(hidden_out),
        _ptr(ws), ws.numel(), _stream(stream)))


def decode_step(model: DeviceModel, token_ids, cache_position, k_cache, v_cache, k_delta, v_delta,
                logits=None, hidden_out=None, ws=None, stream=None):
    B = token_ids.shape[0]
    if ws is None:
        ws = workspace(model, B, 1)
    _check("ark_decode_step", lib().ark_decode_step(
        C.byref(model.c), B, _ptr(token_ids), _pos_array(cache_position), _ptr_array(k_cache),
        _ptr_array(v_cache), _ptr(k_delta), _ptr(v_delta), _ptr(logits), _ptr(hidden_out),
        _ptr(ws), ws.numel(), _stream(stream)))


def decode_step_noalloc(model: DeviceModel, token_ids, cache_position, k_cache, v_cache, k_delta,
                        v_delta, logits=None, hidden_out=None, stream=None):
    """ark_decode_step on the library's static scratch (no workspace)."""
    B = token_ids.shape[0]
    _check("ark_decode_step_noalloc", lib().ark_decode_step_noalloc(
        C.byref(model.c), B, _ptr(token_ids), _pos_array(cache_position), _ptr_array(k_cache),
        _ptr_array(v_cache), _ptr(k_delta), _ptr(v_delta), _ptr(logits), _ptr(hidden_out),
        _stream(stream)))


def decode_check(model: DeviceModel, B: int, ws, stream=None) -> int:
    """Status of the last decode step on ws (synchronises the stream):
    ARK_OK or ARK_E_TIMEOUT; raises on other errors."""
    st = lib().ark_decode_check(C.byref(model.c), B, _ptr(ws), ws.numel(), _stream(stream))
    if st not in (ARK_OK, ARK_E_TIMEOUT):
        _check("ark_decode_check", st)
    return st


def decode_path(model: DeviceModel, B: int) -> int:
    """1: the persistent batch-1 kernel serves B sequences; 0: the multi-kernel path."""
    return _check("ark_decode_path", lib().ark_decode_path(C.byref(model.c), B))


class DumpRecord:
    """Device buffer of a re-anchored parity record and its layout
    (ark_dump_layout); read() copies it to host numpy arrays."""

    def __init__(self, model: DeviceModel, B: int, S: int, layers):
        import torch
        self.model, self.B, self.S = model, B, S
        self.layers = sorted(set(int(l) for l in layers))
        self.mask = 0
        for l in self.layers:
            self.mask |= 1 << l
        f = (C.c_size_t * 13)()
        rec = C.c_size_t()
        head = (C.c_size_t * 4)()
        self.nbytes = lib().ark_dump_layout(C.byref(model.dims), B, S, C.c_uint64(self.mask), f,
                                            C.byref(rec), head)
        if self.nbytes == 0:
            raise ArkError("ark_dump_layout", ARK_E_SHAPE, "invalid dims")
        self.field_off, self.rec, self.head_off = list(f), rec.value, list(head)
        self.buf = torch.zeros(self.nbytes, dtype=torch.uint8, device="cuda")

    def read(self):
        """{layer: {field: array}} and the head record {hn, hc, s, z}; codes
        as uint8 (code - 128 stored, 128 added back)."""
        import torch
        torch.cuda.synchronize()
        raw = self.buf.cpu().numpy()
        cfg = self.model.cfg
        B, R = self.B, self.B * self.S
        H, Q = cfg.hidden, cfg.n_heads * cfg.head_dim
        KV, I = cfg.n_kv_heads * cfg.head_dim, cfg.intermediate
        shapes = {"h1": (R, H), "qkv": (R, Q + 2 * KV), "attn": (R, Q), "x1": (R, H), "h2": (R, H),
                  "a": (R, I), "x2": (R, H), "c1": (R, H), "c2": (R, Q), "c3": (R, H), "c4": (R, I),
                  "s": (4, B), "z": (4, B)}
        out = {}
        for i, l in enumerate(self.layers):
            base = i * self.rec
            d = {}
            for k, name in enumerate(DUMP_FIELDS):
                shp = shapes[name]
                n = int(np.prod(shp))
                o = base + self.field_off[k]
                if name[0] == "c":
                    d[name] = (raw[o:o + n].view(np.int8).astype(np.int16) + 128).astype(np.uint8).reshape(shp)
                elif name == "z":
                    d[name] = raw[o:o + 4 * n].view(np.int32).reshape(shp).copy()
                else:
                    d[name] = raw[o:o + 4 * n].view(np.float32).reshape(shp).copy()
            out[l] = d
        ho = self.head_off
        head = {"hn": raw[ho[0]:ho[0] + 4 * B * H].view(np.float32).reshape(B, H).copy(),
                "hc": (raw[ho[1]:ho[1] + B * H].view(np.int8).astype(np.int16) + 128).astype(np.uint8).reshape(B, H),
                "s": raw[ho[2]:ho[2] + 4 * B].view(np.float32).copy(),
                "z": raw[ho[3]:ho[3] + 4 * B].view(np.int32).copy()}
        return out, head


def prefill_dump(model: DeviceModel, embeds, cache_position, k_cache, v_cache, k_delta, v_delta,
                 rec: DumpRecord, logits=None, hidden_out=None, ws=None, stream=None):
    B, S = embeds.shape[0], embeds.shape[1]
    if ws is None:
        ws = workspace(model, B, S)
    _check("ark_prefill_dump", lib().ark_prefill_dump(
        C.byref(model.c), B, S, _ptr(embeds), _pos_array(cache_position), _ptr_array(k_cache),
        _ptr_array(v_cache), _ptr(k_delta), _ptr(v_delta), _ptr(logits), _ptr(hidden_out),
        _ptr(ws), ws.numel(), _stream(stream), _ptr(rec.buf), rec.nbytes, C.c_uint64(rec.mask)))


def decode_step_dump(model: DeviceModel, token_ids, cache_position, k_cache, v_cache, k_delta,
                     v_delta, rec: DumpRecord, logits=None, hidden_out=None, ws=None, stream=None):
    B = token_ids.shape[0]
    if ws is None:
        ws = workspace(model, B, 1)
    _check("ark_decode_step_dump", lib().ark_decode_step_dump(
        C.byref(model.c), B, _ptr(token_ids), _pos_array(cache_position), _ptr_array(k_cache),
        _ptr_array(v_cache), _ptr(k_delta), _ptr(v_delta), _ptr(logits), _ptr(hidden_out),
        _ptr(ws), ws.numel(), _stream(stream), _ptr(rec.buf), rec.nbytes, C.c_uint64(rec.mask)))


def masked_argmax(logits, mask, out_ids, stream=None):
    B, V = logits.shape
    _check("ark_masked_argmax", lib().ark_masked_argmax(B, V, _ptr(logits), _ptr(mask), _ptr(out_ids),
                                                         _stream(stream)))
    return out_ids


def cache_write(dims: ArkDims, cache_position, k_cache, v_cache, k_delta, v_delta, stream=None):
    B, S = k_delta.shape[1], k_delta.shape[2]
    _check("ark_cache_write", lib().ark_cache_write(
        C.byref(dims), B, S, _pos_array(cache_position), _ptr_array(k_cache), _ptr_array(v_cache),
        _ptr(k_delta), _ptr(v_delta), _stream(stream)))


def greedy_decode(model: DeviceModel, token_ids, cache_position, k_cache, v_cache, k_delta,
                  v_delta, logits, mask, end_id: int, max_steps: int, out_tokens, ws=None,
                  check_every: int = 1, stream=None):
    """Runs the native greedy loop; returns (steps, new cache positions)."""
    B = token_ids.shape[0]
    if ws is None:
        ws = workspace(model, B, 1)
    pos = _pos_array(cache_position)
    n = _check("ark_greedy_decode", lib().ark_greedy_decode(
        C.byref(model.c), B, _ptr(token_ids), pos, _ptr_array(k_cache), _ptr_array(v_cache),
        _ptr(k_delta), _ptr(v_delta), _ptr(logits), _ptr(mask), end_id, max_steps, check_every,
        _ptr(out_tokens), _ptr(ws), ws.numel(), _stream(stream)))
    return n, np.array(pos[:], dtype=np.int32)


def test_dynquant(x, stream=None):
    """x [B][R][K] fp32 -> (codes uint8, scale [B], zp [B]) via the prefill kernels."""
    import torch
    B, R, K = x.shape
    codes = torch.empty((B, R, K), dtype=torch.uint8, device=x.device)
    scale = torch.empty(B, dtype=torch.float32, device=x.device)
    zp = torch.empty(B, dtype=torch.int32, device=x.device)
    ws = torch.empty(lib().ark_test_dynquant_workspace_bytes(), dtype=torch.uint8, device=x.device)
    _check("ark_test_dynquant", lib().ark_test_dynquant(B, R, K, _ptr(x), _ptr(codes), _ptr(scale),
                                                         _ptr(zp), _ptr(ws), ws.numel(), _stream(stream)))
    return codes, scale, zp


def test_qlinear(codes, scale, zp, W: QLinear, use_gemm, stream=None):
    """codes [B][R][k] uint8, scale [B], zp [B] uint8 -> (acc int32, y fp32) [B*R][n].
    use_gemm: 0 decode GEMV, 1 GEMM as dispatched by the decoder, 2 tiled GEMM."""
    import torch
    B, R, k = codes.shape
    n = W.codes.shape[0]
    acc = torch.empty((B * R, n), dtype=torch.int32, device=codes.device)
    y = torch.empty((B * R, n), dtype=torch.float32, device=codes.device)
    nbytes = lib().ark_test_qlinear_workspace_bytes(B * R, k, int(use_gemm))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=codes.device)
    wc = W.c()
    _check("ark_test_qlinear", lib().ark_test_qlinear(B, R, _ptr(codes), _ptr(scale), _ptr(zp), C.byref(wc),
                                                       _ptr(acc), _ptr(y), int(use_gemm), _ptr(ws),
                                                       ws.numel(), _stream(stream)))
    return acc, y


def _stats_ws():
    import torch
    return torch.empty(lib().ark_test_dynquant_workspace_bytes(), dtype=torch.uint8, device="cuda")


def test_layernorm(x, g, b, eps, stream=None):
    """x [B][S][D] -> (y [B][S][D], lo [B], hi [B]) (ark_test_layernorm)."""
    import torch
    B, S, D = x.shape
    y = torch.empty_like(x)
    lo = torch.empty(B, dtype=torch.float32, device=x.device)
    hi = torch.empty_like(lo)
    ws = _stats_ws()
    _check("ark_test_layernorm", lib().ark_test_layernorm(B, S, D, _ptr(x), _ptr(g), _ptr(b), eps,
                                                           _ptr(y), _ptr(lo), _ptr(hi), _ptr(ws),
                                                           ws.numel(), _stream(stream)))
    return y, lo, hi


def test_enc_attention(qkv, H, cos, sin, stream=None):
    """qkv [B][F][3 H 64] -> (out [B][F][H 64], lo [B], hi [B])."""
    import torch
    B, F = qkv.shape[0], qkv.shape[1]
    out = torch.empty((B, F, H * 64), dtype=torch.float32, device=qkv.device)
    lo = torch.empty(B, dtype=torch.float32, device=qkv.device)
    hi = torch.empty_like(lo)
    ws = torch.empty(lib().ark_test_enc_attention_workspace_bytes(B, F, H), dtype=torch.uint8,
                     device=qkv.device)
    _check("ark_test_enc_attention", lib().ark_test_enc_attention(
        B, F, H, _ptr(qkv), _ptr(cos), _ptr(sin), _ptr(out), _ptr(lo), _ptr(hi), _ptr(ws),
        ws.numel(), _stream(stream)))
    return out, lo, hi


def test_swiglu(g, u, stream=None):
    """g, u fp32 device tensors of one shape -> silu(g) * u as the GEMM
    epilogues compute it (fp64 inside, fp32 out)."""
    import torch
    g = g.contiguous()
    u = u.contiguous()
    assert g.shape == u.shape and g.dtype == u.dtype == torch.float32
    y = torch.empty_like(g)
    _check("ark_test_swiglu", lib().ark_test_swiglu(g.numel(), _ptr(g), _ptr(u), _ptr(y),
                                                     _stream(stream)))
    return y


def test_gate_up(codes, scale, zp, gate: QLinear, up: QLinear, stream=None):
    """codes [B][R][k] uint8, scale [B], zp [B] uint8 -> (y [B*R][n] fp32 =
    silu(gate) * up, seq_min [B], seq_max [B] of y) as the prefill computes them."""
    import torch
    B, R, k = codes.shape
    n = gate.codes.shape[0]
    y = torch.empty((B * R, n), dtype=torch.float32, device=codes.device)
    lo = torch.empty(B, dtype=torch.float32, device=codes.device)
    hi = torch.empty(B, dtype=torch.float32, device=codes.device)
    ws = torch.empty(lib().ark_test_gate_up_workspace_bytes(B, R, k), dtype=torch.uint8,
                     device=codes.device)
    gc, uc = gate.c(), up.c()
    _check("ark_test_gate_up", lib().ark_test_gate_up(B, R, _ptr(codes), _ptr(scale), _ptr(zp),
                                                       C.byref(gc), C.byref(uc), _ptr(y), _ptr(lo),
                                                       _ptr(hi), _ptr(ws), ws.numel(),
                                                       _stream(stream)))
    return y, lo, hi


def test_attention(q, k_cache, v_cache, k_delta, v_delta, pos, n_kv_heads: int, stream=None):
    """q [B][S][NH*128]; caches [B][T][NKV][128]; deltas [B][S][NKV][128];
    pos: B host ints -> (out [B*S][NH*128], seq_min [B], seq_max [B])."""
    import torch
    B, S, QD = q.shape
    NH = QD // 128
    T = k_cache.shape[1]
    out = torch.empty((B * S, QD), dtype=torch.float32, device=q.device)
    lo = torch.empty(B, dtype=torch.float32, device=q.device)
    hi = torch.empty(B, dtype=torch.float32, device=q.device)
    ws = torch.empty(lib().ark_test_attention_workspace_bytes(B, S, NH, T), dtype=torch.uint8,
                     device=q.device)
    p = (C.c_int32 * B)(*[int(v) for v in pos])
    _check("ark_test_attention", lib().ark_test_attention(B, S, NH, n_kv_heads, T, p, _ptr(q),
                                                           _ptr(k_cache), _ptr(v_cache),
                                                           _ptr(k_delta), _ptr(v_delta), _ptr(out),
                                                           _ptr(lo), _ptr(hi), _ptr(ws), ws.numel(),
                                                           _stream(stream)))
    return out, lo, hi


# ------------------------------------------------------- instrumentation --
class HipEvents:
    """n pairs of timing hipEvents (created through the HIP runtime) armed
    around the library's dominant decode kernel (ark_profile_arm)."""

    def __init__(self, n_pairs: int):
        self.hip = C.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.hip.hipEventDestroy.argtypes = [C.c_void_p]
        self.n = n_pairs
        self.arr = (C.c_void_p * (2 * n_pairs))()
        for i in range(2 * n_pairs):
            ev = C.c_void_p()
            if self.hip.hipEventCreate(C.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.arr[i] = ev.value

    def arm(self):
        _check("ark_profile_arm", lib().ark_profile_arm(self.arr, self.n))

    @staticmethod
    def disarm():
        lib().ark_profile_arm(None, 0)

    def durations_ms(self):
        """Elapsed ms of every recorded pair (call after synchronising)."""
        k = lib().ark_profile_count()
        out = []
        for i in range(k):
            ms = C.c_float()
            if self.hip.hipEventElapsedTime(C.byref(ms), self.arr[2 * i], self.arr[2 * i + 1]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out.append(ms.value)
        return out

    def close(self):
        for i in range(2 * self.n):
            self.hip.hipEventDestroy(self.arr[i])


def dominant_kernel() -> str:
    return lib().ark_dominant_kernel().decode()


def decode_trace(model: DeviceModel, ws):
    """Phase timestamps of the last traced decode step (ARK_MEGA_TRACE=1):
    numpy uint64 [3][n_layers + 1][32] (workgroups 0, 1 and 255, every
    layer) and [256][16] (every workgroup, one layer) read from the workspace."""
    import torch
    off = lib().ark_decode_trace_offset(C.byref(model.dims))
    n1 = 3 * (model.cfg.n_layers + 1) * 32
    n = n1 + 256 * 16
    torch.cuda.synchronize()
    raw = ws[off:off + n * 8].cpu().numpy().view(np.uint64)
    return raw[:n1].reshape(3, model.cfg.n_layers + 1, 32), raw[n1:].reshape(256, 16)
