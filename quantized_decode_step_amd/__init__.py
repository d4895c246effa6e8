"""Python binding of libocrdec (the decode step of an OCR vision-language
decoder on MI355X / gfx950).

This module only marshals arguments: every step of the decode path runs in the
HIP kernels of ``libocrdec.so``.  PyTorch supplies device memory and streams.
Importing the module fails loudly if the library has not been built
(``python quantized_decode_step_amd/build.py``); there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libocrdec.so")

OCRDEC_OK, OCRDEC_ERR_INVALID_ARG, OCRDEC_ERR_UNSUPPORTED, OCRDEC_ERR_WORKSPACE, OCRDEC_ERR_DEVICE = range(5)
OCRDEC_F16, OCRDEC_Q8_0, OCRDEC_Q4_0, OCRDEC_U8A_G32 = range(4)
OCRDEC_OUT_F32, OCRDEC_OUT_F16 = 0, 1
OCRDEC_DEV_TOKEN_RANGE, OCRDEC_DEV_RESIDUAL, OCRDEC_DEV_LOGIT, OCRDEC_DEV_NO_TOKEN = 1, 2, 4, 8
# ocrdec_kernel
KERNEL_NAMES = ["embed", "qkv", "attn", "attn_merge", "attn_merge_o", "o_proj", "norm", "route", "expert_glu",
                "expert_down", "combine", "dense_glu", "dense_down", "lm_head", "argmax", "other"]

if not os.path.exists(LIB_PATH):
    raise ImportError("libocrdec.so is not built: run `python quantized_decode_step_amd/build.py` "
                      "(hipcc --offload-arch=gfx950)")
try:
    # PyTorch-ROCm carries its own HIP runtime; loading it first makes the
    # library bind to that same runtime (one runtime per process), whatever
    # the caller imports first.
    import torch  # noqa: F401
except ImportError:
    pass
_lib = ctypes.CDLL(LIB_PATH)

_vp, _i32, _i64, _sz, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float


class OcrdecError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("libocrdec status %d: %s" % (status, msg))
        self.status = status


def _check(status: int):
    if status != OCRDEC_OK:
        raise OcrdecError(status, ocrdec_last_error())


# ----------------------------------------------------------------------------
# ABI structs (mirror include/ocrdec.h)
# ----------------------------------------------------------------------------

class QMatDesc(ctypes.Structure):
    _fields_ = [("fmt", _i32), ("n", _i32), ("k", _i32), ("data", _vp)]


class AttnArgs(ctypes.Structure):
    _fields_ = [("rows", _i32), ("n_heads", _i32), ("head_dim", _i32), ("qkv", _vp), ("ld_qkv", _i64),
                ("k_cache", _vp), ("v_cache", _vp), ("prefix_cap", _i32), ("ring_cap", _i32),
                ("prefix_len", _vp), ("gen_index", _vp), ("sink", _vp), ("rope_theta", _f32), ("scale", _f32),
                ("out", _vp), ("ld_out", _i64), ("k_scale", _vp), ("v_scale", _vp)]


class MoeWeights(ctypes.Structure):
    _fields_ = [("hidden", _i32), ("n_experts", _i32), ("top_k", _i32), ("n_shared", _i32), ("d_ff", _i32),
                ("router", QMatDesc), ("router_bias", _vp), ("gate_up", QMatDesc), ("down", QMatDesc),
                ("sh_gate_up", QMatDesc), ("sh_down", QMatDesc)]


class MoeCapture(ctypes.Structure):
    _fields_ = [("topk_idx", _vp), ("topk_w", _vp), ("counts", _vp), ("offsets", _vp), ("perm", _vp)]


class LayerDesc(ctypes.Structure):
    _fields_ = [("attn_norm", _vp), ("wqkv", QMatDesc), ("wo", QMatDesc), ("ffn_norm", _vp), ("is_moe", _i32),
                ("dense_ff", _i32), ("dense_gate_up", QMatDesc), ("dense_down", QMatDesc), ("moe", MoeWeights),
                ("k_cache", _vp), ("v_cache", _vp), ("k_scale", _vp), ("v_scale", _vp)]


class ModelDesc(ctypes.Structure):
    _fields_ = [("n_layers", _i32), ("hidden", _i32), ("n_heads", _i32), ("head_dim", _i32), ("vocab", _i32),
                ("rope_theta", _f32), ("norm_eps", _f32), ("embed", _vp), ("final_norm", _vp),
                ("lm_head", QMatDesc), ("layers", ctypes.POINTER(LayerDesc)), ("embed_q", QMatDesc)]


class StateDesc(ctypes.Structure):
    _fields_ = [("rows", _i32), ("prefix_cap", _i32), ("ring_cap", _i32), ("prefix_len", _vp), ("gen_index", _vp)]


class StepCapture(ctypes.Structure):
    _fields_ = [("topk_idx", _vp), ("topk_w", _vp), ("lm_top2", _vp)]


_P = ctypes.POINTER
_lib.ocrdec_last_error.restype = ctypes.c_char_p
_lib.ocrdec_version.restype = ctypes.c_char_p
_lib.ocrdec_packed_bytes.argtypes = [_i32, _i32, _i32, _P(_sz)]
_lib.ocrdec_pack.argtypes = [_i32, _i32, _i32, _vp, _vp]
_lib.ocrdec_unpack.argtypes = [_i32, _i32, _i32, _vp, _vp]
_lib.ocrdec_gemv_q.argtypes = [_P(QMatDesc), _i32, _vp, _i64, _vp, _i32, _i64, _vp]
_lib.ocrdec_lm_argmax_workspace_bytes.argtypes = [_P(QMatDesc), _i32, _P(_sz)]
_lib.ocrdec_lm_argmax.argtypes = [_P(QMatDesc), _i32, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.ocrdec_attn_workspace_bytes.argtypes = [_P(AttnArgs), _P(_sz)]
_lib.ocrdec_attn_decode.argtypes = [_P(AttnArgs), _vp, _sz, _vp]
_lib.ocrdec_moe_workspace_bytes.argtypes = [_P(MoeWeights), _i32, _P(_sz)]
_lib.ocrdec_moe_layer.argtypes = [_P(MoeWeights), _i32, _vp, _vp, _i32, _vp, _P(MoeCapture), _vp, _sz, _vp]
_lib.ocrdec_step_workspace_bytes.argtypes = [_P(ModelDesc), _P(StateDesc), _P(_sz)]
_lib.ocrdec_decode_step.argtypes = [_P(ModelDesc), _P(StateDesc), _vp, _vp, _vp, _vp, _P(StepCapture), _vp, _sz, _vp]
_lib.ocrdec_prefill_workspace_bytes.argtypes = [_P(ModelDesc), _P(StateDesc), _i32, _P(_sz)]
_lib.ocrdec_prefill_batch_workspace_bytes.argtypes = [_P(ModelDesc), _P(StateDesc), _i32, _vp, _vp, _P(_sz)]
_lib.ocrdec_prefill_batch.argtypes = [_P(ModelDesc), _P(StateDesc), _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      _P(StepCapture), _vp, _sz, _vp]
_lib.ocrdec_round_workspace_bytes.argtypes = [_P(ModelDesc), _P(StateDesc), _i32, _P(_sz)]
_lib.ocrdec_run_round.argtypes = [_P(ModelDesc), _P(StateDesc), _vp, _i32, _vp, _i32, _i32, _vp, _sz, _vp]
_lib.ocrdec_decode_step_noalloc.argtypes = [_P(ModelDesc), _P(StateDesc), _vp, _vp, _vp, _vp, _P(StepCapture), _vp]
class Profile(ctypes.Structure):
    _fields_ = [("events", ctypes.POINTER(_vp)), ("kernels", ctypes.POINTER(_i32)), ("capacity", _i32),
                ("count", _i32)]


_lib.ocrdec_profile_set.argtypes = [ctypes.c_void_p]
_lib.ocrdec_profile_mark.argtypes = [_vp]
_lib.ocrdec_device_status.argtypes = [_vp, _sz, _vp, _P(ctypes.c_uint32)]
_lib.ocrdec_prefill.argtypes = [_P(ModelDesc), _P(StateDesc), _i32, _i32, _vp, _vp, _vp, _vp, _vp, _P(StepCapture),
                                _vp, _sz, _vp]
for _fn in ("ocrdec_packed_bytes", "ocrdec_pack", "ocrdec_unpack", "ocrdec_gemv_q", "ocrdec_lm_argmax_workspace_bytes",
            "ocrdec_lm_argmax", "ocrdec_attn_workspace_bytes",
            "ocrdec_attn_decode", "ocrdec_moe_workspace_bytes", "ocrdec_moe_layer", "ocrdec_step_workspace_bytes",
            "ocrdec_decode_step", "ocrdec_prefill_workspace_bytes", "ocrdec_prefill", "ocrdec_round_workspace_bytes",
            "ocrdec_run_round", "ocrdec_prefill_batch_workspace_bytes", "ocrdec_prefill_batch", "ocrdec_device_status",
            "ocrdec_decode_step_noalloc", "ocrdec_profile_set", "ocrdec_profile_mark"):
    getattr(_lib, _fn).restype = ctypes.c_int

EXPORTED = ["ocrdec_last_error", "ocrdec_version", "ocrdec_packed_bytes", "ocrdec_pack", "ocrdec_unpack",
            "ocrdec_gemv_q", "ocrdec_lm_argmax_workspace_bytes", "ocrdec_lm_argmax", "ocrdec_attn_workspace_bytes",
            "ocrdec_attn_decode", "ocrdec_moe_workspace_bytes",
            "ocrdec_moe_layer", "ocrdec_step_workspace_bytes", "ocrdec_decode_step",
            "ocrdec_prefill_workspace_bytes", "ocrdec_prefill", "ocrdec_round_workspace_bytes", "ocrdec_run_round",
            "ocrdec_prefill_batch_workspace_bytes", "ocrdec_prefill_batch", "ocrdec_device_status", "ocrdec_decode_step_noalloc",
            "ocrdec_profile_set", "ocrdec_profile_mark"]


def _ptr(t) -> int | None:
    """Device/host address of a torch tensor, numpy array or raw int (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


# ----------------------------------------------------------------------------
# Functions with the C names
# ----------------------------------------------------------------------------

def ocrdec_last_error() -> str:
    return _lib.ocrdec_last_error().decode()


def ocrdec_version() -> str:
    return _lib.ocrdec_version().decode()


def ocrdec_packed_bytes(fmt: int, n: int, k: int) -> int:
    b = _sz()
    _check(_lib.ocrdec_packed_bytes(fmt, n, k, ctypes.byref(b)))
    return b.value


def ocrdec_pack(fmt: int, n: int, k: int, canonical: np.ndarray) -> np.ndarray:
    canonical = np.ascontiguousarray(canonical).view(np.uint8)
    out = np.empty(ocrdec_packed_bytes(fmt, n, k), np.uint8)
    _check(_lib.ocrdec_pack(fmt, n, k, canonical.ctypes.data, out.ctypes.data))
    return out


def ocrdec_unpack(fmt: int, n: int, k: int, packed: np.ndarray, canonical_bytes: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed).view(np.uint8)
    out = np.empty(canonical_bytes, np.uint8)
    _check(_lib.ocrdec_unpack(fmt, n, k, packed.ctypes.data, out.ctypes.data))
    return out


def ocrdec_gemv_q(W: QMatDesc, rows: int, x, ldx: int, y, y_type: int, ldy: int, stream=None):
    _check(_lib.ocrdec_gemv_q(ctypes.byref(W), rows, _ptr(x), ldx, _ptr(y), y_type, ldy, _stream(stream)))


def ocrdec_lm_argmax_workspace_bytes(W: QMatDesc, rows: int) -> int:
    b = _sz()
    _check(_lib.ocrdec_lm_argmax_workspace_bytes(ctypes.byref(W), rows, ctypes.byref(b)))
    return b.value


def ocrdec_lm_argmax(W: QMatDesc, rows: int, x, tok_out, top2=None, ws=None, ws_bytes: int = 0, stream=None):
    _check(_lib.ocrdec_lm_argmax(ctypes.byref(W), rows, _ptr(x), _ptr(tok_out), _ptr(top2), _ptr(ws), ws_bytes,
                                 _stream(stream)))


def ocrdec_attn_workspace_bytes(a: AttnArgs) -> int:
    b = _sz()
    _check(_lib.ocrdec_attn_workspace_bytes(ctypes.byref(a), ctypes.byref(b)))
    return b.value


def ocrdec_attn_decode(a: AttnArgs, ws, ws_bytes: int, stream=None):
    _check(_lib.ocrdec_attn_decode(ctypes.byref(a), _ptr(ws), ws_bytes, _stream(stream)))


def ocrdec_moe_workspace_bytes(w: MoeWeights, rows: int) -> int:
    b = _sz()
    _check(_lib.ocrdec_moe_workspace_bytes(ctypes.byref(w), rows, ctypes.byref(b)))
    return b.value


def ocrdec_moe_layer(w: MoeWeights, rows: int, x, h, add_residual: bool, forced_topk=None,
                     capture: MoeCapture | None = None, ws=None, ws_bytes: int = 0, stream=None):
    _check(_lib.ocrdec_moe_layer(ctypes.byref(w), rows, _ptr(x), _ptr(h), int(add_residual), _ptr(forced_topk),
                                 ctypes.byref(capture) if capture is not None else None, _ptr(ws), ws_bytes,
                                 _stream(stream)))


def ocrdec_step_workspace_bytes(m: ModelDesc, st: StateDesc) -> int:
    b = _sz()
    _check(_lib.ocrdec_step_workspace_bytes(ctypes.byref(m), ctypes.byref(st), ctypes.byref(b)))
    return b.value


def ocrdec_decode_step(m: ModelDesc, st: StateDesc, tok_in=None, hidden=None, tok_out=None, forced_topk=None,
                       capture: StepCapture | None = None, ws=None, ws_bytes: int = 0, stream=None):
    _check(_lib.ocrdec_decode_step(ctypes.byref(m), ctypes.byref(st), _ptr(tok_in), _ptr(hidden), _ptr(tok_out),
                                   _ptr(forced_topk), ctypes.byref(capture) if capture is not None else None,
                                   _ptr(ws), ws_bytes, _stream(stream)))


def ocrdec_decode_step_noalloc(m: ModelDesc, st: StateDesc, tok_in=None, hidden=None, tok_out=None, forced_topk=None,
                               capture: StepCapture | None = None, stream=None):
    _check(_lib.ocrdec_decode_step_noalloc(ctypes.byref(m), ctypes.byref(st), _ptr(tok_in), _ptr(hidden),
                                           _ptr(tok_out), _ptr(forced_topk),
                                           ctypes.byref(capture) if capture is not None else None, _stream(stream)))


def ocrdec_profile_set(prof: "Profile | None"):
    _check(_lib.ocrdec_profile_set(ctypes.addressof(prof) if prof is not None else None))


def ocrdec_profile_mark(stream=None):
    _check(_lib.ocrdec_profile_mark(_stream(stream)))


def ocrdec_device_status(ws, ws_bytes: int, stream=None) -> int:
    """Flags (OCRDEC_DEV_*) of the last decode step that used `ws`; synchronises the stream."""
    f = ctypes.c_uint32()
    _check(_lib.ocrdec_device_status(_ptr(ws), ws_bytes, _stream(stream), ctypes.byref(f)))
    return f.value


class Request(ctypes.Structure):
    _fields_ = [("tokens", _vp), ("features", _vp), ("P", _i32), ("max_new", _i32), ("out", _vp), ("n_out", _i32),
                ("stop", _i32)]


def ocrdec_round_workspace_bytes(m: ModelDesc, st: StateDesc, max_P: int) -> int:
    b = _sz()
    _check(_lib.ocrdec_round_workspace_bytes(ctypes.byref(m), ctypes.byref(st), max_P, ctypes.byref(b)))
    return b.value


def ocrdec_run_round(m: ModelDesc, st: StateDesc, reqs, eos=(), keep_eos: bool = False, ws=None, ws_bytes: int = 0,
                     stream=None):
    """reqs: a ctypes array of Request (host), filled in place."""
    eos_arr = (ctypes.c_int32 * max(len(eos), 1))(*eos)
    _check(_lib.ocrdec_run_round(ctypes.byref(m), ctypes.byref(st), ctypes.cast(reqs, _vp), len(reqs),
                                 ctypes.cast(eos_arr, _vp), len(eos), int(keep_eos), _ptr(ws), ws_bytes,
                                 _stream(stream)))


def _i32_array(v):
    return (ctypes.c_int32 * len(v))(*[int(x) for x in v])


def ocrdec_prefill_batch_workspace_bytes(m: ModelDesc, st: StateDesc, rows, P) -> int:
    b = _sz()
    r, p = _i32_array(rows), _i32_array(P)
    _check(_lib.ocrdec_prefill_batch_workspace_bytes(ctypes.byref(m), ctypes.byref(st), len(P), ctypes.cast(r, _vp),
                                                     ctypes.cast(p, _vp), ctypes.byref(b)))
    return b.value


def ocrdec_prefill_batch(m: ModelDesc, st: StateDesc, rows, P, tok=None, emb=None, forced_topk=None, tok_out=None,
                         hidden=None, capture: StepCapture | None = None, ws=None, ws_bytes: int = 0, stream=None):
    r, p = _i32_array(rows), _i32_array(P)
    _check(_lib.ocrdec_prefill_batch(ctypes.byref(m), ctypes.byref(st), len(P), ctypes.cast(r, _vp),
                                     ctypes.cast(p, _vp), _ptr(tok), _ptr(emb), _ptr(forced_topk), _ptr(tok_out),
                                     _ptr(hidden), ctypes.byref(capture) if capture is not None else None, _ptr(ws),
                                     ws_bytes, _stream(stream)))


def ocrdec_prefill_workspace_bytes(m: ModelDesc, st: StateDesc, P: int) -> int:
    b = _sz()
    _check(_lib.ocrdec_prefill_workspace_bytes(ctypes.byref(m), ctypes.byref(st), P, ctypes.byref(b)))
    return b.value


def ocrdec_prefill(m: ModelDesc, st: StateDesc, row: int, P: int, tok=None, emb=None, forced_topk=None, tok_out=None,
                   hidden=None, capture: StepCapture | None = None, ws=None, ws_bytes: int = 0, stream=None):
    _check(_lib.ocrdec_prefill(ctypes.byref(m), ctypes.byref(st), row, P, _ptr(tok), _ptr(emb), _ptr(forced_topk),
                               _ptr(tok_out), _ptr(hidden), ctypes.byref(capture) if capture is not None else None,
                               _ptr(ws), ws_bytes, _stream(stream)))


# ----------------------------------------------------------------------------
# Device-side containers (allocation through torch; packing through the C ABI)
# ----------------------------------------------------------------------------

class DeviceQMat:
    """A packed weight matrix resident on the GPU."""

    def __init__(self, m, device="cuda"):
        import torch
        packed = ocrdec_pack(m.fmt, m.n, m.k, m.data)
        self.tensor = torch.from_numpy(packed).to(device)
        self.fmt, self.n, self.k = m.fmt, m.n, m.k
        self.desc = QMatDesc(m.fmt, m.n, m.k, self.tensor.data_ptr())

    @property
    def nbytes(self) -> int:
        return self.tensor.numel()


def _f16_dev(a, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).astype(np.float16).view(np.int16)).to(device)


def _empty_qmat() -> QMatDesc:
    return QMatDesc(0, 0, 0, None)


def moe_weights(lay, hidden: int, top_k: int, device="cuda"):
    """MoeWeights descriptor (and the tensors it points to) for one MoE layer
    given canonical matrices ``router, exp_gate_up, exp_down, sh_gate_up,
    sh_down`` and optional ``router_bias``."""
    import torch
    keep = {}
    for name in ("router", "exp_gate_up", "exp_down", "sh_gate_up", "sh_down"):
        m = getattr(lay, name, None)
        keep[name] = DeviceQMat(m, device) if m is not None else None
    bias = getattr(lay, "router_bias", None)
    keep["bias"] = torch.from_numpy(np.asarray(bias, np.float32)).to(device) if bias is not None else None
    E = keep["router"].n
    F = keep["exp_down"].k
    S = 0 if keep["sh_gate_up"] is None else keep["sh_gate_up"].n // (2 * F)
    w = MoeWeights(hidden, E, top_k, S, F, keep["router"].desc, _ptr(keep["bias"]), keep["exp_gate_up"].desc,
                   keep["exp_down"].desc,
                   keep["sh_gate_up"].desc if S else _empty_qmat(), keep["sh_down"].desc if S else _empty_qmat())
    return w, keep


class DeviceModel:
    """The decoder's weights on the GPU plus the ABI descriptors."""

    def __init__(self, model, device="cuda"):
        d = model.dims
        self.dims = d
        self.keep = []
        layers = (LayerDesc * len(model.layers))()
        for i, lay in enumerate(model.layers):
            an, fn = _f16_dev(lay.attn_norm, device), _f16_dev(lay.ffn_norm, device)
            wqkv, wo = DeviceQMat(lay.wqkv, device), DeviceQMat(lay.wo, device)
            self.keep += [an, fn, wqkv, wo]
            L = layers[i]
            L.attn_norm, L.ffn_norm = an.data_ptr(), fn.data_ptr()
            L.wqkv, L.wo = wqkv.desc, wo.desc
            L.is_moe = int(lay.is_moe)
            if lay.is_moe:
                mw, keep = moe_weights(lay, d.hidden, d.top_k, device)
                self.keep.append(keep)
                L.moe = mw
                L.dense_ff = 0
                L.dense_gate_up = _empty_qmat()
                L.dense_down = _empty_qmat()
            else:
                gu, dn = DeviceQMat(lay.dense_gate_up, device), DeviceQMat(lay.dense_down, device)
                self.keep += [gu, dn]
                L.dense_ff = lay.dense_down.k
                L.dense_gate_up, L.dense_down = gu.desc, dn.desc
        self.layers = layers
        self.embed = _f16_dev(model.embed, device) if model.embed is not None else None
        self.final_norm = _f16_dev(model.final_norm, device) if model.final_norm is not None else None
        self.lm_head = DeviceQMat(model.lm_head, device) if model.lm_head is not None else None
        eq = getattr(model, "embed_q", None)
        self.embed_q = DeviceQMat(eq, device) if (eq is not None and model.embed is None) else None
        self.desc = ModelDesc(len(model.layers), d.hidden, d.n_heads, d.head_dim, d.vocab, d.rope_theta, d.norm_eps,
                              _ptr(self.embed), _ptr(self.final_norm),
                              self.lm_head.desc if self.lm_head is not None else _empty_qmat(), layers,
                              self.embed_q.desc if self.embed_q is not None else _empty_qmat())

    def layer_view(self, first: int, count: int, with_head: bool):
        """ModelDesc over layers [first, first+count) of this model, sharing its
        device weights (bind the caches first).  The embedding (fp16 or
        quantised) is kept only for first == 0 (otherwise the input comes from `hidden`); the final norm and
        LM head only if with_head."""
        n = self.desc.n_layers
        if not (0 <= first and count >= 1 and first + count <= n):
            raise ValueError("layer range [%d, %d) outside 0..%d" % (first, first + count, n))
        layers = (LayerDesc * count)()
        for i in range(count):
            layers[i] = self.layers[first + i]
        d = self.desc
        view = ModelDesc(count, d.hidden, d.n_heads, d.head_dim, d.vocab, d.rope_theta, d.norm_eps,
                         d.embed if first == 0 else None, d.final_norm if with_head else None,
                         d.lm_head if with_head else _empty_qmat(), layers,
                         d.embed_q if first == 0 else _empty_qmat())
        view._keep_layers = layers
        return view

    def bind_caches(self, k_cache, v_cache, k_scale=None, v_scale=None):
        """Point every layer at its slice of caches [L][R][NH][cap][D] (torch fp16/int16, or int8 codes with
        fp16 scales [L][R][NH][cap])."""
        for i in range(self.desc.n_layers):
            self.layers[i].k_cache = k_cache[i].data_ptr()
            self.layers[i].v_cache = v_cache[i].data_ptr()
            self.layers[i].k_scale = k_scale[i].data_ptr() if k_scale is not None else None
            self.layers[i].v_scale = v_scale[i].data_ptr() if v_scale is not None else None
        self._caches = (k_cache, v_cache, k_scale, v_scale)


class DeviceState:
    """Per-row decode state on the GPU: lengths, generation index and caches."""

    def __init__(self, state, prefix_cap: int, ring_cap: int, device="cuda"):
        import torch
        self.prefix_len = torch.from_numpy(np.asarray(state.prefix_len, np.int32)).to(device)
        self.gen_index = torch.from_numpy(np.asarray(state.gen_index, np.int32)).to(device)
        self.int8 = getattr(state, "k_scale", None) is not None
        if self.int8:
            self.k_cache = torch.from_numpy(np.ascontiguousarray(state.k_cache, np.int8)).to(device)
            self.v_cache = torch.from_numpy(np.ascontiguousarray(state.v_cache, np.int8)).to(device)
            self.k_scale = torch.from_numpy(np.ascontiguousarray(state.k_scale).view(np.int16)).to(device)
            self.v_scale = torch.from_numpy(np.ascontiguousarray(state.v_scale).view(np.int16)).to(device)
        else:
            self.k_cache = torch.from_numpy(np.ascontiguousarray(state.k_cache).view(np.int16)).to(device)
            self.v_cache = torch.from_numpy(np.ascontiguousarray(state.v_cache).view(np.int16)).to(device)
            self.k_scale = self.v_scale = None
        self.rows = int(self.prefix_len.numel())
        self.desc = StateDesc(self.rows, prefix_cap, ring_cap, self.prefix_len.data_ptr(), self.gen_index.data_ptr())
