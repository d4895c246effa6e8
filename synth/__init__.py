"""Seeded synthetic inputs for the OCR-decoder decode step.

This module draws random numbers and encodes them into the storage formats the
decode step reads; it holds none of the step's arithmetic.  Both the GPU
library's tests/bench and the CPU oracle take their inputs from here, so the two
sides see byte-identical weights, caches and tokens.

The random stream is SplitMix64 used as a counter-based generator with a
Box-Muller transform (see synth.c).  Every tensor has its own 64-bit stream id,
derived from (base seed, tensor tag, indices) with BLAKE2b, so a tensor's values
do not depend on which other tensors were generated or in what order.
"""
from __future__ import annotations

import ctypes
import hashlib
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

# Storage-format codes (same numbering as the library's public header).
F16, Q8_0, Q4_0, U8A_G32 = 0, 1, 2, 3
FMT_NAMES = {F16: "F16", Q8_0: "Q8_0", Q4_0: "Q4_0", U8A_G32: "U8A_G32"}
BLOCK_BYTES = {Q8_0: 34, Q4_0: 18, U8A_G32: 36}


def build(force: bool = False) -> str:
    """Compile synth.c into libsynth.so with gcc + OpenMP."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        u64, i64, i32, dbl, vp = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32,
                                  ctypes.c_double, ctypes.c_void_p)
        L.synth_d2h.argtypes, L.synth_d2h.restype = [dbl], ctypes.c_uint16
        L.synth_h2d.argtypes, L.synth_h2d.restype = [ctypes.c_uint16], dbl
        L.synth_draw.argtypes, L.synth_draw.restype = [u64, u64], u64
        L.synth_normal_at.argtypes, L.synth_normal_at.restype = [u64, u64], dbl
        L.synth_normal_f64.argtypes = [u64, i64, dbl, dbl, vp]
        L.synth_normal_f16.argtypes = [u64, i64, dbl, dbl, vp]
        L.synth_uniform_i32.argtypes = [u64, i64, i32, i32, vp]
        for f in (L.synth_q8_0, L.synth_q4_0, L.synth_u8a_g32):
            f.argtypes = [u64, i64, i64, dbl, vp]
        _lib = L
    return _lib


def stream_id(seed: int, tag: str, *idx: int) -> int:
    """64-bit stream id for one tensor: BLAKE2b of (seed, tag, indices)."""
    key = ("%d|%s|%s" % (seed, tag, ",".join(str(int(i)) for i in idx))).encode()
    return int.from_bytes(hashlib.blake2b(key, digest_size=8).digest(), "little")


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def normal_f64(stream: int, shape, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    out = np.empty(shape, np.float64)
    lib().synth_normal_f64(stream, out.size, mean, std, _ptr(out))
    return out


def normal_f16(stream: int, shape, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    out = np.empty(shape, np.float16)
    lib().synth_normal_f16(stream, out.size, mean, std, _ptr(out))
    return out


def uniform_i32(stream: int, shape, lo: int, hi: int) -> np.ndarray:
    out = np.empty(shape, np.int32)
    lib().synth_uniform_i32(stream, out.size, lo, hi, _ptr(out))
    return out


@dataclass
class QMat:
    """A weight matrix W[n][k] in one canonical storage format.

    ``data`` is a flat uint8 array: fp16 values row-major for F16, otherwise the
    canonical 32-weight blocks of each row, rows in order (layouts in synth.c).
    """
    fmt: int
    n: int
    k: int
    data: np.ndarray

    @property
    def nbytes(self) -> int:
        return int(self.data.size)

    def rows(self, r0: int, r1: int) -> "QMat":
        """The sub-matrix of rows [r0, r1) (a view)."""
        per_row = self.nbytes // self.n
        return QMat(self.fmt, r1 - r0, self.k, self.data[r0 * per_row:r1 * per_row])


def qmat_bytes(fmt: int, n: int, k: int) -> int:
    if fmt == F16:
        return n * k * 2
    return n * (k // 32) * BLOCK_BYTES[fmt]


def random_qmat(fmt: int, stream: int, n: int, k: int, std: float = 0.02) -> QMat:
    """W ~ std * N(0,1), stored in ``fmt`` (quantised from the drawn values)."""
    if fmt != F16 and k % 32:
        raise ValueError("k must be a multiple of 32 for block formats")
    out = np.empty(qmat_bytes(fmt, n, k), np.uint8)
    if fmt == F16:
        lib().synth_normal_f16(stream, n * k, 0.0, std, _ptr(out))
    elif fmt == Q8_0:
        lib().synth_q8_0(stream, n, k, std, _ptr(out))
    elif fmt == Q4_0:
        lib().synth_q4_0(stream, n, k, std, _ptr(out))
    elif fmt == U8A_G32:
        lib().synth_u8a_g32(stream, n, k, std, _ptr(out))
    else:
        raise ValueError(fmt)
    return QMat(fmt, n, k, out)


def stack_qmats(mats) -> QMat:
    """Stack matrices with equal k and format along n."""
    m0 = mats[0]
    assert all(m.fmt == m0.fmt and m.k == m0.k for m in mats)
    return QMat(m0.fmt, sum(m.n for m in mats), m0.k, np.concatenate([m.data for m in mats]))


# ----------------------------------------------------------------------------
# Decoder workloads
# ----------------------------------------------------------------------------

@dataclass
class Dims:
    """Shape of the decoder (defaults: the 12-layer OCR decoder)."""
    hidden: int = 1280
    n_heads: int = 10
    head_dim: int = 128
    n_layers: int = 12
    n_dense: int = 1            # layers [0, n_dense) use the dense SwiGLU MLP
    dense_ff: int = 3584
    n_experts: int = 64
    top_k: int = 6
    n_shared: int = 2
    expert_ff: int = 896
    vocab: int = 129280
    prefix_cap: int = 1100
    ring_cap: int = 128
    rope_theta: float = 10000.0
    norm_eps: float = 1e-6
    fmt_attn: int = Q8_0        # QKV and O projections
    fmt_router: int = Q8_0
    fmt_dense: int = Q4_0
    fmt_expert: int = Q4_0      # routed experts
    fmt_shared: int = Q4_0
    fmt_lm: int = F16
    fmt_embed: int = F16        # F16: Model.embed (fp16 array); otherwise Model.embed_q (QMat)
    w_std: float = 0.02


@dataclass
class Layer:
    attn_norm: np.ndarray       # fp16 [H]
    wqkv: QMat                  # [3*NH*D, H]: q rows, then k rows, then v rows
    wo: QMat                    # [H, NH*D]
    ffn_norm: np.ndarray        # fp16 [H]
    is_moe: bool
    dense_gate_up: QMat | None = None   # [2*F, H]: gate rows then up rows
    dense_down: QMat | None = None      # [H, F]
    router: QMat | None = None          # [E, H]
    exp_gate_up: QMat | None = None     # [E*2*F', H]: expert e owns rows [e*2F', (e+1)*2F'), gate first
    exp_down: QMat | None = None        # [E*H, F']: expert e owns rows [e*H, (e+1)*H)
    sh_gate_up: QMat | None = None      # [S*2*F', H]
    sh_down: QMat | None = None         # [S*H, F']
    router_bias: np.ndarray | None = None  # float32 [E] (prefill-shaped MoE only)


@dataclass
class Model:
    dims: Dims
    seed: int
    embed: np.ndarray | None            # fp16 [V, H]
    final_norm: np.ndarray | None       # fp16 [H]
    lm_head: QMat | None                # [V, H]
    layers: list = field(default_factory=list)
    embed_q: QMat | None = None         # [V, H] quantised embedding (when embed is None)


def norm_weight(stream: int, n: int, std: float) -> np.ndarray:
    """RMSNorm gain: 1 + std * N(0,1), stored fp16."""
    return normal_f16(stream, (n,), 1.0, std)


def make_moe_weights(d: Dims, seed: int, layer: int, with_bias: bool = False) -> dict:
    H, E, F = d.hidden, d.n_experts, d.expert_ff
    out = dict(
        router=random_qmat(d.fmt_router, stream_id(seed, "router", layer), E, H, d.w_std),
        exp_gate_up=stack_qmats([random_qmat(d.fmt_expert, stream_id(seed, "exp_gate_up", layer, e), 2 * F, H, d.w_std)
                                 for e in range(E)]),
        exp_down=stack_qmats([random_qmat(d.fmt_expert, stream_id(seed, "exp_down", layer, e), H, F, d.w_std)
                              for e in range(E)]),
        sh_gate_up=stack_qmats([random_qmat(d.fmt_shared, stream_id(seed, "sh_gate_up", layer, s), 2 * F, H, d.w_std)
                                for s in range(d.n_shared)]) if d.n_shared else None,
        sh_down=stack_qmats([random_qmat(d.fmt_shared, stream_id(seed, "sh_down", layer, s), H, F, d.w_std)
                             for s in range(d.n_shared)]) if d.n_shared else None,
    )
    if with_bias:
        out["router_bias"] = normal_f64(stream_id(seed, "router_bias", layer), (E,)).astype(np.float32)
    return out


def make_model(d: Dims, seed: int, with_embed: bool = True, with_lm: bool = True) -> Model:
    H, NH, D = d.hidden, d.n_heads, d.head_dim
    layers = []
    for l in range(d.n_layers):
        lay = Layer(
            attn_norm=norm_weight(stream_id(seed, "attn_norm", l), H, d.w_std),
            wqkv=random_qmat(d.fmt_attn, stream_id(seed, "wqkv", l), 3 * NH * D, H, d.w_std),
            wo=random_qmat(d.fmt_attn, stream_id(seed, "wo", l), H, NH * D, d.w_std),
            ffn_norm=norm_weight(stream_id(seed, "ffn_norm", l), H, d.w_std),
            is_moe=l >= d.n_dense,
        )
        if lay.is_moe:
            for k_, v_ in make_moe_weights(d, seed, l).items():
                setattr(lay, k_, v_)
        else:
            lay.dense_gate_up = random_qmat(d.fmt_dense, stream_id(seed, "dense_gate_up", l), 2 * d.dense_ff, H, d.w_std)
            lay.dense_down = random_qmat(d.fmt_dense, stream_id(seed, "dense_down", l), H, d.dense_ff, d.w_std)
        layers.append(lay)
    embed = embed_q = None
    if with_embed and d.fmt_embed == F16:
        embed = normal_f16(stream_id(seed, "embed"), (d.vocab, H), 0.0, d.w_std)
    elif with_embed:
        embed_q = random_qmat(d.fmt_embed, stream_id(seed, "embed"), d.vocab, H, d.w_std)
    lm = random_qmat(d.fmt_lm, stream_id(seed, "lm_head"), d.vocab, H, d.w_std) if with_lm else None
    fnorm = norm_weight(stream_id(seed, "final_norm"), H, d.w_std) if with_lm else None
    return Model(d, seed, embed, fnorm, lm, layers, embed_q)


@dataclass
class State:
    """Per-row decode state: caches [L][R][NH][prefix_cap + ring_cap][D], fp16,
    or int8 codes with one fp16 scale per (layer, row, head, slot) in k_scale /
    v_scale [L][R][NH][cap]."""
    prefix_len: np.ndarray      # int32 [R]
    gen_index: np.ndarray       # int32 [R]
    k_cache: np.ndarray         # fp16 (or int8) [L, R, NH, cap, D]
    v_cache: np.ndarray
    k_scale: np.ndarray | None = None   # fp16 [L, R, NH, cap] for int8 caches
    v_scale: np.ndarray | None = None

    def copy(self) -> "State":
        return State(self.prefix_len.copy(), self.gen_index.copy(), self.k_cache.copy(), self.v_cache.copy(),
                     None if self.k_scale is None else self.k_scale.copy(),
                     None if self.v_scale is None else self.v_scale.copy())


def make_state(d: Dims, seed: int, prefix_len, gen_index, fill: str = "zero") -> State:
    """Caches ~N(0,1) fp16 over every slot a row has already written.

    Prefix positions [0, prefix_len[r]) and ring slots [0, min(gen_index[r], ring_cap))
    are drawn; the rest are zero (``fill="zero"``) or NaN (``fill="nan"``, used to
    show that nothing outside a row's window is ever read).
    """
    prefix_len = np.asarray(prefix_len, np.int32)
    gen_index = np.asarray(gen_index, np.int32)
    R = prefix_len.size
    L, NH, D, cap = d.n_layers, d.n_heads, d.head_dim, d.prefix_cap + d.ring_cap
    kc = np.empty((L, R, NH, cap, D), np.float16)
    vc = np.empty_like(kc)
    for l in range(L):
        for r in range(R):
            kc[l, r] = normal_f16(stream_id(seed, "k_cache", l, r), (NH, cap, D))
            vc[l, r] = normal_f16(stream_id(seed, "v_cache", l, r), (NH, cap, D))
            valid = np.zeros(cap, bool)
            valid[:prefix_len[r]] = True
            valid[d.prefix_cap:d.prefix_cap + min(int(gen_index[r]), d.ring_cap)] = True
            pad = np.float16(np.nan) if fill == "nan" else np.float16(0)
            kc[l, r][:, ~valid] = pad
            vc[l, r][:, ~valid] = pad
    return State(prefix_len.copy(), gen_index.copy(), kc, vc)


def make_state_int8(d: Dims, seed: int, prefix_len, gen_index) -> State:
    """An int8 KV cache over every slot a row has already written: codes
    round(40 * N(0,1)) clipped to [-127, 127] and scales fp16((1 + 0.1 N(0,1)) / 40),
    so the stored values are about N(0,1).  Unwritten slots hold code 0 and
    scale 0."""
    prefix_len = np.asarray(prefix_len, np.int32)
    gen_index = np.asarray(gen_index, np.int32)
    R = prefix_len.size
    L, NH, D, cap = d.n_layers, d.n_heads, d.head_dim, d.prefix_cap + d.ring_cap
    caches, scales = [], []
    for tag in ("k", "v"):
        c = np.zeros((L, R, NH, cap, D), np.int8)
        s = np.zeros((L, R, NH, cap), np.float16)
        for l in range(L):
            for r in range(R):
                codes = np.clip(np.rint(40.0 * normal_f64(stream_id(seed, tag + "_cache8", l, r), (NH, cap, D))),
                                -127, 127).astype(np.int8)
                sc = ((1.0 + 0.1 * normal_f64(stream_id(seed, tag + "_scale8", l, r), (NH, cap))) / 40.0).astype(np.float16)
                valid = np.zeros(cap, bool)
                valid[:prefix_len[r]] = True
                valid[d.prefix_cap:d.prefix_cap + min(int(gen_index[r]), d.ring_cap)] = True
                c[l, r][:, valid] = codes[:, valid]
                s[l, r][:, valid] = sc[:, valid]
        caches.append(c)
        scales.append(s)
    return State(prefix_len.copy(), gen_index.copy(), caches[0], caches[1], scales[0], scales[1])


def first_tokens(d: Dims, seed: int, rows: int) -> np.ndarray:
    return uniform_i32(stream_id(seed, "tokens0"), (rows,), 0, d.vocab)


# Named workloads ------------------------------------------------------------

def dims_dense_layer() -> Dims:
    """One dense fp16 decoder layer over 256 cached positions."""
    return Dims(n_layers=1, n_dense=1, fmt_attn=F16, fmt_dense=F16, prefix_cap=256, ring_cap=128)


def dims_moe_layer() -> Dims:
    """One Q8_0 MoE decoder layer, prefix 1100 + full 128-slot ring."""
    return Dims(n_layers=1, n_dense=0, fmt_attn=Q8_0, fmt_router=Q8_0, fmt_expert=Q8_0, fmt_shared=Q8_0)


def dims_full() -> Dims:
    """The 12-layer mixed Q4_0 decoder (attention and router Q8_0, LM head fp16)."""
    return Dims()
