"""Oracle primitives and the composed decode step (float64, numpy).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Numeric conventions (shared by every function below):

* Arithmetic is float64.  Values the decode step stores as fp16 are rounded to
  IEEE binary16 with round-to-nearest-even at exactly these points: ``x``
  after each RMSNorm (the input of every projection); q, k, v after RoPE (k
  and v are what the cache holds); the attention output; the SwiGLU
  intermediate.  [UOCR] "Il decoder e il Mixture of Experts": the decode loop
  keeps activations in fp16.
* The residual stream ``h`` is not rounded to fp16.  Reading: the pages do
  not say which tensors "activations" covers; the fp16 ones are taken to be
  the tensors the projections and the cache consume, and the running sum
  between blocks is kept wide, the precision [NCNN] 3.1 gives the residual
  between the blocks of its decoder (the only page that states one).
* Expert outputs, the MoE combine, router logits and LM-head logits are not
  rounded to fp16.  Where floating point decides an integer (top-k routing,
  the LM-head argmax) the decision is taken on logits rounded to float32, the
  precision the GPU kernels compute them in.
"""
from __future__ import annotations

import numpy as np

F16, Q8_0, Q4_0, U8A_G32 = 0, 1, 2, 3
QK = 32  # weights per quantisation block
_BLOCK_BYTES = {Q8_0: 34, Q4_0: 18, U8A_G32: 36}


def f16(x) -> np.ndarray:
    """Round to binary16 (RNE, subnormals kept) and widen back to float64."""
    return np.asarray(x, np.float64).astype(np.float16).astype(np.float64)


def f32(x) -> np.ndarray:
    """Round to binary32 and widen back to float64."""
    return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)


# -----------------------------------------------------------------------------
# Weight formats
# -----------------------------------------------------------------------------

def _half_field(blk: np.ndarray, off: int) -> np.ndarray:
    """Little-endian fp16 stored at byte ``off`` of every block, as float64."""
    raw = blk[..., off].astype(np.uint16) | (blk[..., off + 1].astype(np.uint16) << 8)
    return raw.view(np.float16).astype(np.float64)


def dequant(fmt: int, data: np.ndarray, n: int, k: int) -> np.ndarray:
    """Dense float64 W[n][k] from one of the four storage formats.

    [UOCR] "In sintesi" and "Quantizzazione": fp16, mixed Q8_0 and Q4_0
    profiles, dequantised inside the kernels (no full fp16 copy).  [FALCON]
    "Weights are compressed with NNCF INT8_ASYM": u8 weights with a zero point.
    The pages name the formats but print no bit layout; the 32-weight blocks
    with an fp16 scale, Q4_0 as (q - 8) * d and int8-asymmetric groups of 32
    are the workload's stated definitions.  Readings: the page's "group size
    64" conflicts with the 32-weight Q8_0/Q4_0 blocks and is read as 32; the
    Q4_0 nibble order (byte j holds element j low, element j+16 high) and the
    int8-asymmetric form s * (q - z) with fp16 s and z are our choices.

      F16      w = the stored fp16 value
      Q8_0     block = fp16 d, 32 x int8 q            w_i = d * q_i
      Q4_0     block = fp16 d, 16 bytes of nibbles    w_i = d * (q_i - 8)
      U8A_G32  block = fp16 s, fp16 z, 32 x uint8 q   w_i = s * (q_i - z)
    """
    data = np.asarray(data, np.uint8).reshape(-1)
    if fmt == F16:
        return data.view(np.float16).reshape(n, k).astype(np.float64)
    if k % QK:
        raise ValueError("k must be a multiple of 32")
    nb = k // QK
    blk = data.reshape(n, nb, _BLOCK_BYTES[fmt])
    if fmt == Q8_0:
        d = _half_field(blk, 0)
        q = blk[..., 2:34].view(np.int8).astype(np.float64)
        w = d[..., None] * q
    elif fmt == Q4_0:
        d = _half_field(blk, 0)
        b = blk[..., 2:18]
        q = np.concatenate([b & 0x0F, b >> 4], axis=-1).astype(np.float64)
        w = d[..., None] * (q - 8.0)
    elif fmt == U8A_G32:
        s = _half_field(blk, 0)
        z = _half_field(blk, 2)
        q = blk[..., 4:36].astype(np.float64)
        w = s[..., None] * (q - z[..., None])
    else:
        raise ValueError(fmt)
    return w.reshape(n, k)


def gemv(fmt: int, data: np.ndarray, n: int, k: int, x: np.ndarray) -> np.ndarray:
    """y[r][n] = sum_k W[n][k] * x[r][k] with W dequantised (float64).

    [UOCR] "Quantizzazione": dequantisation happens inside the GEMV; no
    precision is named for the products, which are exact here.
    """
    W = dequant(fmt, data, n, k)
    return np.asarray(x, np.float64) @ W.T


def gemv_qmat(m, x: np.ndarray) -> np.ndarray:
    """``gemv`` on an object with ``fmt, n, k, data`` attributes."""
    return gemv(m.fmt, m.data, m.n, m.k, x)


# -----------------------------------------------------------------------------
# Normalisation, rotary embedding, attention
# -----------------------------------------------------------------------------

def rmsnorm(h: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """x = h / sqrt(mean(h^2) + eps) * gamma over the last axis.

    The decoder layer is pre-normalised with RMSNorm (workload definition of
    the dense layer); eps is not given and is read as 1e-6.
    """
    h = np.asarray(h, np.float64)
    ms = np.mean(h * h, axis=-1, keepdims=True)
    return h / np.sqrt(ms + eps) * np.asarray(gamma, np.float64)


def rope(x: np.ndarray, pos, theta: float, rot_dim: int | None = None) -> np.ndarray:
    """Rotary position embedding, rotate-half convention, over the first
    ``rot_dim`` lanes of the last axis (default: all).

    For i < rot_dim/2 with f_i = theta^(-2i/rot_dim) and a = pos * f_i:
      (x_i, x_{i+rot_dim/2}) <- (x_i cos a - x_{i+half} sin a,
                                 x_{i+half} cos a + x_i sin a).
    RoPE with theta 10000 is part of the workload definition; the convention
    (rotate-half) is our reading.  [NCNN] 3.3: during incremental decoding the
    position is the current linear position, so ``pos`` is the absolute index
    of the new token.
    """
    x = np.asarray(x, np.float64)
    d = x.shape[-1] if rot_dim is None else rot_dim
    half = d // 2
    i = np.arange(half, dtype=np.float64)
    freq = theta ** (-2.0 * i / d)
    a = np.asarray(pos, np.float64)[..., None] * freq
    c, s = np.cos(a), np.sin(a)
    x1, x2 = x[..., :half], x[..., half:d]
    out = x.copy()
    out[..., :half] = x1 * c - x2 * s
    out[..., half:d] = x2 * c + x1 * s
    return out


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
              sink: float | None = None, sink_index: int | None = None) -> np.ndarray:
    """Single-query scaled dot-product attention.

    s_j = scale * (q . k_j);  o = sum_j softmax(s)_j v_j.

    ``sink`` (a logit) adds one more key whose value is zero.  [FALCON] on
    the attention sink: rescaling the output by sigmoid(lse - sink) is the same
    as a softmax over the real keys plus one key with logit = sink and value 0.
    With ``sink_index`` the sink logit is added to the score of that cached key
    (the host seeds the sink at cache index 0 with zero key and zero value),
    which is the page's 65-lane construction with the constant lane factored
    out; without it the sink is a separate extra key.
    """
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    s = (K @ q) * scale
    if sink is not None and sink_index is not None:
        s = s.copy()
        s[sink_index] += sink
        sink = None
    m = s.max() if s.size else -np.inf
    if sink is not None:
        m = max(m, sink)
    e = np.exp(s - m)
    den = e.sum()
    if sink is not None:
        den += np.exp(sink - m)
    return (e @ V) / den


def logsumexp(s: np.ndarray) -> float:
    s = np.asarray(s, np.float64)
    m = s.max()
    return float(m + np.log(np.exp(s - m).sum()))


# -----------------------------------------------------------------------------
# MoE: routing, grouping, experts, combine
# -----------------------------------------------------------------------------

def softmax(v: np.ndarray) -> np.ndarray:
    v = np.asarray(v, np.float64)
    e = np.exp(v - v.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def route(logits: np.ndarray, top_k: int, bias: np.ndarray | None = None):
    """Top-k routing of one token.

    [UOCR] "Il decoder e il Mixture of Experts": 64 routed experts, top-6.
    Workload definition: softmax over the router logits, the top 6 by
    probability, weights renormalised over the chosen 6.  Readings: ties go to
    the lower expert index; the routed scaling factor is 1; an optional
    per-expert bias is added to the logits before the softmax (so it moves both
    the choice and the weights).  The decision is taken on float32-rounded
    logits (see the module docstring).

    Returns (idx[top_k] int32, ordered by probability descending, then index
    ascending; w[top_k] float64).
    """
    l = np.asarray(logits, np.float64)
    if bias is not None:
        l = l + np.asarray(bias, np.float64)
    l = f32(l)
    p = softmax(l)
    order = sorted(range(l.size), key=lambda e: (-p[e], e))
    idx = np.array(order[:top_k], np.int32)
    w = p[idx] / p[idx].sum()
    return idx, w


def route_forced(logits: np.ndarray, idx: np.ndarray, bias: np.ndarray | None = None) -> np.ndarray:
    """Renormalised weights for a given choice of experts (teacher forcing)."""
    l = np.asarray(logits, np.float64)
    if bias is not None:
        l = l + np.asarray(bias, np.float64)
    p = softmax(f32(l))
    idx = np.asarray(idx)
    return p[idx] / p[idx].sum()


def topk_gap(logits: np.ndarray, top_k: int, bias: np.ndarray | None = None) -> float:
    """Smallest gap between adjacent ranks 1..top_k+1 of the routed logits.

    A gap below the near-tie threshold means several routings are correct."""
    l = np.asarray(logits, np.float64)
    if bias is not None:
        l = l + bias
    s = np.sort(l)[::-1][:top_k + 1]
    return float(np.min(s[:-1] - s[1:]))


def group(idx: np.ndarray, n_experts: int):
    """Group (token, rank) pairs by expert: a stable counting sort.

    [UOCR] "Il decoder e il Mixture of Experts": the runtime computes the
    routing, groups the tokens per expert, runs the projections and recombines
    the results.  Reading: within one expert the pairs are ordered by token,
    then by rank.

    idx: int [T][k].  Returns counts[E], offsets[E+1] (exclusive scan),
    perm[T*k] (the flattened pair index t*k + j at each grouped position) and
    inv[T][k] (the grouped position of pair (t, j)).
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    counts = np.zeros(n_experts, np.int64)
    for t in range(T):
        for j in range(k):
            counts[idx[t, j]] += 1
    offsets = np.zeros(n_experts + 1, np.int64)
    for e in range(n_experts):
        offsets[e + 1] = offsets[e] + counts[e]
    fill = offsets[:-1].copy()
    perm = np.zeros(T * k, np.int64)
    inv = np.zeros((T, k), np.int64)
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            perm[fill[e]] = t * k + j
            inv[t, j] = fill[e]
            fill[e] += 1
    return counts.astype(np.int32), offsets.astype(np.int32), perm.astype(np.int32), inv.astype(np.int32)


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def swiglu(gate_up, down, x: np.ndarray, rows=None) -> np.ndarray:
    """One SwiGLU expert on a batch of fp16 inputs.

    g = G x, u = U x, a = fp16(silu(g) * u), y = D a (not rounded).
    ``gate_up`` holds the gate rows then the up rows (F each); ``rows``
    optionally selects the row range [r0, r1) of a stacked matrix.
    [UOCR] "Quantizzazione": dequantisation is fused into the SwiGLU; the
    intermediate is an fp16 activation.
    """
    gu = gemv_qmat(gate_up, x)
    F = gu.shape[-1] // 2
    a = f16(silu(gu[..., :F]) * gu[..., F:])
    return gemv_qmat(down, a)


class _Rows:
    """Row range [r0, r1) of a stacked matrix, as a matrix object."""

    def __init__(self, m, r0, r1):
        per_row = m.data.size // m.n
        self.fmt, self.n, self.k = m.fmt, r1 - r0, m.k
        self.data = m.data[r0 * per_row:r1 * per_row]


def expert_mats(lay, e: int, shared: bool = False):
    """(gate_up, down) of routed expert ``e`` (or shared expert ``e``)."""
    gu = lay.sh_gate_up if shared else lay.exp_gate_up
    dn = lay.sh_down if shared else lay.exp_down
    two_f = gu.n // (lay_n_shared(lay) if shared else lay_n_experts(lay))
    H = dn.n // (lay_n_shared(lay) if shared else lay_n_experts(lay))
    return _Rows(gu, e * two_f, (e + 1) * two_f), _Rows(dn, e * H, (e + 1) * H)


def lay_n_experts(lay) -> int:
    return lay.router.n


def lay_n_shared(lay) -> int:
    return 0 if lay.sh_gate_up is None else lay.sh_gate_up.n // (2 * lay.sh_down.k)


def moe(lay, x: np.ndarray, top_k: int, forced_idx: np.ndarray | None = None):
    """DeepSeek-V2-style MoE on fp16 inputs x[T][H] (not rounded at the end).

    moe(x_t) = sum_s shared_s(x_t) + sum_j w_tj * expert_{idx_tj}(x_t), summed
    shared first, then ranks 0..k-1.  [UOCR] "Il decoder e il Mixture of
    Experts": 64 routed experts, top-6 routing and two shared experts; the
    runtime routes, groups per expert, runs the projections and recombines.

    Returns (out[T][H], idx[T][k], w[T][k], logits[T][E] float64).
    ``forced_idx`` replaces the chosen experts (weights are still this
    side's renormalised probabilities).
    """
    x = np.asarray(x, np.float64)
    T = x.shape[0]
    logits = gemv_qmat(lay.router, x)
    bias = None if lay.router_bias is None else np.asarray(lay.router_bias, np.float64)
    idx = np.zeros((T, top_k), np.int32)
    w = np.zeros((T, top_k))
    for t in range(T):
        if forced_idx is not None and forced_idx[t][0] >= 0:
            idx[t] = forced_idx[t]
            w[t] = route_forced(logits[t], idx[t], bias)
        else:
            idx[t], w[t] = route(logits[t], top_k, bias)
    E = lay_n_experts(lay)
    H = x.shape[1]
    routed = np.zeros((T, top_k, H))
    for e in range(E):
        sel = np.argwhere(idx == e)
        if sel.size == 0:
            continue
        gu, dn = expert_mats(lay, e)
        y = swiglu(gu, dn, x[sel[:, 0]])
        routed[sel[:, 0], sel[:, 1]] = y
    out = np.zeros((T, H))
    for s in range(lay_n_shared(lay)):
        gu, dn = expert_mats(lay, s, shared=True)
        out = out + swiglu(gu, dn, x)
    for j in range(top_k):
        out = out + w[:, j:j + 1] * routed[:, j]
    return out, idx, w, logits


# -----------------------------------------------------------------------------
# Ring KV cache
# -----------------------------------------------------------------------------

def kv_quantise(x: np.ndarray):
    """INT8 KV cache entry of one key or value row (the last axis).

    [FALCON] "How it is meant to be run": the project's CPU service keeps an
    INT8 KV cache; its format is not given.  Reading: symmetric int8 codes with
    one fp16 scale per row (per row of the batch, head and position):
    s = fp16(max|x| / 127), the division in float32; q = round half away from
    zero of float32(x) / float32(s) (float32 division), clamped to [-127, 127];
    a row of zeros has s = 0 and q = 0.  The codes are an integer decision, so
    it is taken in float32, the precision the kernel computes it in.

    Returns (q int8 [..., D], s float16 [...]).
    """
    x32 = np.asarray(x, np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    s = (amax / np.float32(127)).astype(np.float16)
    s32 = s.astype(np.float32)[..., None]
    safe = np.where(s32 > 0, s32, np.float32(1))
    y = np.where(s32 > 0, x32 / safe, np.float32(0)).astype(np.float64)
    q = np.sign(y) * np.floor(np.abs(y) + 0.5)
    return np.clip(q, -127, 127).astype(np.int8), s


def kv_dequant(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Values of INT8 KV cache rows: s * q (exact in float64)."""
    return np.asarray(q, np.float64) * np.asarray(s, np.float64)[..., None]


def ring_slot(t: int, ring_cap: int) -> int:
    """Slot of generated token t in the ring: t mod capacity.

    [UOCR] "Il decoder e il Mixture of Experts": generated tokens live in a
    128-token ring buffer so decode memory stays bounded.
    """
    return t % ring_cap


def window(prefix_len: int, prefix_cap: int, t: int, ring_cap: int) -> np.ndarray:
    """Cache indices a row attends to at generation index t (new token included).

    The fixed prefix [0, prefix_len) plus the ring slots written so far,
    [prefix_cap, prefix_cap + min(t + 1, ring_cap)).  Reading: the ring's
    capacity counts the current token, so after wrapping the window holds the
    last ``ring_cap`` generated tokens.  [NCNN] 3.2: the cache length always
    equals the real token count, so no masked placeholder keys are read.
    """
    n_ring = min(t + 1, ring_cap)
    return np.concatenate([np.arange(prefix_len), prefix_cap + np.arange(n_ring)]).astype(np.int64)


# -----------------------------------------------------------------------------
# The decode step
# -----------------------------------------------------------------------------

class StepResult:
    def __init__(self):
        self.tok = None            # int32 [R] (or None without LM head)
        self.hidden = None         # float64 [R][H] residual after the last layer
        self.layer_in = []         # per layer: float64 [R][H] residual entering the layer
        self.final_x = None        # float64 [R][H] normalised input of the LM head (fp16 values)
        self.lm_top2 = None        # float64 [R][2] best and second logits (float32 values)
        self.topk_idx = []         # per MoE layer: int32 [R][k]
        self.topk_w = []           # per MoE layer: float64 [R][k]
        self.router_gap = []       # per MoE layer: float64 [R]
        self.router_logits = []    # per MoE layer: float64 [R][E]
        self.new_k = []            # per layer: float64 [R][NH][D] (fp16 values)
        self.new_v = []
        self.attn_out = []         # per layer: float64 [R][NH*D] (fp16 values)


def attention_block(lay, dims, h, kc, vc, prefix_len, t, res: StepResult | None = None, ks=None, vs=None):
    """Pre-norm attention with the ring cache for one row; returns new h.

    kc, vc: this row's and layer's caches [NH][prefix_cap + ring_cap][D], fp16
    arrays, updated in place at ring slot t mod ring_cap.  [FALCON] "The KV
    cache is an INPUT": the step only reads the cache and contributes the new
    token's keys and values.  With ``ks``, ``vs`` (fp16 [NH][cap]) the caches
    are INT8 (``kv_quantise``): the new token is stored quantised, and the
    attention reads every key and value, the new one included, as stored.
    """
    H, NH, D = dims.hidden, dims.n_heads, dims.head_dim
    x = f16(rmsnorm(h, lay.attn_norm, dims.norm_eps))
    qkv = gemv_qmat(lay.wqkv, x[None])[0]
    q = qkv[:NH * D].reshape(NH, D)
    k = qkv[NH * D:2 * NH * D].reshape(NH, D)
    v = qkv[2 * NH * D:].reshape(NH, D)
    pos = prefix_len + t
    q = f16(rope(q, pos, dims.rope_theta))
    k = f16(rope(k, pos, dims.rope_theta))
    v = f16(v)
    slot = dims.prefix_cap + ring_slot(t, dims.ring_cap)
    idx = window(prefix_len, dims.prefix_cap, t, dims.ring_cap)
    o = np.zeros((NH, D))
    if ks is None:
        kc[:, slot] = k.astype(np.float16)
        vc[:, slot] = v.astype(np.float16)
        for hh in range(NH):
            o[hh] = attention(q[hh], kc[hh, idx], vc[hh, idx], 1.0 / np.sqrt(D))
    else:
        kc[:, slot], ks[:, slot] = kv_quantise(k)
        vc[:, slot], vs[:, slot] = kv_quantise(v)
        for hh in range(NH):
            o[hh] = attention(q[hh], kv_dequant(kc[hh, idx], ks[hh, idx]), kv_dequant(vc[hh, idx], vs[hh, idx]),
                              1.0 / np.sqrt(D))
    o = f16(o.reshape(-1))
    h = h + gemv_qmat(lay.wo, o[None])[0]
    if res is not None:
        res.new_k[-1].append(k)
        res.new_v[-1].append(v)
        res.attn_out[-1].append(o)
    return h


def dense_mlp_block(lay, dims, h):
    """h + W_d fp16(silu(W_g x) * W_u x) with x the pre-FFN RMSNorm of h.
    [UOCR] "Il decoder e il Mixture of Experts": layer 0 uses a dense MLP."""
    x = f16(rmsnorm(h, lay.ffn_norm, dims.norm_eps))
    return h + swiglu(lay.dense_gate_up, lay.dense_down, x[None])[0]


def decode_step(model, state, tok_in=None, hidden_in=None, forced_topk=None,
                with_lm: bool = True, rows=None) -> StepResult:
    """One autoregressive decode step of the whole decoder, for every row.

    [UOCR] "Il decoder e il Mixture of Experts": 12 layers, hidden 1280,
    10 heads of 128; layer 0 dense, layers 1-11 MoE; activations in fp16; new
    keys/values appended to the cache (the 128-slot ring); the step ends with an
    argmax over the language head.  [FALCON] "How it is meant to be run": rows
    of one round share the weights and nothing else.

    ``state`` (synth.State) is updated in place: ring slots written and
    gen_index incremented.  ``rows`` restricts the step to a subset of rows
    (rows are independent; routing of a row does not depend on the others).
    ``forced_topk`` [n_moe_layers][R][k] (entries < 0: not forced) replaces the
    routing; ``tok_in`` [R] or ``hidden_in`` [R][H] is the input.
    """
    dims = model.dims
    R = state.prefix_len.size
    rows = list(range(R)) if rows is None else list(rows)
    res = StepResult()
    if tok_in is not None:
        h = embed_rows(model, np.asarray(tok_in)[rows])
    else:
        h = f32(np.asarray(hidden_in, np.float64)[rows])
    moe_l = 0
    for l, lay in enumerate(model.layers):
        res.layer_in.append(h.copy())
        res.new_k.append([])
        res.new_v.append([])
        res.attn_out.append([])
        k8 = getattr(state, "k_scale", None) is not None
        for i, r in enumerate(rows):
            h[i] = attention_block(lay, dims, h[i], state.k_cache[l, r], state.v_cache[l, r],
                                   int(state.prefix_len[r]), int(state.gen_index[r]), res,
                                   state.k_scale[l, r] if k8 else None, state.v_scale[l, r] if k8 else None)
        res.new_k[-1] = np.array(res.new_k[-1])
        res.new_v[-1] = np.array(res.new_v[-1])
        res.attn_out[-1] = np.array(res.attn_out[-1])
        if lay.is_moe:
            x = f16(rmsnorm(h, lay.ffn_norm, dims.norm_eps))
            forced = None if forced_topk is None else np.asarray(forced_topk[moe_l])[rows]
            out, idx, w, logits = moe(lay, x, dims.top_k, forced)
            h = h + out
            res.topk_idx.append(idx)
            res.topk_w.append(w)
            res.router_logits.append(logits)
            res.router_gap.append(np.array([topk_gap(lg, dims.top_k) for lg in logits]))
            moe_l += 1
        else:
            for i in range(len(rows)):
                h[i] = dense_mlp_block(lay, dims, h[i])
    res.hidden = h
    if with_lm and model.lm_head is not None:
        x = f16(rmsnorm(h, model.final_norm, dims.norm_eps))
        res.final_x = x
        z = f32(gemv_qmat(model.lm_head, x))
        res.tok = np.array([argmax_lowest(zr) for zr in z], np.int32)
        top2 = np.sort(z, axis=1)[:, ::-1][:, :2]
        res.lm_top2 = top2
    for r in rows:
        state.gen_index[r] += 1
    return res


class PrefillResult:
    def __init__(self):
        self.tok = None          # int32: argmax at the last position (or None without LM head)
        self.lm_top2 = None      # float64 [2]: best and second logit there (float32 values)
        self.hidden = None       # float64 [P][H]: residual after the last layer
        self.k = []              # per layer: float64 [NH][P][D] (fp16 values), cache indices 0..P-1
        self.v = []
        self.topk_idx = []       # per MoE layer: int32 [P][k]
        self.topk_w = []         # per MoE layer: float64 [P][k]
        self.router_gap = []     # per MoE layer: float64 [P]
        self.kq, self.ks = [], []  # INT8 caches: per layer codes int8 [NH][P][D], scales fp16 [NH][P]
        self.vq, self.vs = [], []


def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Causal self-attention of one head over P positions: query i attends
    keys 0..i.  S = scale * Q K^T with the entries above the diagonal masked
    out, softmax per row, O = softmax(S) V.

    [NCNN] 3.2: prefill and incremental decoding use causal masks of
    different shapes; the prompt pass sees every earlier position of the
    prompt and itself.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    P = q.shape[0]
    s = (q @ k.T) * scale
    s[np.triu_indices(P, 1)] = -np.inf
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return (e @ v) / e.sum(axis=1, keepdims=True)


def prefill(model, P: int, tok=None, emb=None, forced_topk=None, with_lm: bool = True,
            int8_kv: bool = False) -> PrefillResult:
    """The prompt pass of one row: P positions through every layer at once.

    [UOCR] (the model needs a prefill before token-by-token generation;
    "Il decoder e il Mixture of Experts" for the layer stack) and [NCNN] 3.2
    (prefill with a causal mask, then one new token per decode call reusing
    the cache of every layer).  Per layer: x = fp16(RMSNorm(h)); q, k, v from
    the QKV projection, RoPE at the linear positions 0..P-1 ([NCNN] 3.3: the
    current linear position), k and v are what the cache keeps at indices
    0..P-1; causal attention; the O projection added to the residual; then
    the dense SwiGLU or the MoE on fp16(RMSNorm(h)) added to the residual.
    The pass ends with the language-head argmax at the last position, the
    first generated token.  Readings: the input is either token ids (the
    embedding table) or the P rows of fp16 input features (``emb``, e.g. the
    image features spliced into the prompt); storage points as in decode.

    ``forced_topk`` [n_moe][P][k] (rows < 0: not forced) replaces the routing.
    With ``int8_kv`` the cache is INT8 (``kv_quantise``): keys and values are
    stored quantised and the attention reads them as stored, as in decode.
    """
    dims = model.dims
    NH, D, eps, theta = dims.n_heads, dims.head_dim, dims.norm_eps, dims.rope_theta
    res = PrefillResult()
    if tok is not None:
        h = embed_rows(model, np.asarray(tok)[:P])
    else:
        h = np.asarray(emb, np.float64)[:P].copy()
    pos = np.arange(P, dtype=np.float64)[:, None]
    moe_l = 0
    for lay in model.layers:
        x = f16(rmsnorm(h, lay.attn_norm, eps))
        qkv = gemv_qmat(lay.wqkv, x)
        q = f16(rope(qkv[:, :NH * D].reshape(P, NH, D), pos, theta))
        k = f16(rope(qkv[:, NH * D:2 * NH * D].reshape(P, NH, D), pos, theta))
        v = f16(qkv[:, 2 * NH * D:].reshape(P, NH, D))
        ka, va = k, v
        if int8_kv:
            kq, ks = kv_quantise(k)
            vq, vs = kv_quantise(v)
            ka, va = kv_dequant(kq, ks), kv_dequant(vq, vs)
            res.kq.append(kq.transpose(1, 0, 2).copy())
            res.ks.append(ks.T.copy())
            res.vq.append(vq.transpose(1, 0, 2).copy())
            res.vs.append(vs.T.copy())
        o = np.zeros((P, NH, D))
        for hh in range(NH):
            o[:, hh] = causal_attention(q[:, hh], ka[:, hh], va[:, hh], 1.0 / np.sqrt(D))
        h = h + gemv_qmat(lay.wo, f16(o.reshape(P, NH * D)))
        res.k.append(k.transpose(1, 0, 2).copy())
        res.v.append(v.transpose(1, 0, 2).copy())
        x = f16(rmsnorm(h, lay.ffn_norm, eps))
        if lay.is_moe:
            forced = None if forced_topk is None else np.asarray(forced_topk[moe_l])[:P]
            out, idx, w, logits = moe(lay, x, dims.top_k, forced)
            h = h + out
            res.topk_idx.append(idx)
            res.topk_w.append(w)
            res.router_gap.append(np.array([topk_gap(lg, dims.top_k) for lg in logits]))
            moe_l += 1
        else:
            h = h + swiglu(lay.dense_gate_up, lay.dense_down, x)
    res.hidden = h
    if with_lm and model.lm_head is not None:
        x = f16(rmsnorm(h[P - 1:P], model.final_norm, eps))
        z = f32(gemv_qmat(model.lm_head, x))[0]
        res.tok = np.int32(argmax_lowest(z))
        res.lm_top2 = np.sort(z)[::-1][:2]
    return res


class _OneRow:
    """Decode state of one row (the attributes decode_step reads)."""

    def __init__(self, dims, P: int, int8_kv: bool = False):
        cap = dims.prefix_cap + dims.ring_cap
        shape = (dims.n_layers, 1, dims.n_heads, cap, dims.head_dim)
        self.prefix_len = np.array([P], np.int32)
        self.gen_index = np.zeros(1, np.int32)
        self.k_cache = np.zeros(shape, np.int8 if int8_kv else np.float16)
        self.v_cache = np.zeros(shape, np.int8 if int8_kv else np.float16)
        self.k_scale = np.zeros(shape[:4], np.float16) if int8_kv else None
        self.v_scale = np.zeros(shape[:4], np.float16) if int8_kv else None


def generate(model, P: int, tok=None, emb=None, max_new: int = 1, eos=(), keep_eos: bool = False,
             int8_kv: bool = False):
    """Greedy generation for one request: the prompt pass, then decode steps
    that feed each token back, until a token of the EOS set or max_new tokens.

    [NCNN] 3.2 (prefill, then one new token per decode call reusing the
    cache) and 3.5 (generation stops at any token of the EOS set before it is
    handed out; a debug mode keeps the end token for comparisons: keep_eos).
    The prompt's keys and values fill cache indices 0..P-1 and decoding
    continues at prefix_len = P, generation index 0.  ``int8_kv``: the cache
    is INT8 throughout (``kv_quantise``).

    Returns (tokens, stop, gaps): stop 1 = EOS, 2 = max_new; gaps[i] is this
    side's top-2 logit gap behind token i (near-ties admit other answers).
    """
    dims = model.dims
    assert 1 <= P <= dims.prefix_cap, "the prompt fills the prefix region"
    pre = prefill(model, P, tok=tok, emb=emb, int8_kv=int8_kv)
    st = _OneRow(dims, P, int8_kv)
    for l in range(dims.n_layers):
        if int8_kv:
            st.k_cache[l, 0][:, :P], st.k_scale[l, 0][:, :P] = pre.kq[l], pre.ks[l]
            st.v_cache[l, 0][:, :P], st.v_scale[l, 0][:, :P] = pre.vq[l], pre.vs[l]
        else:
            st.k_cache[l, 0][:, :P] = pre.k[l].astype(np.float16)
            st.v_cache[l, 0][:, :P] = pre.v[l].astype(np.float16)
    out, gaps = [], []
    t, gap = int(pre.tok), float(pre.lm_top2[0] - pre.lm_top2[1])
    eos = set(int(e) for e in eos)
    while True:
        if t in eos:
            if keep_eos:
                out.append(t)
                gaps.append(gap)
            return out, 1, gaps
        out.append(t)
        gaps.append(gap)
        if len(out) >= max_new:
            return out, 2, gaps
        res = decode_step(model, st, tok_in=np.array([t], np.int32))
        t, gap = int(res.tok[0]), float(res.lm_top2[0, 0] - res.lm_top2[0, 1])


def embed_rows(model, tok) -> np.ndarray:
    """Embedding lookup: row ``tok[i]`` of the table, as float64.

    [UOCR] "In sintesi": the decode loop starts from the embedding lookup, and
    the mixed profiles dequantise inside the kernels.  The fp16 table is read
    as is; a quantised table (``model.embed_q``, any of the four formats) gives
    each looked-up row dequantised exactly as ``dequant`` defines it.
    """
    tok = np.asarray(tok).reshape(-1)
    if getattr(model, "embed", None) is not None:
        return model.embed[tok].astype(np.float64)
    m = model.embed_q
    row_bytes = m.k * 2 if m.fmt == F16 else (m.k // QK) * _BLOCK_BYTES[m.fmt]
    data = np.asarray(m.data, np.uint8).reshape(-1)
    return np.stack([dequant(m.fmt, data[int(t) * row_bytes:(int(t) + 1) * row_bytes], 1, m.k)[0] for t in tok])


def argmax_lowest(z: np.ndarray) -> int:
    """Index of the largest value; ties go to the lowest index.
    [UOCR] the decode loop ends with an argmax over the language head;
    [NCNN] 3.4: greedy selection.  NaN never wins."""
    z = np.asarray(z, np.float64)
    best, bi = -np.inf, -1
    for i in range(z.size):
        if z[i] > best:
            best, bi = z[i], i
    return bi


# -----------------------------------------------------------------------------
# Sink-augmented attention block with int8-asymmetric projections
# -----------------------------------------------------------------------------

def sink_attention_block(wqkv, wo, x, kc, vc, cache_len: int, sink, n_heads: int,
                         head_dim: int, theta: float):
    """One row of the sink-augmented decode attention with u8-asymmetric weights.

    [FALCON]: 8 heads; keys and queries carry one extra constant lane so the
    sink acts as one more key with value 0, seeded by the host at cache index
    0; the cache is an input and the step returns the new token's keys and
    values; weights are INT8_ASYM.  Readings: the cache length ``cache_len``
    counts the sink slot, the new token is appended at index ``cache_len``
    with RoPE position cache_len - 1 (the real tokens before it), and the
    score scale is 1/sqrt(head_dim) (the extra lane is a device, not a
    dimension).  No norm and no residual.

    x: fp16 [H]; kc, vc: fp16 [NH][cap][D] updated in place at cache_len;
    sink: the per-head sink logits [NH].
    Returns (y[H] fp16 values, new_k, new_v, o).
    """
    NH, D = n_heads, head_dim
    qkv = gemv_qmat(wqkv, np.asarray(x, np.float64)[None])[0]
    q = qkv[:NH * D].reshape(NH, D)
    k = qkv[NH * D:2 * NH * D].reshape(NH, D)
    v = qkv[2 * NH * D:].reshape(NH, D)
    pos = cache_len - 1
    q = f16(rope(q, pos, theta))
    k = f16(rope(k, pos, theta))
    v = f16(v)
    kc[:, cache_len] = k.astype(np.float16)
    vc[:, cache_len] = v.astype(np.float16)
    o = np.zeros((NH, D))
    for hh in range(NH):
        o[hh] = attention(q[hh], kc[hh, :cache_len + 1], vc[hh, :cache_len + 1],
                          1.0 / np.sqrt(D), sink=float(sink[hh]), sink_index=0)
    o = f16(o.reshape(-1))
    y = f16(gemv_qmat(wo, o[None])[0])
    return y, k, v, o
