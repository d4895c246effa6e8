"""Pins of the CPU oracle against facts fixed outside it.

Each test states what it pins and why a plausible mistake in the oracle (a
dropped term, a wrong sign or index, a transposed operand, an off-by-one in
the ring window) would fail it.  None of these tests re-type the oracle's
formula: they use hand-built blocks, closed forms, identities, brute force or
constructions whose outcome is known in advance.
"""
import itertools
import os

import numpy as np
import pytest

import oracle as O
from tests.blocks import enc_f16, enc_q4_0, enc_q8_0, enc_u8a

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FMT = {"F16": O.F16, "Q8_0": O.Q8_0, "Q4_0": O.Q4_0, "U8A_G32": O.U8A_G32}


# -----------------------------------------------------------------------------
# fp16 storage rounding
# -----------------------------------------------------------------------------

def test_f16_roundtrip_all_patterns():
    """Every finite binary16 value survives f16() unchanged (no FTZ, no drift)."""
    h = np.arange(65536, dtype=np.uint16).view(np.float16)
    v = h.astype(np.float64)
    fin = np.isfinite(v)
    assert np.array_equal(O.f16(v[fin]), v[fin])
    # subnormals kept
    assert O.f16(2.0 ** -24) == 2.0 ** -24
    assert O.f16(3 * 2.0 ** -24) == 3 * 2.0 ** -24


def test_f16_ties_to_even_and_single_rounding():
    """Halfway cases go to even; rounding is done once, directly from double."""
    assert O.f16(1 + 2.0 ** -11) == 1.0                      # tie -> even (down)
    assert O.f16(1 + 3 * 2.0 ** -11) == 1 + 2.0 ** -9        # tie -> even (up)
    # Just above a tie: a double rounding through float32 would land on the tie
    # and then round to even (1.0); one correct rounding gives 1 + 2^-10.
    assert O.f16(1 + 2.0 ** -11 + 2.0 ** -40) == 1 + 2.0 ** -10
    assert np.isinf(O.f16(65520.0)) and O.f16(65519.0) == 65504.0


# -----------------------------------------------------------------------------
# Block formats
# -----------------------------------------------------------------------------

def _golden_blocks():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            tag, _, rest = line.partition(" ")
            if tag == "case":
                name, fmt = rest.split()
                cur = {"name": name, "fmt": FMT[fmt]}
                cases.append(cur)
            elif tag == "hex":
                cur["bytes"] = bytes.fromhex(rest.replace(" ", ""))
            elif tag == "expect":
                cur["expect"] = np.array([float(t) for t in rest.split()])
    return cases


@pytest.mark.parametrize("case", _golden_blocks(), ids=lambda c: c["name"])
def test_dequant_hand_built_blocks(case):
    """Exact dequantised values of hand-built blocks (tests/golden/blocks.txt)."""
    size = {O.Q8_0: 34, O.Q4_0: 18, O.U8A_G32: 36}[case["fmt"]]
    assert len(case["bytes"]) == size and case["expect"].size == 32
    w = O.dequant(case["fmt"], np.frombuffer(case["bytes"], np.uint8), 1, 32)[0]
    assert np.array_equal(w, case["expect"])


def test_dequant_block_order_along_k():
    """Blocks run along k within a row and rows follow each other: a matrix of
    2 rows x 2 blocks with distinct scales puts each scale where it belongs."""
    d = [[1.0, 2.0], [4.0, 8.0]]
    q = np.full((2, 64), 9)          # code 9 -> value 1 * d
    w = O.dequant(O.Q4_0, enc_q4_0(d, q).data, 2, 64)
    assert np.array_equal(w[0, :32], np.full(32, 1.0)) and np.array_equal(w[0, 32:], np.full(32, 2.0))
    assert np.array_equal(w[1, :32], np.full(32, 4.0)) and np.array_equal(w[1, 32:], np.full(32, 8.0))


def test_embed_rows_quantised_table():
    """Embedding lookup from a quantised table: row t of a Q4_0 table whose row t
    has scales (t+1, 2(t+1)) and every code 9 is (t+1) over the first block and
    2(t+1) over the second; an fp16 table gives its rows as stored; the Q8_0 and
    int8-asymmetric tables give the rows of their dense dequantisation."""
    V, H = 7, 64

    class M:
        embed = None
    m = M()
    d = [[t + 1.0, 2.0 * (t + 1.0)] for t in range(V)]
    m.embed_q = enc_q4_0(d, np.full((V, H), 9))
    tok = np.array([6, 0, 3, 3])
    h = O.embed_rows(m, tok)
    for i, t in enumerate(tok):
        assert np.array_equal(h[i, :32], np.full(32, t + 1.0)) and np.array_equal(h[i, 32:], np.full(32, 2.0 * (t + 1)))
    rng = np.random.default_rng(5)
    w = rng.standard_normal((V, H)) * 0.1
    m.embed_q = enc_f16(w)
    assert np.array_equal(O.embed_rows(m, tok), O.f16(w)[tok])
    for enc in (enc_q8_0, enc_u8a):
        if enc is enc_q8_0:
            m.embed_q = enc(np.abs(w[:, ::32]) + 0.01, rng.integers(-128, 128, (V, H)))
        else:
            m.embed_q = enc(np.abs(w[:, ::32]) + 0.01, np.full((V, 2), 3.0), rng.integers(0, 256, (V, H)))
        dense = O.dequant(m.embed_q.fmt, m.embed_q.data, V, H)
        assert np.array_equal(O.embed_rows(m, tok), dense[tok])
    m2 = M()
    m2.embed = O.f16(w).astype(np.float16)
    assert np.array_equal(O.embed_rows(m2, tok), O.f16(w)[tok])


def test_quantiser_roundtrip_error_bound():
    """Draws quantised by the input generator dequantise to within half a step
    (Q8_0, Q4_0, int8-asymmetric) of the drawn values, plus what the fp16
    rounding of the scale can push past the clamp (at most codes * 2^-11
    steps), and the F16 form is the drawn value rounded once."""
    import synth
    n, k, std = 16, 256, 0.02
    stream = synth.stream_id(5, "roundtrip")
    w = synth.normal_f64(stream, (n, k), 0.0, std)
    for fmt, steps in ((O.Q8_0, 127.0), (O.Q4_0, 7.0)):
        m = synth.random_qmat(fmt, stream, n, k, std)
        deq = O.dequant(fmt, m.data, n, k)
        blk = w.reshape(n, k // 32, 32)
        d = O.f16(np.abs(blk).max(-1) / steps)
        err = np.abs(deq.reshape(n, k // 32, 32) - blk)
        if fmt == O.Q4_0:   # the top code is 7 of [-8, 7]: the clamp side may lose up to one step
            assert np.all(err <= d[..., None] * 1.0 + 1e-12)
        else:
            assert np.all(err <= d[..., None] * (0.5 + 127 * 2.0 ** -11) + 1e-12)
    m = synth.random_qmat(O.U8A_G32, stream, n, k, std)
    deq = O.dequant(O.U8A_G32, m.data, n, k)
    blk = w.reshape(n, k // 32, 32)
    s = O.f16((blk.max(-1) - blk.min(-1)) / 255)
    assert np.all(np.abs(deq.reshape(blk.shape) - blk) <= s[..., None] * (0.5 + 255 * 2.0 ** -11) + 1e-12)
    m = synth.random_qmat(O.F16, stream, n, k, std)
    assert np.array_equal(O.dequant(O.F16, m.data, n, k), O.f16(w))


# -----------------------------------------------------------------------------
# GEMV
# -----------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", ["Q8_0", "Q4_0", "U8A_G32", "F16"])
def test_gemv_permutation_rows(fmt):
    """W with one weight c_n per row at column pi(n): y[r][n] = c_n * x[r][pi(n)]
    exactly.  Catches a transposed W, a wrong block/row stride or a lost scale."""
    rng = np.random.default_rng(1)
    n, k = 48, 96
    pi = rng.permutation(k)[:n]
    c = 2.0 ** rng.integers(-3, 3, size=n)
    x = O.f16(rng.standard_normal((3, k)))
    if fmt == "Q8_0":
        q = np.zeros((n, k), int)
        q[np.arange(n), pi] = 1
        d = np.repeat(c[:, None], k // 32, 1)
        m = enc_q8_0(d, q)
    elif fmt == "Q4_0":
        q = np.full((n, k), 8)
        q[np.arange(n), pi] = 9
        d = np.repeat(c[:, None], k // 32, 1)
        m = enc_q4_0(d, q)
    elif fmt == "U8A_G32":
        q = np.full((n, k), 100)
        q[np.arange(n), pi] = 101
        s = np.repeat(c[:, None], k // 32, 1)
        m = enc_u8a(s, np.full_like(s, 100.0), q)
    else:
        w = np.zeros((n, k))
        w[np.arange(n), pi] = c
        m = enc_f16(w)
    y = O.gemv_qmat(m, x)
    assert np.array_equal(y, c[None, :] * x[:, pi])


def test_gemv_matches_scalar_brute_force():
    """Small random Q4_0 GEMV equals a scalar loop over (row, block, element)
    that reads the nibbles straight from the encoded bytes."""
    rng = np.random.default_rng(2)
    n, k = 5, 64
    q = rng.integers(0, 16, size=(n, k))
    d = O.f16(rng.uniform(0.01, 0.1, size=(n, k // 32)))
    m = enc_q4_0(d, q)
    x = O.f16(rng.standard_normal(k))
    y = O.gemv_qmat(m, x[None])[0]
    raw = m.data.reshape(n, k // 32, 18)
    for r in range(n):
        acc = 0.0
        for b in range(k // 32):
            dd = float(np.frombuffer(raw[r, b, :2].tobytes(), np.float16)[0])
            for j in range(16):
                lo, hi = raw[r, b, 2 + j] & 15, raw[r, b, 2 + j] >> 4
                acc += dd * (int(lo) - 8) * x[b * 32 + j] + dd * (int(hi) - 8) * x[b * 32 + j + 16]
        assert abs(acc - y[r]) <= 1e-12 * max(1.0, abs(acc))


# -----------------------------------------------------------------------------
# RMSNorm, RoPE
# -----------------------------------------------------------------------------

def test_rmsnorm_constant_vector():
    """x = c * 1 -> y = gamma * c / sqrt(c^2 + eps) (closed form)."""
    gamma = np.linspace(0.5, 1.5, 8)
    for c in (0.3, -2.0, 7.0):
        y = O.rmsnorm(np.full(8, c), gamma, 1e-6)
        assert np.allclose(y, gamma * c / np.sqrt(c * c + 1e-6), rtol=1e-15, atol=0)
    # the mean is over the vector, not the sum: [3, 4] has rms 3.5355...
    y = O.rmsnorm(np.array([3.0, 4.0]), np.ones(2), 0.0)
    assert np.allclose(y, np.array([3.0, 4.0]) / np.sqrt(12.5), rtol=1e-15)


def test_rope_closed_forms():
    """pos = 0 is the identity; D = 4, theta = 100, pos = 1 gives the rotation
    angles (1, 0.1) on the lane pairs (0, 2) and (1, 3) (rotate-half)."""
    x = np.array([1.0, 2.0, 3.0, 4.0])
    assert np.array_equal(O.rope(x, 0, 100.0), x)
    y = O.rope(np.array([1.0, 0.0, 0.0, 0.0]), 1, 100.0)
    assert np.allclose(y, [np.cos(1), 0, np.sin(1), 0], atol=1e-15)
    y = O.rope(np.array([0.0, 1.0, 0.0, 0.0]), 1, 100.0)
    assert np.allclose(y, [0, np.cos(0.1), 0, np.sin(0.1)], atol=1e-15)
    y = O.rope(np.array([0.0, 0.0, 1.0, 0.0]), 1, 100.0)
    assert np.allclose(y, [-np.sin(1), 0, np.cos(1), 0], atol=1e-15)


def test_rope_relative_position_property():
    """<R_m q, R_n k> depends only on m - n, and RoPE preserves pair norms."""
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    a = O.rope(q, 1107, 1e4) @ O.rope(k, 1100, 1e4)
    b = O.rope(q, 7, 1e4) @ O.rope(k, 0, 1e4)
    assert abs(a - b) < 1e-9
    y = O.rope(q, 555, 1e4)
    assert np.allclose(y[:64] ** 2 + y[64:] ** 2, q[:64] ** 2 + q[64:] ** 2, rtol=1e-12)
    # a 64-lane rotation on a 65-wide vector leaves the 65th lane alone
    z = np.append(rng.standard_normal(64), 1.0)
    assert O.rope(z, 9, 1e4, rot_dim=64)[64] == 1.0


# -----------------------------------------------------------------------------
# Attention and the sink
# -----------------------------------------------------------------------------

def test_attention_special_cases():
    rng = np.random.default_rng(4)
    q = rng.standard_normal(16)
    K = rng.standard_normal((1, 16))
    V = rng.standard_normal((1, 8))
    assert np.allclose(O.attention(q, K, V, 0.25), V[0], rtol=1e-15)     # one key -> its value
    K = np.zeros((5, 16))
    V = rng.standard_normal((5, 8))
    assert np.allclose(O.attention(q, K, V, 0.25), V.mean(0), rtol=1e-14)  # equal scores -> mean
    # one key far above the rest -> that key's value
    K = np.zeros((4, 16))
    K[2] = 100 * q / np.linalg.norm(q)
    assert np.allclose(O.attention(q, K, V[:4], 1.0), V[2], rtol=1e-12)


def test_attention_softmax_by_hand():
    """Two keys with scores 0 and log 3 -> weights 1/4 and 3/4."""
    q = np.array([1.0, 0.0])
    K = np.array([[0.0, 5.0], [np.log(3.0), -1.0]])
    V = np.array([[4.0], [8.0]])
    assert np.allclose(O.attention(q, K, V, 1.0), [0.25 * 4 + 0.75 * 8], rtol=1e-15)


def test_sink_identity():
    """Softmax with one extra zero-value key of logit sigma equals the plain
    output rescaled by sigmoid(lse - sigma), lse over the real scaled scores
    ([FALCON] paragraph on the attention sink); sigma -> -inf recovers plain."""
    rng = np.random.default_rng(5)
    q = rng.standard_normal(64)
    K = rng.standard_normal((40, 64))
    V = rng.standard_normal((40, 64))
    scale = 1 / 8
    plain = O.attention(q, K, V, scale)
    lse = O.logsumexp(K @ q * scale)
    for sigma in (-1.3, 0.0, 0.7, 2.5):
        with_sink = O.attention(q, K, V, scale, sink=sigma)
        assert np.allclose(with_sink, plain / (1 + np.exp(sigma - lse)), rtol=1e-12)
    assert np.allclose(O.attention(q, K, V, scale, sink=-1e4), plain, rtol=1e-15)


def test_sink_as_65th_lane_equals_sink_logit():
    """The page's construction: queries carry a constant 1 in lane 64, the key
    at cache index 0 carries the sink there (pre-scaled by sqrt(64)) and zero
    elsewhere, its value is 0, other keys have 0 in lane 64.  Plain 65-lane
    attention with scale 1/8 equals the oracle's sink form."""
    rng = np.random.default_rng(6)
    n = 30
    sigma = float(O.f16(0.83))
    q64 = rng.standard_normal(64)
    K64 = rng.standard_normal((n, 64))
    V = rng.standard_normal((n, 64))
    K64[0] = 0.0
    V[0] = 0.0
    q65 = np.append(q64, 1.0)
    K65 = np.concatenate([K64, np.zeros((n, 1))], 1)
    K65[0, 64] = 8.0 * sigma
    literal = O.attention(q65, K65, V, 1 / 8)
    folded = O.attention(q64, K64, V, 1 / 8, sink=sigma, sink_index=0)
    separate = O.attention(q64, K64[1:], V[1:], 1 / 8, sink=sigma)   # sink as an extra key
    # the folded form keeps index 0 (score 0 + sigma, value 0): identical to the extra-key form
    assert np.allclose(literal, folded, rtol=1e-13)
    assert np.allclose(folded, separate, rtol=1e-13)


def _u8a_scaled_identities(scales, H):
    """U8A_G32 matrix [len(scales)*H][H] made of stacked identities, block i
    scaled by scales[i] (s = scale, z = 0, code 1 on the diagonal)."""
    n = len(scales) * H
    q = np.zeros((n, H), np.int64)
    s = np.zeros((n, H // 32))
    for i, sc in enumerate(scales):
        for r in range(H):
            q[i * H + r, r] = 1
            s[i * H + r, :] = sc
    return enc_u8a(s, np.zeros_like(s), q)


def test_sink_block_literal_65_lane_construction():
    """The sink-augmented block against the page's own construction, worked
    out independently ([FALCON] attention-sink paragraph: queries carry a
    constant extra lane, the key at cache index 0 carries the sink logit in
    that lane and its value is 0; the new token's key and value are appended
    after the cache).

    Projections are stacked identities with distinct scales (q = x, k = x/2,
    v = 2x), so the q/k/v slices are known.  Each head's input is nonzero only
    in lane 0, so RoPE moves it within the (0, 32) plane, whose frequency is
    theta^0 = 1: the rotated query is a*(cos p, sin p) for position p.  The
    cached keys sit at known angles in that plane and the cached values are
    one-hot in distinct lanes, so every score and every weight is visible in
    the output.  The expected output is the plain softmax over 65-lane keys
    [0, L] (sink slot, cached keys, new key) with scale 1/8, evaluated here
    from cosines and sines.  A RoPE position of L instead of L - 1, a window
    that drops the new key or a missing sink term each move the output by far
    more than the fp16 rounding allowed below."""
    NH, D, L = 2, 64, 6
    H = NH * D
    wqkv = _u8a_scaled_identities([1.0, 0.5, 2.0], H)
    wo = _u8a_scaled_identities([1.0], H)
    a = np.array([2.0, 1.5])          # lane 0 of each head
    b = np.array([4.0, 3.0])          # magnitude of the cached keys
    phi = np.array([5.0, 1.0, 2.0, 3.0, 4.0])  # angles of cached keys 1..L-1
    sink = np.array([0.75, -0.5])
    x = np.zeros(H)
    x[0], x[D] = a
    cap = L + 1
    kc = np.zeros((NH, cap, D))
    vc = np.zeros((NH, cap, D))
    for h in range(NH):
        for j in range(1, L):
            kc[h, j, 0] = b[h] * np.cos(phi[j - 1])
            kc[h, j, 32] = b[h] * np.sin(phi[j - 1])
            vc[h, j, j] = 1.0 + 0.25 * j
    kc, vc = O.f16(kc), O.f16(vc)
    y, k_new, v_new, _ = O.sink_attention_block(wqkv, wo, x, kc.copy(), vc.copy(), L, sink, NH, D, 10000.0)

    p = L - 1  # real tokens before the new one (the sink slot is not a token)
    f16 = lambda v: np.float64(np.float16(v))
    expect = np.zeros(H)
    for h in range(NH):
        qv = np.zeros(65)
        qv[0], qv[32], qv[64] = f16(a[h] * np.cos(p)), f16(a[h] * np.sin(p)), 1.0
        kn = np.zeros(D)
        kn[0], kn[32] = f16(0.5 * a[h] * np.cos(p)), f16(0.5 * a[h] * np.sin(p))
        assert np.array_equal(k_new[h], kn)
        vn = np.zeros(D)
        vn[0] = f16(2.0 * a[h])
        assert np.array_equal(v_new[h], vn)
        K65 = np.zeros((L + 1, 65))
        V = np.zeros((L + 1, D))
        K65[0, 64] = 8.0 * sink[h]
        K65[1:L, :D] = kc[h, 1:L]
        V[1:L] = vc[h, 1:L]
        K65[L, :D] = kn
        V[L] = vn
        s = K65 @ qv / 8.0
        w = np.exp(s - s.max())
        w /= w.sum()
        expect[h * D:(h + 1) * D] = O.f16(w @ V)
    ulp = np.spacing(np.abs(expect).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(y - expect) <= ulp), np.max(np.abs(y - expect))
    # the new token carries weight (it is attended) and lane 0 is its alone
    assert np.all(np.abs(y[[0, D]]) > 0.1)


# -----------------------------------------------------------------------------
# Near-tie classification
# -----------------------------------------------------------------------------

def test_topk_gap_hand_built():
    """The gap that decides whether two routings are both correct is the
    smallest difference between adjacent ranks 1 .. k+1 of the logits: a
    near-tie between ranks k and k+1 swaps which expert is chosen, one between
    ranks i < k swaps the order of the chosen ones, one below rank k+1 changes
    nothing ([NCNN] section 3.4: a tie rule matters only where the candidates
    are that close)."""
    E, k = 16, 6
    perm = np.random.default_rng(3).permutation(E)

    def place(vals):
        out = np.full(E, -5.0)
        out[perm[:len(vals)]] = vals
        return out

    # only the 6th/7th gap is small
    assert O.topk_gap(place([10, 9, 8, 7, 6, 5, 4.9995, 0]), k) == pytest.approx(5e-4, abs=1e-12)
    # the 2nd/3rd gap is the smallest
    assert O.topk_gap(place([10, 9, 8.9999, 7, 6, 5, 4]), k) == pytest.approx(1e-4, abs=1e-12)
    # a tie below rank k+1 does not count
    assert O.topk_gap(place([10, 9, 8, 7, 6, 5, 4, 3, 3]), k) == pytest.approx(1.0, abs=1e-12)
    # an exact tie at ranks k, k+1
    assert O.topk_gap(place([10, 9, 8, 7, 6, 5, 5]), k) == 0.0
    # the bias is part of the routed logits: all logits equal, the bias separates them
    bias = place([3, 2.5, 2, 1.5, 1, 0.5, 0.4997]) + 5.0
    assert O.topk_gap(np.zeros(E), k, bias) == pytest.approx(3e-4, abs=1e-12)
    # top-1: the gap between the best and the second
    assert O.topk_gap(place([2.0, 1.25]), 1) == pytest.approx(0.75, abs=1e-12)


# -----------------------------------------------------------------------------
# Ring window
# -----------------------------------------------------------------------------

@pytest.mark.parametrize("ring_cap", [4, 128])
def test_ring_equals_linear_window(ring_cap):
    """Writing generated keys g_0..g_t at slot t mod C and attending over the
    oracle's window equals attention over the linear sequence [prefix,
    g_max(0,t-C+1) .. g_t]: while t + 1 <= C that is all generated tokens,
    after wrapping the last C of them."""
    rng = np.random.default_rng(7)
    P_cap, P, D = 9, 6, 16
    gens_k = rng.standard_normal((3 * ring_cap + 2, D))
    gens_v = rng.standard_normal((3 * ring_cap + 2, D))
    pre_k, pre_v = rng.standard_normal((P, D)), rng.standard_normal((P, D))
    q = rng.standard_normal(D)
    cache_k = np.full((P_cap + ring_cap, D), np.nan)
    cache_v = np.full((P_cap + ring_cap, D), np.nan)
    cache_k[:P], cache_v[:P] = pre_k, pre_v
    for t in range(gens_k.shape[0]):
        slot = P_cap + O.ring_slot(t, ring_cap)
        cache_k[slot], cache_v[slot] = gens_k[t], gens_v[t]
        idx = O.window(P, P_cap, t, ring_cap)
        got = O.attention(q, cache_k[idx], cache_v[idx], 0.3)
        lo = max(0, t - ring_cap + 1)
        lin_k = np.concatenate([pre_k, gens_k[lo:t + 1]])
        lin_v = np.concatenate([pre_v, gens_v[lo:t + 1]])
        assert idx.size == P + min(t + 1, ring_cap)
        assert np.allclose(got, O.attention(q, lin_k, lin_v, 0.3), rtol=1e-12)


# -----------------------------------------------------------------------------
# Routing and grouping
# -----------------------------------------------------------------------------

def test_route_brute_force_small():
    """E = 8, k = 3: the chosen set is the 3-subset with the largest total
    probability (brute force over all 56 subsets), ordered by probability;
    weights are the softmax over the chosen logits; sum to 1."""
    rng = np.random.default_rng(8)
    for _ in range(50):
        l = rng.standard_normal(8)
        idx, w = O.route(l, 3)
        p = np.exp(l - l.max()) / np.exp(l - l.max()).sum()
        best = max(itertools.combinations(range(8), 3), key=lambda s: sum(p[list(s)]))
        assert set(idx.tolist()) == set(best)
        assert list(idx) == sorted(best, key=lambda e: -p[e])
        lf = l.astype(np.float32).astype(np.float64)
        ww = np.exp(lf[idx] - lf[idx].max())
        assert np.allclose(w, ww / ww.sum(), rtol=1e-12)
        assert abs(w.sum() - 1) < 1e-15


def test_route_ties_and_top1():
    """Equal logits: the lower expert index wins.  k = 1 is the argmax."""
    l = np.array([0.5, 2.0, 2.0, -1.0, 2.0, 0.0])
    idx, w = O.route(l, 2)
    assert list(idx) == [1, 2] and np.allclose(w, [0.5, 0.5])
    idx, _ = O.route(l, 3)
    assert list(idx) == [1, 2, 4]
    idx, w = O.route(np.array([0.1, 0.9, 0.3]), 1)
    assert list(idx) == [1] and w[0] == 1.0
    # a bias moves the choice: adding 5 to expert 3 selects it first
    idx, _ = O.route(l, 2, bias=np.array([0, 0, 0, 5.0, 0, 0]))
    assert list(idx) == [3, 1]


def test_group_invariants():
    """Counting sort by expert: counts sum to T*k, offsets are the exclusive
    scan, perm is a permutation sorted by (expert, token, rank), and inv
    inverts perm."""
    rng = np.random.default_rng(9)
    T, k, E = 13, 6, 16
    idx = np.array([rng.choice(E, k, replace=False) for _ in range(T)])
    counts, offsets, perm, inv = O.group(idx, E)
    assert counts.sum() == T * k and offsets[0] == 0 and offsets[-1] == T * k
    assert np.array_equal(np.diff(offsets), counts)
    assert sorted(perm.tolist()) == list(range(T * k))
    keys = [(idx[p // k, p % k], p // k, p % k) for p in perm]
    assert keys == sorted(keys)
    for t in range(T):
        for j in range(k):
            assert perm[inv[t, j]] == t * k + j
            e = idx[t, j]
            assert offsets[e] <= inv[t, j] < offsets[e + 1]


# -----------------------------------------------------------------------------
# Experts and the MoE combine
# -----------------------------------------------------------------------------

class _Lay:
    pass


def _small_moe(rng, H=64, F=32, E=8, S=2, fmt=O.Q8_0):
    import synth
    lay = _Lay()
    lay.router = synth.random_qmat(O.Q8_0, 11, E, H, 0.1)
    lay.router_bias = None
    lay.exp_gate_up = synth.random_qmat(fmt, 12, E * 2 * F, H, 0.1)
    lay.exp_down = synth.random_qmat(fmt, 13, E * H, F, 0.1)
    lay.sh_gate_up = synth.random_qmat(fmt, 14, S * 2 * F, H, 0.1)
    lay.sh_down = synth.random_qmat(fmt, 15, S * H, F, 0.1)
    return lay


def test_swiglu_closed_form():
    """Gate row i and up row i are one-hot on input i with scales 1 and 2, the
    down matrix is one-hot back: y_i = fp16(silu(x_i) * 2 x_i) exactly."""
    k = F = 32
    x = O.f16(np.linspace(-3, 3, k))
    q = np.zeros((2 * F, k), int)
    q[np.arange(F), np.arange(F)] = 1
    q[F + np.arange(F), np.arange(F)] = 2
    gu = enc_q8_0(np.ones((2 * F, 1)), q)
    dn = enc_q8_0(np.ones((k, 1)), np.eye(k, dtype=int))
    y = O.swiglu(gu, dn, x[None])[0]
    expect = O.f16(x / (1 + np.exp(-x)) * 2 * x)
    assert np.array_equal(y, expect)


def test_moe_dense_brute_force():
    """Running every expert on every token and keeping the routed ones with
    their weights (no grouping) equals the oracle's grouped MoE."""
    rng = np.random.default_rng(10)
    lay = _small_moe(rng)
    x = O.f16(rng.standard_normal((7, 64)))
    out, idx, w, logits = O.moe(lay, x, 3)
    E = 8
    brute = np.zeros_like(out)
    for t in range(7):
        acc = np.zeros(64)
        for s in range(2):
            gu, dn = O.expert_mats(lay, s, shared=True)
            acc += O.swiglu(gu, dn, x[t:t + 1])[0]
        for e in range(E):
            gu, dn = O.expert_mats(lay, e)
            ye = O.swiglu(gu, dn, x[t:t + 1])[0]
            hit = np.where(idx[t] == e)[0]
            if hit.size:
                acc += w[t, hit[0]] * ye
        brute[t] = acc
    assert np.allclose(out, brute, rtol=1e-12, atol=1e-14)


def test_two_shared_experts_equal_one_of_double_width():
    """Two shared SwiGLU experts of width F equal one of width 2F built by
    concatenating gate, up (rows) and down (columns)."""
    rng = np.random.default_rng(11)
    H, F = 64, 32
    W = {n: O.f16(rng.standard_normal(s) * 0.1) for n, s in
         (("g0", (F, H)), ("u0", (F, H)), ("g1", (F, H)), ("u1", (F, H)), ("d0", (H, F)), ("d1", (H, F)))}
    x = O.f16(rng.standard_normal((3, H)))
    two = (O.swiglu(enc_f16(np.concatenate([W["g0"], W["u0"]])), enc_f16(W["d0"]), x)
           + O.swiglu(enc_f16(np.concatenate([W["g1"], W["u1"]])), enc_f16(W["d1"]), x))
    one = O.swiglu(enc_f16(np.concatenate([W["g0"], W["g1"], W["u0"], W["u1"]])),
                   enc_f16(np.concatenate([W["d0"], W["d1"]], 1)), x)
    assert np.allclose(two, one, rtol=1e-12, atol=1e-15)


# -----------------------------------------------------------------------------
# LM-head argmax
# -----------------------------------------------------------------------------

def test_argmax_lowest_index_and_nan():
    assert O.argmax_lowest(np.array([1.0, 3.0, 3.0, 2.0])) == 1
    assert O.argmax_lowest(np.array([np.nan, -1.0, 5.0, np.nan])) == 2
    z = np.random.default_rng(12).standard_normal(1000)
    assert O.argmax_lowest(z) == int(np.argmax(z))


# -----------------------------------------------------------------------------
# The composed step on constructed models
# -----------------------------------------------------------------------------

def _tiny_dims(**kw):
    import synth
    d = synth.Dims(hidden=64, n_heads=2, head_dim=32, n_layers=2, n_dense=1, dense_ff=64,
                   n_experts=8, top_k=2, n_shared=1, expert_ff=32, vocab=50, prefix_cap=5,
                   ring_cap=4, fmt_attn=O.Q8_0, fmt_router=O.Q8_0, fmt_dense=O.Q4_0,
                   fmt_expert=O.Q4_0, fmt_shared=O.Q4_0, w_std=0.05)
    for k_, v_ in kw.items():
        setattr(d, k_, v_)
    return d


def test_step_planted_token_with_silent_layers():
    """With every projection that writes into the residual set to zero (O and
    the FFN down matrices), each layer returns h unchanged, so the step's token
    is argmax(W_lm . rmsnorm(embed[tok])).  Planting W_lm[v*] = that normalised
    vector makes the step emit v* for every input token."""
    import synth
    d = _tiny_dims()
    m = synth.make_model(d, 21)
    for lay in m.layers:
        lay.wo.data[:] = 0
        (lay.exp_down if lay.is_moe else lay.dense_down).data[:] = 0
        if lay.is_moe:
            lay.sh_down.data[:] = 0
    st = synth.make_state(d, 21, [3, 5], [0, 6])
    tok = np.array([7, 42], np.int32)
    x = O.f16(O.rmsnorm(m.embed[tok].astype(np.float64), m.final_norm, d.norm_eps))
    lm = O.dequant(m.lm_head.fmt, m.lm_head.data, d.vocab, d.hidden).astype(np.float16)
    lm[13] = (4 * x[0] / np.linalg.norm(x[0])).astype(np.float16)
    lm[31] = (4 * x[1] / np.linalg.norm(x[1])).astype(np.float16)
    m.lm_head = synth.QMat(O.F16, d.vocab, d.hidden, lm.reshape(-1).view(np.uint8).copy())
    res = O.decode_step(m, st, tok_in=tok)
    assert np.array_equal(res.hidden, O.f16(m.embed[tok].astype(np.float64)))
    assert list(res.tok) == [13, 31]
    assert list(st.gen_index) == [1, 7]


def test_step_single_key_value_path():
    """Empty prefix and t = 0: the window holds only the new token, so the
    attention output is the new value.  With W_o = identity (Q8_0, d = 1),
    v-rows = 2 * identity and q/k rows zero, the attention block returns
    h + fp16(2 * x) where x = fp16(rmsnorm(h)) (the residual is not rounded);
    this pins that v is the third chunk of the QKV output and that O adds into
    the residual."""
    import synth
    d = _tiny_dims(n_layers=1, n_dense=1)
    m = synth.make_model(d, 22, with_embed=False, with_lm=False)
    lay = m.layers[0]
    H = d.hidden
    q = np.zeros((3 * H, H), int)
    q[2 * H + np.arange(H), np.arange(H)] = 2
    lay.wqkv = enc_q8_0(np.ones((3 * H, H // 32)), q)
    lay.wo = enc_q8_0(np.ones((H, H // 32)), np.eye(H, dtype=int))
    lay.dense_down.data[:] = 0
    st = synth.make_state(d, 22, [0], [0], fill="nan")
    h0 = O.f16(np.random.default_rng(13).standard_normal((1, H)))
    res = O.decode_step(m, st, hidden_in=h0, with_lm=False)
    x = O.f16(O.rmsnorm(h0[0], lay.attn_norm, d.norm_eps))
    assert np.array_equal(res.hidden[0], h0[0] + O.f16(2 * x))
    assert np.array_equal(res.new_v[0][0].reshape(-1), O.f16(2 * x))


def test_step_rows_are_independent():
    """A step over R rows equals R one-row steps (the oracle computes each
    row's arithmetic alone; rows share only the weights)."""
    import synth
    d = _tiny_dims()
    m = synth.make_model(d, 23)
    pl, gi = [5, 0, 3], [2, 9, 0]
    st = synth.make_state(d, 23, pl, gi)
    tok = np.array([1, 2, 3], np.int32)
    full = O.decode_step(m, st.copy(), tok_in=tok)
    for r in range(3):
        one = O.decode_step(m, st.copy(), tok_in=tok, rows=[r])
        assert one.tok[0] == full.tok[r]
        assert np.array_equal(one.hidden[0], full.hidden[r])
        assert np.array_equal(one.topk_idx[0][0], full.topk_idx[0][r])


def test_step_sequence_wraps_ring():
    """Several consecutive steps: the ring slot written at step t is t mod C,
    earlier slots keep their values, and the gen index advances by one."""
    import synth
    d = _tiny_dims()
    m = synth.make_model(d, 24)
    st = synth.make_state(d, 24, [2], [2])
    tok = np.array([4], np.int32)
    for t in range(2, 2 + 2 * d.ring_cap + 1):
        before = st.k_cache.copy()
        res = O.decode_step(m, st, tok_in=tok)
        slot = d.prefix_cap + t % d.ring_cap
        changed = np.argwhere(np.any(before != st.k_cache, axis=-1))
        assert set(changed[:, 3].tolist()) <= {slot}
        assert np.array_equal(st.k_cache[0, 0, :, slot].astype(np.float64), res.new_k[0][0])
        tok = res.tok
    assert st.gen_index[0] == 2 + 2 * d.ring_cap + 1


# --- prefill (the prompt pass) ---------------------------------------------

def _prefill_dims():
    import synth
    return synth.Dims(hidden=64, n_heads=2, head_dim=64, n_layers=3, n_dense=1, dense_ff=128, n_experts=8,
                      top_k=3, n_shared=1, expert_ff=64, vocab=300, prefix_cap=4, ring_cap=24)


@pytest.mark.parametrize("use_emb", [False, True])
def test_prefill_equals_token_by_token_decode(use_emb):
    """The prompt pass over P positions equals P decode steps of one row with
    an empty prefix and a ring large enough to hold them all: step t writes
    ring slot t at position t and attends slots 0..t, which is the causal
    window of position t.  The two forms share no attention or batching
    code (matrix form with a mask against one query at a time)."""
    import synth
    d = _prefill_dims()
    P = 19
    m = synth.make_model(d, 31)
    tok = synth.uniform_i32(synth.stream_id(31, "prompt"), (P,), 0, d.vocab)
    emb = synth.normal_f16(synth.stream_id(31, "emb"), (P, d.hidden)).astype(np.float64) if use_emb else None
    pre = O.prefill(m, P, tok=None if use_emb else tok, emb=emb)
    st = synth.make_state(d, 31, [0], [0])
    steps = []
    for t in range(P):
        if use_emb:
            steps.append(O.decode_step(m, st, hidden_in=emb[t:t + 1]))
        else:
            steps.append(O.decode_step(m, st, tok_in=tok[t:t + 1]))
    for l in range(d.n_layers):
        ring_k = st.k_cache[l, 0][:, d.prefix_cap:d.prefix_cap + P].astype(np.float64)
        ring_v = st.v_cache[l, 0][:, d.prefix_cap:d.prefix_cap + P].astype(np.float64)
        assert np.array_equal(ring_k, pre.k[l])
        assert np.array_equal(ring_v, pre.v[l])
    for ml in range(len(pre.topk_idx)):
        for t in range(P):
            assert np.array_equal(steps[t].topk_idx[ml][0], pre.topk_idx[ml][t])
            assert np.allclose(steps[t].topk_w[ml][0], pre.topk_w[ml][t], rtol=1e-12, atol=0)
    hid = np.array([s.hidden[0] for s in steps])
    assert np.allclose(hid, pre.hidden, rtol=1e-11, atol=1e-12)
    assert steps[-1].tok[0] == pre.tok


def test_prefill_is_causal():
    """Changing the last prompt token changes nothing at earlier positions."""
    import synth
    d = _prefill_dims()
    P = 12
    m = synth.make_model(d, 32)
    tok = synth.uniform_i32(synth.stream_id(32, "prompt"), (P,), 0, d.vocab)
    tok2 = tok.copy()
    tok2[-1] = (tok[-1] + 1) % d.vocab
    a = O.prefill(m, P, tok=tok)
    b = O.prefill(m, P, tok=tok2)
    for l in range(d.n_layers):
        assert np.allclose(a.k[l][:, :P - 1], b.k[l][:, :P - 1], rtol=0, atol=0)
        assert not np.array_equal(a.k[l][:, P - 1], b.k[l][:, P - 1])
    assert np.allclose(a.hidden[:P - 1], b.hidden[:P - 1], rtol=1e-12, atol=1e-13)


def test_causal_attention_cases():
    """One position: the output is its value.  Position i of the masked
    matrix form equals single-query attention over keys 0..i."""
    rng = np.random.default_rng(5)
    q, k, v = rng.standard_normal((3, 9, 16))
    o = O.causal_attention(q, k, v, 0.25)
    assert np.array_equal(O.causal_attention(q[:1], k[:1], v[:1], 0.25)[0], v[0])
    for i in range(9):
        assert np.allclose(o[i], O.attention(q[i], k[:i + 1], v[:i + 1], 0.25), rtol=1e-13, atol=1e-14)


# --- INT8 KV cache ------------------------------------------------------------

def test_kv_quantise_hand_built():
    """s = fp16(2/127) = 1.0078125 * 2^-6; codes by hand: 2/s = 127.008 -> 127,
    -1/s = -63.504 -> -64, 0.5/s = 31.752 -> 32.  With s = 2^-7 exactly
    (amax = 127 * 2^-7) the halves round away from zero: 2.5 -> 3, 0.5 -> 1,
    -0.5 -> -1, 1.5 -> 2."""
    q, s = O.kv_quantise(np.array([[2.0, -1.0, 0.5, 0.0]]))
    assert s[0] == np.float16(0.0157470703125)
    assert q[0].tolist() == [127, -64, 32, 0]
    u = 2.0 ** -7
    q, s = O.kv_quantise(np.array([127 * u, 2.5 * u, 0.5 * u, -0.5 * u, 1.5 * u, -127 * u]))
    assert s == np.float16(u)
    assert q.tolist() == [127, 3, 1, -1, 2, -127]


def test_kv_quantise_zero_row_scaling_and_bound():
    q, s = O.kv_quantise(np.zeros((2, 8)))
    assert np.all(q == 0) and np.all(s == 0)
    rng = np.random.default_rng(9)
    x = rng.standard_normal((50, 128)).astype(np.float16).astype(np.float64)
    q, s = O.kv_quantise(x)
    for k in (-3, 2):
        q2, s2 = O.kv_quantise(x * 2.0 ** k)
        assert np.array_equal(q2, q)
        assert np.array_equal(s2.astype(np.float64), s.astype(np.float64) * 2.0 ** k)
    amax = np.max(np.abs(x), axis=1)
    err = np.abs(O.kv_dequant(q, s) - x)
    assert np.all(err <= 0.5 * s.astype(np.float64)[:, None] + 2.0 ** -11 * amax[:, None] + 1e-15)
    assert np.all(np.max(np.abs(q.astype(int)), axis=1) >= 126)


def test_step_int8_cache_writes_quantised_new_token():
    """With an int8 cache the new slot holds kv_quantise of the same keys and
    values an fp16-cache step computes (the layer-0 projections do not
    depend on the cache), and nothing else in the cache changes."""
    import synth
    d = _tiny_dims()
    m = synth.make_model(d, 41)
    st8 = synth.make_state_int8(d, 41, [5], [2])
    st16 = synth.make_state(d, 41, [5], [2])
    tok = np.array([7], np.int32)
    before = st8.k_cache.copy()
    r8 = O.decode_step(m, st8, tok_in=tok)
    r16 = O.decode_step(m, st16, tok_in=tok)
    slot = d.prefix_cap + 2 % d.ring_cap
    qk, sk = O.kv_quantise(r16.new_k[0][0])
    assert np.array_equal(st8.k_cache[0, 0][:, slot], qk)
    assert np.array_equal(st8.k_scale[0, 0][:, slot], sk)
    changed = np.argwhere(np.any(before != st8.k_cache, axis=-1))
    assert set(changed[:, 3].tolist()) <= {slot}
    assert r8.tok is not None


# --- generation of one request (the round's unit) -----------------------------

def test_generate_first_token_eos_and_budget():
    """max_new = 1 gives the prompt pass's token; a later token of the
    sequence put in the EOS set ends it there (not handed out, or kept with
    keep_eos); the sequence continues the prompt pass with decode steps."""
    import synth
    d = _prefill_dims()
    d.prefix_cap = 16
    m = synth.make_model(d, 51)
    P = 9
    tok = synth.uniform_i32(synth.stream_id(51, "prompt"), (P,), 0, d.vocab)
    pre = O.prefill(m, P, tok=tok)
    one, stop, _ = O.generate(m, P, tok=tok, max_new=1)
    assert one == [int(pre.tok)] and stop == 2
    seq, stop, gaps = O.generate(m, P, tok=tok, max_new=6)
    assert len(seq) == 6 and stop == 2 and len(gaps) == 6 and seq[0] == int(pre.tok)
    # each later token is the prompt pass's argmax over the prompt extended by
    # the tokens generated so far (the hand-off puts the first decode step at
    # position P with the prompt's cache)
    for i in (1, 2):
        ext = np.concatenate([tok, np.array(seq[:i], np.int32)])
        assert seq[i] == int(O.prefill(m, P + i, tok=ext).tok)
    k = next(i for i in range(1, 6) if seq[i] not in seq[:i])  # a token not seen before it
    cut, stop, _ = O.generate(m, P, tok=tok, max_new=6, eos=[seq[k]])
    assert cut == seq[:k] and stop == 1
    kept, stop, _ = O.generate(m, P, tok=tok, max_new=6, eos=[seq[k]], keep_eos=True)
    assert kept == seq[:k + 1] and stop == 1


def test_prefill_int8_equals_token_by_token_decode():
    """With an INT8 cache the prompt pass stores the same codes and scales,
    and leaves the same residual, as P decode steps over an empty prefix with
    an INT8 cache (both quantise the same fp16 keys and values and attend to
    them as stored)."""
    import synth
    d = _prefill_dims()
    P = 15
    m = synth.make_model(d, 33)
    tok = synth.uniform_i32(synth.stream_id(33, "prompt"), (P,), 0, d.vocab)
    pre = O.prefill(m, P, tok=tok, int8_kv=True)
    st = synth.make_state_int8(d, 33, [0], [0])
    steps = [O.decode_step(m, st, tok_in=tok[t:t + 1]) for t in range(P)]
    for l in range(d.n_layers):
        sl = slice(d.prefix_cap, d.prefix_cap + P)
        assert np.array_equal(st.k_cache[l, 0][:, sl], pre.kq[l])
        assert np.array_equal(st.k_scale[l, 0][:, sl], pre.ks[l])
        assert np.array_equal(st.v_cache[l, 0][:, sl], pre.vq[l])
        assert np.array_equal(st.v_scale[l, 0][:, sl], pre.vs[l])
    hid = np.array([s.hidden[0] for s in steps])
    assert np.allclose(hid, pre.hidden, rtol=1e-11, atol=1e-12)
    assert steps[-1].tok[0] == pre.tok
    # and the int8 cache changes the result: the stored values are not the fp16 ones
    assert not np.allclose(O.prefill(m, P, tok=tok).hidden, pre.hidden, rtol=1e-9, atol=0)
