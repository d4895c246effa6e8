"""GPU parity of the C-ABI entry points against the oracle, kernel by kernel.

Every case prints its name, shape and seed before it touches the GPU.
"""
import numpy as np
import pytest

import oracle as O
import synth
from tests.gpu_util import NEAR_TIE, assert_close, assert_close_f16, f16_tensor, from_f16_tensor, log_near_tie

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import torch
    assert torch.cuda.is_available()
    import quantized_decode_step_amd as qd
    return qd


def _say(*a):
    print("[case]", *a, flush=True)


# -----------------------------------------------------------------------------
# ocrdec_gemv_q
# -----------------------------------------------------------------------------

GEMV_CASES = [
    # (fmt, n, k, rows)
    (synth.F16, 40, 96, 1), (synth.Q8_0, 40, 96, 3), (synth.Q4_0, 40, 160, 5), (synth.U8A_G32, 40, 96, 2),
    (synth.Q8_0, 3840, 1280, 1), (synth.Q8_0, 3840, 1280, 24), (synth.Q4_0, 1280, 3584, 1),
    (synth.Q4_0, 1792, 1280, 17), (synth.Q4_0, 1280, 896, 6), (synth.F16, 16200, 1280, 1),
    (synth.F16, 16200, 1280, 12), (synth.U8A_G32, 1536, 512, 24), (synth.U8A_G32, 512, 512, 1),
    (synth.Q8_0, 64, 1280, 32), (synth.Q4_0, 1000, 1280, 40), (synth.F16, 1280, 1280, 33),
]


@pytest.mark.parametrize("fmt,n,k,rows", GEMV_CASES)
@pytest.mark.parametrize("otype", [0, 1])
def test_gemv_q_parity(q, fmt, n, k, rows, otype):
    import torch
    seed = 100 + n + k + rows
    _say("gemv_q", synth.FMT_NAMES[fmt], n, k, rows, "otype", otype, "seed", seed)
    m = synth.random_qmat(fmt, synth.stream_id(seed, "W"), n, k, 0.02)
    x = synth.normal_f16(synth.stream_id(seed, "x"), (rows, k))
    dm = q.DeviceQMat(m)
    xd = f16_tensor(x)
    if otype == 0:
        y = torch.full((rows, n), float("nan"), dtype=torch.float32, device="cuda")
    else:
        y = torch.full((rows, n), -1, dtype=torch.int16, device="cuda")
    q.ocrdec_gemv_q(dm.desc, rows, xd, k, y, otype, n)
    torch.cuda.synchronize()
    ref = O.gemv_qmat(m, x.astype(np.float64))
    got = y.cpu().numpy().astype(np.float64) if otype == 0 else from_f16_tensor(y)
    what = "gemv %s %dx%d rows=%d" % (synth.FMT_NAMES[fmt], n, k, rows)
    if otype == 1:
        assert_close_f16(got, O.f16(ref), what)
    else:
        assert_close(got, ref, what)


def test_gemv_q_rejects_bad_args(q):
    import torch
    m = synth.random_qmat(synth.Q8_0, 1, 32, 64)
    dm = q.DeviceQMat(m)
    x = torch.zeros((2, 64), dtype=torch.int16, device="cuda")
    y = torch.zeros((2, 32), dtype=torch.float32, device="cuda")
    with pytest.raises(q.OcrdecError):
        q.ocrdec_gemv_q(dm.desc, 0, x, 64, y, 0, 32)
    with pytest.raises(q.OcrdecError):
        q.ocrdec_gemv_q(dm.desc, 2, x, 60, y, 0, 32)
    bad = q.QMatDesc(dm.desc.fmt, 32, 48, dm.desc.data)
    with pytest.raises(q.OcrdecError):
        q.ocrdec_gemv_q(bad, 2, x, 64, y, 0, 32)


# -----------------------------------------------------------------------------
# ocrdec_attn_decode
# -----------------------------------------------------------------------------

def _attn_case(q, rows, NH, D, prefix_cap, ring_cap, prefix_len, gen_index, sink, seed, fill="zero"):
    import torch
    cap = prefix_cap + ring_cap
    rng = np.random.default_rng(seed)
    qkv = rng.standard_normal((rows, 3 * NH * D)) * 0.7
    qkv = qkv.astype(np.float32)
    kc = synth.normal_f16(synth.stream_id(seed, "kc"), (rows, NH, cap, D))
    vc = synth.normal_f16(synth.stream_id(seed, "vc"), (rows, NH, cap, D))
    for r in range(rows):
        valid = np.zeros(cap, bool)
        if ring_cap:
            valid[:prefix_len[r]] = True
            valid[prefix_cap:prefix_cap + min(gen_index[r], ring_cap)] = True
        else:
            valid[:prefix_len[r]] = True
        pad = np.float16(np.nan) if fill == "nan" else np.float16(0)
        kc[r][:, ~valid] = pad
        vc[r][:, ~valid] = pad
        if sink is not None:
            kc[r][:, 0] = 0
            vc[r][:, 0] = 0
    kd, vd = f16_tensor(kc), f16_tensor(vc)
    qkv_d = torch.from_numpy(qkv).cuda()
    pl = torch.tensor(prefix_len, dtype=torch.int32, device="cuda")
    gi = torch.tensor(gen_index, dtype=torch.int32, device="cuda")
    sk = torch.tensor(np.asarray(sink, np.float32), device="cuda") if sink is not None else None
    out = torch.full((rows, NH * D), -1, dtype=torch.int16, device="cuda")
    a = q.AttnArgs(rows, NH, D, qkv_d.data_ptr(), 3 * NH * D, kd.data_ptr(), vd.data_ptr(), prefix_cap, ring_cap,
                   pl.data_ptr(), gi.data_ptr(), sk.data_ptr() if sk is not None else None, 10000.0,
                   float(1 / np.sqrt(D)), out.data_ptr(), NH * D)
    wsb = q.ocrdec_attn_workspace_bytes(a)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    q.ocrdec_attn_decode(a, ws, wsb)
    torch.cuda.synchronize()
    got = from_f16_tensor(out)
    kc_after = kd.cpu().numpy().view(np.float16)
    vc_after = vd.cpu().numpy().view(np.float16)
    # oracle
    for r in range(rows):
        qq = qkv[r, :NH * D].reshape(NH, D).astype(np.float64)
        kk = qkv[r, NH * D:2 * NH * D].reshape(NH, D).astype(np.float64)
        vv = qkv[r, 2 * NH * D:].reshape(NH, D).astype(np.float64)
        kcr, vcr = kc[r].copy(), vc[r].copy()
        if ring_cap:
            t = gen_index[r]
            pos = prefix_len[r] + t
            slot = prefix_cap + O.ring_slot(t, ring_cap)
            idx = O.window(prefix_len[r], prefix_cap, t, ring_cap)
        else:
            pos = prefix_len[r] - (1 if sink is not None else 0)
            slot = prefix_len[r]
            idx = np.arange(prefix_len[r] + 1)
        qr = O.f16(O.rope(qq, pos, 10000.0))
        kr = O.f16(O.rope(kk, pos, 10000.0))
        vr = O.f16(vv)
        kcr[:, slot] = kr
        vcr[:, slot] = vr
        ref = np.zeros((NH, D))
        for h in range(NH):
            if sink is not None:
                ref[h] = O.attention(qr[h], kcr[h, idx], vcr[h, idx], 1 / np.sqrt(D), sink=float(sink[h]),
                                     sink_index=0)
            else:
                ref[h] = O.attention(qr[h], kcr[h, idx], vcr[h, idx], 1 / np.sqrt(D))
        assert_close_f16(got[r], O.f16(ref.reshape(-1)), "attn out row %d" % r)
        assert_close_f16(kc_after[r][:, slot].astype(np.float64), kr, "new k row %d" % r)
        assert np.array_equal(vc_after[r][:, slot].astype(np.float64), vr), "new v row %d" % r
        # nothing else in the cache changed
        mask = np.ones(kc.shape[2], bool)
        mask[slot] = False
        assert np.array_equal(kc_after[r][:, mask].view(np.uint16), kc[r][:, mask].view(np.uint16))


@pytest.mark.parametrize("rows,prefix_len,gen_index", [
    (1, [1100], [128]), (1, [256], [0]), (3, [1100, 0, 37], [5, 300, 127]), (24, [1100] * 24, list(range(100, 124))),
])
def test_attn_ring_parity(q, rows, prefix_len, gen_index):
    _say("attn ring", rows, prefix_len[:3], gen_index[:3])
    _attn_case(q, rows, 10, 128, 1100, 128, prefix_len, gen_index, None, 7 + rows, fill="nan")


@pytest.mark.parametrize("rows,L", [(1, 350), (6, 350), (2, 3000), (24, 3000)])
def test_attn_sink_linear_parity(q, rows, L):
    _say("attn sink linear", rows, L)
    sink = O.f16(np.random.default_rng(L + rows).standard_normal(8))
    _attn_case(q, rows, 8, 64, L + 1, 0, [L] * rows, [0] * rows, sink, 11 + rows, fill="nan")


def test_attn_ring_small_cap_wraps(q):
    _say("attn ring small cap")
    _attn_case(q, 4, 2, 128, 70, 4, [0, 70, 3, 64], [0, 3, 4, 9], None, 5, fill="nan")


def _attn_case_int8(q, rows, NH, D, prefix_cap, ring_cap, prefix_len, gen_index, sink, seed):
    """ocrdec_attn_decode over an INT8 KV cache (codes + one fp16 scale per
    row, head and slot) against the oracle reading the same stored values.
    The new value row is fp16(v) on both sides, so its codes and scale must be
    bit-equal; the new key is too where RoPE is the identity (position 0),
    and elsewhere within one code step plus the fp16 rule."""
    import torch
    cap = prefix_cap + ring_cap
    rng = np.random.default_rng(seed)
    qkv = (rng.standard_normal((rows, 3 * NH * D)) * 0.7).astype(np.float32)

    class _D:
        pass
    d = _D()
    d.n_layers, d.n_heads, d.head_dim, d.prefix_cap, d.ring_cap = 1, NH, D, prefix_cap, ring_cap
    if ring_cap == 0:
        # linear mode: the window is [0, prefix_len]; draw codes for [0, prefix_len)
        st = synth.make_state_int8(d, seed, prefix_len, [0] * rows)
    else:
        st = synth.make_state_int8(d, seed, prefix_len, gen_index)
    kc, vc, ks, vs = st.k_cache[0], st.v_cache[0], st.k_scale[0], st.v_scale[0]
    if sink is not None:
        kc[:, :, 0] = 0
        vc[:, :, 0] = 0
    kd = torch.from_numpy(kc.copy()).cuda()
    vd = torch.from_numpy(vc.copy()).cuda()
    ksd = f16_tensor(ks)
    vsd = f16_tensor(vs)
    qkv_d = torch.from_numpy(qkv).cuda()
    pl = torch.tensor(prefix_len, dtype=torch.int32, device="cuda")
    gi = torch.tensor(gen_index, dtype=torch.int32, device="cuda")
    sk = torch.tensor(np.asarray(sink, np.float32), device="cuda") if sink is not None else None
    out = torch.full((rows, NH * D), -1, dtype=torch.int16, device="cuda")
    a = q.AttnArgs(rows, NH, D, qkv_d.data_ptr(), 3 * NH * D, kd.data_ptr(), vd.data_ptr(), prefix_cap, ring_cap,
                   pl.data_ptr(), gi.data_ptr(), sk.data_ptr() if sk is not None else None, 10000.0,
                   float(1 / np.sqrt(D)), out.data_ptr(), NH * D, ksd.data_ptr(), vsd.data_ptr())
    wsb = q.ocrdec_attn_workspace_bytes(a)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    q.ocrdec_attn_decode(a, ws, wsb)
    torch.cuda.synchronize()
    got = from_f16_tensor(out)
    kc_after, vc_after = kd.cpu().numpy(), vd.cpu().numpy()
    ks_after = ksd.cpu().numpy().view(np.float16)
    vs_after = vsd.cpu().numpy().view(np.float16)
    for r in range(rows):
        qq = qkv[r, :NH * D].reshape(NH, D).astype(np.float64)
        kk = qkv[r, NH * D:2 * NH * D].reshape(NH, D).astype(np.float64)
        vv = qkv[r, 2 * NH * D:].reshape(NH, D).astype(np.float64)
        if ring_cap:
            t = gen_index[r]
            pos = prefix_len[r] + t
            slot = prefix_cap + O.ring_slot(t, ring_cap)
            idx = O.window(prefix_len[r], prefix_cap, t, ring_cap)
        else:
            pos = prefix_len[r] - (1 if sink is not None else 0)
            slot = prefix_len[r]
            idx = np.arange(prefix_len[r] + 1)
        qr = O.f16(O.rope(qq, pos, 10000.0))
        kr = O.f16(O.rope(kk, pos, 10000.0))
        vr = O.f16(vv)
        kq, kss = O.kv_quantise(kr)
        vq, vss = O.kv_quantise(vr)
        kcr, vcr, ksr, vsr = kc[r].copy(), vc[r].copy(), ks[r].copy(), vs[r].copy()
        kcr[:, slot], ksr[:, slot] = kq, kss
        vcr[:, slot], vsr[:, slot] = vq, vss
        ref = np.zeros((NH, D))
        for h in range(NH):
            K = O.kv_dequant(kcr[h, idx], ksr[h, idx])
            V = O.kv_dequant(vcr[h, idx], vsr[h, idx])
            if sink is not None:
                ref[h] = O.attention(qr[h], K, V, 1 / np.sqrt(D), sink=float(sink[h]), sink_index=0)
            else:
                ref[h] = O.attention(qr[h], K, V, 1 / np.sqrt(D))
        assert_close_f16(got[r], O.f16(ref.reshape(-1)), "int8 attn out row %d" % r)
        assert np.array_equal(vc_after[r][:, slot], vq), "new v codes row %d" % r
        assert np.array_equal(vs_after[r][:, slot], vss), "new v scales row %d" % r
        if pos == 0:
            assert np.array_equal(kc_after[r][:, slot], kq), "new k codes row %d" % r
            assert np.array_equal(ks_after[r][:, slot], kss), "new k scales row %d" % r
        else:
            gk = O.kv_dequant(kc_after[r][:, slot], ks_after[r][:, slot])
            ok = O.kv_dequant(kq, kss)
            bound = 2e-3 * np.sqrt(np.mean(ok * ok)) + 2 * kss.astype(np.float64)[:, None]
            assert np.all(np.abs(gk - ok) <= bound), "new k row %d" % r
        mask = np.ones(kc.shape[2], bool)
        mask[slot] = False
        assert np.array_equal(kc_after[r][:, mask], kc[r][:, mask])
        assert np.array_equal(ks_after[r][:, mask].view(np.uint16), ks[r][:, mask].view(np.uint16))


@pytest.mark.parametrize("rows,prefix_len,gen_index", [
    (1, [0], [0]), (1, [1100], [128]), (3, [1100, 0, 37], [5, 300, 127]), (24, [1100] * 24, list(range(100, 124))),
])
def test_attn_ring_int8_cache(q, rows, prefix_len, gen_index):
    _say("attn ring int8", rows, prefix_len[:3], gen_index[:3])
    _attn_case_int8(q, rows, 10, 128, 1100, 128, prefix_len, gen_index, None, 31 + rows)


@pytest.mark.parametrize("rows,L", [(1, 350), (6, 3000)])
def test_attn_sink_linear_int8_cache(q, rows, L):
    _say("attn sink linear int8", rows, L)
    sink = O.f16(np.random.default_rng(L + rows).standard_normal(8))
    _attn_case_int8(q, rows, 8, 64, L + 1, 0, [L] * rows, [0] * rows, sink, 41 + rows)


# -----------------------------------------------------------------------------
# ocrdec_moe_layer
# -----------------------------------------------------------------------------

class _Lay:
    pass


def _moe_case(q, rows, seed, H=1280, E=64, K=6, S=2, F=896, fmt=synth.Q8_0, bias=False, residual=True):
    import torch
    d = synth.Dims(hidden=H, n_experts=E, top_k=K, n_shared=S, expert_ff=F, fmt_router=synth.Q8_0,
                   fmt_expert=fmt, fmt_shared=fmt)
    lay = _Lay()
    for k_, v_ in synth.make_moe_weights(d, seed, 0, with_bias=bias).items():
        setattr(lay, k_, v_)
    if not bias:
        lay.router_bias = None
    x = synth.normal_f16(synth.stream_id(seed, "x"), (rows, H))
    h = synth.normal_f16(synth.stream_id(seed, "h"), (rows, H))
    w, keep = q.moe_weights(lay, H, K)
    xd, hd = f16_tensor(x), f16_tensor(h)
    cap_idx = torch.full((rows, K), -1, dtype=torch.int32, device="cuda")
    cap_w = torch.zeros((rows, K), dtype=torch.float32, device="cuda")
    counts = torch.zeros(E, dtype=torch.int32, device="cuda")
    offsets = torch.zeros(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.zeros(rows * K, dtype=torch.int32, device="cuda")
    cap = q.MoeCapture(cap_idx.data_ptr(), cap_w.data_ptr(), counts.data_ptr(), offsets.data_ptr(), perm.data_ptr())
    wsb = q.ocrdec_moe_workspace_bytes(w, rows)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    q.ocrdec_moe_layer(w, rows, xd, hd, residual, None, cap, ws, wsb)
    torch.cuda.synchronize()
    out, idx, wt, logits = O.moe(lay, x.astype(np.float64), K)
    g_idx = cap_idx.cpu().numpy()
    # routing: bit-exact except logged near-ties
    ties = []
    for r in range(rows):
        if not np.array_equal(g_idx[r], idx[r]):
            gap = O.topk_gap(logits[r], K, lay.router_bias)
            assert gap < NEAR_TIE, "row %d routing differs with oracle gap %.3g" % (r, gap)
            log_near_tie("routing", "MoE layer rows=%d row %d" % (rows, r), gap)
            ties.append(r)
    keep_rows = [r for r in range(rows) if r not in ties]
    assert_close(cap_w.cpu().numpy()[keep_rows], wt[keep_rows], "topk weights")
    if not ties:
        c, o, p, _ = O.group(idx, E)
        assert np.array_equal(counts.cpu().numpy(), c)
        assert np.array_equal(offsets.cpu().numpy(), o)
        assert np.array_equal(perm.cpu().numpy(), p)
    ref = O.f16(h + out) if residual else O.f16(out)
    got = from_f16_tensor(hd)
    assert_close_f16(got[keep_rows], ref[keep_rows], "moe out")


@pytest.mark.parametrize("rows", [1, 6, 24])
def test_moe_q8_parity(q, rows):
    _say("moe q8", rows)
    _moe_case(q, rows, 1002 + rows)


# One row with a forced choice that names one expert twice: the one-row
# grouping in the routing kernel gives each of the two tokens its own entry
# (the general grouping would make one entry of two); the output, the
# weights and the captured counts, offsets and permutation are the same.
def test_moe_one_row_forced_repeat(q):
    import torch
    _say("moe one row forced with a repeated expert")
    H, E, K, S, F = 1280, 64, 6, 2, 896
    d = synth.Dims(hidden=H, n_experts=E, top_k=K, n_shared=S, expert_ff=F, fmt_router=synth.Q8_0,
                   fmt_expert=synth.Q4_0, fmt_shared=synth.Q4_0)
    lay = _Lay()
    for k_, v_ in synth.make_moe_weights(d, 1201, 0).items():
        setattr(lay, k_, v_)
    lay.router_bias = None
    x = synth.normal_f16(synth.stream_id(1201, "x"), (1, H))
    h = synth.normal_f16(synth.stream_id(1201, "h"), (1, H))
    forced = np.array([[40, 5, 63, 5, 0, 17]], np.int32)
    w, keep = q.moe_weights(lay, H, K)
    xd, hd = f16_tensor(x), f16_tensor(h)
    ft = torch.from_numpy(forced).cuda()
    cap_w = torch.zeros((1, K), dtype=torch.float32, device="cuda")
    counts = torch.zeros(E, dtype=torch.int32, device="cuda")
    offsets = torch.zeros(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.zeros(K, dtype=torch.int32, device="cuda")
    cap = q.MoeCapture(None, cap_w.data_ptr(), counts.data_ptr(), offsets.data_ptr(), perm.data_ptr())
    wsb = q.ocrdec_moe_workspace_bytes(w, 1)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    q.ocrdec_moe_layer(w, 1, xd, hd, True, ft, cap, ws, wsb)
    torch.cuda.synchronize()
    out, idx, wt, _ = O.moe(lay, x.astype(np.float64), K, forced_idx=forced)
    assert np.array_equal(idx, forced)
    c, o, pm, _ = O.group(idx, E)
    assert c[5] == 2
    assert np.array_equal(counts.cpu().numpy(), c)
    assert np.array_equal(offsets.cpu().numpy(), o)
    assert np.array_equal(perm.cpu().numpy(), pm)
    assert_close(cap_w.cpu().numpy(), wt, "forced weights")
    assert_close_f16(from_f16_tensor(hd), O.f16(h + out), "moe out")


def test_moe_q4_small_parity(q):
    _say("moe q4 small")
    _moe_case(q, 7, 77, H=256, E=16, K=4, S=1, F=128, fmt=synth.Q4_0)


def test_moe_prefill_bias_parity(q):
    _say("moe prefill-shaped 300 rows with bias")
    _moe_case(q, 300, 1005, H=1280, E=64, K=6, S=2, F=896, fmt=synth.Q4_0, bias=True, residual=False)


# the expert GEMM with the other weight formats: an odd number of 128-column
# stages in the down projection (640, 384) and a 2-token last entry (130)
@pytest.mark.parametrize("rows,fmt,F", [(130, synth.Q8_0, 640), (257, synth.F16, 384)])
def test_moe_prefill_formats(q, rows, fmt, F):
    _say("moe prefill-shaped", rows, "rows", synth.FMT_NAMES[fmt], "F", F)
    _moe_case(q, rows, 1100 + rows, H=1024, E=32, K=4, S=1, F=F, fmt=fmt)


# -----------------------------------------------------------------------------
# ocrdec_lm_argmax
# -----------------------------------------------------------------------------

# full-vocabulary heads with up to 16 rows take the CU-balanced kernel, the
# others the general GEMV with the argmax epilogue.  Q4_0 heads of 33000 and
# 36864 rows and a U8A head of 36864 give each of 256 CUs 8-9 tiles: fewer
# than the twelve wavefronts of those forms, so some start with no tile (one
# head ends mid-tile).
@pytest.mark.parametrize("fmt,n,rows", [(synth.F16, 129280, 1), (synth.F16, 129280, 24), (synth.Q8_0, 5000, 7),
                                        (synth.Q4_0, 999, 32), (synth.Q4_0, 129280, 24), (synth.Q8_0, 129280, 1),
                                        (synth.F16, 129280, 16), (synth.Q4_0, 129280, 3),
                                        (synth.U8A_G32, 100000, 2), (synth.Q4_0, 36864, 1), (synth.Q4_0, 33000, 5),
                                        (synth.U8A_G32, 36864, 3)])
def test_lm_argmax_parity(q, fmt, n, rows):
    import torch
    seed = 77 + n + rows
    _say("lm_argmax", synth.FMT_NAMES[fmt], n, rows, "seed", seed)
    m = synth.random_qmat(fmt, synth.stream_id(seed, "W"), n, 1280, 0.02)
    x = synth.normal_f16(synth.stream_id(seed, "x"), (rows, 1280))
    # plant a tie between two rows for row 0: the lower index must win
    dm = q.DeviceQMat(m)
    xd = f16_tensor(x)
    tok = torch.full((rows,), -1, dtype=torch.int32, device="cuda")
    top2 = torch.zeros((rows, 2), dtype=torch.float32, device="cuda")
    wsb = q.ocrdec_lm_argmax_workspace_bytes(dm.desc, rows)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    for rep in range(3):   # the workspace is reused as it is left
        q.ocrdec_lm_argmax(dm.desc, rows, xd, tok, top2, ws, wsb)
        torch.cuda.synchronize()
        z = O.f32(O.gemv_qmat(m, x.astype(np.float64)))
        g = tok.cpu().numpy()
        t2 = top2.cpu().numpy()
        for r in range(rows):
            best = O.argmax_lowest(z[r])
            srt = np.sort(z[r])[::-1]
            if g[r] != best:
                assert srt[0] - srt[1] < NEAR_TIE, "row %d: %d vs %d" % (r, g[r], best)
            assert abs(t2[r, 0] - srt[0]) <= 1e-4 * max(1, abs(srt[0]))
            assert abs(t2[r, 1] - srt[1]) <= 1e-4 * max(1, abs(srt[1]))


@pytest.mark.parametrize("n,k", [(4096, 128), (40000, 256)])
def test_lm_argmax_ties_go_to_lowest_index(q, n, k):
    import torch
    _say("lm_argmax planted ties", n, k)
    rows = 3
    w = np.zeros((n, k), np.float16)
    x = np.zeros((rows, k), np.float16)
    x[:, 0] = 1
    # row r of x: winners planted at several equal maxima (far apart: other
    # workgroups and wavefronts of the CU-balanced kernel hold them)
    for v in (17, 900, 4000, n - 5):
        w[v, 0] = 2.0
    w[3000, 0] = 1.5
    m = synth.QMat(synth.F16, n, k, w.reshape(-1).view(np.uint8).copy())
    dm = q.DeviceQMat(m)
    tok = torch.full((rows,), -1, dtype=torch.int32, device="cuda")
    wsb = q.ocrdec_lm_argmax_workspace_bytes(dm.desc, rows)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    q.ocrdec_lm_argmax(dm.desc, rows, f16_tensor(x), tok, None, ws, wsb)
    torch.cuda.synchronize()
    assert tok.cpu().numpy().tolist() == [17, 17, 17]


def _planted_block_rows(fmt, n, k, vals):
    """Canonical Q8_0 / Q4_0 rows whose only nonzero weight is column 0 of
    the rows in `vals` (value d * q, written exactly)."""
    nb = k // 32
    if fmt == synth.Q8_0:
        blk = np.zeros((n, nb, 34), np.uint8)
        for v, (d, qv) in vals.items():
            blk[v, 0, 0:2] = np.frombuffer(np.float16(d).tobytes(), np.uint8)
            blk[v, 0, 2] = np.uint8(np.int8(qv).view(np.uint8))
    else:
        blk = np.zeros((n, nb, 18), np.uint8)
        blk[:, :, 2:] = 0x88  # every code 8: value 0
        for v, (d, qv) in vals.items():
            blk[v, 0, 0:2] = np.frombuffer(np.float16(d).tobytes(), np.uint8)
            blk[v, 0, 2] = 0x80 | (qv + 8)  # element 0 in the low nibble of byte 0
    return synth.QMat(fmt, n, k, blk.reshape(-1).copy())


# block formats: five chunks per row against the ring of four, so tiles end
# inside a pass of the ring
@pytest.mark.parametrize("fmt,k", [(synth.Q8_0, 320), (synth.Q4_0, 640)])
def test_lm_argmax_block_ties_go_to_lowest_index(q, fmt, k):
    import torch
    n, rows = 40000, 3
    _say("lm_argmax planted ties", synth.FMT_NAMES[fmt], n, k)
    # four rows at 2.0 (d = 1, q = 2), one at 1.5 (d = 0.5, q = 3)
    vals = {v: (1.0, 2) for v in (17, 900, 4000, n - 5)}
    vals[3000] = (0.5, 3)
    m = _planted_block_rows(fmt, n, k, vals)
    x = np.zeros((rows, k), np.float16)
    x[:, 0] = 1
    z = O.gemv_qmat(m, x.astype(np.float64))
    assert z[0, 17] == 2.0 and z[0, 3000] == 1.5 and np.count_nonzero(z[0]) == 5
    dm = q.DeviceQMat(m)
    tok = torch.full((rows,), -1, dtype=torch.int32, device="cuda")
    top2 = torch.zeros((rows, 2), dtype=torch.float32, device="cuda")
    wsb = q.ocrdec_lm_argmax_workspace_bytes(dm.desc, rows)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    q.ocrdec_lm_argmax(dm.desc, rows, f16_tensor(x), tok, top2, ws, wsb)
    torch.cuda.synchronize()
    assert tok.cpu().numpy().tolist() == [17, 17, 17]
    assert top2.cpu().numpy().tolist() == [[2.0, 2.0]] * rows
