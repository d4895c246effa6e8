"""GPU parity of ocrdec_decode_step against the oracle over several steps.

Protocol (teacher forcing): every step feeds both sides the oracle's tokens and
gives the GPU the oracle's routing as forced experts, while the GPU still
reports the experts it would have chosen itself.  Its own choices and its
argmax tokens must equal the oracle's bit for bit, except where the oracle's
own logit gap is below the near-tie threshold (such cases are printed).  All
floating-point state (the final hidden state, every new cache slot, the routing
weights) is compared at every step.
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


def small_dims(**kw):
    d = synth.Dims(hidden=256, n_heads=2, head_dim=128, n_layers=3, n_dense=1, dense_ff=512, n_experts=16, top_k=6,
                   n_shared=2, expert_ff=128, vocab=1000, prefix_cap=40, ring_cap=8)
    for k_, v_ in kw.items():
        setattr(d, k_, v_)
    return d


def run_steps(q, d, seed, prefix_len, gen_index, n_steps, forced=True, sample_rows=None, check_cache=True,
              int8_kv=False):
    import torch
    R = len(prefix_len)
    print("[case] step", d.n_layers, "layers", "H", d.hidden, "V", d.vocab, "R", R, "steps", n_steps, "seed", seed,
          "int8 kv" if int8_kv else "", flush=True)
    model = synth.make_model(d, seed)
    st = synth.make_state_int8(d, seed, prefix_len, gen_index) if int8_kv else synth.make_state(d, seed, prefix_len,
                                                                                                    gen_index)
    dm = q.DeviceModel(model)
    ds = q.DeviceState(st, d.prefix_cap, d.ring_cap)
    dm.bind_caches(ds.k_cache, ds.v_cache, ds.k_scale, ds.v_scale)
    if int8_kv:
        check_cache = False  # the new slots are compared as stored values below
    wsb = q.ocrdec_step_workspace_bytes(dm.desc, ds.desc)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    n_moe = sum(1 for l in model.layers if l.is_moe)
    K = d.top_k
    cap_idx = torch.zeros((max(n_moe, 1), R, K), dtype=torch.int32, device="cuda")
    cap_w = torch.zeros((max(n_moe, 1), R, K), dtype=torch.float32, device="cuda")
    top2 = torch.zeros((R, 2), dtype=torch.float32, device="cuda")
    cap = q.StepCapture(cap_idx.data_ptr(), cap_w.data_ptr(), top2.data_ptr())
    hidden = torch.zeros((R, d.hidden), dtype=torch.float32, device="cuda")
    tok_out = torch.full((R,), -1, dtype=torch.int32, device="cuda")
    rows = list(range(R)) if sample_rows is None else list(sample_rows)
    tok = synth.first_tokens(d, seed, R)
    ost = st.copy()
    ties = []
    for step in range(n_steps):
        res = O.decode_step(model, ost, tok_in=tok, rows=rows)
        tok_in = torch.from_numpy(tok.astype(np.int32)).cuda()
        forced_t = None
        if forced and n_moe:
            f = np.full((n_moe, R, K), -1, np.int32)
            for ml in range(n_moe):
                f[ml, rows] = res.topk_idx[ml]
            forced_t = torch.from_numpy(f).cuda()
        q.ocrdec_decode_step(dm.desc, ds.desc, tok_in, hidden, tok_out, forced_t, cap, ws, wsb)
        torch.cuda.synchronize()
        g_tok = tok_out.cpu().numpy()[rows]
        g_hid = hidden.cpu().numpy().astype(np.float64)[rows]
        g_idx = cap_idx.cpu().numpy()[:, rows]
        g_w = cap_w.cpu().numpy()[:, rows]
        # routing decisions
        for ml in range(n_moe):
            for i, r in enumerate(rows):
                if not np.array_equal(g_idx[ml, i], res.topk_idx[ml][i]):
                    gap = res.router_gap[ml][i]
                    assert gap < NEAR_TIE, "step %d layer %d row %d: routing differs, oracle gap %.3g" % (
                        step, ml, r, gap)
                    ties.append(("route", step, ml, r, gap))
            assert_close(g_w[ml], res.topk_w[ml], "step %d moe layer %d weights" % (step, ml))
        # tokens
        for i, r in enumerate(rows):
            if g_tok[i] != res.tok[i]:
                gap = res.lm_top2[i, 0] - res.lm_top2[i, 1]
                assert gap < NEAR_TIE, "step %d row %d: token %d vs oracle %d, oracle gap %.3g" % (
                    step, r, g_tok[i], res.tok[i], gap)
                ties.append(("token", step, r, gap))
        e_hid = assert_close(g_hid, res.hidden, "step %d hidden" % step)
        if int8_kv:
            print("[int8 kv] step %d hidden max|gpu-oracle|/rms %.3g" % (step, e_hid), flush=True)
        if check_cache:
            kc = ds.k_cache.cpu().numpy().view(np.float16)
            vc = ds.v_cache.cpu().numpy().view(np.float16)
            for l in range(d.n_layers):
                for i, r in enumerate(rows):
                    t = int(st.gen_index[r]) + step
                    slot = d.prefix_cap + t % d.ring_cap
                    assert_close_f16(kc[l, r, :, slot].astype(np.float64), res.new_k[l][i],
                                     "step %d layer %d k" % (step, l))
                    assert_close_f16(vc[l, r, :, slot].astype(np.float64), res.new_v[l][i],
                                     "step %d layer %d v" % (step, l))
        if int8_kv:
            kc, ks = ds.k_cache.cpu().numpy(), ds.k_scale.cpu().numpy().view(np.float16)
            vc, vs = ds.v_cache.cpu().numpy(), ds.v_scale.cpu().numpy().view(np.float16)
            for l in range(d.n_layers):
                for i, r in enumerate(rows):
                    t = int(st.gen_index[r]) + step
                    slot = d.prefix_cap + t % d.ring_cap
                    for what, c, s, oc, os_ in (("k", kc, ks, ost.k_cache, ost.k_scale),
                                                ("v", vc, vs, ost.v_cache, ost.v_scale)):
                        g = O.kv_dequant(c[l, r, :, slot], s[l, r, :, slot])
                        o = O.kv_dequant(oc[l, r, :, slot], os_[l, r, :, slot])
                        bound = 2e-3 * np.sqrt(np.mean(o * o)) + 2 * os_[l, r, :, slot].astype(np.float64)[:, None]
                        assert np.all(np.abs(g - o) <= bound), "step %d layer %d new %s" % (step, l, what)
                # The codes are rounding decisions: a value within fp32 rounding
                # of a code boundary may take either code, and both are correct.
                # The device cache continues from the oracle's codes and scales
                # for the new slot (oracle values into the device state, never
                # the reverse), so that later steps compare attention over the
                # same cache instead of carrying such a flip forward.
                for i, r in enumerate(rows):
                    t = int(st.gen_index[r]) + step
                    slot = d.prefix_cap + t % d.ring_cap
                    for dc, dsc, oc, os_ in ((ds.k_cache, ds.k_scale, ost.k_cache, ost.k_scale),
                                             (ds.v_cache, ds.v_scale, ost.v_cache, ost.v_scale)):
                        dc[l, r, :, slot] = torch.from_numpy(np.ascontiguousarray(oc[l, r, :, slot], np.int8)).cuda()
                        dsc[l, r, :, slot] = torch.from_numpy(
                            np.ascontiguousarray(os_[l, r, :, slot], np.float16).view(np.int16)).cuda()
        gi = ds.gen_index.cpu().numpy()
        assert np.array_equal(gi[rows], ost.gen_index[rows])
        nxt = tok.copy()
        nxt[rows] = res.tok
        tok = nxt
    for t_ in ties:
        log_near_tie(t_[0], "step " + " ".join(str(v) for v in t_[1:-1]), t_[-1])
    return ties


def test_step_small_forced_ragged(q):
    d = small_dims()
    run_steps(q, d, 501, prefix_len=[40, 0, 17, 33, 1], gen_index=[0, 5, 7, 20, 3], n_steps=12)


def test_step_small_unforced(q):
    d = small_dims()
    run_steps(q, d, 502, prefix_len=[12, 40], gen_index=[6, 0], n_steps=10, forced=False)


def test_step_small_rows_32(q):
    d = small_dims(n_layers=2)
    run_steps(q, d, 503, prefix_len=[(7 * i) % 41 for i in range(32)], gen_index=[3 * i for i in range(32)],
              n_steps=3)


# Launch paths by row count: up to 16 rows the norms are formed inside the
# consuming kernels, from 17 rows the separate norm kernels run; up to 24
# rows the attention merge runs inside the O projection (in workgroups of four
# rows), from 25 rows the separate merge and O projection run; up to 32 rows
# the MoE down projection adds into the residual itself.  One row
# takes the single-row grouping.  Shared-expert counts 0..2 and top-k 1..8
# exercise the slot lists.
@pytest.mark.parametrize("R,ns,k", [(1, 0, 8), (1, 1, 1), (3, 2, 6), (5, 2, 6), (16, 2, 6), (17, 2, 6),
                                    (17, 1, 8), (24, 2, 6), (25, 2, 6)])
def test_step_rows_around_folded_combine(q, R, ns, k):
    d = small_dims(n_shared=ns, top_k=k)
    run_steps(q, d, 530 + 16 * R + 4 * ns + k, prefix_len=[(11 * i + 5) % 41 for i in range(R)],
              gen_index=[(5 * i + 2) % 9 for i in range(R)], n_steps=4)


# INT8 KV cache through the whole step (fused and separate combine paths)
@pytest.mark.parametrize("R", [1, 5])
def test_step_int8_kv_cache(q, R):
    d = small_dims()
    run_steps(q, d, 540 + R, prefix_len=[(13 * i + 7) % 41 for i in range(R)], gen_index=[(3 * i + 4) % 11 for i in range(R)],
              n_steps=10, int8_kv=True)


# quantised embedding tables and LM heads through the whole step (tokens from
# the table, argmax over the quantised head)
@pytest.mark.parametrize("fe,fl", [(synth.Q4_0, synth.Q4_0), (synth.Q8_0, synth.Q8_0), (synth.U8A_G32, synth.F16),
                                   (synth.F16, synth.Q4_0)])
def test_step_small_quantised_embed_and_head(q, fe, fl):
    d = small_dims(fmt_embed=fe, fmt_lm=fl)
    run_steps(q, d, 510 + 4 * fe + fl, prefix_len=[40, 9, 25], gen_index=[2, 7, 30], n_steps=6)


# a full-size vocabulary: the step's LM head runs on the CU-balanced kernel
def test_step_full_vocab_head(q):
    d = small_dims(n_layers=2, vocab=129280)
    run_steps(q, d, 520, prefix_len=[40, 3, 22, 31], gen_index=[1, 4, 9, 6], n_steps=3)


def test_step_single_dense_layer_fp16(q):
    """One dense fp16 decoder layer over 256 cached positions (no embedding or
    LM head: the hidden state goes in and comes out)."""
    import torch
    d = synth.dims_dense_layer()
    seed = 1001
    print("[case] dense fp16 layer", flush=True)
    model = synth.make_model(d, seed, with_embed=False, with_lm=False)
    st = synth.make_state(d, seed, [256], [0])
    h0 = synth.normal_f16(synth.stream_id(seed, "h0"), (1, d.hidden))
    dm = q.DeviceModel(model)
    ds = q.DeviceState(st, d.prefix_cap, d.ring_cap)
    dm.bind_caches(ds.k_cache, ds.v_cache)
    wsb = q.ocrdec_step_workspace_bytes(dm.desc, ds.desc)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    hidden = torch.from_numpy(h0.astype(np.float32)).cuda()
    q.ocrdec_decode_step(dm.desc, ds.desc, None, hidden, None, None, None, ws, wsb)
    torch.cuda.synchronize()
    res = O.decode_step(model, st.copy(), hidden_in=h0.astype(np.float64), with_lm=False)
    assert_close(hidden.cpu().numpy(), res.hidden, "dense layer hidden")


def test_step_single_moe_layer_q8(q):
    """One Q8_0 MoE decoder layer, prefix 1100 + a full ring (t = 128)."""
    import torch
    d = synth.dims_moe_layer()
    seed = 1002
    print("[case] moe q8 layer", flush=True)
    model = synth.make_model(d, seed, with_embed=False, with_lm=False)
    st = synth.make_state(d, seed, [1100], [128])
    h0 = synth.normal_f16(synth.stream_id(seed, "h0"), (1, d.hidden))
    dm = q.DeviceModel(model)
    ds = q.DeviceState(st, d.prefix_cap, d.ring_cap)
    dm.bind_caches(ds.k_cache, ds.v_cache)
    wsb = q.ocrdec_step_workspace_bytes(dm.desc, ds.desc)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    hidden = torch.from_numpy(h0.astype(np.float32)).cuda()
    cap_idx = torch.zeros((1, 1, d.top_k), dtype=torch.int32, device="cuda")
    cap = q.StepCapture(cap_idx.data_ptr(), None, None)
    # the oracle's routing is forced, so a near-tie (where both choices are
    # correct) cannot part the two results; the GPU still reports its own
    # choice, which must be the oracle's unless the oracle's gap is a near-tie
    res = O.decode_step(model, st.copy(), hidden_in=h0.astype(np.float64), with_lm=False)
    forced = torch.from_numpy(np.array(res.topk_idx, np.int32).reshape(1, 1, d.top_k)).cuda()
    q.ocrdec_decode_step(dm.desc, ds.desc, None, hidden, None, forced, cap, ws, wsb)
    torch.cuda.synchronize()
    if not np.array_equal(cap_idx.cpu().numpy()[0, 0], res.topk_idx[0][0]):
        assert res.router_gap[0][0] < NEAR_TIE
        log_near_tie("routing", "single MoE layer (Q8_0)", res.router_gap[0][0])
    assert_close(hidden.cpu().numpy(), res.hidden, "moe layer hidden")
