"""Parity at full size, in the launch configurations the benchmark times.

* The 12-layer decoder at 1, 6, 12 and 24 rows (prefix 1100), layer by
  layer: each layer run alone from the oracle's own input to that layer, for
  the sampled rows, at generation index 124 and 128 (ring just wrapped),
  against tests/golden/decode_layers_r24.npz and decode_layers_r1_6_12.npz
  (written by make_decode_fixture.py from the oracle alone).  Each layer's
  residual must be within 2e-3 * rms.  The row counts cover every launch
  path of the step (one row, norms staged in the consumers and the merge in
  the O projection up to 16 rows, the separate kernels above).
* One row over 64 consecutive steps from generation index 100 (the ring wraps
  at step 28), teacher-forced, against decode_r1_64.npz.
* The same decoder composed over 8 steps (the ring wraps after four), rows
  0, 11 and 23 against tests/golden/decode_full_r24.npz, with tokens and the
  sampled rows' routing forced to the oracle's: the GPU's own routing and
  tokens bit-exact except near-ties within TRAJ_NEAR_TIE; the composed
  hidden state, routing weights and the last layer's new keys within
  TRAJ_TOL; both bounds derived from the oracle's own sensitivity (below).
* The prefill-shaped MoE layer: 2048 tokens, router bias, Q4_0 experts.
* The sink-augmented attention block with int8-asymmetric projections:
  hidden 512, 8 heads of 64, 350 and 3000 cached positions.
"""
import os

import numpy as np
import pytest

import oracle as O
import synth
from tests.gpu_util import NEAR_TIE, assert_close, assert_close_f16, f16_tensor, from_f16_tensor, log_near_tie

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# The composed 12-layer residual cannot meet 2e-3 * rms against the oracle for
# any fp32 implementation: perturbing only the oracle's own matrix-vector
# products by relative noise of 3e-7 (fp32 accumulation size), with its routing
# held fixed, moves its hidden state by up to 5.0e-3 * rms (median <= 1e-3)
# and its router logits by up to 3.3e-3, because the fp16 storage points turn
# the noise into whole-ulp flips that compound from layer to layer
# (tests/golden/decode_sensitivity.py measures it).  The trajectory bounds are
# twice the hidden-state spread and three times the logit spread (a decision
# compares two logits); each single layer, from the oracle's input, is held to
# 2e-3 * rms and the 1e-3 near-tie rule.
TRAJ_TOL = 1e-2
TRAJ_MEDIAN_TOL = 2e-3
TRAJ_NEAR_TIE = 1e-2


@pytest.fixture(scope="module")
def q():
    import torch
    assert torch.cuda.is_available()
    import quantized_decode_step_amd as qd
    return qd


@pytest.fixture(scope="module")
def full_model(q):
    fx = np.load(os.path.join(GOLDEN, "decode_layers_r24.npz"))
    d = synth.dims_full()
    model = synth.make_model(d, int(fx["seed"]))
    return d, model, q.DeviceModel(model)


class _Prefixed:
    """Keys of one row count in a fixture file that holds several."""

    def __init__(self, fx, prefix):
        self.fx, self.prefix = fx, prefix

    def __getitem__(self, k):
        return self.fx[self.prefix + k] if k not in ("seed",) else self.fx[k]


def _layer_fixture(R):
    if R == 24:
        fx = np.load(os.path.join(GOLDEN, "decode_layers_r24.npz"))
        return fx, [int(r) for r in fx["sampled"]], int(fx["seed"])
    fx = np.load(os.path.join(GOLDEN, "decode_layers_r1_6_12.npz"))
    pf = _Prefixed(fx, "r%d_" % R)
    return pf, [int(r) for r in pf["sampled"]], int(fx["seed"])


@pytest.mark.parametrize("R", [1, 6, 12, 24])
@pytest.mark.parametrize("case", ["a", "b"])
def test_decode_full_each_layer(q, full_model, R, case):
    """Every layer of the full decoder, run alone (launch as in the benchmark
    at that row count) from the oracle's residual entering it; the last one
    also runs the final norm, the LM head and the argmax."""
    import torch
    fx, sampled, seed = _layer_fixture(R)
    t = int(fx[case + "_t"])
    d, model, dm = full_model
    print("[case] full decoder per layer R=%d t=%d sampled=%s seed=%d" % (R, t, sampled, seed), flush=True)
    st = synth.make_state(d, seed, [d.prefix_cap] * R, [t] * R)
    ds = q.DeviceState(st, d.prefix_cap, d.ring_cap)
    del st
    dm.bind_caches(ds.k_cache, ds.v_cache)
    K, H = d.top_k, d.hidden
    cap_idx = torch.zeros((1, R, K), dtype=torch.int32, device="cuda")
    cap_w = torch.zeros((1, R, K), dtype=torch.float32, device="cuda")
    top2 = torch.zeros((R, 2), dtype=torch.float32, device="cuda")
    cap = q.StepCapture(cap_idx.data_ptr(), cap_w.data_ptr(), top2.data_ptr())
    tok_out = torch.zeros(R, dtype=torch.int32, device="cuda")
    layer_in = fx[case + "_layer_in"].astype(np.float64)      # [L][2][H]
    slot = d.prefix_cap + t % d.ring_cap
    moe_l = 0
    worst = 0.0
    for l in range(d.n_layers):
        last = l == d.n_layers - 1
        view = dm.layer_view(l, 1, with_head=last)
        ds.gen_index.fill_(t)
        if l == 0:
            hidden = torch.zeros((R, H), dtype=torch.float32, device="cuda")
            tin = torch.from_numpy(fx[case + "_tok_in"].astype(np.int32)).cuda()
        else:
            # rows that are not sampled carry unrelated inputs of the same scale
            scale = np.sqrt(np.mean(layer_in[l] ** 2))
            h_in = synth.normal_f64(synth.stream_id(seed, "layer-fill", t, l), (R, H)) * scale
            h_in[sampled] = layer_in[l]
            hidden = torch.from_numpy(h_in.astype(np.float32)).cuda()
            tin = None
        wsb = q.ocrdec_step_workspace_bytes(view, ds.desc)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        q.ocrdec_decode_step(view, ds.desc, tin, hidden, tok_out if last else None, None, cap, ws, wsb)
        torch.cuda.synchronize()
        assert np.all(ds.gen_index.cpu().numpy() == t + 1)
        g_hid = hidden.cpu().numpy().astype(np.float64)
        ref_out = fx[case + "_hidden"] if last else fx[case + "_layer_in"][l + 1]
        kc = ds.k_cache[l].cpu().numpy().view(np.float16)
        vc = ds.v_cache[l].cpu().numpy().view(np.float16)
        for i, r in enumerate(sampled):
            what = "case %s layer %d row %d" % (case, l, r)
            assert_close_f16(kc[r, :, slot].astype(np.float64), fx[case + "_new_k"][l][i], what + " new k")
            assert_close_f16(vc[r, :, slot].astype(np.float64), fx[case + "_new_v"][l][i], what + " new v")
            if model.layers[l].is_moe:
                g_idx = cap_idx[0, r].cpu().numpy()
                if not np.array_equal(g_idx, fx[case + "_topk_idx"][moe_l][i]):
                    gap = fx[case + "_router_gap"][moe_l][i]
                    assert gap < NEAR_TIE, "%s: routing differs (gap %.3g)" % (what, gap)
                    log_near_tie("routing", what, gap)
                    continue
                assert_close(cap_w[0, r].cpu().numpy(), fx[case + "_topk_w"][moe_l][i], what + " routing weights")
            worst = max(worst, assert_close(g_hid[r], ref_out[i], what + " residual"))
            if last:
                g_tok = int(tok_out[r].item())
                if g_tok != fx[case + "_tok"][i]:
                    gap = fx[case + "_lm_top2"][i][0] - fx[case + "_lm_top2"][i][1]
                    assert gap < NEAR_TIE, "%s: token %d vs %d (gap %.3g)" % (what, g_tok, fx[case + "_tok"][i], gap)
                    log_near_tie("token", what, gap)
        if model.layers[l].is_moe:
            moe_l += 1
    print("[result] R=%d case %s: worst per-layer residual error %.3g rms" % (R, case, worst))


def test_decode_full_12_layers_24_rows(q, full_model):
    """Eight composed steps; tokens are teacher-forced and the sampled rows'
    routing is forced to the oracle's, so a near-tie (where both choices are
    correct) does not part the trajectories.  The GPU still reports its own
    choice, which must equal the oracle's except at logged near-ties."""
    import torch
    fx = np.load(os.path.join(GOLDEN, "decode_full_r24.npz"))
    seed, R, t0, steps = int(fx["seed"]), int(fx["rows"]), int(fx["t0"]), int(fx["steps"])
    sampled = [int(r) for r in fx["sampled"]]
    print("[case] full decoder R=%d t0=%d steps=%d sampled=%s seed=%d" % (R, t0, steps, sampled, seed), flush=True)
    d, _, dm = full_model
    assert seed == int(np.load(os.path.join(GOLDEN, "decode_layers_r24.npz"))["seed"])
    st = synth.make_state(d, seed, [d.prefix_cap] * R, [t0] * R)
    ds = q.DeviceState(st, d.prefix_cap, d.ring_cap)
    del st
    dm.bind_caches(ds.k_cache, ds.v_cache)
    wsb = q.ocrdec_step_workspace_bytes(dm.desc, ds.desc)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    n_moe = int(fx["n_moe"])
    K = d.top_k
    cap_idx = torch.zeros((n_moe, R, K), dtype=torch.int32, device="cuda")
    cap_w = torch.zeros((n_moe, R, K), dtype=torch.float32, device="cuda")
    top2 = torch.zeros((R, 2), dtype=torch.float32, device="cuda")
    cap = q.StepCapture(cap_idx.data_ptr(), cap_w.data_ptr(), top2.data_ptr())
    hidden = torch.zeros((R, d.hidden), dtype=torch.float32, device="cuda")
    tok_out = torch.zeros(R, dtype=torch.int32, device="cuda")
    tok = synth.first_tokens(d, seed, R)
    ties = 0
    for step in range(steps):
        tok[sampled] = fx["tok_in"][step]
        forced = np.full((n_moe, R, K), -1, np.int32)
        forced[:, sampled] = fx["topk_idx"][step]
        q.ocrdec_decode_step(dm.desc, ds.desc, torch.from_numpy(tok).cuda(), hidden, tok_out,
                             torch.from_numpy(forced).cuda(), cap, ws, wsb)
        torch.cuda.synchronize()
        g_tok = tok_out.cpu().numpy()
        assert np.all((g_tok >= 0) & (g_tok < d.vocab))
        g_idx, g_w = cap_idx.cpu().numpy(), cap_w.cpu().numpy()
        g_hid = hidden.cpu().numpy().astype(np.float64)
        kc = ds.k_cache.cpu().numpy().view(np.float16) if step in (0, steps - 1) else None
        for i, r in enumerate(sampled):
            # the GPU's own routing: bit-exact unless the oracle's gap is a near-tie
            for ml in range(n_moe):
                if not np.array_equal(g_idx[ml, r], fx["topk_idx"][step][ml][i]):
                    gap = fx["router_gap"][step][ml][i]
                    assert gap < TRAJ_NEAR_TIE, "step %d layer %d row %d: routing differs (gap %.3g)" % (
                        step, ml, r, gap)
                    log_near_tie("routing", "R=24 trajectory step %d layer %d row %d" % (step, ml, r), gap)
                    ties += 1
            assert_close(g_w[:, r], fx["topk_w"][step][:, i], "step %d row %d routing weights" % (step, r),
                         tol=TRAJ_TOL)
            assert_close(g_hid[r], fx["hidden"][step][i], "step %d row %d hidden" % (step, r), tol=TRAJ_TOL)
            dev = np.abs(g_hid[r] - fx["hidden"][step][i]) / np.sqrt(np.mean(fx["hidden"][step][i] ** 2.0))
            assert np.median(dev) <= TRAJ_MEDIAN_TOL, "step %d row %d hidden: median %.3g" % (step, r, np.median(dev))
            if g_tok[r] != fx["tok"][step][i]:
                gap = fx["lm_top2"][step][i][0] - fx["lm_top2"][step][i][1]
                assert gap < TRAJ_NEAR_TIE, "step %d row %d: token %d vs %d (gap %.3g)" % (
                    step, r, g_tok[r], fx["tok"][step][i], gap)
                log_near_tie("token", "R=24 trajectory step %d row %d" % (step, r), gap)
            if kc is not None:
                slot = d.prefix_cap + (t0 + step) % d.ring_cap
                assert_close_f16(kc[0, r, :, slot].astype(np.float64), fx["new_k_first"][step][i], "layer 0 new k")
                assert_close_f16(kc[-1, r, :, slot].astype(np.float64), fx["new_k_last"][step][i], "last layer new k",
                                 tol=TRAJ_TOL)
        tok = g_tok.copy()
    decisions = steps * n_moe * len(sampled)
    assert ties <= 0.05 * decisions, "%d routing near-ties among %d decisions" % (ties, decisions)
    assert np.all(ds.gen_index.cpu().numpy() == t0 + steps)


def test_decode_full_one_row_64_steps(q, full_model):
    """One row, 64 consecutive steps from generation index 100: the ring wraps
    at step 28 and the window then slides over the ring.  Tokens are
    teacher-forced and routing forced to the oracle's (so a near-tie cannot
    part the two runs); the GPU's own routing and tokens must equal the
    oracle's except at near-ties; the hidden state and routing weights are
    held to the composed-decoder bounds above."""
    import torch
    fx = np.load(os.path.join(GOLDEN, "decode_r1_64.npz"))
    seed, t0, steps = int(fx["seed"]), int(fx["t0"]), int(fx["steps"])
    key_steps = [int(s) for s in fx["key_steps"]]
    print("[case] full decoder R=1 t0=%d steps=%d seed=%d" % (t0, steps, seed), flush=True)
    d, _, dm = full_model
    st = synth.make_state(d, seed, [d.prefix_cap], [t0])
    ds = q.DeviceState(st, d.prefix_cap, d.ring_cap)
    del st
    dm.bind_caches(ds.k_cache, ds.v_cache)
    wsb = q.ocrdec_step_workspace_bytes(dm.desc, ds.desc)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    n_moe, K = d.n_layers - d.n_dense, d.top_k
    cap_idx = torch.zeros((n_moe, 1, K), dtype=torch.int32, device="cuda")
    cap_w = torch.zeros((n_moe, 1, K), dtype=torch.float32, device="cuda")
    top2 = torch.zeros((1, 2), dtype=torch.float32, device="cuda")
    cap = q.StepCapture(cap_idx.data_ptr(), cap_w.data_ptr(), top2.data_ptr())
    hidden = torch.zeros((1, d.hidden), dtype=torch.float32, device="cuda")
    tok_out = torch.zeros(1, dtype=torch.int32, device="cuda")
    ties, worst, medians = 0, 0.0, []
    for step in range(steps):
        forced = torch.from_numpy(fx["topk_idx"][step].reshape(n_moe, 1, K).astype(np.int32)).cuda()
        q.ocrdec_decode_step(dm.desc, ds.desc, torch.from_numpy(fx["tok_in"][step].astype(np.int32)).cuda(), hidden,
                             tok_out, forced, cap, ws, wsb)
        torch.cuda.synchronize()
        g_idx, g_w = cap_idx.cpu().numpy()[:, 0], cap_w.cpu().numpy()[:, 0]
        for ml in range(n_moe):
            if not np.array_equal(g_idx[ml], fx["topk_idx"][step][ml][0]):
                gap = fx["router_gap"][step][ml][0]
                assert gap < TRAJ_NEAR_TIE, "step %d layer %d: routing differs (gap %.3g)" % (step, ml, gap)
                log_near_tie("routing", "R=1 64-step run step %d layer %d" % (step, ml), gap)
                ties += 1
        assert_close(g_w, fx["topk_w"][step][:, 0], "step %d routing weights" % step, tol=TRAJ_TOL)
        g_hid = hidden.cpu().numpy()[0].astype(np.float64)
        ref = fx["hidden"][step][0]
        worst = max(worst, assert_close(g_hid, ref, "step %d hidden" % step, tol=TRAJ_TOL))
        medians.append(np.median(np.abs(g_hid - ref)) / np.sqrt(np.mean(ref ** 2.0)))
        assert medians[-1] <= TRAJ_MEDIAN_TOL, "step %d hidden: median %.3g" % (step, medians[-1])
        g_tok = int(tok_out.item())
        if g_tok != fx["tok"][step][0]:
            gap = fx["lm_top2"][step][0][0] - fx["lm_top2"][step][0][1]
            assert gap < TRAJ_NEAR_TIE, "step %d: token %d vs %d (gap %.3g)" % (step, g_tok, fx["tok"][step][0], gap)
            log_near_tie("token", "R=1 64-step run step %d" % step, gap)
        if step in key_steps:
            slot = d.prefix_cap + (t0 + step) % d.ring_cap
            kc = ds.k_cache[-1, 0, :, slot].cpu().numpy().view(np.float16).astype(np.float64)
            assert_close_f16(kc, fx["new_k_last"][key_steps.index(step)][0], "step %d last layer new k" % step,
                             tol=TRAJ_TOL)
    assert int(ds.gen_index.item()) == t0 + steps
    assert ties <= 0.05 * steps * n_moe
    print("[result] R=1 64 steps: worst hidden %.3g rms, worst median %.3g, routing near-ties %d" % (
        worst, max(medians), ties))


class _Lay:
    pass


def test_moe_prefill_2048_tokens(q):
    import torch
    seed, T = 1005, 2048
    print("[case] prefill-shaped MoE T=%d seed=%d" % (T, seed), flush=True)
    d = synth.Dims(fmt_router=synth.Q8_0, fmt_expert=synth.Q4_0, fmt_shared=synth.Q4_0)
    lay = _Lay()
    for k_, v_ in synth.make_moe_weights(d, seed, 0, with_bias=True).items():
        setattr(lay, k_, v_)
    x = synth.normal_f16(synth.stream_id(seed, "x"), (T, d.hidden))
    w, keep = q.moe_weights(lay, d.hidden, d.top_k)
    xd = f16_tensor(x)
    out = torch.zeros((T, d.hidden), dtype=torch.int16, device="cuda")
    cap_idx = torch.zeros((T, d.top_k), dtype=torch.int32, device="cuda")
    counts = torch.zeros(d.n_experts, dtype=torch.int32, device="cuda")
    offsets = torch.zeros(d.n_experts + 1, dtype=torch.int32, device="cuda")
    perm = torch.zeros(T * d.top_k, dtype=torch.int32, device="cuda")
    cap = q.MoeCapture(cap_idx.data_ptr(), None, counts.data_ptr(), offsets.data_ptr(), perm.data_ptr())
    wsb = q.ocrdec_moe_workspace_bytes(w, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    q.ocrdec_moe_layer(w, T, xd, out, False, None, cap, ws, wsb)
    torch.cuda.synchronize()
    ref, idx, wt, logits = O.moe(lay, x.astype(np.float64), d.top_k)
    g_idx = cap_idx.cpu().numpy()
    ties = [t for t in range(T) if not np.array_equal(g_idx[t], idx[t])]
    for t in ties:
        gap = O.topk_gap(logits[t], d.top_k, lay.router_bias)
        assert gap < NEAR_TIE, "token %d routing differs with gap %.3g" % (t, gap)
        log_near_tie("routing", "prefill-shaped MoE token %d" % t, gap)
    if not ties:
        c, o, p, _ = O.group(idx, d.n_experts)
        assert np.array_equal(counts.cpu().numpy(), c)
        assert np.array_equal(offsets.cpu().numpy(), o)
        assert np.array_equal(perm.cpu().numpy(), p)
    keep_rows = np.array([t for t in range(T) if t not in set(ties)])
    assert_close_f16(from_f16_tensor(out)[keep_rows], O.f16(ref)[keep_rows], "prefill MoE output")
    # the bias skews the loads: the busiest expert gets several times the mean
    cnt = np.bincount(idx.reshape(-1), minlength=d.n_experts)
    assert cnt.max() > 2 * cnt.mean()


@pytest.mark.parametrize("rows,L", [(1, 350), (24, 350), (6, 3000), (24, 3000)])
def test_sink_attention_block_u8a(q, rows, L):
    """x -> int8-asymmetric QKV -> RoPE(64) -> append at index L -> attention
    over the sink (index 0) and the L cached + 1 new keys -> int8-asymmetric O."""
    import torch
    seed = 1004
    H, NH, D = 512, 8, 64
    print("[case] sink block rows=%d L=%d seed=%d" % (rows, L, seed), flush=True)
    wqkv = synth.random_qmat(synth.U8A_G32, synth.stream_id(seed, "wqkv"), 3 * H, H)
    wo = synth.random_qmat(synth.U8A_G32, synth.stream_id(seed, "wo"), H, H)
    sink = O.f16(synth.normal_f64(synth.stream_id(seed, "sink"), (NH,)))
    x = synth.normal_f16(synth.stream_id(seed, "x", rows), (rows, H))
    cap = L + 1
    kc = synth.normal_f16(synth.stream_id(seed, "kc", L), (rows, NH, cap, D))
    vc = synth.normal_f16(synth.stream_id(seed, "vc", L), (rows, NH, cap, D))
    kc[:, :, 0] = 0    # the sink slot: zero key, zero value
    vc[:, :, 0] = 0
    kc[:, :, L:] = 0
    vc[:, :, L:] = 0
    dq, do = q.DeviceQMat(wqkv), q.DeviceQMat(wo)
    xd = f16_tensor(x)
    qkv = torch.zeros((rows, 3 * H), dtype=torch.float32, device="cuda")
    q.ocrdec_gemv_q(dq.desc, rows, xd, H, qkv, q.OCRDEC_OUT_F32, 3 * H)
    kd, vd = f16_tensor(kc), f16_tensor(vc)
    pl = torch.full((rows,), L, dtype=torch.int32, device="cuda")
    sk = torch.from_numpy(sink.astype(np.float32)).cuda()
    o = torch.zeros((rows, H), dtype=torch.int16, device="cuda")
    a = q.AttnArgs(rows, NH, D, qkv.data_ptr(), 3 * H, kd.data_ptr(), vd.data_ptr(), cap, 0, pl.data_ptr(), None,
                   sk.data_ptr(), 10000.0, 1.0 / 8.0, o.data_ptr(), H)
    wsb = q.ocrdec_attn_workspace_bytes(a)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    q.ocrdec_attn_decode(a, ws, wsb)
    y = torch.zeros((rows, H), dtype=torch.int16, device="cuda")
    q.ocrdec_gemv_q(do.desc, rows, o, H, y, q.OCRDEC_OUT_F16, H)
    torch.cuda.synchronize()
    g_y = from_f16_tensor(y)
    g_k = kd.cpu().numpy().view(np.float16)
    for r in range(rows):
        kcr, vcr = kc[r].copy(), vc[r].copy()
        ref_y, ref_k, ref_v, _ = O.sink_attention_block(wqkv, wo, x[r].astype(np.float64), kcr, vcr, L, sink, NH, D,
                                                        10000.0)
        assert_close_f16(g_y[r], ref_y, "sink block y row %d" % r)
        assert_close_f16(g_k[r][:, L].astype(np.float64), ref_k, "sink block new k row %d" % r)
