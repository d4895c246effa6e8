"""GPU parity of ocrdec_prefill (the prompt pass of one row) against the oracle.

Routing is teacher-forced to the oracle's choice while the GPU still reports
its own choice, which must equal the oracle's except at logged near-ties.
Compared: every layer's keys and values at cache indices 0..P-1 (fp16 rule),
the residual after the last layer at every position (fp32 rule), the argmax at
the last position, and that nothing else in the caches changed.
"""
import numpy as np
import pytest

import oracle as O
import synth
from tests.gpu_util import NEAR_TIE, assert_close, assert_close_f16, f16_tensor, log_near_tie

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import torch
    assert torch.cuda.is_available()
    import quantized_decode_step_amd as qd
    return qd


def small_dims(**kw):
    d = synth.Dims(hidden=256, n_heads=2, head_dim=128, n_layers=3, n_dense=1, dense_ff=512, n_experts=16, top_k=6,
                   n_shared=2, expert_ff=128, vocab=1000, prefix_cap=300, ring_cap=8)
    for k_, v_ in kw.items():
        setattr(d, k_, v_)
    return d


# Prompt passes into INT8 caches: every key and value row is quantised, and a
# value within rounding noise of a code boundary flips a whole code step that
# the next layers amplify.  The oracle's own residual moves by up to 8.4e-3 rms
# under float32-size input noise (tests/golden/int8_prefill_sensitivity.py),
# so the residual is held to 2e-2 rms and decisions may differ where the
# oracle's gap is below 1e-2 (as for the composed 12-layer decoder).
INT8_TOL, INT8_TIE = 2e-2, 1e-2


def run_prefill(q, d, seed, P, row=0, rows=1, use_emb=False, forced=True, int8_kv=False):
    import torch
    print("[case] prefill", d.n_layers, "layers H", d.hidden, "P", P, "row", row, "of", rows, "emb", use_emb,
          "int8 kv" if int8_kv else "", "seed", seed, flush=True)
    model = synth.make_model(d, seed)
    if int8_kv:
        st = synth.make_state_int8(d, seed, [d.prefix_cap // 2] * rows, [3] * rows)
    else:
        st = synth.make_state(d, seed, [d.prefix_cap // 2] * rows, [3] * rows)
    tok = synth.uniform_i32(synth.stream_id(seed, "prompt"), (P,), 0, d.vocab)
    emb = synth.normal_f16(synth.stream_id(seed, "prompt_emb"), (P, d.hidden)) if use_emb else None
    res = O.prefill(model, P, tok=None if use_emb else tok, emb=None if emb is None else emb.astype(np.float64),
                    int8_kv=int8_kv)
    n_moe = len(res.topk_idx)
    dm = q.DeviceModel(model)
    ds = q.DeviceState(st, d.prefix_cap, d.ring_cap)
    dm.bind_caches(ds.k_cache, ds.v_cache, ds.k_scale, ds.v_scale)
    k_before = ds.k_cache.cpu().numpy().copy()
    wsb = q.ocrdec_prefill_workspace_bytes(dm.desc, ds.desc, P)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    K = d.top_k
    cap_idx = torch.zeros((max(n_moe, 1), P, K), dtype=torch.int32, device="cuda")
    cap_w = torch.zeros((max(n_moe, 1), P, K), dtype=torch.float32, device="cuda")
    top2 = torch.zeros((1, 2), dtype=torch.float32, device="cuda")
    cap = q.StepCapture(cap_idx.data_ptr(), cap_w.data_ptr(), top2.data_ptr())
    hidden = torch.zeros((P, d.hidden), dtype=torch.float32, device="cuda")
    tok_out = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    forced_t = torch.from_numpy(np.array(res.topk_idx, np.int32)).cuda() if (forced and n_moe) else None
    tok_t = torch.from_numpy(tok.astype(np.int32)).cuda()
    emb_t = f16_tensor(emb) if use_emb else None
    q.ocrdec_prefill(dm.desc, ds.desc, row, P, tok=None if use_emb else tok_t, emb=emb_t, forced_topk=forced_t,
                     tok_out=tok_out, hidden=hidden, capture=cap, ws=ws, ws_bytes=wsb)
    torch.cuda.synchronize()
    kc = ds.k_cache.cpu().numpy()
    if int8_kv:
        vc = ds.v_cache.cpu().numpy()
        ks = ds.k_scale.cpu().numpy().view(np.float16)
        vs = ds.v_scale.cpu().numpy().view(np.float16)
        for l in range(d.n_layers):
            for what, c, s, oq, os_ in (("keys", kc, ks, res.kq[l], res.ks[l]), ("values", vc, vs, res.vq[l], res.vs[l])):
                g = O.kv_dequant(c[l, row, :, :P], s[l, row, :, :P])
                o = O.kv_dequant(oq, os_)
                bound = 2e-3 * np.sqrt(np.mean(o * o)) + 2 * os_.astype(np.float64)[..., None]
                assert np.all(np.abs(g - o) <= bound), "layer %d %s" % (l, what)
                if l == 0:
                    # first layer: both sides quantise fp16 keys that rarely differ, so codes rarely do;
                    # deeper layers inherit the residual's 1e-3-level differences, one code step apart
                    # wherever a value sits near a rounding boundary
                    assert np.mean(c[l, row, :, :P] == oq) > 0.99, "layer %d %s codes" % (l, what)
    else:
        vc = ds.v_cache.cpu().numpy().view(np.float16)
        for l in range(d.n_layers):
            assert_close_f16(kc.view(np.float16)[l, row, :, :P].astype(np.float64), res.k[l], "layer %d keys" % l)
            assert_close_f16(vc[l, row, :, :P].astype(np.float64), res.v[l], "layer %d values" % l)
    # nothing outside row `row`, indices 0..P-1 was written
    mask = np.ones(kc.shape, bool)
    mask[:, row, :, :P] = False
    assert np.array_equal(kc[mask], k_before[mask])
    ties = []
    tie, tol = (INT8_TIE, INT8_TOL) if int8_kv else (NEAR_TIE, 2e-3)
    g_idx = cap_idx.cpu().numpy()
    for ml in range(n_moe):
        for t in range(P):
            if not np.array_equal(g_idx[ml, t], res.topk_idx[ml][t]):
                gap = res.router_gap[ml][t]
                assert gap < tie, "moe layer %d position %d: routing differs, oracle gap %.3g" % (ml, t, gap)
                ties.append(("route", ml, t, gap))
        assert_close(cap_w.cpu().numpy()[ml], res.topk_w[ml], "moe layer %d weights" % ml, tol)
    assert_close(hidden.cpu().numpy(), res.hidden, "hidden after the last layer", tol)
    g_tok = int(tok_out.cpu().numpy()[0])
    if g_tok != int(res.tok):
        gap = res.lm_top2[0] - res.lm_top2[1]
        assert gap < tie, "token %d vs oracle %d, oracle gap %.3g" % (g_tok, res.tok, gap)
        ties.append(("token", gap))
    for t_ in ties:
        log_near_tie(t_[0], "prompt pass " + " ".join(str(v) for v in t_[1:-1]), t_[-1])
    return res, dm, ds, model, st


# P = 1 (one position), a ragged block of 19 (the MoE's single-workgroup
# routing), 64 (one full query block), 70 and 257 (several query blocks and
# the MoE's GEMM path)
@pytest.mark.parametrize("P", [1, 19, 64, 70, 257])
def test_prefill_small_tokens(q, P):
    run_prefill(q, small_dims(), 600 + P, P)


def test_prefill_input_features_row_offset(q):
    """fp16 input features instead of tokens, written into row 2 of 3."""
    run_prefill(q, small_dims(), 611, 45, row=2, rows=3, use_emb=True)


def test_prefill_unforced_head_dim_64(q):
    d = small_dims(n_heads=4, head_dim=64)
    run_prefill(q, d, 612, 100, forced=False)


def test_prefill_quantised_embed_and_head(q):
    d = small_dims(fmt_embed=synth.Q4_0, fmt_lm=synth.Q8_0)
    run_prefill(q, d, 613, 33)


@pytest.mark.parametrize("P", [40, 257])
def test_prefill_int8_kv_cache(q, P):
    """The prompt pass into INT8 caches: codes and scales as the oracle stores
    them (dequantised within one code step plus the fp16 rule), and the
    residual after attending over the stored values."""
    run_prefill(q, small_dims(), 630 + P, P, row=1, rows=2, int8_kv=True)


def test_prefill_full_width_two_layers(q):
    """Full hidden size and head layout, one dense and one MoE layer, a
    1100-position prompt (the decode workload's prefix)."""
    d = synth.dims_full()
    d.n_layers = 2
    d.vocab = 5000
    run_prefill(q, d, 614, 1100, use_emb=True)


def test_prefill_then_decode(q):
    """After the prompt pass, decode steps continue from it: the state says
    prefix_len = P, gen_index = 0, and the step's token goes to RoPE position P."""
    import torch
    d = small_dims()
    P = 37
    res, dm, ds, model, st = run_prefill(q, d, 615, P)
    ost = st.copy()
    ost.prefix_len[0] = P
    ost.gen_index[0] = 0
    kc = ds.k_cache.cpu().numpy().view(np.float16)
    vc = ds.v_cache.cpu().numpy().view(np.float16)
    ost.k_cache[:, 0] = kc[:, 0]
    ost.v_cache[:, 0] = vc[:, 0]
    ds.prefix_len.fill_(P)
    ds.gen_index.zero_()
    wsb = q.ocrdec_step_workspace_bytes(dm.desc, ds.desc)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    tok = np.array([res.tok], np.int32)
    for step in range(3):
        ores = O.decode_step(model, ost, tok_in=tok)
        tok_out = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        hidden = torch.zeros((1, d.hidden), dtype=torch.float32, device="cuda")
        forced = torch.from_numpy(np.array(ores.topk_idx, np.int32)).cuda()
        q.ocrdec_decode_step(dm.desc, ds.desc, torch.from_numpy(tok).cuda(), hidden, tok_out, forced, None, ws, wsb)
        torch.cuda.synchronize()
        assert_close(hidden.cpu().numpy(), ores.hidden, "decode step %d hidden" % step)
        g = int(tok_out.cpu().numpy()[0])
        if g != int(ores.tok[0]):
            assert ores.lm_top2[0, 0] - ores.lm_top2[0, 1] < NEAR_TIE
        tok = ores.tok.astype(np.int32)


@pytest.mark.parametrize("Ps,rows_used,use_emb", [([19, 70, 3], [2, 0, 3], False), ([130, 64, 257, 1], [1, 3, 0, 2], True)])
def test_prefill_batch_matches_each_sequence(q, Ps, rows_used, use_emb):
    """Several prompt passes in one call: every sequence's caches, residual,
    routing and first token equal the oracle's prompt pass of that sequence
    alone (routing teacher-forced, packed in sequence order)."""
    import torch
    d = small_dims()
    seed = 620 + len(Ps)
    print("[case] prefill batch", Ps, "rows", rows_used, "emb", use_emb, flush=True)
    model = synth.make_model(d, seed)
    st = synth.make_state(d, seed, [d.prefix_cap // 2] * 4, [3] * 4)
    res, toks, embs = [], [], []
    for i, P in enumerate(Ps):
        tk = synth.uniform_i32(synth.stream_id(seed, "prompt", i), (P,), 0, d.vocab)
        em = synth.normal_f16(synth.stream_id(seed, "prompt_emb", i), (P, d.hidden))
        toks.append(tk)
        embs.append(em)
        res.append(O.prefill(model, P, tok=None if use_emb else tk, emb=em.astype(np.float64) if use_emb else None))
    T = sum(Ps)
    n_moe = len(res[0].topk_idx)
    forced = np.concatenate([np.array(r.topk_idx, np.int32) for r in res], axis=1)
    dm = q.DeviceModel(model)
    ds = q.DeviceState(st, d.prefix_cap, d.ring_cap)
    dm.bind_caches(ds.k_cache, ds.v_cache)
    wsb = q.ocrdec_prefill_batch_workspace_bytes(dm.desc, ds.desc, rows_used, Ps)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    K = d.top_k
    cap_idx = torch.zeros((n_moe, T, K), dtype=torch.int32, device="cuda")
    top2 = torch.zeros((len(Ps), 2), dtype=torch.float32, device="cuda")
    cap = q.StepCapture(cap_idx.data_ptr(), None, top2.data_ptr())
    hidden = torch.zeros((T, d.hidden), dtype=torch.float32, device="cuda")
    tok_out = torch.full((len(Ps),), -1, dtype=torch.int32, device="cuda")
    tok_t = torch.from_numpy(np.concatenate(toks).astype(np.int32)).cuda()
    emb_t = f16_tensor(np.concatenate(embs))
    q.ocrdec_prefill_batch(dm.desc, ds.desc, rows_used, Ps, tok=None if use_emb else tok_t,
                           emb=emb_t if use_emb else None, forced_topk=torch.from_numpy(forced).cuda(),
                           tok_out=tok_out, hidden=hidden, capture=cap, ws=ws, ws_bytes=wsb)
    torch.cuda.synchronize()
    kc = ds.k_cache.cpu().numpy().view(np.float16)
    vc = ds.v_cache.cpu().numpy().view(np.float16)
    hid = hidden.cpu().numpy()
    g_idx = cap_idx.cpu().numpy()
    g_tok = tok_out.cpu().numpy()
    off = 0
    for i, P in enumerate(Ps):
        r = rows_used[i]
        for l in range(d.n_layers):
            assert_close_f16(kc[l, r, :, :P].astype(np.float64), res[i].k[l], "seq %d layer %d keys" % (i, l))
            assert_close_f16(vc[l, r, :, :P].astype(np.float64), res[i].v[l], "seq %d layer %d values" % (i, l))
        assert_close(hid[off:off + P], res[i].hidden, "seq %d hidden" % i)
        for ml in range(n_moe):
            for t_ in range(P):
                if not np.array_equal(g_idx[ml, off + t_], res[i].topk_idx[ml][t_]):
                    assert res[i].router_gap[ml][t_] < NEAR_TIE
        if g_tok[i] != int(res[i].tok):
            assert res[i].lm_top2[0] - res[i].lm_top2[1] < NEAR_TIE
        off += P
