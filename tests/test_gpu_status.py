"""Reproducibility of the decode step and its device status word.

* Two runs of the same steps from identical inputs give the same bits: the
  tokens, every layer's routing and weights, the hidden state and the new
  cache slots.  The residual is accumulated in exact fixed point, so the
  order in which workgroups add their parts (atomic adds) cannot show.  Row
  counts cover every launch path of the step: the norm staged in the
  consumers and the merge inside the O projection (up to 16 rows), the
  separate merge, O projection and norm kernels (17-32 rows), and the down
  projection adding into the residual (up to 32 rows).
* ocrdec_device_status reports what the step cannot return synchronously
  (Falcon-OCR card, "Two traps the host must avoid": wrong inputs give
  degenerate output, not an error): a token id outside the vocabulary, a
  non-finite value entering the residual, a non-finite language-head logit.
  The conditions are made with ordinary arithmetic on the inputs (a NaN weight
  row, an out-of-range id, a huge hidden value), never with a fault.
"""
import numpy as np
import pytest

import oracle as O
import synth

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


def _run(q, dm, st, d, tok, n_steps):
    """n_steps decode steps from a fresh copy of st with tokens fed back on the
    device; returns every output as host arrays."""
    import torch
    R = len(st.prefix_len)
    ds = q.DeviceState(st.copy(), d.prefix_cap, d.ring_cap)
    dm.bind_caches(ds.k_cache, ds.v_cache)
    wsb = q.ocrdec_step_workspace_bytes(dm.desc, ds.desc)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    n_moe = d.n_layers - d.n_dense
    K = d.top_k
    out = []
    toks = torch.from_numpy(tok.astype(np.int32)).cuda()
    for _ in range(n_steps):
        cap_idx = torch.zeros((n_moe, R, K), dtype=torch.int32, device="cuda")
        cap_w = torch.zeros((n_moe, R, K), dtype=torch.float32, device="cuda")
        top2 = torch.zeros((R, 2), dtype=torch.float32, device="cuda")
        cap = q.StepCapture(cap_idx.data_ptr(), cap_w.data_ptr(), top2.data_ptr())
        hidden = torch.zeros((R, d.hidden), dtype=torch.float32, device="cuda")
        q.ocrdec_decode_step(dm.desc, ds.desc, toks, hidden, toks, None, cap, ws, wsb)
        torch.cuda.synchronize()
        out.append((toks.cpu().numpy().copy(), cap_idx.cpu().numpy(), cap_w.cpu().numpy(), top2.cpu().numpy(),
                    hidden.cpu().numpy()))
    assert q.ocrdec_device_status(ws, wsb) == 0
    return out, ds.k_cache.cpu().numpy(), ds.v_cache.cpu().numpy()


@pytest.mark.parametrize("R", [1, 6, 16, 17, 32])
def test_step_bitwise_reproducible(q, R):
    d = small_dims()
    seed = 600 + R
    print("[case] reproducibility R=%d seed=%d" % (R, seed), flush=True)
    model = synth.make_model(d, seed)
    st = synth.make_state(d, seed, [(7 * i + 3) % 41 for i in range(R)], [(5 * i + 1) % 13 for i in range(R)])
    tok = synth.first_tokens(d, seed, R)
    dm = q.DeviceModel(model)
    a, ka, va = _run(q, dm, st, d, tok, 4)
    b, kb, vb = _run(q, dm, st, d, tok, 4)
    for s, (x, y) in enumerate(zip(a, b)):
        for name, u, v in zip(("tokens", "routing", "routing weights", "top-2 logits", "hidden"), x, y):
            assert np.array_equal(u.view(np.uint8), v.view(np.uint8)), "step %d: %s differ between runs" % (s, name)
    assert np.array_equal(ka.view(np.uint8), kb.view(np.uint8)) and np.array_equal(va.view(np.uint8), vb.view(np.uint8))


def test_device_status_flags(q):
    import torch
    d = small_dims(n_layers=2)
    seed = 650
    print("[case] device status seed=%d" % seed, flush=True)
    model = synth.make_model(d, seed)
    R = 2
    st = synth.make_state(d, seed, [40, 12], [3, 0])
    # a NaN weight row in the language head: its logit is NaN for every row
    nan_row = 17
    lm = model.lm_head.data.view(np.float16).reshape(d.vocab, d.hidden)
    lm[nan_row, 5] = np.nan
    dm = q.DeviceModel(model)
    ds = q.DeviceState(st.copy(), d.prefix_cap, d.ring_cap)
    dm.bind_caches(ds.k_cache, ds.v_cache)
    wsb = q.ocrdec_step_workspace_bytes(dm.desc, ds.desc)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    tok_out = torch.zeros(R, dtype=torch.int32, device="cuda")
    tok = synth.first_tokens(d, seed, R)

    # 1. the NaN row: flagged, never chosen; the tokens equal the oracle's
    #    argmax over the other rows
    q.ocrdec_decode_step(dm.desc, ds.desc, torch.from_numpy(tok).cuda(), None, tok_out, None, None, ws, wsb)
    flags = q.ocrdec_device_status(ws, wsb)
    assert flags == q.OCRDEC_DEV_LOGIT, flags
    res = O.decode_step(model, st.copy(), tok_in=tok)
    g = tok_out.cpu().numpy()
    assert np.all(g != nan_row)
    for r in range(R):
        if g[r] != res.tok[r]:
            assert res.lm_top2[r, 0] - res.lm_top2[r, 1] < 1e-3

    # 2. a token id outside the vocabulary (clamped) is reported as well
    bad_tok = np.array([d.vocab + 5, 3], np.int32)
    q.ocrdec_decode_step(dm.desc, ds.desc, torch.from_numpy(bad_tok).cuda(), None, tok_out, None, None, ws, wsb)
    assert q.ocrdec_device_status(ws, wsb) == q.OCRDEC_DEV_LOGIT | q.OCRDEC_DEV_TOKEN_RANGE
    neg_tok = np.array([5, -1], np.int32)
    q.ocrdec_decode_step(dm.desc, ds.desc, torch.from_numpy(neg_tok).cuda(), None, tok_out, None, None, ws, wsb)
    assert q.ocrdec_device_status(ws, wsb) & q.OCRDEC_DEV_TOKEN_RANGE

    # 3. a clean head: no flags, and each step clears the previous step's bits
    model.lm_head.data.view(np.float16).reshape(d.vocab, d.hidden)[nan_row, 5] = 0.0
    dm2 = q.DeviceModel(model)
    dm2.bind_caches(ds.k_cache, ds.v_cache)
    q.ocrdec_decode_step(dm2.desc, ds.desc, torch.from_numpy(tok).cuda(), None, tok_out, None, None, ws, wsb)
    assert q.ocrdec_device_status(ws, wsb) == 0

    # 4. a hidden input beyond the residual's range (2^31) is replaced and reported
    h = np.zeros((R, d.hidden), np.float32)
    h[:] = synth.normal_f64(synth.stream_id(seed, "h"), (R, d.hidden)).astype(np.float32)
    h[1, 7] = 2.0 ** 31
    hd = torch.from_numpy(h).cuda()
    q.ocrdec_decode_step(dm2.desc, ds.desc, None, hd, tok_out, None, None, ws, wsb)
    assert q.ocrdec_device_status(ws, wsb) == q.OCRDEC_DEV_RESIDUAL
    h[1, 7] = np.nan
    hd = torch.from_numpy(h).cuda()
    q.ocrdec_decode_step(dm2.desc, ds.desc, None, hd, tok_out, None, None, ws, wsb)
    assert q.ocrdec_device_status(ws, wsb) == q.OCRDEC_DEV_RESIDUAL
