"""ocrdec_decode_step_noalloc (static scratch, no workspace argument) against
ocrdec_decode_step with a caller workspace: the same steps from the same
inputs must give the same bits (the step is deterministic), on two calls in a
row, the second with fewer rows (the scratch keeps the first call's contents,
which the second must not depend on)."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import torch
    assert torch.cuda.is_available()
    import quantized_decode_step_amd as qd
    return qd


def _dims():
    return synth.Dims(hidden=256, n_heads=2, head_dim=128, n_layers=3, n_dense=1, dense_ff=512, n_experts=16, top_k=6,
                      n_shared=2, expert_ff=128, vocab=1000, prefix_cap=40, ring_cap=8)


def _step(q, dm, d, st, tok, noalloc):
    import torch
    R = len(st.prefix_len)
    ds = q.DeviceState(st.copy(), d.prefix_cap, d.ring_cap)
    dm.bind_caches(ds.k_cache, ds.v_cache)
    n_moe = d.n_layers - d.n_dense
    cap_idx = torch.zeros((n_moe, R, d.top_k), dtype=torch.int32, device="cuda")
    cap_w = torch.zeros((n_moe, R, d.top_k), dtype=torch.float32, device="cuda")
    cap = q.StepCapture(cap_idx.data_ptr(), cap_w.data_ptr(), None)
    hidden = torch.zeros((R, d.hidden), dtype=torch.float32, device="cuda")
    toks = torch.from_numpy(tok.astype(np.int32)).cuda()
    for _ in range(2):  # two steps, tokens fed back on the device
        if noalloc:
            q.ocrdec_decode_step_noalloc(dm.desc, ds.desc, toks, hidden, toks, None, cap)
        else:
            wsb = q.ocrdec_step_workspace_bytes(dm.desc, ds.desc)
            ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
            q.ocrdec_decode_step(dm.desc, ds.desc, toks, hidden, toks, None, cap, ws, wsb)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (toks, cap_idx, cap_w, hidden, ds.k_cache, ds.v_cache, ds.gen_index)]


def test_noalloc_step_matches_workspace_step(q):
    d = _dims()
    seed = 700
    model = synth.make_model(d, seed)
    dm = q.DeviceModel(model)
    for R in (6, 2):  # the second call has fewer rows
        print("[case] no-alloc step R=%d seed=%d" % (R, seed), flush=True)
        st = synth.make_state(d, seed + R, [(9 * i + 4) % 41 for i in range(R)], [(3 * i + 2) % 11 for i in range(R)])
        tok = synth.first_tokens(d, seed + R, R)
        want = _step(q, dm, d, st, tok, noalloc=False)
        got = _step(q, dm, d, st, tok, noalloc=True)
        for name, a, b in zip(("tokens", "routing", "routing weights", "hidden", "k cache", "v cache", "gen_index"),
                              got, want):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), "R=%d: %s differ" % (R, name)


def test_noalloc_rejects_a_step_beyond_the_scratch(q):
    fake = 1 << 20
    m = q.ModelDesc()
    m.n_layers, m.hidden, m.n_heads, m.head_dim, m.vocab = 1, 1280, 10, 128, 1000
    m.rope_theta, m.norm_eps = 10000.0, 1e-6
    layers = (q.LayerDesc * 1)()
    L = layers[0]
    L.attn_norm = L.ffn_norm = fake
    L.wqkv, L.wo = q.QMatDesc(1, 3840, 1280, fake), q.QMatDesc(1, 1280, 1280, fake)
    L.k_cache = L.v_cache = fake
    L.is_moe, L.dense_ff = 0, 3584
    L.dense_gate_up, L.dense_down = q.QMatDesc(2, 7168, 1280, fake), q.QMatDesc(2, 1280, 3584, fake)
    m.layers = layers
    st = q.StateDesc(32, 65536 - 128, 128, fake, fake)
    with pytest.raises(q.OcrdecError) as e:
        q.ocrdec_decode_step_noalloc(m, st, fake, None, None, None, None, stream=0)
    assert e.value.status == q.OCRDEC_ERR_WORKSPACE
    assert "static scratch" in q.ocrdec_last_error()
