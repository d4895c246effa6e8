"""Measures how far the oracle's own 12-layer decode step moves when every
quantised matrix-vector product is perturbed by relative noise of 3e-7 (the
size of fp32 accumulation error; the GEMV kernels measure about 5e-7 of the
output rms).  The fp16 storage points of the decoder (normalised activations,
q/k/v, attention output, SwiGLU product) turn such noise into whole-ulp
flips, and the flips compound from layer to layer: this sets the floor for
comparing any fp32 implementation with the oracle on the composed hidden
state and on routing decisions taken from it, and the bounds of the
multi-layer trajectory test are derived from it.  The perturbed runs keep the
exact run's routing (forced), as the trajectory test does.  Uses the oracle
and the input generator only.

Run from the repo root:  python tests/golden/decode_sensitivity.py
Prints, per sampled row and noise seed, max and median of
|perturbed - exact| / rms(exact) of the residual after 1, 2, 4, 8 and 12
layers and the largest router-logit change; then each layer alone from its
exact input.
"""
import copy
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
import oracle.core as C  # noqa: E402
import synth  # noqa: E402

SEED = 1003
ROWS = 24
SAMPLED = [0, 11, 23]
T0 = 124
REL = 3e-7
NOISE_SEEDS = 4


def noisy_gemv(exact, tag, *key):
    calls = [0]

    def f(m, x):
        y = exact(m, x)
        calls[0] += 1
        e = synth.normal_f64(synth.stream_id(SEED, tag, *key, calls[0]), y.shape)
        return y * (1.0 + REL * e)
    return f


def main():
    d = synth.dims_full()
    model = synth.make_model(d, SEED)
    st = synth.make_state(d, SEED, [d.prefix_cap] * ROWS, [T0] * ROWS)
    tok = synth.first_tokens(d, SEED, ROWS)
    exact = C.gemv_qmat
    n_moe = d.n_layers - d.n_dense
    ref = O.decode_step(model, st.copy(), tok_in=tok, rows=SAMPLED, with_lm=False)
    forced = np.full((n_moe, ROWS, d.top_k), -1, np.int64)
    forced[:, SAMPLED] = np.array(ref.topk_idx)
    deep = [np.array(ref.layer_in[l]) for l in range(1, d.n_layers)] + [ref.hidden]
    worst_h = {}
    worst_lg = 0.0
    for ns in range(NOISE_SEEDS):
        C.gemv_qmat = noisy_gemv(exact, "gemv-noise", ns)
        try:
            res = O.decode_step(model, st.copy(), tok_in=tok, rows=SAMPLED, forced_topk=forced, with_lm=False)
        finally:
            C.gemv_qmat = exact
        dlg = np.array([np.max(np.abs(np.array(a) - np.array(b)), axis=1)
                        for a, b in zip(res.router_logits, ref.router_logits)])     # [n_moe][rows]
        worst_lg = max(worst_lg, float(dlg.max()))
        for i, r in enumerate(SAMPLED):
            line = []
            for depth in (1, 2, 4, 8, 12):
                h0 = deep[depth - 1][i]
                h1 = (np.array(res.layer_in[depth]) if depth < d.n_layers else res.hidden)[i]
                e = np.abs(h1 - h0) / np.sqrt(np.mean(h0 ** 2))
                worst_h[depth] = max(worst_h.get(depth, 0.0), e.max())
                line.append("L%-2d max %.2e p50 %.2e" % (depth, e.max(), np.median(e)))
            print("noise %d row %2d: %s | router logit max change %.2e" % (ns, r, " | ".join(line), dlg[:, i].max()),
                  flush=True)
    print("composed, worst over seeds and rows: " + " ".join("L%d %.2e" % kv for kv in sorted(worst_h.items())) +
          " | router logits %.2e" % worst_lg, flush=True)
    # one layer at a time, each from the exact input of that layer
    for l in range(d.n_layers):
        sub = copy.copy(model)
        sub.layers = model.layers[l:l + 1]
        sub.embed = model.embed if l == 0 else None
        sd = copy.copy(d)
        sd.n_layers = 1
        sub.dims = sd
        sst = synth.State(st.prefix_len.copy(), st.gen_index.copy(), st.k_cache[l:l + 1].copy(),
                          st.v_cache[l:l + 1].copy())
        h_in = None
        if l > 0:
            h_in = np.zeros((ROWS, d.hidden))
            h_in[SAMPLED] = ref.layer_in[l]
        worst = 0.0
        for ns in range(NOISE_SEEDS):
            C.gemv_qmat = noisy_gemv(exact, "gemv-noise-layer", ns, l)
            try:
                res = O.decode_step(sub, sst.copy(), tok_in=tok if l == 0 else None, hidden_in=h_in, rows=SAMPLED,
                                    with_lm=False)
            finally:
                C.gemv_qmat = exact
            for i in range(len(SAMPLED)):
                h0 = deep[l][i]
                worst = max(worst, float(np.max(np.abs(res.hidden[i] - h0)) / np.sqrt(np.mean(h0 ** 2))))
        print("layer %2d alone, from its exact input: worst max %.2e" % (l, worst), flush=True)


if __name__ == "__main__":
    main()
