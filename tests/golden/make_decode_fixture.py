"""Writes the oracle fixtures of the full 12-layer decoder at 24 rows (prefix
1100) for sampled rows, from the oracle and the input generator alone:

* decode_full_r24.npz: an 8-step trajectory of rows 0, 11 and 23 from
  generation index 124 (the ring wraps after four steps), teacher-forced on
  the oracle's own tokens; per step the tokens, routing, final hidden state
  and new keys.
* decode_layers_r24.npz: single steps of rows 0 and 23 at generation index
  124 and 128 (just wrapped), with the residual entering every layer and the
  final LM-head input, so each layer can be checked from the oracle's own
  inputs.

Run from the repo root:  python tests/golden/make_decode_fixture.py
(about five minutes on 8 cores; --layers-only / --trajectory-only write one).
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
import synth  # noqa: E402

SEED = 1003
ROWS = 24
SAMPLED = [0, 23]
TRAJ_SAMPLED = [0, 11, 23]
T0 = 124
STEPS = 8
HERE = os.path.dirname(os.path.abspath(__file__))


def trajectory(d, model):
    SAMPLED = TRAJ_SAMPLED
    st = synth.make_state(d, SEED, [d.prefix_cap] * ROWS, [T0] * ROWS)
    tok = synth.first_tokens(d, SEED, ROWS)
    n_moe = d.n_layers - d.n_dense
    out = {k: [] for k in ("tok_in", "tok", "lm_top2", "hidden", "topk_idx", "topk_w", "router_gap",
                           "new_k_first", "new_k_last")}
    for step in range(STEPS):
        res = O.decode_step(model, st, tok_in=tok, rows=SAMPLED)
        out["tok_in"].append(tok[SAMPLED].copy())
        out["tok"].append(res.tok)
        out["lm_top2"].append(res.lm_top2)
        out["hidden"].append(res.hidden.astype(np.float32))
        out["topk_idx"].append(np.array(res.topk_idx, np.int32))       # [n_moe][2][k]
        out["topk_w"].append(np.array(res.topk_w, np.float64))
        out["router_gap"].append(np.array(res.router_gap, np.float64))  # [n_moe][2]
        out["new_k_first"].append(res.new_k[0].astype(np.float32))     # [2][NH][D]
        out["new_k_last"].append(res.new_k[-1].astype(np.float32))
        nxt = tok.copy()
        nxt[SAMPLED] = res.tok
        tok = nxt
        print("step", step, "tokens", res.tok.tolist(), flush=True)
    np.savez_compressed(os.path.join(HERE, "decode_full_r24.npz"), seed=SEED, rows=ROWS, sampled=np.array(SAMPLED),
                        t0=T0, steps=STEPS, n_moe=n_moe, **{k: np.array(v) for k, v in out.items()})


def per_layer(d, model):
    out = {}
    for case, t in (("a", 124), ("b", 128)):
        st = synth.make_state(d, SEED, [d.prefix_cap] * ROWS, [t] * ROWS)
        tok = synth.first_tokens(d, SEED + t, ROWS)
        res = O.decode_step(model, st, tok_in=tok, rows=SAMPLED)
        out[case + "_t"] = t
        out[case + "_tok_in"] = tok
        out[case + "_layer_in"] = np.array(res.layer_in, np.float32)       # [L][2][H]
        out[case + "_hidden"] = res.hidden.astype(np.float32)              # [2][H]
        out[case + "_final_x"] = res.final_x.astype(np.float16)            # [2][H] (fp16 values)
        out[case + "_tok"] = res.tok
        out[case + "_lm_top2"] = res.lm_top2
        out[case + "_topk_idx"] = np.array(res.topk_idx, np.int32)
        out[case + "_topk_w"] = np.array(res.topk_w, np.float64)
        out[case + "_router_gap"] = np.array(res.router_gap, np.float64)
        out[case + "_new_k"] = np.array(res.new_k, np.float32)             # [L][2][NH][D]
        out[case + "_new_v"] = np.array(res.new_v, np.float32)
        print("case", case, "t", t, "tokens", res.tok.tolist(), flush=True)
    np.savez_compressed(os.path.join(HERE, "decode_layers_r24.npz"), seed=SEED, rows=ROWS,
                        sampled=np.array(SAMPLED), **out)


def main():
    d = synth.dims_full()
    model = synth.make_model(d, SEED)
    if "--trajectory-only" not in sys.argv:
        per_layer(d, model)
    if "--layers-only" not in sys.argv:
        trajectory(d, model)
    print("done")


if __name__ == "__main__":
    main()
