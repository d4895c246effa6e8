"""Writes decode_full_r24.npz: the oracle's trajectory of two sampled rows of
the full 12-layer decoder (24-row launch, prefix 1100, ring from t = 124 so it
wraps after four steps), teacher-forced on the oracle's own tokens.

Calls only the oracle and the input generator.  Run from the repo root:
    python tests/golden/make_decode_fixture.py
(about two minutes on 8 cores).
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
T0 = 124
STEPS = 8
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "decode_full_r24.npz")


def main():
    d = synth.dims_full()
    model = synth.make_model(d, SEED)
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
    np.savez_compressed(OUT, seed=SEED, rows=ROWS, sampled=np.array(SAMPLED), t0=T0, steps=STEPS,
                        n_moe=n_moe, **{k: np.array(v) for k, v in out.items()})
    print("wrote", OUT)


if __name__ == "__main__":
    main()
