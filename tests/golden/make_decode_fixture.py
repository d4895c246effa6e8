"""Writes the oracle fixtures of the full 12-layer decoder (prefix 1100) for
sampled rows, from the oracle and the input generator alone:

* decode_full_r24.npz: an 8-step trajectory of rows 0, 11 and 23 from
  generation index 124 (the ring wraps after four steps), teacher-forced on
  the oracle's own tokens; per step the tokens, routing, final hidden state
  and new keys.
* decode_layers_r24.npz: single steps of rows 0 and 23 at generation index
  124 and 128 (just wrapped), with the residual entering every layer and the
  final LM-head input, so each layer can be checked from the oracle's own
  inputs.
* decode_layers_r1_6_12.npz: the same at 1, 6 and 12 rows (sampled rows: the
  first and the last), the batch sizes of the decode rows sweep.
* decode_r1_64.npz: 64 consecutive steps of one row from generation index 100
  (the ring wraps at step 28), teacher-forced on the oracle's own tokens: per
  step the tokens, routing and final hidden state, and the last layer's new
  keys at steps 0, 27, 28 and 63.

Run from the repo root:  python tests/golden/make_decode_fixture.py
(about five minutes on 8 cores for the 24-row files and as long again for the
64-step trajectory; --layers-only / --trajectory-only / --small-rows /
--r1-64 write one of them).
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


def per_layer(d, model, rows=ROWS, sampled=SAMPLED, prefix=""):
    out = {}
    for case, t in (("a", 124), ("b", 128)):
        st = synth.make_state(d, SEED, [d.prefix_cap] * rows, [t] * rows)
        tok = synth.first_tokens(d, SEED + t, rows)
        res = O.decode_step(model, st, tok_in=tok, rows=sampled)
        case = prefix + case
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
    return out


SMALL_ROWS = {1: [0], 6: [0, 5], 12: [0, 11]}
R1_T0, R1_STEPS = 100, 64
R1_KEY_STEPS = [0, 27, 28, 63]


def trajectory_r1(d, model):
    """64 steps of one row across the ring wrap (t = 100 .. 163)."""
    st = synth.make_state(d, SEED, [d.prefix_cap], [R1_T0])
    tok = synth.first_tokens(d, SEED, 1)
    out = {k: [] for k in ("tok_in", "tok", "lm_top2", "hidden", "topk_idx", "topk_w", "router_gap")}
    new_k_last = []
    for step in range(R1_STEPS):
        res = O.decode_step(model, st, tok_in=tok, rows=[0])
        out["tok_in"].append(tok.copy())
        out["tok"].append(res.tok)
        out["lm_top2"].append(res.lm_top2)
        out["hidden"].append(res.hidden.astype(np.float32))
        out["topk_idx"].append(np.array(res.topk_idx, np.int32))
        out["topk_w"].append(np.array(res.topk_w, np.float64))
        out["router_gap"].append(np.array(res.router_gap, np.float64))
        if step in R1_KEY_STEPS:
            new_k_last.append(res.new_k[-1].astype(np.float32))
        tok = np.array(res.tok, np.int32)
        print("r1 step", step, "token", int(res.tok[0]), flush=True)
    np.savez_compressed(os.path.join(HERE, "decode_r1_64.npz"), seed=SEED, t0=R1_T0, steps=R1_STEPS,
                        key_steps=np.array(R1_KEY_STEPS), new_k_last=np.array(new_k_last),
                        **{k: np.array(v) for k, v in out.items()})


def main():
    d = synth.dims_full()
    model = synth.make_model(d, SEED)
    only = [a for a in sys.argv[1:] if a.startswith("--")]
    if not only or "--layers-only" in only:
        out = per_layer(d, model)
        np.savez_compressed(os.path.join(HERE, "decode_layers_r24.npz"), seed=SEED, rows=ROWS,
                            sampled=np.array(SAMPLED), **out)
    if not only or "--trajectory-only" in only:
        trajectory(d, model)
    if not only or "--small-rows" in only:
        out = {}
        for R, smp in SMALL_ROWS.items():
            out.update(per_layer(d, model, R, smp, "r%d_" % R))
            out["r%d_sampled" % R] = np.array(smp)
        np.savez_compressed(os.path.join(HERE, "decode_layers_r1_6_12.npz"), seed=SEED,
                            rows=np.array(sorted(SMALL_ROWS)), **out)
    if not only or "--r1-64" in only:
        trajectory_r1(d, model)
    print("done")


if __name__ == "__main__":
    main()
