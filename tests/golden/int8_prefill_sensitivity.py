"""How far the oracle's own INT8 prompt pass moves under float32-size input noise.

Used to derive the comparison rule for prompt passes into INT8 caches: every
key and value row is quantised to codes one step (max|row| / 127) apart, so a
value within rounding noise of a code boundary flips a whole step, and the
next layer amplifies it.  This script calls only the oracle: it perturbs the
prompt's embedding rows by relative Gaussian noise of 3e-7 (the size of fp32
accumulation error) with the routing held fixed, and prints the largest
residual deviation over three noise draws and the fraction of flipped codes.

    python tests/golden/int8_prefill_sensitivity.py
"""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import oracle as O  # noqa: E402
import synth  # noqa: E402


def main():
    d = synth.Dims(hidden=256, n_heads=2, head_dim=128, n_layers=3, n_dense=1, dense_ff=512, n_experts=16, top_k=6,
                   n_shared=2, expert_ff=128, vocab=1000, prefix_cap=300, ring_cap=8)
    for P, seed in ((40, 670), (257, 887)):
        m = synth.make_model(d, seed)
        tok = synth.uniform_i32(synth.stream_id(seed, "prompt"), (P,), 0, d.vocab)
        base = O.prefill(m, P, tok=tok, int8_kv=True)
        emb = O.embed_rows(m, tok)
        rms = np.sqrt(np.mean(base.hidden ** 2))
        worst, flips = 0.0, []
        for s in range(3):
            e = emb * (1 + 3e-7 * np.random.default_rng(s).standard_normal(emb.shape))
            r = O.prefill(m, P, emb=e, int8_kv=True, forced_topk=base.topk_idx)
            worst = max(worst, float(np.max(np.abs(r.hidden - base.hidden)) / rms))
            flips.append(np.mean([np.mean(r.kq[l] != base.kq[l]) for l in range(d.n_layers)]))
        print("P %d: worst residual deviation %.2e rms, flipped key codes %.3f" % (P, worst, float(np.mean(flips))))


if __name__ == "__main__":
    main()
