"""Helpers shared by the GPU parity tests (comparison rules, device uploads).

Comparison rule for floating point:
  * fp32 outputs: max |gpu - oracle| <= 2e-3 * rms(oracle).
  * fp16-stored outputs: every element within 2e-3 * rms(oracle) + one fp16
    ulp of the oracle's value.  Both sides compute the same real number up to
    fp32 accumulation order and then round it to fp16; when that number lies
    within their accumulation difference of a rounding boundary, the two
    roundings land on neighbouring fp16 values, one ulp apart.  For elements
    above about 2 * rms an ulp exceeds 2e-3 * rms, so the stated tolerance
    alone cannot hold for a tensor stored in fp16.  Such flips must stay rare:
    at most 1% of the elements may exceed 2e-3 * rms.
"""
import json
import os

import numpy as np

REL_TOL = 2e-3
FLIP_FRACTION = 0.01
# Routing and argmax decisions may differ only where the oracle's own gap
# between the competing logits is below this (a logged near-tie).
NEAR_TIE = 1e-3


def rel_err(gpu, ref) -> float:
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    if rms == 0:
        return float(np.max(np.abs(gpu - ref)))
    return float(np.max(np.abs(gpu - ref)) / rms)


def ulp16(v) -> np.ndarray:
    """Spacing of binary16 at |v| (2^-24 in the subnormal range)."""
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)


def assert_close(gpu, ref, what: str, tol: float = REL_TOL):
    """fp32 outputs: max |gpu - ref| <= tol * rms(ref)."""
    gpu = np.asarray(gpu, np.float64)
    e = rel_err(gpu, ref)
    assert np.all(np.isfinite(gpu)), "%s: non-finite GPU values" % what
    assert e <= tol, "%s: max|gpu-oracle|/rms = %.3g > %.3g" % (what, e, tol)
    return e


def assert_close_f16(gpu, ref, what: str, tol: float = REL_TOL):
    """fp16-stored outputs: |gpu - ref| <= tol * rms(ref) + ulp16(ref) per
    element, with at most FLIP_FRACTION of the elements beyond tol * rms."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(gpu)), "%s: non-finite GPU values" % what
    rms = np.sqrt(np.mean(ref * ref))
    err = np.abs(gpu - ref)
    bound = tol * rms + ulp16(ref)
    bad = err > bound
    assert not np.any(bad), "%s: %d elements beyond 2e-3*rms + 1 ulp (worst %.3g rms)" % (
        what, int(bad.sum()), float(np.max(err) / max(rms, 1e-300)))
    flips = int(np.sum(err > tol * rms))
    assert flips <= FLIP_FRACTION * err.size, "%s: %d of %d elements beyond 2e-3*rms" % (what, flips, err.size)
    return float(np.max(err) / max(rms, 1e-300)), flips


def f16_tensor(a, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.float16)).view(np.int16)).to(device)


def from_f16_tensor(t) -> np.ndarray:
    return t.cpu().numpy().view(np.float16).astype(np.float64)


# near-ties accepted in this session (the parity report lists them)
NEAR_TIES = []


def log_near_tie(kind: str, what: str, gap: float):
    """Records an accepted near-tie (a routing or argmax decision that differs
    from the oracle's where the oracle's own gap is below the threshold) in
    the JSONL log named by OCRDEC_NEAR_TIE_LOG (default
    gpurun_out/near_ties.jsonl) and on stdout."""
    rec = {"kind": kind, "case": what, "oracle_gap": float(gap)}
    NEAR_TIES.append(rec)
    print("[near-tie]", json.dumps(rec), flush=True)
    path = os.environ.get("OCRDEC_NEAR_TIE_LOG", os.path.join("gpurun_out", "near_ties.jsonl"))
    try:
        os.makedirs(os.path.dirname(path) or ".", exist_ok=True)
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")
    except OSError:
        pass
