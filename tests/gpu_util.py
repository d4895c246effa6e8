"""Helpers shared by the GPU parity tests (comparison rules, device uploads)."""
import numpy as np

# Floating-point outputs: max |gpu - oracle| <= 2e-3 * rms(oracle) per tensor,
# with fp32 accumulation on the GPU.
REL_TOL = 2e-3
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


def assert_close(gpu, ref, what: str, tol: float = REL_TOL):
    e = rel_err(gpu, ref)
    assert np.all(np.isfinite(np.asarray(gpu, np.float64))), "%s: non-finite GPU values" % what
    assert e <= tol, "%s: max|gpu-oracle|/rms = %.3g > %.3g" % (what, e, tol)
    return e


def f16_tensor(a, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.float16)).view(np.int16)).to(device)


def from_f16_tensor(t) -> np.ndarray:
    return t.cpu().numpy().view(np.float16).astype(np.float64)
