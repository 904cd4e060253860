"""Helpers for the GPU parity tests (comparisons and device set-up)."""
import numpy as np

REL_TOL = 1e-3          # per-output relative error bound for GEMM and attention outputs
LOGIT_ABS_TOL = 5e-2    # max |delta logit|
ARGMAX_GAP = 1e-3       # argmax must agree where the oracle's top-2 gap exceeds this


def floored_rel_err(got, ref):
    """|got - ref| / max(|ref|, 1e-3 * rms(ref)) elementwise.

    The floor keeps outputs within 0.1 % of the tensor's rms from turning the
    relative error into a ratio of two rounding noises.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    den = np.maximum(np.abs(ref), 1e-3 * rms)
    den = np.where(den == 0.0, 1.0, den)
    return np.abs(got - ref) / den


def assert_rel(got, ref, tol=REL_TOL, what=""):
    err = floored_rel_err(got, ref)
    worst = float(err.max()) if err.size else 0.0
    assert np.all(np.isfinite(np.asarray(got, dtype=np.float64))), f"{what}: non-finite output"
    assert worst <= tol, f"{what}: max floored relative error {worst:.3e} > {tol:.0e}"
    return worst


def top2_gap(logits_row):
    s = np.sort(np.asarray(logits_row, dtype=np.float64))
    return float(s[-1] - s[-2])


def sync():
    import torch
    torch.cuda.synchronize()


def ws(nbytes):
    """Zeroed device workspace (uint8)."""
    import torch
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device="cuda")
