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


def assert_rel(got, ref, tol=REL_TOL, what="", slack=None):
    """Floored relative error <= tol, after subtracting `slack` (an absolute
    allowance per element, see f16_rounding_slack) from |got - ref|."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    if slack is None:
        err = floored_rel_err(got, ref)
    else:
        rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
        den = np.maximum(np.abs(ref), 1e-3 * rms)
        den = np.where(den == 0.0, 1.0, den)
        err = np.maximum(np.abs(got - ref) - slack, 0.0) / den
    worst = float(err.max()) if err.size else 0.0
    assert worst <= tol, f"{what}: max floored relative error {worst:.3e} > {tol:.0e}"
    return worst


F32_DECIDES = 2.0 ** -20   # relative distance to an fp16 midpoint that fp32 arithmetic cannot resolve


def f16_rounding_slack(pre, rel=F32_DECIDES):
    """Where rounding `pre` (fp64) to fp16 is too close to call for an fp32
    computation of the same value (within rel*|pre| of the midpoint between two
    neighbouring fp16 values), |other neighbour - chosen|; elsewhere 0.  Either
    rounding is then a correct result of the kernel."""
    v = np.asarray(pre, dtype=np.float64)
    r16 = v.astype(np.float16)
    r = r16.astype(np.float64)
    toward = np.where(v >= r, np.float16(np.inf), np.float16(-np.inf))
    nb = np.nextafter(r16, toward).astype(np.float64)
    amb = np.abs(v - 0.5 * (r + nb)) <= rel * np.abs(v)
    return np.where(amb & np.isfinite(nb), np.abs(nb - r), 0.0)


def propagate_slack(slack_in, n_out, w_dense):
    """Bound on |delta Y| for Y = X W^T (n_out outputs) when X may move by
    slack_in: slack_in |W|^T.  w_dense() gives W; it is only called when some
    slack is non-zero."""
    if not np.any(slack_in):
        return np.zeros((slack_in.shape[0], n_out))
    return slack_in @ np.abs(w_dense()).T


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


U32 = 2.0 ** -24    # unit roundoff of fp32


def rope_fp32_slack(x, pos, base):
    """Bound on |fp32 rotation - exact rotation| of x [heads, D] at pos, for a
    kernel that rounds cos and sin once to fp32 and rotates in fp32: each
    output x_i c -/+ x_j s carries at most 4 roundings of the size of its two
    products (cos / sin, two products, one sum).  Near a cancellation this is
    far more than one fp16 ulp of the (small) result."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    i = np.arange(half, dtype=np.float64)
    a = float(pos) * base ** (-2.0 * i / d)
    c, s = np.abs(np.cos(a)), np.abs(np.sin(a))
    x1, x2 = np.abs(x[..., :half]), np.abs(x[..., half:])
    mag = np.concatenate([x1 * c + x2 * s, x2 * c + x1 * s], axis=-1)
    return 4.0 * U32 * mag


def attention_fp32_slack(q, k, v, scale):
    """First-order bound on |O_fp32 - O_exact| for one sequence (q [Hq, D],
    k, v [Hkv, n, D] as the kernel reads them) caused by computing the scores
    in fp32: a D-term dot product is within (D + 4) u sum_d |q_d k_d| of
    exact (any summation order, plus the per-block scale and the softmax
    scale), and O = sum_t p_t v_t moves by sum_t p_t ds_t (v_t - O) when the
    scores move by ds.  Where one key holds a large share of the softmax and
    a very different value, this exceeds 1e-3 of O; elsewhere it is tiny."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    hq, hkv, d = q.shape[0], k.shape[0], q.shape[1]
    out = np.zeros_like(q)
    for h in range(hq):
        g = h // (hq // hkv)
        s = scale * (k[g] @ q[h])
        p = np.exp(s - s.max())
        p /= p.sum()
        o = p @ v[g]
        ds = (d + 4) * U32 * scale * (np.abs(k[g]) @ np.abs(q[h]))
        out[h] = (p * ds) @ np.abs(v[g] - o)
    return out
