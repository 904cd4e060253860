"""The comparison helpers the GPU parity tests rely on (CPU only)."""
import numpy as np

from tests.gpu_util import assert_rel, f16_rounding_slack, floored_rel_err, propagate_slack


def test_rounding_slack_only_at_midpoints():
    ulp1 = 2.0 ** -10                      # fp16 spacing in [1, 2)
    mid = 1.0 + ulp1 / 2
    v = np.array([mid, mid * (1 + 2.0 ** -22), mid * (1 + 2.0 ** -15), 1.0, 0.75, -(0.5 + 2.0 ** -12)])
    s = f16_rounding_slack(v)
    assert s[0] == ulp1 and s[1] == ulp1      # on, or within fp32 reach of, the midpoint
    assert s[2] == 0 and s[3] == 0 and s[4] == 0
    assert s[5] == 2.0 ** -11                 # spacing in [0.5, 1)


def test_slack_propagates_through_a_product():
    w = np.array([[1.0, -2.0], [0.5, 0.0]])
    got = propagate_slack(np.array([[0.0, 0.25]]), 2, lambda: w)
    assert np.allclose(got, [[0.5, 0.0]])
    assert propagate_slack(np.zeros((3, 2)), 5, lambda: 1 / 0).shape == (3, 5)   # W never built


def test_assert_rel_with_slack():
    ref = np.array([1.0, 100.0])
    got = ref + np.array([0.5, 0.0])
    assert floored_rel_err(got, ref)[0] == 0.5
    assert_rel(got, ref, slack=np.array([0.5, 0.0]))


def test_rope_fp32_slack_covers_an_fp32_rotation():
    # the rotation done the way an fp32 kernel does it (cos / sin rounded once
    # to fp32, products and difference in fp32) stays within the slack of the
    # exact rotation, including elements where x_i c and x_j s nearly cancel
    from oracle import ops as OO
    from tests.gpu_util import rope_fp32_slack
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((64, 128)) * 20).astype(np.float32).astype(np.float64)
    pos, base = 2417, 1e6
    half = 64
    i = np.arange(half, dtype=np.float64)
    a = pos * base ** (-2.0 * i / 128)
    c32, s32 = np.cos(a).astype(np.float32), np.sin(a).astype(np.float32)
    x32 = x.astype(np.float32)
    # make some pairs cancel: x_j = x_i cos / sin (to fp32)
    x32[:8, half:] = (x32[:8, :half] * c32 / s32).astype(np.float32)
    x = x32.astype(np.float64)
    lo = (x32[:, :half] * c32).astype(np.float32) - (x32[:, half:] * s32).astype(np.float32)
    hi = (x32[:, half:] * c32).astype(np.float32) + (x32[:, :half] * s32).astype(np.float32)
    got = np.concatenate([lo, hi], axis=1).astype(np.float64)
    want = OO.rope(x, pos, base)
    slack = rope_fp32_slack(x, pos, base)
    assert (np.abs(got - want) <= slack).all()
    # and near the cancellations the error is more than one fp16 ulp of the result
    r16 = np.abs(np.spacing(want[:8, :half].astype(np.float16)).astype(np.float64))
    assert (np.abs(got - want)[:8, :half] > r16).any()


def test_attention_fp32_slack_covers_fp32_scores_near_a_tie():
    # one cached key of a large value whose score lands next to the best other
    # score: fp32 scores move O by more than 1e-3 of |O|, inside the slack;
    # away from the tie the slack is far below 1e-3 of |O|
    from oracle import ops as OO
    from tests.gpu_util import attention_fp32_slack
    rng = np.random.default_rng(12)
    d, n = 128, 301
    k = rng.standard_normal((1, n, d))
    v = rng.standard_normal((1, n, d))
    q = (rng.standard_normal((1, d)) * 20).astype(np.float16).astype(np.float64)
    scale = d ** -0.5
    s = scale * (k[0] @ q[0])
    big = 60.0 * np.sign(q[0])                    # a key with a huge score magnitude ...
    k[0, -1] = big * ((np.max(s) - 2.2) / (scale * (big @ q[0])))   # ... next to the best other key (p ~ 0.1)
    v[0, -1] = 55.0
    k = k.astype(np.float16).astype(np.float64)
    exact = OO.attention(q, k, v, scale)
    k32, q32 = k.astype(np.float32), q.astype(np.float32)
    s32 = (k32[0] @ q32[0]).astype(np.float32) * np.float32(scale)
    p = np.exp(s32.astype(np.float64) - s32.max())
    p /= p.sum()
    got = p @ v[0]
    slack = attention_fp32_slack(q, k, v, scale)
    assert (np.abs(got - exact[0]) <= slack[0] + 1e-12).all()
    assert (slack[0] / np.abs(exact[0])).max() > 1e-3
    far = attention_fp32_slack(q, k[:, :-1], v[:, :-1], scale)
    assert far.max() < 1e-4 * np.abs(OO.attention(q, k[:, :-1], v[:, :-1], scale)).max()
