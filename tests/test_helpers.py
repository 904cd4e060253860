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
