"""The parity bar's helpers on the CPU: what they accept and what they reject."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def H():
    from tests import gpu_helpers
    return gpu_helpers


def _outputs(seed=0, n=20000, peak=9.5):
    r = np.random.default_rng(seed).standard_normal(n)
    r[17] = peak * np.sqrt(np.mean(r * r))  # one heavy-tailed output
    return r


def test_correctly_rounded_output_meets_bar(H):
    from oracle import round_bf16
    r = _outputs()
    g = round_bf16(r)
    m = H.check_close(g, r, "rounded")
    assert m["max_abs_over_rms"] > 2e-2   # the rounding alone is over 2e-2 RMS at the peak
    H.check_ulp(g, r, "rounded")


def test_bar_rejects_a_real_error(H):
    from oracle import round_bf16
    r = _outputs(1)
    g = round_bf16(r)
    g[5] += 0.03 * np.sqrt(np.mean(r * r))
    with pytest.raises(AssertionError):
        H.check_close(g, r, "planted")
    with pytest.raises(AssertionError):
        H.check_ulp(g, r, "planted")


def test_bar_rejects_a_two_ulp_error_at_the_peak(H):
    from oracle import round_bf16
    r = _outputs(2)
    g = round_bf16(r)
    g[17] += 2 * H.bf16_ulp(r[17])
    with pytest.raises(AssertionError):
        H.check_close(g, r, "two ulp")
