"""The issue-rate probe (ss2d_probe_issue_rates) through the C ABI: its rates are positive,
consistent with one another and within what the chip can issue.

The bounds are those of the issue model the roofline diagnostics use: a SIMD issues one
wave64 fp32 instruction per 4 cycles (16 lanes per cycle), so fused multiply-adds run at most
CUs x 4 x 16 x the clock; an exponential costs at least one such slot; a group of 4
multiply-adds and one exponential costs at least 5.
"""
import pytest

from tests.gpu_util import log

pytestmark = pytest.mark.gpu


def test_issue_rates_are_within_the_issue_model():
    import selective_scan_ss2d_amd as ss
    r = ss.probe_issue_rates()
    log(f"issue rates: {r}")
    clock = r["clock_hz"]
    assert 0.5e9 < clock < 3.5e9, r
    cus = r["compute_units"]
    assert cus > 0, r
    peak = cus * 4 * 16 * clock
    # allow 10% for the clock reading being taken from one launch of the three
    assert 0.2 * peak < r["fma_per_s"] <= 1.1 * peak, (r, peak)
    assert 0.0 < r["exp_per_s"] <= 1.02 * r["fma_per_s"], r
    assert 0.0 < r["update_mix_per_s"] <= 1.02 * r["fma_per_s"] / 5, r
