"""Pins of the oracle's log-normaliser and of the probabilities it reports.

The tempered softmax is fixed by the sampling rule (softmax(z / T) on both
sides).  The oracle's value is checked against scipy's logsumexp, an
independent library routine, and against exact invariances.
"""
import numpy as np
import pytest
from scipy import special

import workloads as W


def _rows(rng, n, V, dtype, scale):
    z = (rng.standard_normal((n, V)) * scale).astype(np.float32)
    return W.bf16_bits(z) if dtype == "bf16" else z


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [0.7, 0.8, 1.0, 2.0])
def test_log_normaliser_matches_scipy(orc, dtype, T):
    rng = np.random.default_rng(11)
    for row in _rows(rng, 6, 5000, dtype, 3.0):
        z = W.as_f32(row).astype(np.float64)
        ref = special.logsumexp(z / T)
        got = orc.row_log_normaliser(row, T)
        assert abs(got - ref) <= 1e-13 * max(1.0, abs(ref)), (got, ref)


def test_log_normaliser_masked_entries(orc):
    z = np.full(100, -np.inf, np.float32)
    z[[3, 50]] = [1.0, 2.0]
    ref = special.logsumexp(np.array([1.0, 2.0]) / 0.5)
    assert abs(orc.row_log_normaliser(z, 0.5) - ref) < 1e-14


def test_temperature_power_of_two_is_exact(orc):
    """softmax_T(z) = softmax_1(z / T): for T = 1/2 the scaled row 2z is exact in
    bf16, so both evaluations run the same arithmetic and agree to the bit."""
    rng = np.random.default_rng(3)
    for row in _rows(rng, 4, 3000, "bf16", 2.0):
        z = W.as_f32(row)
        doubled = W.bf16_bits(2.0 * z)
        np.testing.assert_array_equal(W.as_f32(doubled), 2.0 * z)
        assert orc.row_log_normaliser(row, 0.5) == orc.row_log_normaliser(doubled, 1.0)


def test_reported_probabilities_match_scipy(orc):
    case = W.make_case("p", b=3, K=4, V=3000, dtype="bf16", target_scale=2.5,
                       draft_sigma=0.7, T=0.7, seed=5)
    res = orc.sample_accept(case.target, case.draft, case.draft_tokens, case.T, case.seeds)
    for s in range(case.b):
        for i in range(case.K):
            x = case.draft_tokens[s, i]
            p = special.softmax(W.as_f32(case.target[s, i]).astype(np.float64) / case.T)[x]
            q = special.softmax(W.as_f32(case.draft[s, i]).astype(np.float64) / case.T)[x]
            assert res["p_draft"][s, i] == pytest.approx(p, rel=1e-12)
            assert res["q_draft"][s, i] == pytest.approx(q, rel=1e-12)
            assert res["r"][s, i] == pytest.approx(p / q, rel=1e-11)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("residual", [False, True])
def test_draw_cdf_matches_scipy(orc, dtype, residual):
    """The running sums the draw inverts: of softmax(p_n / T) (target mode) or
    of max(0, softmax(p_n / T) - softmax(q_n / T)) (residual mode), against
    scipy's softmax summed by numpy."""
    rng = np.random.default_rng(29)
    b, K, V, T = 2, 3, 3000, 0.8
    target = _rows(rng, b * (K + 1), V, dtype, 2.5).reshape(b, K + 1, V)
    draft = _rows(rng, b * K, V, dtype, 2.5).reshape(b, K, V)
    for s in range(b):
        for slot in range(K if residual else K + 1):
            F = orc.draw_cdf(target, draft, T, s, slot, residual)
            p = special.softmax(W.as_f32(target[s, slot]).astype(np.float64) / T)
            w = p
            if residual:
                q = special.softmax(W.as_f32(draft[s, slot]).astype(np.float64) / T)
                w = np.maximum(0.0, p - q)
            ref = np.cumsum(w)
            assert np.abs(F - ref).max() <= 1e-13, (s, slot, np.abs(F - ref).max())
            assert np.all(np.diff(F) >= 0.0)


def test_draw_cdf_rejects_bad_arguments(orc):
    rng = np.random.default_rng(30)
    target = _rows(rng, 3, 50, "f32", 1.0).reshape(1, 3, 50)
    draft = _rows(rng, 2, 50, "f32", 1.0).reshape(1, 2, 50)
    with pytest.raises(ValueError):
        orc.draw_cdf(target, draft, 0.0, 0, 0, False)        # T must be > 0
    with pytest.raises(ValueError):
        orc.draw_cdf(target, draft, 1.0, 0, 2, True)         # no residual at the bonus slot


@pytest.mark.parametrize("offset", [0.0, 3.0e5, 2.0e6])
def test_tied_maxima_at_a_tiny_temperature(orc, offset):
    """Closed form: a row whose two largest logits are equal and every other
    entry sits at least 1 below them has, at T = 1e-6, p = 1/2 at each
    maximum (the rest weigh exp(-1e6)), whatever common offset the row
    carries.  z / T reaches 2e12 at the largest offset, so a log-sum-exp
    taken on z / T before the maximum is subtracted loses about 1e-4 here."""
    V, T = 4099, 1.0e-6
    rng = np.random.default_rng(17)
    row = (offset + rng.uniform(-8.0, -1.0, V)).astype(np.float32)
    top = np.float32(offset + 0.75)
    row[[1000, 2048]] = top
    target = np.stack([row, row]).reshape(1, 2, V)               # rows p_1 and the bonus row
    draft = row.reshape(1, 1, V).copy()
    for x in (1000, 2048):
        res = orc.sample_accept(target, draft, np.array([[x]], np.int32), T, np.array([7], np.uint64))
        assert res["p_draft"][0, 0] == pytest.approx(0.5, rel=1e-12)
        assert res["q_draft"][0, 0] == pytest.approx(0.5, rel=1e-12)
        assert res["n_accepted"][0] == 1                         # p(x) = q(x): always accepted
    assert orc.row_log_normaliser(row, T) == pytest.approx(float(top) / T + np.log(2.0), rel=1e-15)
