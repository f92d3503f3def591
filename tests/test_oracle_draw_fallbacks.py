"""Pins of the oracle's two draw fallbacks.

1. Zero residual mass.  A slot is rejected while max(0, p_n - q_n) is zero
   everywhere: with identical target and draft rows and a draft token masked
   (-inf) in both, p(x) = 0 rejects the slot and the residual has no mass.
   In exact arithmetic the published rule (Leviathan et al. 2023; Chen et al.
   2023) never reaches this case with p != q, and the pages' policy is
   lossless ("dspark-mlx 0.1.0", dspark_mlx/adapter.py docstring), so the
   committed token must still follow the target: the oracle draws it from
   p_n itself.  Pinned by one-hot fixtures (tests/golden/sampling_hand.json,
   the two "zero residual mass" cases) and by chi-square against p_n at
   slots 0 and 1.

2. The rounding fallback of the inverse-CDF search.  The running sum walks
   the same weights in the same order as the total R, so it reaches R
   exactly, and t = u' * R < R whenever u' * R rounds below R.  It can only
   round up to R when R is subnormal with few significant bits and u' is
   close to 1; then no running sum exceeds t and the draw takes the last
   entry of positive weight, which is also the exact-arithmetic answer for
   such u'.  Pinned on rows whose residual mass is about 1e-322 (float32
   logits near -740, so only a double oracle sees it).

Negative controls: oracle builds with a planted mistake in each branch
(ORACLE_MUTANT 6, 7, 8; see spec_oracle.c) must fail these pins.
"""
import json
import os

import numpy as np
import pytest
from scipy import special, stats

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
NINF = -np.inf


def _golden_zero_mass_cases():
    with open(os.path.join(GOLDEN, "sampling_hand.json")) as f:
        cases = json.load(f)["cases"]
    return [c for c in cases if c["name"].startswith("zero residual mass")]


def _run_golden(orc, c, nseeds=8):
    tgt = np.array(c["target"], dtype=np.float32)[None]
    drf = np.array(c["draft"], dtype=np.float32)[None]
    tok = np.array(c["draft_tokens"], dtype=np.int32)[None]
    out = []
    for seed in range(nseeds):
        res = orc.sample_accept(tgt, drf, tok, c["temperature"], np.array([seed], np.uint64))
        out.append((int(res["n_accepted"][0]), res["tokens"][0].tolist(), float(res["R"][0]),
                    float(res["residual"][0])))
    return out


def test_zero_mass_golden_cases_take_the_fallback(orc):
    cases = _golden_zero_mass_cases()
    assert len(cases) == 2
    for c in cases:
        for n, tok, R, resid in _run_golden(orc, c):
            assert n == c["n_accepted"] and tok == c["tokens"], c["name"]
            # the draw used p_n (residual flag 0), whose mass is 1
            assert resid == 0.0 and R == pytest.approx(1.0, abs=1e-15), c["name"]


def _zero_mass_block(rng, V=8, K=2, slot=0, N=200_000, T=0.9):
    """N sequences sharing one block whose slot `slot` has identical target
    and draft rows with the draft token masked in both; earlier slots have
    identical rows with a finite draft token (ratio exactly 1, accepted)."""
    zt = (rng.standard_normal((K + 1, V)) * 1.3).astype(np.float32)
    zd = zt[:K].copy()
    x = np.zeros(K, np.int32)
    for i in range(K):
        x[i] = int(rng.integers(0, V))
    zt[slot, x[slot]] = NINF
    zd[slot] = zt[slot]
    for i in range(slot):
        zd[i] = zt[i]
    for i in range(slot + 1, K):          # later slots: arbitrary draft rows
        zd[i] = (zt[i] + rng.standard_normal(V) * 0.5).astype(np.float32)
    target = np.ascontiguousarray(np.broadcast_to(zt, (N, K + 1, V)))
    draft = np.ascontiguousarray(np.broadcast_to(zd, (N, K, V)))
    tokens = np.ascontiguousarray(np.broadcast_to(x, (N, K)))
    seeds = np.arange(N, dtype=np.uint64) * np.uint64(104729) + np.uint64(3)
    p = special.softmax(zt.astype(np.float64) / T, axis=-1)
    return dict(target=target, draft=draft, tokens=tokens, seeds=seeds, T=T, p=p, slot=slot, V=V, K=K)


def _zero_mass_pvalue(orc, blk):
    """Chi-square p-value of the token drawn at the zero-mass slot against
    p_n; 0 when a token outside p_n's support (or no token) was drawn."""
    res = orc.sample_accept(blk["target"], blk["draft"], blk["tokens"], blk["T"], blk["seeds"])
    slot = blk["slot"]
    n, tok = res["n_accepted"], res["tokens"]
    assert (n == slot).all()
    y = tok[:, slot]
    p = blk["p"][slot]
    if (y < 0).any() or (p[np.maximum(y, 0)] == 0.0).any():
        return 0.0
    counts = np.bincount(y, minlength=blk["V"])
    pos = p > 0
    return stats.chisquare(counts[pos], p[pos] * len(n)).pvalue


@pytest.mark.parametrize("slot", [0, 1])
def test_zero_mass_draw_follows_p_n(orc, slot):
    blk = _zero_mass_block(np.random.default_rng(40 + slot), slot=slot)
    pv = _zero_mass_pvalue(orc, blk)
    assert pv > 0.01, pv


@pytest.mark.parametrize("mutant", [6, 7])
def test_planted_mistakes_fail_zero_mass_pins(tmp_path, mutant):
    mut = oracle.Oracle(oracle.build(str(tmp_path / f"mut{mutant}.so"), mutant=mutant))
    golden_ok = all(n == c["n_accepted"] and tok == c["tokens"]
                    for c in _golden_zero_mass_cases() for n, tok, _, _ in _run_golden(mut, c, 2))
    pvals = [_zero_mass_pvalue(mut, _zero_mass_block(np.random.default_rng(40 + s), slot=s, N=20_000))
             for s in (0, 1)]
    assert not golden_ok, mutant
    assert min(pvals) < 1e-6, (mutant, pvals)


# ---------------------------------------------------------------- rounding fallback


def _subnormal_residual_block(N=4000):
    """Slot 0: the draft token (4) has p = 0 and a tiny q, so it is rejected;
    entries 0..3 are identical in both rows (zero residual); entries 5 and 6
    carry the whole residual mass, exp(-740 - C) and exp(-740.5 - C), about
    1e-322 together: a subnormal with a few significant bits."""
    zt = np.array([[0.5, -0.25, 1.0, 0.0, NINF, -740.0, -740.5, NINF],
                   [0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0]], np.float32)
    zd = np.array([[0.5, -0.25, 1.0, 0.0, -740.0, NINF, NINF, NINF]], np.float32)
    target = np.ascontiguousarray(np.broadcast_to(zt, (N, 2, 8)))
    draft = np.ascontiguousarray(np.broadcast_to(zd, (N, 1, 8)))
    tokens = np.full((N, 1), 4, np.int32)
    return target, draft, tokens, np.arange(N, dtype=np.uint64)


def test_rounding_fallback_takes_last_positive_weight(orc):
    target, draft, tokens, seeds = _subnormal_residual_block()
    res = orc.sample_accept(target, draft, tokens, 1.0, seeds)
    assert (res["n_accepted"] == 0).all() and (res["residual"] == 1.0).all()
    R = res["R"]
    assert (R > 0).all() and (R < np.finfo(np.float64).tiny).all()    # subnormal mass
    y = res["tokens"][:, 0]
    assert set(np.unique(y).tolist()) <= {5, 6}                       # only positive-weight entries
    fell_back = res["t"] == R                                         # u' * R rounded up to R
    assert fell_back.sum() >= 20
    assert (y[fell_back] == 6).all()                                  # the last positive entry
    # u' that high lies above entry 5's exact share 1 / (1 + e^-0.5), so 6 is
    # also the exact-arithmetic answer
    assert (res["u2"][fell_back] > 1.0 / (1.0 + np.exp(-0.5))).all()


def test_planted_first_positive_fails_rounding_pin(tmp_path):
    mut = oracle.Oracle(oracle.build(str(tmp_path / "mut8.so"), mutant=8))
    target, draft, tokens, seeds = _subnormal_residual_block()
    res = mut.sample_accept(target, draft, tokens, 1.0, seeds)
    fell_back = res["t"] == res["R"]
    assert fell_back.any()
    assert (res["tokens"][fell_back, 0] != 6).all()
