"""Pins of the oracle's per-sequence draft length (ragged blocks).

A drafter with a confidence head may stop its block early, and a draft cap
limits it ("mlx-dspark 0.0.1" sdist diff, README "Tuning", and its
__main__.py flags --max-draft and --confidence-threshold; the confidence
output of "dspark-mlx 0.1.0", DraftBackbone.forward_spec).  A sequence with
Ks < K draft tokens verifies the block made of target rows 0..Ks and draft
rows 0..Ks-1, row Ks being its bonus position; Ks = 0 is a plain decode step.

Pinned without retyping the oracle: a ragged sequence must give what the
(separately pinned) fixed-K oracle gives on the truncated block; a Ks = 0
sequence must give numpy's argmax of row 0 (greedy) or a draw that follows
softmax(row 0 / T) (sampling, chi-square); storage past the block is never
read (poisoned with NaN and out-of-range tokens); Ks outside [0, K] makes
only its own sequence invalid.
"""
import numpy as np
import pytest
from scipy import special, stats

import workloads as W


def _truncated(case, k):
    """The batch cut to k draft tokens (every sequence, same batch indices)."""
    return (np.ascontiguousarray(case.target[:, :k + 1]), np.ascontiguousarray(case.draft[:, :k]),
            np.ascontiguousarray(case.draft_tokens[:, :k]))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ragged_equals_fixed_k_on_truncated_block(orc, dtype):
    K = 6
    case = W.make_case("ragged", b=48, K=K, V=1500, dtype=dtype, target_scale=2.0,
                       draft_sigma=0.5, T=0.8, seed=33)
    rng = np.random.default_rng(7)
    lens = rng.integers(1, K + 1, size=case.b).astype(np.int32)
    temps = np.where(np.arange(case.b) % 3 == 0, 0.0, 0.8)
    res = orc.mixed_accept(case.target, case.draft, case.draft_tokens, temps, case.seeds, lens)
    for k in range(1, K + 1):
        t, d, x = _truncated(case, k)
        n_g, tok_g, am_g = orc.greedy_accept(t, x)
        smp = orc.sample_accept(t, d, x, 0.8, case.seeds)
        for s in np.nonzero(lens == k)[0]:
            n = res["n_accepted"][s]
            if temps[s] == 0.0:
                assert n == n_g[s]
                assert (res["tokens"][s, :k + 1] == tok_g[s]).all()
                assert (res["argmax"][s, :k + 1] == am_g[s]).all()
                assert (res["argmax"][s, k + 1:] == -1).all()
            else:
                assert n == smp["n_accepted"][s]
                assert (res["tokens"][s, :k + 1] == smp["tokens"][s]).all()
                assert (res["p_draft"][s, :k] == smp["p_draft"][s]).all()
                assert (res["q_draft"][s, :k] == smp["q_draft"][s]).all()
                assert np.isnan(res["p_draft"][s, k:]).all() and np.isnan(res["q_draft"][s, k:]).all()
            assert (res["tokens"][s, k + 1:] == -1).all()
    # K_s = K everywhere is the same call as no lengths at all
    full = orc.mixed_accept(case.target, case.draft, case.draft_tokens, temps, case.seeds,
                            np.full(case.b, K, np.int32))
    ref = orc.mixed_accept(case.target, case.draft, case.draft_tokens, temps, case.seeds)
    for key in ("n_accepted", "tokens", "argmax"):
        assert (full[key] == ref[key]).all()


def test_storage_past_the_block_is_not_read(orc):
    K = 5
    case = W.make_case("poison", b=24, K=K, V=900, dtype="f32", target_scale=2.0,
                       draft_sigma=0.5, T=0.8, seed=34)
    lens = (np.arange(case.b) % (K + 1)).astype(np.int32)
    temps = np.where(np.arange(case.b) % 2 == 0, 0.0, 0.8)
    clean = orc.mixed_accept(case.target, case.draft, case.draft_tokens, temps, case.seeds, lens)
    t, d, x = case.target.copy(), case.draft.copy(), case.draft_tokens.copy()
    for s, k in enumerate(lens):
        t[s, k + 1:] = np.nan
        d[s, k:] = np.nan
        x[s, k:] = -7
    dirty = orc.mixed_accept(t, d, x, temps, case.seeds, lens)
    assert (clean["n_accepted"] >= 0).all()
    for key in ("n_accepted", "tokens", "argmax"):
        assert (dirty[key] == clean[key]).all()
    ok = ~np.isnan(clean["p_draft"])
    assert (dirty["p_draft"][ok] == clean["p_draft"][ok]).all()


def test_zero_length_greedy_is_argmax_of_first_row(orc):
    case = W.make_case("k0g", b=16, K=3, V=777, dtype="bf16", target_scale=2.0,
                       draft_sigma=0.5, T=0.8, seed=35)
    lens = np.zeros(case.b, np.int32)
    res = orc.mixed_accept(case.target, case.draft, case.draft_tokens, np.zeros(case.b),
                           case.seeds, lens)
    A0 = np.argmax(W.as_f32(case.target)[:, 0], axis=-1)
    assert (res["n_accepted"] == 0).all()
    assert (res["tokens"][:, 0] == A0).all() and (res["tokens"][:, 1:] == -1).all()
    assert (res["argmax"][:, 0] == A0).all() and (res["argmax"][:, 1:] == -1).all()


def test_zero_length_sampling_follows_first_row_law(orc):
    """With no draft tokens the committed token is a draw from p_1."""
    nseq, K, V, T = 200_000, 2, 8, 0.7
    rng = np.random.default_rng(36)
    zt = (rng.standard_normal((K + 1, V)) * 1.2).astype(np.float32)
    target = np.ascontiguousarray(np.broadcast_to(zt, (nseq, K + 1, V)))
    draft = np.zeros((nseq, K, V), np.float32)
    tokens = np.zeros((nseq, K), np.int32)
    seeds = np.arange(nseq, dtype=np.uint64) * np.uint64(104729) + np.uint64(5)
    res = orc.mixed_accept(target, draft, tokens, np.full(nseq, T), seeds,
                           np.zeros(nseq, np.int32))
    assert (res["n_accepted"] == 0).all() and (res["tokens"][:, 1:] == -1).all()
    p1 = special.softmax(zt[0].astype(np.float64) / T)
    counts = np.bincount(res["tokens"][:, 0], minlength=V)
    assert stats.chisquare(counts, p1 * nseq).pvalue > 1e-4


def test_length_out_of_range_invalidates_only_its_sequence(orc):
    K = 4
    case = W.make_case("badlen", b=8, K=K, V=600, dtype="f32", target_scale=2.0,
                       draft_sigma=0.5, T=0.8, seed=37)
    lens = np.full(case.b, K, np.int32)
    lens[2], lens[5] = -1, K + 1
    temps = np.array([0.0, 0.8] * 4)
    res = orc.mixed_accept(case.target, case.draft, case.draft_tokens, temps, case.seeds, lens)
    ref = orc.mixed_accept(case.target, case.draft, case.draft_tokens, temps, case.seeds)
    for s in range(case.b):
        if s in (2, 5):
            assert res["n_accepted"][s] == -1 and (res["tokens"][s] == -1).all()
        else:
            assert res["n_accepted"][s] == ref["n_accepted"][s]
            assert (res["tokens"][s] == ref["tokens"][s]).all()
