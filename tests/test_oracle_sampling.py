"""Pins of the oracle's speculative-sampling accept (statistical and exact).

The pages assert the property the rule must have: decoding is lossless, the
target's verify forward being the only token source ("DeepSeek-V4-Flash
DSpark drafter" model card; the "lossless accept policy" of "dspark-mlx
0.1.0", dspark_mlx/adapter.py).  The rule is the published speculative-
sampling rule (Leviathan et al. 2023; Chen et al. 2023).  Its laws are pinned
here without retyping the oracle's formulas:

* losslessness: with drafts x_i ~ q_i the committed token at every slot that
  is reached follows p_i (chi-square over 10^6 seeded sequences, V=8, K=3);
* a multi-block Markov-chain generation whose joint law must be the target
  chain's;
* closed forms: P(accept slot 1) = sum_v min(p, q); E[n] = sum_j prod_{i<=j} alpha_i;
  the token drawn after a rejection at slot 1 follows normalise(max(0, p - q));
* the special case draft == target (every slot accepted, bonus ~ p_{K+1});
* hand-made deterministic fixtures (one-hot rows);
* negative controls: builds of the oracle with a planted mistake must fail.
"""
import json
import os

import numpy as np
import pytest
from scipy import special, stats

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
NSEQ = 1_000_000


def _draw(rng, probs, n):
    """n iid draws from a categorical law (inverse CDF of numpy uniforms)."""
    cdf = np.cumsum(probs)
    cdf[-1] = 1.0
    return np.searchsorted(cdf, rng.random(n), side="right").astype(np.int32)


@pytest.fixture(scope="module")
def fixed_block():
    """One [K+1, V] target block and [K, V] draft block shared by all sequences."""
    rng = np.random.default_rng(2024)
    K, V, T = 3, 8, 0.7
    zt = (rng.standard_normal((K + 1, V)) * 1.2).astype(np.float32)
    zd = (zt[:K] + rng.standard_normal((K, V)) * 0.6).astype(np.float32)
    p = special.softmax(zt.astype(np.float64) / T, axis=-1)
    q = special.softmax(zd.astype(np.float64) / T, axis=-1)
    tokens = np.stack([_draw(rng, q[i], NSEQ) for i in range(K)], axis=1)
    target = np.ascontiguousarray(np.broadcast_to(zt, (NSEQ, K + 1, V)))
    draft = np.ascontiguousarray(np.broadcast_to(zd, (NSEQ, K, V)))
    seeds = np.arange(NSEQ, dtype=np.uint64) * np.uint64(7919) + np.uint64(11)
    return dict(K=K, V=V, T=T, p=p, q=q, target=target, draft=draft, tokens=tokens, seeds=seeds)


def _slot_pvalues(res, blk):
    """Chi-square p-value of the committed token at each slot j against p_{j+1},
    over the sequences that reached slot j."""
    n, tok = res["n_accepted"], res["tokens"]
    out = []
    for j in range(blk["K"] + 1):
        reached = n >= j
        counts = np.bincount(tok[reached, j], minlength=blk["V"])
        exp = blk["p"][j] * reached.sum()
        out.append(stats.chisquare(counts, exp).pvalue)
    return out


def _run(orc, blk):
    return orc.sample_accept(blk["target"], blk["draft"], blk["tokens"], blk["T"], blk["seeds"])


@pytest.fixture(scope="module")
def fixed_result(orc, fixed_block):
    return _run(orc, fixed_block)


def test_lossless_every_slot(fixed_block, fixed_result):
    pv = _slot_pvalues(fixed_result, fixed_block)
    assert min(pv) > 0.01, pv
    # every slot, including the bonus, is reached often enough to test
    assert (fixed_result["n_accepted"] == fixed_block["K"]).sum() > 50_000


def test_closed_form_acceptance(fixed_block, fixed_result):
    p, q, K = fixed_block["p"], fixed_block["q"], fixed_block["K"]
    alpha = np.minimum(p[:K], q).sum(axis=1)           # 1 - TV(p_i, q_i)
    n = fixed_result["n_accepted"]
    acc0 = (n >= 1).mean()
    z = (acc0 - alpha[0]) / np.sqrt(alpha[0] * (1 - alpha[0]) / NSEQ)
    assert abs(z) < 4.5, (acc0, alpha[0])
    En = sum(np.prod(alpha[:j]) for j in range(1, K + 1))
    z = (n.mean() - En) / (n.std() / np.sqrt(NSEQ))
    assert abs(z) < 4.5, (n.mean(), En)
    for j in range(1, K + 1):              # P(n >= j) = prod_{i<j} alpha_i
        pj = np.prod(alpha[:j])
        z = ((n >= j).mean() - pj) / np.sqrt(pj * (1 - pj) / NSEQ)
        assert abs(z) < 4.5, (j, (n >= j).mean(), pj)


def test_residual_law_after_rejection(fixed_block, fixed_result):
    p, q, V = fixed_block["p"][0], fixed_block["q"][0], fixed_block["V"]
    w = np.maximum(0.0, p - q)
    rej = fixed_result["n_accepted"] == 0
    counts = np.bincount(fixed_result["tokens"][rej, 0], minlength=V)
    assert counts[w == 0].sum() == 0            # zero-weight tokens are never drawn
    pos = w > 0
    pv = stats.chisquare(counts[pos], w[pos] / w.sum() * rej.sum()).pvalue
    assert pv > 0.01, pv


def test_accept_decisions_consistent_with_diagnostics(fixed_result, fixed_block):
    n, r, u = fixed_result["n_accepted"], fixed_result["r"], fixed_result["u"]
    K = fixed_block["K"]
    idx = np.arange(K)[None, :]
    acc = u < np.minimum(1.0, r)
    assert (acc | (idx >= n[:, None])).all()
    rej_at_n = np.take_along_axis(acc, np.minimum(n, K - 1)[:, None], axis=1)[:, 0]
    assert not rej_at_n[n < K].any()


@pytest.mark.parametrize("mutant", [1, 2, 3, 5])
def test_planted_mistakes_fail_losslessness(tmp_path, fixed_block, mutant):
    mut = oracle.Oracle(oracle.build(str(tmp_path / f"mut{mutant}.so"), mutant=mutant))
    pv = _slot_pvalues(_run(mut, fixed_block), fixed_block)
    assert min(pv) < 1e-6, (mutant, pv)


def test_draft_equal_to_target_accepts_all(orc):
    """q == p bitwise: every ratio is exactly 1, so every slot is accepted and
    the committed bonus follows p_{K+1}."""
    rng = np.random.default_rng(99)
    K, V, T, N = 3, 8, 1.0, 200_000
    zt = W.bf16_bits((rng.standard_normal((K + 1, V)) * 1.5).astype(np.float32))
    p = special.softmax(W.as_f32(zt).astype(np.float64) / T, axis=-1)
    target = np.ascontiguousarray(np.broadcast_to(zt, (N, K + 1, V)))
    draft = np.ascontiguousarray(target[:, :K])
    tokens = np.stack([_draw(rng, p[i], N) for i in range(K)], axis=1)
    res = orc.sample_accept(target, draft, tokens, T, np.arange(N, dtype=np.uint64))
    assert (res["n_accepted"] == K).all()
    assert (res["r"] == 1.0).all()
    counts = np.bincount(res["tokens"][:, K], minlength=V)
    assert stats.chisquare(counts, p[K] * N).pvalue > 0.01


def test_markov_chain_generation_is_lossless(orc):
    """Honest multi-block generation on an 8-state chain: the target block rows
    are P[previous token] along the drafted prefix, the draft rows Q[...].
    The joint law of the first three generated tokens must be the target
    chain's (chi-square over cells with expectation >= 5)."""
    rng = np.random.default_rng(5)
    V, K, L, N = 8, 2, 3, 400_000
    P = rng.dirichlet(np.full(V, 0.7), size=V)
    Q = 0.5 * P + 0.5 * rng.dirichlet(np.full(V, 0.7), size=V)
    logP = np.log(P).astype(np.float32)
    logQ = np.log(Q).astype(np.float32)
    # exp(float32(log P)) is the law actually fed; use it for the expectation
    Pf = special.softmax(logP.astype(np.float64), axis=-1)
    Qf = special.softmax(logQ.astype(np.float64), axis=-1)
    out = np.full((N, L), -1, np.int32)
    count = np.zeros(N, np.int32)
    last = np.zeros(N, np.int32)            # start token 0
    cycle = 0
    while (count < L).any():
        act = np.nonzero(count < L)[0]
        b = len(act)
        x = np.zeros((b, K), np.int32)
        prev = last[act]
        for i in range(K):
            cdf = np.cumsum(Qf[prev], axis=1)
            x[:, i] = (rng.random((b, 1)) > cdf).sum(axis=1).clip(max=V - 1)
            prev = x[:, i]
        ctx = np.concatenate([last[act][:, None], x], axis=1)      # [b, K+1]
        target = np.ascontiguousarray(logP[ctx])                   # rows P[ctx_i]
        draft = np.ascontiguousarray(logQ[ctx[:, :K]])
        seeds = (act.astype(np.uint64) << np.uint64(8)) + np.uint64(cycle)
        res = orc.sample_accept(target, draft, x, 1.0, seeds)
        n = res["n_accepted"]
        for j in range(K + 1):
            take = (n >= j) & (count[act] < L)
            rows = act[take]
            out[rows, count[rows]] = res["tokens"][take, j]
            count[rows] += 1
        done = np.arange(b)
        last[act] = res["tokens"][done, n]
        cycle += 1
    cell = out[:, 0] * V * V + out[:, 1] * V + out[:, 2]
    counts = np.bincount(cell, minlength=V ** 3)
    a, bb, c = np.meshgrid(np.arange(V), np.arange(V), np.arange(V), indexing="ij")
    expected = (Pf[0][a] * Pf[a, bb] * Pf[bb, c]).reshape(-1) * N
    keep = expected >= 5
    obs = counts[keep].astype(np.float64)
    exp_k = expected[keep]
    chi2 = ((obs - exp_k) ** 2 / exp_k).sum()
    chi2 += (counts[~keep].sum() - expected[~keep].sum()) ** 2 / max(expected[~keep].sum(), 1e-9)
    dof = keep.sum()
    assert stats.chi2.sf(chi2, dof) > 0.01, (chi2, dof)


def test_sampling_hand_fixtures(orc):
    """One-hot rows make every decision independent of the uniforms."""
    with open(os.path.join(GOLDEN, "sampling_hand.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        tgt = np.array(c["target"], dtype=np.float32)[None]
        drf = np.array(c["draft"], dtype=np.float32)[None]
        tok = np.array(c["draft_tokens"], dtype=np.int32)[None]
        for seed in range(5):
            res = orc.sample_accept(tgt, drf, tok, c["temperature"], np.array([seed], np.uint64))
            assert res["n_accepted"][0] == c["n_accepted"], c["name"]
            assert res["tokens"][0].tolist() == c["tokens"], c["name"]


def test_invalid_inputs(orc):
    case = W.make_case("inv", b=5, K=2, V=64, dtype="f32", seed=1)
    t, d, x = case.target.copy(), case.draft.copy(), case.draft_tokens.copy()
    t[0, 2, 7] = np.nan          # bonus row holds NaN
    d[1, 0, :] = -np.inf         # draft row without a finite entry
    t[2, 1, 0] = np.inf
    x[3, 1] = -1                 # token outside the vocabulary
    res = orc.sample_accept(t, d, x, 1.0, case.seeds)
    assert list(res["n_accepted"][:4]) == [-1] * 4
    assert (res["tokens"][:4] == -1).all()
    assert res["n_accepted"][4] >= 0
    with pytest.raises(ValueError):
        orc.sample_accept(t, d, x, 0.0, case.seeds)
    with pytest.raises(ValueError):
        orc.sample_accept(t, d, x, float("inf"), case.seeds)


def test_mixed_batch_is_per_sequence_dispatch(orc):
    """A mixed batch (temperature 0 = greedy, else sampling) gives every
    sequence what the single-rule oracle gives it at the same batch index;
    a negative or non-finite temperature invalidates only its sequence."""
    case = W.make_case("mix", b=10, K=3, V=2000, dtype="bf16", target_scale=2.0,
                       draft_sigma=0.6, T=0.8, seed=21)
    temps = np.array([0.0, 0.8] * 5)
    temps[9] = -1.0
    res = orc.mixed_accept(case.target, case.draft, case.draft_tokens, temps, case.seeds)
    n_g, tok_g, am_g = orc.greedy_accept(case.target, case.draft_tokens)
    smp = orc.sample_accept(case.target, case.draft, case.draft_tokens, 0.8, case.seeds)
    for s in range(10):
        if s == 9:
            assert res["n_accepted"][s] == -1 and (res["tokens"][s] == -1).all()
        elif temps[s] == 0.0:
            assert res["n_accepted"][s] == n_g[s]
            assert (res["tokens"][s] == tok_g[s]).all() and (res["argmax"][s] == am_g[s]).all()
            assert np.isnan(res["p_draft"][s]).all()
        else:
            assert res["n_accepted"][s] == smp["n_accepted"][s]
            assert (res["tokens"][s] == smp["tokens"][s]).all()
            assert (res["p_draft"][s] == smp["p_draft"][s]).all()
            assert (res["argmax"][s] == -1).all()
