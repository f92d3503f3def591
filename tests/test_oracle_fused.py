"""Pins of the fused-verify oracle (lm_head logits + softcap, then accept).

The logits are defined by the Gemma-4 drafter code of "dspark-mlx 0.1.0"
(dspark_mlx/arch/gemma4.py): a bias-free Linear(hidden_size, vocab_size)
with weight [V, D] on float32 hidden states, then c * tanh(a / c).  Pinned
without retyping the oracle's formula:

* one-hot hidden rows select one weight column exactly (closed form);
* a tiny case summed exactly in rational arithmetic (brute force);
* the softcap against math.tanh, its odd symmetry, its bound |.| < c and its
  small-argument expansion a - a^3 / (3 c^2);
* the float32 accumulation bound: numpy's float32 product of the same inputs
  (an independent float32 computation) stays within gamma_D * sum |h w|;
* planted workloads: each target row's planted token is the argmax the
  construction makes it, so the greedy oracle accepts every agreeing draft.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle.fused as F
import workloads as W


def test_one_hot_hidden_selects_weight_column():
    rng = np.random.default_rng(3)
    b, K, D, V = 3, 2, 48, 700
    weight = W.bf16_bits(rng.standard_normal((V, D), dtype=np.float32))
    hidden = np.zeros((b, K + 1, D), np.float32)
    cols = rng.integers(0, D, size=(b, K + 1))
    amps = np.array([1.0, -2.0, 0.5, 4.0, -0.25, 8.0, 3.0, -1.5, 0.75])
    for n, (s, i) in enumerate(np.ndindex(b, K + 1)):
        hidden[s, i, cols[s, i]] = amps[n]
    z = F.lm_head_logits(W.bf16_bits(hidden), weight, 0.0)
    wf = W.bf16_to_f32(weight).astype(np.float64)
    for n, (s, i) in enumerate(np.ndindex(b, K + 1)):
        assert (z[s, i] == amps[n] * wf[:, cols[s, i]]).all()


def test_exact_rational_sum():
    rng = np.random.default_rng(4)
    b, K, D, V = 2, 1, 9, 5
    h = (rng.integers(-40, 40, size=(b, K + 1, D)) / 8.0).astype(np.float32)
    w = (rng.integers(-40, 40, size=(V, D)) / 16.0).astype(np.float32)
    z = F.lm_head_logits(W.bf16_bits(h), W.bf16_bits(w), 0.0)
    for s, i, v in np.ndindex(b, K + 1, V):
        exact = sum(Fraction(float(h[s, i, d])) * Fraction(float(w[v, d])) for d in range(D))
        assert z[s, i, v] == float(exact)


def test_softcap_properties():
    c = 30.0
    xs = np.array([-200.0, -31.0, -1.0, -1e-3, 0.0, 1e-3, 2.5, 29.0, 90.0])
    y = F.softcap(xs, c)
    assert y[4] == 0.0
    for x, v in zip(xs, y):
        assert v == pytest.approx(c * math.tanh(x / c), rel=1e-15, abs=1e-300)
    assert (np.abs(y) < c).all()
    assert (F.softcap(-xs, c) == -y).all()
    small = np.array([1e-3, -2e-2, 0.1])
    assert np.allclose(F.softcap(small, c), small - small ** 3 / (3 * c * c), rtol=1e-9, atol=0)
    assert (F.softcap(xs, 0.0) == xs).all()


@pytest.mark.parametrize("D", [64, 1000, 3840])
def test_float32_accumulation_within_gamma_bound(D):
    rng = np.random.default_rng(D)
    b, K, V = 2, 3, 2000
    hidden = W.bf16_bits(rng.standard_normal((b, K + 1, D), dtype=np.float32))
    weight = W.bf16_bits(rng.standard_normal((V, D), dtype=np.float32) * np.float32(3 / np.sqrt(D)))
    z64 = F.lm_head_logits(hidden, weight, 0.0)
    H32 = W.bf16_to_f32(hidden).reshape(-1, D)
    z32 = (H32 @ W.bf16_to_f32(weight).T).reshape(b, K + 1, V)   # numpy float32 product
    bound = F.gamma(D) * F.abs_products(hidden, weight)
    err = np.abs(z32.astype(np.float64) - z64)
    assert (err <= bound).all()
    assert err.max() > 0.0       # the float32 product does round


def test_planted_rows_accept_every_agreeing_draft():
    case = W.make_fused_case("pin", b=6, K=4, V=3000, D=512, softcap=30.0, gain=(24.0, 28.0),
                             agree=1.0, rule=W.GREEDY, seed=5)
    res = F.fused_mixed_accept(case.hidden, case.weight, case.softcap, case.draft,
                               case.draft_tokens, case.temps, case.seeds)
    assert (res["argmax"] == case.planted).all()
    assert (res["n_accepted"] == case.K).all()
    assert (res["tokens"][:, :case.K] == case.planted[:, :case.K]).all()
    assert (res["tokens"][:, case.K] == case.planted[:, case.K]).all()


def test_sequence_subset_matches_full_batch():
    case = W.make_fused_case("sub", b=6, K=3, V=2500, D=256, rule=[0, 1, 0, 1, 1, 0], seed=6)
    full = F.fused_mixed_accept(case.hidden, case.weight, case.softcap, case.draft,
                                case.draft_tokens, case.temps, case.seeds)
    sub = F.fused_mixed_accept(case.hidden, case.weight, case.softcap, case.draft,
                               case.draft_tokens, case.temps, case.seeds, seqs=[1, 2, 5])
    for j, s in enumerate([1, 2, 5]):
        assert sub["n_accepted"][s] == full["n_accepted"][s]
        assert (sub["tokens"][s] == full["tokens"][s]).all()
        assert (sub["logits32"][j] == full["logits32"][s]).all()
