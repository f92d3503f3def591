"""Pins of the oracle's greedy accept.

The pages fix greedy accept by its result: the committed tokens are the
target's own argmax chain, so the output equals plain greedy decoding
("mlx-dspark 0.0.1" sdist diff, README "How it works";
benchmark.py takes the plain greedy token as argmax of the raw logits).  The
block convention ([K+1, V], row K the bonus position) is the one of
"dspark-mlx 0.1.0", dspark_mlx/adapter.py.  Pinned against numpy.argmax
(first index among equal maxima), by brute force and by hand-made fixtures.
"""
import json
import os

import numpy as np
import pytest

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _expected(target, tokens):
    z = W.as_f32(target)
    A = np.argmax(z, axis=-1)                 # numpy: first index of the max
    b, K = tokens.shape
    n = np.zeros(b, np.int32)
    out = np.full((b, K + 1), -1, np.int32)
    for s in range(b):
        k = 0
        while k < K and tokens[s, k] == A[s, k]:
            k += 1
        n[s] = k
        out[s, :k] = tokens[s, :k]
        out[s, k] = A[s, k]
    return n, out, A


def _with_ties(rng, b, K, V, dtype):
    z = np.round(rng.standard_normal((b, K + 1, V)) * 2.0).astype(np.float32)  # many exact ties
    tgt = W.bf16_bits(z) if dtype == "bf16" else z
    A = np.argmax(W.as_f32(tgt), axis=-1)
    tokens = A[:, :K].copy()
    # break the chain at a random place in half the sequences, sometimes with
    # a token that ties the maximum at a higher index (must be rejected)
    for s in range(b):
        if s % 2 == 0:
            continue
        j = rng.integers(K)
        row = W.as_f32(tgt[s, j])
        tied = np.nonzero(row == row.max())[0]
        tokens[s, j] = tied[-1] if len(tied) > 1 else (A[s, j] + 1) % V
    return tgt, tokens.astype(np.int32)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_greedy_matches_numpy_argmax_chain(orc, dtype):
    rng = np.random.default_rng(1)
    tgt, tok = _with_ties(rng, 40, 5, 257, dtype)
    n, out, am = orc.greedy_accept(tgt, tok)
    en, eout, eA = _expected(tgt, tok)
    np.testing.assert_array_equal(am, eA)
    np.testing.assert_array_equal(n, en)
    np.testing.assert_array_equal(out, eout)
    assert (n < 5).any() and (n == 5).any()


def test_greedy_chain_invariants_on_workload(orc):
    case = W.config(2, b=4, V=4096)
    n, out, am = orc.greedy_accept(case.target, case.draft_tokens)
    for s in range(case.b):
        k = n[s]
        assert 0 <= k <= case.K
        assert (out[s, :k] == case.draft_tokens[s, :k]).all()
        assert (out[s, :k + 1] == am[s, :k + 1]).all()     # the target argmax chain
        assert (out[s, k + 1:] == -1).all()
        assert (k == case.K) == bool((case.draft_tokens[s] == am[s, :case.K]).all())


def test_greedy_tie_breaking_mutant_is_caught(tmp_path):
    mut = oracle.Oracle(oracle.build(str(tmp_path / "mut4.so"), mutant=4))
    rng = np.random.default_rng(1)
    tgt, tok = _with_ties(rng, 40, 5, 257, "bf16")
    n, out, am = mut.greedy_accept(tgt, tok)
    en, eout, eA = _expected(tgt, tok)
    assert not np.array_equal(am, eA)


def test_greedy_invalid_rows(orc):
    V, K = 16, 3
    base = np.arange(4 * (K + 1) * V, dtype=np.float32).reshape(4, K + 1, V) % 7
    tok = np.zeros((4, K), np.int32)
    t = base.copy()
    t[0, 1, 5] = np.nan
    t[1, 3, :] = -np.inf
    t[2, 0, 2] = np.inf
    t[3, 2, :4] = -np.inf          # masked entries are allowed
    n, out, am = orc.greedy_accept(t, tok)
    assert list(n[:3]) == [-1, -1, -1] and (out[:3] == -1).all()
    assert n[3] >= 0
    bad = tok.copy()
    bad[3, 1] = V                   # token outside the vocabulary
    n2, out2, _ = orc.greedy_accept(t, bad)
    assert n2[3] == -1 and (out2[3] == -1).all()


def test_greedy_hand_fixtures(orc):
    with open(os.path.join(GOLDEN, "greedy_hand.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        tgt = np.array(c["target"], dtype=np.float32)[None]
        tok = np.array(c["draft_tokens"], dtype=np.int32)[None]
        n, out, _ = orc.greedy_accept(tgt, tok)
        assert n[0] == c["n_accepted"], c["name"]
        assert out[0].tolist() == c["tokens"], c["name"]
