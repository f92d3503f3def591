"""Pins of the draft-side Markov block-decode oracle.

The structure is fixed by the pages (a rank-r previous-token correction to
the parallel backbone's logits, sampled one position after another; a
confidence head on [hidden ; markov features]); the readings are listed in
oracle/markov.py.  Pinned without retyping the oracle:

* a zero table leaves the base logits: greedy tokens are numpy's argmax;
* one-hot W1 rows select one table column exactly (closed form);
* sampling follows the chain's law: the first token ~ softmax((L_0 +
  W2 W1[anchor]) / T) and the second, given the first, ~ softmax((L_1 + W2
  W1[x_0]) / T) (chi-square over 2 * 10^5 seeds);
* the confidence is the logistic function of the stated dot product
  (brute force), and the threshold truncates at the first position below it.
"""
import math

import numpy as np
import pytest
from scipy import special, stats

import oracle.markov as OM
import workloads as W


def _tables(rng, V, r, scale=1.0):
    w1 = W.bf16_bits(rng.standard_normal((V, r), dtype=np.float32))
    w2 = W.bf16_bits(rng.standard_normal((V, r), dtype=np.float32) * np.float32(scale / np.sqrt(r)))
    return w1, w2


def test_zero_table_is_plain_argmax():
    rng = np.random.default_rng(1)
    b, K, V, r = 5, 4, 300, 16
    base = rng.standard_normal((b, K, V)).astype(np.float32)
    w1, _ = _tables(rng, V, r)
    w2 = np.zeros((V, r), np.uint16)
    res = OM.block_decode(base, rng.integers(0, V, b), w1, w2, np.zeros(b), np.arange(b, dtype=np.uint64))
    assert (res["tokens"] == np.argmax(base, axis=-1)).all()
    assert (res["logits"] == base).all()


def test_one_hot_feature_selects_table_column():
    rng = np.random.default_rng(2)
    V, r = 50, 8
    w1 = np.zeros((V, r), np.float32)
    cols = rng.integers(0, r, V)
    amps = rng.choice([1.0, -2.0, 0.5, 4.0], V)
    w1[np.arange(V), cols] = amps
    _, w2 = _tables(rng, V, r)
    prev = rng.integers(0, V, 12)
    corr = OM.markov_correction(W.bf16_bits(w1), w2, prev)
    w2f = W.bf16_to_f32(w2).astype(np.float64)
    for n, p in enumerate(prev):
        assert (corr[n] == amps[p] * w2f[:, cols[p]]).all()


def test_chain_law_first_two_positions():
    nseq, V, r, T = 200_000, 6, 4, 0.9
    rng = np.random.default_rng(3)
    base1 = rng.standard_normal((2, V)).astype(np.float32)
    base = np.ascontiguousarray(np.broadcast_to(base1, (nseq, 2, V)))
    w1, w2 = _tables(rng, V, r, scale=2.0)
    anchor = 2
    res = OM.block_decode(base, np.full(nseq, anchor), w1, w2, np.full(nseq, T),
                          np.arange(nseq, dtype=np.uint64) * np.uint64(7) + np.uint64(1))
    x0, x1 = res["tokens"][:, 0], res["tokens"][:, 1]
    corr = OM.markov_correction(w1, w2, np.arange(V))                 # [prev, V]
    p0 = special.softmax((base1[0].astype(np.float64) + corr[anchor]) / T)
    assert stats.chisquare(np.bincount(x0, minlength=V), p0 * nseq).pvalue > 1e-4
    for v in range(V):
        sel = x0 == v
        if sel.sum() < 2000:
            continue
        p1 = special.softmax((base1[1].astype(np.float64) + corr[v]) / T)
        assert stats.chisquare(np.bincount(x1[sel], minlength=V), p1 * sel.sum()).pvalue > 1e-4


def test_confidence_and_threshold():
    rng = np.random.default_rng(4)
    b, K, V, r, D = 3, 5, 40, 4, 6
    base = rng.standard_normal((b, K, V)).astype(np.float32)
    w1, w2 = _tables(rng, V, r)
    hidden = W.bf16_bits(rng.standard_normal((b, K, D), dtype=np.float32))
    cw = W.bf16_bits(rng.standard_normal(D + r, dtype=np.float32))
    anchors = rng.integers(0, V, b)
    res = OM.block_decode(base, anchors, w1, w2, np.zeros(b), np.arange(b, dtype=np.uint64),
                          hidden=hidden, conf_w=cw, conf_b=0.25, threshold=0.5)
    hf, cf, w1f = W.bf16_to_f32(hidden), W.bf16_to_f32(cw), W.bf16_to_f32(w1)
    toks = res["tokens"]
    for s in range(b):
        for i in range(K):
            prev = anchors[s] if i == 0 else toks[s, i - 1]
            logit = sum(float(hf[s, i, d]) * float(cf[d]) for d in range(D))
            logit += sum(float(w1f[prev, j]) * float(cf[D + j]) for j in range(r))
            want = 1.0 / (1.0 + math.exp(-(logit + 0.25)))
            assert res["confidence"][s, i] == pytest.approx(want, rel=1e-12)
        k = 0
        while k < K and res["confidence"][s, k] >= 0.5:
            k += 1
        assert res["lengths"][s] == k
