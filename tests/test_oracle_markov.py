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
* the confidence head in closed form: a one-hot weight on hidden feature d
  gives expit(+-h[d] + c) (scipy's logistic), a one-hot weight on Markov
  feature j gives expit(W1[previous token, j] + c) with the previous token
  the anchor at position 0, zero weights give expit(c); a planted crossing
  fixes the draft length, no threshold keeps all K, and a confidence equal
  to the threshold counts.
"""

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


def _conf_case(seed, b=4, K=6, V=40, r=8, D=16):
    rng = np.random.default_rng(seed)
    base = (rng.standard_normal((b, K, V)) * 2.0).astype(np.float32)
    w1, w2 = _tables(rng, V, r)
    hidden = W.bf16_bits(rng.standard_normal((b, K, D), dtype=np.float32) * np.float32(2.0))
    anchors = rng.integers(0, V, b)
    return base, w1, w2, hidden, anchors


def _one_hot_w(n, j, value=1.0):
    w = np.zeros(n, np.float32)
    w[j] = value
    return W.bf16_bits(w)


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_confidence_of_one_hidden_feature(sign):
    """conf_w = +-e_d selects hidden feature d: conf_i = expit(+-h_i[d] + c),
    exactly (one exact product, zeros elsewhere), by scipy's logistic."""
    base, w1, w2, hidden, anchors = _conf_case(11)
    b, K, D = hidden.shape
    r = w1.shape[1]
    d0, c = 5, 0.375
    res = OM.block_decode(base, anchors, w1, w2, np.zeros(b), np.arange(b, dtype=np.uint64),
                          hidden=hidden, conf_w=_one_hot_w(D + r, d0, sign), conf_b=c)
    want = special.expit(sign * W.bf16_to_f32(hidden)[:, :, d0].astype(np.float64) + c)
    np.testing.assert_allclose(res["confidence"], want, rtol=1e-15, atol=0)


def test_confidence_of_one_markov_feature_is_the_previous_token():
    """conf_w = e_{D+j} selects Markov feature j, which belongs to the token
    BEFORE each position: W1[anchor] at position 0, W1[x_{i-1}] at position
    i.  The wrong shift (W1[x_i]) must disagree somewhere, so the pin has
    power."""
    base, w1, w2, hidden, anchors = _conf_case(12)
    b, K, D = hidden.shape
    r = w1.shape[1]
    j, c = 3, -0.5
    temps = np.array([0.0, 0.7, 1.0, 0.0])
    res = OM.block_decode(base, anchors, w1, w2, temps, np.arange(b, dtype=np.uint64) + np.uint64(5),
                          hidden=hidden, conf_w=_one_hot_w(D + r, D + j), conf_b=c)
    toks = res["tokens"]
    prev = np.concatenate([np.asarray(anchors)[:, None], toks[:, :-1]], axis=1)
    w1f = W.bf16_to_f32(w1).astype(np.float64)
    np.testing.assert_allclose(res["confidence"], special.expit(w1f[prev, j] + c), rtol=1e-15, atol=0)
    wrong = special.expit(w1f[toks, j] + c)
    assert not np.allclose(res["confidence"], wrong)


def test_confidence_without_weights_is_the_bias():
    base, w1, w2, hidden, anchors = _conf_case(13)
    b, K, D = hidden.shape
    r = w1.shape[1]
    res = OM.block_decode(base, anchors, w1, w2, np.zeros(b), np.arange(b, dtype=np.uint64),
                          hidden=hidden, conf_w=np.zeros(D + r, np.uint16), conf_b=1.25)
    assert (res["confidence"] == special.expit(1.25)).all()


def test_threshold_truncates_at_the_first_low_position():
    """Hidden feature d0 planted +8 before position k_s and -8 at it (random
    after): with conf_w = e_{d0}, no bias and threshold 0.5 the draft length
    is k_s; without a threshold it is K; a confidence exactly at the
    threshold (logit 0, conf 1/2) still counts (conf >= threshold)."""
    base, w1, w2, hidden, anchors = _conf_case(14)
    b, K, D = hidden.shape
    r = w1.shape[1]
    d0 = 2
    h = W.bf16_to_f32(hidden).copy()
    ks = np.array([0, 3, K - 1, K])
    for s in range(b):
        h[s, :ks[s], d0] = 8.0
        if ks[s] < K:
            h[s, ks[s], d0] = -8.0
    hb = W.bf16_bits(h)
    cw = _one_hot_w(D + r, d0)
    kw = dict(hidden=hb, conf_w=cw, conf_b=0.0)
    seeds = np.arange(b, dtype=np.uint64)
    res = OM.block_decode(base, anchors, w1, w2, np.zeros(b), seeds, threshold=0.5, **kw)
    assert res["lengths"].tolist() == ks.tolist()
    res0 = OM.block_decode(base, anchors, w1, w2, np.zeros(b), seeds, threshold=0.0, **kw)
    assert (res0["lengths"] == K).all()
    h[:, :, d0] = 0.0
    res_tie = OM.block_decode(base, anchors, w1, w2, np.zeros(b), seeds, threshold=0.5,
                              hidden=W.bf16_bits(h), conf_w=cw, conf_b=0.0)
    assert (res_tie["confidence"] == 0.5).all() and (res_tie["lengths"] == K).all()
