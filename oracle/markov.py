"""Oracle of the draft-side block decode with the Markov head (test
infrastructure only).

What the pages fix ("dspark-mlx 0.1.0" wheel diff, dspark_mlx/arch/gemma4.py
and the README "How it works"; "mlx-dspark 0.0.1" sdist diff, __init__.py;
the ds4 DSpark drafter model card, "What's in the file" and "Files"): the
parallel backbone proposes base logits for all K positions at once (its
lm_head on float32 hidden states, then the softcap); a rank-r Markov head
(r = 256, tensors markov_w1 and the markov_w2 table) adds a low-rank
correction conditioned on the previous token, which is why the block is
then sampled one position after another; a confidence head with bias on
[hidden_size + markov_rank] features scores each position, and a threshold
on it truncates the block.

Readings (the listing of draft_block_decode is not on the pages):
  u_i      = W1[x_{i-1}]                       rank-r feature, x_{-1} = the anchor
  q_i      = L_i + W2 u_i                      corrected draft logits (float32)
  x_i      = argmax q_i (T = 0, lowest index)  or a draw from softmax(q_i / T)
             by inverse CDF over ascending index at t = U * R, U the Philox
             uniform at (position i, batch row s, tag 2)
  conf_i   = sigmoid(w . [h_i ; u_i] + c)
  length   = leading positions with conf_i >= threshold (all K without one)
with W1 [V, r] (one row per previous token), W2 stored as [V, r] (row v
holds the table's column for vocabulary entry v), L [b, K, V] float32.

The correction is formed in float64 from the exactly widened bf16 tables
(numpy matmul as the library step) and the corrected logits are rounded once
to float32, the drafter's logit precision; the draw reuses the C oracle's
Philox and CDF.
"""
from __future__ import annotations

import numpy as np

from . import default as _default

TAG_DRAFT = 2


def _widen(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def markov_correction(w1: np.ndarray, w2: np.ndarray, prev_tokens: np.ndarray) -> np.ndarray:
    """W2 u for u = W1[prev] of each previous token: float64 [n, V]."""
    U = _widen(w1[np.asarray(prev_tokens)])          # [n, r]
    return U @ _widen(w2).T


def draw_index(z32: np.ndarray, T: float, u: float) -> int:
    """Inverse-CDF draw from softmax(z / T) at t = u * R (first index whose
    running sum exceeds t; the last index of positive weight if rounding
    leaves none)."""
    orc = _default()
    row = np.ascontiguousarray(z32, dtype=np.float32)[None, None, :]
    F = orc.draw_cdf(row, np.zeros((1, 0, row.shape[-1]), np.float32), T, 0, 0, False)
    t = u * F[-1]
    y = int(np.searchsorted(F, t, side="right"))
    if y >= len(F):
        pos = np.nonzero(np.diff(np.concatenate([[0.0], F])) > 0.0)[0]
        y = int(pos[-1]) if len(pos) else len(F) - 1
    return y


def block_decode(base: np.ndarray, anchors: np.ndarray, w1: np.ndarray, w2: np.ndarray,
                 temperatures: np.ndarray, seeds: np.ndarray, hidden=None, conf_w=None,
                 conf_b: float = 0.0, threshold: float = 0.0) -> dict:
    """Sequential block decode of b sequences.  Returns tokens [b, K] int32,
    logits [b, K, V] float32 (the corrected q_i), logits64, confidence
    [b, K] (when hidden and conf_w are given) and lengths [b]."""
    orc = _default()
    b, K, V = base.shape
    tokens = np.zeros((b, K), np.int32)
    q32 = np.zeros((b, K, V), np.float32)
    q64 = np.zeros((b, K, V), np.float64)
    conf = np.full((b, K), np.nan)
    feats = np.zeros((b, K, w1.shape[1]), np.float64)
    prev = np.asarray(anchors, np.int64).copy()
    for i in range(K):
        corr = markov_correction(w1, w2, prev)
        feats[:, i] = _widen(w1[prev])
        for s in range(b):
            z = base[s, i].astype(np.float64) + corr[s]
            q64[s, i] = z
            q32[s, i] = z.astype(np.float32)
            T = float(temperatures[s])
            if T == 0.0:
                tokens[s, i] = int(np.argmax(q32[s, i]))
            else:
                tokens[s, i] = draw_index(q32[s, i], T, orc.uniform(int(seeds[s]), s, i, TAG_DRAFT))
        prev = tokens[:, i].astype(np.int64)
    lengths = np.full(b, K, np.int32)
    if hidden is not None and conf_w is not None:
        x = np.concatenate([_widen(hidden), feats], axis=-1)        # [b, K, D + r]
        logit = x @ _widen(conf_w) + float(conf_b)
        conf = 1.0 / (1.0 + np.exp(-logit))
        if threshold > 0.0:
            for s in range(b):
                k = 0
                while k < K and conf[s, k] >= threshold:
                    k += 1
                lengths[s] = k
    return {"tokens": tokens, "logits": q32, "logits64": q64, "confidence": conf, "lengths": lengths,
            "features": feats}
