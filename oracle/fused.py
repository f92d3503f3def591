"""Oracle of the fused verify (test infrastructure only).

The fused verify takes the verify forward's final hidden states and the
lm_head weight instead of a materialised target logit block.  What it
computes is fixed by the Gemma-4 drafter code of "dspark-mlx 0.1.0" (wheel
diff, dspark_mlx/arch/gemma4.py): the lm_head is a bias-free
Linear(hidden_size, vocab_size) with weight [V, D], applied to hidden states
cast to float32, and the final-logit softcap maps a logit a to
c * tanh(a / c) when c is set (30 for Gemma-4).  The logits the accept policy
consumes are therefore float32 values of

    z[s, i, v] = softcap( sum_d hidden[s, i, d] * weight[v, d] ).

This oracle forms that definition in float64 (numpy matmul as the only
library step; bf16 inputs widen exactly, their products are exact in
float64), applies the softcap in float64, and rounds once to float32: the
float32 logits closest to the definition.  The accept step that follows is
the C oracle's mixed accept (spec_oracle.c) on those logits, unchanged.

An accelerator computes the same sum in float32 in its own order.  Any
ordering of D exactly-formed products accumulated in float32 differs from the
exact sum by at most gamma_D * sum_d |hidden * weight| with
gamma_D = D u / (1 - D u), u = 2^-24 (the standard floating-point summation
bound); abs_products() provides that sum of magnitudes for the tests'
tolerance.

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
module; the product path never does.
"""
from __future__ import annotations

import numpy as np

from . import mixed_accept as _mixed_accept

U32 = 2.0 ** -24
_SLAB = 8192          # vocabulary rows per float64 slab (bounds host memory)


def _widen(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) or float32 -> float64, exactly."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if a.dtype == np.float32:
        return a.astype(np.float64)
    raise TypeError(a.dtype)


def softcap(a: np.ndarray, c: float) -> np.ndarray:
    """The final-logit softcap c * tanh(a / c); identity when c <= 0."""
    if c and c > 0.0:
        return c * np.tanh(a / c)
    return a


def lm_head_logits(hidden: np.ndarray, weight: np.ndarray, cap: float, seqs=None) -> np.ndarray:
    """float64 logits softcap(hidden @ weight.T) for hidden [b, K+1, D] and
    weight [V, D]; only the sequences in `seqs` (all when None), returned in
    that order as [len(seqs), K+1, V]."""
    b, K1, D = hidden.shape
    V = weight.shape[0]
    idx = np.arange(b) if seqs is None else np.asarray(seqs)
    H = _widen(np.ascontiguousarray(hidden[idx])).reshape(-1, D)
    out = np.empty((H.shape[0], V), np.float64)
    for v0 in range(0, V, _SLAB):
        v1 = min(V, v0 + _SLAB)
        out[:, v0:v1] = H @ _widen(weight[v0:v1]).T
    return softcap(out, cap).reshape(len(idx), K1, V)


def abs_products(hidden: np.ndarray, weight: np.ndarray, seqs=None) -> np.ndarray:
    """sum_d |hidden[s, i, d] * weight[v, d]| in float64, shaped like
    lm_head_logits (no softcap: the softcap is 1-Lipschitz)."""
    b, K1, D = hidden.shape
    V = weight.shape[0]
    idx = np.arange(b) if seqs is None else np.asarray(seqs)
    H = np.abs(_widen(np.ascontiguousarray(hidden[idx])).reshape(-1, D))
    out = np.empty((H.shape[0], V), np.float64)
    for v0 in range(0, V, _SLAB):
        v1 = min(V, v0 + _SLAB)
        out[:, v0:v1] = H @ np.abs(_widen(weight[v0:v1])).T
    return out.reshape(len(idx), K1, V)


def lm_head_logits_and_abs(hidden: np.ndarray, weight: np.ndarray, cap: float, seqs=None):
    """lm_head_logits and abs_products in one pass over the weight (each
    slab widened once): the same two float64 arrays."""
    b, K1, D = hidden.shape
    V = weight.shape[0]
    idx = np.arange(b) if seqs is None else np.asarray(seqs)
    H = _widen(np.ascontiguousarray(hidden[idx])).reshape(-1, D)
    Ha = np.abs(H)
    out = np.empty((H.shape[0], V), np.float64)
    absout = np.empty((H.shape[0], V), np.float64)
    for v0 in range(0, V, _SLAB):
        v1 = min(V, v0 + _SLAB)
        Wt = _widen(weight[v0:v1]).T
        out[:, v0:v1] = H @ Wt
        np.abs(Wt, out=Wt)
        absout[:, v0:v1] = Ha @ Wt
    return softcap(out, cap).reshape(len(idx), K1, V), absout.reshape(len(idx), K1, V)


def gamma(n: int) -> float:
    """gamma_n = n u / (1 - n u) for float32 (u = 2^-24)."""
    return n * U32 / (1.0 - n * U32)


def fused_mixed_accept(hidden, weight, cap, draft, draft_tokens, temperatures, seeds,
                       draft_lengths=None, seqs=None, with_abs: bool = False) -> dict:
    """Mixed-rule accept on the lm_head logits rounded to float32.

    With `seqs`, only those sequences' logits are formed; the other target
    rows are left at zero and their results are meaningless (the accept of a
    sequence reads only its own rows, and Philox rows stay the batch
    indices).  Returns the C oracle's result dict plus 'logits64' and
    'logits32' of the formed sequences ([len(seqs), K+1, V]), and with
    `with_abs` also 'abs_products' (abs_products of the same sequences)."""
    b, K1, D = hidden.shape
    V = weight.shape[0]
    idx = np.arange(b) if seqs is None else np.asarray(seqs)
    if with_abs:
        z64, absp = lm_head_logits_and_abs(hidden, weight, cap, idx)
    else:
        z64, absp = lm_head_logits(hidden, weight, cap, idx), None
    z32 = z64.astype(np.float32)
    target = np.zeros((b, K1, V), np.float32)
    target[idx] = z32
    res = _mixed_accept(target, np.ascontiguousarray(draft, dtype=np.float32), draft_tokens,
                        temperatures, seeds, draft_lengths)
    res["logits64"] = z64
    res["logits32"] = z32
    if absp is not None:
        res["abs_products"] = absp
    res["seqs"] = idx
    return res
