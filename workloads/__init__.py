"""Seeded synthetic inputs for the verify/accept step.

This module only produces input bytes: target logit blocks [b, K+1, V], draft
logit blocks [b, K, V], draft tokens [b, K], per-sequence Philox seeds and the
per-sequence rule (greedy or sampling).  It holds none of the accept rule's
arithmetic and serves the tests, the benchmark and the oracle alike.

Draft tokens are produced the way a drafter would produce them: the argmax of
the stored draft row (greedy rows) or a draw from softmax(z_d / T) of the
stored draft row (sampling rows), the draw taken with the Gumbel-max trick
(argmax of z_d / T + Gumbel noise, Gumbel's 1954 extreme-value construction),
so no softmax is evaluated here.  All randomness is numpy PCG64.

Stored logits are bf16 (returned as their raw uint16 bit patterns, rounded to
nearest even from float32) or float32.

The five named workloads mirror the shapes of the pages' own settings: a
262144-entry vocabulary and a 7-token block (the Gemma-4 DSpark drafter
arguments, "dspark-mlx 0.1.0" wheel diff, dspark_mlx/arch/gemma4.py), and a
draft cap of 4 ("mlx-dspark 0.0.1" README, Tuning).  They stand in for the
pages' end-to-end decoding workloads (prompt suites that are not available
here): logits are synthetic, drawn as described per workload.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence, Tuple, Union

import numpy as np

GREEDY = 0
SAMPLING = 1


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); return uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    # process in slabs to bound temporaries
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 24
    for i in range(0, flat_u.size, step):
        s = flat_u[i:i + step]
        nan = (s & 0x7FFFFFFF) > 0x7F800000
        r = (s + (0x7FFF + ((s >> 16) & 1))) >> 16
        r = r.astype(np.uint16)
        r[nan] = ((s[nan] >> 16) | 0x0040).astype(np.uint16)  # keep NaN quiet
        flat_o[i:i + step] = r
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def as_f32(a: np.ndarray) -> np.ndarray:
    """Stored logits (float32 or bf16 bits) as float32 values."""
    return a if a.dtype == np.float32 else bf16_to_f32(a)


@dataclass
class Case:
    """One verify batch: every array is host memory (numpy)."""
    name: str
    dtype: str                      # "f32" or "bf16"
    b: int
    K: int
    V: int
    T: float
    target: np.ndarray              # [b, K+1, V] float32 or uint16 bf16 bits
    draft: np.ndarray               # [b, K, V]
    draft_tokens: np.ndarray        # [b, K] int32
    seeds: np.ndarray               # [b] uint64
    rule: np.ndarray                # [b] GREEDY / SAMPLING
    meta: dict = field(default_factory=dict)

    def rows(self, rule: int) -> np.ndarray:
        return np.nonzero(self.rule == rule)[0]

    def take(self, idx: Sequence[int]) -> "Case":
        idx = np.asarray(idx)
        return Case(self.name, self.dtype, len(idx), self.K, self.V, self.T,
                    np.ascontiguousarray(self.target[idx]),
                    np.ascontiguousarray(self.draft[idx]),
                    np.ascontiguousarray(self.draft_tokens[idx]),
                    np.ascontiguousarray(self.seeds[idx]),
                    np.ascontiguousarray(self.rule[idx]), dict(self.meta))

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


def _zipf_rows(rng: np.random.Generator, nrows: int, V: int, slope: float,
               jitter: float) -> np.ndarray:
    """Rows whose sorted log-probabilities fall as -slope*ln(rank), ranks in a
    random order per row, plus N(0, jitter^2)."""
    base = (-slope * np.log(np.arange(1, V + 1, dtype=np.float64))).astype(np.float32)
    out = np.empty((nrows, V), np.float32)
    for r in range(nrows):
        out[r] = base[rng.permutation(V)]
        out[r] += rng.standard_normal(V, dtype=np.float32) * np.float32(jitter)
    return out


def _gumbel_draw(rng: np.random.Generator, z: np.ndarray, T: float) -> int:
    """One draw from softmax(z / T) by the Gumbel-max trick."""
    u = rng.random(z.shape[-1], dtype=np.float64)
    with np.errstate(divide="ignore"):
        g = -np.log(-np.log(u))
    return int(np.argmax(z.astype(np.float64) / T + g))


def make_case(name: str, *, b: int, K: int, V: int, dtype: str = "bf16",
              target_kind: str = "normal", target_scale: float = 1.0,
              zipf_slope: float = 1.1, zipf_jitter: float = 0.3,
              draft_sigma: Union[float, Tuple[float, float]] = 0.5,
              rule: Union[int, Sequence[int]] = SAMPLING, T: float = 1.0,
              seed: int = 0, philox_seeds: Optional[Sequence[int]] = None,
              equal_draft_rows: Sequence[int] = (), spike_prob: float = 0.0,
              spike_height: float = 20.0, greedy_draft: str = "argmax") -> Case:
    """Generate one seeded batch.

    target_kind  "normal": iid N(0, target_scale^2); "zipf": see _zipf_rows.
    draft_sigma  scalar, or (lo, hi) for a per-sequence sigma ~ U[lo, hi];
                 draft = target (before rounding) + N(0, sigma^2).
    rule         per-sequence GREEDY / SAMPLING (scalar = all the same).
    equal_draft_rows  sequences whose draft block is bitwise the target's first K rows.
    spike_prob   each target row gets +spike_height on one uniform token with
                 this probability (at least one row when > 0); drafts are
                 derived from the rows before the spike.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if np.isscalar(rule):
        rules = np.full(b, int(rule), np.int32)
    else:
        rules = np.asarray(rule, np.int32)
        assert rules.shape == (b,)
    if isinstance(draft_sigma, tuple):
        sig = rng.uniform(draft_sigma[0], draft_sigma[1], size=b)
    else:
        sig = np.full(b, float(draft_sigma))

    tgt_bits = None
    tgt_f = np.empty((b, K + 1, V), np.float32)
    drf_f = np.empty((b, K, V), np.float32)
    for s in range(b):
        if target_kind == "normal":
            rows = rng.standard_normal((K + 1, V), dtype=np.float32) * np.float32(target_scale)
        elif target_kind == "zipf":
            rows = _zipf_rows(rng, K + 1, V, zipf_slope, zipf_jitter)
        else:
            raise ValueError(target_kind)
        tgt_f[s] = rows
        noise = rng.standard_normal((K, V), dtype=np.float32) * np.float32(sig[s])
        drf_f[s] = rows[:K] + noise

    spiked = []
    if spike_prob > 0.0:
        hits = rng.random(b * (K + 1)) < spike_prob
        if not hits.any():
            hits[rng.integers(b * (K + 1))] = True
        for flat in np.nonzero(hits)[0]:
            s, i = divmod(int(flat), K + 1)
            v = int(rng.integers(V))
            tgt_f[s, i, v] += np.float32(spike_height)
            spiked.append((s, i, v))

    if dtype == "bf16":
        target = bf16_bits(tgt_f)
        draft = bf16_bits(drf_f)
    elif dtype == "f32":
        target = tgt_f
        draft = drf_f
    else:
        raise ValueError(dtype)
    del tgt_f, drf_f
    for s in equal_draft_rows:
        draft[s] = target[s, :K]

    tokens = np.empty((b, K), np.int32)
    for s in range(b):
        for i in range(K):
            z = as_f32(draft[s, i])
            if rules[s] == GREEDY and greedy_draft == "argmax":
                tokens[s, i] = int(np.argmax(z))
            else:
                tokens[s, i] = _gumbel_draw(rng, z, T)

    if philox_seeds is None:
        seeds = np.arange(b, dtype=np.uint64)
    else:
        seeds = np.asarray(philox_seeds, dtype=np.uint64)
    meta = {"draft_sigma": sig, "spiked": spiked, "seed": seed,
            "target_kind": target_kind}
    return Case(name, dtype, b, K, V, float(T), target, draft, tokens, seeds, rules, meta)


# ---------------------------------------------------------------------------
# The five named workloads.  Data seed 1000 * id + 1.

CONFIG_TEXT = {
    1: "b=1 K=7 V=151936 fp32, target N(0,2^2), draft = target + N(0,0.5^2), "
       "tokens ~ draft softmax, T=1.0, Philox seed 0, greedy and sampling",
    2: "b=8 K=7 V=262144 bf16, Zipf target (-1.1 ln rank + N(0,0.3^2)), "
       "draft = target + N(0,0.8^2), tokens = draft argmax, greedy",
    3: "b=32 K=7 V=151936 bf16, target N(0,2.5^2), per-row draft sigma ~ U[0.2,1.5], "
       "sampling T=0.7, Philox seed per row",
    4: "b=64 K=4 V=129280 bf16, Zipf target, draft = target + N(0,0.5^2), rows 0..31 "
       "draft == target, sampling T=1.0",
    5: "b=128 K=7 V=262144 bf16, target N(0,3^2) with 1% of rows spiked +20, per-row "
       "draft sigma ~ U[0.1,2.0], rows 0..63 greedy / 64..127 sampling, T=0.8",
}


def config(cid: int, b: Optional[int] = None, V: Optional[int] = None) -> Case:
    """Workload `cid` (1..5).  `b` / `V` shrink it for quick runs (same recipe)."""
    seed = 1000 * cid + 1
    if cid == 1:
        bb, VV = b or 1, V or 151936
        # b=1: both rules run on the same sequence; rule marks the sampling call.
        return make_case("c1", b=bb, K=7, V=VV, dtype="f32", target_kind="normal",
                         target_scale=2.0, draft_sigma=0.5, rule=SAMPLING, T=1.0,
                         seed=seed, philox_seeds=[0] * bb)
    if cid == 2:
        bb, VV = b or 8, V or 262144
        return make_case("c2", b=bb, K=7, V=VV, dtype="bf16", target_kind="zipf",
                         draft_sigma=0.8, rule=GREEDY, T=1.0, seed=seed)
    if cid == 3:
        bb, VV = b or 32, V or 151936
        return make_case("c3", b=bb, K=7, V=VV, dtype="bf16", target_kind="normal",
                         target_scale=2.5, draft_sigma=(0.2, 1.5), rule=SAMPLING,
                         T=0.7, seed=seed)
    if cid == 4:
        bb, VV = b or 64, V or 129280
        return make_case("c4", b=bb, K=4, V=VV, dtype="bf16", target_kind="zipf",
                         draft_sigma=0.5, rule=SAMPLING, T=1.0, seed=seed,
                         equal_draft_rows=range(bb // 2))
    if cid == 5:
        bb, VV = b or 128, V or 262144
        rules = np.array([GREEDY] * (bb // 2) + [SAMPLING] * (bb - bb // 2), np.int32)
        return make_case("c5", b=bb, K=7, V=VV, dtype="bf16", target_kind="normal",
                         target_scale=3.0, draft_sigma=(0.1, 2.0), rule=rules, T=0.8,
                         seed=seed, spike_prob=0.01)
    raise ValueError(f"unknown workload {cid}")



def make_zero_mass_case(name: str, *, b: int, K: int, V: int, dtype: str = "bf16",
                        T: float = 0.9, seed: int = 0) -> Case:
    """A batch whose draws hit zero residual mass.  Every draft block is
    bitwise its target's first K rows, so every accept ratio is exactly 1;
    sequence s then masks (-inf, in the target and the draft row alike) its
    draft token at slot j_s = s mod (K+1) when j_s < K.  That slot has
    p(x) = 0 and is rejected, and max(0, p - q) is zero over the whole row, so
    the token is drawn from p_{j_s}; sequences with j_s = K accept every slot
    and draw the bonus.  meta["slot"] holds j_s."""
    case = make_case(name, b=b, K=K, V=V, dtype=dtype, target_scale=2.0, draft_sigma=0.5,
                     T=T, seed=seed, equal_draft_rows=range(b))
    ninf = np.uint16(0xFF80) if case.target.dtype == np.uint16 else np.float32(-np.inf)
    slot = np.arange(b) % (K + 1)
    for s in range(b):
        j = int(slot[s])
        if j < K:
            x = int(case.draft_tokens[s, j])
            case.target[s, j, x] = ninf
            case.draft[s, j, x] = ninf
    case.meta["slot"] = slot
    return case

# ---------------------------------------------------------------------------
# Fused verify inputs: the verify forward's final hidden states and the
# lm_head weight instead of a materialised target logit block.
#
# The lm_head is a bias-free Linear(hidden_size, vocab_size) followed by the
# final-logit softcap; hidden_size 3840, vocab_size 262144, softcap 30 are
# the Gemma-4 drafter arguments ("dspark-mlx 0.1.0" wheel diff,
# dspark_mlx/arch/gemma4.py).  The drafter's logits arrive in float32 (it
# applies its lm_head to float32 hidden states, same file).
#
# Recipe (no product of hidden and weight is formed here):
#   hidden      iid N(0, 1), bf16
#   weight      iid N(0, scale^2 / D), bf16, so background logits ~ N(0, scale^2)
#   planted     each target row (s, i) gets its own token t[s, i] (distinct
#               tokens); weight row t[s, i] is set to bf16(g / D * hidden[s, i])
#               with a gain g ~ U[gain_lo, gain_hi], so that row's logit at
#               t[s, i] is about g and elsewhere about N(0, scale^2)
#   draft       float32 [b, K, V]: iid N(0, draft_scale^2) plus, at t[s, i],
#               0.9 g + N(0, 1) (a drafter that mostly agrees)
#   tokens      greedy sequences: t[s, i] with probability agree, else another
#               uniform token; sampling sequences: a draw from softmax(draft / T)
#               (Gumbel-max)
#   temps       0 for greedy sequences, T for sampling sequences


@dataclass
class FusedCase:
    name: str
    b: int
    K: int
    V: int
    D: int
    softcap: float
    T: float
    hidden: np.ndarray              # [b, K+1, D] uint16 bf16 bits
    weight: np.ndarray              # [V, D] uint16 bf16 bits
    draft: np.ndarray               # [b, K, V] float32
    draft_tokens: np.ndarray        # [b, K] int32
    seeds: np.ndarray               # [b] uint64
    temps: np.ndarray               # [b] float64 (0 = greedy)
    planted: np.ndarray             # [b, K+1] int32
    meta: dict = field(default_factory=dict)


def make_fused_case(name: str, *, b: int, K: int, V: int, D: int, softcap: float = 30.0,
                    scale: float = 3.0, gain: Tuple[float, float] = (10.0, 24.0),
                    draft_scale: float = 3.0, agree: float = 0.85,
                    rule: Union[int, Sequence[int]] = SAMPLING, T: float = 0.8,
                    seed: int = 0) -> FusedCase:
    if V < b * (K + 1):
        raise ValueError("need V >= b*(K+1) for distinct planted tokens")
    rng = np.random.Generator(np.random.PCG64(seed))
    rules = np.full(b, int(rule), np.int32) if np.isscalar(rule) else np.asarray(rule, np.int32)
    assert rules.shape == (b,)
    hidden = bf16_bits(rng.standard_normal((b, K + 1, D), dtype=np.float32))
    weight = np.empty((V, D), np.uint16)
    wscale = np.float32(scale / np.sqrt(D))
    slab = max(1, (1 << 24) // D)
    for v0 in range(0, V, slab):
        v1 = min(V, v0 + slab)
        weight[v0:v1] = bf16_bits(rng.standard_normal((v1 - v0, D), dtype=np.float32) * wscale)
    planted = rng.choice(V, size=b * (K + 1), replace=False).astype(np.int32).reshape(b, K + 1)
    g = rng.uniform(gain[0], gain[1], size=(b, K + 1))
    hf = bf16_to_f32(hidden)
    for s in range(b):
        for i in range(K + 1):
            weight[planted[s, i]] = bf16_bits(hf[s, i] * np.float32(g[s, i] / D))
    draft = np.empty((b, K, V), np.float32)
    for s in range(b):
        draft[s] = rng.standard_normal((K, V), dtype=np.float32) * np.float32(draft_scale)
        for i in range(K):
            draft[s, i, planted[s, i]] = np.float32(0.9 * g[s, i] + rng.standard_normal())
    tokens = np.empty((b, K), np.int32)
    for s in range(b):
        for i in range(K):
            if rules[s] == GREEDY:
                if rng.random() < agree:
                    tokens[s, i] = planted[s, i]
                else:
                    tokens[s, i] = (planted[s, i] + 1 + int(rng.integers(V - 1))) % V
            else:
                tokens[s, i] = _gumbel_draw(rng, draft[s, i], T)
    temps = np.where(rules == GREEDY, 0.0, float(T))
    meta = {"seed": seed, "gain": g, "scale": scale}
    return FusedCase(name, b, K, V, D, float(softcap), float(T), hidden, weight, draft, tokens,
                     np.arange(b, dtype=np.uint64), temps, planted, meta)


FUSED_TEXT = ("b=128 K=7 V=262144 D=3840: bf16 hidden states [b, K+1, D] N(0,1) and bf16 lm_head "
              "weight [V, D] N(0, 3^2/D) with one planted token per target row (gain ~ U[10,24]), "
              "final-logit softcap 30, fp32 drafter logits, rows 0..63 greedy / 64..127 sampling "
              "T=0.8")


def fused_config(b: int = 128, K: int = 7, V: int = 262144, D: int = 3840) -> FusedCase:
    """The fused verify workload at the 262144-entry Gemma-4 vocabulary (data
    seed 6001); smaller b / V / D keep the recipe."""
    rules = np.array([GREEDY] * (b // 2) + [SAMPLING] * (b - b // 2), np.int32)
    return make_fused_case("fused", b=b, K=K, V=V, D=D, softcap=30.0, rule=rules, T=0.8, seed=6001)


# ---------------------------------------------------------------------------
# Draft-side block decode inputs: the parallel backbone's base logits, the
# rank-r Markov head tables and the confidence head (rank 256, the Gemma-4
# drafter's markov_rank, "dspark-mlx 0.1.0" wheel diff, arch/gemma4.py).
#
#   base     float32 [b, K, V] iid N(0, scale^2)
#   w1       bf16 [V, r] iid N(0, 1)                 (previous-token features)
#   w2       bf16 [V, r] iid N(0, (gain / sqrt r)^2) (the table, row v = entry v)
#   hidden   bf16 [b, K, D] iid N(0, 1), conf_w bf16 [D + r] iid N(0, 1/(D + r)),
#            conf_b = 1.0
#   anchors  uniform tokens; temps 0 (greedy) or T per sequence; seeds = index


@dataclass
class MarkovCase:
    name: str
    b: int
    K: int
    V: int
    r: int
    D: int
    base: np.ndarray
    anchors: np.ndarray
    w1: np.ndarray
    w2: np.ndarray
    hidden: np.ndarray
    conf_w: np.ndarray
    conf_b: float
    temps: np.ndarray
    seeds: np.ndarray
    meta: dict = field(default_factory=dict)


def make_markov_case(name: str, *, b: int, K: int, V: int, r: int = 256, D: int = 64,
                     scale: float = 3.0, gain: float = 3.0, rule: Union[int, Sequence[int]] = SAMPLING,
                     T: float = 0.8, seed: int = 0) -> MarkovCase:
    rng = np.random.Generator(np.random.PCG64(seed))
    rules = np.full(b, int(rule), np.int32) if np.isscalar(rule) else np.asarray(rule, np.int32)
    base = np.empty((b, K, V), np.float32)
    for s in range(b):
        base[s] = rng.standard_normal((K, V), dtype=np.float32) * np.float32(scale)
    w1 = np.empty((V, r), np.uint16)
    w2 = np.empty((V, r), np.uint16)
    slab = max(1, (1 << 24) // r)
    for v0 in range(0, V, slab):
        v1 = min(V, v0 + slab)
        w1[v0:v1] = bf16_bits(rng.standard_normal((v1 - v0, r), dtype=np.float32))
        w2[v0:v1] = bf16_bits(rng.standard_normal((v1 - v0, r), dtype=np.float32) * np.float32(gain / np.sqrt(r)))
    hidden = bf16_bits(rng.standard_normal((b, K, D), dtype=np.float32))
    conf_w = bf16_bits(rng.standard_normal(D + r, dtype=np.float32) * np.float32(1.0 / np.sqrt(D + r)))
    anchors = rng.integers(0, V, b).astype(np.int32)
    temps = np.where(rules == GREEDY, 0.0, float(T))
    return MarkovCase(name, b, K, V, r, D, base, anchors, w1, w2, hidden, conf_w, 1.0, temps,
                      np.arange(b, dtype=np.uint64), {"seed": seed})


MARKOV_TEXT = ("b=128 K=7 V=262144 r=256 D=3840: float32 base logits N(0,3^2), bf16 Markov tables "
               "W1 [V,r] N(0,1) and W2 [V,r] N(0,(3/16)^2), confidence head on [hidden; u], "
               "rows 0..63 greedy / 64..127 sampled at T=0.8")


def markov_config(b: int = 128, K: int = 7, V: int = 262144, r: int = 256, D: int = 3840) -> MarkovCase:
    rules = np.array([GREEDY] * (b // 2) + [SAMPLING] * (b - b // 2), np.int32)
    return make_markov_case("markov", b=b, K=K, V=V, r=r, D=D, rule=rules, T=0.8, seed=7001)
