"""Helpers shared by the GPU parity tests: move a seeded workload to the GPU,
run the HIP path through the C ABI (via the Python binding), run the oracle
on the same bytes, and compare element by element.

Decisions are compared bit-exactly.  A disagreement is tolerated only when
the oracle itself sits within a near-tie band of that decision, and every
such case is counted and reported:

* accept test of slot i: |u_i - min(1, r_i)| < 1e-6 (r_i the oracle's ratio);
* drawn token (residual or bonus): the oracle's t lies within
  1e-6 * R + 2 E of a step of the oracle's CDF between the two answers (R
  the total mass, E the bound on the kernel's fp32 weight error below), and
  the GPU's token lies in the support of p_n.

E: the kernel takes each weight as exp2 of an exponent e = log2 p(v) that
carries its last two fp32 roundings, 2 * 2^-24 |e| absolute, and v_exp_f32's
own ulp, so |p_f(v) - p(v)| <= 2^-24 p(v) (2 ln2 |log2 p(v)| + 2) to first
order; summed over v this is 2^-24 (1.39 H2(p) + 2), H2 the entropy in bits.
With q's term and the rounding of p_f - q_f (2^-24 (p + q)),
E = 2^-24 (1.39 (H2(p_n) + H2(q_n)) + 6) + V 2^-124 (entries that underflow
fp32 altogether).  The GPU's CDF and its t = u' R_gpu then lie within E of
the oracle's.  Where R itself is below E the kernel cannot resolve the
residual: its masses may round to zero, and it then draws from p_n.

After a tolerated disagreement the rest of that sequence is not compared.
Probabilities p_i(x_i), q_i(x_i) must agree within 1e-5 relative.
"""
from __future__ import annotations

import json
import os
from dataclasses import dataclass, field

import numpy as np
import torch

import oracle
import workloads as W

ACCEPT_BAND = 1e-6
DRAW_BAND = 1e-6
PROB_RTOL = 1e-5


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def seeds_to_device(seeds: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(seeds, dtype=np.uint64).view(np.int64)).to(device)


@dataclass
class Report:
    sequences: int = 0
    greedy_sequences: int = 0
    sampling_sequences: int = 0
    exact_sequences: int = 0
    accept_slots_in_band: int = 0        # slots whose |u - min(1,r)| < band (reported, any outcome)
    accept_near_tie_mismatch: int = 0    # tolerated accept-decision disagreements
    draw_near_tie_mismatch: int = 0      # tolerated drawn-token disagreements
    draws: int = 0
    residual_draws: int = 0
    bonus_draws: int = 0
    max_prob_rel_err: float = 0.0
    failures: list = field(default_factory=list)

    def merge(self, o: "Report") -> "Report":
        for k, v in o.__dict__.items():
            if k == "failures":
                self.failures += v
            elif k == "max_prob_rel_err":
                self.max_prob_rel_err = max(self.max_prob_rel_err, v)
            else:
                setattr(self, k, getattr(self, k) + v)
        return self

    def save(self, name: str) -> None:
        out = os.environ.get("SPEC_PARITY_REPORT_DIR")
        if out:
            os.makedirs(out, exist_ok=True)
            with open(os.path.join(out, f"{name}.json"), "w") as f:
                json.dump(self.__dict__, f, indent=1, default=str)
        print(f"[parity {name}] {json.dumps({k: v for k, v in self.__dict__.items() if k != 'failures'})}",
              flush=True)


def compare_greedy(case: W.Case, n_g, tok_g, am_g, name: str) -> Report:
    n_o, tok_o, am_o = oracle.greedy_accept(case.target, case.draft_tokens)
    rep = Report(sequences=case.b, greedy_sequences=case.b)
    bad = np.nonzero((n_g != n_o) | (tok_g != tok_o).any(axis=1) | (am_g != am_o).any(axis=1))[0]
    rep.exact_sequences = case.b - len(bad)
    for s in bad[:10]:
        rep.failures.append(dict(case=name, seq=int(s), n_gpu=int(n_g[s]), n_oracle=int(n_o[s]),
                                 tok_gpu=tok_g[s].tolist(), tok_oracle=tok_o[s].tolist(),
                                 am_gpu=am_g[s].tolist(), am_oracle=am_o[s].tolist()))
    return rep


def _softmax64(row: np.ndarray, T: float) -> np.ndarray:
    z = W.as_f32(row).astype(np.float64)
    fin = z[np.isfinite(z)]
    if fin.size == 0:
        return np.zeros_like(z)
    w = np.exp((z - fin.max()) / T)
    return w / w.sum()


def _entropy_bits(p: np.ndarray) -> float:
    p = p[p > 0]
    return float(-(p * np.log2(p)).sum())


def draw_error_bound(case: W.Case, s: int, slot: int, T: float, residual: bool):
    """E of the module docstring for the draw at `slot` of sequence s, and p_n."""
    p = _softmax64(case.target[s, slot], T)
    H = _entropy_bits(p)
    if residual:
        H += _entropy_bits(_softmax64(case.draft[s, slot], T))
    return 2.0 ** -24 * (1.39 * H + 6.0) + case.V * 2.0 ** -124, p


def _draw_near_tie(case: W.Case, res: dict, s: int, slot: int, y_g: int, T: float) -> bool:
    if y_g < 0 or y_g >= case.V:
        return False
    residual = bool(res["residual"][s])
    F = oracle.draw_cdf(case.target, case.draft, T, s, slot, residual)
    t, R, y_o = res["t"][s], res["R"][s], res["tokens"][s, slot]
    E, p = draw_error_bound(case, s, slot, T, residual)
    if not p[y_g] > 0.0:
        return False
    if y_g > y_o:
        margin = F[y_g - 1] - t
    else:
        margin = t - F[y_g]
    return 0.0 <= margin <= DRAW_BAND * R + 2.0 * E


def compare_sample(case: W.Case, n_g, tok_g, p_g, q_g, name: str, res: dict = None,
                   temps=None, lens=None) -> Report:
    """Sampling sequences of `case` (all of them, or those with temps > 0);
    sequence s has lens[s] draft tokens (all K when lens is None)."""
    if res is None:
        res = oracle.sample_accept(case.target, case.draft, case.draft_tokens, case.T, case.seeds)
    if temps is None:
        temps = np.full(case.b, case.T)
    seqs = [s for s in range(case.b) if temps[s] != 0.0]
    n_o, tok_o = res["n_accepted"], res["tokens"]
    rep = Report(sequences=len(seqs), sampling_sequences=len(seqs))
    with np.errstate(invalid="ignore"):
        band = np.abs(res["u"] - np.minimum(1.0, res["r"])) < ACCEPT_BAND
    for s in seqs:
        K = case.K if lens is None else int(lens[s])
        # probabilities of every slot of the block; NaN past it
        if n_o[s] >= 0:
            if not (np.isnan(p_g[s, K:]).all() and np.isnan(q_g[s, K:]).all()):
                rep.failures.append(dict(case=name, seq=s, what="probabilities past the block"))
            for arr_g, arr_o in ((p_g, res["p_draft"]), (q_g, res["q_draft"])):
                g, o = arr_g[s, :K].astype(np.float64), arr_o[s, :K]
                ok = np.isclose(g, o, rtol=PROB_RTOL, atol=1e-37)
                rel = np.abs(g - o) / np.maximum(np.abs(o), 1e-300)
                rep.max_prob_rel_err = max(rep.max_prob_rel_err, float(rel[o > 1e-30].max(initial=0.0)))
                if not ok.all():
                    rep.failures.append(dict(case=name, seq=s, what="probability", gpu=g.tolist(),
                                             oracle=o.tolist()))
        else:
            if not (np.isnan(p_g[s]).all() and np.isnan(q_g[s]).all()):
                rep.failures.append(dict(case=name, seq=s, what="invalid sequence probabilities"))
        nb = int(band[s, :max(0, min(n_o[s], K - 1)) + 1].sum()) if n_o[s] >= 0 else 0
        rep.accept_slots_in_band += nb
        if n_o[s] >= 0:
            rep.draws += 1
            if n_o[s] < K:
                rep.residual_draws += 1
            else:
                rep.bonus_draws += 1
        if n_g[s] == n_o[s] and (tok_g[s] == tok_o[s]).all():
            rep.exact_sequences += 1
            continue
        if n_g[s] != n_o[s]:
            j = int(min(n_g[s], n_o[s]))
            if n_o[s] >= 0 and n_g[s] >= 0 and j < K and band[s, j] and \
                    (tok_g[s, :j] == tok_o[s, :j]).all():
                rep.accept_near_tie_mismatch += 1
                continue
            rep.failures.append(dict(case=name, seq=s, what="accepted length", n_gpu=int(n_g[s]),
                                     n_oracle=int(n_o[s]), u=res["u"][s].tolist(), r=res["r"][s].tolist()))
            continue
        n = int(n_o[s])
        if (tok_g[s, :n] == tok_o[s, :n]).all() and (tok_g[s, n + 1:] == -1).all() and \
                _draw_near_tie(case, res, s, n, int(tok_g[s, n]), float(temps[s])):
            rep.draw_near_tie_mismatch += 1
            continue
        rep.failures.append(dict(case=name, seq=s, what="tokens", n=n, tok_gpu=tok_g[s].tolist(),
                                 tok_oracle=tok_o[s].tolist(), t=float(res["t"][s]), R=float(res["R"][s])))
    return rep


def compare_mixed(case: W.Case, temps: np.ndarray, n_g, tok_g, p_g, q_g, am_g, name: str,
                  lens=None) -> Report:
    res = oracle.mixed_accept(case.target, case.draft, case.draft_tokens, temps, case.seeds, lens)
    rep = compare_sample(case, n_g, tok_g, p_g, q_g, name, res=res, temps=temps, lens=lens)
    greedy = np.nonzero(temps == 0.0)[0]
    rep.sequences += len(greedy)
    rep.greedy_sequences += len(greedy)
    for s in greedy:
        ok = (n_g[s] == res["n_accepted"][s] and (tok_g[s] == res["tokens"][s]).all()
              and (am_g[s] == res["argmax"][s]).all() and np.isnan(p_g[s]).all() and np.isnan(q_g[s]).all())
        if ok:
            rep.exact_sequences += 1
        else:
            rep.failures.append(dict(case=name, seq=int(s), what="greedy in mixed", n_gpu=int(n_g[s]),
                                     n_oracle=int(res["n_accepted"][s]), tok_gpu=tok_g[s].tolist(),
                                     tok_oracle=res["tokens"][s].tolist()))
    sampling = np.nonzero(temps != 0.0)[0]
    if not (am_g[sampling] == -1).all():
        rep.failures.append(dict(case=name, what="argmax of sampling sequences must be -1"))
    return rep


def run_gpu_mixed(case: W.Case, temps: np.ndarray, target_dev=None, draft_dev=None, lens=None,
                  draft_tokens=None):
    import lossless_draft_verification_amd as L
    t = to_device(case.target) if target_dev is None else target_dev
    d = to_device(case.draft) if draft_dev is None else draft_dev
    x = torch.from_numpy(case.draft_tokens if draft_tokens is None else draft_tokens).cuda()
    sd = seeds_to_device(case.seeds)
    T = torch.from_numpy(np.ascontiguousarray(temps, dtype=np.float64)).cuda()
    kl = None if lens is None else torch.from_numpy(np.ascontiguousarray(lens, dtype=np.int32)).cuda()
    r = L.mixed_accept(t, d, x, T, sd, draft_lengths=kl)
    torch.cuda.synchronize()
    return (r.n_accepted.cpu().numpy(), r.tokens.cpu().numpy(), r.p_draft.cpu().numpy(),
            r.q_draft.cpu().numpy(), r.argmax.cpu().numpy())


def run_gpu_greedy(case: W.Case, target_dev=None):
    import lossless_draft_verification_amd as L
    t = to_device(case.target) if target_dev is None else target_dev
    x = torch.from_numpy(case.draft_tokens).cuda()
    r = L.greedy_accept(t, x)
    torch.cuda.synchronize()
    return r.n_accepted.cpu().numpy(), r.tokens.cpu().numpy(), r.argmax.cpu().numpy()


def run_gpu_sample(case: W.Case, target_dev=None, draft_dev=None):
    import lossless_draft_verification_amd as L
    t = to_device(case.target) if target_dev is None else target_dev
    d = to_device(case.draft) if draft_dev is None else draft_dev
    x = torch.from_numpy(case.draft_tokens).cuda()
    sd = seeds_to_device(case.seeds)
    r = L.speculative_sample_accept(t, d, x, case.T, sd)
    torch.cuda.synchronize()
    return (r.n_accepted.cpu().numpy(), r.tokens.cpu().numpy(), r.p_draft.cpu().numpy(),
            r.q_draft.cpu().numpy())


# ------------------------------------------------------------- fused verify
#
# The fused path forms its float32 logits in its own summation order, so they
# differ from the oracle's (the float64 definition rounded once) by at most
# the float32 summation bound plus the softcap's evaluation error:
#     tol(v) = gamma_{D+1} * sum_d |h_d w_vd| + 4 * 2^-23 * c + 2^-23 * |z(v)|
# (gamma_n = n 2^-24 / (1 - n 2^-24); the last term is the rounding of the
# result).  A decision may then differ from the oracle's only where the
# oracle sits within that perturbation of the decision boundary:
#   argmax       z(v_gpu) + tol(v_gpu) >= z(v_oracle) - tol(v_oracle);
#   accept test  |u - min(1, r)| <= min(1, r) * expm1(delta) + 1e-6,
#                delta = (tol(x) + max_v tol(v)) / T;
#   drawn token  t within 2 * expm1(2 max_v tol(v) / T) + 1e-6 R of a CDF
#                step between the two answers.
# Probabilities p(x) must agree to expm1(delta) + 1e-5 relative, q(x) to 1e-5.


def fused_tolerance(hidden, weight, cap, z64, seqs, absp=None) -> np.ndarray:
    import oracle.fused as F
    D = hidden.shape[-1]
    if absp is None:
        absp = F.abs_products(hidden, weight, seqs)
    tol = F.gamma(D + 1) * absp
    tol += 4.0 * 2.0 ** -23 * cap + 2.0 ** -23 * np.abs(z64)
    return tol


def _cdf_near_tie(F, t, R, y_g, y_o, band_abs) -> bool:
    if y_g < 0 or y_g >= len(F):
        return False
    margin = (F[y_g - 1] - t) if y_g > y_o else (t - F[y_g])
    return margin <= band_abs + 1e-6 * R


def compare_fused(case, res_o: dict, tol: np.ndarray, n_g, tok_g, p_g, q_g, am_g, name: str,
                  lens=None) -> Report:
    """GPU fused results against the oracle's on the sequences the oracle
    formed (res_o['seqs']); tol[j] is fused_tolerance for seqs[j]."""
    seqs = list(res_o["seqs"])
    rep = Report()
    n_o, tok_o, am_o = res_o["n_accepted"], res_o["tokens"], res_o["argmax"]
    K = case.K
    for j, s in enumerate(seqs):
        T = float(case.temps[s])
        Ks = K if lens is None else int(lens[s])
        z, tl = res_o["logits64"][j], tol[j]
        rep.sequences += 1
        if n_o[s] < 0:
            if n_g[s] == -1 and (tok_g[s] == -1).all():
                rep.exact_sequences += 1
            else:
                rep.failures.append(dict(case=name, seq=s, what="invalid sequence", n_gpu=int(n_g[s])))
            continue
        if T == 0.0:
            rep.greedy_sequences += 1
            diff = np.nonzero(am_g[s, :Ks + 1] != am_o[s, :Ks + 1])[0]
            if len(diff) == 0:
                if n_g[s] == n_o[s] and (tok_g[s] == tok_o[s]).all() and (am_g[s] == am_o[s]).all():
                    rep.exact_sequences += 1
                else:
                    rep.failures.append(dict(case=name, seq=s, what="greedy tokens", n_gpu=int(n_g[s]),
                                             n_oracle=int(n_o[s])))
                continue
            i = int(diff[0])
            vg, vo = int(am_g[s, i]), int(am_o[s, i])
            ok = 0 <= vg < case.V and z[i, vg] + tl[i, vg] >= z[i, vo] - tl[i, vo]
            m = min(i, int(n_g[s]), int(n_o[s]))
            if ok and (tok_g[s, :m] == tok_o[s, :m]).all():
                rep.accept_near_tie_mismatch += 1
            else:
                rep.failures.append(dict(case=name, seq=s, what="greedy argmax", row=i, gpu=vg, oracle=vo,
                                         z_gpu_choice=float(z[i, vg]), z_max=float(z[i, vo])))
            continue
        rep.sampling_sequences += 1
        tmax = tl.max(axis=1)
        x = case.draft_tokens[s]
        ok_prob = True
        for i in range(Ks):
            d = (tl[i, x[i]] + tmax[i]) / T
            po, qo = res_o["p_draft"][s, i], res_o["q_draft"][s, i]
            if not abs(p_g[s, i] - po) <= po * (np.expm1(d) + 1e-5) + 1e-37:
                ok_prob = False
            if not abs(q_g[s, i] - qo) <= qo * PROB_RTOL + 1e-37:
                ok_prob = False
        if not ok_prob:
            rep.failures.append(dict(case=name, seq=s, what="probabilities", p_gpu=p_g[s].tolist(),
                                     p_oracle=res_o["p_draft"][s].tolist()))
            continue
        if n_g[s] != n_o[s]:
            i = int(min(n_g[s], n_o[s]))
            if 0 <= i < Ks:
                d = (tl[i, x[i]] + tmax[i]) / T
                u, r = res_o["u"][s, i], min(1.0, res_o["r"][s, i])
                if abs(u - r) <= r * np.expm1(d) + 1e-6 and (tok_g[s, :i] == tok_o[s, :i]).all():
                    rep.accept_near_tie_mismatch += 1
                    continue
            rep.failures.append(dict(case=name, seq=s, what="accepted length", n_gpu=int(n_g[s]),
                                     n_oracle=int(n_o[s])))
            continue
        n = int(n_o[s])
        rep.draws += 1
        if n < Ks:
            rep.residual_draws += 1
        else:
            rep.bonus_draws += 1
        if (tok_g[s] == tok_o[s]).all():
            rep.exact_sequences += 1
            continue
        if not ((tok_g[s, :n] == tok_o[s, :n]).all() and (tok_g[s, n + 1:] == -1).all()):
            rep.failures.append(dict(case=name, seq=s, what="tokens", tok_gpu=tok_g[s].tolist(),
                                     tok_oracle=tok_o[s].tolist()))
            continue
        resid = bool(res_o["residual"][s])
        t1 = np.ascontiguousarray(res_o["logits32"][j:j + 1])
        d1 = np.ascontiguousarray(case.draft[s:s + 1])
        F = oracle.draw_cdf(t1, d1, T, 0, n, resid)
        band = 2.0 * np.expm1(2.0 * tmax[n] / T)
        if _cdf_near_tie(F, res_o["t"][s], res_o["R"][s], int(tok_g[s, n]), int(tok_o[s, n]), band):
            rep.draw_near_tie_mismatch += 1
        else:
            rep.failures.append(dict(case=name, seq=s, what="drawn token", gpu=int(tok_g[s, n]),
                                     oracle=int(tok_o[s, n])))
    return rep
