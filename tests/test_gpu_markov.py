"""GPU parity of the draft-side Markov block decode against the oracle.

The corrected logits q_i = L_i + W2 W1[x_{i-1}] are formed on the matrix
cores in float32 (bf16 products exact, sums in any order), so they differ
from the oracle's float64 definition by at most
    tol(v) = gamma_{r} * sum_j |W1[x_{i-1}, j] W2[v, j]| + 2^-23 * |q(v)|
(the float32 summation bound, plus the rounding of the sum and of adding
the base logit).  Positions are compared in order; tokens must be equal,
except where the oracle sits within that perturbation of its decision (an
argmax within tol of the runner-up, or a draw within the perturbed CDF's
reach), which is counted and ends the comparison of that sequence (the
next positions condition on a different token).  Confidences agree to
1e-6 and the draft lengths exactly, except at a confidence within 1e-6 of
the threshold.
"""
import numpy as np
import pytest
import torch

import oracle
import oracle.markov as OM
import workloads as W
from parity import Report, seeds_to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    import lossless_draft_verification_amd  # noqa: F401


def _bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _run(case: W.MarkovCase, threshold: float, anchors=None, temps=None):
    import lossless_draft_verification_amd as L
    anchors = case.anchors if anchors is None else anchors
    temps = case.temps if temps is None else temps
    r = L.markov_block_decode(torch.from_numpy(case.base).cuda(), torch.from_numpy(anchors).cuda(),
                              _bf16_dev(case.w1), _bf16_dev(case.w2),
                              torch.from_numpy(np.ascontiguousarray(temps, np.float64)).cuda(),
                              seeds_to_device(case.seeds), hidden=_bf16_dev(case.hidden),
                              conf_w=_bf16_dev(case.conf_w), conf_b=case.conf_b, threshold=threshold)
    torch.cuda.synchronize()
    return (r.tokens.cpu().numpy(), r.logits.cpu().numpy(), r.confidence.cpu().numpy(),
            r.lengths.cpu().numpy())


def _compare(case: W.MarkovCase, gpu, res, threshold, name) -> Report:
    tok_g, q_g, conf_g, len_g = gpu
    tok_o, q_o = res["tokens"], res["logits64"]
    w1f = W.bf16_to_f32(case.w1).astype(np.float64)
    w2a = np.abs(W.bf16_to_f32(case.w2).astype(np.float64))
    g_r = OM_gamma(case.r)
    rep = Report()
    max_ratio = 0.0
    for s in range(case.b):
        rep.sequences += 1
        T = float(case.temps[s])
        if T == 0.0:
            rep.greedy_sequences += 1
        else:
            rep.sampling_sequences += 1
        diverged = False
        for i in range(case.K):
            prev = case.anchors[s] if i == 0 else tok_o[s, i - 1]
            # non-finite oracle entries (a base logit masked with -inf) must be
            # matched exactly; the bound applies to the finite ones
            fin = np.isfinite(q_o[s, i])
            tol = np.where(fin, g_r * (np.abs(w1f[prev]) @ w2a.T) + 2.0 ** -23 * np.abs(np.where(fin, q_o[s, i], 0.0)),
                           0.0)
            err = np.where(fin, np.abs(q_g[s, i].astype(np.float64) - np.where(fin, q_o[s, i], 0.0)), 0.0)
            max_ratio = max(max_ratio, float((err / np.where(fin, tol, 1.0)).max()))
            if not ((err <= tol).all() and (q_g[s, i][~fin] == q_o[s, i][~fin]).all()):
                rep.failures.append(dict(case=name, seq=s, pos=i, what="corrected logits",
                                         worst=float((err / np.where(fin, tol, 1.0)).max())))
                diverged = True
                break
            if abs(conf_g[s, i] - res["confidence"][s, i]) > 1e-6:
                rep.failures.append(dict(case=name, seq=s, pos=i, what="confidence",
                                         gpu=float(conf_g[s, i]), oracle=float(res["confidence"][s, i])))
            if tok_g[s, i] == tok_o[s, i]:
                continue
            yg, yo = int(tok_g[s, i]), int(tok_o[s, i])
            z = q_o[s, i]
            if T == 0.0:
                ok = 0 <= yg < case.V and z[yg] + tol[yg] >= z[yo] - tol[yo]
            else:
                zz = np.ascontiguousarray(res["logits"][s, i])[None, None, :]
                F = oracle.draw_cdf(zz, np.zeros((1, 0, case.V), np.float32), T, 0, 0, False)
                u = oracle.uniform(int(case.seeds[s]), s, i, OM.TAG_DRAFT)
                t = u * F[-1]
                band = 2.0 * np.expm1(2.0 * tol.max() / T) * F[-1] + 1e-6 * F[-1]
                margin = (F[yg - 1] - t) if yg > yo else (t - F[yg])
                ok = 0 <= yg < case.V and margin <= band
            if ok:
                rep.draw_near_tie_mismatch += 1
            else:
                rep.failures.append(dict(case=name, seq=s, pos=i, what="token", gpu=yg, oracle=yo))
            diverged = True
            break
        if not diverged:
            rep.exact_sequences += 1
            if threshold > 0.0 and len_g[s] != res["lengths"][s]:
                k = int(min(len_g[s], res["lengths"][s]))
                if not abs(res["confidence"][s, k] - threshold) < 1e-6:
                    rep.failures.append(dict(case=name, seq=s, what="length", gpu=int(len_g[s]),
                                             oracle=int(res["lengths"][s])))
    rep.max_prob_rel_err = max_ratio      # here: the largest logit error as a fraction of its bound
    return rep


def OM_gamma(n: int) -> float:
    u = 2.0 ** -24
    return (n + 1) * u / (1.0 - (n + 1) * u)


def _check(rep: Report, name: str, max_near_tie_frac: float = 0.02):
    rep.save(name)
    assert not rep.failures, rep.failures[:3]
    ties = rep.accept_near_tie_mismatch + rep.draw_near_tie_mismatch
    assert ties <= max(1, max_near_tie_frac * max(rep.sequences, 1)), rep


MARKOV_CASES = [
    # name, b, K, V, r, D, threshold
    ("small_ragged_vocab", 12, 5, 5000, 64, 32, 0.5),
    ("rank256", 40, 7, 20012, 256, 128, 0.6),
    ("rank256_odd_vocab_tiled_kernel", 40, 7, 20011, 256, 128, 0.6),
    ("two_row_tiles", 300, 3, 3000, 128, 16, 0.0),
    ("rank320", 20, 4, 3001, 320, 16, 0.5),
    ("rank192_two_seq_tiles", 130, 3, 4099, 192, 16, 0.5),
    ("rank384_tiled_kernel", 16, 3, 2500, 384, 16, 0.5),
    ("vocab4", 3, 2, 4, 64, 8, 0.5),
    ("one_tile_and_a_bit", 5, 3, 132, 128, 8, 0.5),
    ("single_sequence", 1, 7, 4096, 256, 16, 0.5),
    ("vocab_over_1M_segments_in_memory", 2, 2, 1100000, 64, 8, 0.5),
    ("three_seq_tiles_many_vocab_tiles", 300, 2, 100000, 64, 8, 0.5),
]


@pytest.mark.parametrize("spec", MARKOV_CASES, ids=[c[0] for c in MARKOV_CASES])
def test_markov_block_decode(spec):
    name, b, K, V, r, D, thr = spec
    rule = np.array([W.GREEDY, W.SAMPLING] * (b // 2) + [W.SAMPLING] * (b % 2))
    case = W.make_markov_case(name, b=b, K=K, V=V, r=r, D=D, rule=rule, T=0.8, seed=61 + b)
    gpu = _run(case, thr)
    res = OM.block_decode(case.base, case.anchors, case.w1, case.w2, case.temps, case.seeds, hidden=case.hidden,
                          conf_w=case.conf_w, conf_b=case.conf_b, threshold=thr)
    _check(_compare(case, gpu, res, thr, f"markov_{name}"), f"markov_{name}")


def test_markov_extreme_temperatures_and_masked_vocab():
    """Temperatures from 0.02 to 50 next to greedy rows on the streaming
    correction kernel (r = 256), and sequences 5..9 with base logits masked
    to -inf on columns 1000..8999 (q = -inf there): no draw or argmax may
    land in the mask."""
    import dataclasses
    case = W.make_markov_case("mext", b=10, K=5, V=20012, r=256, D=32, rule=W.SAMPLING, T=1.0, seed=71)
    temps = np.array([0.0, 0.02, 0.05, 20.0, 50.0, 0.0, 0.02, 0.7, 20.0, 1.0])
    base = case.base.copy()
    base[5:, :, 1000:9000] = -np.inf
    case = dataclasses.replace(case, base=base, temps=temps)
    gpu = _run(case, 0.5)
    tok = gpu[0][5:]
    assert (tok >= 0).all() and not ((tok >= 1000) & (tok < 9000)).any()
    res = OM.block_decode(case.base, case.anchors, case.w1, case.w2, case.temps, case.seeds, hidden=case.hidden,
                          conf_w=case.conf_w, conf_b=case.conf_b, threshold=0.5)
    _check(_compare(case, gpu, res, 0.5, "markov_extreme_masked"), "markov_extreme_masked")


def test_markov_invalid_inputs():
    """An invalid temperature or anchor gives -1 tokens for that sequence only."""
    case = W.make_markov_case("bad", b=6, K=3, V=2000, r=64, D=8, rule=W.GREEDY, seed=66)
    temps = case.temps.copy()
    temps[1] = -1.0
    anchors = case.anchors.copy()
    anchors[3] = case.V + 5
    tok = _run(case, 0.0, anchors=anchors, temps=temps)[0]
    assert (tok[1] == -1).all() and (tok[3] == -1).all()
    ok = [0, 2, 4, 5]
    res = OM.block_decode(case.base[ok], anchors[ok], case.w1, case.w2, temps[ok], case.seeds[ok])
    assert (tok[ok] == res["tokens"]).all()


def test_markov_full_size():
    """b=128, K=7, V=262144, r=256, D=3840; rows 0..63 greedy, 64..127 sampled."""
    case = W.markov_config()
    gpu = _run(case, 0.6)
    res = OM.block_decode(case.base, case.anchors, case.w1, case.w2, case.temps, case.seeds, hidden=case.hidden,
                          conf_w=case.conf_w, conf_b=case.conf_b, threshold=0.6)
    _check(_compare(case, gpu, res, 0.6, "markov_full"), "markov_full")


def test_markov_deterministic_repeat():
    """Two calls on the same inputs give the same tokens, logits, confidences
    and lengths, bit for bit."""
    case = W.make_markov_case("mdet", b=40, K=5, V=9000, r=128, D=32,
                              rule=np.array([W.GREEDY, W.SAMPLING] * 20), T=0.9, seed=67)
    a, c = _run(case, 0.5), _run(case, 0.5)
    for x, y in zip(a, c):
        np.testing.assert_array_equal(x, y)


def _markov_sweep_case(k: int):
    """Seeded random b, K, V, rank (both correction kernels), per-sequence
    rule and temperature, and confidence threshold.  (Invalid inputs are
    covered by test_markov_invalid_inputs: the oracle numbers the Philox rows
    by position in the batch it is given, so the sweep keeps every row.)"""
    rng = np.random.default_rng(7000 + k)
    b = int(rng.integers(1, 150))
    K = int(rng.integers(1, 8))
    if k % 2 == 0:                       # the streaming kernel: rank <= 256, 16-byte aligned base rows
        V = int(rng.choice([4, 64, 1000, 4096, 9000, 20012]))
        r = int(rng.choice([64, 128, 192, 256]))
    else:
        V = int(rng.choice([3, 64, 129, 1000, 4097, 9000, 20011]))
        r = int(rng.choice([64, 128, 192, 256, 320, 384]))
    rules = np.where(rng.random(b) < 0.5, W.GREEDY, W.SAMPLING).astype(np.int32)
    case = W.make_markov_case(f"msweep{k}", b=b, K=K, V=V, r=r, D=int(rng.choice([8, 32, 64])), rule=rules,
                              T=float(rng.choice([0.3, 0.8, 2.0])), seed=int(rng.integers(1 << 30)))
    return case, float(rng.choice([0.0, 0.5, 0.7]))


@pytest.mark.parametrize("k", range(8))
def test_markov_seeded_sweep(k):
    """Eight seeded random Markov block decodes against the oracle."""
    case, thr = _markov_sweep_case(k)
    gpu = _run(case, thr)
    res = OM.block_decode(case.base, case.anchors, case.w1, case.w2, case.temps, case.seeds, hidden=case.hidden,
                          conf_w=case.conf_w, conf_b=case.conf_b, threshold=thr)
    _check(_compare(case, gpu, res, thr, f"markov_sweep_{k}"), f"markov_sweep_{k}")
