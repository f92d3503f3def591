"""GPU parity of the fused verify (lm_head GEMM on the matrix cores with the
verify's row statistics in its epilogue) against the oracle.

The GEMM's float32 logits are checked element by element against the
float64 definition within the float32 summation bound (see
tests/parity.py, fused_tolerance); decisions are compared exactly except
where the oracle sits within that perturbation of a decision boundary, and
every such case is counted.
"""
import numpy as np
import pytest
import torch

import oracle.fused as OF
import workloads as W
from parity import Report, compare_fused, fused_tolerance, seeds_to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    import lossless_draft_verification_amd  # noqa: F401


def _bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _check(rep: Report, name: str, max_near_tie_frac: float = 0.02):
    rep.save(name)
    assert not rep.failures, rep.failures[:3]
    ties = rep.accept_near_tie_mismatch + rep.draw_near_tie_mismatch
    assert ties <= max(1, max_near_tie_frac * max(rep.sequences, 1)), rep


# -------------------------------------------------------------- the GEMM alone

LOGIT_CASES = [
    # name, rows, V, D, softcap
    ("tiny", 5, 1000, 64, 0.0),
    ("two_row_tiles_ragged_vocab", 300, 70000, 256, 30.0),
    ("gemma_width", 17, 4099, 3840, 30.0),
    ("exact_tiles", 256, 8192, 128, 0.0),
]


@pytest.mark.parametrize("spec", LOGIT_CASES, ids=[c[0] for c in LOGIT_CASES])
def test_lm_head_logits_within_bound(spec):
    import lossless_draft_verification_amd as L
    name, rows, V, D, cap = spec
    rng = np.random.default_rng(rows * 7 + D)
    h = W.bf16_bits(rng.standard_normal((rows, 1, D), dtype=np.float32))
    w = W.bf16_bits(rng.standard_normal((V, D), dtype=np.float32) * np.float32(3.0 / np.sqrt(D)))
    z = L.lm_head_logits(_bf16_dev(h[:, 0]), _bf16_dev(w), softcap=cap)
    torch.cuda.synchronize()
    zg = z.cpu().numpy().astype(np.float64)
    z64 = OF.lm_head_logits(h, w, cap)[:, 0]
    tol = fused_tolerance(h, w, cap, z64[:, None], None)[:, 0]
    err = np.abs(zg - z64)
    ratio = float((err / tol).max())
    print(f"[logits {name}] max |err| = {err.max():.3e}, max err/bound = {ratio:.3e}", flush=True)
    assert (err <= tol).all(), np.unravel_index(np.argmax(err / tol), err.shape)


# -------------------------------------------------------------- fused accept


def _run_fused(case: W.FusedCase, lens=None):
    import lossless_draft_verification_amd as L
    kl = None if lens is None else torch.from_numpy(np.ascontiguousarray(lens, np.int32)).cuda()
    r = L.fused_mixed_accept(
        _bf16_dev(case.hidden), _bf16_dev(case.weight), torch.from_numpy(case.draft).cuda(),
        torch.from_numpy(case.draft_tokens).cuda(), torch.from_numpy(case.temps).cuda(),
        seeds_to_device(case.seeds), softcap=case.softcap, draft_lengths=kl)
    torch.cuda.synchronize()
    return (r.n_accepted.cpu().numpy(), r.tokens.cpu().numpy(), r.p_draft.cpu().numpy(),
            r.q_draft.cpu().numpy(), r.argmax.cpu().numpy())


def _oracle(case: W.FusedCase, seqs=None, lens=None):
    res = OF.fused_mixed_accept(case.hidden, case.weight, case.softcap, case.draft, case.draft_tokens,
                                case.temps, case.seeds, lens, seqs, with_abs=True)
    tol = fused_tolerance(case.hidden, case.weight, case.softcap, res["logits64"], res["seqs"],
                          res.pop("abs_products"))
    return res, tol


@pytest.mark.parametrize("cap", [0.0, 30.0])
def test_fused_small_mixed(cap):
    """Both rules, invalid temperatures, V with a ragged last tile, hidden rows
    spanning two row tiles (b*(K+1) = 300)."""
    b, K = 60, 4
    rule = np.array([W.GREEDY, W.SAMPLING] * (b // 2))
    case = W.make_fused_case("fsmall", b=b, K=K, V=20011, D=256, softcap=cap, rule=rule, T=0.8, seed=71)
    case.temps[5] = -1.0
    case.temps[8] = np.inf
    case.temps[9] = 1.3
    out = _run_fused(case)
    res, tol = _oracle(case)
    assert out[0][5] == -1 and out[0][8] == -1
    rep = compare_fused(case, res, tol, *out, f"fused_small_cap{int(cap)}")
    _check(rep, f"fused_small_cap{int(cap)}")


def test_fused_ragged_lengths():
    b, K = 24, 5
    rule = np.array([W.GREEDY, W.SAMPLING, W.SAMPLING] * (b // 3))
    case = W.make_fused_case("fragged", b=b, K=K, V=9000, D=192, softcap=30.0, rule=rule, T=1.0, seed=72)
    lens = (np.arange(b) % (K + 1)).astype(np.int32)
    lens[-1] = K + 2
    out = _run_fused(case, lens)
    res, tol = _oracle(case, lens=lens)
    assert out[0][-1] == -1
    _check(compare_fused(case, res, tol, *out, "fused_ragged", lens=lens), "fused_ragged")


_FULL = {}


def _full_case():
    if "c" not in _FULL:
        _FULL["c"] = W.fused_config()
    return _FULL["c"]


@pytest.mark.timeout(900)
def test_fused_full_size_all_sequences():
    """b=128, K=7, V=262144, D=3840, softcap 30, rows 0..63 greedy and
    64..127 sampled at T=0.8 in one call (the benchmark's launch); the oracle
    forms the float64 logits of all 128 sequences (about 4 TFLOP on the host,
    in vocabulary slabs) and every sequence is compared."""
    case = _full_case()
    out = _run_fused(case)
    res, tol = _oracle(case)
    assert len(res["seqs"]) == case.hidden.shape[0] == 128
    rep = compare_fused(case, res, tol, *out, "fused_full")
    assert rep.sequences == 128 and rep.greedy_sequences == 64 and rep.sampling_sequences == 64
    _check(rep, "fused_full")


def test_fused_deterministic_repeat():
    """Two calls on the same inputs give the same bytes (every merge is in a
    fixed order; there are no floating-point atomics)."""
    b, K = 40, 5
    rule = np.array([W.GREEDY, W.SAMPLING] * (b // 2))
    case = W.make_fused_case("fdet", b=b, K=K, V=12000, D=256, softcap=30.0, rule=rule, T=0.9, seed=74)
    a, c = _run_fused(case), _run_fused(case)
    for x, y in zip(a, c):
        np.testing.assert_array_equal(x, y)


def _fused_sweep_case(k: int):
    """Seeded random b, K, V, D (a multiple of 64), softcap, per-sequence
    rule and temperature (some invalid) and, in odd cases, draft lengths."""
    rng = np.random.default_rng(9000 + k)
    K = int(rng.integers(1, 8))
    V = int(rng.choice([7, 300, 4097, 9000, 20011]))
    b = int(rng.integers(1, min(70, V // (K + 1)) + 1)) if V >= K + 1 else 1   # distinct planted tokens
    if V < b * (K + 1):
        V = b * (K + 1)
    D = int(rng.choice([64, 128, 192, 256, 512]))
    cap = float(rng.choice([0.0, 30.0]))
    rule = np.where(rng.random(b) < 0.5, W.GREEDY, W.SAMPLING).astype(np.int32)
    case = W.make_fused_case(f"fsweep{k}", b=b, K=K, V=V, D=D, softcap=cap, rule=rule,
                             T=float(rng.choice([0.5, 0.8, 1.5])), seed=int(rng.integers(1 << 30)))
    bad = rng.random(b) < 0.08
    case.temps[bad] = rng.choice([-1.0, np.inf], size=int(bad.sum()))
    lens = rng.integers(0, K + 1, size=b).astype(np.int32) if k % 2 else None
    return case, lens


@pytest.mark.parametrize("k", range(6))
def test_fused_seeded_sweep(k):
    """Six seeded random fused calls (one row tile to several, V from 7 to a
    ragged 20011, D from 64 to 512, softcap on and off) against the oracle."""
    case, lens = _fused_sweep_case(k)
    out = _run_fused(case, lens)
    res, tol = _oracle(case, lens=lens)
    _check(compare_fused(case, res, tol, *out, f"fused_sweep_{k}", lens=lens), f"fused_sweep_{k}")

