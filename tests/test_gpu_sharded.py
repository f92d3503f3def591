"""GPU parity of the vocabulary-sharded verify (shards in separate buffers,
per-shard row and residual passes, one record per row per shard merged in
shard order) against the oracle on the concatenated vocabulary, and against
the unsharded call on the same bytes.
"""
import numpy as np
import pytest
import torch

import workloads as W
from parity import Report, compare_mixed, seeds_to_device, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    import lossless_draft_verification_amd  # noqa: F401


def _check(rep: Report, name: str, max_near_tie_frac: float = 0.02):
    rep.save(name)
    assert not rep.failures, rep.failures[:3]
    ties = rep.accept_near_tie_mismatch + rep.draw_near_tie_mismatch
    assert ties <= max(1, max_near_tie_frac * max(rep.sequences, 1)), rep


def _shards(case: W.Case, widths):
    """Column slices of the target and draft blocks, each a separate buffer."""
    assert sum(widths) == case.V
    cuts = np.cumsum([0] + list(widths))
    t = [to_device(np.ascontiguousarray(case.target[:, :, a:b])) for a, b in zip(cuts[:-1], cuts[1:])]
    d = [to_device(np.ascontiguousarray(case.draft[:, :, a:b])) for a, b in zip(cuts[:-1], cuts[1:])]
    return t, d


def _run(case, temps, widths, lens=None):
    import lossless_draft_verification_amd as L
    ts, ds = _shards(case, widths)
    kl = None if lens is None else torch.from_numpy(np.ascontiguousarray(lens, np.int32)).cuda()
    r = L.sharded_mixed_accept(ts, ds, torch.from_numpy(case.draft_tokens).cuda(),
                               torch.from_numpy(np.ascontiguousarray(temps, np.float64)).cuda(),
                               seeds_to_device(case.seeds), draft_lengths=kl)
    torch.cuda.synchronize()
    return (r.n_accepted.cpu().numpy(), r.tokens.cpu().numpy(), r.p_draft.cpu().numpy(),
            r.q_draft.cpu().numpy(), r.argmax.cpu().numpy())


def _run_unsharded(case, temps, lens=None):
    import lossless_draft_verification_amd as L
    kl = None if lens is None else torch.from_numpy(np.ascontiguousarray(lens, np.int32)).cuda()
    r = L.mixed_accept(to_device(case.target), to_device(case.draft), torch.from_numpy(case.draft_tokens).cuda(),
                       torch.from_numpy(np.ascontiguousarray(temps, np.float64)).cuda(),
                       seeds_to_device(case.seeds), draft_lengths=kl)
    torch.cuda.synchronize()
    return (r.n_accepted.cpu().numpy(), r.tokens.cpu().numpy(), r.p_draft.cpu().numpy(),
            r.q_draft.cpu().numpy(), r.argmax.cpu().numpy())


SPLITS = [
    # name, dtype, V, widths
    ("one_shard", "bf16", 20011, [20011]),
    ("uneven_bf16", "bf16", 20011, [7001, 9000, 4010]),
    ("uneven_f32", "f32", 20011, [1, 12000, 8010]),
    ("many_small", "bf16", 3000, [200] * 15),
    ("aligned_8", "bf16", 65536, [8192] * 8),
]


@pytest.mark.parametrize("spec", SPLITS, ids=[s[0] for s in SPLITS])
def test_sharded_matches_oracle_and_unsharded(spec):
    name, dt, V, widths = spec
    b, K = 24, 5
    case = W.make_case("shard", b=b, K=K, V=V, dtype=dt, target_scale=2.5, draft_sigma=(0.2, 1.5), T=0.8,
                       seed=81 + len(widths))
    temps = np.where(np.arange(b) % 3 == 0, 0.0, 0.8)
    temps[4] = 1.3
    temps[7] = -1.0
    out = _run(case, temps, widths)
    _check(compare_mixed(case, temps, *out, f"sharded_{name}"), f"sharded_{name}")
    ref = _run_unsharded(case, temps)
    for a, r in zip((out[0], out[1], out[4]), (ref[0], ref[1], ref[4])):
        np.testing.assert_array_equal(a, r)
    ok = ~np.isnan(ref[2])
    np.testing.assert_allclose(out[2][ok], ref[2][ok], rtol=1e-6)


def test_sharded_ragged_lengths():
    b, K = 20, 6
    case = W.make_case("shard_rag", b=b, K=K, V=12000, dtype="bf16", target_scale=2.5, draft_sigma=(0.2, 1.5),
                       T=1.0, seed=91)
    temps = np.where(np.arange(b) % 2 == 0, 0.0, 1.0)
    lens = (np.arange(b) % (K + 1)).astype(np.int32)
    out = _run(case, temps, [5000, 4000, 3000], lens)
    _check(compare_mixed(case, temps, *out, "sharded_ragged", lens=lens), "sharded_ragged")
    ref = _run_unsharded(case, temps, lens)
    np.testing.assert_array_equal(out[1], ref[1])


def test_sharded_workload_c5_eight_shards():
    """b=128, K=7, V=262144 bf16, rows 0..63 greedy / 64..127 sampling, split
    into 8 shards of 32768 columns (a tensor-parallel degree of 8)."""
    case = W.config(5)
    temps = np.where(case.rule == W.GREEDY, 0.0, case.T)
    out = _run(case, temps, [32768] * 8)
    _check(compare_mixed(case, temps, *out, "c5_sharded8"), "workload_c5_sharded8")
    ref = _run_unsharded(case, temps)
    for a, r in zip((out[0], out[1], out[4]), (ref[0], ref[1], ref[4])):
        np.testing.assert_array_equal(a, r)


def test_sharded_deterministic_repeat():
    """Two calls on the same shards give the same bytes."""
    b, K = 20, 5
    case = W.make_case("shard_det", b=b, K=K, V=12000, dtype="bf16", target_scale=2.5, draft_sigma=(0.2, 1.5),
                       T=0.8, seed=93)
    temps = np.where(np.arange(b) % 2 == 0, 0.0, 0.8)
    a, c = _run(case, temps, [4000, 5000, 3000]), _run(case, temps, [4000, 5000, 3000])
    for x, y in zip(a, c):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("k", range(6))
def test_sharded_seeded_sweep(k):
    """Six seeded random splits (1 to 12 shards of uneven widths, some of one
    column), both dtypes, per-sequence rules and temperatures, draft lengths
    in odd cases: equal to the oracle and to the unsharded call."""
    rng = np.random.default_rng(11000 + k)
    b, K = int(rng.integers(1, 40)), int(rng.integers(1, 9))
    V = int(rng.choice([50, 3000, 20011, 40000]))
    G = int(rng.integers(1, min(12, V) + 1))
    cuts = np.sort(rng.choice(np.arange(1, V), size=G - 1, replace=False)) if G > 1 else np.array([], int)
    widths = [int(x) for x in np.diff(np.concatenate([[0], cuts, [V]]))]
    dt = str(rng.choice(["bf16", "f32"]))
    case = W.make_case(f"shsweep{k}", b=b, K=K, V=V, dtype=dt, target_scale=2.5, draft_sigma=(0.1, 1.5), T=0.8,
                       seed=int(rng.integers(1 << 30)))
    temps = np.where(rng.random(b) < 0.4, 0.0, rng.choice([0.5, 0.8, 1.3], size=b))
    lens = rng.integers(0, K + 1, size=b).astype(np.int32) if k % 2 else None
    out = _run(case, temps, widths, lens)
    _check(compare_mixed(case, temps, *out, f"sharded_sweep_{k}", lens=lens), f"sharded_sweep_{k}")
    ref = _run_unsharded(case, temps, lens)
    for a, r in zip((out[0], out[1], out[4]), (ref[0], ref[1], ref[4])):
        np.testing.assert_array_equal(a, r)



def test_sharded_zero_residual_mass():
    """The zero-residual-mass fallback through the sharded call: every shard's
    residual mass is zero, so the shard selection falls back to the target
    masses of slot n.  Integer results equal the unsharded call's."""
    case = W.make_zero_mass_case("zmass_sh", b=18, K=5, V=20011, dtype="bf16", T=0.9, seed=19)
    temps = np.where(np.arange(case.b) % 4 == 3, 0.0, case.T)
    widths = [7001, 9000, 4010]
    out = _run(case, temps, widths)
    ref = _run_unsharded(case, temps)
    for a, b_ in zip((out[0], out[1], out[4]), (ref[0], ref[1], ref[4])):
        np.testing.assert_array_equal(a, b_)
    _check(compare_mixed(case, temps, *out, "sharded_zero_mass"), "sharded_zero_mass")
