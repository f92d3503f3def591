"""The allocation-free mixed accept (spec_mixed_accept_noalloc, the library's
fixed device scratch instead of a caller workspace) against the workspace
entry point spec_mixed_accept and the oracle.

Two calls in a row through the C ABI: first the b=128, K=7, V=262144 bf16
mixed workload (greedy sequences 0..63, sampling 64..127 at T=0.8), then a
smaller float32 call with ragged draft lengths, so the second call runs over
scratch the first one left behind.  Each must equal the workspace call bit
for bit (same kernels) and meet the oracle parity bar.
"""
import numpy as np
import pytest
import torch

import workloads as W
from parity import compare_mixed, run_gpu_mixed, seeds_to_device, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    import lossless_draft_verification_amd  # noqa: F401


def _run_noalloc(case, temps, lens=None):
    import lossless_draft_verification_amd as L
    b, K = case.b, case.K
    dev = torch.device("cuda")
    out = L.AcceptResult(torch.full((b,), -7, dtype=torch.int32, device=dev),
                         torch.full((b, K + 1), -7, dtype=torch.int32, device=dev),
                         p_draft=torch.full((b, K), 7.0, device=dev),
                         q_draft=torch.full((b, K), 7.0, device=dev),
                         argmax=torch.full((b, K + 1), -7, dtype=torch.int32, device=dev))
    kl = None if lens is None else torch.from_numpy(np.ascontiguousarray(lens, np.int32)).cuda()
    L.mixed_accept_noalloc(to_device(case.target), to_device(case.draft),
                           torch.from_numpy(case.draft_tokens).cuda(),
                           torch.from_numpy(np.ascontiguousarray(temps, np.float64)).cuda(),
                           seeds_to_device(case.seeds), draft_lengths=kl, out=out)
    torch.cuda.synchronize()
    return (out.n_accepted.cpu().numpy(), out.tokens.cpu().numpy(), out.p_draft.cpu().numpy(),
            out.q_draft.cpu().numpy(), out.argmax.cpu().numpy())


def test_noalloc_two_calls_match_workspace_call():
    import lossless_draft_verification_amd as L
    big = W.config(5)
    temps_big = np.where(big.rule == W.GREEDY, 0.0, big.T)
    small = W.make_case("noalloc_small", b=6, K=3, V=3001, dtype="f32", target_scale=2.0,
                        draft_sigma=(0.2, 1.5), T=0.9, seed=23)
    temps_small = np.array([0.0, 0.9, 0.9, 0.0, 1.4, 0.9])
    lens_small = np.array([3, 0, 2, 1, 3, 1], np.int32)
    assert L.mixed_workspace_bytes(big.b, big.K, big.V, torch.bfloat16) <= L.SCRATCH_BYTES
    for case, temps, lens, name in ((big, temps_big, None, "noalloc_c5"),
                                    (small, temps_small, lens_small, "noalloc_small_f32")):
        print(f"[noalloc] {name}: b={case.b} K={case.K} V={case.V} {case.dtype}", flush=True)
        got = _run_noalloc(case, temps, lens)
        ref = run_gpu_mixed(case, temps, lens=lens)
        for g, r in zip(got, ref):
            np.testing.assert_array_equal(g, r)
        rep = compare_mixed(case, temps, *got, name, lens=lens)
        rep.save(name)
        assert not rep.failures, rep.failures[:3]
        ties = rep.accept_near_tie_mismatch + rep.draw_near_tie_mismatch
        assert ties <= max(1, 0.02 * rep.sequences), rep
