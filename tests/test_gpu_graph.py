"""Graph capture of the verify step.

A serving loop can capture the step once in a HIP graph and replay it with
new logits written into the same buffers.  The path's kernels take only the
call's pointers and sizes, keep no host-side state between them, and clear
what must start at zero with their own stores (the residual work list's
count is cleared by the row pass), so every replay of a captured call must
give the eager call's bits on whatever the buffers hold at replay time.
Replays alternate between two batches, with eager work and synchronisations
between them, through the workspace entry point and the allocation-free one,
with and without per-sequence draft lengths.
"""
import numpy as np
import pytest
import torch

import workloads as W
from parity import seeds_to_device, to_device

pytestmark = pytest.mark.gpu

FIELDS = ("n_accepted", "tokens", "p_draft", "q_draft", "argmax")


def _case(seed: int, b: int = 24, K: int = 5, V: int = 20011) -> W.Case:
    return W.make_case("graph", b=b, K=K, V=V, dtype="bf16", target_scale=2.5, draft_sigma=(0.2, 1.5),
                       rule=np.array([W.GREEDY, W.SAMPLING, W.SAMPLING] * (b // 3)), T=0.8, seed=seed,
                       philox_seeds=np.arange(b, dtype=np.uint64) * np.uint64(7919) + np.uint64(seed))


def _result(b: int, K: int):
    import lossless_draft_verification_amd as L
    return L.AcceptResult(torch.empty(b, dtype=torch.int32, device="cuda"),
                          torch.empty(b, K + 1, dtype=torch.int32, device="cuda"),
                          p_draft=torch.empty(b, K, dtype=torch.float32, device="cuda"),
                          q_draft=torch.empty(b, K, dtype=torch.float32, device="cuda"),
                          argmax=torch.empty(b, K + 1, dtype=torch.int32, device="cuda"))


def _host(r) -> dict:
    return {f: getattr(r, f).cpu().numpy().copy() for f in FIELDS}


@pytest.mark.parametrize("ragged", [False, True], ids=["full", "ragged"])
@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
def test_captured_step_replays_eager_bits(noalloc, ragged):
    import lossless_draft_verification_amd as L
    cases = [_case(71), _case(72)]
    b, K, V = cases[0].b, cases[0].K, cases[0].V
    temps = torch.from_numpy(np.where(cases[0].rule == W.GREEDY, 0.0, 0.8)).cuda()
    lens = (torch.from_numpy(np.random.default_rng(73).integers(0, K + 1, size=b).astype(np.int32)).cuda()
            if ragged else None)

    # the eager results of both batches, each call on its own buffers
    want = []
    for case in cases:
        r = L.mixed_accept(to_device(case.target), to_device(case.draft),
                           torch.from_numpy(case.draft_tokens).cuda(), temps, seeds_to_device(case.seeds),
                           draft_lengths=lens)
        torch.cuda.synchronize()
        want.append(_host(r))
    assert not all(np.array_equal(want[0][f], want[1][f]) for f in FIELDS)

    # the buffers the graph reads and writes
    tgt, drf = to_device(cases[0].target), to_device(cases[0].draft)
    x = torch.from_numpy(cases[0].draft_tokens).cuda()
    seeds = seeds_to_device(cases[0].seeds)
    out = _result(b, K)
    ws = torch.empty(L.mixed_workspace_bytes(b, K, V, tgt.dtype), dtype=torch.uint8, device="cuda")

    def call():
        if noalloc:
            L.mixed_accept_noalloc(tgt, drf, x, temps, seeds, draft_lengths=lens, out=out)
        else:
            L.mixed_accept(tgt, drf, x, temps, seeds, draft_lengths=lens, out=out, workspace=ws)

    # one call outside the capture first (device set-up, such as the scratch
    # address, happens on a first call)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()

    for rnd in range(3):
        for k in (1, 0) if rnd % 2 else (0, 1):
            case = cases[k]
            tgt.copy_(to_device(case.target))
            drf.copy_(to_device(case.draft))
            x.copy_(torch.from_numpy(case.draft_tokens).cuda())
            seeds.copy_(seeds_to_device(case.seeds))
            for f in FIELDS:                                    # stale bits must not survive a replay
                getattr(out, f).fill_(-7)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            got = _host(out)
            for f in FIELDS:
                np.testing.assert_array_equal(got[f], want[k][f], err_msg=f"replay {rnd} batch {k} {f}")
