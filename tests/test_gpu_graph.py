"""Graph capture of the verify step and of the other entry points.

A serving loop can capture the step once in a HIP graph and replay it with
new logits written into the same buffers.  The path's kernels take only the
call's pointers and sizes, keep no host-side state between them, and clear
what must start at zero with their own stores (the residual work list's
count is cleared by the row pass), so every replay of a captured call must
give the eager call's bits on whatever the buffers hold at replay time.
Replays alternate between two batches, with eager work and synchronisations
between them, through the workspace entry point and the allocation-free one,
with and without per-sequence draft lengths, and through the fused,
vocabulary-sharded and Markov entry points (each captured with its
workspace).
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


# ------------------------------------------------ the other entry points


def _bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _replay(bufs: dict, loads: list, call, outputs, want: list):
    """Capture call() once, then for each round and batch k copy loads[k]
    (name -> device tensor) into the captured buffers, poison the outputs,
    replay and compare outputs() with want[k] bit for bit."""
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
            for name, t in loads[k].items():
                bufs[name].copy_(t)
            for t in outputs().values():
                t.fill_(-7)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            got = {f: t.cpu().numpy() for f, t in outputs().items()}
            for f in got:
                np.testing.assert_array_equal(got[f], want[k][f], err_msg=f"replay {rnd} batch {k} {f}")


def test_captured_fused_call():
    import lossless_draft_verification_amd as L
    b, K, V, D = 24, 5, 9000, 192
    rule = np.array([W.GREEDY, W.SAMPLING, W.SAMPLING] * (b // 3))
    cases = [W.make_fused_case(f"gfused{k}", b=b, K=K, V=V, D=D, softcap=30.0, rule=rule, T=1.0, seed=81 + k)
             for k in range(2)]
    loads = [{"h": _bf16_dev(c.hidden), "w": _bf16_dev(c.weight), "d": torch.from_numpy(c.draft).cuda(),
              "x": torch.from_numpy(c.draft_tokens).cuda(), "t": torch.from_numpy(c.temps).cuda(),
              "s": seeds_to_device(c.seeds)} for c in cases]
    want = []
    for ld in loads:
        r = L.fused_mixed_accept(ld["h"].clone(), ld["w"].clone(), ld["d"].clone(), ld["x"].clone(), ld["t"].clone(),
                                 ld["s"].clone(), softcap=30.0)
        torch.cuda.synchronize()
        want.append(_host(r))
    bufs = {k: v.clone() for k, v in loads[0].items()}
    out = _result(b, K)
    ws = torch.empty(L.fused_workspace_bytes(b, K, V, D), dtype=torch.uint8, device="cuda")
    _replay(bufs, loads,
            lambda: L.fused_mixed_accept(bufs["h"], bufs["w"], bufs["d"], bufs["x"], bufs["t"], bufs["s"],
                                         softcap=30.0, out=out, workspace=ws),
            lambda: {f: getattr(out, f) for f in FIELDS}, want)


def test_captured_sharded_call():
    import lossless_draft_verification_amd as L
    widths = [7001, 9000, 4010]
    cases = [_case(91), _case(92)]
    b, K, V = cases[0].b, cases[0].K, cases[0].V
    cuts = np.cumsum([0] + widths)
    temps = torch.from_numpy(np.where(cases[0].rule == W.GREEDY, 0.0, 0.8)).cuda()

    def load(c):
        ld = {"x": torch.from_numpy(c.draft_tokens).cuda(), "s": seeds_to_device(c.seeds)}
        for g, (a0, a1) in enumerate(zip(cuts[:-1], cuts[1:])):
            ld[f"t{g}"] = to_device(np.ascontiguousarray(c.target[:, :, a0:a1]))
            ld[f"d{g}"] = to_device(np.ascontiguousarray(c.draft[:, :, a0:a1]))
        return ld
    loads = [load(c) for c in cases]
    G = len(widths)
    want = []
    for ld in loads:
        r = L.sharded_mixed_accept([ld[f"t{g}"].clone() for g in range(G)], [ld[f"d{g}"].clone() for g in range(G)],
                                   ld["x"].clone(), temps, ld["s"].clone())
        torch.cuda.synchronize()
        want.append(_host(r))
    bufs = {k: v.clone() for k, v in loads[0].items()}
    out = _result(b, K)
    ws = torch.empty(L.sharded_workspace_bytes(widths, b, K, torch.bfloat16), dtype=torch.uint8, device="cuda")
    _replay(bufs, loads,
            lambda: L.sharded_mixed_accept([bufs[f"t{g}"] for g in range(G)], [bufs[f"d{g}"] for g in range(G)],
                                           bufs["x"], temps, bufs["s"], out=out, workspace=ws),
            lambda: {f: getattr(out, f) for f in FIELDS}, want)


def test_captured_markov_decode():
    import lossless_draft_verification_amd as L
    b, K, V, r, D = 6, 3, 4096, 256, 16
    rule = np.array([W.GREEDY, W.SAMPLING] * (b // 2))
    cases = [W.make_markov_case(f"gmarkov{k}", b=b, K=K, V=V, r=r, D=D, rule=rule, T=0.8, seed=95 + k)
             for k in range(2)]
    conf_b = cases[0].conf_b
    loads = [{"base": torch.from_numpy(c.base).cuda(), "anc": torch.from_numpy(c.anchors).cuda(),
              "w1": _bf16_dev(c.w1), "w2": _bf16_dev(c.w2),
              "t": torch.from_numpy(np.ascontiguousarray(c.temps, np.float64)).cuda(),
              "s": seeds_to_device(c.seeds), "h": _bf16_dev(c.hidden), "cw": _bf16_dev(c.conf_w)} for c in cases]
    fields = ("tokens", "logits", "confidence", "lengths")
    want = []
    for ld in loads:
        res = L.markov_block_decode(ld["base"].clone(), ld["anc"].clone(), ld["w1"].clone(), ld["w2"].clone(),
                                    ld["t"].clone(), ld["s"].clone(), hidden=ld["h"].clone(), conf_w=ld["cw"].clone(),
                                    conf_b=conf_b, threshold=0.5)
        torch.cuda.synchronize()
        want.append({f: getattr(res, f).cpu().numpy().copy() for f in fields})
    bufs = {k: v.clone() for k, v in loads[0].items()}
    out = L.DraftBlock(torch.empty(b, K, dtype=torch.int32, device="cuda"),
                       torch.empty(b, K, V, dtype=torch.float32, device="cuda"),
                       torch.empty(b, K, dtype=torch.float32, device="cuda"),
                       torch.empty(b, dtype=torch.int32, device="cuda"))
    ws = torch.empty(L.markov_workspace_bytes(b, K, V, r), dtype=torch.uint8, device="cuda")
    _replay(bufs, loads,
            lambda: L.markov_block_decode(bufs["base"], bufs["anc"], bufs["w1"], bufs["w2"], bufs["t"], bufs["s"],
                                          hidden=bufs["h"], conf_w=bufs["cw"], conf_b=conf_b, threshold=0.5,
                                          out=out, workspace=ws),
            lambda: {f: getattr(out, f) for f in fields}, want)
