"""Calls from several host threads at once.

The boundary keeps no state between calls: each call's kernels take only
its own pointers and sizes, and the profiling events are per host thread.
So host threads that call the entry points at the same time, each on its
own stream with its own workspace and outputs, must each get the bits a
lone call gives.  Three threads run side by side (ctypes drops the GIL for
the foreign call, so their host code really overlaps and their kernels run
on three streams): the plain mixed call, a mixed call with per-sequence
draft lengths (the listed row pass) and a vocabulary-sharded call.  Each
repeats its call and checks every result.
"""
import threading

import numpy as np
import pytest
import torch

import workloads as W
from parity import seeds_to_device, to_device

pytestmark = pytest.mark.gpu

FIELDS = ("n_accepted", "tokens", "p_draft", "q_draft", "argmax")
REPEATS = 20
WIDTHS = [6001, 8000, 6010]


def _case(seed: int, b: int = 30, K: int = 6, V: int = 20011) -> W.Case:
    return W.make_case("threads", b=b, K=K, V=V, dtype="bf16", target_scale=2.5, draft_sigma=(0.2, 1.5),
                       rule=np.array([W.GREEDY, W.SAMPLING, W.SAMPLING] * (b // 3)), T=0.8, seed=seed,
                       philox_seeds=np.arange(b, dtype=np.uint64) * np.uint64(104729) + np.uint64(seed))


def _host(r) -> dict:
    return {f: getattr(r, f).cpu().numpy().copy() for f in FIELDS}


def _result(b: int, K: int):
    import lossless_draft_verification_amd as L
    return L.AcceptResult(torch.empty(b, dtype=torch.int32, device="cuda"),
                          torch.empty(b, K + 1, dtype=torch.int32, device="cuda"),
                          p_draft=torch.empty(b, K, dtype=torch.float32, device="cuda"),
                          q_draft=torch.empty(b, K, dtype=torch.float32, device="cuda"),
                          argmax=torch.empty(b, K + 1, dtype=torch.int32, device="cuda"))


def _caller(kind: str, case: W.Case, lens_seed: int):
    """A function that makes one call of `kind` on `case` into the given
    outputs and workspace (on the current stream), and the workspace size."""
    import lossless_draft_verification_amd as L
    b, K, V = case.b, case.K, case.V
    temps = torch.from_numpy(np.where(case.rule == W.GREEDY, 0.0, 0.8)).cuda()
    x = torch.from_numpy(case.draft_tokens).cuda()
    seeds = seeds_to_device(case.seeds)
    if kind == "sharded":
        cuts = np.cumsum([0] + WIDTHS)
        tg = [to_device(np.ascontiguousarray(case.target[:, :, a0:a1])) for a0, a1 in zip(cuts[:-1], cuts[1:])]
        dr = [to_device(np.ascontiguousarray(case.draft[:, :, a0:a1])) for a0, a1 in zip(cuts[:-1], cuts[1:])]
        nbytes = L.sharded_workspace_bytes(WIDTHS, b, K, torch.bfloat16)

        def call(out=None, workspace=None):
            return L.sharded_mixed_accept(tg, dr, x, temps, seeds, out=out, workspace=workspace)
        return call, nbytes
    tgt, drf = to_device(case.target), to_device(case.draft)
    lens = None
    if kind == "ragged":
        lens = torch.from_numpy(np.random.default_rng(lens_seed).integers(0, K + 1, size=b).astype(np.int32)).cuda()
    nbytes = L.mixed_workspace_bytes(b, K, V, tgt.dtype)

    def call(out=None, workspace=None):
        return L.mixed_accept(tgt, drf, x, temps, seeds, draft_lengths=lens, out=out, workspace=workspace)
    return call, nbytes


def test_host_threads_on_their_own_streams():
    kinds = [("plain", 301), ("ragged", 302), ("sharded", 303)]
    assert sum(WIDTHS) == 20011
    # each call alone first: the bits every threaded repeat must give
    callers, want = [], []
    for kind, seed in kinds:
        call, nbytes = _caller(kind, _case(seed), seed + 1000)
        r = call()
        torch.cuda.synchronize()
        callers.append((call, nbytes))
        want.append(_host(r))
    # the three calls differ, so a result landing in the wrong thread's buffers shows
    assert not np.array_equal(want[0]["tokens"], want[2]["tokens"])

    errors = []
    start = threading.Barrier(len(kinds))

    def worker(k):
        try:
            call, nbytes = callers[k]
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                b, K1 = want[k]["tokens"].shape
                out = _result(b, K1 - 1)
                ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
                st.synchronize()
                start.wait(timeout=60)
                for rep in range(REPEATS):
                    for f in FIELDS:                          # stale bits must not pass
                        getattr(out, f).fill_(-7)
                    call(out=out, workspace=ws)
                    st.synchronize()
                    got = _host(out)
                    for f in FIELDS:
                        if not np.array_equal(got[f], want[k][f], equal_nan=True):
                            errors.append(f"{kinds[k][0]}: repeat {rep} field {f} differs")
                            return
        except Exception as e:                                # reported by the main thread
            start.abort()                                     # no thread waits for this one
            errors.append(f"{kinds[k][0]}: {type(e).__name__}: {e}")

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(len(kinds))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a caller thread did not finish"
    assert not errors, errors
