"""Replay of a recorded verify step.

The drafter card describes checking a change by replaying a recorded trace
and requiring identical per-record accepts ("DeepSeek-V4-Flash DSpark
drafter" model card, "Files").  Here one mixed call (greedy and sampled
sequences, ragged draft lengths, bf16) is recorded to disk -- its inputs and
its outputs, as a serving log would hold them -- and then replayed from the
files alone: a fresh call on the loaded inputs must give the recorded
outputs bit for bit, through the workspace entry point and the
allocation-free one, and the recorded outputs must meet the oracle parity bar
on the loaded inputs.
"""
import numpy as np
import pytest
import torch

import workloads as W
from parity import compare_mixed, seeds_to_device, to_device

pytestmark = pytest.mark.gpu

FIELDS = ("n_accepted", "tokens", "p_draft", "q_draft", "argmax")


def _call(case_arrays, noalloc=False):
    import lossless_draft_verification_amd as L
    tgt, drf, x, temps, seeds, lens = case_arrays
    args = (to_device(tgt), to_device(drf), torch.from_numpy(x).cuda(),
            torch.from_numpy(temps).cuda(), seeds_to_device(seeds))
    kl = torch.from_numpy(lens).cuda()
    r = (L.mixed_accept_noalloc if noalloc else L.mixed_accept)(*args, draft_lengths=kl)
    torch.cuda.synchronize()
    return {f: getattr(r, f).cpu().numpy() for f in FIELDS}


def test_replay_recorded_step(tmp_path):
    b, K, V = 48, 7, 65537
    case = W.make_case("replay", b=b, K=K, V=V, dtype="bf16", target_scale=2.5, draft_sigma=(0.2, 1.5),
                       rule=np.array([W.GREEDY, W.SAMPLING, W.SAMPLING] * (b // 3)), T=0.8, seed=97,
                       philox_seeds=np.arange(b, dtype=np.uint64) * np.uint64(1000003) + np.uint64(11))
    temps = np.where(case.rule == W.GREEDY, 0.0, 0.8)
    lens = np.random.default_rng(98).integers(0, K + 1, size=b).astype(np.int32)
    arrays = (case.target, case.draft, case.draft_tokens, temps, case.seeds, lens)

    # record
    out = _call(arrays)
    path = tmp_path / "trace.npz"
    np.savez(path, target=case.target, draft=case.draft, draft_tokens=case.draft_tokens, temperatures=temps,
             seeds=case.seeds, draft_lengths=lens, **{"out_" + f: out[f] for f in FIELDS})

    # replay from the file alone
    rec = np.load(path)
    loaded = (rec["target"], rec["draft"], rec["draft_tokens"], rec["temperatures"], rec["seeds"],
              rec["draft_lengths"])
    for noalloc in (False, True):
        again = _call(loaded, noalloc=noalloc)
        for f in FIELDS:
            np.testing.assert_array_equal(again[f], rec["out_" + f], err_msg=f"{f} (noalloc={noalloc})")

    # and the recorded accepts against the oracle on the loaded inputs
    import dataclasses
    replayed = dataclasses.replace(case, target=rec["target"], draft=rec["draft"],
                                   draft_tokens=rec["draft_tokens"], seeds=rec["seeds"])
    rep = compare_mixed(replayed, rec["temperatures"], rec["out_n_accepted"], rec["out_tokens"],
                        rec["out_p_draft"], rec["out_q_draft"], rec["out_argmax"], "replay",
                        lens=rec["draft_lengths"])
    rep.save("replay")
    assert not rep.failures, rep.failures[:3]
    assert rep.accept_near_tie_mismatch + rep.draw_near_tie_mismatch <= 1
    assert rep.draws > 0 and rep.greedy_sequences == b // 3
