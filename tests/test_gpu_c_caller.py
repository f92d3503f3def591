"""The boundary from plain C.

tests/c_abi_caller.c (built by build() with gcc into tests/_bin/) calls
spec_mixed_accept through include/specverify.h alone, on device buffers it
allocates with the HIP runtime's C API: no Python and no torch in that
process.  The test writes a seeded mixed call's inputs to a file, runs the
program as a child process, and checks its outputs against the oracle (the
parity bar of the other tests) and bit for bit against the Python binding's
call on the same inputs.  bf16 and fp32 logits, with and without draft
lengths.
"""
import os
import subprocess

import numpy as np
import pytest

import workloads as W
from parity import compare_mixed, run_gpu_mixed

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CALLER = os.path.join(ROOT, "tests", "_bin", "c_abi_caller")
DTYPE_CODE = {"f32": 0, "bf16": 1}


def _write_inputs(path, case, temps, lens):
    b, K, V = case.b, case.K, case.V
    with open(path, "wb") as f:
        f.write(np.array([b, K, V, DTYPE_CODE[case.dtype], lens is not None], dtype="<i4").tobytes())
        f.write(np.ascontiguousarray(case.target).tobytes())
        f.write(np.ascontiguousarray(case.draft).tobytes())
        f.write(np.ascontiguousarray(case.draft_tokens, dtype="<i4").tobytes())
        f.write(np.ascontiguousarray(temps, dtype="<f8").tobytes())
        if lens is not None:
            f.write(np.ascontiguousarray(lens, dtype="<i4").tobytes())
        f.write(np.ascontiguousarray(case.seeds, dtype="<u8").tobytes())


def _read_outputs(path, b, K):
    raw = open(path, "rb").read()
    off = 0

    def take(dtype, n):
        nonlocal off
        a = np.frombuffer(raw, dtype=dtype, count=n, offset=off)
        off += a.nbytes
        return a

    status = int(take("<i4", 1)[0])
    n = take("<i4", b)
    tok = take("<i4", b * (K + 1)).reshape(b, K + 1)
    p = take("<f4", b * K).reshape(b, K)
    q = take("<f4", b * K).reshape(b, K)
    am = take("<i4", b * (K + 1)).reshape(b, K + 1)
    assert off == len(raw), (off, len(raw))
    return status, (n, tok, p, q, am)


@pytest.mark.parametrize("ragged", [False, True], ids=["full", "lengths"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_plain_c_caller_matches_binding_and_oracle(tmp_path, dtype, ragged):
    assert os.path.exists(CALLER), f"{CALLER} is missing: run __graft_entry__.build()"
    b, K, V = 18, 5, 12007
    case = W.make_case("c_caller", b=b, K=K, V=V, dtype=dtype, target_scale=2.5, draft_sigma=(0.2, 1.5),
                       T=0.8, seed=401 + int(ragged) + 2 * (dtype == "f32"))
    temps = np.where(np.arange(b) % 3 == 0, 0.0, 0.8)
    lens = np.random.default_rng(402).integers(0, K + 1, size=b).astype(np.int32) if ragged else None
    fin, fout = str(tmp_path / "in.bin"), str(tmp_path / "out.bin")
    _write_inputs(fin, case, temps, lens)
    print(f"c_abi_caller: dtype={dtype} lengths={ragged} b={b} K={K} V={V}", flush=True)
    proc = subprocess.run([CALLER, fin, fout], capture_output=True, text=True, timeout=120)
    assert proc.returncode == 0, (proc.returncode, proc.stderr)
    status, got = _read_outputs(fout, b, K)
    assert status == 0

    # the same call through the Python binding: the same bits
    want = run_gpu_mixed(case, temps, lens=lens)
    for name, g, w in zip(("n_accepted", "tokens", "p_draft", "q_draft", "argmax"), got, want):
        np.testing.assert_array_equal(g, w, err_msg=name)

    # and the oracle's parity bar
    rep = compare_mixed(case, temps, *got, f"c_caller_{dtype}_{'lengths' if ragged else 'full'}", lens=lens)
    assert not rep.failures, rep.failures[:3]
    assert rep.accept_near_tie_mismatch + rep.draw_near_tie_mismatch <= 1, rep
