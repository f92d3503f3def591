"""CPU oracle for the verify/accept step (test infrastructure only).

Thin ctypes wrapper over ``spec_oracle.c``: a plain single-threaded C
implementation in double precision of greedy accept and lossless
speculative-sampling accept, plus the Philox4x32-10 uniform stream.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (``lossless_draft_verification_amd``)
never does, and the two share no code.

What is computed, and where the pages fix it, is stated in the header of
``spec_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "spec_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_spec.so")

F32 = 0
BF16 = 1


def build(path: str = _LIB, mutant: int = 0, sanitize: bool = False) -> str:
    """Compile the oracle with gcc -O2 (single-threaded, no fast-math).

    `mutant` > 0 builds a planted-mistake variant (see the header of
    spec_oracle.c) for the tests' negative controls; the default is 0.
    `sanitize` builds it with AddressSanitizer and UndefinedBehaviorSanitizer
    (-O1 -g); a process loading that build preloads gcc's libasan.
    """
    tmp = path + ".tmp"
    opt = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer"] if sanitize else ["-O2"]
    subprocess.check_call(
        ["gcc", *opt, "-std=c11", "-Wall", "-Wextra", f"-DORACLE_MUTANT={int(mutant)}",
         "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, path)
    return path


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:  # raw bf16 bits
        return BF16
    raise TypeError(f"logits must be float32 or uint16 (bf16 bits), got {a.dtype}")


class Oracle:
    """One loaded build of spec_oracle.c."""

    def __init__(self, path: str = _LIB):
        if path == _LIB and not os.path.exists(path):
            build(path)
        lib = ctypes.CDLL(path)
        vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.oracle_philox4x32_10.argtypes = [vp, vp, vp]
        lib.oracle_philox4x32_10.restype = None
        lib.oracle_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                       ctypes.c_uint32]
        lib.oracle_uniform.restype = dbl
        lib.oracle_uniform_grid.argtypes = [ctypes.c_uint64, ctypes.c_uint32, i32, ctypes.c_uint32, i32,
                                            ctypes.c_uint32, vp]
        lib.oracle_uniform_grid.restype = None
        lib.oracle_greedy_accept.argtypes = [vp, i32, i64, i64, vp, i32, i32, i32, vp, vp, vp]
        lib.oracle_greedy_accept.restype = i32
        lib.oracle_sample_accept.argtypes = [vp, vp, i32, i64, i64, i64, i64, vp, i32, i32, i32,
                                             dbl, vp, vp, vp, vp, vp, vp]
        lib.oracle_sample_accept.restype = i32
        lib.oracle_mixed_accept.argtypes = [vp, vp, i32, i64, i64, i64, i64, vp, i32, i32, i32,
                                            vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.oracle_mixed_accept.restype = i32
        lib.oracle_draw_cdf.argtypes = [vp, vp, i32, i64, i64, i64, i64, i32, i32, dbl,
                                        i32, i32, i32, vp]
        lib.oracle_draw_cdf.restype = i32
        lib.oracle_row_log_normaliser.argtypes = [vp, i32, i32, dbl]
        lib.oracle_row_log_normaliser.restype = dbl
        self.lib = lib
        self.path = path

    def philox4x32_10(self, counter, key) -> np.ndarray:
        """Philox4x32-10 block: four 32-bit counter words, two key words."""
        c = np.ascontiguousarray(np.asarray(counter, dtype=np.uint32))
        k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32))
        out = np.zeros(4, dtype=np.uint32)
        self.lib.oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
        return out

    def uniform(self, seed: int, row: int, pos: int, tag: int) -> float:
        """U(seed, row, pos, tag) = (word0 >> 8) * 2^-24 of Philox at (pos, row, tag, 0)."""
        return self.lib.oracle_uniform(int(seed), int(row), int(pos), int(tag))

    def uniform_grid(self, seed: int, row0: int, nrow: int, pos0: int, npos: int, tag: int) -> np.ndarray:
        """U(seed, row0 + r, pos0 + p, tag) as a float64 [nrow, npos] array."""
        out = np.zeros((nrow, npos), np.float64)
        self.lib.oracle_uniform_grid(int(seed) & (2 ** 64 - 1), int(row0) & 0xFFFFFFFF, int(nrow),
                                     int(pos0) & 0xFFFFFFFF, int(npos), int(tag) & 0xFFFFFFFF, _ptr(out))
        return out

    def row_log_normaliser(self, row: np.ndarray, T: float) -> float:
        """C = m + ln sum exp(z/T - m) of one logit row (float32 or bf16 bits)."""
        row = np.ascontiguousarray(row)
        return self.lib.oracle_row_log_normaliser(_ptr(row), _dtype_code(row), row.shape[-1],
                                                  float(T))

    def greedy_accept(self, target: np.ndarray, draft_tokens: np.ndarray):
        """Greedy accept over target [b, K+1, V] and draft tokens [b, K].

        Returns (n_accepted [b], tokens [b, K+1], argmax [b, K+1]).
        """
        target = np.ascontiguousarray(target)
        x = np.ascontiguousarray(draft_tokens, dtype=np.int32)
        b, K1, V = target.shape
        K = K1 - 1
        assert x.shape == (b, K)
        n = np.zeros(b, np.int32)
        tok = np.zeros((b, K + 1), np.int32)
        am = np.zeros((b, K + 1), np.int32)
        rc = self.lib.oracle_greedy_accept(_ptr(target), _dtype_code(target), K1 * V, V,
                                           _ptr(x), b, K, V, _ptr(n), _ptr(tok), _ptr(am))
        if rc != 0:
            raise ValueError("oracle_greedy_accept rejected its arguments")
        return n, tok, am

    def sample_accept(self, target: np.ndarray, draft: np.ndarray, draft_tokens: np.ndarray,
                      temperature: float, seeds: np.ndarray) -> dict:
        """Speculative-sampling accept.

        target [b, K+1, V], draft [b, K, V] (same dtype), draft tokens [b, K],
        seeds [b] (uint64).  Returns a dict with n_accepted, tokens, p_draft,
        q_draft and the per-sequence diagnostics (ratios r, uniforms u, t, R,
        u2, residual flag).
        """
        target = np.ascontiguousarray(target)
        draft = np.ascontiguousarray(draft)
        x = np.ascontiguousarray(draft_tokens, dtype=np.int32)
        seeds = np.ascontiguousarray(seeds, dtype=np.uint64)
        b, K1, V = target.shape
        K = K1 - 1
        assert draft.shape == (b, K, V) and draft.dtype == target.dtype
        assert x.shape == (b, K) and seeds.shape == (b,)
        n = np.zeros(b, np.int32)
        tok = np.zeros((b, K + 1), np.int32)
        p = np.zeros((b, K), np.float64)
        q = np.zeros((b, K), np.float64)
        diag = np.zeros((b, 2 * K + 4), np.float64)
        rc = self.lib.oracle_sample_accept(_ptr(target), _ptr(draft), _dtype_code(target),
                                           K1 * V, V, K * V, V, _ptr(x), b, K, V,
                                           float(temperature), _ptr(seeds), _ptr(n), _ptr(tok),
                                           _ptr(p), _ptr(q), _ptr(diag))
        if rc != 0:
            raise ValueError("oracle_sample_accept rejected its arguments")
        return {
            "n_accepted": n, "tokens": tok, "p_draft": p, "q_draft": q,
            "r": diag[:, :K].copy(), "u": diag[:, K:2 * K].copy(),
            "t": diag[:, 2 * K].copy(), "R": diag[:, 2 * K + 1].copy(),
            "u2": diag[:, 2 * K + 2].copy(), "residual": diag[:, 2 * K + 3].copy(),
        }

    def mixed_accept(self, target: np.ndarray, draft: np.ndarray, draft_tokens: np.ndarray,
                     temperatures: np.ndarray, seeds: np.ndarray, draft_lengths=None) -> dict:
        """Mixed batch: greedy where temperatures[s] == 0, sampling at
        temperatures[s] > 0; sequence s uses draft_lengths[s] <= K draft
        tokens (all K when None).  Same outputs as sample_accept plus argmax."""
        target = np.ascontiguousarray(target)
        draft = np.ascontiguousarray(draft)
        x = np.ascontiguousarray(draft_tokens, dtype=np.int32)
        temps = np.ascontiguousarray(temperatures, dtype=np.float64)
        seeds = np.ascontiguousarray(seeds, dtype=np.uint64)
        b, K1, V = target.shape
        K = K1 - 1
        assert draft.shape == (b, K, V) and draft.dtype == target.dtype
        assert x.shape == (b, K) and seeds.shape == (b,) and temps.shape == (b,)
        n = np.zeros(b, np.int32)
        tok = np.zeros((b, K + 1), np.int32)
        p = np.zeros((b, K), np.float64)
        q = np.zeros((b, K), np.float64)
        am = np.zeros((b, K + 1), np.int32)
        diag = np.zeros((b, 2 * K + 4), np.float64)
        lens = None
        if draft_lengths is not None:
            lens = np.ascontiguousarray(draft_lengths, dtype=np.int32)
            assert lens.shape == (b,)
        rc = self.lib.oracle_mixed_accept(_ptr(target), _ptr(draft), _dtype_code(target),
                                          K1 * V, V, K * V, V, _ptr(x), b, K, V, _ptr(temps),
                                          _ptr(lens) if lens is not None else None,
                                          _ptr(seeds), _ptr(n), _ptr(tok), _ptr(p), _ptr(q),
                                          _ptr(am), _ptr(diag))
        if rc != 0:
            raise ValueError("oracle_mixed_accept rejected its arguments")
        return {
            "n_accepted": n, "tokens": tok, "p_draft": p, "q_draft": q, "argmax": am,
            "r": diag[:, :K].copy(), "u": diag[:, K:2 * K].copy(),
            "t": diag[:, 2 * K].copy(), "R": diag[:, 2 * K + 1].copy(),
            "u2": diag[:, 2 * K + 2].copy(), "residual": diag[:, 2 * K + 3].copy(),
        }

    def draw_cdf(self, target: np.ndarray, draft: np.ndarray, temperature: float, s: int,
                 slot: int, residual: bool) -> np.ndarray:
        """Running sums F_v of the oracle's draw weights for sequence s at `slot`."""
        target = np.ascontiguousarray(target)
        draft = np.ascontiguousarray(draft)
        b, K1, V = target.shape
        K = K1 - 1
        F = np.zeros(V, np.float64)
        rc = self.lib.oracle_draw_cdf(_ptr(target), _ptr(draft), _dtype_code(target),
                                      K1 * V, V, K * V, V, K, V, float(temperature),
                                      int(s), int(slot), int(bool(residual)), _ptr(F))
        if rc != 0:
            raise ValueError("oracle_draw_cdf rejected its arguments")
        return F


_default = None


def default() -> Oracle:
    """The regular (non-mutant) oracle build, compiled on first use if absent;
    SPEC_ORACLE_LIBRARY names another build of it (the sanitizer build)."""
    global _default
    if _default is None:
        _default = Oracle(os.environ.get("SPEC_ORACLE_LIBRARY") or _LIB)
    return _default


def philox4x32_10(counter, key):
    return default().philox4x32_10(counter, key)


def uniform(seed, row, pos, tag):
    return default().uniform(seed, row, pos, tag)


def row_log_normaliser(row, T):
    return default().row_log_normaliser(row, T)


def greedy_accept(target, draft_tokens):
    return default().greedy_accept(target, draft_tokens)


def sample_accept(target, draft, draft_tokens, temperature, seeds):
    return default().sample_accept(target, draft, draft_tokens, temperature, seeds)


def mixed_accept(target, draft, draft_tokens, temperatures, seeds, draft_lengths=None):
    return default().mixed_accept(target, draft, draft_tokens, temperatures, seeds, draft_lengths)


def draw_cdf(target, draft, temperature, s, slot, residual):
    return default().draw_cdf(target, draft, temperature, s, slot, residual)
