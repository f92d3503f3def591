"""Verify/accept for block speculative decoding on MI355X (gfx950).

Python binding of the C ABI in ``include/specverify.h``: argument marshalling
only.  Every step of the accept path runs in the HIP kernels of
``libspecverify.so``; PyTorch provides device memory and streams.

The names mirror the accept policy's exports on "dspark-mlx 0.1.0" wheel
diff, dspark_mlx/__init__.py: ``greedy_accept``,
``speculative_sample_accept`` and ``AcceptResult``.  Their input is the
target logit block [b, K+1, V] (row 0 = p_1 from the anchor step, rows
1..K = p_2..p_{K+1} from one verify forward, row K the bonus position; same
page, dspark_mlx/adapter.py, "Logit conventions"), the drafter's [b, K, V]
logits and its K tokens.  ``n_accepted`` is the ``n_keep`` that
``BaseModelAdapter.kv_rollback`` takes; the committed tokens are
``tokens[:, :n_accepted + 1]``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

__all__ = ["AcceptResult", "greedy_accept", "speculative_sample_accept", "mixed_accept",
           "mixed_accept_noalloc", "SCRATCH_BYTES",
           "fused_mixed_accept", "lm_head_logits", "fused_workspace_bytes",
           "sharded_mixed_accept", "sharded_workspace_bytes",
           "DraftBlock", "markov_block_decode", "markov_workspace_bytes",
           "workspace_bytes", "mixed_workspace_bytes",
           "set_stage_events", "stream_copy", "stream_read", "philox_uniforms", "library_path", "SpecError"]

_PKG = os.path.dirname(os.path.abspath(__file__))
# SPEC_LIBRARY names another build of the same library (the host-sanitizer
# build of _build.build(sanitize=True)); it must exist like the default one.
_LIB_PATH = os.environ.get("SPEC_LIBRARY") or os.path.join(_PKG, "libspecverify.so")

SPEC_F32 = 0
SPEC_BF16 = 1
SPEC_MAX_K = 32
SCRATCH_BYTES = 8 << 20        # SPEC_SCRATCH_BYTES: the fixed device scratch of mixed_accept_noalloc


class SpecError(RuntimeError):
    """A non-zero status from the C ABI."""


def library_path() -> str:
    return _LIB_PATH


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64, sz, dbl = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t,
                             ctypes.c_double)
    lib.spec_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.spec_workspace_bytes.restype = sz
    lib.spec_status_string.argtypes = [i32]
    lib.spec_status_string.restype = ctypes.c_char_p
    lib.spec_greedy_accept.argtypes = [vp, i32, i64, i64, vp, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.spec_greedy_accept.restype = i32
    lib.spec_sample_accept.argtypes = [vp, vp, i32, i64, i64, i64, i64, vp, i32, i32, i32, dbl, vp,
                                       vp, vp, vp, vp, vp, sz, vp]
    lib.spec_sample_accept.restype = i32
    lib.spec_mixed_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.spec_mixed_workspace_bytes.restype = sz
    lib.spec_mixed_accept.argtypes = [vp, vp, i32, i64, i64, i64, i64, vp, i32, i32, i32, vp, vp, vp,
                                      vp, vp, vp, vp, vp, vp, sz, vp]
    lib.spec_mixed_accept.restype = i32
    lib.spec_mixed_accept_noalloc.argtypes = [vp, vp, i32, i64, i64, i64, i64, vp, i32, i32, i32, vp, vp,
                                              vp, vp, vp, vp, vp, vp, vp]
    lib.spec_mixed_accept_noalloc.restype = i32
    f32 = ctypes.c_float
    lib.spec_fused_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.spec_fused_workspace_bytes.restype = sz
    lib.spec_fused_mixed_accept.argtypes = [vp, i64, i64, vp, i64, i32, f32, vp, i64, i64, vp, i32, i32,
                                            i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.spec_fused_mixed_accept.restype = i32
    lib.spec_lm_head_logits.argtypes = [vp, i64, i32, vp, i64, i32, i32, f32, vp, i64, vp]
    lib.spec_lm_head_logits.restype = i32
    lib.spec_sharded_workspace_bytes.argtypes = [i32, vp, i32, i32, i32]
    lib.spec_sharded_workspace_bytes.restype = sz
    lib.spec_sharded_mixed_accept.argtypes = [i32, vp, vp, vp, vp, vp, i32, vp, i32, i32, vp, vp, vp, vp, vp,
                                              vp, vp, vp, vp, sz, vp]
    lib.spec_sharded_mixed_accept.restype = i32
    lib.spec_markov_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.spec_markov_workspace_bytes.restype = sz
    lib.spec_markov_block_decode.argtypes = [vp, i64, i64, vp, vp, i64, vp, i64, i32, i32, i32, i32, vp, vp, vp, i64,
                                             i64, i32, vp, f32, f32, vp, vp, i64, i64, vp, vp, vp, sz, vp]
    lib.spec_markov_block_decode.restype = i32
    lib.spec_set_stage_events.argtypes = [vp, i32]
    lib.spec_set_stage_events.restype = i32
    lib.spec_stream_copy.argtypes = [vp, vp, sz, vp]
    lib.spec_stream_copy.restype = i32
    lib.spec_stream_read.argtypes = [vp, sz, vp, vp]
    lib.spec_stream_read.restype = i32
    lib.spec_philox_uniforms.argtypes = [ctypes.c_uint64, ctypes.c_uint32, i32, ctypes.c_uint32, i32,
                                         ctypes.c_uint32, vp, vp]
    lib.spec_philox_uniforms.restype = i32
    return lib


_lib = _load()


def _check(rc: int) -> None:
    if rc != 0:
        raise SpecError(f"status {rc}: {_lib.spec_status_string(rc).decode()}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SPEC_BF16
    if t.dtype == torch.float32:
        return SPEC_F32
    raise TypeError(f"logits must be bfloat16 or float32, got {t.dtype}")


def _stream_handle(device: torch.device, stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return int(s.cuda_stream)


def _on_gpu(*ts: torch.Tensor) -> None:
    for t in ts:
        if not t.is_cuda:
            raise ValueError("every tensor must live on the GPU")


@dataclass
class AcceptResult:
    """Result of one accept call (device tensors).

    n_accepted  [b] int32: accepted draft tokens (-1 for an invalid sequence)
    tokens      [b, K+1] int32: committed tokens, -1 after position n_accepted
    p_draft     [b, K] float32: p_i(x_i) of every slot (sampling rule)
    q_draft     [b, K] float32: q_i(x_i) of every slot (sampling rule)
    argmax      [b, K+1] int32: target argmax of every row (greedy rule)
    """
    n_accepted: torch.Tensor
    tokens: torch.Tensor
    p_draft: Optional[torch.Tensor] = None
    q_draft: Optional[torch.Tensor] = None
    argmax: Optional[torch.Tensor] = None


def workspace_bytes(b: int, K: int, V: int, dtype: torch.dtype, sampling: bool) -> int:
    code = SPEC_BF16 if dtype == torch.bfloat16 else SPEC_F32
    n = _lib.spec_workspace_bytes(b, K, V, code, int(bool(sampling)))
    if n == 0:
        raise ValueError(f"sizes out of range: b={b} K={K} V={V}")
    return n


def mixed_workspace_bytes(b: int, K: int, V: int, dtype: torch.dtype) -> int:
    code = SPEC_BF16 if dtype == torch.bfloat16 else SPEC_F32
    n = _lib.spec_mixed_workspace_bytes(b, K, V, code)
    if n == 0:
        raise ValueError(f"sizes out of range: b={b} K={K} V={V}")
    return n


def _workspace(ws: Optional[torch.Tensor], need: int, device) -> torch.Tensor:
    if ws is None:
        return torch.empty(need, dtype=torch.uint8, device=device)
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace holds {ws.numel() * ws.element_size()} bytes, needs {need}")
    return ws


def greedy_accept(target: torch.Tensor, draft_tokens: torch.Tensor, *, want_argmax: bool = True,
                  out: Optional[AcceptResult] = None, workspace: Optional[torch.Tensor] = None,
                  stream=None) -> AcceptResult:
    """Greedy accept of target [b, K+1, V] against draft tokens [b, K]."""
    _on_gpu(target, draft_tokens)
    if target.dim() != 3 or target.stride(2) != 1:
        raise ValueError("target must be [b, K+1, V] with V contiguous")
    b, K1, V = target.shape
    K = K1 - 1
    if draft_tokens.shape != (b, K) or draft_tokens.dtype != torch.int32 or not draft_tokens.is_contiguous():
        raise ValueError("draft_tokens must be a contiguous int32 [b, K] tensor")
    dev = target.device
    if out is None:
        out = AcceptResult(torch.empty(b, dtype=torch.int32, device=dev),
                           torch.empty(b, K1, dtype=torch.int32, device=dev),
                           argmax=torch.empty(b, K1, dtype=torch.int32, device=dev) if want_argmax else None)
    need = workspace_bytes(b, K, V, target.dtype, False)
    ws = _workspace(workspace, need, dev)
    rc = _lib.spec_greedy_accept(
        target.data_ptr(), _dtype_code(target), target.stride(0), target.stride(1),
        draft_tokens.data_ptr(), b, K, V, out.n_accepted.data_ptr(), out.tokens.data_ptr(),
        out.argmax.data_ptr() if out.argmax is not None else None,
        ws.data_ptr(), ws.numel() * ws.element_size(), _stream_handle(dev, stream))
    _check(rc)
    return out


def speculative_sample_accept(target: torch.Tensor, draft: torch.Tensor, draft_tokens: torch.Tensor,
                              temperature: float, seeds: torch.Tensor, *,
                              out: Optional[AcceptResult] = None,
                              workspace: Optional[torch.Tensor] = None, stream=None) -> AcceptResult:
    """Lossless speculative-sampling accept; temperature 0 falls back to greedy.

    seeds: [b] int64 or uint64 Philox keys (bit patterns are used as given).
    """
    if temperature == 0.0:
        return greedy_accept(target, draft_tokens, workspace=workspace, stream=stream)
    _on_gpu(target, draft, draft_tokens, seeds)
    if target.dim() != 3 or draft.dim() != 3 or target.stride(2) != 1 or draft.stride(2) != 1:
        raise ValueError("target [b, K+1, V] and draft [b, K, V] need V contiguous")
    b, K1, V = target.shape
    K = K1 - 1
    if draft.shape != (b, K, V) or draft.dtype != target.dtype:
        raise ValueError("draft must be [b, K, V] with the target's dtype")
    if draft_tokens.shape != (b, K) or draft_tokens.dtype != torch.int32 or not draft_tokens.is_contiguous():
        raise ValueError("draft_tokens must be a contiguous int32 [b, K] tensor")
    if seeds.shape != (b,) or seeds.element_size() != 8 or not seeds.is_contiguous():
        raise ValueError("seeds must be a contiguous 64-bit [b] tensor")
    dev = target.device
    if out is None:
        out = AcceptResult(torch.empty(b, dtype=torch.int32, device=dev),
                           torch.empty(b, K1, dtype=torch.int32, device=dev),
                           p_draft=torch.empty(b, K, dtype=torch.float32, device=dev),
                           q_draft=torch.empty(b, K, dtype=torch.float32, device=dev))
    need = workspace_bytes(b, K, V, target.dtype, True)
    ws = _workspace(workspace, need, dev)
    rc = _lib.spec_sample_accept(
        target.data_ptr(), draft.data_ptr(), _dtype_code(target), target.stride(0), target.stride(1),
        draft.stride(0), draft.stride(1), draft_tokens.data_ptr(), b, K, V, float(temperature),
        seeds.data_ptr(), out.n_accepted.data_ptr(), out.tokens.data_ptr(),
        out.p_draft.data_ptr() if out.p_draft is not None else None,
        out.q_draft.data_ptr() if out.q_draft is not None else None,
        ws.data_ptr(), ws.numel() * ws.element_size(), _stream_handle(dev, stream))
    _check(rc)
    return out


def mixed_accept(target: torch.Tensor, draft: torch.Tensor, draft_tokens: torch.Tensor,
                 temperatures: torch.Tensor, seeds: torch.Tensor, *,
                 draft_lengths: Optional[torch.Tensor] = None, out: Optional[AcceptResult] = None,
                 workspace: Optional[torch.Tensor] = None, stream=None) -> AcceptResult:
    """Mixed batch: sequence s is greedy when temperatures[s] == 0 and sampled
    at temperatures[s] otherwise (float64 device tensor [b]).  Philox rows are
    the sequences' indices in this batch.  draft_lengths (int32 device tensor
    [b], or None for all K): sequence s verifies only its first
    draft_lengths[s] draft tokens (0..K; anything else marks it invalid)."""
    _on_gpu(target, draft, draft_tokens, temperatures, seeds)
    if target.dim() != 3 or draft.dim() != 3 or target.stride(2) != 1 or draft.stride(2) != 1:
        raise ValueError("target [b, K+1, V] and draft [b, K, V] need V contiguous")
    b, K1, V = target.shape
    K = K1 - 1
    if draft.shape != (b, K, V) or draft.dtype != target.dtype:
        raise ValueError("draft must be [b, K, V] with the target's dtype")
    if draft_tokens.shape != (b, K) or draft_tokens.dtype != torch.int32 or not draft_tokens.is_contiguous():
        raise ValueError("draft_tokens must be a contiguous int32 [b, K] tensor")
    if temperatures.shape != (b,) or temperatures.dtype != torch.float64 or not temperatures.is_contiguous():
        raise ValueError("temperatures must be a contiguous float64 [b] tensor")
    if seeds.shape != (b,) or seeds.element_size() != 8 or not seeds.is_contiguous():
        raise ValueError("seeds must be a contiguous 64-bit [b] tensor")
    if draft_lengths is not None:
        _on_gpu(draft_lengths)
        if (draft_lengths.shape != (b,) or draft_lengths.dtype != torch.int32
                or not draft_lengths.is_contiguous()):
            raise ValueError("draft_lengths must be a contiguous int32 [b] tensor")
    dev = target.device
    if out is None:
        out = AcceptResult(torch.empty(b, dtype=torch.int32, device=dev),
                           torch.empty(b, K1, dtype=torch.int32, device=dev),
                           p_draft=torch.empty(b, K, dtype=torch.float32, device=dev),
                           q_draft=torch.empty(b, K, dtype=torch.float32, device=dev),
                           argmax=torch.empty(b, K1, dtype=torch.int32, device=dev))
    need = mixed_workspace_bytes(b, K, V, target.dtype)
    ws = _workspace(workspace, need, dev)
    rc = _lib.spec_mixed_accept(
        target.data_ptr(), draft.data_ptr(), _dtype_code(target), target.stride(0), target.stride(1),
        draft.stride(0), draft.stride(1), draft_tokens.data_ptr(), b, K, V, temperatures.data_ptr(),
        draft_lengths.data_ptr() if draft_lengths is not None else None,
        seeds.data_ptr(), out.n_accepted.data_ptr(), out.tokens.data_ptr(),
        out.p_draft.data_ptr() if out.p_draft is not None else None,
        out.q_draft.data_ptr() if out.q_draft is not None else None,
        out.argmax.data_ptr() if out.argmax is not None else None,
        ws.data_ptr(), ws.numel() * ws.element_size(), _stream_handle(dev, stream))
    _check(rc)
    return out


def mixed_accept_noalloc(target: torch.Tensor, draft: torch.Tensor, draft_tokens: torch.Tensor,
                         temperatures: torch.Tensor, seeds: torch.Tensor, *,
                         draft_lengths: Optional[torch.Tensor] = None, out: Optional[AcceptResult] = None,
                         stream=None) -> AcceptResult:
    """mixed_accept without a workspace: the C entry point runs in the
    library's fixed device scratch (SCRATCH_BYTES per GPU) and allocates
    nothing; pass `out` to keep this wrapper from allocating the results.
    Calls that overlap on one GPU race on that scratch."""
    _on_gpu(target, draft, draft_tokens, temperatures, seeds)
    if target.dim() != 3 or draft.dim() != 3 or target.stride(2) != 1 or draft.stride(2) != 1:
        raise ValueError("target [b, K+1, V] and draft [b, K, V] need V contiguous")
    b, K1, V = target.shape
    K = K1 - 1
    if draft.shape != (b, K, V) or draft.dtype != target.dtype:
        raise ValueError("draft must be [b, K, V] with the target's dtype")
    if draft_tokens.shape != (b, K) or draft_tokens.dtype != torch.int32 or not draft_tokens.is_contiguous():
        raise ValueError("draft_tokens must be a contiguous int32 [b, K] tensor")
    if temperatures.shape != (b,) or temperatures.dtype != torch.float64 or not temperatures.is_contiguous():
        raise ValueError("temperatures must be a contiguous float64 [b] tensor")
    if seeds.shape != (b,) or seeds.element_size() != 8 or not seeds.is_contiguous():
        raise ValueError("seeds must be a contiguous 64-bit [b] tensor")
    if draft_lengths is not None:
        _on_gpu(draft_lengths)
        if (draft_lengths.shape != (b,) or draft_lengths.dtype != torch.int32
                or not draft_lengths.is_contiguous()):
            raise ValueError("draft_lengths must be a contiguous int32 [b] tensor")
    dev = target.device
    if out is None:
        out = AcceptResult(torch.empty(b, dtype=torch.int32, device=dev),
                           torch.empty(b, K1, dtype=torch.int32, device=dev),
                           p_draft=torch.empty(b, K, dtype=torch.float32, device=dev),
                           q_draft=torch.empty(b, K, dtype=torch.float32, device=dev),
                           argmax=torch.empty(b, K1, dtype=torch.int32, device=dev))
    rc = _lib.spec_mixed_accept_noalloc(
        target.data_ptr(), draft.data_ptr(), _dtype_code(target), target.stride(0), target.stride(1),
        draft.stride(0), draft.stride(1), draft_tokens.data_ptr(), b, K, V, temperatures.data_ptr(),
        draft_lengths.data_ptr() if draft_lengths is not None else None,
        seeds.data_ptr(), out.n_accepted.data_ptr(), out.tokens.data_ptr(),
        out.p_draft.data_ptr() if out.p_draft is not None else None,
        out.q_draft.data_ptr() if out.q_draft is not None else None,
        out.argmax.data_ptr() if out.argmax is not None else None,
        _stream_handle(dev, stream))
    _check(rc)
    return out


def philox_uniforms(seed: int, row0: int, nrow: int, pos0: int, npos: int, tag: int, *, device="cuda",
                    stream=None) -> torch.Tensor:
    """U(seed, row0 + r, pos0 + p, tag) from the library's device Philox, as a
    float64 [nrow, npos] tensor (diagnostic: the uniforms the accept test and
    the draws take)."""
    dev = torch.device(device)
    out = torch.empty(nrow, npos, dtype=torch.float64, device=dev)
    _check(_lib.spec_philox_uniforms(int(seed) & (2 ** 64 - 1), int(row0) & 0xFFFFFFFF, int(nrow),
                                     int(pos0) & 0xFFFFFFFF, int(npos), int(tag) & 0xFFFFFFFF,
                                     out.data_ptr(), _stream_handle(dev, stream)))
    return out


def fused_workspace_bytes(b: int, K: int, V: int, D: int) -> int:
    n = _lib.spec_fused_workspace_bytes(b, K, V, D)
    if n == 0:
        raise ValueError(f"sizes out of range: b={b} K={K} V={V} D={D} (D a multiple of 64)")
    return n


def fused_mixed_accept(hidden: torch.Tensor, weight: torch.Tensor, draft: torch.Tensor,
                       draft_tokens: torch.Tensor, temperatures: torch.Tensor, seeds: torch.Tensor, *,
                       softcap: float = 0.0, draft_lengths: Optional[torch.Tensor] = None,
                       out: Optional[AcceptResult] = None, workspace: Optional[torch.Tensor] = None,
                       stream=None) -> AcceptResult:
    """Fused verify: target logits softcap(hidden @ weight.T) formed inside
    the call (bf16 hidden [b, K+1, D], bf16 weight [V, D]), then the mixed
    accept of mixed_accept with float32 drafter logits draft [b, K, V]."""
    _on_gpu(hidden, weight, draft, draft_tokens, temperatures, seeds)
    if hidden.dim() != 3 or hidden.dtype != torch.bfloat16 or hidden.stride(2) != 1:
        raise ValueError("hidden must be bf16 [b, K+1, D] with D contiguous")
    if weight.dim() != 2 or weight.dtype != torch.bfloat16 or weight.stride(1) != 1:
        raise ValueError("weight must be bf16 [V, D] with D contiguous")
    b, K1, D = hidden.shape
    K = K1 - 1
    V = weight.shape[0]
    if weight.shape[1] != D:
        raise ValueError("hidden and weight disagree on D")
    if draft.shape != (b, K, V) or draft.dtype != torch.float32 or draft.stride(2) != 1:
        raise ValueError("draft must be float32 [b, K, V] with V contiguous")
    if draft_tokens.shape != (b, K) or draft_tokens.dtype != torch.int32 or not draft_tokens.is_contiguous():
        raise ValueError("draft_tokens must be a contiguous int32 [b, K] tensor")
    if temperatures.shape != (b,) or temperatures.dtype != torch.float64 or not temperatures.is_contiguous():
        raise ValueError("temperatures must be a contiguous float64 [b] tensor")
    if seeds.shape != (b,) or seeds.element_size() != 8 or not seeds.is_contiguous():
        raise ValueError("seeds must be a contiguous 64-bit [b] tensor")
    if draft_lengths is not None:
        _on_gpu(draft_lengths)
        if (draft_lengths.shape != (b,) or draft_lengths.dtype != torch.int32
                or not draft_lengths.is_contiguous()):
            raise ValueError("draft_lengths must be a contiguous int32 [b] tensor")
    dev = hidden.device
    if out is None:
        out = AcceptResult(torch.empty(b, dtype=torch.int32, device=dev),
                           torch.empty(b, K1, dtype=torch.int32, device=dev),
                           p_draft=torch.empty(b, K, dtype=torch.float32, device=dev),
                           q_draft=torch.empty(b, K, dtype=torch.float32, device=dev),
                           argmax=torch.empty(b, K1, dtype=torch.int32, device=dev))
    ws = _workspace(workspace, fused_workspace_bytes(b, K, V, D), dev)
    rc = _lib.spec_fused_mixed_accept(
        hidden.data_ptr(), hidden.stride(0), hidden.stride(1), weight.data_ptr(), weight.stride(0), D,
        float(softcap), draft.data_ptr(), draft.stride(0), draft.stride(1), draft_tokens.data_ptr(), b, K, V,
        temperatures.data_ptr(), draft_lengths.data_ptr() if draft_lengths is not None else None,
        seeds.data_ptr(), out.n_accepted.data_ptr(), out.tokens.data_ptr(),
        out.p_draft.data_ptr() if out.p_draft is not None else None,
        out.q_draft.data_ptr() if out.q_draft is not None else None,
        out.argmax.data_ptr() if out.argmax is not None else None,
        ws.data_ptr(), ws.numel() * ws.element_size(), _stream_handle(dev, stream))
    _check(rc)
    return out


def lm_head_logits(hidden: torch.Tensor, weight: torch.Tensor, *, softcap: float = 0.0,
                   out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """float32 logits softcap(hidden @ weight.T) for bf16 hidden [rows, D] and
    weight [V, D]: the fused call's GEMM on its own.  Returns [rows, V] (a
    view of a buffer whose row stride is V rounded up to 4)."""
    _on_gpu(hidden, weight)
    if hidden.dim() != 2 or hidden.dtype != torch.bfloat16 or hidden.stride(1) != 1:
        raise ValueError("hidden must be bf16 [rows, D] with D contiguous")
    if weight.dim() != 2 or weight.dtype != torch.bfloat16 or weight.stride(1) != 1:
        raise ValueError("weight must be bf16 [V, D] with D contiguous")
    rows, D = hidden.shape
    V = weight.shape[0]
    if out is None:
        out = torch.empty(rows, (V + 3) // 4 * 4, dtype=torch.float32, device=hidden.device)[:, :V]
    if out.shape != (rows, V) or out.dtype != torch.float32 or out.stride(1) != 1:
        raise ValueError("out must be float32 [rows, V] with V contiguous")
    rc = _lib.spec_lm_head_logits(hidden.data_ptr(), hidden.stride(0), rows, weight.data_ptr(), weight.stride(0),
                                  V, D, float(softcap), out.data_ptr(), out.stride(0),
                                  _stream_handle(hidden.device, stream))
    _check(rc)
    return out


def sharded_workspace_bytes(shard_V: Sequence[int], b: int, K: int, dtype: torch.dtype) -> int:
    G = len(shard_V)
    arr = (ctypes.c_int * G)(*[int(v) for v in shard_V])
    code = SPEC_BF16 if dtype == torch.bfloat16 else SPEC_F32
    n = _lib.spec_sharded_workspace_bytes(G, ctypes.cast(arr, ctypes.c_void_p), b, K, code)
    if n == 0:
        raise ValueError(f"sizes out of range: G={G} b={b} K={K} widths={list(shard_V)}")
    return n


def sharded_mixed_accept(target_shards: Sequence[torch.Tensor], draft_shards: Sequence[torch.Tensor],
                         draft_tokens: torch.Tensor, temperatures: torch.Tensor, seeds: torch.Tensor, *,
                         draft_lengths: Optional[torch.Tensor] = None, out: Optional[AcceptResult] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None) -> AcceptResult:
    """Vocabulary-sharded mixed accept: shard g holds columns [col0_g,
    col0_g + V_g) of every target row ([b, K+1, V_g]) and draft row
    ([b, K, V_g]); the result is mixed_accept's on the concatenation."""
    G = len(target_shards)
    if G != len(draft_shards) or G < 1:
        raise ValueError("need as many draft shards as target shards, at least one")
    _on_gpu(*target_shards, *draft_shards, draft_tokens, temperatures, seeds)
    t0 = target_shards[0]
    b, K1 = t0.shape[0], t0.shape[1]
    K = K1 - 1
    widths = []
    for t, d in zip(target_shards, draft_shards):
        if t.dim() != 3 or d.dim() != 3 or t.stride(2) != 1 or d.stride(2) != 1:
            raise ValueError("each shard needs its columns contiguous")
        if t.shape[:2] != (b, K1) or d.shape != (b, K, t.shape[2]) or t.dtype != t0.dtype or d.dtype != t0.dtype:
            raise ValueError("shards must be [b, K+1, V_g] / [b, K, V_g] with one dtype")
        widths.append(int(t.shape[2]))
    if draft_tokens.shape != (b, K) or draft_tokens.dtype != torch.int32 or not draft_tokens.is_contiguous():
        raise ValueError("draft_tokens must be a contiguous int32 [b, K] tensor")
    if temperatures.shape != (b,) or temperatures.dtype != torch.float64 or not temperatures.is_contiguous():
        raise ValueError("temperatures must be a contiguous float64 [b] tensor")
    if seeds.shape != (b,) or seeds.element_size() != 8 or not seeds.is_contiguous():
        raise ValueError("seeds must be a contiguous 64-bit [b] tensor")
    if draft_lengths is not None:
        _on_gpu(draft_lengths)
        if (draft_lengths.shape != (b,) or draft_lengths.dtype != torch.int32
                or not draft_lengths.is_contiguous()):
            raise ValueError("draft_lengths must be a contiguous int32 [b] tensor")
    dev = t0.device
    if out is None:
        out = AcceptResult(torch.empty(b, dtype=torch.int32, device=dev),
                           torch.empty(b, K1, dtype=torch.int32, device=dev),
                           p_draft=torch.empty(b, K, dtype=torch.float32, device=dev),
                           q_draft=torch.empty(b, K, dtype=torch.float32, device=dev),
                           argmax=torch.empty(b, K1, dtype=torch.int32, device=dev))
    ws = _workspace(workspace, sharded_workspace_bytes(widths, b, K, t0.dtype), dev)
    tp = (ctypes.c_void_p * G)(*[t.data_ptr() for t in target_shards])
    dp = (ctypes.c_void_p * G)(*[d.data_ptr() for d in draft_shards])
    vw = (ctypes.c_int * G)(*widths)
    ts = (ctypes.c_int64 * (2 * G))(*[x for t in target_shards for x in (t.stride(0), t.stride(1))])
    ds = (ctypes.c_int64 * (2 * G))(*[x for d in draft_shards for x in (d.stride(0), d.stride(1))])
    rc = _lib.spec_sharded_mixed_accept(
        G, ctypes.cast(tp, ctypes.c_void_p), ctypes.cast(dp, ctypes.c_void_p), ctypes.cast(vw, ctypes.c_void_p),
        ctypes.cast(ts, ctypes.c_void_p), ctypes.cast(ds, ctypes.c_void_p), _dtype_code(t0),
        draft_tokens.data_ptr(), b, K, temperatures.data_ptr(),
        draft_lengths.data_ptr() if draft_lengths is not None else None, seeds.data_ptr(),
        out.n_accepted.data_ptr(), out.tokens.data_ptr(),
        out.p_draft.data_ptr() if out.p_draft is not None else None,
        out.q_draft.data_ptr() if out.q_draft is not None else None,
        out.argmax.data_ptr() if out.argmax is not None else None,
        ws.data_ptr(), ws.numel() * ws.element_size(), _stream_handle(dev, stream))
    _check(rc)
    return out


@dataclass
class DraftBlock:
    """Result of markov_block_decode (device tensors).

    tokens      [b, K] int32 draft tokens (-1 from the first invalid position on)
    logits      [b, K, V] float32 corrected draft logits q_i (the verify's draft block)
    confidence  [b, K] float32 confidence of each position, or None
    lengths     [b] int32 draft length from the confidence threshold, or None
    """
    tokens: torch.Tensor
    logits: torch.Tensor
    confidence: Optional[torch.Tensor] = None
    lengths: Optional[torch.Tensor] = None


def markov_workspace_bytes(b: int, K: int, V: int, r: int) -> int:
    n = _lib.spec_markov_workspace_bytes(b, K, V, r)
    if n == 0:
        raise ValueError(f"sizes out of range: b={b} K={K} V={V} r={r} (r a multiple of 64)")
    return n


def markov_block_decode(base: torch.Tensor, anchors: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor,
                        temperatures: torch.Tensor, seeds: torch.Tensor, *, hidden: Optional[torch.Tensor] = None,
                        conf_w: Optional[torch.Tensor] = None, conf_b: float = 0.0, threshold: float = 0.0,
                        out: Optional[DraftBlock] = None, workspace: Optional[torch.Tensor] = None,
                        stream=None) -> DraftBlock:
    """Draft-side block decode with the Markov head: q_i = base_i + W2 W1[x_{i-1}]
    (x_{-1} = anchor), x_i = argmax q_i (temperature 0) or a draw from
    softmax(q_i / T); base float32 [b, K, V], w1 and w2 bf16 [V, r].  With
    hidden [b, K, D] and conf_w [D + r] (bf16) also the confidence
    sigmoid(conf_w . [h_i ; W1[x_{i-1}]] + conf_b) and the draft length."""
    _on_gpu(base, anchors, w1, w2, temperatures, seeds)
    if base.dim() != 3 or base.dtype != torch.float32 or base.stride(2) != 1:
        raise ValueError("base must be float32 [b, K, V] with V contiguous")
    b, K, V = base.shape
    if w1.dim() != 2 or w1.dtype != torch.bfloat16 or w1.stride(1) != 1 or w1.shape[0] != V:
        raise ValueError("w1 must be bf16 [V, r] with r contiguous")
    r = w1.shape[1]
    if w2.shape != (V, r) or w2.dtype != torch.bfloat16 or w2.stride(1) != 1:
        raise ValueError("w2 must be bf16 [V, r] with r contiguous")
    if anchors.shape != (b,) or anchors.dtype != torch.int32 or not anchors.is_contiguous():
        raise ValueError("anchors must be a contiguous int32 [b] tensor")
    if temperatures.shape != (b,) or temperatures.dtype != torch.float64 or not temperatures.is_contiguous():
        raise ValueError("temperatures must be a contiguous float64 [b] tensor")
    if seeds.shape != (b,) or seeds.element_size() != 8 or not seeds.is_contiguous():
        raise ValueError("seeds must be a contiguous 64-bit [b] tensor")
    want_conf = hidden is not None and conf_w is not None
    D = 0
    if want_conf:
        _on_gpu(hidden, conf_w)
        if hidden.dim() != 3 or hidden.shape[:2] != (b, K) or hidden.dtype != torch.bfloat16 or hidden.stride(2) != 1:
            raise ValueError("hidden must be bf16 [b, K, D] with D contiguous")
        D = hidden.shape[2]
        if conf_w.shape != (D + r,) or conf_w.dtype != torch.bfloat16 or not conf_w.is_contiguous():
            raise ValueError("conf_w must be a contiguous bf16 [D + r] tensor")
    dev = base.device
    if out is None:
        out = DraftBlock(torch.empty(b, K, dtype=torch.int32, device=dev),
                         torch.empty(b, K, (V + 3) // 4 * 4, dtype=torch.float32, device=dev)[:, :, :V],
                         torch.empty(b, K, dtype=torch.float32, device=dev) if want_conf else None,
                         torch.empty(b, dtype=torch.int32, device=dev) if want_conf else None)
    ws = _workspace(workspace, markov_workspace_bytes(b, K, V, r), dev)
    q = out.logits
    rc = _lib.spec_markov_block_decode(
        base.data_ptr(), base.stride(0), base.stride(1), anchors.data_ptr(), w1.data_ptr(), w1.stride(0),
        w2.data_ptr(), w2.stride(0), r, b, K, V, temperatures.data_ptr(), seeds.data_ptr(),
        hidden.data_ptr() if want_conf else None, hidden.stride(0) if want_conf else 0,
        hidden.stride(1) if want_conf else 0, D, conf_w.data_ptr() if want_conf else None, float(conf_b),
        float(threshold), out.tokens.data_ptr(), q.data_ptr(), q.stride(0), q.stride(1),
        out.confidence.data_ptr() if out.confidence is not None else None,
        out.lengths.data_ptr() if out.lengths is not None else None,
        ws.data_ptr(), ws.numel() * ws.element_size(), _stream_handle(dev, stream))
    _check(rc)
    return out


_stage_keepalive = None


def set_stage_events(events: Optional[Sequence[torch.cuda.Event]]) -> None:
    """Register torch CUDA events as the calling thread's stage markers (see
    spec_set_stage_events); None unregisters.  Events must already exist on
    the device (record them once, or create them with enable_timing=True and
    call .record() beforehand)."""
    global _stage_keepalive
    if not events:
        _stage_keepalive = None
        _check(_lib.spec_set_stage_events(None, 0))
        return
    arr = (ctypes.c_void_p * len(events))(*[int(e.cuda_event) for e in events])
    _stage_keepalive = (arr, list(events))
    _check(_lib.spec_set_stage_events(ctypes.cast(arr, ctypes.c_void_p), len(events)))


def stream_read(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Read-only stream over src with the row pass's load shape (bandwidth
    ceiling); sink is a device int32 tensor the kernel may write."""
    _on_gpu(src, sink)
    if sink.dtype != torch.int32 or sink.numel() < 1:
        raise ValueError("sink must be a device int32 tensor")
    n = src.numel() * src.element_size()
    _check(_lib.spec_stream_read(src.data_ptr(), n, sink.data_ptr(), _stream_handle(src.device, stream)))


def stream_copy(dst: torch.Tensor, src: torch.Tensor, stream=None) -> None:
    """Device copy through the library's 16-byte streaming kernel."""
    _on_gpu(dst, src)
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n:
        raise ValueError("dst smaller than src")
    _check(_lib.spec_stream_copy(dst.data_ptr(), src.data_ptr(), n, _stream_handle(src.device, stream)))
