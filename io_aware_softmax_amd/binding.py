"""ctypes binding of libattn.so with the C ABI's names (argument marshalling only).

Every computation runs in the library's HIP kernels.  PyTorch supplies device
memory and the current HIP stream; nothing here computes attention, and there
is no fallback: if the library is missing, every call raises
``AttnLibraryMissing``.
"""

from __future__ import annotations

import ctypes
import math
import os
import threading
from pathlib import Path
from typing import Optional, Tuple

import torch

# IO_AWARE_SOFTMAX_LIB names another build of the same library (the CPU
# tests run the host-sanitized build this way); by default the in-tree one.
LIB_PATH = Path(os.environ.get("IO_AWARE_SOFTMAX_LIB") or (Path(__file__).resolve().parent / "libattn.so"))

ATTN_F32, ATTN_F16, ATTN_BF16 = 0, 1, 2
ATTN_MAX_SPLITS = 256
ATTN_NOALLOC_SCRATCH_BYTES = 16 << 20
_DTYPE_CODES = {torch.float32: ATTN_F32, torch.float16: ATTN_F16, torch.bfloat16: ATTN_BF16}
EXPORTED = ("attn_fwd", "attn_decode_fwd", "attn_decode_fwd_noalloc", "attn_decode_varlen_fwd", "attn_bwd", "attn_fwd_ex", "attn_bwd_ex",
            "attn_decode_auto_splits", "attn_prefill_split_plan", "attn_strerror")
ATTN_MASK_NONE, ATTN_MASK_BOOL, ATTN_MASK_ADD = 0, 1, 2

_lock = threading.Lock()
_lib: Optional[ctypes.CDLL] = None


class AttnLibraryMissing(RuntimeError):
    """libattn.so has not been built (run ``__graft_entry__.build()``)."""


class AttnError(RuntimeError):
    """A negative status from the C ABI."""

    def __init__(self, status: int, message: str):
        super().__init__(f"attn status {status}: {message}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libattn.so once and declare the C signatures."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not LIB_PATH.exists():
            raise AttnLibraryMissing(
                f"{LIB_PATH} not found; build it with `python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(str(LIB_PATH))
        vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, i]
        lib.attn_fwd.restype = i
        lib.attn_decode_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i]
        lib.attn_decode_fwd.restype = i
        lib.attn_decode_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i]
        lib.attn_decode_fwd_noalloc.restype = i
        lib.attn_decode_varlen_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i]
        lib.attn_decode_varlen_fwd.restype = i
        lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, i]
        lib.attn_bwd.restype = i
        u64, u32 = ctypes.c_ulonglong, ctypes.c_uint
        lib.attn_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, i, i, i, f, u64, u32, vp, i]
        lib.attn_fwd_ex.restype = i
        lib.attn_bwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, i, i, i, f, u64, u32,
                                    vp, i]
        lib.attn_bwd_ex.restype = i
        lib.attn_decode_auto_splits.argtypes = [i, i, i, i]
        lib.attn_decode_auto_splits.restype = i
        ip = ctypes.POINTER(ctypes.c_int)
        lib.attn_prefill_split_plan.argtypes = [i, i, i, i, i, i, i, ip, ip]
        lib.attn_prefill_split_plan.restype = i
        lib.attn_strerror.argtypes = [i]
        lib.attn_strerror.restype = ctypes.c_char_p
        _lib = lib
        return lib


def attn_strerror(status: int) -> str:
    return load().attn_strerror(int(status)).decode()


def attn_prefill_split_plan(B: int, H: int, Lq: int, Lk: int, causal: bool, num_cus: int, forced: int = 0):
    """Key ranges per 256-row query tile that attn_fwd uses for this prefill
    on a device with num_cus compute units, and the work items per
    (batch, head).  Host arithmetic only."""
    nqt = (max(Lq, 1) + 255) // 256
    ranges = (ctypes.c_int * nqt)()
    items = ctypes.c_int()
    _check(load().attn_prefill_split_plan(int(B), int(H), int(Lq), int(Lk), int(bool(causal)), int(num_cus),
                                          int(forced), ranges, ctypes.byref(items)))
    return list(ranges), items.value


def _check(status: int) -> None:
    if status != 0:
        raise AttnError(status, attn_strerror(status))


def _stream_handle(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _is_tensor(t) -> bool:
    return isinstance(t, torch.Tensor)


def _dims(q):
    """(B, H, Lq, D) of q, which must be a 4-d tensor."""
    if not _is_tensor(q) or q.dim() != 4:
        raise ValueError("q must be a [B, H, L, D] tensor")
    return tuple(q.shape)


def _keys(k):
    """Lk of k, which must be a 4-d tensor."""
    if not _is_tensor(k) or k.dim() != 4:
        raise ValueError("k must be a [B, H, L, D] tensor")
    return k.shape[2]


def _prep(q, k, v, out, lse, Lq, place=True):
    """Check q, k, v (and a caller's out / lse) against the shapes the C ABI
    takes from q.shape and k.shape: the kernels trust those sizes, so any
    mismatch here would become an out-of-bounds access on the device.
    Structure (shape, dtype, layout) is checked before placement so the
    messages name the first real problem; place=False leaves the device
    check to the caller (which checks more tensors first).  Returns
    (out, lse), allocated when not given (place=True only)."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not _is_tensor(t):
            raise ValueError(f"{name} must be a torch tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, L, D]")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dtype not in _DTYPE_CODES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one of float32, float16, bfloat16")
    B, H, Lq_q, D = q.shape
    if Lq_q != Lq:
        raise ValueError(f"q must have {Lq} queries per (batch, head)")
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != D:
        raise ValueError("k must be [B, H, Lk, D] with q's B, H and D")
    if v.shape != k.shape:
        raise ValueError("v must have the shape of k")
    if out is not None:
        if not _is_tensor(out) or tuple(out.shape) != (B, H, Lq, D) or out.dtype != q.dtype:
            raise ValueError("out must be [B, H, Lq, D] with q's dtype")
        if not out.is_contiguous():
            raise ValueError("out must be contiguous")
    if lse is not None:
        if not _is_tensor(lse) or tuple(lse.shape) != (B, H, Lq) or lse.dtype != torch.float32:
            raise ValueError("lse must be a float32 tensor [B, H, Lq]")
        if not lse.is_contiguous():
            raise ValueError("lse must be contiguous")
    if not place:
        return out, lse
    _same_gpu(q, ("k", k), ("v", v), ("out", out), ("lse", lse))
    if out is None:
        out = torch.empty((B, H, Lq, D), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device)
    return out, lse


def _same_gpu(q, *named):
    """q is a GPU tensor and every other (non-None) tensor is on q's device."""
    if not q.is_cuda:
        raise ValueError("q must be a GPU tensor")
    for name, t in named:
        if t is not None and t.device != q.device:
            raise ValueError(f"{name} must be a GPU tensor on q's device ({q.device})")


def _bwd_prep(q, k, v, out, lse, dout, dq, dk, dv):
    """Checks of the backward entry points (beyond _prep's): out and dout
    shaped and typed like q, lse [B, H, Lq] float32, and caller-supplied
    gradients shaped and typed like their inputs, all on q's device.
    Returns (dq, dk, dv), allocated when not given."""
    _prep(q, k, v, out, lse, _dims(q)[2], place=False)
    if out is None or lse is None:
        raise ValueError("out and lse (the forward's outputs) are required")
    if not _is_tensor(dout) or dout.shape != q.shape or dout.dtype != q.dtype:
        raise ValueError("dout must be shaped and typed like q")
    if not dout.is_contiguous():
        raise ValueError("dout must be contiguous")
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t is None:
            continue
        if not _is_tensor(t) or t.shape != ref.shape or t.dtype != ref.dtype or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor shaped and typed like its input")
    _same_gpu(q, ("k", k), ("v", v), ("out", out), ("lse", lse), ("dout", dout), ("dq", dq), ("dk", dk),
              ("dv", dv))
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    return dq, dk, dv


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
             scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
             lse: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """O, LSE = attention(q, k, v) through ``attn_fwd`` of the C ABI.

    q [B,H,Lq,D], k and v [B,H,Lk,D], contiguous, on the GPU.  Returns the
    output [B,H,Lq,D] (dtype of q) and the log-sum-exp [B,H,Lq] (float32).
    ``scale`` defaults to 1/sqrt(D).  Asynchronous on ``stream`` (default:
    torch's current stream).
    """
    lib = load()
    B, H, Lq, D = _dims(q)
    Lk = _keys(k)
    out, lse = _prep(q, k, v, out, lse, Lq)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                        B, H, Lq, Lk, D, int(bool(causal)), scale, _stream_handle(stream),
                        _DTYPE_CODES[q.dtype]))
    return out, lse


def attn_decode_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: Optional[float] = None,
                    num_splits: int = 0, out: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Split-KV single-query attention through ``attn_decode_fwd``.

    q [B,H,1,D]; ``num_splits`` 0 lets the library choose.
    """
    lib = load()
    B, H, Lq, D = _dims(q)
    if Lq != 1:
        raise ValueError("attn_decode_fwd takes one query per (batch, head)")
    Lk = _keys(k)
    out, lse = _prep(q, k, v, out, lse, 1)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib.attn_decode_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                               lse.data_ptr(), B, H, Lk, D, scale, int(num_splits),
                               _stream_handle(stream), _DTYPE_CODES[q.dtype]))
    return out, lse


def attn_decode_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                            lse: torch.Tensor, scale: Optional[float] = None, num_splits: int = 0,
                            stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """``attn_decode_fwd_noalloc``: the split-KV decode with its partials in
    the library's fixed device scratch (no allocation in the library).

    The caller passes ``out`` [B,H,1,D] and ``lse`` [B,H,1] (nothing is
    allocated here either).  Same results as ``attn_decode_fwd`` with the
    same ``num_splits``.
    """
    lib = load()
    B, H, Lq, D = _dims(q)
    if Lq != 1:
        raise ValueError("attn_decode_fwd_noalloc takes one query per (batch, head)")
    if out is None or lse is None:
        raise ValueError("out and lse are required (this entry point allocates nothing)")
    Lk = _keys(k)
    out, lse = _prep(q, k, v, out, lse, 1)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib.attn_decode_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                       lse.data_ptr(), B, H, Lk, D, scale, int(num_splits),
                                       _stream_handle(stream), _DTYPE_CODES[q.dtype]))
    return out, lse


def attn_decode_varlen_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seqlens: torch.Tensor,
                           scale: Optional[float] = None, num_splits: int = 0,
                           out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                           stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Single-query attention over a KV cache with per-sequence lengths,
    through ``attn_decode_varlen_fwd``.

    q [B,H,1,D]; k and v [B,H,Lk_max,D]; seqlens an int32 GPU tensor [B]
    (each clamped to [0, Lk_max] by the library).
    """
    lib = load()
    B, H, Lq, D = _dims(q)
    if Lq != 1:
        raise ValueError("attn_decode_varlen_fwd takes one query per (batch, head)")
    if (not _is_tensor(seqlens) or seqlens.dtype != torch.int32 or tuple(seqlens.shape) != (B,)
            or not seqlens.is_contiguous()):
        raise ValueError("seqlens must be a contiguous int32 tensor of shape [B]")
    Lk = _keys(k)
    out, lse = _prep(q, k, v, out, lse, 1)
    _same_gpu(q, ("seqlens", seqlens))
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib.attn_decode_varlen_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                      lse.data_ptr(), seqlens.data_ptr(), B, H, Lk, D, scale,
                                      int(num_splits), _stream_handle(stream), _DTYPE_CODES[q.dtype]))
    return out, lse


def attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, lse: torch.Tensor,
             dout: torch.Tensor, causal: bool = False, scale: Optional[float] = None,
             dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
             dv: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """dq, dk, dv of attention through ``attn_bwd``.

    ``out`` and ``lse`` are what ``attn_fwd`` returned for the same q, k, v,
    causal and scale; ``dout`` is the gradient of the loss with respect to
    ``out`` (same shape and dtype).  float16 / bfloat16 only.
    """
    lib = load()
    dq, dk, dv = _bwd_prep(q, k, v, out, lse, dout, dq, dk, dv)
    B, H, Lq, D = _dims(q)
    Lk = _keys(k)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
                        lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Lq, Lk, D,
                        int(bool(causal)), scale, _stream_handle(stream), _DTYPE_CODES[q.dtype]))
    return dq, dk, dv


def _mask_args(mask, q, B, H, Lq, Lk):
    """(pointer, kind, mask_b, mask_h) of an optional mask tensor: bool or
    uint8 -> boolean mask, float32 -> additive mask; shape [1|B, 1|H, Lq, Lk]
    on q's device."""
    if mask is None:
        return None, ATTN_MASK_NONE, 1, 1
    if not _is_tensor(mask) or not mask.is_contiguous() or mask.dim() != 4:
        raise ValueError("mask must be a contiguous 4-d tensor")
    if mask.dtype in (torch.bool, torch.uint8):
        kind = ATTN_MASK_BOOL
    elif mask.dtype == torch.float32:
        kind = ATTN_MASK_ADD
    else:
        raise ValueError("mask dtype must be bool, uint8 (keep / drop) or float32 (additive)")
    mb, mh, mq, mk = mask.shape
    if mq != Lq or mk != Lk or mb not in (1, B) or mh not in (1, H):
        raise ValueError("mask must be [1 or B, 1 or H, Lq, Lk]")
    _same_gpu(q, ("mask", mask))
    return mask.data_ptr(), kind, mb, mh


def attn_fwd_ex(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                scale: Optional[float] = None, mask: Optional[torch.Tensor] = None, dropout_p: float = 0.0,
                seed: int = 0, offset: int = 0, out: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Attention with a general mask and dropout through ``attn_fwd_ex``.

    mask: None, a bool / uint8 tensor (nonzero = attend) or a float32 tensor
    added to the scaled scores, shaped [1 or B, 1 or H, Lq, Lk].  dropout_p
    in [0, 1) with the Philox key ``seed`` (64-bit) and counter word
    ``offset`` (32-bit).  float16 / bfloat16 only.
    """
    lib = load()
    B, H, Lq, D = _dims(q)
    Lk = _keys(k)
    _prep(q, k, v, out, lse, Lq, place=False)
    mp, kind, mb, mh = _mask_args(mask, q, B, H, Lq, Lk)
    out, lse = _prep(q, k, v, out, lse, Lq)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib.attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, Lq, Lk,
                           D, int(bool(causal)), scale, mp, kind, mb, mh, float(dropout_p), int(seed), int(offset),
                           _stream_handle(stream), _DTYPE_CODES[q.dtype]))
    return out, lse


def attn_bwd_ex(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, lse: torch.Tensor,
                dout: torch.Tensor, causal: bool = False, scale: Optional[float] = None,
                mask: Optional[torch.Tensor] = None, dropout_p: float = 0.0, seed: int = 0, offset: int = 0,
                dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                dv: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """dq, dk, dv of ``attn_fwd_ex`` (same mask and dropout arguments)."""
    lib = load()
    dq, dk, dv = _bwd_prep(q, k, v, out, lse, dout, dq, dk, dv)
    B, H, Lq, D = _dims(q)
    Lk = _keys(k)
    mp, kind, mb, mh = _mask_args(mask, q, B, H, Lq, Lk)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib.attn_bwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
                           lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Lq, Lk, D,
                           int(bool(causal)), scale, mp, kind, mb, mh, float(dropout_p), int(seed), int(offset),
                           _stream_handle(stream), _DTYPE_CODES[q.dtype]))
    return dq, dk, dv


def attn_decode_auto_splits(B: int, H: int, Lk: int, D: int) -> int:
    s = load().attn_decode_auto_splits(B, H, Lk, D)
    _check(min(s, 0))
    return s


def raw_attn_fwd(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, B: int, H: int,
                 Lq: int, Lk: int, D: int, causal: int, scale: float, stream: int, dtype: int) -> int:
    """The C entry point with plain integers for pointers; returns the status."""
    return load().attn_fwd(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, Lq, Lk, D, causal, scale,
                           stream, dtype)


def raw_attn_decode_fwd(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, B: int, H: int,
                        Lk: int, D: int, scale: float, num_splits: int, stream: int, dtype: int) -> int:
    return load().attn_decode_fwd(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, Lk, D, scale, num_splits,
                                  stream, dtype)


def library_loaded_path() -> str:
    """Absolute path of the loaded library (for provenance checks)."""
    load()
    return os.fspath(LIB_PATH)
