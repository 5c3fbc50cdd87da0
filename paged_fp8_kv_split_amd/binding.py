"""ctypes binding of ``libpfkv.so``: argument marshalling only.

Every step of the computation runs in the HIP kernels behind the C ABI declared
in ``include/pfkv.h``; torch is used here for device memory (``out`` and the
workspace) and for the current stream. There is no fallback: if the library is
not built, or a call fails, a Python exception is raised.

The call mirrors ``mtp_verify_attn_fwd_asm(q, k_cache, v_cache, block_tables,
seq_lens, cu_seqlens_q, k_descale, v_descale, softmax_scale, num_segments=None,
out=None)`` of aiter PR #5190 ("gfx950 assembly MTP-verify attention for head_dim
256 fp8 paged KV"), section Modifications.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libpfkv.so"
_lib = None

STATUS_NAMES = {0: "OK", 1: "INVALID", 2: "UNSUPPORTED", 3: "DEVICE", 4: "LAUNCH"}


class PfkvError(RuntimeError):
    """A non-zero status from the library; ``status`` holds the code."""

    def __init__(self, status: int, message: str):
        super().__init__(f"pfkv {STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class PfkvPrefillArgs(ctypes.Structure):
    """Mirror of ``pfkv_prefill_args`` in include/pfkv_prefill.h (same field order and types)."""

    _fields_ = [
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("cu_seqlens_q", ctypes.c_void_p),
        ("cu_seqlens_k", ctypes.c_void_p),
        ("q_descale", ctypes.c_void_p),
        ("k_descale", ctypes.c_void_p),
        ("v_descale", ctypes.c_void_p),
        ("q_stride_token", ctypes.c_int64),
        ("q_stride_head", ctypes.c_int64),
        ("k_stride_token", ctypes.c_int64),
        ("k_stride_head", ctypes.c_int64),
        ("v_stride_token", ctypes.c_int64),
        ("v_stride_head", ctypes.c_int64),
        ("out_stride_token", ctypes.c_int64),
        ("out_stride_head", ctypes.c_int64),
        ("num_seqs", ctypes.c_int32),
        ("total_q", ctypes.c_int32),
        ("total_k", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim_qk", ctypes.c_int32),
        ("head_dim_v", ctypes.c_int32),
        ("max_seqlen_q", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("causal", ctypes.c_int32),
    ]


class PfkvArgs(ctypes.Structure):
    """Mirror of ``pfkv_args`` in include/pfkv.h (same field order and types)."""

    _fields_ = [
        ("q", ctypes.c_void_p),
        ("k_cache", ctypes.c_void_p),
        ("v_cache", ctypes.c_void_p),
        ("block_tables", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("cu_seqlens_q", ctypes.c_void_p),
        ("k_descale", ctypes.c_void_p),
        ("v_descale", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("q_stride_token", ctypes.c_int64),
        ("q_stride_head", ctypes.c_int64),
        ("out_stride_token", ctypes.c_int64),
        ("out_stride_head", ctypes.c_int64),
        ("block_table_stride", ctypes.c_int64),
        ("workspace_size", ctypes.c_uint64),
        ("num_seqs", ctypes.c_int32),
        ("total_q", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("num_segments", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("precision", ctypes.c_int32),
        ("lse", ctypes.c_void_p),
        ("sinks", ctypes.c_void_p),
        ("window_keys", ctypes.c_int32),
        ("softcap", ctypes.c_float),
        ("max_q_len", ctypes.c_int32),
        ("balance_segments", ctypes.c_int32),
        ("merge_sync", ctypes.c_void_p),
        ("merge_sync_size", ctypes.c_uint64),
        ("merge_wait_us", ctypes.c_int32),
    ]


def library_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def load_library():
    """Load ``libpfkv.so`` once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
                           "from the repository root")
    lib = ctypes.CDLL(path)
    lib.pfkv_check_args.argtypes = [ctypes.POINTER(PfkvArgs), ctypes.c_char_p, ctypes.c_int]
    lib.pfkv_check_args.restype = ctypes.c_int
    lib.pfkv_verify_attn_fwd.argtypes = [ctypes.POINTER(PfkvArgs), ctypes.c_void_p]
    lib.pfkv_verify_attn_fwd.restype = ctypes.c_int
    lib.pfkv_verify_attn_fwd_noalloc.argtypes = [ctypes.POINTER(PfkvArgs), ctypes.c_void_p]
    lib.pfkv_verify_attn_fwd_noalloc.restype = ctypes.c_int
    for name in ("pfkv_splitkv_main", "pfkv_segment_reduce"):
        getattr(lib, name).argtypes = [ctypes.POINTER(PfkvArgs), ctypes.c_void_p]
        getattr(lib, name).restype = ctypes.c_int
    lib.pfkv_num_segments.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.pfkv_num_segments.restype = ctypes.c_int
    lib.pfkv_workspace_bytes.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.pfkv_workspace_bytes.restype = ctypes.c_uint64
    lib.pfkv_merge_sync_bytes.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.pfkv_partials_row_major.argtypes = [ctypes.c_int] * 4
    lib.pfkv_partials_row_major.restype = ctypes.c_int
    lib.pfkv_merge_sync_bytes.restype = ctypes.c_uint64
    lib.pfkv_last_error.argtypes = []
    lib.pfkv_last_error.restype = ctypes.c_char_p
    lib.pfkv_device_info.argtypes = [ctypes.c_int, ctypes.c_char_p, ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    lib.pfkv_device_info.restype = ctypes.c_int
    lib.pfkv_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p,
                                     ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    lib.pfkv_stream_read.restype = ctypes.c_int
    lib.pfkv_set_debug.argtypes = [ctypes.c_int]
    lib.pfkv_set_debug.restype = ctypes.c_int
    lib.pfkv_prefill_check_args.argtypes = [ctypes.POINTER(PfkvPrefillArgs), ctypes.c_char_p, ctypes.c_int]
    lib.pfkv_prefill_check_args.restype = ctypes.c_int
    lib.pfkv_prefill_fwd.argtypes = [ctypes.POINTER(PfkvPrefillArgs), ctypes.c_void_p]
    lib.pfkv_prefill_fwd.restype = ctypes.c_int
    _lib = lib
    return lib


def set_debug(on: bool) -> bool:
    """Switch the library's debug mode (a device-side precondition check before
    every launch; synchronizing, not for graph capture). Returns the previous setting."""
    return bool(load_library().pfkv_set_debug(1 if on else 0))


def _raise_on(status: int):
    if status != 0:
        msg = load_library().pfkv_last_error()
        raise PfkvError(status, msg.decode() if msg else "")


def last_error() -> str:
    msg = load_library().pfkv_last_error()
    return msg.decode() if msg else ""


def device_info(device: Optional[int] = None):
    """(gcnArchName, CU count) of a HIP device as the library sees it."""
    if device is None:
        device = torch.cuda.current_device()
    buf = ctypes.create_string_buffer(128)
    cus = ctypes.c_int(0)
    _raise_on(load_library().pfkv_device_info(int(device), buf, 128, ctypes.byref(cus)))
    return buf.value.decode(), cus.value


def num_segments(num_cus: int, num_seqs: int, num_kv_heads: int) -> int:
    """The library's segment-count heuristic (one work-group per CU)."""
    return int(load_library().pfkv_num_segments(int(num_cus), int(num_seqs), int(num_kv_heads)))


def workspace_bytes(num_segments_: int, total_q: int, num_q_heads: int) -> int:
    return int(load_library().pfkv_workspace_bytes(int(num_segments_), int(total_q), int(num_q_heads)))


def partials_row_major(precision: int, head_dim: int, page_size: int, num_segments_: int) -> bool:
    """Whether a call with these arguments leaves its workspace partials
    row-major ([T][Hq][S][...]) rather than segment-major ([S][T][Hq][...])."""
    return bool(load_library().pfkv_partials_row_major(int(precision), int(head_dim), int(page_size),
                                                       int(num_segments_)))


def merge_sync_bytes(num_seqs: int, num_q_heads: int) -> int:
    return int(load_library().pfkv_merge_sync_bytes(int(num_seqs), int(num_q_heads)))


def merge_sync_buffer(num_seqs: int, num_q_heads: int, device) -> torch.Tensor:
    """Zeroed sync words for the in-launch merge (``merge_sync=`` of
    :func:`verify_attn`), for calls of up to ``num_seqs`` sequences and
    ``num_q_heads`` query heads. Keep it and pass it to every call on one
    stream: each call leaves it ready for the next."""
    return torch.zeros(max(merge_sync_bytes(num_seqs, num_q_heads), 256), dtype=torch.uint8, device=device)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _as_bytes(cache: torch.Tensor) -> torch.Tensor:
    if cache.dtype == torch.float8_e4m3fn:
        return cache.view(torch.uint8)
    if cache.dtype != torch.uint8:
        raise TypeError(f"KV cache must be float8_e4m3fn or uint8 codes, got {cache.dtype}")
    return cache


PRECISION_16BIT = 0   # bf16 Q x exact-bf16 K, fp16 P x exact-fp16 V (default)
PRECISION_FP8_P = 1   # scores as the default, e4m3 P x e4m3 V on the fp8 MFMA
PRECISION_FP8 = 2     # e4m3 Q (per-row scale) and e4m3 P on the fp8 MFMA


def build_args(q, k_cache, v_cache, block_tables, seq_lens, cu_seqlens_q, k_descale, v_descale,
               softmax_scale, num_segments_, out, workspace, precision=PRECISION_16BIT, lse=None,
               sinks=None, window_left=-1, softcap=0.0, max_q_len=0, balance_segments=0, merge_sync=None,
               merge_wait_us=0) -> PfkvArgs:
    """Fill a ``pfkv_args`` from torch tensors (shapes and dtypes checked here).

    ``lse`` (optional) is a contiguous float32 ``[Hq, T]`` tensor on q's device,
    ``sinks`` (optional) a contiguous float32 ``[Hq]`` tensor on q's device.
    ``workspace`` may be None (pointer NULL, size 0) for the allocation-free call.
    ``merge_sync`` (optional) is a contiguous uint8 tensor on q's device
    (:func:`merge_sync_buffer`).
    """
    k_cache, v_cache = _as_bytes(k_cache), _as_bytes(v_cache)
    if q.dtype != torch.bfloat16 or q.dim() != 3 or q.stride(2) != 1:
        raise TypeError("q must be bf16 [T, Hq, D] with unit last stride")
    if out.dtype != torch.bfloat16 or out.shape != q.shape or out.stride(2) != 1:
        raise TypeError("out must be bf16 with q's shape and unit last stride")
    if k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise TypeError("k_cache / v_cache must be [num_pages, page_size, Hkv, D] of equal shape")
    if not (k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise TypeError("k_cache / v_cache must be contiguous")
    if k_cache.shape[3] != q.shape[2]:
        raise TypeError(f"k_cache / v_cache head_dim ({k_cache.shape[3]}) must equal q's ({q.shape[2]})")
    for name, t in (("block_tables", block_tables), ("seq_lens", seq_lens), ("cu_seqlens_q", cu_seqlens_q)):
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32")
    if block_tables.dim() != 2 or block_tables.stride(1) != 1:
        raise TypeError("block_tables must be [N, max_pages] with unit column stride")
    if not (seq_lens.is_contiguous() and cu_seqlens_q.is_contiguous()):
        raise TypeError("seq_lens / cu_seqlens_q must be contiguous")
    for name, t in (("k_descale", k_descale), ("v_descale", v_descale)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.numel() != 1:
            raise TypeError(f"{name} must be a one-element float32 tensor")
        if t.device != q.device:
            raise ValueError(f"{name} must be on q's device ({q.device}), got {t.device}")
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache), ("block_tables", block_tables),
                    ("seq_lens", seq_lens), ("cu_seqlens_q", cu_seqlens_q), ("out", out),
                    ("workspace", workspace)):
        if t is None:
            continue
        if t.device != q.device:
            raise ValueError(f"{name} must be on q's device ({q.device}), got {t.device}")
    if workspace is not None and (workspace.dtype != torch.uint8 or not workspace.is_contiguous()):
        raise TypeError("workspace must be a contiguous uint8 tensor")
    if lse is not None:
        if lse.dtype != torch.float32 or tuple(lse.shape) != (q.shape[1], q.shape[0]) or not lse.is_contiguous():
            raise TypeError("lse must be a contiguous float32 [Hq, T] tensor")
        if lse.device != q.device:
            raise ValueError(f"lse must be on q's device ({q.device}), got {lse.device}")
    a = PfkvArgs()
    a.q, a.k_cache, a.v_cache = q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr()
    a.block_tables, a.seq_lens, a.cu_seqlens_q = (block_tables.data_ptr(), seq_lens.data_ptr(),
                                                  cu_seqlens_q.data_ptr())
    a.k_descale, a.v_descale = k_descale.data_ptr(), v_descale.data_ptr()
    a.workspace = workspace.data_ptr() if workspace is not None else None
    a.out = out.data_ptr()
    a.q_stride_token, a.q_stride_head = q.stride(0), q.stride(1)
    a.out_stride_token, a.out_stride_head = out.stride(0), out.stride(1)
    a.block_table_stride = block_tables.stride(0)
    a.workspace_size = workspace.numel() if workspace is not None else 0
    a.num_seqs = seq_lens.numel()
    a.total_q = q.shape[0]
    a.num_q_heads = q.shape[1]
    a.num_kv_heads = k_cache.shape[2]
    a.head_dim = q.shape[2]
    a.page_size = k_cache.shape[1]
    a.num_pages = k_cache.shape[0]
    a.max_pages_per_seq = block_tables.shape[1]
    a.num_segments = int(num_segments_)
    a.softmax_scale = float(softmax_scale)
    a.precision = int(precision)
    a.lse = lse.data_ptr() if lse is not None else None
    if sinks is not None:
        if sinks.dtype != torch.float32 or tuple(sinks.shape) != (q.shape[1],) or not sinks.is_contiguous():
            raise TypeError("sinks must be a contiguous float32 [Hq] tensor")
        if sinks.device != q.device:
            raise ValueError(f"sinks must be on q's device ({q.device}), got {sinks.device}")
    a.sinks = sinks.data_ptr() if sinks is not None else None
    a.window_keys = int(window_left) + 1 if window_left >= 0 else 0   # left window W -> W + 1 keys
    a.softcap = float(softcap)
    a.max_q_len = int(max_q_len)
    a.balance_segments = 1 if balance_segments else 0
    if merge_sync is not None:
        if merge_sync.dtype != torch.uint8 or not merge_sync.is_contiguous():
            raise TypeError("merge_sync must be a contiguous uint8 tensor")
        if merge_sync.device != q.device:
            raise ValueError(f"merge_sync must be on q's device ({q.device}), got {merge_sync.device}")
        a.merge_sync = merge_sync.data_ptr()
        a.merge_sync_size = merge_sync.numel()
    a.merge_wait_us = int(merge_wait_us)
    return a


def verify_attn(q, k_cache, v_cache, block_tables, seq_lens, cu_seqlens_q, k_descale, v_descale,
                softmax_scale, num_segments=None, out=None, workspace=None, stream=None,
                precision=PRECISION_16BIT, return_lse=False, lse=None, sinks=None, window_left=-1,
                softcap=0.0, max_q_len=0, balance_segments=False, merge_sync=None, merge_wait_us=0):
    """Split-KV verify attention; returns ``out`` (bf16 ``[T, Hq, 256]``), or
    ``(out, lse)`` when ``return_lse`` is set or an ``lse`` buffer is given.

    ``lse`` is float32 ``[Hq, T]``: the natural-log sum of exp(scores) over each
    row's visible keys, -inf for a row without one (``include/pfkv.h``).
    ``sinks`` (float32 ``[Hq]``), ``window_left`` (a left window of that many
    positions when >= 0; passed as ``window_keys = window_left + 1``) and
    ``softcap`` (> 0 to enable) are the options described in ``include/pfkv.h``.
    ``max_q_len`` bounds every sequence's query tokens (0 = 4, at most 8).
    ``num_segments=None`` picks the library heuristic from the device's CU count.
    ``balance_segments=True`` gives each sequence segments in proportion to its
    pages, with ``num_segments`` as the cap per sequence (``None``: 128).
    ``precision`` selects the main kernel's arithmetic (``PRECISION_16BIT``,
    ``PRECISION_FP8_P`` or ``PRECISION_FP8``, see ``include/pfkv.h``).
    ``workspace`` (uint8, at least :func:`workspace_bytes` bytes) is allocated with
    torch when not given. ``merge_sync`` (:func:`merge_sync_buffer`, kept across
    calls) runs the merge inside the main launch where the call allows it
    (``include/pfkv.h``); ``merge_wait_us`` bounds its waits. The call is
    enqueued on ``stream`` (default: torch's current stream) and does not
    synchronize.
    """
    lib = load_library()
    if not q.is_cuda:
        raise ValueError("q must be a GPU tensor")
    if num_segments is None:
        if balance_segments:
            num_segments = 128
        else:
            _, cus = device_info(q.device.index)
            num_segments = num_segments_for(cus, seq_lens.numel(), k_cache.shape[2])
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        need = workspace_bytes(num_segments, q.shape[0], q.shape[1])
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
    a = build_args(q, k_cache, v_cache, block_tables, seq_lens, cu_seqlens_q, k_descale, v_descale,
                   softmax_scale, num_segments, out, workspace, precision, lse, sinks, window_left, softcap,
                   max_q_len, balance_segments, merge_sync, merge_wait_us)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    _raise_on(lib.pfkv_verify_attn_fwd(ctypes.byref(a), ctypes.c_void_p(handle)))
    return (out, lse) if lse is not None else out


def verify_attn_noalloc(q, k_cache, v_cache, block_tables, seq_lens, cu_seqlens_q, k_descale, v_descale,
                        softmax_scale, num_segments, out, stream=None, precision=PRECISION_16BIT, lse=None,
                        sinks=None, window_left=-1, softcap=0.0, max_q_len=0, balance_segments=False,
                        merge_sync=None, merge_wait_us=0):
    """The allocation-free call (``pfkv_verify_attn_fwd_noalloc``): the caller
    passes ``out`` (and ``lse`` if wanted) and an explicit ``num_segments``;
    the partials go to the library's own device array, so neither this wrapper
    nor the library allocates. Calls that overlap on one GPU race."""
    lib = load_library()
    if not q.is_cuda:
        raise ValueError("q must be a GPU tensor")
    a = build_args(q, k_cache, v_cache, block_tables, seq_lens, cu_seqlens_q, k_descale, v_descale,
                   softmax_scale, num_segments, out, None, precision, lse, sinks, window_left, softcap,
                   max_q_len, balance_segments, merge_sync, merge_wait_us)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    _raise_on(lib.pfkv_verify_attn_fwd_noalloc(ctypes.byref(a), ctypes.c_void_p(handle)))
    return (out, lse) if lse is not None else out


def num_segments_for(num_cus: int, num_seqs: int, num_kv_heads: int) -> int:
    return num_segments(num_cus, num_seqs, num_kv_heads)


def check_args(args: PfkvArgs, arch: str = "gfx950:sramecc+:xnack-", num_cus: int = 256) -> int:
    """Run the library's pure host validation (no GPU needed); returns the status."""
    return int(load_library().pfkv_check_args(ctypes.byref(args), arch.encode(), int(num_cus)))


def stream_read(buf: torch.Tensor, variant: int, page_order: Optional[torch.Tensor] = None,
                sink: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Launch one streaming-read pass over ``buf`` (see ``pfkv_stream_read``)."""
    lib = load_library()
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=buf.device)
    if stream is None:
        stream = torch.cuda.current_stream(buf.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    n_pages = 0 if page_order is None else page_order.numel()
    _raise_on(lib.pfkv_stream_read(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                                   int(variant), ctypes.c_void_p(_ptr(page_order) or 0), n_pages,
                                   ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(handle)))
    return sink


# ---------------------------------------------------------------- prefill
def build_prefill_args(q, k, v, q_descale, k_descale, v_descale, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                       softmax_scale, causal, out, lse=None) -> PfkvPrefillArgs:
    """Fill a ``pfkv_prefill_args`` from torch tensors (shapes and dtypes checked here)."""
    q, k, v = _as_bytes(q), _as_bytes(k), _as_bytes(v)
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 3 or t.stride(2) != 1:
            raise TypeError(f"{name} must be [tokens, heads, dim] with unit last stride")
    if k.shape[:2] != v.shape[:2] or q.shape[2] != k.shape[2]:
        raise TypeError("k / v must share [total_k, Hkv] and q / k their head dim")
    if out.dtype != torch.bfloat16 or out.dim() != 3 or out.stride(2) != 1 or \
            tuple(out.shape) != (q.shape[0], q.shape[1], v.shape[2]):
        raise TypeError("out must be bf16 [total_q, Hq, Dv] with unit last stride")
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous int32 vector")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 2:
        raise TypeError("cu_seqlens_q / cu_seqlens_k must both hold num_seqs + 1 entries")
    for name, t in (("q_descale", q_descale), ("k_descale", k_descale), ("v_descale", v_descale)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.numel() != 1:
            raise TypeError(f"{name} must be a one-element float32 tensor")
    for name, t in (("k", k), ("v", v), ("out", out), ("cu_seqlens_q", cu_seqlens_q),
                    ("cu_seqlens_k", cu_seqlens_k), ("q_descale", q_descale), ("k_descale", k_descale),
                    ("v_descale", v_descale)):
        if t.device != q.device:
            raise ValueError(f"{name} must be on q's device ({q.device}), got {t.device}")
    if lse is not None:
        if lse.dtype != torch.float32 or tuple(lse.shape) != (q.shape[1], q.shape[0]) or not lse.is_contiguous():
            raise TypeError("lse must be a contiguous float32 [Hq, total_q] tensor")
        if lse.device != q.device:
            raise ValueError(f"lse must be on q's device ({q.device}), got {lse.device}")
    a = PfkvPrefillArgs()
    a.q, a.k, a.v, a.out = q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr()
    a.lse = lse.data_ptr() if lse is not None else None
    a.cu_seqlens_q, a.cu_seqlens_k = cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr()
    a.q_descale, a.k_descale, a.v_descale = q_descale.data_ptr(), k_descale.data_ptr(), v_descale.data_ptr()
    a.q_stride_token, a.q_stride_head = q.stride(0), q.stride(1)
    a.k_stride_token, a.k_stride_head = k.stride(0), k.stride(1)
    a.v_stride_token, a.v_stride_head = v.stride(0), v.stride(1)
    a.out_stride_token, a.out_stride_head = out.stride(0), out.stride(1)
    a.num_seqs = cu_seqlens_q.numel() - 1
    a.total_q, a.total_k = q.shape[0], k.shape[0]
    a.num_q_heads, a.num_kv_heads = q.shape[1], k.shape[1]
    a.head_dim_qk, a.head_dim_v = q.shape[2], v.shape[2]
    a.max_seqlen_q = int(max_seqlen_q)
    a.softmax_scale = float(softmax_scale)
    a.causal = 1 if causal else 0
    return a


def prefill_attn(q, k, v, q_descale, k_descale, v_descale, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                 max_seqlen_k=None, softmax_scale=None, is_causal=False, return_lse=False, out=None, lse=None):
    """fp8 varlen prefill attention; returns ``out`` (bf16 ``[total_q, Hq, 128]``),
    or ``(out, lse)`` with ``return_lse`` (or an ``lse`` buffer given).

    Same argument list as ``fmha_fwd_fp8_varlen_asm(q, k, v, q_descale, k_descale,
    v_descale, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
    softmax_scale=None, is_causal=False, return_lse=False, out=None)`` of aiter
    PR #7375 (Changes). q / k / v: ``float8_e4m3fn`` (or uint8 codes) packed
    ``[tokens, heads, dim]`` views with unit last stride (qk dim 192, v dim 128);
    descales: one-element float32 tensors on q's device; softmax_scale defaults to
    1 / sqrt(192). ``max_seqlen_k`` is accepted for the same signature and unused.
    """
    del max_seqlen_k
    if out is None:
        out = torch.empty((q.shape[0], q.shape[1], v.shape[2]), dtype=torch.bfloat16, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
    if softmax_scale is None:
        softmax_scale = 1.0 / float(q.shape[2]) ** 0.5
    a = build_prefill_args(q, k, v, q_descale, k_descale, v_descale, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                           softmax_scale, is_causal, out, lse)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _raise_on(load_library().pfkv_prefill_fwd(ctypes.byref(a), ctypes.c_void_p(stream)))
    return (out, lse) if lse is not None else out


def check_prefill_args(args: PfkvPrefillArgs, arch: str = "gfx950:sramecc+:xnack-", num_cus: int = 256) -> int:
    """Host-only validation (no GPU): the library's status code for ``args``."""
    return int(load_library().pfkv_prefill_check_args(ctypes.byref(args), arch.encode(), int(num_cus)))
