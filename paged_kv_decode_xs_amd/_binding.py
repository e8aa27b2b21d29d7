"""ctypes binding of libxs.so: argument marshalling only.

Each function takes torch tensors, reads their shapes and device pointers, and calls the C
function of the same name in libxs.so (declared in include/xs/xs.h). Every step of the
computation runs in the library's HIP kernels. There is no fallback path: if the library is
not built, or the library rejects a call, these functions raise.

torch is imported before the library is loaded. libxs.so then binds to the HIP runtime that
torch already loaded (both carry the soname libamdhip64.so.7), so the library and torch share
one runtime, one device context and the same streams.
"""

from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

LIB_NAME = "libxs.so"
# XS_LIBRARY names another build of the same library (the host-sanitized one the ABI tests run
# under); there is no fallback either way.
LIB_PATH = os.environ.get("XS_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)

XS_F32 = 0
XS_BF16 = 1
STATUS = {0: "XS_OK", 1: "XS_EINVAL", 2: "XS_EUNSUPPORTED", 3: "XS_ELAUNCH"}

_lock = threading.Lock()
_lib: Optional[ctypes.CDLL] = None

_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float

class XsStepDesc(ctypes.Structure):
    """Mirror of xs_step_desc in include/xs/xs.h (field order and types must match)."""

    _fields_ = [
        ("q", ctypes.c_void_p), ("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p),
        ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p), ("block_tables", ctypes.c_void_p),
        ("context_lens", ctypes.c_void_p), ("sinks", ctypes.c_void_p), ("window_size", ctypes.c_int),
        ("scale", ctypes.c_float), ("out", ctypes.c_void_p), ("part_o", ctypes.c_void_p),
        ("part_m", ctypes.c_void_p), ("part_l", ctypes.c_void_p), ("batch", ctypes.c_int),
        ("num_q_heads", ctypes.c_int), ("num_kv_heads", ctypes.c_int), ("head_dim", ctypes.c_int),
        ("block_size", ctypes.c_int), ("max_blocks_per_seq", ctypes.c_int), ("num_blocks", ctypes.c_int),
        ("partition_size", ctypes.c_int), ("max_partitions", ctypes.c_int), ("dtype", ctypes.c_int),
        ("fused", ctypes.c_int),
    ]


SIGNATURES = {
    "xs_kv_append": [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp],
    "xs_paged_attn_decode": [_vp, _vp, _vp, _vp, _vp, _f, _vp, _vp, _vp, _vp,
                             _i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _vp],
    "xs_paged_attn_decode_append": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _f, _vp, _vp, _vp, _vp,
                                    _i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _vp],
    "xs_paged_attn_reduce": [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp],
    "xs_paged_attn_decode_append_noalloc": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _f, _vp,
                                            _i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _vp],
    "xs_paged_attn_decode_sinks": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _f, _vp, _vp, _vp, _vp,
                                   _i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _vp],
    "xs_paged_attn_reduce_sinks": [_vp, _vp, _vp, _vp, _vp, _i, _vp, _i, _i, _i, _i, _i, _i, _vp],
    "xs_stream_read_probe": [_vp, ctypes.c_size_t, _vp, _i, _i, _vp],
    "xs_kv_swap_out": [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp],
    "xs_kv_swap_in": [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp],
    "xs_step_graph_create": [ctypes.POINTER(XsStepDesc), _i, ctypes.POINTER(ctypes.c_void_p)],
    "xs_step_graph_launch": [_vp, _vp],
    "xs_step_graph_destroy": [_vp],
    "xs_kv_append_chunk": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _vp],
    "xs_paged_attn_prefill": [_vp, _vp, _vp, _vp, _vp, _vp, _f, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _i, _vp],
    "xs_paged_attn_prefill_split": [_vp, _vp, _vp, _vp, _vp, _vp, _f, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i,
                                    _i, _i, _i, _vp],
    "xs_paged_attn_prefill_sinks": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _f, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i,
                                    _i, _i, _i, _i, _i, _vp],
    "xs_last_error": [],
    "xs_version": [],
}


class XsError(RuntimeError):
    def __init__(self, func: str, status: int, message: str):
        super().__init__(f"{func} returned {STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


def library_path() -> str:
    return LIB_PATH


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libxs.so once (raises if it is missing: build it with __graft_entry__.build())."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(f"{p} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
        lib = ctypes.CDLL(p)
        for name, args in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_char_p if name == "xs_last_error" else ctypes.c_int
        if path is None:
            _lib = lib
        return lib


def xs_last_error() -> str:
    return load_library().xs_last_error().decode()


def xs_version() -> int:
    return load_library().xs_version()


def _check(func: str, status: int) -> None:
    if status != 0:
        raise XsError(func, status, xs_last_error())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return XS_BF16
    if t.dtype == torch.float32:
        return XS_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return stream or None
    return stream.cuda_stream or None


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _dev(*ts: Optional[torch.Tensor]) -> None:
    for t in ts:
        if t is None:
            continue
        _need(t.is_cuda, "all tensors must be on the GPU")
        _need(t.is_contiguous(), "all tensors must be contiguous")


def xs_kv_append(k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                 block_tables: torch.Tensor, context_lens: torch.Tensor, stream=None) -> None:
    """Write each sequence's new K/V row into slot context_lens[b] - 1 of the paged pools."""
    _dev(k_new, v_new, k_cache, v_cache, block_tables, context_lens)
    NB, Hkv, BS, D = k_cache.shape
    B = k_new.shape[0]
    _need(k_new.shape == (B, Hkv, D) and v_new.shape == (B, Hkv, D), "k_new/v_new must be [batch, Hkv, D]")
    _need(v_cache.shape == k_cache.shape, "k_cache and v_cache must have the same shape")
    _need(len({k_new.dtype, v_new.dtype, k_cache.dtype, v_cache.dtype}) == 1, "K/V dtypes differ")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and block_tables.shape[0] == B,
          "block_tables must be int32 [batch, max_blocks_per_seq]")
    _need(context_lens.dtype == torch.int32 and context_lens.shape == (B,), "context_lens must be int32 [batch]")
    lib = load_library()
    _check("xs_kv_append", lib.xs_kv_append(
        _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        B, Hkv, D, BS, block_tables.shape[1], NB, _dtype_code(k_cache), _stream_handle(stream)))


def _decode_common(q, k_cache, v_cache, block_tables, context_lens, out, part_o, part_m, part_l, partition_size):
    _dev(q, k_cache, v_cache, block_tables, context_lens, out, part_o, part_m, part_l)
    B, Hq, D = q.shape
    NB, Hkv, BS, D2 = k_cache.shape
    _need(D2 == D and v_cache.shape == k_cache.shape, "pool shapes do not match q")
    _need(len({q.dtype, k_cache.dtype, v_cache.dtype}) == 1, "q and pool dtypes differ")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and block_tables.shape[0] == B,
          "block_tables must be int32 [batch, max_blocks_per_seq]")
    _need(context_lens.dtype == torch.int32 and context_lens.shape == (B,), "context_lens must be int32 [batch]")
    NP = 0
    if partition_size > 0:
        _need(part_o is not None and part_m is not None and part_l is not None, "split-K needs part_o/m/l")
        NP = part_m.shape[-1]
        _need(part_o.shape == (B, Hq, NP, D) and part_m.shape == (B, Hq, NP) and part_l.shape == (B, Hq, NP),
              "partials must be [B, Hq, NP, D], [B, Hq, NP], [B, Hq, NP]")
        _need(all(t.dtype == torch.float32 for t in (part_o, part_m, part_l)), "partials are float32")
    else:
        _need(out is not None and out.shape == (B, Hq, D) and out.dtype == q.dtype, "out must be q-shaped")
    return B, Hq, Hkv, D, BS, NB, NP


def xs_paged_attn_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                         block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                         out: Optional[torch.Tensor] = None, part_o: Optional[torch.Tensor] = None,
                         part_m: Optional[torch.Tensor] = None, part_l: Optional[torch.Tensor] = None,
                         partition_size: int = 0, stream=None) -> None:
    """Decode attention. partition_size == 0 writes `out`; otherwise the split-K partials."""
    B, Hq, Hkv, D, BS, NB, NP = _decode_common(q, k_cache, v_cache, block_tables, context_lens, out, part_o,
                                               part_m, part_l, partition_size)
    lib = load_library()
    _check("xs_paged_attn_decode", lib.xs_paged_attn_decode(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens), float(scale), _ptr(out),
        _ptr(part_o), _ptr(part_m), _ptr(part_l), B, Hq, Hkv, D, BS, block_tables.shape[1], NB,
        int(partition_size), NP, _dtype_code(q), _stream_handle(stream)))


def xs_paged_attn_decode_append(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor,
                                v_cache: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                                scale: float, out: Optional[torch.Tensor] = None,
                                part_o: Optional[torch.Tensor] = None, part_m: Optional[torch.Tensor] = None,
                                part_l: Optional[torch.Tensor] = None, partition_size: int = 0, stream=None) -> None:
    """The KV append and the decode attention in one launch (same results as the two calls)."""
    B, Hq, Hkv, D, BS, NB, NP = _decode_common(q, k_cache, v_cache, block_tables, context_lens, out, part_o,
                                               part_m, part_l, partition_size)
    _dev(k_new, v_new)
    _need(k_new.shape == (B, Hkv, D) and v_new.shape == (B, Hkv, D), "k_new/v_new must be [batch, Hkv, D]")
    _need(k_new.dtype == q.dtype and v_new.dtype == q.dtype, "k_new/v_new dtype differs from q")
    lib = load_library()
    _check("xs_paged_attn_decode_append", lib.xs_paged_attn_decode_append(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        float(scale), _ptr(out), _ptr(part_o), _ptr(part_m), _ptr(part_l), B, Hq, Hkv, D, BS,
        block_tables.shape[1], NB, int(partition_size), NP, _dtype_code(q), _stream_handle(stream)))


def xs_paged_attn_decode_append_noalloc(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                                        k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
                                        context_lens: torch.Tensor, scale: float, out: torch.Tensor,
                                        partition_size: int = 0, max_partitions: Optional[int] = None,
                                        stream=None) -> None:
    """Append + decode (+ the reduce with split-K) into `out`, the partials kept in the library's
    own device scratch: nothing is allocated. max_partitions defaults to what the block table can
    hold (max_blocks_per_seq * block_size / partition_size)."""
    B, Hq, Hkv, D, BS, NB, _ = _decode_common(q, k_cache, v_cache, block_tables, context_lens, out, None, None,
                                              None, 0)
    _dev(k_new, v_new)
    _need(k_new.shape == (B, Hkv, D) and v_new.shape == (B, Hkv, D), "k_new/v_new must be [batch, Hkv, D]")
    _need(k_new.dtype == q.dtype and v_new.dtype == q.dtype, "k_new/v_new dtype differs from q")
    NP = 0
    if partition_size > 0:
        NP = max_partitions if max_partitions is not None else num_partitions(block_tables.shape[1] * BS,
                                                                              partition_size)
    lib = load_library()
    _check("xs_paged_attn_decode_append_noalloc", lib.xs_paged_attn_decode_append_noalloc(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        float(scale), _ptr(out), B, Hq, Hkv, D, BS, block_tables.shape[1], NB, int(partition_size), int(NP),
        _dtype_code(q), _stream_handle(stream)))


def xs_paged_attn_reduce(part_o: torch.Tensor, part_m: torch.Tensor, part_l: torch.Tensor,
                         context_lens: torch.Tensor, out: torch.Tensor, partition_size: int, stream=None) -> None:
    """Log-sum-exp merge of the split-K partials into `out`."""
    _dev(part_o, part_m, part_l, context_lens, out)
    B, Hq, NP, D = part_o.shape
    _need(part_m.shape == (B, Hq, NP) and part_l.shape == (B, Hq, NP), "partial shapes differ")
    _need(out.shape == (B, Hq, D), "out must be [B, Hq, D]")
    _need(context_lens.dtype == torch.int32 and context_lens.shape == (B,), "context_lens must be int32 [batch]")
    lib = load_library()
    _check("xs_paged_attn_reduce", lib.xs_paged_attn_reduce(
        _ptr(part_o), _ptr(part_m), _ptr(part_l), _ptr(context_lens), _ptr(out), B, Hq, D,
        int(partition_size), NP, _dtype_code(out), _stream_handle(stream)))


def xs_paged_attn_decode_sinks(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                               block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                               sinks: Optional[torch.Tensor] = None, window_size: int = 0,
                               out: Optional[torch.Tensor] = None, part_o: Optional[torch.Tensor] = None,
                               part_m: Optional[torch.Tensor] = None, part_l: Optional[torch.Tensor] = None,
                               partition_size: int = 0, k_new: Optional[torch.Tensor] = None,
                               v_new: Optional[torch.Tensor] = None, stream=None) -> None:
    """Decode attention with per-head sinks (bf16 [Hq] or None) and a sliding window (0: none),
    plus the fused append when k_new/v_new are given."""
    B, Hq, Hkv, D, BS, NB, NP = _decode_common(q, k_cache, v_cache, block_tables, context_lens, out, part_o,
                                               part_m, part_l, partition_size)
    _dev(sinks, k_new, v_new)
    if sinks is not None:
        _need(sinks.shape == (Hq,) and sinks.dtype == torch.bfloat16, "sinks must be bfloat16 [num_q_heads]")
    if k_new is not None or v_new is not None:
        _need(k_new is not None and v_new is not None, "give both k_new and v_new, or neither")
        _need(k_new.shape == (B, Hkv, D) and v_new.shape == (B, Hkv, D), "k_new/v_new must be [batch, Hkv, D]")
        _need(k_new.dtype == q.dtype and v_new.dtype == q.dtype, "k_new/v_new dtype differs from q")
    lib = load_library()
    _check("xs_paged_attn_decode_sinks", lib.xs_paged_attn_decode_sinks(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        _ptr(sinks), int(window_size), float(scale), _ptr(out), _ptr(part_o), _ptr(part_m), _ptr(part_l),
        B, Hq, Hkv, D, BS, block_tables.shape[1], NB, int(partition_size), NP, _dtype_code(q),
        _stream_handle(stream)))


def xs_paged_attn_reduce_sinks(part_o: torch.Tensor, part_m: torch.Tensor, part_l: torch.Tensor,
                               context_lens: torch.Tensor, out: torch.Tensor, partition_size: int,
                               sinks: Optional[torch.Tensor] = None, window_size: int = 0, stream=None) -> None:
    """The merge of xs_paged_attn_decode_sinks' partials (same sinks and window)."""
    _dev(part_o, part_m, part_l, context_lens, out, sinks)
    B, Hq, NP, D = part_o.shape
    _need(part_m.shape == (B, Hq, NP) and part_l.shape == (B, Hq, NP), "partial shapes differ")
    _need(out.shape == (B, Hq, D), "out must be [B, Hq, D]")
    _need(context_lens.dtype == torch.int32 and context_lens.shape == (B,), "context_lens must be int32 [batch]")
    if sinks is not None:
        _need(sinks.shape == (Hq,) and sinks.dtype == torch.bfloat16, "sinks must be bfloat16 [num_q_heads]")
    lib = load_library()
    _check("xs_paged_attn_reduce_sinks", lib.xs_paged_attn_reduce_sinks(
        _ptr(part_o), _ptr(part_m), _ptr(part_l), _ptr(context_lens), _ptr(sinks), int(window_size), _ptr(out),
        B, Hq, D, int(partition_size), NP, _dtype_code(out), _stream_handle(stream)))


def xs_stream_read_probe(buf: torch.Tensor, sink: torch.Tensor, nontemporal: bool = True, shape: int = 0,
                         stream=None) -> None:
    """Read all of `buf` with 16-byte loads (a bandwidth reference); `sink` is a 4-byte device buffer.
    shape 0: 16 workgroups per CU on 256 KiB chunks; shape 1: two per CU on 16 KiB chunks."""
    _dev(buf, sink)
    nbytes = buf.numel() * buf.element_size()
    _need(sink.numel() * sink.element_size() >= 4, "sink must hold 4 bytes")
    _check("xs_stream_read_probe", load_library().xs_stream_read_probe(
        _ptr(buf), nbytes - nbytes % 16, _ptr(sink), int(bool(nontemporal)), int(shape), _stream_handle(stream)))


def _swap_checks(k_cache, v_cache, k_host, v_host, src, dst):
    _dev(k_cache, v_cache, src, dst)
    _need(v_cache.shape == k_cache.shape and k_cache.dim() == 4, "pools must be [NB, Hkv, BS, D] and alike")
    for t in (k_host, v_host):
        _need(not t.is_cuda and t.is_pinned() and t.is_contiguous(), "the swap space must be pinned, contiguous host tensors")
    _need(k_host.shape[1:] == k_cache.shape[1:] and v_host.shape == k_host.shape,
          "swap space must be [slots, Hkv, BS, D] like the pools")
    _need(len({k_cache.dtype, v_cache.dtype, k_host.dtype, v_host.dtype}) == 1, "pool and swap-space dtypes differ")
    _need(src.dtype == torch.int32 and dst.dtype == torch.int32 and src.dim() == 1 and src.shape == dst.shape,
          "index lists must be int32 [num_pairs] device tensors of equal length")
    NB, Hkv, BS, D = k_cache.shape
    return NB, k_host.shape[0], Hkv, BS, D


def xs_kv_swap_out(k_cache: torch.Tensor, v_cache: torch.Tensor, k_host: torch.Tensor, v_host: torch.Tensor,
                   src_blocks: torch.Tensor, dst_slots: torch.Tensor, stream=None) -> None:
    """Copy pool blocks src_blocks[i] into host slots dst_slots[i] (K and V), one launch."""
    NB, S, Hkv, BS, D = _swap_checks(k_cache, v_cache, k_host, v_host, src_blocks, dst_slots)
    _check("xs_kv_swap_out", load_library().xs_kv_swap_out(
        _ptr(k_cache), _ptr(v_cache), _ptr(k_host), _ptr(v_host), _ptr(src_blocks), _ptr(dst_slots),
        src_blocks.numel(), NB, S, Hkv, BS, D, _dtype_code(k_cache), _stream_handle(stream)))


def xs_kv_swap_in(k_host: torch.Tensor, v_host: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                  src_slots: torch.Tensor, dst_blocks: torch.Tensor, stream=None) -> None:
    """Copy host slots src_slots[i] into pool blocks dst_blocks[i] (K and V), one launch."""
    NB, S, Hkv, BS, D = _swap_checks(k_cache, v_cache, k_host, v_host, src_slots, dst_blocks)
    _check("xs_kv_swap_in", load_library().xs_kv_swap_in(
        _ptr(k_host), _ptr(v_host), _ptr(k_cache), _ptr(v_cache), _ptr(src_slots), _ptr(dst_blocks),
        src_slots.numel(), NB, S, Hkv, BS, D, _dtype_code(k_cache), _stream_handle(stream)))


def xs_step_graph_create(descs) -> int:
    """Capture decode steps (a sequence of XsStepDesc, run in order) as one HIP graph; returns the handle."""
    arr = (XsStepDesc * len(descs))(*descs)
    handle = ctypes.c_void_p()
    _check("xs_step_graph_create", load_library().xs_step_graph_create(arr, len(descs), ctypes.byref(handle)))
    return handle.value


def xs_step_graph_launch(handle: int, stream=None) -> None:
    _check("xs_step_graph_launch", load_library().xs_step_graph_launch(handle, _stream_handle(stream)))


def xs_step_graph_destroy(handle: int) -> None:
    _check("xs_step_graph_destroy", load_library().xs_step_graph_destroy(handle))


def _chunk_checks(B, block_tables, start_pos, chunk_lens):
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and block_tables.shape[0] == B,
          "block_tables must be int32 [batch, max_blocks_per_seq]")
    _need(start_pos.dtype == torch.int32 and start_pos.shape == (B,), "start_pos must be int32 [batch]")
    _need(chunk_lens.dtype == torch.int32 and chunk_lens.shape == (B,), "chunk_lens must be int32 [batch]")


def xs_kv_append_chunk(k_src: torch.Tensor, v_src: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                       block_tables: torch.Tensor, start_pos: torch.Tensor, chunk_lens: torch.Tensor,
                       stream=None) -> None:
    """Write rows i < chunk_lens[b] of k_src/v_src [batch, Hkv, chunk, D] to positions start_pos[b] + i."""
    _dev(k_src, v_src, k_cache, v_cache, block_tables, start_pos, chunk_lens)
    NB, Hkv, BS, D = k_cache.shape
    B, C = k_src.shape[0], k_src.shape[2]
    _need(k_src.shape == (B, Hkv, C, D) and v_src.shape == k_src.shape, "k_src/v_src must be [batch, Hkv, chunk, D]")
    _need(v_cache.shape == k_cache.shape, "k_cache and v_cache must have the same shape")
    _need(len({k_src.dtype, v_src.dtype, k_cache.dtype, v_cache.dtype}) == 1, "K/V dtypes differ")
    _chunk_checks(B, block_tables, start_pos, chunk_lens)
    _check("xs_kv_append_chunk", load_library().xs_kv_append_chunk(
        _ptr(k_src), _ptr(v_src), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(start_pos),
        _ptr(chunk_lens), B, Hkv, D, C, BS, block_tables.shape[1], NB, _dtype_code(k_cache), _stream_handle(stream)))


def xs_paged_attn_prefill(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
                          start_pos: torch.Tensor, chunk_lens: torch.Tensor, scale: float,
                          out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Causal attention of q [batch, Hq, chunk, D] (row i at position start_pos[b] + i) over the pools."""
    _dev(q, k_cache, v_cache, block_tables, start_pos, chunk_lens, out)
    B, Hq, C, D = q.shape
    NB, Hkv, BS, D2 = k_cache.shape
    _need(D2 == D and v_cache.shape == k_cache.shape, "pool shapes do not match q")
    _need(q.dtype == k_cache.dtype == v_cache.dtype, "q and the pools must have the same dtype")
    _chunk_checks(B, block_tables, start_pos, chunk_lens)
    if out is None:
        out = torch.empty_like(q)
    _dev(out)
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    _check("xs_paged_attn_prefill", load_library().xs_paged_attn_prefill(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(start_pos), _ptr(chunk_lens), float(scale),
        _ptr(out), B, Hq, Hkv, D, C, BS, block_tables.shape[1], NB, _dtype_code(q), _stream_handle(stream)))
    return out


def xs_paged_attn_prefill_split(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                block_tables: torch.Tensor, start_pos: torch.Tensor, chunk_lens: torch.Tensor,
                                scale: float, partition_size: int, out: Optional[torch.Tensor] = None,
                                part_o: Optional[torch.Tensor] = None, part_ml: Optional[torch.Tensor] = None,
                                stream=None) -> torch.Tensor:
    """xs_paged_attn_prefill with split-K over the key range (pieces of partition_size positions).
    part_o [batch, Hq, chunk, NP, D] / part_ml [batch, Hq, chunk, NP, 2] fp32 scratch, NP =
    ceil(max_blocks_per_seq * block_size / partition_size); allocated here when not given."""
    _dev(q, k_cache, v_cache, block_tables, start_pos, chunk_lens, out, part_o, part_ml)
    B, Hq, C, D = q.shape
    NB, Hkv, BS, D2 = k_cache.shape
    _need(D2 == D and v_cache.shape == k_cache.shape, "pool shapes do not match q")
    _need(q.dtype == k_cache.dtype == v_cache.dtype, "q and the pools must have the same dtype")
    _chunk_checks(B, block_tables, start_pos, chunk_lens)
    MBPS = block_tables.shape[1]
    _need(int(partition_size) > 0, "partition_size must be positive")
    NP = num_partitions(MBPS * BS, int(partition_size))
    if out is None:
        out = torch.empty_like(q)
    if part_o is None:
        part_o = torch.empty((B, Hq, C, NP, D), dtype=torch.float32, device=q.device)
    if part_ml is None:
        part_ml = torch.empty((B, Hq, C, NP, 2), dtype=torch.float32, device=q.device)
    _dev(out, part_o, part_ml)
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    _need(part_o.dtype == torch.float32 and part_ml.dtype == torch.float32 and part_o.is_contiguous()
          and part_ml.is_contiguous(), "partials must be contiguous fp32")
    NP = part_o.shape[3] if part_o.dim() == 5 else NP
    _need(part_o.shape == (B, Hq, C, NP, D) and part_ml.shape == (B, Hq, C, NP, 2), "partial shapes do not match")
    _check("xs_paged_attn_prefill_split", load_library().xs_paged_attn_prefill_split(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(start_pos), _ptr(chunk_lens), float(scale),
        _ptr(out), _ptr(part_o), _ptr(part_ml), B, Hq, Hkv, D, C, BS, MBPS, NB, int(partition_size), NP,
        _dtype_code(q), _stream_handle(stream)))
    return out


def xs_paged_attn_prefill_sinks(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                block_tables: torch.Tensor, start_pos: torch.Tensor, chunk_lens: torch.Tensor,
                                scale: float, sinks: Optional[torch.Tensor] = None, window_size: int = 0,
                                partition_size: int = 0, out: Optional[torch.Tensor] = None,
                                part_o: Optional[torch.Tensor] = None, part_ml: Optional[torch.Tensor] = None,
                                stream=None) -> torch.Tensor:
    """Chunked-prefill attention with per-head sinks (bf16 [Hq] or None) and a sliding window
    (0: none); partition_size 0 runs unsplit, > 0 split-K with partials as in
    xs_paged_attn_prefill_split (allocated here when not given)."""
    _dev(q, k_cache, v_cache, block_tables, start_pos, chunk_lens, sinks, out, part_o, part_ml)
    B, Hq, C, D = q.shape
    NB, Hkv, BS, D2 = k_cache.shape
    _need(D2 == D and v_cache.shape == k_cache.shape, "pool shapes do not match q")
    _need(q.dtype == k_cache.dtype == v_cache.dtype, "q and the pools must have the same dtype")
    _chunk_checks(B, block_tables, start_pos, chunk_lens)
    if sinks is not None:
        _need(sinks.shape == (Hq,) and sinks.dtype == torch.bfloat16 and sinks.is_contiguous(),
              "sinks must be contiguous bfloat16 [num_q_heads]")
    MBPS = block_tables.shape[1]
    P = int(partition_size)
    _need(P >= 0, "partition_size must be >= 0")
    if out is None:
        out = torch.empty_like(q)
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    NP = 0
    if P > 0:
        NP = num_partitions(MBPS * BS, P)
        if part_o is None:
            part_o = torch.empty((B, Hq, C, NP, D), dtype=torch.float32, device=q.device)
        if part_ml is None:
            part_ml = torch.empty((B, Hq, C, NP, 2), dtype=torch.float32, device=q.device)
        _dev(part_o, part_ml)
        _need(part_o.dtype == torch.float32 and part_ml.dtype == torch.float32 and part_o.is_contiguous()
              and part_ml.is_contiguous(), "partials must be contiguous fp32")
        NP = part_o.shape[3] if part_o.dim() == 5 else NP
        _need(part_o.shape == (B, Hq, C, NP, D) and part_ml.shape == (B, Hq, C, NP, 2), "partial shapes do not match")
    _check("xs_paged_attn_prefill_sinks", load_library().xs_paged_attn_prefill_sinks(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(start_pos), _ptr(chunk_lens), _ptr(sinks),
        int(window_size), float(scale), _ptr(out), _ptr(part_o), _ptr(part_ml), B, Hq, Hkv, D, C, BS, MBPS, NB, P, NP,
        _dtype_code(q), _stream_handle(stream)))
    return out


def num_partitions(max_context_len: int, partition_size: int) -> int:
    """Partition slots the split-K call needs for contexts up to max_context_len."""
    return max(1, -(-int(max_context_len) // int(partition_size)))
