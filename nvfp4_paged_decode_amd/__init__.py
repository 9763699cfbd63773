"""NVFP4 paged KV cache for AMD MI355X (gfx950).

Thin ctypes binding of ``libkvfp4.so`` (see ``include/kvfp4.h`` for the
contract).  Functions carry the C ABI's names; they only marshal torch
tensors into pointers and sizes, pass torch's current HIP stream, and turn
a negative status into :class:`KvFp4Error`.  Every step of the computation
runs in the library's HIP kernels; there is no Python or CPU fallback: if
the library is not built, every call raises.

Build the library with ``python -m nvfp4_paged_decode_amd.build``.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvfp4.so")

KVFP4_OK = 0
KVFP4_ERR_INVALID_ARG = -1
KVFP4_ERR_UNSUPPORTED = -2
KVFP4_ERR_WORKSPACE = -3
KVFP4_ERR_HIP = -4
KVFP4_ROWS_BF16 = 0
KVFP4_ROWS_FP8_E4M3 = 1

#: Every function the header declares (checked by the CPU tests).
EXPORTS = (
    "kvfp4_hot_page_bytes", "kvfp4_packed_page_bytes", "kvfp4_quantize_pages",
    "kvfp4_dequantize_pages", "kvfp4_sort_page_list", "kvfp4_append_quantize",
    "kvfp4_gather_dequantize",
    "kvfp4_packed_page_bytes_rope", "kvfp4_quantize_pages_rope", "kvfp4_dequantize_pages_rope",
    "kvfp4_decode_workspace_bytes",
    "kvfp4_paged_decode_attention", "kvfp4_paged_decode_attention_noalloc",
    "kvfp4_status_string", "kvfp4_last_error_message",
)


class Geometry(ctypes.Structure):
    """``kvfp4_geometry``: (num_kv_tensors, page_size, num_kv_heads, head_dim)."""

    _fields_ = [("num_kv_tensors", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32)]

    @classmethod
    def of(cls, g) -> "Geometry":
        return g if isinstance(g, cls) else cls(*[int(v) for v in g])


KVFP4_ROPE_NVFP4 = 0
KVFP4_ROPE_BF16 = 1
KVFP4_ROPE_2FP4 = 2


class RopeLayout(ctypes.Structure):
    """``kvfp4_rope_layout``: (rope_dims, mode)."""

    _fields_ = [("rope_dims", ctypes.c_int32), ("mode", ctypes.c_int32)]

    @classmethod
    def of(cls, r) -> "RopeLayout":
        return r if isinstance(r, cls) else cls(*[int(v) for v in r])


class KvFp4Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load libkvfp4.so once.  torch is imported first so that the library
    binds to the HIP runtime torch already loaded (same soname)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run: python -m nvfp4_paged_decode_amd.build")
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    G = ctypes.POINTER(Geometry)
    lib.kvfp4_hot_page_bytes.argtypes = [G]
    lib.kvfp4_hot_page_bytes.restype = SZ
    lib.kvfp4_packed_page_bytes.argtypes = [G]
    lib.kvfp4_packed_page_bytes.restype = SZ
    codec = [G, P, I32, P, P, I32, P, I32, P, P]
    lib.kvfp4_quantize_pages.argtypes = codec
    lib.kvfp4_quantize_pages.restype = I32
    lib.kvfp4_dequantize_pages.argtypes = codec
    lib.kvfp4_dequantize_pages.restype = I32
    lib.kvfp4_sort_page_list.argtypes = [P, P, I32, P, P, P]
    lib.kvfp4_sort_page_list.restype = I32
    lib.kvfp4_append_quantize.argtypes = [G, P, I32, I32, P, P, P, I32, P, P]
    lib.kvfp4_append_quantize.restype = I32
    lib.kvfp4_gather_dequantize.argtypes = [G, P, I32, P, P, I32, P, I32, P, P]
    lib.kvfp4_gather_dequantize.restype = I32
    RL = ctypes.POINTER(RopeLayout)
    lib.kvfp4_packed_page_bytes_rope.argtypes = [G, RL]
    lib.kvfp4_packed_page_bytes_rope.restype = SZ
    lib.kvfp4_quantize_pages_rope.argtypes = [G, RL] + codec[1:]
    lib.kvfp4_quantize_pages_rope.restype = I32
    lib.kvfp4_dequantize_pages_rope.argtypes = [G, RL] + codec[1:]
    lib.kvfp4_dequantize_pages_rope.restype = I32
    lib.kvfp4_decode_workspace_bytes.argtypes = [G, I32, I32, I32, I32]
    lib.kvfp4_decode_workspace_bytes.restype = SZ
    lib.kvfp4_paged_decode_attention.argtypes = [G, P, I32, P, P, I32, I32, I32, P, I32, P, I32,
                                                 F, P, P, P, SZ, P]
    lib.kvfp4_paged_decode_attention.restype = I32
    lib.kvfp4_paged_decode_attention_noalloc.argtypes = [G, P, I32, P, P, I32, I32, I32, P, I32,
                                                         P, I32, F, P, P, P]
    lib.kvfp4_paged_decode_attention_noalloc.restype = I32
    lib.kvfp4_status_string.argtypes = [I32]
    lib.kvfp4_status_string.restype = ctypes.c_char_p
    lib.kvfp4_last_error_message.argtypes = []
    lib.kvfp4_last_error_message.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int) -> int:
    if status != KVFP4_OK:
        lib = load_library()
        msg = lib.kvfp4_last_error_message().decode() or lib.kvfp4_status_string(status).decode()
        raise KvFp4Error(status, msg)
    return status


def _ptr(t, host_ok: bool = False) -> Optional[int]:
    """Device pointer of a contiguous GPU tensor (None -> NULL).  With
    ``host_ok`` a pinned host tensor is accepted too: pinned host memory is
    mapped into the GPU's address space at the same address."""
    if t is None:
        return None
    if not t.is_cuda and not (host_ok and t.is_pinned()):
        raise ValueError("tensor must live on the GPU" +
                         (" or in pinned host memory" if host_ok else ""))
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _int32(t, name: str, min_numel: int):
    """Check an index tensor before its pointer is taken: the kernels read
    int32, so an int64 tensor (torch's default integer type) would be read
    as pairs of halves."""
    if t is None:
        return
    import torch
    if t.dtype != torch.int32:
        raise ValueError(f"{name} must be int32, got {t.dtype}")
    if t.numel() < min_numel:
        raise ValueError(f"{name} holds {t.numel()} entries, needs at least {min_numel}")


def _check_decode_args(g: "Geometry", q, out, lse, block_table, seq_lens, vd: int) -> None:
    """Shapes and dtypes of the decode call's tensors, checked before any
    pointer is taken (the library sees only pointers and sizes)."""
    import torch
    if q.dim() != 3 or q.element_size() != 2:
        raise ValueError("q must be a 3-d tensor [batch, num_q_heads, head_dim] of 2-byte "
                         f"elements (bf16 bits), got shape {tuple(q.shape)} and {q.dtype}")
    if int(q.shape[-1]) != g.head_dim:
        raise ValueError(f"q.shape[-1] = {int(q.shape[-1])} differs from head_dim {g.head_dim}")
    B, Hq = int(q.shape[0]), int(q.shape[1])
    if out.element_size() != 2:
        raise ValueError(f"out must hold 2-byte elements (bf16 bits), got {out.dtype}")
    if out.numel() < B * Hq * vd:
        raise ValueError(f"out holds {out.numel()} elements, needs {B} x {Hq} x {vd}")
    if lse is not None:
        if lse.dtype != torch.float32:
            raise ValueError(f"lse must be float32, got {lse.dtype}")
        if lse.numel() < B * Hq:
            raise ValueError(f"lse holds {lse.numel()} elements, needs {B} x {Hq}")
    if block_table.dim() != 2:
        raise ValueError(f"block_table must be 2-d [batch, max_pages], got {tuple(block_table.shape)}")
    _int32(block_table, "block_table", 1)
    if int(block_table.shape[0]) < B:
        raise ValueError(f"block_table has {int(block_table.shape[0])} rows, needs {B}")
    _int32(seq_lens, "seq_lens", B)


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


def _scales(global_scale: Sequence[float], n: int):
    vals = [float(v) for v in list(global_scale)[:n]]
    if len(vals) < n:
        raise ValueError(f"global_scale needs {n} values")
    return (ctypes.c_float * n)(*vals)


def _pages(pool, page_bytes: int) -> int:
    nbytes = pool.numel() * pool.element_size()
    return nbytes // page_bytes if page_bytes else 0


def kvfp4_hot_page_bytes(geometry) -> int:
    return int(load_library().kvfp4_hot_page_bytes(ctypes.byref(Geometry.of(geometry))))


def kvfp4_packed_page_bytes(geometry) -> int:
    return int(load_library().kvfp4_packed_page_bytes(ctypes.byref(Geometry.of(geometry))))


def kvfp4_quantize_pages(geometry, hot_pool, packed_pool, num_pages: int, global_scale,
                         src_slots=None, dst_slots=None, stream=None) -> None:
    """Encode ``num_pages`` bf16 pages of ``hot_pool`` into ``packed_pool``
    (device memory, or pinned host memory: the offload path)."""
    lib = load_library()
    g = Geometry.of(geometry)
    _int32(src_slots, "src_slots", int(num_pages))
    _int32(dst_slots, "dst_slots", int(num_pages))
    _check(lib.kvfp4_quantize_pages(
        ctypes.byref(g), _ptr(hot_pool), _pages(hot_pool, kvfp4_hot_page_bytes(g)), _ptr(src_slots),
        _ptr(packed_pool, host_ok=True), _pages(packed_pool, kvfp4_packed_page_bytes(g)),
        _ptr(dst_slots),
        int(num_pages), _scales(global_scale, g.num_kv_tensors), _stream(stream)))


def kvfp4_dequantize_pages(geometry, packed_pool, hot_pool, num_pages: int, global_scale,
                           src_slots=None, dst_slots=None, stream=None) -> None:
    """Decode ``num_pages`` packed pages of ``packed_pool`` (device memory, or
    pinned host memory: the onboard path) into ``hot_pool``."""
    lib = load_library()
    g = Geometry.of(geometry)
    _int32(src_slots, "src_slots", int(num_pages))
    _int32(dst_slots, "dst_slots", int(num_pages))
    _check(lib.kvfp4_dequantize_pages(
        ctypes.byref(g), _ptr(packed_pool, host_ok=True),
        _pages(packed_pool, kvfp4_packed_page_bytes(g)),
        _ptr(src_slots), _ptr(hot_pool), _pages(hot_pool, kvfp4_hot_page_bytes(g)),
        _ptr(dst_slots), int(num_pages), _scales(global_scale, g.num_kv_tensors), _stream(stream)))


def kvfp4_sort_page_list(key, key_out, other=None, other_out=None, num_pages=None,
                         stream=None) -> None:
    """Sort the pairs (key[i], other[i]) by key into (key_out, other_out):
    ascending as unsigned 32-bit values, equal keys in input order.  Pass
    the codec calls' hot-pool slots as ``key``; the codec then takes the
    pages in slot order."""
    lib = load_library()
    n = int(key.numel() if num_pages is None else num_pages)
    _int32(key, "key", n)
    _int32(key_out, "key_out", n)
    if (other is None) != (other_out is None):
        raise ValueError("other and other_out must both be given or both be None")
    _int32(other, "other", n)
    _int32(other_out, "other_out", n)
    _check(lib.kvfp4_sort_page_list(_ptr(key), _ptr(other), n, _ptr(key_out), _ptr(other_out),
                                    _stream(stream)))


def kvfp4_packed_page_bytes_rope(geometry, rope) -> int:
    return int(load_library().kvfp4_packed_page_bytes_rope(
        ctypes.byref(Geometry.of(geometry)), ctypes.byref(RopeLayout.of(rope))))


def kvfp4_quantize_pages_rope(geometry, rope, hot_pool, packed_pool, num_pages: int,
                              global_scale, src_slots=None, dst_slots=None, stream=None) -> None:
    """kvfp4_quantize_pages into slots of a RoPE layout ``(rope_dims, mode)``."""
    lib = load_library()
    g, r = Geometry.of(geometry), RopeLayout.of(rope)
    _int32(src_slots, "src_slots", int(num_pages))
    _int32(dst_slots, "dst_slots", int(num_pages))
    _check(lib.kvfp4_quantize_pages_rope(
        ctypes.byref(g), ctypes.byref(r), _ptr(hot_pool), _pages(hot_pool, kvfp4_hot_page_bytes(g)),
        _ptr(src_slots), _ptr(packed_pool, host_ok=True),
        _pages(packed_pool, kvfp4_packed_page_bytes_rope(g, r)), _ptr(dst_slots), int(num_pages),
        _scales(global_scale, g.num_kv_tensors), _stream(stream)))


def kvfp4_dequantize_pages_rope(geometry, rope, packed_pool, hot_pool, num_pages: int,
                                global_scale, src_slots=None, dst_slots=None,
                                stream=None) -> None:
    """kvfp4_dequantize_pages from slots of a RoPE layout ``(rope_dims, mode)``."""
    lib = load_library()
    g, r = Geometry.of(geometry), RopeLayout.of(rope)
    _int32(src_slots, "src_slots", int(num_pages))
    _int32(dst_slots, "dst_slots", int(num_pages))
    _check(lib.kvfp4_dequantize_pages_rope(
        ctypes.byref(g), ctypes.byref(r), _ptr(packed_pool, host_ok=True),
        _pages(packed_pool, kvfp4_packed_page_bytes_rope(g, r)), _ptr(src_slots), _ptr(hot_pool),
        _pages(hot_pool, kvfp4_hot_page_bytes(g)), _ptr(dst_slots), int(num_pages),
        _scales(global_scale, g.num_kv_tensors), _stream(stream)))


def kvfp4_append_quantize(geometry, rows, token_slots, token_rows, packed_pool, global_scale,
                          rows_dtype: Optional[int] = None, stream=None) -> None:
    """Quantize ``rows`` (``[num_tokens, n_t, H, D]``: 2-byte elements are
    bf16 bits, 1-byte elements E4M3FN codes unless ``rows_dtype`` says so)
    into row ``token_rows[i]`` of packed slot ``token_slots[i]``."""
    lib = load_library()
    g = Geometry.of(geometry)
    n = int(token_slots.shape[0])
    if int(token_rows.shape[0]) != n:
        raise ValueError("token_slots and token_rows differ in length")
    _int32(token_slots, "token_slots", n)
    _int32(token_rows, "token_rows", n)
    if rows_dtype is None:
        rows_dtype = KVFP4_ROWS_FP8_E4M3 if rows.element_size() == 1 else KVFP4_ROWS_BF16
    width = 1 if rows_dtype == KVFP4_ROWS_FP8_E4M3 else 2
    per_token = g.num_kv_tensors * g.num_kv_heads * g.head_dim
    if rows.numel() * rows.element_size() != n * per_token * width:
        raise ValueError(f"rows holds {rows.numel() * rows.element_size()} bytes, expected "
                         f"{n} tokens x {per_token} values x {width} bytes")
    _check(lib.kvfp4_append_quantize(
        ctypes.byref(g), _ptr(rows), int(rows_dtype), n, _ptr(token_slots), _ptr(token_rows),
        _ptr(packed_pool),
        _pages(packed_pool, kvfp4_packed_page_bytes(g)), _scales(global_scale, g.num_kv_tensors),
        _stream(stream)))


def kvfp4_gather_dequantize(geometry, packed_pool, token_slots, token_rows, out, global_scale,
                            out_dtype: Optional[int] = None, stream=None) -> None:
    """Dequantize row ``token_rows[i]`` of packed slot ``token_slots[i]`` into
    ``out[i]`` (``[num_tokens, n_t, H, D]``: 2-byte elements get bf16 bits,
    1-byte elements E4M3FN codes unless ``out_dtype`` says so)."""
    lib = load_library()
    g = Geometry.of(geometry)
    n = int(token_slots.shape[0])
    if int(token_rows.shape[0]) != n:
        raise ValueError("token_slots and token_rows differ in length")
    _int32(token_slots, "token_slots", n)
    _int32(token_rows, "token_rows", n)
    if out_dtype is None:
        out_dtype = KVFP4_ROWS_FP8_E4M3 if out.element_size() == 1 else KVFP4_ROWS_BF16
    width = 1 if out_dtype == KVFP4_ROWS_FP8_E4M3 else 2
    per_token = g.num_kv_tensors * g.num_kv_heads * g.head_dim
    if out.numel() * out.element_size() != n * per_token * width:
        raise ValueError(f"out holds {out.numel() * out.element_size()} bytes, expected "
                         f"{n} tokens x {per_token} values x {width} bytes")
    _check(lib.kvfp4_gather_dequantize(
        ctypes.byref(g), _ptr(packed_pool), _pages(packed_pool, kvfp4_packed_page_bytes(g)),
        _ptr(token_slots), _ptr(token_rows), n, _ptr(out), int(out_dtype),
        _scales(global_scale, g.num_kv_tensors), _stream(stream)))


def kvfp4_decode_workspace_bytes(geometry, batch: int, num_q_heads: int, v_dim: int,
                                 max_seq_len_hint: int) -> int:
    return int(load_library().kvfp4_decode_workspace_bytes(
        ctypes.byref(Geometry.of(geometry)), int(batch), int(num_q_heads), int(v_dim),
        int(max_seq_len_hint)))


def kvfp4_paged_decode_attention(geometry, packed_pool, global_scale, q, block_table, seq_lens,
                                 max_seq_len_hint: int, softmax_scale: float, out, lse=None,
                                 workspace=None, v_dim: Optional[int] = None,
                                 stream=None) -> None:
    """Decode attention over the packed cache; writes ``out`` (bf16 bits or
    bf16 tensor ``[B, Hq, v_dim]``) and, if given, ``lse`` (fp32 ``[B, Hq]``)."""
    lib = load_library()
    g = Geometry.of(geometry)
    vd = int(v_dim if v_dim is not None else out.shape[-1])
    _check_decode_args(g, q, out, lse, block_table, seq_lens, vd)
    B, Hq = int(q.shape[0]), int(q.shape[1])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.kvfp4_paged_decode_attention(
        ctypes.byref(g), _ptr(packed_pool), _pages(packed_pool, kvfp4_packed_page_bytes(g)),
        _scales(global_scale, g.num_kv_tensors), _ptr(q), B, Hq, vd, _ptr(block_table),
        int(block_table.shape[1]), _ptr(seq_lens), int(max_seq_len_hint), float(softmax_scale),
        _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)))


def kvfp4_paged_decode_attention_noalloc(geometry, packed_pool, global_scale, q, block_table,
                                         seq_lens, max_seq_len_hint: int, softmax_scale: float,
                                         out, lse=None, v_dim: Optional[int] = None,
                                         stream=None) -> None:
    """kvfp4_paged_decode_attention with the library's own scratch instead
    of a workspace (for callers that cannot allocate; see the header for the
    size limit and the rule that calls on one device must not overlap)."""
    lib = load_library()
    g = Geometry.of(geometry)
    vd = int(v_dim if v_dim is not None else out.shape[-1])
    _check_decode_args(g, q, out, lse, block_table, seq_lens, vd)
    B, Hq = int(q.shape[0]), int(q.shape[1])
    _check(lib.kvfp4_paged_decode_attention_noalloc(
        ctypes.byref(g), _ptr(packed_pool), _pages(packed_pool, kvfp4_packed_page_bytes(g)),
        _scales(global_scale, g.num_kv_tensors), _ptr(q), B, Hq, vd, _ptr(block_table),
        int(block_table.shape[1]), _ptr(seq_lens), int(max_seq_len_hint), float(softmax_scale),
        _ptr(out), _ptr(lse), _stream(stream)))
