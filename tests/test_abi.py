"""Host-only checks of the C ABI: the library loads, exports every function
include/kvfp4.h declares, and rejects invalid arguments before launching
anything (no GPU needed; no call here reaches a kernel launch)."""

import ctypes
import os
import re

import pytest

import nvfp4_paged_decode_amd as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    src = open(os.path.join(ROOT, "include", "kvfp4.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvfp4_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(K.library_path()):
        pytest.fail("libkvfp4.so is not built (python -m nvfp4_paged_decode_amd.build)")
    return K.load_library()


def test_exports_every_declared_function(lib):
    declared = _header_functions()
    assert declared == sorted(K.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_page_sizes(lib):
    g = K.Geometry(2, 64, 8, 128)
    assert lib.kvfp4_hot_page_bytes(ctypes.byref(g)) == 262144
    assert lib.kvfp4_packed_page_bytes(ctypes.byref(g)) == 73728
    mla = K.Geometry(1, 64, 1, 576)
    assert lib.kvfp4_packed_page_bytes(ctypes.byref(mla)) == 64 * 576 * 9 // 16
    for bad in [(3, 64, 8, 128), (2, 64, 8, 120), (2, 0, 8, 128), (2, 64, -1, 128)]:
        assert lib.kvfp4_packed_page_bytes(ctypes.byref(K.Geometry(*bad))) == 0
    assert lib.kvfp4_hot_page_bytes(None) == 0


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def _q(lib, g, num_pages=4, gs=(1.0, 1.0), hot=FAKE, packed=FAKE, hot_pages=8, packed_pages=8):
    arr = (ctypes.c_float * 2)(*gs)
    return lib.kvfp4_quantize_pages(ctypes.byref(g) if g is not None else None, hot, hot_pages,
                                    None, packed, packed_pages, None, num_pages, arr, None)


@pytest.mark.parametrize("case,msg", [
    (dict(n=-1), "num_pages"),
    (dict(key=None), "NULL key"),
    (dict(key_out=None), "NULL key"),
    (dict(other_out=None), "both"),                     # other given, other_out missing
    (dict(other=None), "both"),
    (dict(key_out=FAKE + 8), "overlap"),               # into key's 16 bytes
    (dict(other_out=0x3000 - 4), "overlap"),           # ends inside key_out
    (dict(other_out=0x2000), "overlap"),               # same as other
])
def test_sort_rejects_invalid_arguments(lib, case, msg):
    """kvfp4_sort_page_list validates before launching anything (pointers
    are never dereferenced: every call here fails validation)."""
    a = dict(key=FAKE, other=0x2000, n=4, key_out=0x3000, other_out=0x4000)
    a.update(case)
    st = lib.kvfp4_sort_page_list(a["key"], a["other"], a["n"], a["key_out"], a["other_out"],
                                  None)
    assert st == K.KVFP4_ERR_INVALID_ARG
    assert msg in lib.kvfp4_last_error_message().decode()


def test_sort_zero_pages_is_a_noop(lib):
    assert lib.kvfp4_sort_page_list(None, None, 0, None, None, None) == K.KVFP4_OK


@pytest.mark.parametrize("case", [
    dict(g=None),
    dict(g=K.Geometry(2, 64, 8, 100)),
    dict(g=K.Geometry(0, 64, 8, 128)),
    dict(num_pages=-1),
    dict(hot=None),
    dict(packed=None),
    dict(hot=FAKE, packed=FAKE),  # aliasing pools
    dict(num_pages=9),            # more pages than the pool with identity slots
    dict(gs=(0.0, 1.0)),
    dict(gs=(1.0, -2.0)),
    dict(gs=(float("nan"), 1.0)),
    dict(gs=(float("inf"), 1.0)),
    dict(gs=(1e36, 1.0)),         # 2688 * gs overflows fp32
])
def test_codec_rejects_invalid_arguments(lib, case):
    g = case.pop("g", K.Geometry(2, 64, 8, 128))
    if case.get("hot") == FAKE and case.get("packed") == FAKE:
        st = _q(lib, g, **case)
    else:
        case.setdefault("packed", FAKE + 0x100)
        st = _q(lib, g, **case)
    assert st == K.KVFP4_ERR_INVALID_ARG
    assert lib.kvfp4_last_error_message().decode() != ""
    # the same validation guards the dequantizer
    arr = (ctypes.c_float * 2)(*case.get("gs", (1.0, 1.0)))
    st2 = lib.kvfp4_dequantize_pages(ctypes.byref(g) if g is not None else None,
                                     case.get("packed", FAKE + 0x100), 8, None,
                                     case.get("hot", FAKE), 8, None, case.get("num_pages", 4),
                                     arr, None)
    assert st2 == K.KVFP4_ERR_INVALID_ARG


def test_codec_zero_pages_is_a_noop(lib):
    g = K.Geometry(2, 64, 8, 128)
    arr = (ctypes.c_float * 2)(1.0, 1.0)
    assert lib.kvfp4_quantize_pages(ctypes.byref(g), None, 0, None, None, 0, None, 0, arr,
                                    None) == K.KVFP4_OK


def _append(lib, g, num_tokens=4, gs=(1.0, 1.0), rows=FAKE, slots=FAKE + 0x200,
            prows=FAKE + 0x300, packed=FAKE + 0x400, packed_pages=8, dtype=K.KVFP4_ROWS_BF16):
    arr = (ctypes.c_float * 2)(*gs)
    return lib.kvfp4_append_quantize(ctypes.byref(g) if g is not None else None, rows, dtype,
                                     num_tokens, slots, prows, packed, packed_pages, arr, None)


@pytest.mark.parametrize("case", [
    dict(g=None),
    dict(g=K.Geometry(2, 64, 8, 120)),
    dict(num_tokens=-1),
    dict(packed_pages=-1),
    dict(rows=None),
    dict(slots=None),
    dict(prows=None),
    dict(packed=None),
    dict(rows=FAKE + 8),              # rows must be 16-byte aligned
    dict(rows=FAKE + 8, dtype=K.KVFP4_ROWS_FP8_E4M3),
    dict(dtype=2),
    dict(dtype=-1),
    dict(num_tokens=1 << 30),         # 2^30 tokens x 2048 values overflow the index space
    dict(gs=(0.0, 1.0)),
    dict(gs=(1.0, float("nan"))),
    dict(gs=(1e36, 1.0)),
])
def test_append_rejects_invalid_arguments(lib, case):
    g = case.pop("g", K.Geometry(2, 64, 8, 128))
    assert _append(lib, g, **case) == K.KVFP4_ERR_INVALID_ARG
    assert lib.kvfp4_last_error_message().decode() != ""


def test_append_zero_tokens_is_a_noop(lib):
    assert _append(lib, K.Geometry(2, 64, 8, 128), num_tokens=0, rows=None, slots=None,
                   prows=None, packed=None) == K.KVFP4_OK


def _gather(lib, g, num_tokens=4, gs=(1.0, 1.0), packed=FAKE, slots=FAKE + 0x200,
            prows=FAKE + 0x300, out=FAKE + 0x400, packed_pages=8, dtype=K.KVFP4_ROWS_BF16):
    arr = (ctypes.c_float * 2)(*gs)
    return lib.kvfp4_gather_dequantize(ctypes.byref(g) if g is not None else None, packed,
                                       packed_pages, slots, prows, num_tokens, out, dtype, arr,
                                       None)


@pytest.mark.parametrize("case", [
    dict(g=None),
    dict(g=K.Geometry(1, 64, 1, 500)),
    dict(num_tokens=-1),
    dict(packed_pages=-1),
    dict(packed=None),
    dict(slots=None),
    dict(prows=None),
    dict(out=None),
    dict(out=FAKE + 8),                               # bf16 rows need 16-byte alignment
    dict(out=FAKE + 4, dtype=K.KVFP4_ROWS_FP8_E4M3),  # FP8 rows need 8
    dict(dtype=7),
    dict(num_tokens=1 << 30),
    dict(gs=(-1.0, 1.0)),
])
def test_gather_rejects_invalid_arguments(lib, case):
    g = case.pop("g", K.Geometry(2, 64, 8, 128))
    assert _gather(lib, g, **case) == K.KVFP4_ERR_INVALID_ARG
    assert lib.kvfp4_last_error_message().decode() != ""


def test_gather_zero_tokens_is_a_noop(lib):
    assert _gather(lib, K.Geometry(2, 64, 8, 128), num_tokens=0, packed=None, slots=None,
                   prows=None, out=None) == K.KVFP4_OK


def _decode(lib, g, gs=(1.0, 1.0), batch=2, hq=32, v_dim=128, hint=1024, ws=0, wsptr=None,
            pool=FAKE, q=FAKE, bt=FAKE, sl=FAKE, out=FAKE, scale=0.088, max_pages=16,
            pool_pages=64):
    arr = (ctypes.c_float * 2)(*gs)
    return lib.kvfp4_paged_decode_attention(
        ctypes.byref(g) if g is not None else None, pool, pool_pages, arr, q, batch, hq, v_dim,
        bt, max_pages, sl, hint, ctypes.c_float(scale), out, None, wsptr, ws, None)


@pytest.mark.parametrize("case,code", [
    (dict(g=None), K.KVFP4_ERR_INVALID_ARG),
    (dict(hq=30), K.KVFP4_ERR_INVALID_ARG),      # not a multiple of 8 KV heads
    (dict(v_dim=64), K.KVFP4_ERR_INVALID_ARG),   # K and V need v_dim == head_dim
    (dict(v_dim=0), K.KVFP4_ERR_INVALID_ARG),
    (dict(batch=-1), K.KVFP4_ERR_INVALID_ARG),
    (dict(hint=-5), K.KVFP4_ERR_INVALID_ARG),
    (dict(q=None), K.KVFP4_ERR_INVALID_ARG),
    (dict(bt=None), K.KVFP4_ERR_INVALID_ARG),
    (dict(out=None), K.KVFP4_ERR_INVALID_ARG),
    (dict(max_pages=0), K.KVFP4_ERR_INVALID_ARG),
    (dict(pool_pages=0), K.KVFP4_ERR_INVALID_ARG),
    (dict(scale=float("nan")), K.KVFP4_ERR_INVALID_ARG),
    (dict(gs=(1.0, 0.0)), K.KVFP4_ERR_INVALID_ARG),
    (dict(ws=0), K.KVFP4_ERR_WORKSPACE),          # workspace too small
    (dict(ws=1 << 30, wsptr=FAKE + 4), K.KVFP4_ERR_INVALID_ARG),  # misaligned workspace
    (dict(ws=1 << 30, wsptr=FAKE, q=FAKE + 2), K.KVFP4_ERR_INVALID_ARG),  # misaligned q
    (dict(g=K.Geometry(2, 64, 8, 640), v_dim=640), K.KVFP4_ERR_UNSUPPORTED),
])
def test_decode_rejects_invalid_arguments(lib, case, code):
    g = case.pop("g", K.Geometry(2, 64, 8, 128))
    assert _decode(lib, g, **case) == code
    assert lib.kvfp4_last_error_message().decode() != ""


def test_decode_workspace_size(lib):
    g = K.Geometry(2, 64, 8, 128)
    n = lib.kvfp4_decode_workspace_bytes(ctypes.byref(g), 32, 32, 128, 8192)
    # partials (128 fp16 dims, fp32 m and l) for (workgroups + batch) x 32
    # heads, then the merge index (first/last workgroup per sequence and the
    # page count)
    index = -(-(2 * 32 + 1) * 4 // 16) * 16
    assert n > index and (n - index) % (32 * (128 * 2 + 2 * 4)) == 0
    assert lib.kvfp4_decode_workspace_bytes(ctypes.byref(g), 32, 30, 128, 8192) == 0
    assert lib.kvfp4_decode_workspace_bytes(ctypes.byref(g), 0, 32, 128, 8192) == 0


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4, 7):
        assert lib.kvfp4_status_string(s).decode()


def test_python_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(K, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(K, "_lib", None)
    with pytest.raises(ImportError):
        K.load_library()


def test_binding_rejects_pageable_host_tensors():
    import torch
    t = torch.zeros(16, dtype=torch.uint8)
    with pytest.raises(ValueError):
        K._ptr(t)
    with pytest.raises(ValueError):
        K._ptr(t, host_ok=True)  # pageable host memory is not mapped for the GPU
    assert K._ptr(None) is None


def test_rope_page_sizes(lib):
    g = K.Geometry(1, 64, 1, 576)
    base = 64 * 576 * 9 // 16
    sizes = [K.kvfp4_packed_page_bytes_rope(g, (64, m)) for m in range(3)]
    assert sizes == [base, base + 64 * 64 * 2, base + 64 * 64 * 9 // 16]
    for bad in [(0, 1), (8, 1), (592, 1), (64, 3), (64, -1)]:
        assert K.kvfp4_packed_page_bytes_rope(g, bad) == 0
    assert lib.kvfp4_packed_page_bytes_rope(ctypes.byref(g), None) == 0


@pytest.mark.parametrize("rope,code", [
    (None, K.KVFP4_ERR_INVALID_ARG),
    ((0, 2), K.KVFP4_ERR_INVALID_ARG),
    ((24, 2), K.KVFP4_ERR_INVALID_ARG),
    ((144, 2), K.KVFP4_ERR_INVALID_ARG),   # more than head_dim
    ((64, 5), K.KVFP4_ERR_INVALID_ARG),
])
def test_rope_codec_rejects_invalid_layouts(lib, rope, code):
    g = K.Geometry(2, 64, 8, 128)
    arr = (ctypes.c_float * 2)(1.0, 1.0)
    r = ctypes.byref(K.RopeLayout(*rope)) if rope is not None else None
    for fn in (lib.kvfp4_quantize_pages_rope, lib.kvfp4_dequantize_pages_rope):
        st = fn(ctypes.byref(g), r, FAKE, 8, None, FAKE + 0x100, 8, None, 4, arr, None)
        assert st == code
        assert lib.kvfp4_last_error_message().decode() != ""


def test_rope_codec_needs_16_byte_slots(lib):
    # 4 tokens x 1 head x 16 dims: a 36-byte plain slot
    g = K.Geometry(1, 4, 1, 16)
    arr = (ctypes.c_float * 1)(1.0)
    st = lib.kvfp4_quantize_pages_rope(ctypes.byref(g), ctypes.byref(K.RopeLayout(16, 2)), FAKE,
                                       8, None, FAKE + 0x100, 8, None, 4, arr, None)
    assert st == K.KVFP4_ERR_UNSUPPORTED
    # the plain codec takes the same geometry
    assert lib.kvfp4_quantize_pages(ctypes.byref(g), None, 0, None, None, 0, None, 0, arr,
                                    None) == K.KVFP4_OK


@pytest.mark.parametrize("geom,hq,balanced", [
    ((2, 64, 8, 128), 32, True),      # 4 query heads per KV head
    ((2, 64, 8, 128), 8, True),       # one query head per KV head: padded columns
    ((2, 64, 4, 128), 28, True),      # 7 per KV head
    ((2, 16, 2, 128), 16, True),      # 2 KV heads: padded KV-head slots
    ((2, 16, 10, 128), 40, True),     # 10 KV heads
    ((1, 64, 1, 576), 128, True),     # MLA
    ((2, 16, 16, 128), 256, False),   # 16 x 16: more wave groups than a workgroup has
    ((2, 64, 4, 256), 16, False),     # head_dim 256
])
def test_decode_routing_by_workspace(lib, geom, hq, balanced):
    """The workspace size tells which plan a shape gets: the balanced
    kernels hold (workgroups + batch) partial rows (fp16 outputs, fp32 max
    and sum) and the merge index, the generic kernel batch x heads x splits
    rows of fp32.  Without a GPU the plan assumes 256 compute units."""
    g = K.Geometry(*geom)
    batch, hint = 4, 1024
    v = 512 if geom[0] == 1 else geom[3]
    n = lib.kvfp4_decode_workspace_bytes(ctypes.byref(g), batch, hq, v, hint)
    row = hq * (v * 2 + 2 * 4)
    index = -(-(2 * batch + 1) * 4 // 16) * 16
    pages = batch * -(-hint // geom[1])
    balanced_bytes = (min(256, pages) + batch) * row + index
    if balanced:
        assert n == balanced_bytes
    else:
        assert n != balanced_bytes and n % (hq * (v + 2) * 4) == 0


# --- the Python binding's checks, made before any pointer is taken --------
# CPU tensors stand in for device tensors: every call below is turned away
# by a shape or dtype check that runs before the pointer check.

def _decode_call(**over):
    torch = pytest.importorskip("torch")
    B, Hq, D = 2, 8, 128
    args = dict(
        geometry=(2, 64, 2, D), packed_pool=torch.zeros(4, 64, dtype=torch.uint8),
        global_scale=[1.0, 1.0], q=torch.zeros(B, Hq, D, dtype=torch.int16),
        block_table=torch.zeros(B, 4, dtype=torch.int32),
        seq_lens=torch.zeros(B, dtype=torch.int32), max_seq_len_hint=256,
        softmax_scale=0.1, out=torch.zeros(B, Hq, D, dtype=torch.int16),
        lse=torch.zeros(B, Hq, dtype=torch.float32), workspace=None, v_dim=D)
    args.update(over)
    K.kvfp4_paged_decode_attention(**args)


@pytest.mark.parametrize("name,make,msg", [
    ("block_table", lambda t: t.zeros(2, 4, dtype=t.int64), "int32"),
    ("block_table", lambda t: t.zeros(8, dtype=t.int32), "2-d"),
    ("block_table", lambda t: t.zeros(1, 4, dtype=t.int32), "rows"),
    ("seq_lens", lambda t: t.zeros(2, dtype=t.int64), "int32"),
    ("seq_lens", lambda t: t.zeros(1, dtype=t.int32), "at least 2"),
    ("q", lambda t: t.zeros(2, 8, 128, dtype=t.float32), "2-byte"),
    ("q", lambda t: t.zeros(2, 8, 64, dtype=t.int16), "head_dim"),
    ("q", lambda t: t.zeros(16, 128, dtype=t.int16), "3-d"),
    ("out", lambda t: t.zeros(2 * 8 * 128 - 1, dtype=t.int16), "needs"),
    ("out", lambda t: t.zeros(2, 8, 128, dtype=t.float32), "2-byte"),
    ("lse", lambda t: t.zeros(2, 7, dtype=t.float32), "needs"),
    ("lse", lambda t: t.zeros(2, 8, dtype=t.float64), "float32"),
])
def test_binding_rejects_decode_tensor(lib, name, make, msg):
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError, match=msg):
        _decode_call(**{name: make(torch)})


@pytest.mark.parametrize("fn", ["kvfp4_quantize_pages", "kvfp4_dequantize_pages"])
@pytest.mark.parametrize("which,make,msg", [
    ("src_slots", lambda t: t.arange(4, dtype=t.int64), "int32"),
    ("dst_slots", lambda t: t.arange(4, dtype=t.int64), "int32"),
    ("src_slots", lambda t: t.arange(3, dtype=t.int32), "at least 4"),
    ("dst_slots", lambda t: t.arange(3, dtype=t.int32), "at least 4"),
])
def test_binding_rejects_codec_slots(lib, fn, which, make, msg):
    torch = pytest.importorskip("torch")
    g = (2, 64, 8, 128)
    a = torch.zeros(8, 16, dtype=torch.uint8)
    b = torch.zeros(8, 16, dtype=torch.uint8)
    with pytest.raises(ValueError, match=msg):
        getattr(K, fn)(g, a, b, 4, [1.0, 1.0], **{which: make(torch)})


@pytest.mark.parametrize("fn", ["kvfp4_quantize_pages_rope", "kvfp4_dequantize_pages_rope"])
def test_binding_rejects_rope_codec_slots(lib, fn):
    torch = pytest.importorskip("torch")
    a = torch.zeros(8, 16, dtype=torch.uint8)
    b = torch.zeros(8, 16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="int32"):
        getattr(K, fn)((2, 64, 8, 128), (64, 1), a, b, 4, [1.0, 1.0],
                       src_slots=torch.arange(4, dtype=torch.int64))


@pytest.mark.parametrize("fn", ["kvfp4_append_quantize", "kvfp4_gather_dequantize"])
@pytest.mark.parametrize("which", ["token_slots", "token_rows"])
def test_binding_rejects_token_index_dtype(lib, fn, which):
    torch = pytest.importorskip("torch")
    n = 4
    idx = {"token_slots": torch.zeros(n, dtype=torch.int32),
           "token_rows": torch.zeros(n, dtype=torch.int32)}
    idx[which] = torch.zeros(n, dtype=torch.int64)
    rows = torch.zeros(n, 2, 8, 128, dtype=torch.int16)
    pool = torch.zeros(8, 16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="int32"):
        if fn == "kvfp4_append_quantize":
            K.kvfp4_append_quantize((2, 64, 8, 128), rows, idx["token_slots"], idx["token_rows"],
                                    pool, [1.0, 1.0])
        else:
            K.kvfp4_gather_dequantize((2, 64, 8, 128), pool, idx["token_slots"],
                                      idx["token_rows"], rows, [1.0, 1.0])


def test_noalloc_rejects_sizes_beyond_its_scratch(lib):
    """Sizes whose split-K workspace exceeds the allocation-free entry
    point's 96 MiB scratch are rejected before anything is launched (the
    pointers below are never dereferenced)."""
    g = K.Geometry(1, 64, 1, 576)
    need = lib.kvfp4_decode_workspace_bytes(ctypes.byref(g), 4096, 128, 512, 16384)
    assert need > 96 << 20
    gs = (ctypes.c_float * 1)(1.0)
    st = lib.kvfp4_paged_decode_attention_noalloc(
        ctypes.byref(g), FAKE, 8, gs, FAKE, 4096, 128, 512, FAKE + 0x100, 256, FAKE + 0x200,
        16384, 0.04, FAKE + 0x300, None, None)
    assert st == K.KVFP4_ERR_WORKSPACE
    assert "allocation-free" in lib.kvfp4_last_error_message().decode()
