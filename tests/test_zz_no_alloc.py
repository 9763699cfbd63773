"""The allocation-free decode entry point (kvfp4_paged_decode_attention_noalloc),
called through the C ABI, against the workspace entry point on the same
inputs: the same kernels and split-K plan, so every output and lse must be
bit-identical.  Two calls in a row on one device, the second smaller, so the
second reads a scratch array the first left full."""

import ctypes

import numpy as np
import pytest

import nvfp4_paged_decode_amd as K
from nvfp4_paged_decode_amd import workloads as W
from tests.gpu_common import dev, host, oracle_packed_pages, poison_unread, require_gpu, torch

pytestmark = pytest.mark.gpu


def _pool(wl, gs):
    packed = oracle_packed_pages(wl.hot_pool, wl.geometry, gs, np.arange(wl.num_slots))
    poison_unread(packed, wl, np.random.default_rng(5))
    return packed


def _noalloc_abi(wl, packed_d, gs, q_d, bt_d, sl_d, out, lse):
    """One call of the C entry point itself (ctypes, no binding helper)."""
    lib = K.load_library()
    g = K.Geometry(*wl.geometry)
    gsa = (ctypes.c_float * len(gs))(*[float(v) for v in gs])
    st = lib.kvfp4_paged_decode_attention_noalloc(
        ctypes.byref(g), packed_d.data_ptr(), int(packed_d.shape[0]), gsa, q_d.data_ptr(),
        wl.batch, wl.num_q_heads, wl.v_dim, bt_d.data_ptr(), int(bt_d.shape[1]),
        sl_d.data_ptr(), int(wl.seq_lens.max()), float(wl.softmax_scale), out.data_ptr(),
        lse.data_ptr(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.kvfp4_last_error_message().decode()


def _both(wl):
    gs = wl.gs_calibrated
    packed_d = dev(_pool(wl, gs))
    q_d = dev(wl.q.view(np.int16))
    bt_d, sl_d = dev(wl.block_table), dev(wl.seq_lens)
    B, Hq, hint = wl.batch, wl.num_q_heads, int(wl.seq_lens.max())
    ws = torch.empty(max(16, K.kvfp4_decode_workspace_bytes(wl.geometry, B, Hq, wl.v_dim, hint)),
                     dtype=torch.uint8, device="cuda")
    out_ws = torch.empty((B, Hq, wl.v_dim), dtype=torch.int16, device="cuda")
    lse_ws = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    K.kvfp4_paged_decode_attention(wl.geometry, packed_d, gs, q_d, bt_d, sl_d, hint,
                                   wl.softmax_scale, out_ws, lse_ws, ws, v_dim=wl.v_dim)
    out_na = torch.full((B, Hq, wl.v_dim), 0x7FC0, dtype=torch.int16, device="cuda")
    lse_na = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    _noalloc_abi(wl, packed_d, gs, q_d, bt_d, sl_d, out_na, lse_na)
    return host(out_ws), host(lse_ws), host(out_na), host(lse_na)


CASES = {
    "gqa": [lambda: W.llama3_8b(seed=31, batch=12, context=3000),
            lambda: W.llama3_8b(seed=32, batch=3, context=200)],
    "mla": [lambda: W.mla(seed=33, batch=6, context=900),
            lambda: W.mla(seed=34, batch=2, context=130)],
}


@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_equals_workspace_entry_point(name):
    require_gpu()
    for make in CASES[name]:  # the second call is smaller than the first
        wl = make()
        o_ws, l_ws, o_na, l_na = _both(wl)
        assert np.array_equal(o_na, o_ws), f"{name} {wl.name}: outputs differ"
        assert np.array_equal(l_na.view(np.uint32), l_ws.view(np.uint32)), f"{name}: lse differs"
