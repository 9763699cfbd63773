"""The whole step (encode pages, decode attention, decode pages) captured
into a HIP graph through torch and replayed: every replay must reproduce
the eager results bit for bit.  The calls allocate nothing, launch no
memset, and set their kernels' LDS limits outside capture (first eager
call), so a serving loop can capture them."""

import numpy as np
import pytest

import nvfp4_paged_decode_amd as K
from nvfp4_paged_decode_amd import workloads as W
from tests.gpu_common import dev, require_gpu, torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["llama", "mla"])
def test_step_replays_from_a_graph(name):
    require_gpu()
    if name == "llama":
        wl = W.llama3_8b(seed=12, batch=4, context=1000)
    else:
        wl = W.mla(seed=13, batch=2, context=700, num_q_heads=32)
    gs = [float(v) for v in wl.gs_calibrated]
    hot = dev(wl.hot_pool.view(np.int16))
    slots = dev(wl.used_slots.astype(np.int32))
    n = int(wl.used_slots.shape[0])
    pb = K.kvfp4_packed_page_bytes(wl.geometry)
    packed = torch.zeros((wl.num_slots, pb), dtype=torch.uint8, device="cuda")
    back = torch.zeros_like(hot)
    q, bt = dev(wl.q.view(np.int16)), dev(wl.block_table)
    sl = dev(wl.seq_lens.astype(np.int32))
    hint = int(wl.seq_lens.max())
    ws = torch.empty(max(4, K.kvfp4_decode_workspace_bytes(wl.geometry, wl.batch, wl.num_q_heads,
                                                           wl.v_dim, hint)),
                     dtype=torch.uint8, device="cuda")
    out = torch.zeros((wl.batch, wl.num_q_heads, wl.v_dim), dtype=torch.int16, device="cuda")
    lse = torch.zeros((wl.batch, wl.num_q_heads), dtype=torch.float32, device="cuda")

    def step():
        K.kvfp4_quantize_pages(wl.geometry, hot, packed, n, gs, slots, slots)
        K.kvfp4_paged_decode_attention(wl.geometry, packed, gs, q, bt, sl, hint, wl.softmax_scale,
                                       out, lse, ws, v_dim=wl.v_dim)
        K.kvfp4_dequantize_pages(wl.geometry, packed, back, n, gs, slots, slots)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (packed, out, lse, back)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for replay in range(3):
        for t in (packed, out, lse, back):  # eager work between replays
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for what, got, want in zip(("packed", "out", "lse", "back"), (packed, out, lse, back), ref):
            assert torch.equal(got, want), f"replay {replay}: {what} differs"
