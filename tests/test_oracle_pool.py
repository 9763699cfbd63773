"""The process-pool front end of the oracle gives exactly the serial
oracle's results (chunking, ordering and worker start-up are plumbing only)."""

import numpy as np

from nvfp4_paged_decode_amd import workloads as W
from oracle import attention as A
from oracle import nvfp4 as O
from tests import oracle_pool as P


def test_pool_matches_serial_oracle():
    wl = W.llama3_8b(seed=41, batch=3, context=300)
    gs = wl.gs_calibrated
    g = O.Geometry(*wl.geometry)
    slots = wl.used_slots
    serial = np.zeros((len(slots), O.packed_page_bytes(g)), np.uint8)
    O.quantize_pages(wl.hot_pool[slots], g, len(slots), gs, serial)
    with P.make_pool(2) as pool:
        enc = P.encode_pages(pool, wl.hot_pool, wl.geometry, gs, slots)
        assert np.array_equal(enc, serial)
        dec = P.decode_pages(pool, enc, wl.geometry, gs)
        packed = np.zeros((wl.num_slots, O.packed_page_bytes(g)), np.uint8)
        packed[slots] = enc
        out, lse = P.decode_attention_all(pool, packed, wl, gs)
    ref_dec = np.zeros_like(dec)
    O.dequantize_pages(serial, g, len(slots), gs, ref_dec)
    assert np.array_equal(dec, ref_dec)
    ref, ref_lse = A.decode_attention(packed, g, gs, wl.q, wl.block_table, wl.seq_lens,
                                      wl.softmax_scale, wl.v_dim)
    assert np.array_equal(out, ref) and np.array_equal(lse, ref_lse)


def test_worker_count_is_bounded():
    assert 1 <= P.workers() <= P.MAX_WORKERS
