"""GPU parity of paged NVFP4 decode attention against the fp64 oracle:
every output within 1e-2 + 1e-2 |ref|, lse within 1e-3 + 1e-3 |ref|."""

import numpy as np
import pytest

import nvfp4_paged_decode_amd as K
from nvfp4_paged_decode_amd import workloads as W
from oracle import nvfp4 as O
from tests import oracle_pool as P
from tests.gpu_common import (assert_attention_close, dev, host, oracle_attention,
                              oracle_packed_pages, poison_unread, require_gpu, torch)

pytestmark = pytest.mark.gpu


def gpu_decode(wl, packed_d, gs, hint=None, seq_lens=None):
    B, Hq = wl.batch, wl.num_q_heads
    hint = int(wl.seq_lens.max()) if hint is None else hint
    ws_bytes = K.kvfp4_decode_workspace_bytes(wl.geometry, B, Hq, wl.v_dim, hint)
    ws = torch.empty(max(ws_bytes, 4), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, wl.v_dim), dtype=torch.int16, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    sl = wl.seq_lens if seq_lens is None else seq_lens
    K.kvfp4_paged_decode_attention(wl.geometry, packed_d, gs, dev(wl.q.view(np.int16)),
                                   dev(wl.block_table), dev(sl.astype(np.int32)), hint,
                                   wl.softmax_scale, out, lse, ws, v_dim=wl.v_dim)
    return host(out).view(np.uint16), host(lse)


def oracle_pool(wl, gs, poison_seed=0):
    packed = oracle_packed_pages(wl.hot_pool, wl.geometry, gs, np.arange(wl.num_slots))
    poison_unread(packed, wl, np.random.default_rng(poison_seed))
    return packed


def check(wl, gs, packed, out, lse, batch_indices=None, head_indices=None, what=""):
    ref, ref_lse = oracle_attention(packed, wl, gs, batch_indices, head_indices)
    bi = slice(None) if batch_indices is None else np.asarray(batch_indices)
    o = out[bi]
    l = lse[bi]
    if head_indices is not None:
        o = o[:, np.asarray(head_indices)]
        l = l[:, np.asarray(head_indices)]
    assert_attention_close(o, ref, what)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(l)), f"{what}: lse finiteness"
    assert np.all(np.abs(l[fin] - ref_lse[fin]) <= 1e-3 + 1e-3 * np.abs(ref_lse[fin])), what


SMALL = {
    "tiny": lambda: W.tiny(),
    "llama3_ragged": lambda: W.llama3_8b(seed=12, batch=3, context=300),
    "qwen3_ragged": lambda: W.qwen3_8b_long(seed=13, batch=3, lo=1, hi=700),
    "mla_ragged": lambda: W.mla(seed=15, batch=2, context=200),
    "mla_16_heads": lambda: W.mla(seed=16, batch=3, context=130, num_q_heads=16),
}


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("gs_kind", ["unit", "calibrated"])
def test_decode_small_all_outputs(name, gs_kind):
    require_gpu()
    wl = SMALL[name]()
    gs = wl.gs_unit if gs_kind == "unit" else wl.gs_calibrated
    packed = oracle_pool(wl, gs)
    out, lse = gpu_decode(wl, dev(packed), gs)
    check(wl, gs, packed, out, lse, what=f"{name}/{gs_kind}")


def test_decode_edge_lengths():
    """Empty sequences, one token, exact page multiples and a page-table row
    used to the last entry, in one batch."""
    require_gpu()
    wl = W.llama3_8b(seed=17, batch=6, context=256)
    wl.seq_lens[:] = [0, 1, 64, 256, 63, 65]
    gs = wl.gs_calibrated
    packed = oracle_pool(wl, gs)
    out, lse = gpu_decode(wl, dev(packed), gs, hint=256)
    check(wl, gs, packed, out, lse, what="edge lengths")
    assert np.all(out[0] == 0) and np.all(lse[0] == -np.inf)


def test_decode_hint_larger_than_lengths():
    require_gpu()
    wl = W.qwen3_8b_long(seed=18, batch=2, lo=50, hi=300)
    gs = wl.gs_unit
    packed = oracle_pool(wl, gs)
    out, lse = gpu_decode(wl, dev(packed), gs, hint=int(wl.max_pages_per_seq * wl.page_size))
    check(wl, gs, packed, out, lse, what="large hint")


# (nt, T, H, D, Hq, v_dim): every decode kernel and its template variants
GEOMETRIES = {
    "mfma_gqa_T16_H4": (2, 16, 4, 128, 16, 128),
    "mfma_gqa_T32_H16": (2, 32, 16, 128, 64, 128),
    "mfma_gqa_T128_H32": (2, 128, 32, 128, 128, 128),
    "mfma_gqa_G8_H8_T64": (2, 64, 8, 128, 64, 128),
    "mfma_gqa_G8_H4_T32": (2, 32, 4, 128, 32, 128),
    "mfma_gqa_G8_H16_T16": (2, 16, 16, 128, 128, 128),
    "mfma_gqa_G16_H4_T16": (2, 16, 4, 128, 64, 128),
    "mfma_gqa_G16_H8_T64": (2, 64, 8, 128, 128, 128),
    "mfma_gqa_D64_T16_H4": (2, 16, 4, 64, 16, 64),
    "mfma_gqa_D64_G8_H8_T32": (2, 32, 8, 64, 64, 64),
    "mfma_gqa_D64_G16_H8_T64": (2, 64, 8, 64, 128, 64),
    "mfma_gqa_D64_T128_H32": (2, 128, 32, 64, 128, 64),
    "generic_G16_H16": (2, 16, 16, 128, 256, 128),  # 16 wave groups: past the MFMA kernel
    "mfma_gqa_G1_H8": (2, 64, 8, 128, 8, 128),      # padded query columns: 1 of 4 used
    "mfma_gqa_G2_H16": (2, 32, 16, 128, 32, 128),
    "mfma_gqa_G3_H32_D64": (2, 16, 32, 64, 96, 64),
    "mfma_gqa_G5_H8": (2, 64, 8, 128, 40, 128),       # 5 of 8 columns
    "mfma_gqa_G7_H4": (2, 16, 4, 128, 28, 128),       # 28 q / 4 KV heads
    "mfma_gqa_G10_H8": (2, 16, 8, 128, 80, 128),      # 10 of 16 columns
    "mfma_gqa_G12_H4": (2, 16, 4, 128, 48, 128),
    "mfma_gqa_H2_G8": (2, 16, 2, 128, 16, 128),       # KV-head slots padded to 4
    "mfma_gqa_H2_G6_D64": (2, 32, 2, 64, 12, 64),
    "mfma_gqa_H3_G7": (2, 16, 3, 128, 21, 128),
    "mfma_gqa_H1_G16": (2, 16, 1, 128, 16, 128),
    "mfma_gqa_H6_G2": (2, 64, 6, 128, 12, 128),
    "mfma_gqa_H10_G4": (2, 16, 10, 128, 40, 128),     # 16 slots, 10 KV heads
    "valu_gqa_G1_H2": (2, 32, 2, 128, 2, 128),
    "valu_gqa_G2_H2": (2, 32, 2, 128, 4, 128),
    "valu_gqa_G4_H2": (2, 16, 2, 128, 8, 128),
    "generic_G3_D64_T8": (2, 8, 2, 64, 6, 64),
    "generic_D256": (2, 64, 1, 256, 4, 256),
    "generic_mla_v448": (1, 32, 1, 576, 8, 448),
    "mla_32_heads_T64": (1, 64, 1, 576, 32, 512),
    "mla_64_heads_T256": (1, 256, 1, 576, 64, 512),
}


@pytest.mark.parametrize("name", list(GEOMETRIES))
def test_decode_geometries(name):
    """Ragged lengths (one token, a partial first tile, page multiples and
    a partial last page) for each kernel the shape routes to."""
    require_gpu()
    nt, T, H, D, Hq, v_dim = GEOMETRIES[name]
    lens = [1, 17, 2 * T, 3 * T + 5, 300]
    wl = W.geometry_case(40 + len(name), nt=nt, T=T, H=H, D=D, Hq=Hq, v_dim=v_dim, lens=lens)
    gs = wl.gs_calibrated
    packed = oracle_pool(wl, gs)
    out, lse = gpu_decode(wl, dev(packed), gs)
    check(wl, gs, packed, out, lse, what=name)


# (nt, T, H, D, Hq, v_dim): the largest page the MFMA and MLA kernels take
# (4096 tokens: 256 sixteen-token tiles, 128 MLA tiles), and the generic
# kernel at the same page size
LARGEST_PAGE = {
    "mfma_gqa_T4096_H4": (2, 4096, 4, 128, 16, 128),
    "mfma_gqa_D64_T4096_H8": (2, 4096, 8, 64, 64, 64),
    "mla_T4096": (1, 4096, 1, 576, 128, 512),
    "generic_D256_T4096": (2, 4096, 1, 256, 4, 256),
}


@pytest.mark.parametrize("name", list(LARGEST_PAGE))
def test_decode_largest_page(name):
    """One token, a partial first tile, exactly one page, one page and a few
    tokens, and a partial page, at 4096 tokens a page."""
    require_gpu()
    nt, T, H, D, Hq, v_dim = LARGEST_PAGE[name]
    lens = [1, 17, T, T + 5, 300]
    wl = W.geometry_case(60 + len(name), nt=nt, T=T, H=H, D=D, Hq=Hq, v_dim=v_dim, lens=lens)
    gs = wl.gs_calibrated
    packed = oracle_pool(wl, gs)
    out, lse = gpu_decode(wl, dev(packed), gs)
    check(wl, gs, packed, out, lse, what=name)


# (nt, T, H, D, Hq, v_dim) for the balanced kernels
MANY = {
    "mfma_gqa_D128": (2, 64, 8, 128, 32, 128),
    "mfma_gqa_D64": (2, 16, 8, 64, 32, 64),
    "mla_128_heads": (1, 64, 1, 576, 128, 512),
}


@pytest.mark.parametrize("name", list(MANY))
def test_decode_more_sequences_than_workgroups(name):
    """300 short sequences (about a tenth of them empty) over at most 256
    workgroups: a workgroup then walks several whole sequences one after
    another, the page-range scan covers the batch in 64-lane chunks, and
    empty sequences sit between the others."""
    require_gpu()
    nt, T, H, D, Hq, v_dim = MANY[name]
    rng = np.random.default_rng(77)
    lens = rng.integers(1, 3 * T, 300)
    lens[rng.random(300) < 0.1] = 0
    wl = W.geometry_case(90 + len(name), nt=nt, T=T, H=H, D=D, Hq=Hq, v_dim=v_dim, lens=lens)
    gs = wl.gs_calibrated
    packed = oracle_pool(wl, gs)
    out, lse = gpu_decode(wl, dev(packed), gs)
    check(wl, gs, packed, out, lse, what=name)
    empty = np.asarray(lens) == 0
    assert np.all(out[empty] == 0) and np.all(lse[empty] == -np.inf)


def inner_boundaries(lens, T, nwg):
    """Sequence starts that fall strictly inside a workgroup's range of the
    plain balanced split (pages [floor(w P / nwg), floor((w+1) P / nwg)))."""
    npg = [(int(L) + T - 1) // T for L in lens]
    P = sum(npg)
    starts = {(w * P) // nwg for w in range(nwg + 1)}
    out, s = [], 0
    for n in npg:
        if n > 0 and s > 0 and s not in starts:
            out.append(s)
        s += n
    return out


# (nt, T, H, D, Hq, v_dim), one per balanced kernel
PADDED = {
    "valu_gqa": (2, 16, 2, 128, 4, 128),
    "mfma_gqa": (2, 16, 8, 128, 32, 128),
    "mla": (1, 64, 1, 576, 128, 512),
}


@pytest.mark.parametrize("name", list(PADDED))
def test_decode_sequence_boundaries_inside_ranges(name):
    """Ragged sequences with more pages than workgroups: sequence starts
    fall inside workgroup ranges, where the split inserts pad pages (the
    workgroups around such a start take fewer real pages), with empty and
    one-page sequences between the others."""
    require_gpu()
    nt, T, H, D, Hq, v_dim = PADDED[name]
    unit = 16 if T == 16 else 64
    lens = np.array([700, 1900, 33, 0, 1250, 2600, 411, 1, 977], dtype=np.int64) * unit // 16
    hint = int(lens.max())
    nwg = min(torch.cuda.get_device_properties(0).multi_processor_count,
              len(lens) * ((hint + T - 1) // T))
    assert inner_boundaries(lens, T, nwg), "no sequence start inside a range"
    wl = W.geometry_case(110 + len(name), nt=nt, T=T, H=H, D=D, Hq=Hq, v_dim=v_dim, lens=lens)
    gs = wl.gs_calibrated
    packed = oracle_pool(wl, gs)
    out, lse = gpu_decode(wl, dev(packed), gs)
    check(wl, gs, packed, out, lse, what=name)


NO_LSE = {
    "valu_tiny": lambda: W.tiny(seed=21),
    "mfma_gqa": lambda: W.llama3_8b(seed=22, batch=3, context=300),
    "mla": lambda: W.mla(seed=23, batch=2, context=150),
    "generic_D256": lambda: W.geometry_case(24, nt=2, T=64, H=1, D=256, Hq=4, v_dim=256,
                                            lens=[0, 1, 70, 200]),
}


@pytest.mark.parametrize("name", list(NO_LSE))
def test_decode_without_lse(name):
    """lse is optional: without it the outputs are bit-identical to a call
    that writes it (empty sequences included)."""
    require_gpu()
    wl = NO_LSE[name]()
    gs = wl.gs_calibrated
    packed = oracle_pool(wl, gs)
    out_ref, _ = gpu_decode(wl, dev(packed), gs)
    B, Hq = wl.batch, wl.num_q_heads
    hint = int(wl.seq_lens.max())
    ws_bytes = K.kvfp4_decode_workspace_bytes(wl.geometry, B, Hq, wl.v_dim, hint)
    ws = torch.empty(max(ws_bytes, 4), dtype=torch.uint8, device="cuda")
    out = torch.full((B, Hq, wl.v_dim), 0x7FC0, dtype=torch.int16, device="cuda")
    K.kvfp4_paged_decode_attention(wl.geometry, dev(packed), gs, dev(wl.q.view(np.int16)),
                                   dev(wl.block_table), dev(wl.seq_lens), hint,
                                   wl.softmax_scale, out, None, ws, v_dim=wl.v_dim)
    assert np.array_equal(host(out).view(np.uint16), out_ref), name


BAD_PAGES = {  # (nt, T, H, D, Hq, v_dim), one per decode kernel
    "valu_gqa": (2, 16, 2, 128, 4, 128),
    "mfma_gqa": (2, 64, 8, 128, 32, 128),
    "mla": (1, 64, 1, 576, 128, 512),
    "generic_D256": (2, 64, 1, 256, 4, 256),
}


@pytest.mark.parametrize("name", list(BAD_PAGES))
def test_decode_out_of_range_pages_contribute_nothing(name):
    """Page-table entries outside [0, pool pages) make their page's tokens
    take no part: the result equals the oracle on the same sequences with
    those pages left out (a middle page, a first page, a one-token last
    page, and a sequence's only page, which leaves it empty)."""
    require_gpu()
    import dataclasses
    nt, T, H, D, Hq, v_dim = BAD_PAGES[name]
    lens = [3 * T + 5, 2 * T, 4 * T + 1, T, 2 * T + 3]
    wl = W.geometry_case(110 + len(name), nt=nt, T=T, H=H, D=D, Hq=Hq, v_dim=v_dim, lens=lens)
    gs = wl.gs_calibrated
    packed = oracle_pool(wl, gs)
    bt_bad = wl.block_table.copy()
    bt_ref = wl.block_table.copy()
    lens_ref = wl.seq_lens.copy()
    # (sequence, page, bad id); the reference drops that page from the row
    for b, pg, bad in [(0, 1, -1), (1, 0, wl.num_slots), (2, 4, 1 << 30), (3, 0, -5)]:
        n_pages = -(-int(wl.seq_lens[b]) // T)
        bt_bad[b, pg] = bad
        row = [int(s) for j, s in enumerate(wl.block_table[b, :n_pages]) if j != pg]
        bt_ref[b, :len(row)] = row
        rows_on_page = min(T, int(wl.seq_lens[b]) - pg * T)
        lens_ref[b] -= rows_on_page
    assert list(lens_ref[:4]) == [2 * T + 5, T, 4 * T, 0]
    wl_bad = dataclasses.replace(wl, block_table=bt_bad)
    wl_ref = dataclasses.replace(wl, block_table=bt_ref, seq_lens=lens_ref)
    out, lse = gpu_decode(wl_bad, dev(packed), gs)
    check(wl_ref, gs, packed, out, lse, what=f"{name} out-of-range pages")
    assert np.all(out[3] == 0) and np.all(lse[3] == -np.inf)


@pytest.mark.parametrize("name", list(BAD_PAGES))
def test_decode_out_of_range_lengths_are_clamped(name):
    """A negative length reads as 0 (out = 0, lse = -inf); a length past
    max_pages_per_seq * T reads as that bound.  The pool is encoded without
    poisoned rows, so the clamped sequence's last page is data throughout."""
    require_gpu()
    import dataclasses
    nt, T, H, D, Hq, v_dim = BAD_PAGES[name]
    lens = [3 * T + 5, 2 * T, 4 * T + 1, 40]
    wl = W.geometry_case(130 + len(name), nt=nt, T=T, H=H, D=D, Hq=Hq, v_dim=v_dim, lens=lens)
    gs = wl.gs_calibrated
    packed = oracle_packed_pages(wl.hot_pool, wl.geometry, gs, np.arange(wl.num_slots))
    cap = wl.block_table.shape[1] * T
    assert cap == 5 * T  # sequence 2 uses every entry of its page-table row
    lens_bad = np.array([-3, 2 * T, cap + 100, 40], np.int32)
    lens_ref = np.array([0, 2 * T, cap, 40], np.int32)
    out, lse = gpu_decode(wl, dev(packed), gs, hint=cap + 100, seq_lens=lens_bad)
    check(dataclasses.replace(wl, seq_lens=lens_ref), gs, packed, out, lse,
          what=f"{name} clamped lengths")
    assert np.all(out[0] == 0) and np.all(lse[0] == -np.inf)


def test_decode_unaligned_output():
    """An output buffer that is only 2-byte aligned takes the merge's
    one-column-per-thread path; results are the same."""
    require_gpu()
    wl = W.llama3_8b(seed=19, batch=3, context=200)
    gs = wl.gs_calibrated
    packed = oracle_pool(wl, gs)
    B, Hq = wl.batch, wl.num_q_heads
    hint = int(wl.seq_lens.max())
    ws_bytes = K.kvfp4_decode_workspace_bytes(wl.geometry, B, Hq, wl.v_dim, hint)
    ws = torch.empty(max(ws_bytes, 4), dtype=torch.uint8, device="cuda")
    flat = torch.empty(B * Hq * wl.v_dim + 1, dtype=torch.int16, device="cuda")
    out = flat[1:].view(B, Hq, wl.v_dim)
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    K.kvfp4_paged_decode_attention(wl.geometry, dev(packed), gs, dev(wl.q.view(np.int16)),
                                   dev(wl.block_table), dev(wl.seq_lens), hint,
                                   wl.softmax_scale, out, lse, ws, v_dim=wl.v_dim)
    check(wl, gs, packed, host(out).view(np.uint16), host(lse), what="unaligned out")


FULL = {
    "llama3_8b": lambda: W.llama3_8b(),
    "qwen3_8b_long": lambda: W.qwen3_8b_long(),
    "mla": lambda: W.mla(),
}


@pytest.mark.parametrize("name", list(FULL))
def test_decode_full_size_all_outputs(name):
    """Full-size workloads in the bench's launch configuration, every output
    of every sequence and query head: the whole pool is encoded by the
    oracle (process pool), bytes no decode may read are poisoned, the GPU
    decodes the batch in one call, and the oracle computes every
    (sequence, head) result in the pool."""
    require_gpu()
    wl = FULL[name]()
    gs = wl.gs_calibrated
    g = O.Geometry(*wl.geometry)
    with P.make_pool() as pool:
        packed = np.zeros((wl.num_slots, O.packed_page_bytes(g)), np.uint8)
        packed[wl.used_slots] = P.encode_pages(pool, wl.hot_pool, wl.geometry, gs,
                                               wl.used_slots)
        poison_unread(packed, wl, np.random.default_rng(3))
        out, lse = gpu_decode(wl, dev(packed), gs)
        ref, ref_lse = P.decode_attention_all(pool, packed, wl, gs)
    assert_attention_close(out, ref, f"{name} full size")
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(lse)), f"{name}: lse finiteness"
    assert np.all(np.abs(lse[fin] - ref_lse[fin]) <= 1e-3 + 1e-3 * np.abs(ref_lse[fin])), name


def test_decode_workspace_reused_across_calls():
    """Two different batches decoded back to back through the same
    workspace, each sequence split over many workgroups: the second call's
    outputs match the oracle (no partial or arrival count of the first call
    leaks into it), and a third call on unchanged inputs reproduces them bit
    for bit."""
    require_gpu()
    wa = W.llama3_8b(seed=31, batch=4, context=2048)
    wb = W.llama3_8b(seed=32, batch=4, context=2048)
    B, Hq = wb.batch, wb.num_q_heads
    hint = int(max(wa.seq_lens.max(), wb.seq_lens.max()))
    ws_bytes = K.kvfp4_decode_workspace_bytes(wb.geometry, B, Hq, wb.v_dim, hint)
    ws = torch.empty(max(ws_bytes, 4), dtype=torch.uint8, device="cuda")
    outs = []
    for wl in (wa, wb, wb):
        gs = wl.gs_calibrated
        packed = oracle_pool(wl, gs)
        out = torch.empty((B, Hq, wl.v_dim), dtype=torch.int16, device="cuda")
        lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        K.kvfp4_paged_decode_attention(wl.geometry, dev(packed), gs, dev(wl.q.view(np.int16)),
                                       dev(wl.block_table), dev(wl.seq_lens), hint,
                                       wl.softmax_scale, out, lse, ws, v_dim=wl.v_dim)
        outs.append((host(out).view(np.uint16), host(lse), packed))
    out_b, lse_b, packed_b = outs[1]
    check(wb, wb.gs_calibrated, packed_b, out_b, lse_b, what="second call, reused workspace")
    assert np.array_equal(outs[2][0], out_b) and np.array_equal(outs[2][1], lse_b)


@pytest.mark.parametrize("name", list(BAD_PAGES))
def test_decode_late_dominant_score(name):
    """A token near the end of a long sequence whose key equals a query row
    scores far above every token before it (for MLA about 24 nats, past the
    fp16 headroom of the first tiles' maximum): the kernels' running-maximum
    updates (rescales, or a second pass over the segment) must give the
    oracle's result; the head's output is then close to that token's value."""
    require_gpu()
    nt, T, H, D, Hq, v_dim = BAD_PAGES[name]
    lens = [6 * T + 7, 3 * T, 2 * T + 1]
    wl = W.geometry_case(150 + len(name), nt=nt, T=T, H=H, D=D, Hq=Hq, v_dim=v_dim, lens=lens)
    G = Hq // H
    for b, h in [(0, 0), (2, Hq - 1)]:
        # three quarters into the second-to-last page: a later tile of its
        # page than the page's first (each workgroup may own a single page)
        j = (-(-int(wl.seq_lens[b]) // T) - 2) * T + (3 * T) // 4
        slot, row = int(wl.block_table[b, j // T]), j % T
        wl.hot_pool[slot, 0, row, h // G] = wl.q[b, h]  # key row = query row
    gs = wl.gs_calibrated
    packed = oracle_pool(wl, gs)
    out, lse = gpu_decode(wl, dev(packed), gs)
    check(wl, gs, packed, out, lse, what=f"{name} late dominant score")


# (nt, T, H, D, Hq, v_dim): every balanced kernel
FULL_SCALE = {
    "valu_gqa": (2, 16, 2, 128, 4, 128),
    "mfma_gqa": (2, 64, 8, 128, 32, 128),
    "mfma_gqa_D64": (2, 16, 8, 64, 32, 64),
    "mla": (1, 64, 1, 576, 128, 512),
}


@pytest.mark.parametrize("gs_last", [1.0 / 2688.0, 2.0 ** -8])
@pytest.mark.parametrize("name", list(FULL_SCALE))
def test_decode_full_scale_values(name, gs_last):
    """Every value of the last tensor (V; for MLA the latent, so the keys
    too) encodes to the format's largest finite magnitude, E2M1 6 times
    E4M3 448 = 2688, with random signs: the partials the kernels hand to
    the merge (o / l before the tensor scale: fp16 for MLA) span the
    format's whole range.  The tensor scale, applied after the merge, keeps
    the outputs O(1) (values of 1 and 10.5), where the absolute part of the
    tolerance is meaningful: at |v| = 2688 any 16-bit rounding of the
    probabilities would exceed it for outputs that cancel to near zero."""
    require_gpu()
    nt, T, H, D, Hq, v_dim = FULL_SCALE[name]
    lens = [7 * T + 3, 2 * T, 5]
    wl = W.geometry_case(180 + len(name), nt=nt, T=T, H=H, D=D, Hq=Hq, v_dim=v_dim, lens=lens)
    rng = np.random.default_rng(181)
    neg = rng.random(wl.hot_pool[:, nt - 1].shape) < 0.5
    top = np.float32(round(2688.0 * gs_last, 6))  # 1 and 10.5: exact in bf16
    wl.hot_pool[:, nt - 1] = W.f32_to_bf16_bits(np.where(neg, -top, top).astype(np.float32))
    gs = np.ones(nt, np.float32)
    gs[-1] = gs_last
    packed = oracle_pool(wl, gs)
    g = O.Geometry(*wl.geometry)
    full = wl.block_table[0, :int(wl.seq_lens[0]) // T]  # sequence 0's full pages
    for slot in full:
        _, sc = O.split_packed_page(packed[slot], g)
        assert np.all(sc[-1] == 0x7E), "every block of the last tensor at scale 448"
    out, lse = gpu_decode(wl, dev(packed), gs)
    check(wl, gs, packed, out, lse, what=f"{name} full-scale values, gs {gs_last}")
