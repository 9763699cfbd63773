"""GPU parity of the page codec against the oracle: packed bytes, scale
bytes and dequantized bf16 bits must be identical."""

import os

import numpy as np
import pytest

import nvfp4_paged_decode_amd as K
from nvfp4_paged_decode_amd import workloads as W
from oracle import nvfp4 as O
from tests import oracle_pool as P
from tests.gpu_common import dev, host, require_gpu, torch, oracle_packed_pages

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def gpu_quantize(hot: np.ndarray, geometry, gs, num_pages=None, src=None, dst=None,
                 packed_slots=None):
    g = O.Geometry(*geometry)
    n = hot.shape[0] if num_pages is None else num_pages
    slots = hot.shape[0] if packed_slots is None else packed_slots
    assert all(a is None or len(a) >= n for a in (src, dst)), "slot arrays shorter than num_pages"
    hot_d = dev(hot.view(np.int16))
    packed_d = torch.zeros((slots, O.packed_page_bytes(g)), dtype=torch.uint8, device="cuda")
    K.kvfp4_quantize_pages(geometry, hot_d, packed_d, n, gs,
                           None if src is None else dev(src.astype(np.int32)),
                           None if dst is None else dev(dst.astype(np.int32)))
    return host(packed_d)


def gpu_dequantize(packed: np.ndarray, geometry, gs, num_pages=None, src=None, dst=None,
                   hot_slots=None, fill=0):
    g = O.Geometry(*geometry)
    n = packed.shape[0] if num_pages is None else num_pages
    slots = packed.shape[0] if hot_slots is None else hot_slots
    assert all(a is None or len(a) >= n for a in (src, dst)), "slot arrays shorter than num_pages"
    hot_d = torch.full((slots, *g.row_shape), fill, dtype=torch.int16, device="cuda")
    K.kvfp4_dequantize_pages(geometry, dev(packed), hot_d, n, gs,
                             None if src is None else dev(src.astype(np.int32)),
                             None if dst is None else dev(dst.astype(np.int32)))
    return host(hot_d).view(np.uint16)


def test_golden_page():
    require_gpu()
    z = np.load(os.path.join(GOLDEN, "tiny_page.npz"))
    geom = tuple(int(v) for v in z["geometry"])
    packed = gpu_quantize(z["hot"], geom, z["gs"])
    assert np.array_equal(packed[0], z["packed"])
    back = gpu_dequantize(z["packed"][None], geom, z["gs"])
    assert np.array_equal(back, z["dequant"])


def _block_zoo(rng, gs, n_pages, geometry):
    """Pages of adversarial blocks: quotients on E4M3 and E2M1 rounding
    midpoints (for the given gs), saturation, zeros, signed zeros, subnormal
    inputs, and random blocks over 12 decades."""
    g = O.Geometry(*geometry)
    nblk = n_pages * g.elems // 16
    e4 = O.E4M3_FINITE
    blocks = []
    for c in range(126):
        mid = (e4[c] + e4[c + 1]) / 2.0
        blk = np.zeros(16)
        blk[rng.integers(16)] = mid * 6.0 * gs
        blk[rng.integers(16)] = -mid * 6.0 * gs
        blocks.append(blk)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0])
    for s in O.E4M3_FINITE[1:]:
        vals = rng.choice(mids, 16) * s * gs * rng.choice([-1, 1], 16)
        vals[0] = 6.0 * s * gs
        blocks.append(vals)
    blocks = np.array(blocks, dtype=np.float64)
    special = [np.zeros(16), np.full(16, 3e38), np.full(16, 1e-40), np.full(16, -1e-39)]
    rest = nblk - len(blocks) - len(special)
    mag = 10.0 ** rng.uniform(-8, 4, size=(rest, 1))
    rand = rng.standard_normal((rest, 16)) * mag
    allb = np.concatenate([blocks, np.array(special), rand])
    bits = W.f32_to_bf16_bits(allb.astype(np.float32))
    bits[len(blocks) + 1, :8] = 0x8000  # negative zeros
    bits[rng.integers(0, bits.shape[0], 50), rng.integers(0, 16, 50)] = 0x8000
    perm = rng.permutation(bits.shape[0])
    return bits[perm].reshape(n_pages, *g.row_shape)


# (1, 3, 1, 16) and (2, 5, 1, 48): 3 and 30 blocks a page, so the last
# group of four scale bytes is cut by the page end, and pages are 27 and
# 270 bytes (not dword-aligned).  The decoder splits larger pages into runs
# of about 4096 half-blocks: 4 a page for (2, 64, 8, 128), 2 of 2304 for
# (1, 64, 1, 576), 3 of 2880 for (2, 16, 9, 240); smaller pages are grouped.
@pytest.mark.parametrize("geometry", [(2, 16, 1, 128), (2, 64, 8, 128), (1, 64, 1, 576),
                                      (2, 8, 3, 48), (1, 3, 1, 16), (2, 5, 1, 48),
                                      (2, 16, 9, 240)])
@pytest.mark.parametrize("gs_val", [1.0, 2.0 ** -3, float(np.float32(0.0123456)),
                                    float(np.float32(3.1e-5)), 2.0 ** -110,
                                    float(np.float32(1e30))])
def test_quantize_dequantize_bit_exact(geometry, gs_val):
    require_gpu()
    rng = np.random.default_rng(hash((geometry, gs_val)) % 2 ** 32)
    g = O.Geometry(*geometry)
    n_pages = max(3, -(-3000 * 16 // g.elems))
    hot = _block_zoo(rng, gs_val, n_pages, geometry)
    gs = [gs_val, float(np.float32(gs_val * 1.37))][:g.num_kv_tensors]
    ref = np.zeros((n_pages, O.packed_page_bytes(g)), np.uint8)
    O.quantize_pages(hot, g, n_pages, gs, ref)
    got = gpu_quantize(hot, geometry, gs)
    mism = np.nonzero(got != ref)
    assert got.shape == ref.shape
    assert mism[0].size == 0, f"{mism[0].size} packed bytes differ, first at {mism[0][0]},{mism[1][0]}"
    back_ref = np.zeros_like(hot)
    O.dequantize_pages(ref, g, n_pages, gs, back_ref)
    back = gpu_dequantize(ref, geometry, gs)
    assert np.array_equal(back, back_ref)


def test_slots_and_out_of_range_pages_are_skipped():
    require_gpu()
    geometry = (2, 16, 2, 64)
    g = O.Geometry(*geometry)
    rng = np.random.default_rng(4)
    hot = W.f32_to_bf16_bits(rng.standard_normal((6, *g.row_shape)).astype(np.float32))
    src = np.array([5, 2, 0, 1, 9], np.int32)   # 9 is out of range: skipped
    dst = np.array([3, 0, 4, -1, 1], np.int32)  # -1 is out of range: skipped
    gs = [1.0, 0.5]
    got = gpu_quantize(hot, geometry, gs, num_pages=5, src=src, dst=dst, packed_slots=5)
    ref = np.zeros((5, O.packed_page_bytes(g)), np.uint8)
    O.quantize_pages(hot, g, 3, gs, ref, src[:3], dst[:3])
    assert np.array_equal(got, ref)  # slots 2 (untouched) and 1 (skipped page) stay zero
    back = gpu_dequantize(ref, geometry, gs, num_pages=3, src=dst[:3], dst=src[:3], hot_slots=6,
                          fill=0x1234)
    ref_back = np.full((6, *g.row_shape), 0x1234, np.uint16)
    O.dequantize_pages(ref, g, 3, gs, ref_back, dst[:3], src[:3])
    assert np.array_equal(back, ref_back)


def test_zero_pages_launches_nothing():
    require_gpu()
    geometry = (2, 16, 1, 128)
    hot = np.zeros((1, *O.Geometry(*geometry).row_shape), np.uint16)
    got = gpu_quantize(hot, geometry, [1.0, 1.0], num_pages=0)
    assert np.all(got == 0)


@pytest.mark.parametrize("gs_kind", ["unit", "calibrated"])
def test_cold_pages_full_size(gs_kind):
    """The 4096-page cold-page workload in the launch configuration the bench
    times (source and destination slots permuted): every packed page equals
    the oracle's encoding, and every decoded page the oracle's decoding of
    it, byte for byte (oracle in a process pool)."""
    require_gpu()
    wl = W.cold_pages()
    gs = wl.gs_unit if gs_kind == "unit" else wl.gs_calibrated
    packed = gpu_quantize(wl.hot_pool, wl.geometry, gs, src=wl.src_slots, dst=wl.dst_slots)
    with P.make_pool() as pool:
        ref = P.encode_pages(pool, wl.hot_pool, wl.geometry, gs, wl.src_slots)
        bad = np.nonzero(np.any(packed[wl.dst_slots] != ref, axis=1))[0]
        assert bad.size == 0, f"{bad.size} of {wl.num_pages} packed pages differ (first {bad[:5]})"
        pool_in = np.zeros_like(packed)
        pool_in[wl.dst_slots] = ref  # the decoder's input is the oracle's encoding
        back = gpu_dequantize(pool_in, wl.geometry, gs, src=wl.dst_slots, dst=wl.src_slots)
        ref_back = P.decode_pages(pool, ref, wl.geometry, gs)
    bad = np.nonzero(np.any((back[wl.src_slots] != ref_back).reshape(wl.num_pages, -1), axis=1))[0]
    assert bad.size == 0, f"{bad.size} of {wl.num_pages} decoded pages differ (first {bad[:5]})"


def gpu_append(rows: np.ndarray, geometry, gs, slots, page_rows, pool: np.ndarray) -> np.ndarray:
    """Append through the C ABI into a device copy of ``pool``; returns the pool."""
    pool_d = dev(pool)
    K.kvfp4_append_quantize(geometry, dev(rows.view(np.int16)), dev(np.asarray(slots, np.int32)),
                            dev(np.asarray(page_rows, np.int32)), pool_d, gs)
    return host(pool_d)


@pytest.mark.parametrize("geometry,num_tokens", [
    ((2, 64, 8, 128), 64),    # one decode step of a 64-sequence batch
    ((2, 8, 3, 48), 37),      # 36 half-blocks a token: ragged last wave
    ((1, 64, 1, 576), 129),   # MLA latent rows
    ((2, 16, 1, 16), 5),      # one block a row
    ((2, 8, 3, 48), 2001),    # past the one-half-block-a-lane size: 4 a lane, ragged
])
def test_append_bit_exact_and_touches_only_its_rows(geometry, num_tokens):
    """Appended rows match the oracle byte for byte, over a pool filled with
    noise: every byte outside the appended rows must keep its noise."""
    require_gpu()
    g = O.Geometry(*geometry)
    rng = np.random.default_rng(num_tokens)
    n_slots = 2 * num_tokens // g.page_size + 3
    pool = rng.integers(0, 256, (n_slots, O.packed_page_bytes(g)), dtype=np.uint8)
    cells = rng.choice(n_slots * g.page_size, num_tokens, replace=False)
    slots, page_rows = (cells // g.page_size).astype(np.int32), (cells % g.page_size).astype(np.int32)
    per_token = g.num_kv_tensors * g.num_kv_heads * g.head_dim
    zoo_pages = max(-(-num_tokens * per_token // g.elems), -(-300 * 16 // g.elems))
    zoo = _block_zoo(rng, 0.37, zoo_pages, geometry).reshape(-1)[:num_tokens * per_token]
    rows = np.ascontiguousarray(zoo.reshape(num_tokens, g.num_kv_tensors, g.num_kv_heads,
                                            g.head_dim))
    gs = [float(np.float32(0.37)), float(np.float32(0.011))][:g.num_kv_tensors]
    ref = pool.copy()
    O.append_quantize(rows, g, gs, ref, slots, page_rows)
    got = gpu_append(rows, geometry, gs, slots, page_rows, pool)
    mism = np.nonzero(got != ref)
    assert mism[0].size == 0, f"{mism[0].size} bytes differ, first at {mism[0][0]},{mism[1][0]}"


def test_append_skips_bad_slots_and_rows():
    require_gpu()
    geometry = (2, 16, 2, 64)
    g = O.Geometry(*geometry)
    rng = np.random.default_rng(21)
    rows = W.f32_to_bf16_bits(rng.standard_normal((6, 2, 2, 64)).astype(np.float32))
    slots = np.array([0, -1, 3, 1, 2, 1], np.int32)    # -1 and 3 are outside a 3-slot pool
    page_rows = np.array([5, 0, 0, 16, -2, 15], np.int32)  # 16 and -2 are outside the page
    pool = np.full((3, O.packed_page_bytes(g)), 0x5A, np.uint8)
    ref = pool.copy()
    O.append_quantize(rows, g, [1.0, 0.25], ref, slots, page_rows)
    got = gpu_append(rows, geometry, [1.0, 0.25], slots, page_rows, pool)
    assert np.array_equal(got, ref)
    changed = np.nonzero(np.any(ref != 0x5A, axis=1))[0]
    assert changed.tolist() == [0, 1]  # only tokens 0 and 5 landed


def test_append_prefill_full_size():
    """A 16384-token prefill of Llama-3-8B KV rows (8 KV heads x 128) into
    256 scattered 64-token pages: more half-blocks than the grid covers in
    one pass.  Sampled tokens are checked against the oracle; the whole pool
    must equal quantizing the assembled bf16 pages page by page."""
    require_gpu()
    geometry = (2, 64, 8, 128)
    g = O.Geometry(*geometry)
    n_pages, n_tok = 256, 16384
    rng = np.random.default_rng(5)
    hot = W.f32_to_bf16_bits((rng.standard_normal((n_pages, *g.row_shape))
                              * rng.uniform(0.1, 8.0, (n_pages, 2, 1, 8, 1))).astype(np.float32))
    dst = rng.permutation(n_pages + 7)[:n_pages].astype(np.int32)
    tok = np.arange(n_tok)
    slots, page_rows = dst[tok // 64], (tok % 64).astype(np.int32)
    rows = np.ascontiguousarray(hot.transpose(0, 2, 1, 3, 4).reshape(n_tok, 2, 8, 128))
    gs = [float(np.float32(0.05)), float(np.float32(0.02))]
    pool = np.zeros((n_pages + 7, O.packed_page_bytes(g)), np.uint8)
    got = gpu_append(rows, geometry, gs, slots, page_rows, pool)
    whole = gpu_quantize(hot, geometry, gs, dst=dst, packed_slots=n_pages + 7)
    assert np.array_equal(got, whole)
    sample = np.concatenate([[0, n_tok - 1], rng.choice(n_tok, 40, replace=False)])
    ref = np.zeros_like(pool)
    O.append_quantize(rows[sample], g, gs, ref, slots[sample], page_rows[sample])
    data_idx, scale_idx = O.split_packed_page(np.arange(O.packed_page_bytes(g)), g)
    for i in sample:
        s, r = slots[i], page_rows[i]
        idx = np.concatenate([data_idx[:, r].reshape(-1), scale_idx[:, r].reshape(-1)])
        assert np.array_equal(got[s, idx], ref[s, idx]), f"token {i}"


@pytest.mark.parametrize("geometry,num_tokens", [((2, 64, 8, 128), 96), ((2, 8, 3, 48), 37),
                                                 ((1, 64, 1, 576), 40), ((2, 64, 8, 128), 300)])
@pytest.mark.parametrize("gs_pair", [(1.0, 1.0), (float(np.float32(0.0123)), 2.0 ** -7),
                                     (float(np.float32(3.3)), float(np.float32(0.71)))])
def test_append_fp8_rows_bit_exact(geometry, num_tokens, gs_pair):
    """FP8 (E4M3FN) input rows: every finite code appears, in blocks of mixed
    and of uniform magnitude range, over a noise-filled pool."""
    require_gpu()
    g = O.Geometry(*geometry)
    rng = np.random.default_rng(num_tokens * 7 + int(gs_pair[0] * 100))
    per_token = g.num_kv_tensors * g.num_kv_heads * g.head_dim
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    codes = rng.choice(finite, num_tokens * per_token)
    codes[:finite.size] = finite
    blocks = codes.reshape(-1, 16)
    nb = blocks.shape[0]
    # blocks drawn from one binade band each: small (subnormal) to large codes
    for i in rng.choice(nb, nb // 2, replace=False):
        lo = rng.integers(0, 0x70)
        blocks[i] = rng.integers(lo, lo + 16, 16) | (rng.integers(0, 2, 16) << 7)
    blocks[blocks == 0x7F] = 0x7E
    blocks[blocks == 0xFF] = 0xFE
    rows = np.ascontiguousarray(blocks.reshape(num_tokens, g.num_kv_tensors, g.num_kv_heads,
                                               g.head_dim).astype(np.uint8))
    n_slots = num_tokens // g.page_size + 3
    pool = rng.integers(0, 256, (n_slots, O.packed_page_bytes(g)), dtype=np.uint8)
    cells = rng.choice(n_slots * g.page_size, num_tokens, replace=False)
    slots, page_rows = (cells // g.page_size).astype(np.int32), (cells % g.page_size).astype(np.int32)
    gs = list(gs_pair)[:g.num_kv_tensors]
    ref = pool.copy()
    O.append_quantize(rows, g, gs, ref, slots, page_rows)
    pool_d = dev(pool)
    K.kvfp4_append_quantize(geometry, dev(rows), dev(slots), dev(page_rows), pool_d, gs)
    got = host(pool_d)
    mism = np.nonzero(got != ref)
    assert mism[0].size == 0, f"{mism[0].size} bytes differ, first at {mism[0][0]},{mism[1][0]}"


def _valid_pool(rng, g, n_slots, gs):
    """Packed slots holding encoder output of random data, with some scale
    bytes negated (the decoder's sign flip); no NaN scale codes."""
    hot = W.f32_to_bf16_bits((rng.standard_normal((n_slots, *g.row_shape))
                              * 10.0 ** rng.uniform(-3, 3, (n_slots, g.num_kv_tensors, 1, 1, 1)))
                             .astype(np.float32))
    pool = np.zeros((n_slots, O.packed_page_bytes(g)), np.uint8)
    O.quantize_pages(hot, g, n_slots, gs, pool)
    nd = g.elems // 2
    sc = pool[:, nd:]
    neg = rng.random(sc.shape) < 0.05
    sc[neg & (sc != 0x7F)] |= 0x80
    return pool


@pytest.mark.parametrize("geometry,num_tokens", [((2, 64, 8, 128), 100), ((2, 8, 3, 48), 37),
                                                 ((1, 64, 1, 576), 70), ((2, 8, 3, 48), 2001)])
@pytest.mark.parametrize("out_dtype", ["bf16", "fp8"])
def test_gather_bit_exact(geometry, num_tokens, out_dtype):
    """Gathered rows match the oracle bit for bit, bf16 and FP8, including
    tokens with a bad slot (negative or past the pool) or row (zero rows)
    and repeated tokens."""
    require_gpu()
    g = O.Geometry(*geometry)
    rng = np.random.default_rng(num_tokens + (7 if out_dtype == "fp8" else 0))
    gs = [float(np.float32(0.37)), float(np.float32(0.011))][:g.num_kv_tensors]
    n_slots = 2 * num_tokens // g.page_size + 3
    pool = _valid_pool(rng, g, n_slots, gs)
    slots = rng.integers(0, n_slots, num_tokens).astype(np.int32)
    page_rows = rng.integers(0, g.page_size, num_tokens).astype(np.int32)
    slots[::17] = -1
    slots[3::23] = n_slots  # one past the pool
    page_rows[5::19] = g.page_size
    ref = O.gather_dequantize(pool, g, gs, slots, page_rows, out_dtype)
    dt = torch.int16 if out_dtype == "bf16" else torch.uint8
    out = torch.full(ref.shape, 0x55, dtype=dt, device="cuda")
    K.kvfp4_gather_dequantize(geometry, dev(pool), dev(slots), dev(page_rows), out, gs)
    got = host(out)
    got = got.view(np.uint16) if out_dtype == "bf16" else got
    mism = np.nonzero(got.reshape(num_tokens, -1) != ref.reshape(num_tokens, -1))
    assert mism[0].size == 0, f"{mism[0].size} values differ, first at token {mism[0][0]}"


def test_gather_prefix_full_size():
    """The extend-path gather at Llama-3-8B size: the 8192-token prefixes of
    4 sequences of 64-token pages (32768 rows) in bf16 and FP8.  The bf16
    rows must equal the page dequantizer's pages; sampled rows of both
    outputs are checked against the oracle."""
    require_gpu()
    geometry = (2, 64, 8, 128)
    g = O.Geometry(*geometry)
    rng = np.random.default_rng(8)
    n_pages, n_slots = 512, 600
    gs = [float(np.float32(0.05)), float(np.float32(0.02))]
    hot = W.f32_to_bf16_bits(rng.standard_normal((n_pages, *g.row_shape)).astype(np.float32))
    dst = rng.permutation(n_slots)[:n_pages].astype(np.int32)
    packed = gpu_quantize(hot, geometry, gs, dst=dst, packed_slots=n_slots)
    tok = np.arange(n_pages * 64)
    slots, page_rows = dst[tok // 64], (tok % 64).astype(np.int32)
    pool_d = dev(packed)
    out16 = torch.empty((tok.size, 2, 8, 128), dtype=torch.int16, device="cuda")
    out8 = torch.empty((tok.size, 2, 8, 128), dtype=torch.uint8, device="cuda")
    K.kvfp4_gather_dequantize(geometry, pool_d, dev(slots), dev(page_rows), out16, gs)
    K.kvfp4_gather_dequantize(geometry, pool_d, dev(slots), dev(page_rows), out8, gs)
    got16, got8 = host(out16).view(np.uint16), host(out8)
    pages = gpu_dequantize(packed, geometry, gs, num_pages=n_pages, src=dst,
                           dst=np.arange(n_pages), hot_slots=n_pages)
    assert np.array_equal(got16, pages.transpose(0, 2, 1, 3, 4).reshape(tok.size, 2, 8, 128))
    sample = np.concatenate([[0, tok.size - 1], rng.choice(tok.size, 40, replace=False)])
    for dt, got in (("bf16", got16), ("fp8", got8)):
        ref = O.gather_dequantize(packed, g, gs, slots[sample], page_rows[sample], dt)
        assert np.array_equal(got[sample], ref), dt


def test_offload_to_pinned_host_and_back():
    """The cold-page path with the packed pool in pinned host memory: the
    encoder writes across the host link and the decoder reads back across
    it.  The host bytes must equal the oracle's (sampled pages) and the
    device-pool encoding (every page), and the decoded pages the device
    decoder's."""
    require_gpu()
    geometry = (2, 64, 8, 128)
    g = O.Geometry(*geometry)
    rng = np.random.default_rng(9)
    n_pages = 96
    gs = [float(np.float32(0.03)), float(np.float32(0.01))]
    hot = W.f32_to_bf16_bits(rng.standard_normal((n_pages, *g.row_shape)).astype(np.float32))
    src = rng.permutation(n_pages).astype(np.int32)
    dst = rng.permutation(n_pages + 5)[:n_pages].astype(np.int32)
    hot_d = dev(hot.view(np.int16))
    pb = O.packed_page_bytes(g)
    host_pool = torch.zeros((n_pages + 5, pb), dtype=torch.uint8).pin_memory()
    dev_pool = torch.zeros((n_pages + 5, pb), dtype=torch.uint8, device="cuda")
    K.kvfp4_quantize_pages(geometry, hot_d, host_pool, n_pages, gs, dev(src), dev(dst))
    K.kvfp4_quantize_pages(geometry, hot_d, dev_pool, n_pages, gs, dev(src), dev(dst))
    torch.cuda.synchronize()
    got = host_pool.numpy().copy()
    assert np.array_equal(got, host(dev_pool))
    sample = rng.choice(n_pages, 6, replace=False)
    ref = np.zeros((n_pages + 5, pb), np.uint8)
    O.quantize_pages(hot, g, len(sample), gs, ref, src[sample], dst[sample])
    assert np.array_equal(got[dst[sample]], ref[dst[sample]])
    back_h = torch.zeros_like(hot_d)
    back_d = torch.zeros_like(hot_d)
    K.kvfp4_dequantize_pages(geometry, host_pool, back_h, n_pages, gs, dev(dst), dev(src))
    K.kvfp4_dequantize_pages(geometry, dev_pool, back_d, n_pages, gs, dev(dst), dev(src))
    assert np.array_equal(host(back_h), host(back_d))
