"""GPU parity of the page codec against the oracle: packed bytes, scale
bytes and dequantized bf16 bits must be identical."""

import os

import numpy as np
import pytest

import nvfp4_paged_decode_amd as K
from nvfp4_paged_decode_amd import workloads as W
from oracle import nvfp4 as O
from tests.gpu_common import dev, host, require_gpu, torch, oracle_packed_pages

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def gpu_quantize(hot: np.ndarray, geometry, gs, num_pages=None, src=None, dst=None,
                 packed_slots=None):
    g = O.Geometry(*geometry)
    n = hot.shape[0] if num_pages is None else num_pages
    slots = hot.shape[0] if packed_slots is None else packed_slots
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


@pytest.mark.parametrize("geometry", [(2, 16, 1, 128), (2, 64, 8, 128), (1, 64, 1, 576),
                                      (2, 8, 3, 48)])
@pytest.mark.parametrize("gs_val", [1.0, 2.0 ** -3, float(np.float32(0.0123456)),
                                    float(np.float32(3.1e-5)), 2.0 ** -110, 1e30])
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
    times: every packed page is checked against the oracle on a sample of
    pages, and the whole pool against the round-trip property."""
    require_gpu()
    wl = W.cold_pages()
    gs = wl.gs_unit if gs_kind == "unit" else wl.gs_calibrated
    g = O.Geometry(*wl.geometry)
    packed = gpu_quantize(wl.hot_pool, wl.geometry, gs, src=wl.src_slots, dst=wl.dst_slots)
    rng = np.random.default_rng(0)
    sample = np.concatenate([[0, wl.num_pages - 1], rng.choice(wl.num_pages, 30, replace=False)])
    ref = oracle_packed_pages(wl.hot_pool, wl.geometry, gs, wl.src_slots[sample])
    assert np.array_equal(packed[wl.dst_slots[sample]], ref)
    back = gpu_dequantize(packed, wl.geometry, gs, src=wl.dst_slots, dst=wl.src_slots)
    ref_back = np.zeros((len(sample), *g.row_shape), np.uint16)
    O.dequantize_pages(ref, g, len(sample), gs, ref_back)
    assert np.array_equal(back[wl.src_slots[sample]], ref_back)
    # whole pool: a second round trip changes nothing outside E4M3's two
    # smallest subnormal scales
    packed2 = gpu_quantize(back, wl.geometry, gs, src=wl.src_slots, dst=wl.dst_slots)
    nd, nb = g.elems // 2, g.elems // 16
    data1, sc1 = packed[:, :nd].reshape(-1, nb, 8), packed[:, nd:]
    data2, sc2 = packed2[:, :nd].reshape(-1, nb, 8), packed2[:, nd:]
    changed = np.any(data1 != data2, axis=-1) | (sc1 != sc2)
    assert set(np.unique(sc1[changed]).tolist()) <= {1, 2}
