"""GPU parity of the RoPE-part storage variants of the cold-page codec
(RoPE dims kept at bf16, and 2FP4) against the oracle: packed slots and
decoded pages bit for bit."""

import numpy as np
import pytest

import nvfp4_paged_decode_amd as K
from nvfp4_paged_decode_amd import workloads as W
from oracle import nvfp4 as O
from oracle import rope as RP
from tests.gpu_common import dev, host, require_gpu, torch

pytestmark = pytest.mark.gpu


def _pages(rng, g, n, gs):
    """bf16 pages over several decades, with K's RoPE dims salted with
    signed zeros, values the first layer holds exactly and E2M1 midpoints."""
    x = rng.standard_normal((n, *g.row_shape)).astype(np.float32)
    x *= (10.0 ** rng.uniform(-4, 3, (n, g.num_kv_tensors, 1, g.num_kv_heads, 1))).astype(np.float32)
    bits = W.f32_to_bf16_bits(x)
    k = bits[:, 0]  # a view: K (or the latent) of every page
    idx = np.unravel_index(rng.choice(k.size, k.size // 25, replace=False), k.shape)
    q = idx[0].size // 3
    k[tuple(c[:q] for c in idx)] = 0x8000          # -0
    k[tuple(c[q:2 * q] for c in idx)] = 0x0000     # +0
    # values e2m1 * sb * gs[0], held exactly by the first layer when their
    # block's scale is sb (a power of two times gs[0], bf16 when gs[0] is)
    v = rng.choice([0.5, 1.5, 3.0, 6.0], size=idx[0].size - 2 * q) * 2.0 ** rng.integers(-6, 3)
    k[tuple(c[2 * q:] for c in idx)] = W.f32_to_bf16_bits((v * gs[0]).astype(np.float32))
    return bits


@pytest.mark.parametrize("geometry,rope_dims", [((1, 64, 1, 576), 64), ((2, 16, 8, 128), 128),
                                                ((2, 16, 4, 128), 64)])
@pytest.mark.parametrize("mode", [K.KVFP4_ROPE_NVFP4, K.KVFP4_ROPE_BF16, K.KVFP4_ROPE_2FP4])
def test_rope_layouts_bit_exact(geometry, rope_dims, mode):
    require_gpu()
    g = O.Geometry(*geometry)
    rope = RP.RopeLayout(rope_dims, mode)
    rng = np.random.default_rng(rope_dims + 10 * mode)
    n = 3
    gs = [float(np.float32(0.0173)), float(np.float32(2.5))][:g.num_kv_tensors]
    hot = _pages(rng, g, n, gs)
    # two more pages that must be skipped: a negative source slot, and a
    # destination one past the pool; the reference encodes the valid three
    src = np.array([2, 0, 1, -1, 1], np.int32)
    dst = np.array([1, 3, 0, 2, 4], np.int32)
    pb = RP.packed_page_bytes(g, rope)
    assert K.kvfp4_packed_page_bytes_rope(geometry, (rope_dims, mode)) == pb
    ref = np.zeros((4, pb), np.uint8)
    RP.quantize_pages(hot, g, rope, n, gs, ref, src[:n], dst[:n])
    pool = torch.zeros((4, pb), dtype=torch.uint8, device="cuda")
    K.kvfp4_quantize_pages_rope(geometry, (rope_dims, mode), dev(hot.view(np.int16)), pool, n + 2,
                                gs, dev(src), dev(dst))
    got = host(pool)
    mism = np.nonzero(got != ref)
    assert mism[0].size == 0, f"{mism[0].size} bytes differ, first at {mism[0][0]},{mism[1][0]}"
    back_ref = np.full((4, *g.row_shape), 0x1234, np.uint16)
    # packed slots in, hot slots out; again two skipped pages (a source
    # past the pool, a negative destination)
    dsrc = np.array([1, 3, 0, 7, 0], np.int32)
    ddst = np.array([2, 0, 1, 3, -2], np.int32)
    RP.dequantize_pages(ref, g, rope, n, gs, back_ref, dsrc[:n], ddst[:n])
    back = torch.full((4, *g.row_shape), 0x1234, dtype=torch.int16, device="cuda")
    K.kvfp4_dequantize_pages_rope(geometry, (rope_dims, mode), dev(ref), back, n + 2, gs,
                                  dev(dsrc), dev(ddst))
    got_back = host(back).view(np.uint16)
    mism = np.nonzero(got_back != back_ref)
    assert mism[0].size == 0, f"{mism[0].size} values differ, first at {[m[0] for m in mism]}"
