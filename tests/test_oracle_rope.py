"""Pins for the RoPE-part storage variants of the cold-page codec oracle
(oracle/rope.py): kept-at-bf16 RoPE dims, and 2FP4 (a second NVFP4 layer
holding the first one's rounding error)."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import nvfp4 as O
from oracle import rope as RP
from tests import exact as X
from nvfp4_paged_decode_amd.workloads import f32_to_bf16_bits


def _hot(rng, g, n):
    x = rng.standard_normal((n, *g.row_shape)).astype(np.float32)
    x *= (10.0 ** rng.uniform(-3, 2, (n, g.num_kv_tensors, 1, g.num_kv_heads, 1))).astype(np.float32)
    return f32_to_bf16_bits(x)


def _round_trip(g, rope, hot, gs):
    pool = np.zeros((hot.shape[0], RP.packed_page_bytes(g, rope)), np.uint8)
    RP.quantize_pages(hot, g, rope, hot.shape[0], gs, pool)
    back = np.zeros_like(hot)
    RP.dequantize_pages(pool, g, rope, hot.shape[0], gs, back)
    return pool, back


def test_page_sizes():
    g = O.Geometry(1, 64, 1, 576)  # MLA latent, 64 RoPE dims
    base = 64 * 576 * 9 // 16
    assert RP.packed_page_bytes(g, RP.RopeLayout(64, RP.ROPE_NVFP4)) == base
    assert RP.packed_page_bytes(g, RP.RopeLayout(64, RP.ROPE_BF16)) == base + 64 * 64 * 2
    assert RP.packed_page_bytes(g, RP.RopeLayout(64, RP.ROPE_2FP4)) == base + 64 * 64 * 9 // 16


@pytest.mark.parametrize("mode", [RP.ROPE_NVFP4, RP.ROPE_BF16, RP.ROPE_2FP4])
def test_base_region_and_non_rope_values_are_the_plain_codec(mode):
    g = O.Geometry(2, 8, 2, 64)
    rng = np.random.default_rng(40 + mode)
    hot = _hot(rng, g, 2)
    gs = [float(np.float32(0.02)), float(np.float32(0.5))]
    rope = RP.RopeLayout(32, mode)
    pool, back = _round_trip(g, rope, hot, gs)
    plain = np.zeros((2, O.packed_page_bytes(g)), np.uint8)
    O.quantize_pages(hot, g, 2, gs, plain)
    assert np.array_equal(pool[:, :O.packed_page_bytes(g)], plain)
    plain_back = np.zeros_like(hot)
    O.dequantize_pages(plain, g, 2, gs, plain_back)
    assert np.array_equal(back[:, 1], plain_back[:, 1])            # V untouched
    assert np.array_equal(back[:, 0, ..., :32], plain_back[:, 0, ..., :32])  # K's other dims
    if mode == RP.ROPE_BF16:
        assert np.array_equal(back[:, 0, ..., 32:], hot[:, 0, ..., 32:])  # kept exactly


def test_2fp4_second_layer_is_the_exact_residual_quantized():
    """Each block of the extension region equals an exact-rational
    brute-force quantization of r = x - D1 (nearest E4M3 scale for
    amax/(6 gs), nearest E2M1 for |r|/(sb gs), ties even), and the decoded
    value is the bf16 nearest to D1 + D2."""
    g = O.Geometry(1, 4, 2, 48)
    rng = np.random.default_rng(41)
    hot = _hot(rng, g, 1)
    gsf = float(np.float32(0.0371))
    rope = RP.RopeLayout(32, RP.ROPE_2FP4)
    pool, back = _round_trip(g, rope, hot, [gsf])
    gs = Fraction(gsf)
    data, scales = O.split_packed_page(pool[0][:O.packed_page_bytes(g)], g)
    e_data, e_scales = RP.split_extension(pool[0], g, rope)

    def vals(d, s):
        nib = [(int(b) >> (4 * k)) & 0xF for b in d for k in (0, 1)]
        return [(-1 if n & 8 else 1) * X.E2M1[n & 7] * X.E4M3[int(s[i // 16])] * gs
                for i, n in enumerate(nib)]

    for t in range(g.page_size):
        for h in range(g.num_kv_heads):
            x = [X.bf16_fraction(int(b)) for b in hot[0, 0, t, h, 16:]]
            d1 = vals(data[0, t, h, 8:], scales[0, t, h, 1:])
            r = [a - b for a, b in zip(x, d1)]
            d2 = vals(e_data[t, h], e_scales[t, h])
            for blk in range(2):
                rb = r[16 * blk:16 * blk + 16]
                sb = X.nearest_even(max(abs(v) for v in rb) / (6 * gs), X.E4M3)
                assert int(e_scales[t, h, blk]) == sb
                for i, v in enumerate(rb):
                    want = 0 if X.E4M3[sb] == 0 else X.nearest_even(abs(v) / (X.E4M3[sb] * gs), X.E2M1)
                    got = vals(e_data[t, h], e_scales[t, h])[16 * blk + i]
                    assert abs(got) == X.E2M1[want] * X.E4M3[sb] * gs
            for i in range(32):
                assert int(back[0, 0, t, h, 16 + i]) == X.bf16_round_exact(d1[i] + d2[i]) or \
                    (d1[i] + d2[i] == 0)


def test_2fp4_never_increases_the_error_and_keeps_exact_values():
    g = O.Geometry(1, 16, 1, 64)
    rng = np.random.default_rng(42)
    hot = _hot(rng, g, 3)
    rope = RP.RopeLayout(64, RP.ROPE_2FP4)
    gs = [float(np.float32(0.011))]
    _, back2 = _round_trip(g, rope, hot, gs)
    _, back0 = _round_trip(g, RP.RopeLayout(64, RP.ROPE_NVFP4), hot, gs)
    x = O.bf16_bits_to_f64(hot)
    e2 = np.abs(O.bf16_bits_to_f64(back2) - x)
    e0 = np.abs(O.bf16_bits_to_f64(back0) - x)
    # |x - (D1 + D2)| <= |x - D1| before the final bf16 rounding (0 is on the
    # second layer's grid), and the rounding adds at most half a bf16 ulp
    half_ulp = np.abs(x) * 2.0 ** -8
    assert np.all(e2 <= e0 + half_ulp)
    assert e2.mean() < e0.mean() / 4
    # values the first layer holds exactly (and signed zeros) come back as
    # they were (a tensor scale of few bits keeps them bf16 values)
    gs = [0.375]
    vals = np.outer([0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, 0.0], [1.0]) * 0.25 * gs[0]
    blk = np.resize(vals.reshape(-1), 64)
    blk[0] = 6.0 * 0.25 * gs[0]  # the block maximum fixes scale 0.25 exactly
    blk[16] = blk[32] = blk[48] = blk[0]
    xs = np.tile(blk, (1, 1, 16, 1, 1)).reshape(1, *g.row_shape) * np.where(
        np.arange(64) % 3 == 0, -1.0, 1.0)
    bits = O.f64_to_bf16_rne(xs)
    assert np.array_equal(O.bf16_bits_to_f64(bits), xs)
    pool, back = _round_trip(g, rope, bits, gs)
    assert np.array_equal(back, bits)
    _, e_scales = RP.split_extension(pool[0], g, rope)
    assert np.all(e_scales == 0)


def test_fraction_rounding_matches_the_fp64_rounding_on_fp64_values():
    rng = np.random.default_rng(43)
    v = rng.standard_normal(2000) * 10.0 ** rng.uniform(-40, 38, 2000)
    ours = [RP.fraction_to_bf16_rne(Fraction(float(a))) for a in v]
    assert ours == O.f64_to_bf16_rne(v).astype(int).tolist()
