"""Pins for the oracle's block and page codec."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import nvfp4 as O
from tests import exact as X
from nvfp4_paged_decode_amd.workloads import f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _random_blocks(rng, n, lo=-6, hi=3):
    mag = 10.0 ** rng.uniform(lo, hi, size=(n, 1))
    return f32_to_bf16_bits((rng.standard_normal((n, 16)) * mag).astype(np.float32))


def _adversarial_blocks(rng, gs):
    """Blocks whose quotients sit exactly on E4M3 / E2M1 rounding midpoints,
    at saturation, at zero, and with signed zeros."""
    out = []
    e4 = O.E4M3_FINITE
    for c in range(0, 126):
        mid = (e4[c] + e4[c + 1]) / 2.0
        amax = np.float32(mid * 6.0 * gs)  # exact when gs is a power of two
        blk = np.full(16, 0.0, np.float32)
        blk[rng.integers(16)] = amax
        blk[rng.integers(16)] = -amax
        out.append(f32_to_bf16_bits(blk))
    sb = O.E4M3_FINITE[rng.integers(1, 127, 64)]
    for s in sb:  # element quotients exactly on E2M1 midpoints
        mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0])
        vals = rng.choice(mids, 16) * s * gs * rng.choice([-1, 1], 16)
        vals[0] = 6.0 * s * gs
        out.append(f32_to_bf16_bits(vals.astype(np.float32)))
    out.append(np.zeros(16, np.uint16))                       # all +0
    out.append(np.full(16, 0x8000, np.uint16))                # all -0
    out.append(f32_to_bf16_bits(np.full(16, 3e38, np.float32)))  # saturating
    out.append(f32_to_bf16_bits(np.array([1e-40] * 8 + [-1e-40] * 8, np.float32)))
    return np.stack(out)


@pytest.mark.parametrize("gs", [1.0, 0.5, 2.0 ** -12, float(np.float32(0.0123456)),
                                float(np.float32(7.77e-3)), float(np.float32(3.0))])
def test_block_quantizer_equals_exact_rational_brute_force(gs):
    rng = np.random.default_rng(int(gs * 1e6) % 1000 + 7)
    blocks = np.concatenate([_random_blocks(rng, 1500), _adversarial_blocks(rng, gs)])
    data, scales = O.quantize_rows(blocks, gs)
    gsf = Fraction(gs)
    for i in range(blocks.shape[0]):
        nibs, sb = X.quantize_block_exact(blocks[i], gsf)
        assert scales[i, 0] == sb, (i, blocks[i])
        packed = [nibs[2 * k] | (nibs[2 * k + 1] << 4) for k in range(8)]
        assert list(data[i]) == packed, (i, blocks[i])


def test_all_zero_block_gives_scale_zero():
    data, scales = O.quantize_rows(np.zeros((3, 32), np.uint16), 1.0)
    assert np.all(scales == 0) and np.all(data == 0)
    # -0.0 keeps its sign bit in every nibble
    data, scales = O.quantize_rows(np.full((1, 16), 0x8000, np.uint16), 1.0)
    assert np.all(scales == 0) and np.all(data == 0x88)
    assert np.all(O.dequantize_rows(data, scales, 1.0) == 0x8000)


@pytest.mark.parametrize("gs", [1.0, 0.25, 1.5, 2.0 ** -20])
def test_representable_values_round_trip_exactly(gs):
    # x = c * sb * gs with a block maximum of 6 is a fixed point: quantize
    # returns sb and c, dequantize returns x
    rng = np.random.default_rng(11)
    for _ in range(400):
        sbc = int(rng.integers(1, 127))
        codes = rng.integers(0, 8, 16)
        codes[rng.integers(16)] = 7
        sign = rng.integers(0, 2, 16)
        vals = O.E2M1_GRID[codes] * O.E4M3_FINITE[sbc] * gs * np.where(sign == 1, -1.0, 1.0)
        bits = O.f64_to_bf16_rne(vals)
        if not np.array_equal(O.bf16_bits_to_f64(bits), vals):
            continue  # not representable in bf16 (deep subnormal); skip
        data, scales = O.quantize_rows(bits[None], gs)
        assert scales[0, 0] == sbc
        nib = (sign << 3) | codes
        assert list(data[0]) == [int(nib[2 * k] | (nib[2 * k + 1] << 4)) for k in range(8)]
        assert np.array_equal(O.dequantize_rows(data, scales, gs)[0], bits)


@pytest.mark.parametrize("gs", [1.0, float(np.float32(0.0123456))])
def test_round_trips_do_not_accumulate_error(gs):
    # "KV Cache Compression in TensorRT LLM", Evaluation / Accuracy, Figure 15:
    # after the first round trip the next one changes nothing.  Under the
    # readings here this holds for every block whose scale is at least
    # 3 * 2**-9; the two smallest E4M3 subnormals are the one exception
    # (there the re-quantized block maximum can tie down to scale 0).
    rng = np.random.default_rng(5)
    x = _random_blocks(rng, 20000, lo=-5, hi=2)
    d1, s1 = O.quantize_rows(x, gs)
    y1 = O.dequantize_rows(d1, s1, gs)
    d2, s2 = O.quantize_rows(y1, gs)
    y2 = O.dequantize_rows(d2, s2, gs)
    changed = ~np.all(y2 == y1, axis=1)
    assert set(np.unique(s1[changed, 0])) <= {1, 2}
    assert not np.any(changed & (s1[:, 0] >= 3))
    d3, s3 = O.quantize_rows(y2, gs)
    y3 = O.dequantize_rows(d3, s3, gs)
    assert np.array_equal(y3, y2)  # stable from the second trip on


def test_storage_accounting_matches_the_pages():
    with open(os.path.join(GOLDEN, "page_figures.json")) as f:
        fig = json.load(f)
    g = O.Geometry(2, 64, 8, 128)  # {K,V} x 64 tokens x 8 heads x 128 dims
    per_value = O.packed_page_bytes(g) / g.elems
    assert per_value == fig["bytes_per_value_nvfp4"]["value"]
    assert 8 * per_value == fig["bits_per_value"]["value"]
    assert O.packed_page_bytes(O.Geometry(1, 1, 1, 16)) == fig["bytes_per_block_of_16"]["value"]
    fp8, bf16 = g.elems * 1, O.hot_page_bytes(g)
    assert round(100 * (1 - O.packed_page_bytes(g) / fp8), 2) == fig["reduction_vs_fp8_pct"]["value"]
    assert round(100 * (1 - O.packed_page_bytes(g) / bf16), 1) == fig["reduction_vs_bf16_pct"]["value"]
    assert round(100 * O.packed_page_bytes(g) / fp8) == fig["share_of_fp8_pct"]["value"]
    assert round(fp8 / O.packed_page_bytes(g), 2) == fig["capacity_vs_fp8"]["value"]
    assert O.packed_page_bytes(g) == 73728 and O.hot_page_bytes(g) == 262144


def test_page_codec_layout_and_slots():
    g = O.Geometry(2, 4, 2, 32)
    rng = np.random.default_rng(3)
    hot = _random_blocks(rng, 6 * g.elems // 16).reshape(6, *g.row_shape)
    packed = np.zeros((6, O.packed_page_bytes(g)), np.uint8)
    src = np.array([4, 0, 5]); dst = np.array([1, 3, 2])
    gs = [1.0, float(np.float32(0.03))]
    O.quantize_pages(hot, g, 3, gs, packed, src, dst)
    for i in range(3):
        page = packed[dst[i]]
        for t in range(2):
            d, s = O.quantize_rows(hot[src[i], t], gs[t])
            nd = g.elems // 2
            assert np.array_equal(page[t * nd // 2:(t + 1) * nd // 2], d.reshape(-1))
            ns = g.elems // 16
            assert np.array_equal(page[nd + t * ns // 2: nd + (t + 1) * ns // 2], s.reshape(-1))
    assert np.all(packed[[0, 4, 5]] == 0)  # untouched slots
    back = np.zeros_like(hot)
    O.dequantize_pages(packed, g, 3, gs, back, dst, src)
    for i in range(3):
        for t in range(2):
            d, s = O.quantize_rows(hot[src[i], t], gs[t])
            assert np.array_equal(back[src[i], t], O.dequantize_rows(d, s, gs[t]))


def test_golden_page_bytes_are_stable():
    z = np.load(os.path.join(GOLDEN, "tiny_page.npz"))
    g = O.Geometry(*[int(v) for v in z["geometry"]])
    packed = np.zeros((1, O.packed_page_bytes(g)), np.uint8)
    O.quantize_pages(z["hot"], g, 1, z["gs"], packed)
    assert np.array_equal(packed[0], z["packed"])
    back = np.zeros_like(z["hot"])
    O.dequantize_pages(packed, g, 1, z["gs"], back)
    assert np.array_equal(back, z["dequant"])


def test_append_rows_rebuild_the_page_and_touch_nothing_else():
    """Appending a page's tokens one at a time, in any order, gives the same
    bytes as encoding the whole page (a block never spans two tokens), and
    each append writes only its own row's data and scale bytes."""
    g = O.Geometry(2, 8, 3, 32)
    rng = np.random.default_rng(11)
    hot = _random_blocks(rng, g.elems // 16).reshape(1, *g.row_shape)
    gs = [float(np.float32(0.7)), float(np.float32(0.02))]
    whole = np.zeros((1, O.packed_page_bytes(g)), np.uint8)
    O.quantize_pages(hot, g, 1, gs, whole)
    rows = np.ascontiguousarray(hot[0].transpose(1, 0, 2, 3))  # [T, n_t, H, D]
    order = rng.permutation(g.page_size)
    built = np.full((2, O.packed_page_bytes(g)), 0xA5, np.uint8)
    for r in order:
        before = built.copy()
        O.append_quantize(rows[r:r + 1], g, gs, built, [0], [r])
        changed = np.nonzero(before[0] != built[0])[0]
        data, scales = O.split_packed_page(np.arange(O.packed_page_bytes(g)), g)
        allowed = set(data[:, r].reshape(-1)) | set(scales[:, r].reshape(-1))
        assert set(changed.tolist()) <= allowed
        assert np.array_equal(before[1], built[1])  # other slot untouched
    assert np.array_equal(built[0], whole[0])


def test_append_skips_bad_slots_and_rows():
    g = O.Geometry(1, 4, 1, 16)
    rng = np.random.default_rng(12)
    rows = _random_blocks(rng, 3).reshape(3, 1, 1, 16)
    pool = np.zeros((2, O.packed_page_bytes(g)), np.uint8)
    O.append_quantize(rows, g, [1.0], pool, [2, -1, 0], [0, 1, 4])
    assert np.all(pool == 0)
    O.append_quantize(rows, g, [1.0], pool, [1, 1, 1], [3, 3, 0])
    d, s = O.quantize_rows(rows[2, 0], 1.0)
    data, scales = O.split_packed_page(pool[1], g)
    assert np.array_equal(data[0, 0], d) and np.array_equal(scales[0, 0], s)


def test_gather_returns_representable_rows_exactly():
    """Rows whose values are exactly e2m1 * e4m3 * gs (and bf16) come back
    from the gather bit for bit, in any token order; bad slots and rows give
    zero rows."""
    g = O.Geometry(2, 8, 2, 32)
    rng = np.random.default_rng(31)
    gs = [1.0, 0.375]
    n_tok = 10
    x = np.zeros((n_tok, 2, 2, 32))
    for t in range(2):
        sb = O.E4M3_FINITE[rng.integers(40, 110, size=(n_tok, 2, 2))]
        codes = rng.integers(0, 8, size=(n_tok, 2, 32))
        codes[:, :, 0] = 7  # the block maximum maps onto 6 exactly
        codes[:, :, 16] = 7
        vals = O.E2M1_GRID[codes] * np.repeat(sb, 16, axis=-1) * gs[t]
        x[:, t] = vals * rng.choice([-1.0, 1.0], size=vals.shape)
    bits = O.f64_to_bf16_rne(x)
    assert np.array_equal(O.bf16_bits_to_f64(bits), x)  # representable
    pool = np.zeros((3, O.packed_page_bytes(g)), np.uint8)
    cells = rng.choice(3 * g.page_size, n_tok, replace=False)
    slots, rows = cells // g.page_size, cells % g.page_size
    O.append_quantize(bits, g, gs, pool, slots, rows)
    order = rng.permutation(n_tok)
    got = O.gather_dequantize(pool, g, gs, slots[order], rows[order], "bf16")
    assert np.array_equal(got, bits[order])
    bad = O.gather_dequantize(pool, g, gs, [3, -1, 0], [0, 0, 8], "fp8")
    assert bad.shape == (3, 2, 2, 32) and np.all(bad == 0)


def test_gather_fp8_equals_torch_cast_of_exact_values():
    """FP8 output: each value is the exact e2m1 * e4m3 * gs rounded once to
    E4M3FN.  With gs = 1 every such value fits bf16 exactly, so torch's
    bfloat16 -> float8_e4m3fn cast of the bf16 gather is an independent
    rounding of the same value (it matches below 464, where torch saturates
    to NaN instead)."""
    import torch
    g = O.Geometry(2, 16, 2, 64)
    rng = np.random.default_rng(32)
    hot = _random_blocks(rng, g.elems // 16, lo=-4, hi=3).reshape(1, *g.row_shape)
    gs = [1.0, 1.0]
    pool = np.zeros((1, O.packed_page_bytes(g)), np.uint8)
    O.quantize_pages(hot, g, 1, gs, pool)
    slots, rows = np.zeros(16, np.int64), np.arange(16)
    b16 = O.gather_dequantize(pool, g, gs, slots, rows, "bf16")
    f8 = O.gather_dequantize(pool, g, gs, slots, rows, "fp8")
    v = O.bf16_bits_to_f64(b16)
    keep = np.abs(v) < 464
    ref = torch.from_numpy(b16.view(np.int16)).view(torch.bfloat16).to(torch.float8_e4m3fn)
    ref = ref.view(torch.uint8).numpy()
    assert keep.mean() > 0.9 and np.array_equal(f8[keep], ref[keep])
    assert np.all((f8[~keep] & 0x7F) == 0x7E)  # saturated to +-448


@pytest.mark.parametrize("gs", [0.7, 1.0 / 3.0, 1.2345e-3, 37.5])
def test_dequantize_rows_equals_exact_rational_rounding(gs):
    """Every (code, scale) pair at a non-power-of-two tensor scale: the
    oracle's bf16 value is the bf16 nearest (ties to even) to the exact
    rational product e2m1 * e4m3 * gs, found by the brute-force rounding of
    tests/exact.py."""
    from fractions import Fraction
    from tests.exact import E2M1, E4M3, bf16_round_exact
    gs32 = float(np.float32(gs))
    gsf = Fraction(gs32)
    nibs = np.arange(16, dtype=np.int64)
    codes = np.arange(127, dtype=np.uint8)  # every finite scale code
    # one 16-value block per scale code holding all 16 nibbles
    data = np.tile((nibs[0::2] | (nibs[1::2] << 4)).astype(np.uint8), (127, 1))
    got = O.dequantize_rows(data, codes[:, None], gs32)
    for c in range(127):
        for n in range(16):
            v = E2M1[n & 7] * E4M3[c] * gsf
            want = bf16_round_exact(-v if n & 8 else v)
            if v == 0 and n & 8:
                want = 0x8000  # -0 keeps its sign
            assert int(got[c, n]) == want, (gs, c, n)
