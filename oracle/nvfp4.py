"""NVFP4 format and page codec -- plain fp64 CPU oracle (TEST INFRASTRUCTURE ONLY).

The format ("Accelerating Long-Context and Agentic Inference with NVFP4 KV
Cache", introduction / Figure 1; NVFP4 KV Decode Attention Kernel
Implementation): four-bit E2M1 values, one E4M3 (FP8) scale per block of 16
values, and one FP32 scale per tensor.  A block occupies eight bytes of
packed codes plus one scale byte (same page, kernel section), i.e. 0.5625
bytes per value ("KV Cache Compression in TensorRT LLM", Evaluation /
Performance, Figure 10).

Readings of what the pages leave open:

* E2M1 is the OCP 4-bit float: 1 sign, 2 exponent bits (bias 1), 1 mantissa
  bit, no inf/NaN; magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.  Code bits are
  ``sign<<3 | exp<<1 | mant``, so a magnitude code equals its grid index.
* E4M3 is OCP E4M3FN: bias 7, max 448, no inf, 0x7F / 0xFF are NaN.
* The tensor scale ``gs`` is a decode multiplier supplied by the caller:
  ``x ~= e2m1 * e4m3 * gs``.  The block scale maps the block's largest
  magnitude onto E2M1's largest, 6:  ``sb = E4M3(amax / (6 gs))``.
* Every rounding is round-to-nearest, ties to the even code, from the exact
  real quotient, saturating at the format's largest finite value.
* A block whose scale rounds to 0 stores magnitude code 0 for every element;
  every nibble keeps the sign bit of its bf16 input (so -0.0 gives 0x8).
* The block axis is 16 consecutive elements along head_dim of one
  (tensor, token, head) row; element 2k is the low nibble of byte k.
* Dequantization returns ``bf16_RNE(+-e2m1 * e4m3 * gs)``, one rounding from
  the exact product (IEEE overflow to +-inf).

Why fp64 is exact here.  ``6*gs``, ``sb*gs`` and every ``grid*sb*gs`` have at
most 31 significant bits, so fp64 holds them exactly.  A bf16 input has at
most 8 significant bits.  The quotient ``amax/(6 gs)`` (or ``|x|/(sb gs)``)
either equals a rounding midpoint exactly -- then the correctly rounded fp64
division returns that midpoint exactly -- or it differs from every midpoint by
at least 2**-31 relative, far above fp64's 2**-53 division error.  So one
fp64 division followed by exact comparisons with the midpoints rounds the
exact real quotient.  tests/test_oracle_codec.py checks this against an
exact-rational brute force.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# ----------------------------------------------------------------------------
# Element formats
# ----------------------------------------------------------------------------


def e2m1_magnitude(code: int) -> float:
    """Value of a 3-bit E2M1 magnitude code (exp 2 bits, bias 1; mant 1 bit)."""
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:  # subnormal: m * 2**-1
        return m * 0.5
    return (1.0 + m / 2.0) * 2.0 ** (e - 1)


#: E2M1 magnitudes indexed by magnitude code 0..7.
E2M1_GRID = np.array([e2m1_magnitude(c) for c in range(8)], dtype=np.float64)


def e4m3fn_decode(code: int) -> float:
    """Value of an OCP E4M3FN byte (bias 7, no inf, S.1111.111 is NaN)."""
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        v = (m / 8.0) * 2.0 ** -6
    else:
        v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


#: The 127 finite non-negative E4M3FN values, indexed by code 0x00..0x7E.
E4M3_FINITE = np.array([e4m3fn_decode(c) for c in range(127)], dtype=np.float64)

#: Full 256-entry decode table (NaN for 0x7F and 0xFF).
E4M3_TABLE = np.array([e4m3fn_decode(c) for c in range(256)], dtype=np.float64)


def round_half_even_to_grid(q: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index of the grid value nearest to each q >= 0, ties to the even index.

    ``grid`` is increasing and starts at 0; q above the last value saturates.
    The grid index is the format's code, so "even index" is "even code".
    """
    q = np.asarray(q, dtype=np.float64)
    i = np.searchsorted(grid, q, side="right") - 1  # largest i with grid[i] <= q
    i = np.clip(i, 0, len(grid) - 1)
    last = len(grid) - 1
    hi = np.minimum(i + 1, last)
    mid = (grid[i] + grid[hi]) / 2.0  # exact: grid values have few bits
    up = (q > mid) | ((q == mid) & (i % 2 == 1))
    out = np.where((i < last) & up, i + 1, i)
    return out.astype(np.int64)


# ----------------------------------------------------------------------------
# bf16 helpers
# ----------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_rne(v: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 (8 significant bits, exponent range of fp32),
    nearest with ties to even, once, including subnormals; overflow gives inf.
    Returns uint16 bit patterns.  Negative zero stays negative."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, e = np.frexp(a)  # a = f * 2**e, f in [0.5, 1)
    # bf16 normal numbers in binade [2**(e-1), 2**e) have spacing 2**(e-8);
    # below 2**-126 the spacing is fixed at 2**-133.
    ulp_exp = np.maximum(e - 8, -133)
    r = np.round(np.ldexp(a, -ulp_exp))  # numpy rounds half to even
    mag = np.ldexp(r, ulp_exp)
    out = np.where(np.signbit(v), -mag, mag)
    # every finite result is now exactly a bf16 value, hence exactly an fp32
    # value; values rounded to 2**128 or beyond become inf in fp32.
    with np.errstate(over="ignore"):
        f32 = out.astype(np.float32)
    bits = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return bits


def e4m3_codes_to_bf16_bits(codes: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of OCP E4M3FN bytes, exactly.

    Every finite E4M3 value (4 significant bits, magnitudes 2**-9 .. 448) is
    a bf16 value, so the widening is exact; a NaN code is refused.  This is
    how FP8 K/V (the pages' prefill and workspace type, "Accelerating
    Long-Context and Agentic Inference with NVFP4 KV Cache", Path 1) enter
    the NVFP4 encoder: as the bf16 values they equal.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    v = E4M3_TABLE[codes.astype(np.int64)]
    if np.any(np.isnan(v)):
        raise ValueError("E4M3 NaN codes (0x7F, 0xFF) are outside the contract")
    bits = f64_to_bf16_rne(v)
    assert np.array_equal(bf16_bits_to_f64(bits), v)
    return bits


# ----------------------------------------------------------------------------
# Block codec
# ----------------------------------------------------------------------------

BLOCK = 16


def tensor_scale(gs) -> float:
    """The FP32 tensor scale as a float.  The format fixes it as an FP32 value
    and the exactness argument above needs its 24-bit significand, so a value
    that FP32 cannot hold exactly is refused rather than silently used."""
    v = float(gs)
    if not (np.isfinite(v) and v > 0.0 and float(np.float32(v)) == v):
        raise ValueError(f"tensor scale {v!r} is not a positive finite FP32 value")
    return v


def encode_block_scale(amax: np.ndarray, gs: float) -> np.ndarray:
    """E4M3 scale code for blocks with largest magnitude ``amax``.

    ``sb = E4M3_RNE_SAT(amax / (6 gs))``: the block maximum maps onto E2M1's
    largest magnitude (6) after the tensor scale is taken out.
    """
    q = np.asarray(amax, dtype=np.float64) / (6.0 * tensor_scale(gs))
    return round_half_even_to_grid(q, E4M3_FINITE)


def encode_magnitudes(absx: np.ndarray, scale_value: np.ndarray, gs: float) -> np.ndarray:
    """E2M1 magnitude codes of ``|x| / (sb * gs)``; all zero where sb == 0."""
    absx = np.asarray(absx, dtype=np.float64)
    denom = np.asarray(scale_value, dtype=np.float64) * tensor_scale(gs)
    safe = np.where(denom > 0, denom, 1.0)
    y = absx / safe
    codes = round_half_even_to_grid(y, E2M1_GRID)
    return np.where(denom > 0, codes, 0)


def quantize_rows(xbits: np.ndarray, gs: float):
    """Quantize bf16 rows (last axis = head_dim, a multiple of 16).

    Returns ``(data, scales)``: uint8 arrays of shape ``[..., D/2]`` (two
    nibbles per byte, even element low) and ``[..., D/16]`` (E4M3 codes).
    """
    xbits = np.asarray(xbits, dtype=np.uint16)
    D = xbits.shape[-1]
    assert D % BLOCK == 0
    x = bf16_bits_to_f64(xbits)
    blocks = x.reshape(*x.shape[:-1], D // BLOCK, BLOCK)
    amax = np.max(np.abs(blocks), axis=-1)
    sb_code = encode_block_scale(amax, gs)
    sb_val = E4M3_FINITE[sb_code]
    mags = encode_magnitudes(np.abs(blocks), sb_val[..., None], gs)
    sign = ((xbits >> np.uint16(15)) & np.uint16(1)).astype(np.int64)
    nib = (sign.reshape(mags.shape) << 3) | mags
    nib = nib.reshape(*x.shape[:-1], D)
    data = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    return data, sb_code.astype(np.uint8)


def dequantize_rows(data: np.ndarray, scales: np.ndarray, gs: float) -> np.ndarray:
    """Inverse of :func:`quantize_rows`: bf16 bits of +-e2m1 * e4m3 * gs."""
    data = np.asarray(data, dtype=np.uint8)
    D = data.shape[-1] * 2
    nib = np.empty((*data.shape[:-1], D), dtype=np.int64)
    nib[..., 0::2] = data & 0xF
    nib[..., 1::2] = data >> 4
    v = exact_values(nib, scales, gs)
    return f64_to_bf16_rne(v)


def exact_values(nib: np.ndarray, scales: np.ndarray, gs: float) -> np.ndarray:
    """Exact fp64 values of nibbles ``nib[..., D]`` with scale codes
    ``scales[..., D/16]`` (at most 30 significant bits: exact in fp64)."""
    nib = np.asarray(nib, dtype=np.int64)
    D = nib.shape[-1]
    mag = E2M1_GRID[nib & 7]
    sval = E4M3_TABLE[np.asarray(scales, dtype=np.int64)]
    sval = np.repeat(sval, BLOCK, axis=-1).reshape(*nib.shape[:-1], D)
    v = mag * sval * tensor_scale(gs)
    return np.where((nib >> 3) & 1 == 1, -v, v)


# ----------------------------------------------------------------------------
# Pages
# ----------------------------------------------------------------------------


@dataclass(frozen=True)
class Geometry:
    """Page geometry: ``num_kv_tensors`` (2: K and V; 1: one shared MLA
    latent), tokens per page, KV heads, head_dim (multiple of 16)."""

    num_kv_tensors: int
    page_size: int
    num_kv_heads: int
    head_dim: int

    @property
    def elems(self) -> int:  # E: elements per page
        return self.num_kv_tensors * self.page_size * self.num_kv_heads * self.head_dim

    @property
    def row_shape(self):
        return (self.num_kv_tensors, self.page_size, self.num_kv_heads, self.head_dim)


def hot_page_bytes(g: Geometry) -> int:
    """bf16 page: 2 bytes per value."""
    return 2 * g.elems


def packed_page_bytes(g: Geometry) -> int:
    """One fixed-size block per page: 8 data bytes + 1 scale byte per 16
    values ("KV Cache Compression in TensorRT LLM", How It Works, one block
    per page; "Accelerating Long-Context ...", NVFP4 KV Decode Attention Kernel
    Implementation)."""
    return g.elems // 2 + g.elems // BLOCK


def split_packed_page(page: np.ndarray, g: Geometry):
    """Views ``(data [n_t,T,H,D/2], scales [n_t,T,H,D/16])`` of one packed page:
    the data region comes first, the scale region follows it."""
    nt, T, H, D = g.row_shape
    nd = g.elems // 2
    data = page[:nd].reshape(nt, T, H, D // 2)
    scales = page[nd:nd + g.elems // BLOCK].reshape(nt, T, H, D // BLOCK)
    return data, scales


def quantize_pages(hot_pool: np.ndarray, g: Geometry, num_pages: int, gs,
                   packed_pool: np.ndarray, src_slots=None, dst_slots=None) -> None:
    """Encode ``num_pages`` hot pages into packed slots, in place.

    ``hot_pool``: uint16 bf16 bits ``[slots, n_t, T, H, D]``;
    ``packed_pool``: uint8 ``[slots, packed_page_bytes]``.  Page i reads hot
    slot ``src_slots[i]`` (identity when None) and writes packed slot
    ``dst_slots[i]``.  ``gs[t]`` is the tensor scale of tensor t.
    """
    for i in range(num_pages):
        s = i if src_slots is None else int(src_slots[i])
        d = i if dst_slots is None else int(dst_slots[i])
        data, scales = split_packed_page(packed_pool[d], g)
        for t in range(g.num_kv_tensors):
            dt, sc = quantize_rows(hot_pool[s, t], float(gs[t]))
            data[t] = dt
            scales[t] = sc


def dequantize_pages(packed_pool: np.ndarray, g: Geometry, num_pages: int, gs,
                     hot_pool: np.ndarray, src_slots=None, dst_slots=None) -> None:
    """Decode ``num_pages`` packed pages back into bf16 hot slots, in place."""
    for i in range(num_pages):
        s = i if src_slots is None else int(src_slots[i])
        d = i if dst_slots is None else int(dst_slots[i])
        data, scales = split_packed_page(packed_pool[s], g)
        for t in range(g.num_kv_tensors):
            hot_pool[d, t] = dequantize_rows(data[t], scales[t], float(gs[t]))


def append_quantize(rows: np.ndarray, g: Geometry, gs, packed_pool: np.ndarray,
                    token_slots, token_rows) -> None:
    """Quantize new tokens' K/V rows into rows of packed pages, in place.

    The write path of the cache ("Accelerating Long-Context and Agentic
    Inference with NVFP4 KV Cache", Path 1 / Path 3: each step's new K/V are
    quantized into the NVFP4 pool as they are written).  A block is 16
    values of one (tensor, token, head) row, so a token's blocks never share
    a byte or a scale with another token: appending writes exactly that
    token's data and scale bytes and leaves the rest of the page as it was.

    ``rows``: ``[num_tokens, n_t, H, D]`` of uint16 bf16 bits, or of uint8
    E4M3FN codes (FP8 K/V), which are encoded as the bf16 values they equal;
    token i goes to packed slot ``token_slots[i]``, page row
    ``token_rows[i]``; a token whose slot is outside the pool or whose row is
    outside ``[0, page_size)`` is skipped.
    """
    rows = np.asarray(rows)
    if rows.dtype == np.uint8:
        rows = e4m3_codes_to_bf16_bits(rows)
    rows = np.asarray(rows, dtype=np.uint16)
    for i in range(rows.shape[0]):
        s, r = int(token_slots[i]), int(token_rows[i])
        if not (0 <= s < packed_pool.shape[0] and 0 <= r < g.page_size):
            continue
        data, scales = split_packed_page(packed_pool[s], g)
        for t in range(g.num_kv_tensors):
            dt, sc = quantize_rows(rows[i, t], float(gs[t]))
            data[t, r] = dt
            scales[t, r] = sc


def f64_to_e4m3_rne(v: np.ndarray) -> np.ndarray:
    """OCP E4M3FN codes of exact fp64 values: the magnitude rounded once to
    the nearest finite E4M3 value, ties to the even code, saturating at 448
    (never NaN); the sign bit is the value's sign bit (-0.0 gives 0x80)."""
    v = np.asarray(v, dtype=np.float64)
    mag = round_half_even_to_grid(np.abs(v), E4M3_FINITE)
    return (mag | (np.signbit(v).astype(np.int64) << 7)).astype(np.uint8)


def gather_dequantize(packed_pool: np.ndarray, g: Geometry, gs, token_slots, token_rows,
                      out_dtype: str = "bf16") -> np.ndarray:
    """Rows of packed pages gathered into a contiguous workspace.

    The extend path ("Accelerating Long-Context and Agentic Inference with
    NVFP4 KV Cache", Path 2: Chunked prefill / Extend): the cached prefix's
    NVFP4 entries are gathered, dequantized and written to a workspace that
    prefill attention reads (the page's workspace type is FP8; bf16 is the
    lossless alternative).  Output row i is row ``token_rows[i]`` of packed
    slot ``token_slots[i]``, ``[n_t, H, D]``, each value the exact
    ``+-e2m1 * e4m3 * gs[t]`` rounded once: to bf16 (``"bf16"``, uint16
    bits, as :func:`dequantize_rows`) or to E4M3FN (``"fp8"``, uint8 codes,
    :func:`f64_to_e4m3_rne`).  A token whose slot is outside the pool or whose
    row is outside ``[0, page_size)`` gives an all-zero row.
    """
    n = len(token_slots)
    nt, T, H, D = g.row_shape
    dt = np.uint16 if out_dtype == "bf16" else np.uint8
    out = np.zeros((n, nt, H, D), dtype=dt)
    for i in range(n):
        s, r = int(token_slots[i]), int(token_rows[i])
        if not (0 <= s < packed_pool.shape[0] and 0 <= r < T):
            continue
        data, scales = split_packed_page(packed_pool[s], g)
        for t in range(nt):
            d = np.asarray(data[t, r], dtype=np.uint8)
            nib = np.empty((H, D), dtype=np.int64)
            nib[:, 0::2] = d & 0xF
            nib[:, 1::2] = d >> 4
            v = exact_values(nib, scales[t, r], float(gs[t]))
            out[i, t] = f64_to_bf16_rne(v) if out_dtype == "bf16" else f64_to_e4m3_rne(v)
    return out
