"""RoPE-part storage variants of the cold-page codec -- plain CPU oracle
(TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU baseline, never by the product path).

"KV Cache Compression in TensorRT LLM", How It Works / The RoPE part of K:
the position-encoded part of each K vector is the most sensitive to
quantization.  By default it is quantized like the rest; it can instead be
kept at its original precision (a lower compression ratio), or stored as
two FP4 components where the second holds the first one's rounding error
(2FP4).  Readings of what the page leaves open:

* The RoPE part is the last ``rope_dims`` dimensions of every head row of
  tensor 0 (K; for MLA the shared latent, whose last 64 of 576 dimensions
  carry the rotary embedding).  ``rope_dims`` is a multiple of 16, so RoPE
  blocks never mix with the rest.
* The page keeps the base layout (every value encoded as NVFP4, data region
  then scale region) and appends one extension region for the RoPE part,
  ``[T][H][rope_dims]`` per page:
    - mode BF16: the original bf16 values (2 bytes each); decoding takes
      them as they are;
    - mode 2FP4: a second NVFP4 layer, data ``[T][H][R/2]`` then scales
      ``[T][H][R/16]``, encoding the exact residual ``r = x - D1`` of the
      first layer ``D1 = +-e2m1 * e4m3 * gs`` with the same rules and the
      same tensor scale; decoding returns ``bf16_RNE(D1 + D2)``, one rounding
      of the exact sum.
* A residual of exactly zero takes the sign of ``x``, so that a signed zero
  (or a value the first layer holds exactly) keeps its sign through both
  layers; a zero sum keeps the sign IEEE addition gives it.

Exactness.  ``x`` (bf16, 8 significant bits) and ``D1`` (at most 30) are
within a few binades of each other whenever ``D1 != 0``, so ``r`` is exact in
fp64.  ``r`` has up to about 40 significant bits, so unlike a bf16 input its
quotient by ``6 gs`` is not decided exactly by one fp64 division: the
residual layer is therefore decided by exact comparisons against the
rounding midpoints times the scales (each product exact in fp64).  The sum
``D1 + D2`` can need more than 53 bits, so it is formed as a Fraction.
"""

from __future__ import annotations

from dataclasses import dataclass
from fractions import Fraction

import numpy as np

from oracle import nvfp4 as O

ROPE_NVFP4 = 0  # quantized like the rest: no extension region
ROPE_BF16 = 1   # kept at original precision
ROPE_2FP4 = 2   # two FP4 layers, the second the first one's rounding error


@dataclass(frozen=True)
class RopeLayout:
    rope_dims: int
    mode: int


def extension_bytes(g: O.Geometry, rope: RopeLayout) -> int:
    n = g.page_size * g.num_kv_heads * rope.rope_dims
    if rope.mode == ROPE_BF16:
        return 2 * n
    if rope.mode == ROPE_2FP4:
        return n // 2 + n // O.BLOCK
    return 0


def packed_page_bytes(g: O.Geometry, rope: RopeLayout) -> int:
    return O.packed_page_bytes(g) + extension_bytes(g, rope)


def split_extension(page: np.ndarray, g: O.Geometry, rope: RopeLayout):
    """The extension region of one page: ``bf16 [T, H, R]`` (uint8 view
    reinterpreted by the caller) for mode BF16, ``(data [T,H,R/2], scales
    [T,H,R/16])`` for mode 2FP4."""
    base = O.packed_page_bytes(g)
    T, H, R = g.page_size, g.num_kv_heads, rope.rope_dims
    ext = page[base:base + extension_bytes(g, rope)]
    if rope.mode == ROPE_BF16:
        return ext.reshape(T, H, R, 2)
    nd = T * H * R // 2
    return ext[:nd].reshape(T, H, R // 2), ext[nd:].reshape(T, H, R // O.BLOCK)


def _round_even_by_thresholds(x: np.ndarray, th: np.ndarray) -> np.ndarray:
    """Index of the interval of ``x`` between increasing exact thresholds
    (the midpoints between consecutive codes): the number of thresholds below
    ``x``; at a threshold exactly, the even one of the two codes."""
    i = np.searchsorted(th, x, side="left")  # thresholds < x
    tie = (i < len(th)) & (th[np.minimum(i, len(th) - 1)] == x)
    return np.where(tie & (i % 2 == 1), i + 1, i).astype(np.int64)


def quantize_residual(r: np.ndarray, gs: float):
    """NVFP4 encoding of exact fp64 values ``r[..., R]`` (blocks of 16 along
    the last axis), with every rounding decided by exact comparisons.
    Returns ``(data [..., R/2], scales [..., R/16])`` like quantize_rows."""
    gs = O.tensor_scale(gs)
    r = np.asarray(r, dtype=np.float64)
    R = r.shape[-1]
    blocks = r.reshape(*r.shape[:-1], R // O.BLOCK, O.BLOCK)
    amax = np.max(np.abs(blocks), axis=-1)
    e4 = O.E4M3_FINITE
    mids6 = (e4[:-1] + e4[1:]) / 2.0 * 6.0 * gs  # exact: <= 5 + 2 + 24 bits
    sb = _round_even_by_thresholds(amax, mids6)
    sbv = e4[sb]
    g = O.E2M1_GRID
    mu = (g[:-1] + g[1:]) / 2.0
    th = mu[None, :] * (sbv.reshape(-1, 1) * gs)  # exact: <= 3 + 4 + 24 bits
    ax = np.abs(blocks).reshape(-1, O.BLOCK)
    codes = np.stack([_round_even_by_thresholds(ax[i], th[i]) for i in range(ax.shape[0])])
    codes = np.where(sbv.reshape(-1, 1) > 0, codes, 0).reshape(blocks.shape)
    sign = np.signbit(blocks).astype(np.int64)
    nib = ((sign << 3) | codes).reshape(r.shape)
    data = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    return data, sb.astype(np.uint8)


def fraction_to_bf16_rne(q: Fraction, negative_zero: bool = False) -> int:
    """bf16 bits of an exact rational, rounded once to nearest, ties even."""
    if q == 0:
        return 0x8000 if negative_zero else 0
    s = 0x8000 if q < 0 else 0
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1  # now 2**e <= a < 2**(e+1)
    ulp = max(e - 7, -133)
    k = round(a / Fraction(2) ** ulp)  # Fraction rounds half to even
    v = float(Fraction(k) * Fraction(2) ** ulp)
    with np.errstate(over="ignore"):
        f = np.float32(v)
    return s | int(np.array([f]).view(np.uint32)[0] >> 16)


def _values(data, scales, gs):
    d = np.asarray(data, dtype=np.uint8)
    nib = np.empty((*d.shape[:-1], d.shape[-1] * 2), dtype=np.int64)
    nib[..., 0::2] = d & 0xF
    nib[..., 1::2] = d >> 4
    return O.exact_values(nib, scales, gs)


def quantize_pages(hot_pool, g: O.Geometry, rope: RopeLayout, num_pages: int, gs,
                   packed_pool, src_slots=None, dst_slots=None) -> None:
    """Base encoding of every value (as O.quantize_pages) plus the RoPE
    extension region of each page."""
    R = rope.rope_dims
    for i in range(num_pages):
        s = i if src_slots is None else int(src_slots[i])
        d = i if dst_slots is None else int(dst_slots[i])
        page = packed_pool[d]
        base = page[:O.packed_page_bytes(g)]
        O.quantize_pages(hot_pool[s:s + 1], g, 1, gs, base[None])
        if rope.mode == ROPE_NVFP4:
            continue
        x = hot_pool[s, 0][..., -R:]  # [T, H, R] bf16 bits of K's RoPE part
        if rope.mode == ROPE_BF16:
            split_extension(page, g, rope)[...] = np.ascontiguousarray(x).view(np.uint8) \
                .reshape(g.page_size, g.num_kv_heads, R, 2)
            continue
        data, scales = O.split_packed_page(base, g)
        D = g.head_dim
        d1 = _values(data[0][..., (D - R) // 2:], scales[0][..., (D - R) // 16:], gs[0])
        xv = O.bf16_bits_to_f64(x)
        r = xv - d1  # exact (see module notes)
        r = np.where(r == 0, np.copysign(0.0, xv), r)
        d2, s2 = quantize_residual(r, gs[0])
        e_data, e_scales = split_extension(page, g, rope)
        e_data[...] = d2
        e_scales[...] = s2


def dequantize_pages(packed_pool, g: O.Geometry, rope: RopeLayout, num_pages: int, gs,
                     hot_pool, src_slots=None, dst_slots=None) -> None:
    """Base decoding (as O.dequantize_pages) with K's RoPE part taken from
    the extension region."""
    R, D = rope.rope_dims, g.head_dim
    for i in range(num_pages):
        s = i if src_slots is None else int(src_slots[i])
        d = i if dst_slots is None else int(dst_slots[i])
        page = packed_pool[s]
        base = page[:O.packed_page_bytes(g)]
        out = np.empty((1, *g.row_shape), np.uint16)
        O.dequantize_pages(base[None], g, 1, gs, out)
        if rope.mode == ROPE_BF16:
            out[0, 0, ..., D - R:] = split_extension(page, g, rope).copy().view(np.uint16) \
                .reshape(g.page_size, g.num_kv_heads, R)
        elif rope.mode == ROPE_2FP4:
            data, scales = O.split_packed_page(base, g)
            d1 = _values(data[0][..., (D - R) // 2:], scales[0][..., (D - R) // 16:], gs[0])
            e_data, e_scales = split_extension(page, g, rope)
            d2 = _values(e_data, e_scales, gs[0])
            flat = out[0, 0, ..., D - R:].reshape(-1)
            a, b = d1.reshape(-1), d2.reshape(-1)
            for j in range(flat.size):
                q = Fraction(float(a[j])) + Fraction(float(b[j]))
                neg0 = bool(np.signbit(a[j]) and np.signbit(b[j]))  # IEEE: -0 + -0 = -0
                flat[j] = fraction_to_bf16_rne(q, negative_zero=neg0)
            out[0, 0, ..., D - R:] = flat.reshape(g.page_size, g.num_kv_heads, R)
        hot_pool[d] = out[0]
