"""Seeded synthetic inputs for the five workloads (tests, bench, smoke).

This module only draws inputs: bf16 pages, page tables, sequence lengths,
queries and the caller's tensor scales.  It holds none of the codec's or the
attention's arithmetic, and it is the only code the HIP path and the CPU
oracle share.

Draw order for a decode workload (one ``numpy.random.default_rng(seed)``):
page permutation, sequence lengths, K, V, outlier / scale draws, Q.  Normals
are drawn in fp32, scaled in fp32, then rounded once to bf16 (nearest, ties
to even) by :func:`f32_to_bf16_bits`.

Workloads (sizes as the page geometry ``[tensors, tokens, heads, dim]``):

* ``tiny``        -- 1 sequence, 1 KV head, 4 query heads, head_dim 128,
  256 tokens, 16-token pages; N(0, 1) everywhere.
* ``llama3_8b``   -- batch 32, 32 q / 8 KV heads, head_dim 128, 8192 tokens,
  64-token pages in a seeded permutation; per tensor, 1 % of the (head, dim)
  channels (10 of 1024) are x20 outliers on every token.
* ``qwen3_8b_long`` -- batch 8, 32 q / 8 KV heads, head_dim 128, lengths
  uniform in [4096, 65536], 64-token pages; every (tensor, KV head) is scaled
  by 10**U(-1, 1), shared across sequences.
* ``cold_pages``  -- 4096 pages of {K, V} x 64 tokens x 8 heads x 128 dims,
  N(0, 1) with each value x50 with probability 0.001.
* ``mla``         -- batch 64, 128 query heads over one 576-dim latent (512 +
  64 rope) per token, values = first 512 dims, 16384 tokens, 64-token pages.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 bit patterns (nearest, ties to even)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class DecodeWorkload:
    name: str
    num_kv_tensors: int
    page_size: int
    num_kv_heads: int
    head_dim: int
    batch: int
    num_q_heads: int
    v_dim: int
    softmax_scale: float
    hot_pool: np.ndarray      # uint16 [slots, n_t, T, H, D]
    block_table: np.ndarray   # int32 [B, max_pages_per_seq]
    seq_lens: np.ndarray      # int32 [B]
    q: np.ndarray             # uint16 [B, Hq, D]
    gs_unit: np.ndarray       # float32 [n_t]
    gs_calibrated: np.ndarray  # float32 [n_t]
    used_slots: np.ndarray    # int32, the pool slots some sequence reads
    poison_slot: int          # a spare slot; unused block-table entries point here
    meta: dict = field(default_factory=dict)

    @property
    def geometry(self):
        return (self.num_kv_tensors, self.page_size, self.num_kv_heads, self.head_dim)

    @property
    def num_slots(self) -> int:
        return self.hot_pool.shape[0]

    @property
    def max_pages_per_seq(self) -> int:
        return self.block_table.shape[1]


@dataclass
class CodecWorkload:
    name: str
    num_kv_tensors: int
    page_size: int
    num_kv_heads: int
    head_dim: int
    hot_pool: np.ndarray      # uint16 [pages, n_t, T, H, D]
    src_slots: np.ndarray     # int32 [pages] (a permutation)
    dst_slots: np.ndarray     # int32 [pages] (a permutation)
    gs_unit: np.ndarray
    gs_calibrated: np.ndarray

    @property
    def geometry(self):
        return (self.num_kv_tensors, self.page_size, self.num_kv_heads, self.head_dim)

    @property
    def num_pages(self) -> int:
        return self.hot_pool.shape[0]


def calibrated_scales(hot_pool: np.ndarray, slots=None) -> np.ndarray:
    """The caller's per-tensor scale fp32(amax / (6 * 448)): the tensor's
    largest magnitude lands on the largest E2M1 value times the largest E4M3
    value.  Only the slots in ``slots`` count (all when None)."""
    pool = hot_pool if slots is None else hot_pool[slots]
    nt = pool.shape[1]
    out = np.empty(nt, dtype=np.float32)
    for t in range(nt):
        amax = float(np.max(np.abs(bf16_bits_to_f32(pool[:, t]))))
        out[t] = np.float32(amax / (6.0 * 448.0)) if amax > 0 else np.float32(1.0)
    return out


def _normal_bf16(rng, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def _decode_workload(name, seed, *, nt, T, H, D, B, Hq, v_dim, lens_fn, kv_fn,
                     softmax_scale) -> DecodeWorkload:
    rng = np.random.default_rng(seed)
    # sizes are needed before the first draw: sequence lengths come second,
    # so the permutation is drawn over an upper bound of the slot count.
    lens_hint = lens_fn(None)
    max_pages = -(-lens_hint // T)
    pages_bound = B * max_pages
    spare = max(2, pages_bound // 64)
    num_slots = pages_bound + spare
    perm = rng.permutation(num_slots).astype(np.int32)
    seq_lens = np.asarray(lens_fn(rng), dtype=np.int32).reshape(B)
    need = -(-seq_lens // T)
    poison_slot = int(perm[-1])
    block_table = np.full((B, max_pages), poison_slot, dtype=np.int32)
    cursor = 0
    for b in range(B):
        block_table[b, :need[b]] = perm[cursor:cursor + need[b]]
        cursor += int(need[b])
    used = perm[:cursor].copy()
    hot = kv_fn(rng, num_slots)  # uint16 [slots, nt, T, H, D]
    q = _normal_bf16(rng, (B, Hq, D))
    gs_cal = calibrated_scales(hot, used)
    return DecodeWorkload(name, nt, T, H, D, B, Hq, v_dim, softmax_scale, hot,
                          block_table, seq_lens, q, np.ones(nt, np.float32), gs_cal,
                          used, poison_slot)


def geometry_case(seed: int, *, nt: int, T: int, H: int, D: int, Hq: int, v_dim: int,
                  lens) -> DecodeWorkload:
    """A small decode workload of any page geometry: N(0, 1) K/V (or latent)
    and queries, the given sequence lengths, pages in a seeded permutation.
    For covering every kernel a shape can be routed to."""
    lens = np.asarray(lens, dtype=np.int64)

    def lens_fn(rng):
        return int(lens.max()) if rng is None else lens

    def kv(rng, slots):
        return _normal_bf16(rng, (slots, nt, T, H, D))

    return _decode_workload(f"geom_nt{nt}_T{T}_H{H}_D{D}_Hq{Hq}", seed, nt=nt, T=T, H=H, D=D,
                            B=len(lens), Hq=Hq, v_dim=v_dim, lens_fn=lens_fn, kv_fn=kv,
                            softmax_scale=1.0 / np.sqrt(float(D)))


def tiny(seed: int = 1) -> DecodeWorkload:
    """1 sequence, 1 KV head, 4 query heads, head_dim 128, 256 tokens, page 16."""
    def lens(rng):
        return 256

    def kv(rng, slots):
        k = _normal_bf16(rng, (slots, 1, 16, 1, 128))
        v = _normal_bf16(rng, (slots, 1, 16, 1, 128))
        return np.concatenate([k, v], axis=1)

    return _decode_workload("tiny", seed, nt=2, T=16, H=1, D=128, B=1, Hq=4, v_dim=128,
                            lens_fn=lens, kv_fn=kv, softmax_scale=1.0 / np.sqrt(128.0))


def llama3_8b(seed: int = 2, batch: int = 32, context: int = 8192) -> DecodeWorkload:
    """Llama-3-8B-shaped layer decode (32 q / 8 KV heads, head_dim 128)."""
    H, D = 8, 128

    def lens(rng):
        return context if rng is None else np.full(batch, context)

    def kv(rng, slots):
        parts = []
        for _t in range(2):
            parts.append(rng.standard_normal((slots, 1, 64, H, D), dtype=np.float32))
        n_out = int(round(0.01 * H * D))
        for t in range(2):
            ch = rng.choice(H * D, size=n_out, replace=False)
            x = parts[t].reshape(slots, 64, H * D)
            x[:, :, ch] *= np.float32(20.0)
        return f32_to_bf16_bits(np.concatenate(parts, axis=1))

    return _decode_workload(f"llama3_8b_b{batch}_l{context}", seed, nt=2, T=64, H=H, D=D,
                            B=batch, Hq=32, v_dim=D, lens_fn=lens, kv_fn=kv,
                            softmax_scale=1.0 / np.sqrt(128.0))


def qwen3_8b_long(seed: int = 3, batch: int = 8, lo: int = 4096, hi: int = 65536) -> DecodeWorkload:
    """Qwen3-8B-shaped long-context decode, lengths uniform in [lo, hi]."""
    H, D = 8, 128

    def lens(rng):
        return hi if rng is None else rng.integers(lo, hi, size=batch, endpoint=True)

    def kv(rng, slots):
        parts = [rng.standard_normal((slots, 1, 64, H, D), dtype=np.float32) for _ in range(2)]
        scale = (10.0 ** rng.uniform(-1.0, 1.0, size=(2, H))).astype(np.float32)
        for t in range(2):
            parts[t] *= scale[t][None, None, None, :, None]
        return f32_to_bf16_bits(np.concatenate(parts, axis=1))

    return _decode_workload(f"qwen3_8b_long_b{batch}", seed, nt=2, T=64, H=H, D=D, B=batch,
                            Hq=32, v_dim=D, lens_fn=lens, kv_fn=kv,
                            softmax_scale=1.0 / np.sqrt(128.0))


def mla(seed: int = 5, batch: int = 64, context: int = 16384, num_q_heads: int = 128) -> DecodeWorkload:
    """MLA-style decode: one 576-dim latent (512 + 64 rope), values = first 512."""
    def lens(rng):
        return context if rng is None else np.full(batch, context)

    def kv(rng, slots):
        return _normal_bf16(rng, (slots, 1, 64, 1, 576))

    return _decode_workload(f"mla_b{batch}_l{context}", seed, nt=1, T=64, H=1, D=576, B=batch,
                            Hq=num_q_heads, v_dim=512, lens_fn=lens, kv_fn=kv,
                            softmax_scale=1.0 / np.sqrt(576.0))


def cold_pages(seed: int = 4, pages: int = 4096) -> CodecWorkload:
    """Cold-page round trip: pages of {K, V} x 64 tokens x 8 heads x 128 dims."""
    rng = np.random.default_rng(seed)
    src = rng.permutation(pages).astype(np.int32)
    dst = rng.permutation(pages).astype(np.int32)
    x = rng.standard_normal((pages, 2, 64, 8, 128), dtype=np.float32)
    hit = rng.random(x.shape, dtype=np.float32) < np.float32(0.001)
    x[hit] *= np.float32(50.0)
    hot = f32_to_bf16_bits(x)
    return CodecWorkload("cold_pages", 2, 64, 8, 128, hot, src, dst,
                         np.ones(2, np.float32), calibrated_scales(hot))


#: The five workloads at full size, in order.
FULL = {
    "tiny": tiny,
    "llama3_8b": llama3_8b,
    "qwen3_8b_long": qwen3_8b_long,
    "cold_pages": cold_pages,
    "mla": mla,
}
