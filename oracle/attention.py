"""Single-token decode attention over a paged NVFP4 K/V cache -- plain fp64
CPU oracle (TEST INFRASTRUCTURE ONLY).

What is computed ("Accelerating Long-Context and Agentic Inference with NVFP4
KV Cache", Path 3: Decode; NVFP4 KV Decode Attention Kernel Implementation /
Figure 3): bf16 queries attend to K/V read from the NVFP4 cache and
dequantized with their E4M3 block scales; the per-tensor K and V scales enter
as scalar multipliers of the two products.  This oracle uses the exact
dequantized values (``e2m1 * e4m3 * gs`` in fp64), so it is the plain
definition

    s_j = sigma * sum_d q[d] * k_j[d],   o = sum_j softmax(s)_j * v_j,
    lse = log(sum_j exp(s_j))

for every (sequence, query head), with query head h reading KV head
``h // (num_q_heads // num_kv_heads)``.

Readings of what the pages leave open: the query attends to exactly ``seq_lens[b]``
cached tokens, found through ``block_table[b][j // page_size]`` at row
``j % page_size``; with one KV tensor (MLA) the latent row is the key and its
first ``v_dim`` elements are the value; ``seq_lens[b] == 0`` gives ``o = 0``
and ``lse = -inf``.
"""

from __future__ import annotations

import numpy as np

from .nvfp4 import Geometry, bf16_bits_to_f64, exact_values, split_packed_page


def gather_rows(packed_pool: np.ndarray, g: Geometry, gs, block_table_row,
                seq_len: int, tensor: int) -> np.ndarray:
    """Exact fp64 rows ``[seq_len, H, D]`` of one K/V tensor of one sequence."""
    T = g.page_size
    rows = np.empty((seq_len, g.num_kv_heads, g.head_dim), dtype=np.float64)
    for j0 in range(0, seq_len, T):
        slot = int(block_table_row[j0 // T])
        data, scales = split_packed_page(packed_pool[slot], g)
        n = min(T, seq_len - j0)
        d = data[tensor, :n]
        nib = np.empty((n, g.num_kv_heads, g.head_dim), dtype=np.int64)
        nib[..., 0::2] = d & 0xF
        nib[..., 1::2] = d >> 4
        rows[j0:j0 + n] = exact_values(nib, scales[tensor, :n], float(gs[tensor]))
    return rows


def decode_attention(packed_pool: np.ndarray, g: Geometry, gs, q_bits: np.ndarray,
                     block_table: np.ndarray, seq_lens: np.ndarray,
                     softmax_scale: float, v_dim: int, batch_indices=None,
                     head_indices=None):
    """Decode attention for the selected sequences and query heads.

    ``q_bits``: uint16 bf16 bits ``[B, Hq, D]``.  Returns ``(out, lse)`` as
    fp64 arrays ``[len(batch), len(heads), v_dim]`` and
    ``[len(batch), len(heads)]`` (all sequences / heads when None).
    """
    B, Hq, D = q_bits.shape
    H = g.num_kv_heads
    assert D == g.head_dim and Hq % H == 0
    group = Hq // H
    bsel = range(B) if batch_indices is None else batch_indices
    hsel = range(Hq) if head_indices is None else head_indices
    bsel, hsel = list(bsel), list(hsel)
    out = np.zeros((len(bsel), len(hsel), v_dim), dtype=np.float64)
    lse = np.full((len(bsel), len(hsel)), -np.inf, dtype=np.float64)
    for bi, b in enumerate(bsel):
        L = int(seq_lens[b])
        if L == 0:
            continue
        K = gather_rows(packed_pool, g, gs, block_table[b], L, 0)
        if g.num_kv_tensors == 2:
            V = gather_rows(packed_pool, g, gs, block_table[b], L, 1)
        else:
            V = K
        q = bf16_bits_to_f64(q_bits[b])  # [Hq, D]
        for hi, h in enumerate(hsel):
            kv = h // group
            s = softmax_scale * (K[:, kv, :] @ q[h])  # [L]
            m = np.max(s)
            w = np.exp(s - m)
            denom = np.sum(w)
            out[bi, hi] = (w @ V[:, kv, :v_dim]) / denom
            lse[bi, hi] = m + np.log(denom)
    return out, lse


def merge_partials(outs, lses):
    """Combine attention results over disjoint token sets into the result
    over their union (the log-sum-exp merge)."""
    lses = np.asarray(lses, dtype=np.float64)
    m = np.max(lses)
    if m == -np.inf:
        return np.zeros_like(np.asarray(outs[0], dtype=np.float64)), -np.inf
    w = np.exp(lses - m)
    o = sum(wi * np.asarray(oi, dtype=np.float64) for wi, oi in zip(w, outs)) / np.sum(w)
    return o, m + np.log(np.sum(w))
