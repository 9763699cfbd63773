"""The oracle at full size, in a pool of worker processes (test
infrastructure).

The oracle's page encoding is independent per page and its decode attention
independent per sequence, so full-size references are computed in parallel:
pages in chunks, sequences one task each (longest first).  Workers are
started fresh (spawn) and import only numpy and the oracle, never a GPU
runtime; inputs go to them by value.  The worker count follows the CPUs this
process may use (affinity and cgroup quota), at most 16.
"""

from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np

MAX_WORKERS = 16


def cpu_share() -> int:
    """CPUs this process may use: affinity, then the cgroup v2 quota."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            quota, period = f.read().split()
        if quota != "max":
            n = min(n, max(1, int(quota) // int(period)))
    except (OSError, ValueError):
        pass
    return max(1, n)


def workers() -> int:
    return min(MAX_WORKERS, cpu_share())


def make_pool(n: int | None = None):
    return mp.get_context("spawn").Pool(n or workers())


# --- worker functions (module level, so spawned workers can import them) ---

def _encode_chunk(args):
    hot, geometry, gs = args
    from oracle import nvfp4 as O
    g = O.Geometry(*geometry)
    out = np.zeros((hot.shape[0], O.packed_page_bytes(g)), np.uint8)
    O.quantize_pages(hot, g, hot.shape[0], gs, out)
    return out


def _decode_chunk(args):
    packed, geometry, gs = args
    from oracle import nvfp4 as O
    g = O.Geometry(*geometry)
    out = np.zeros((packed.shape[0], *g.row_shape), np.uint16)
    O.dequantize_pages(packed, g, packed.shape[0], gs, out)
    return out


def _attention_one(args):
    b, pages, geometry, gs, q_row, seq_len, softmax_scale, v_dim = args
    from oracle import nvfp4 as O
    from oracle import attention as A
    g = O.Geometry(*geometry)
    table = np.arange(pages.shape[0], dtype=np.int32)[None, :]
    out, lse = A.decode_attention(pages, g, gs, q_row[None], table,
                                  np.asarray([seq_len], np.int32), softmax_scale, v_dim)
    return b, out[0], lse[0]


def _chunks(n: int, parts: int):
    bounds = np.linspace(0, n, min(n, parts) + 1).astype(int) if n else np.zeros(1, int)
    return [(int(a), int(c)) for a, c in zip(bounds[:-1], bounds[1:]) if c > a]


def encode_pages(pool, hot_pool: np.ndarray, geometry, gs, slots) -> np.ndarray:
    """Oracle-encoded packed pages of hot_pool[slots], in slot order."""
    slots = np.asarray(slots)
    gs = [float(v) for v in gs]
    parts = _chunks(len(slots), 8 * getattr(pool, "_processes", workers()))
    res = pool.map(_encode_chunk, [(hot_pool[slots[a:c]], tuple(geometry), gs) for a, c in parts])
    return np.concatenate(res) if res else np.zeros((0, 0), np.uint8)


def decode_pages(pool, packed: np.ndarray, geometry, gs) -> np.ndarray:
    """Oracle-decoded bf16 pages of every row of packed."""
    gs = [float(v) for v in gs]
    parts = _chunks(packed.shape[0], 8 * getattr(pool, "_processes", workers()))
    res = pool.map(_decode_chunk, [(packed[a:c], tuple(geometry), gs) for a, c in parts])
    return np.concatenate(res)


def decode_attention_all(pool, packed_pool: np.ndarray, wl, gs):
    """Oracle decode attention of every sequence and query head of a decode
    workload: (out [B, Hq, v_dim], lse [B, Hq]) in fp64."""
    B, Hq = wl.batch, wl.num_q_heads
    T = wl.page_size
    gs = [float(v) for v in gs]
    out = np.zeros((B, Hq, wl.v_dim), np.float64)
    lse = np.full((B, Hq), -np.inf, np.float64)
    order = sorted(range(B), key=lambda b: -int(wl.seq_lens[b]))
    tasks = []
    for b in order:
        L = int(wl.seq_lens[b])
        if L == 0:
            continue
        pages = packed_pool[wl.block_table[b, :-(-L // T)]]
        tasks.append((b, pages, tuple(wl.geometry), gs, wl.q[b], L, wl.softmax_scale,
                      wl.v_dim))
    for b, o, l in pool.imap_unordered(_attention_one, tasks):
        out[b], lse[b] = o, l
    return out, lse
