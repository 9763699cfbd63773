#!/usr/bin/env python3
"""Benchmark of the NVFP4 paged-KV hot path on one MI355X.

One step = the whole hot path over one batch of synthetic input resident in
HBM: encode the batch's bf16 K/V pages into the packed NVFP4 pool
(kvfp4_quantize_pages), run single-token decode attention over the packed
pool (kvfp4_paged_decode_attention, dequantizing in-kernel), and decode the
pages back to bf16 (kvfp4_dequantize_pages).  Headline workload: the
Llama-3-8B-shaped layer (batch 32, 32 q / 8 KV heads, head_dim 128, 8192
tokens, 64-token pages in a seeded permutation; 4096 pages); the other four
workloads are timed the same way and reported under ``workloads``.

Timing (steady state): each leg runs K calls back to back on the stream,
between one pair of HIP events, cycling over three copies of its buffers
(as a model step cycles over its layers' caches).  A set's bytes were last
touched two calls earlier, after more than the 256 MiB Infinity Cache of
other traffic, so they come from HBM; a call also pays for writing back what
the calls before it left dirty, as it does in a running server.  The
per-call time is the block's time over K; an untimed 1 GiB read before each
block writes back what the previous block left dirty.  Also reported, as
``isolated``:
single calls after an untimed 1 GiB read that evicts the caches, each
between its own events.  ``value`` is the step's algorithmic bytes over the
summed steady-state leg times.  Prints one JSON line.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
COPY_CALLS = 4          # 1 GiB device copies timed as the practical ceiling
COPY_BYTES = 1 << 30
PROFILES = os.path.join(ROOT, "profiles")
SETS = 3                # buffer copies each leg cycles over
ISOLATED_CALLS = 10
HEADLINE = "llama3_8b"
WORKLOADS = ["tiny", "llama3_8b", "qwen3_8b_long", "cold_pages", "mla"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default=HEADLINE, choices=WORKLOADS,
                   help="the workload whose step is the headline")
    p.add_argument("--only", action="store_true",
                   help="time only --workload (the other workloads are skipped)")
    p.add_argument("--gs", default="calibrated", choices=["calibrated", "unit"])
    p.add_argument("--no-isolated", action="store_true",
                   help="skip the single-call (cache-evicted) timings")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=20.0,
                   help="approximate host time budget of the oracle sample")
    p.add_argument("--no-copy-yardstick", action="store_true",
                   help="skip timing plain streams (the practical HBM ceilings)")
    p.add_argument("--extras-only", action="store_true",
                   help="time only the paths reported beside the step (no step, no JSON "
                        "metric line); for profiling those kernels on their own")
    p.add_argument("--no-append", action="store_true",
                   help="skip timing the paths reported beside the step (append-quantize, "
                        "gather-dequantize, host offload, RoPE layouts)")
    return p.parse_args()


def decode_bytes(wl) -> dict:
    """Algorithmic bytes of one decode call: the packed K/V rows of every
    cached token, Q, the output, the used page-table entries and lengths."""
    nt, T, H, D = wl.geometry
    L = wl.seq_lens.astype(np.int64)
    kv = int(L.sum()) * nt * H * D * 9 // 16
    q = wl.batch * wl.num_q_heads * D * 2
    out = wl.batch * wl.num_q_heads * wl.v_dim * 2 + wl.batch * wl.num_q_heads * 4
    bt = int(np.sum(-(-L // T))) * 4 + wl.batch * 4
    flops = 2 * int(L.sum()) * wl.num_q_heads * (D + wl.v_dim)
    return {"bytes": kv + q + out + bt, "kv_bytes": kv, "flops": flops}


def codec_bytes(geometry, pages: int) -> int:
    nt, T, H, D = geometry
    e = nt * T * H * D
    return pages * (2 * e + e * 9 // 16)


def append_bytes(geometry, tokens: int, elem_bytes: int) -> int:
    """Algorithmic bytes of appending (or gathering) `tokens` rows: the bf16
    or FP8 rows, their packed data and scale bytes, the two int32 slot/row
    entries."""
    nt, T, H, D = geometry
    per = nt * H * D
    return tokens * (per * elem_bytes + per * 9 // 16 + 8)


# Each streaming leg's traffic mix, for reading its bandwidth against a plain
# stream of the same mix: decode reads (the merge's few writes aside); the
# encoder reads 32 bytes of bf16 for every 9 it writes, the decoder the
# reverse.  The page-list sort (a few KiB) has none.
LEG_MIX = {"decode": "read", "quantize": "read4_write1", "dequantize": "read1_write4"}
YARDSTICK_KINDS = {"read": (0, 1.0), "write": (1, 1.0), "read4_write1": (2, 1.25),
                   "read1_write4": (3, 1.25)}


def stream_yardsticks(torch, src, dst, stream, calls=COPY_CALLS):
    """Plain streams of 1 GiB per traffic mix (libkvfp4_yardstick.so), timed
    like the legs: one untimed call, then `calls` back to back between one
    pair of events.  GB/s counts both directions (read 1 GiB + write 256 MiB
    for read4_write1)."""
    import ctypes
    lib_path = os.path.join(ROOT, "nvfp4_paged_decode_amd", "libkvfp4_yardstick.so")
    if not os.path.exists(lib_path):
        return None
    lib = ctypes.CDLL(lib_path)
    lib.kvfp4_yardstick.restype = ctypes.c_int
    lib.kvfp4_yardstick.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    sink = torch.empty(1024, dtype=torch.uint8, device=src.device)
    nbytes = src.numel()
    out = {}
    for name, (kind, factor) in YARDSTICK_KINDS.items():
        def call():
            rc = lib.kvfp4_yardstick(kind, src.data_ptr(), dst.data_ptr(), sink.data_ptr(), nbytes,
                                     ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError(f"kvfp4_yardstick({name}) failed: {rc}")
        ms = time_block(torch, stream, [call], calls, 1)
        moved = factor * nbytes
        out[name] = {"bytes": int(moved), "avg_us": round(ms * 1e3, 2),
                     "GB/s": round(moved / (ms * 1e-3) / 1e9, 1),
                     "frac_hbm_peak": round(moved / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    return out


#: Untimed warm-up lasts at least this long as well as at least W steps, so
#: that a timed block never starts from a GPU that idled through the seconds
#: of host-side input generation.
WARM_SECONDS = 0.25


def warm_up(torch, step, min_calls, seconds=WARM_SECONDS):
    """Run step() at least min_calls times and for at least `seconds` of
    wall time, synchronizing at the end."""
    t0 = time.perf_counter()
    i = 0
    while i < min_calls or time.perf_counter() - t0 < seconds:
        step(i)
        i += 1
        if i >= min_calls:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def time_block(torch, stream, calls, k, warmup):
    """Average ms of one call when `k` calls run back to back, cycling over
    `calls` (one per buffer set), between one pair of events on `stream`;
    before them at least `warmup` calls and WARM_SECONDS of them, untimed."""
    n = len(calls)
    warm_up(torch, lambda i: calls[i % n](), warmup)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(k):
        calls[i % n]()
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / k


def time_append(K, torch, wl, geometry, gs, hot, packed, stream, evict, steps, warmup):
    """The token-row paths, timed beside the step (not part of it).  Write
    path: a prefill of up to 256 of the workload's pages appended token by
    token (bf16 rows, and the same values as FP8 rows), and one decode step
    that rewrites the last cached token of every sequence.  Extend path: the
    same pages' rows gathered back into a bf16 and an FP8 workspace."""
    nt, T, H, D = geometry
    dev = hot.device
    used = torch.from_numpy(wl.used_slots[:256].astype(np.int64)).to(dev)
    n_pages = int(used.shape[0])
    pages = hot.view(wl.num_slots, nt, T, H, D)[used]
    rows = pages.permute(0, 2, 1, 3, 4).reshape(n_pages * T, nt, H, D).contiguous()
    tok_slots = used.to(torch.int32).repeat_interleave(T)
    tok_rows = torch.arange(T, dtype=torch.int32, device=dev).repeat(n_pages)
    amax = rows.view(torch.bfloat16).float().abs().max().clamp_min(1e-30)
    rows8 = (rows.view(torch.bfloat16).float() * (448.0 / amax)).to(torch.float8_e4m3fn)
    rows8 = rows8.view(torch.uint8).contiguous()
    L = wl.seq_lens.astype(np.int64)
    last = np.maximum(L - 1, 0)
    dslots = torch.from_numpy(wl.block_table[np.arange(wl.batch), last // T].astype(np.int32)).to(dev)
    drows = torch.from_numpy((last % T).astype(np.int32)).to(dev)
    drow_data = rows[:wl.batch].contiguous()
    g16 = torch.empty_like(rows)
    g8 = torch.empty_like(rows8)
    cases = [("append", "prefill_bf16", rows, tok_slots, tok_rows, 2),
             ("append", "prefill_fp8", rows8, tok_slots, tok_rows, 1),
             ("append", "decode_step_bf16", drow_data, dslots, drows, 2),
             ("gather", "prefix_bf16", g16, tok_slots, tok_rows, 2),
             ("gather", "prefix_fp8", g8, tok_slots, tok_rows, 1)]
    res = {"append": {}, "gather": {}}
    for kind, name, r, ts, tr, eb in cases:
        def fn():
            if kind == "append":
                K.kvfp4_append_quantize(geometry, r, ts, tr, packed, gs)
            else:
                K.kvfp4_gather_dequantize(geometry, packed, ts, tr, r, gs)
        for _ in range(warmup):
            fn()
        evs = []
        for _ in range(steps):
            evict()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        us = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3
        ntok = int(ts.shape[0])
        b = append_bytes(geometry, ntok, eb)
        res[kind][name] = {"tokens": ntok, "avg_us": round(us, 2), "bytes": b,
                           "GB/s": round(b / (us * 1e-6) / 1e9, 1)}
    return res


def time_offload(K, torch, wl, geometry, gs, hot, stream, steps, warmup, pages=256):
    """Cold-page offload and onboard with the packed pool in pinned host
    memory (timed beside the step): the encoder writes each packed page
    across the host link and the decoder reads it back.  The yardstick is a
    plain copy of the same packed bytes each way between device and pinned
    host memory."""
    dev = hot.device
    pages = min(pages, int(wl.used_slots.shape[0]))
    pb = K.kvfp4_packed_page_bytes(geometry)
    slots = torch.from_numpy(wl.used_slots[:pages].astype(np.int32)).to(dev)
    idx = torch.arange(pages, dtype=torch.int32, device=dev)
    host_pool = torch.empty((pages, pb), dtype=torch.uint8).pin_memory()
    dev_pool = torch.empty((pages, pb), dtype=torch.uint8, device=dev)
    back = torch.empty((pages,) + tuple(hot.shape[1:]), dtype=hot.dtype, device=dev)
    cases = {
        "offload_quantize_to_host": lambda: K.kvfp4_quantize_pages(
            geometry, hot, host_pool, pages, gs, slots, idx),
        "onboard_dequantize_from_host": lambda: K.kvfp4_dequantize_pages(
            geometry, host_pool, back, pages, gs, idx, idx),
        "copy_device_to_host": lambda: host_pool.copy_(dev_pool, non_blocking=True),
        "copy_host_to_device": lambda: dev_pool.copy_(host_pool, non_blocking=True),
    }
    res = {"pages": pages, "packed_bytes": pages * pb}
    for name, fn in cases.items():
        for _ in range(warmup):
            fn()
        evs = []
        for _ in range(steps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        us = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3
        res[name] = {"avg_us": round(us, 1),
                     "host_link_GB/s": round(pages * pb / (us * 1e-6) / 1e9, 2)}
    return res


def time_rope_layouts(K, torch, wl, geometry, gs, hot, stream, evict, steps, warmup, pages=1024):
    """Cold-page codec with K's last 64 dims (the MLA latent's RoPE part) in
    each storage variant, timed beside the step on up to 1024 pages: bytes
    are the hot page read or written plus the packed slot with its
    extension."""
    dev = hot.device
    pages = min(pages, int(wl.used_slots.shape[0]))
    slots = torch.from_numpy(wl.used_slots[:pages].astype(np.int32)).to(dev)
    idx = torch.arange(pages, dtype=torch.int32, device=dev)
    back = torch.empty((pages,) + tuple(hot.shape[1:]), dtype=hot.dtype, device=dev)
    hot_b = K.kvfp4_hot_page_bytes(geometry)
    res = {"pages": pages, "rope_dims": 64}
    for mode, name in ((1, "bf16"), (2, "2fp4")):
        rope = (64, mode)
        pb = K.kvfp4_packed_page_bytes_rope(geometry, rope)
        pool = torch.empty((pages, pb), dtype=torch.uint8, device=dev)
        legs = {"quantize": lambda: K.kvfp4_quantize_pages_rope(geometry, rope, hot, pool, pages,
                                                                 gs, slots, idx),
                "dequantize": lambda: K.kvfp4_dequantize_pages_rope(geometry, rope, pool, back,
                                                                     pages, gs, idx, idx)}
        out = {"slot_bytes": pb}
        for leg, fn in legs.items():
            for _ in range(warmup):
                fn()
            evs = []
            for _ in range(steps):
                evict()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                evs.append((e0, e1))
            torch.cuda.synchronize()
            us = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3
            out[leg] = {"avg_us": round(us, 1),
                        "GB/s": round(pages * (hot_b + pb) / (us * 1e-6) / 1e9, 1)}
        res[name] = out
    return res


def _oracle_encode(task):
    """Pool worker: encode a chunk of hot pages with the oracle."""
    from oracle import nvfp4 as O
    hot, geometry, gs = task
    g = O.Geometry(*geometry)
    out = np.zeros((hot.shape[0], O.packed_page_bytes(g)), np.uint8)
    O.quantize_pages(hot, g, hot.shape[0], gs, out)
    return out


def _oracle_decode(task):
    """Pool worker: decode a chunk of packed pages with the oracle."""
    from oracle import nvfp4 as O
    packed, geometry, gs = task
    g = O.Geometry(*geometry)
    back = np.zeros((packed.shape[0], *g.row_shape), np.uint16)
    O.dequantize_pages(packed, g, packed.shape[0], gs, back)
    return back.shape[0]


def _oracle_attend(task):
    """Pool worker: decode attention of one sequence (all query heads)."""
    from oracle import nvfp4 as O
    from oracle import attention as A
    packed, geometry, gs, q, L, scale, v_dim = task
    g = O.Geometry(*geometry)
    bt = np.arange(packed.shape[0], dtype=np.int32)[None, :]
    A.decode_attention(packed, g, gs, q, bt, np.array([L], np.int32), scale, v_dim,
                       batch_indices=[0])
    return L


def cgroup_cpu_quota() -> float | None:
    """CPUs' worth of time the process's cgroup may use (cpu.max), or None
    when it is unlimited or not readable."""
    try:
        quota, period = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        if quota != "max":
            return int(quota) / int(period)
    except (OSError, ValueError):
        pass
    return None


#: Processes the oracle may start on the benchmark's host: the CPU share one
#: GPU has on the MI355X hosts this runs on (their cores are shared between
#: the GPUs of the machine).
CPU_SHARE_PER_GPU = 16


def oracle_processes() -> tuple[int, dict]:
    """Worker count for the oracle: every core the process may run on, up to
    the cgroup's CPU quota and the one-GPU CPU share; and the host's own
    figures, reported beside it."""
    affinity = len(os.sched_getaffinity(0))
    quota = cgroup_cpu_quota()
    n = affinity
    if quota is not None:
        n = min(n, max(1, int(quota)))
    n = max(1, min(n, CPU_SHARE_PER_GPU))
    return n, {"host_logical_cpus": os.cpu_count(), "affinity_cpus": affinity,
               "cgroup_cpu_quota": quota, "cpu_share_per_gpu": CPU_SHARE_PER_GPU}


def cpu_baseline(wl, gs, budget_s: float, step_unit_bytes: dict, dec_bytes_per_token: float,
                 step_bytes: float) -> dict:
    """The oracle as it stands, on the host's cores, over a bounded sample of
    the same workload.  A pool of processes (one per core the process may
    use, within the cgroup quota and the one-GPU share, each with one BLAS
    thread) encodes chunks of 16 pages,
    decodes them back, and runs decode attention for whole sequences (all
    query heads); the sample sizes come from a short single-process timing
    so that the three legs take about a quarter, a quarter and a half of
    `budget_s` of wall time.  Each leg's rate is scaled to that leg's bytes
    in one step, and the figure is the step's algorithmic bytes over the
    summed time."""
    import multiprocessing as mp
    from threadpoolctl import threadpool_limits
    from oracle import nvfp4 as O
    g = O.Geometry(*wl.geometry)
    per_page = codec_bytes(wl.geometry, 1)
    chunk = 16
    cores, host = oracle_processes()
    used = wl.used_slots
    n_chunks = used.shape[0] // chunk
    seq_packed = {}

    def enc_task(i):
        return (wl.hot_pool[used[i * chunk:(i + 1) * chunk]], wl.geometry, gs)

    def seq_pages(b):
        need = -(-int(wl.seq_lens[b]) // wl.page_size)
        return (wl.hot_pool[wl.block_table[b, :need]], wl.geometry, gs)

    def att_task(b):
        if b not in seq_packed:
            seq_packed[b] = _oracle_encode(seq_pages(b))
        return (seq_packed[b], wl.geometry, gs, wl.q[b:b + 1], int(wl.seq_lens[b]),
                wl.softmax_scale, wl.v_dim)

    # single-process timing of one task of each kind sizes the samples
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        packed0 = _oracle_encode(enc_task(0))
        t_enc = time.perf_counter() - t0
        t0 = time.perf_counter()
        _oracle_decode((packed0, wl.geometry, gs))
        t_dec = time.perf_counter() - t0
        task0 = att_task(0)
        t0 = time.perf_counter()
        _oracle_attend(task0)
        t_att = time.perf_counter() - t0
    # tasks that keep every process busy for about the leg's share of the budget
    n_enc = int(max(1, min(n_chunks, cores * max(1, int(budget_s / 4 / t_enc)))))
    n_att = int(max(1, min(wl.batch, cores * max(1, int(budget_s / 2 / t_att)))))

    env = dict(os.environ)
    os.environ["OMP_NUM_THREADS"] = "1"  # the workers inherit one BLAS thread each
    try:
        ctx = mp.get_context("spawn")
        pool = ctx.Pool(cores)
        try:
            pool.map(_oracle_decode, [(packed0, wl.geometry, gs)] * cores)  # workers up
            t0 = time.perf_counter()
            packed = pool.map(_oracle_encode, [enc_task(i) for i in range(n_enc)])
            q_s = time.perf_counter() - t0
            t0 = time.perf_counter()
            pool.map(_oracle_decode, [(p, wl.geometry, gs) for p in packed])
            dq_s = time.perf_counter() - t0
            # the sampled sequences' pages, encoded first (untimed: that is
            # the encode leg's work)
            for b, pk in zip(range(1, n_att), pool.map(_oracle_encode,
                                                       [seq_pages(b) for b in range(1, n_att)])):
                seq_packed[b] = pk
            tasks = [att_task(b) for b in range(n_att)]
            t0 = time.perf_counter()
            tokens = sum(pool.map(_oracle_attend, tasks))
            dec_s = time.perf_counter() - t0
        finally:
            # the workers finish and exit on their own (no SIGTERM, which a
            # preloaded profiler's signal handler in the children can stall)
            pool.close()
            pool.join()
    finally:
        os.environ.clear()
        os.environ.update(env)
    n_q = n_enc * chunk
    t_step = (step_unit_bytes["quantize"] / (n_q * per_page)) * q_s + \
             (step_unit_bytes["dequantize"] / (n_q * per_page)) * dq_s + \
             (step_unit_bytes["decode"] / (tokens * dec_bytes_per_token)) * dec_s
    cpu = "unknown CPU"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(step_bytes / t_step / 1e9, 6), "unit": "GB/s", "cores": cores,
            "kind": "oracle", "processes": cores, **host,
            "sample": (f"oracle (NumPy fp64) in {cores} processes, one thread each, on {cpu}: "
                       f"encode {n_q} pages ({q_s:.1f} s), decode {n_q} pages ({dq_s:.1f} s), "
                       f"attention for {n_att} sequence(s) ({tokens} tokens, all "
                       f"{wl.num_q_heads} q heads, {dec_s:.1f} s) of wall time; each leg "
                       f"scaled to the step's bytes of that leg"),
            "seconds": round(q_s + dq_s + dec_s, 2)}


class Legs:
    """Device buffers and calls of one workload's three legs, over SETS
    copies of the hot pool, the packed pool and the decoded pool."""

    def __init__(self, K, torch, name, gs_kind):
        from nvfp4_paged_decode_amd import workloads as W
        t0 = time.perf_counter()
        self.name = name
        if name == "cold_pages":
            cw = W.cold_pages()
            self.wl = None
            self.geometry = cw.geometry
            self.gs = [float(v) for v in (cw.gs_calibrated if gs_kind == "calibrated"
                                          else cw.gs_unit)]
            host_pool = cw.hot_pool
            self.pages = cw.num_pages
            src, dst = cw.src_slots, cw.dst_slots
            self.num_slots = cw.num_pages
        else:
            wl = W.FULL[name]()
            self.wl = wl
            self.geometry = wl.geometry
            self.gs = [float(v) for v in (wl.gs_calibrated if gs_kind == "calibrated"
                                          else wl.gs_unit)]
            host_pool = wl.hot_pool
            self.pages = int(wl.used_slots.shape[0])
            src = dst = wl.used_slots.astype(np.int32)
            self.num_slots = wl.num_slots
        self.gen_s = time.perf_counter() - t0
        dev = torch.device("cuda")
        self.dev = dev
        hot0 = torch.from_numpy(host_pool.view(np.int16)).to(dev)
        self.hot = [hot0] + [hot0.clone() for _ in range(SETS - 1)]
        self.src = torch.from_numpy(np.ascontiguousarray(src, np.int32)).to(dev)
        self.dst = torch.from_numpy(np.ascontiguousarray(dst, np.int32)).to(dev)
        # The step's first leg sorts the page list by hot slot (the library's
        # kvfp4_sort_page_list); both codec legs take the sorted list, so
        # the workgroups running at once touch neighbouring slots.
        self.src_sorted = torch.empty_like(self.src)
        self.dst_sorted = torch.empty_like(self.dst)
        K.kvfp4_sort_page_list(self.src, self.src_sorted, self.dst, self.dst_sorted,
                               num_pages=self.pages)
        pb = K.kvfp4_packed_page_bytes(self.geometry)
        self.packed = [torch.zeros((self.num_slots, pb), dtype=torch.uint8, device=dev)
                       for _ in range(SETS)]
        self.back = [torch.empty_like(hot0) for _ in range(SETS)]
        self.K = K
        G, gs = self.geometry, self.gs
        sort = lambda: K.kvfp4_sort_page_list(self.src, self.src_sorted, self.dst,
                                              self.dst_sorted, num_pages=self.pages)
        self.calls = {
            "sort": [sort] * SETS,
            "quantize": [lambda r=r: K.kvfp4_quantize_pages(G, self.hot[r], self.packed[r],
                                                            self.pages, gs, self.src_sorted,
                                                            self.dst_sorted)
                         for r in range(SETS)],
            "dequantize": [lambda r=r: K.kvfp4_dequantize_pages(G, self.packed[r], self.back[r],
                                                                self.pages, gs, self.dst_sorted,
                                                                self.src_sorted)
                           for r in range(SETS)],
        }
        # the sort reads both lists and writes their sorted copies
        self.leg_bytes = {"sort": 16 * self.pages, "quantize": codec_bytes(G, self.pages),
                          "dequantize": codec_bytes(G, self.pages)}
        if self.wl is not None:
            wl = self.wl
            self.q = torch.from_numpy(wl.q.view(np.int16)).to(dev)
            self.bt = torch.from_numpy(wl.block_table).to(dev)
            self.sl = torch.from_numpy(wl.seq_lens).to(dev)
            self.hint = int(wl.seq_lens.max())
            ws_n = K.kvfp4_decode_workspace_bytes(G, wl.batch, wl.num_q_heads, wl.v_dim,
                                                  self.hint)
            self.ws = torch.empty(max(ws_n, 16), dtype=torch.uint8, device=dev)
            self.out = torch.empty((wl.batch, wl.num_q_heads, wl.v_dim), dtype=torch.int16,
                                   device=dev)
            self.lse = torch.empty((wl.batch, wl.num_q_heads), dtype=torch.float32, device=dev)
            self.calls["decode"] = [
                lambda r=r: K.kvfp4_paged_decode_attention(G, self.packed[r], gs, self.q,
                                                           self.bt, self.sl, self.hint,
                                                           wl.softmax_scale, self.out, self.lse,
                                                           self.ws, v_dim=wl.v_dim)
                for r in range(SETS)]
            self.db = decode_bytes(wl)
            self.leg_bytes["decode"] = self.db["bytes"]
        self.order = [k for k in ("sort", "quantize", "decode", "dequantize") if k in self.calls]

    def describe(self) -> str:
        if self.wl is None:
            return (f"cold_pages: {self.pages} pages x {self.geometry} (tensors, tokens, heads, "
                    f"dims); step = sort the page list by hot slot + encode + decode of every "
                    f"page")
        wl = self.wl
        nt, T, H, D = self.geometry
        return (f"{self.name}: batch {wl.batch}, {wl.num_q_heads} q / {H} KV heads, head_dim "
                f"{D}, v_dim {wl.v_dim}, context {int(wl.seq_lens.min())}-"
                f"{int(wl.seq_lens.max())} (sum {int(wl.seq_lens.sum())}), page {T}; step = "
                f"sort the page list by hot slot + encode {self.pages} pages + decode "
                f"attention + decode {self.pages} pages")

    def free(self):
        for k in list(vars(self)):
            if k not in ("name", "wl", "geometry", "gs", "pages", "leg_bytes", "db", "gen_s",
                         "order", "num_slots"):
                delattr(self, k)


def leg_report(legs, name, ms, iso=None, mixes=None, copy=None) -> dict:
    """Rates of one leg from its per-call time `ms` (and the isolated-call
    figures `iso`, a list of ms)."""
    b = legs.leg_bytes[name]
    gbs = b / (ms * 1e-3) / 1e9
    r = {"avg_us": round(ms * 1e3, 2), "bytes": b, "GB/s": round(gbs, 1),
         "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    if mixes and LEG_MIX.get(name) in mixes:
        r["frac_mix_yardstick"] = round(gbs / mixes[LEG_MIX[name]]["GB/s"], 4)
    if copy is not None:
        r["frac_copy_yardstick"] = round(gbs / copy["GB/s"], 4)
    if name == "decode":
        wl, t = legs.wl, ms * 1e-3
        r["tokens_per_s"] = round(wl.batch / t, 1)
        r["context_tokens_per_s"] = round(float(wl.seq_lens.sum()) / t, 1)
        r["TFLOP/s"] = round(legs.db["flops"] / t / 1e12, 2)
        r["frac_bf16_mfma_peak"] = round(legs.db["flops"] / t / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)
    if iso:
        r["isolated"] = {"avg_us": round(float(np.mean(iso)) * 1e3, 2),
                         "median_us": round(float(np.median(iso)) * 1e3, 2),
                         "min_us": round(float(np.min(iso)) * 1e3, 2),
                         "frac_hbm_peak": round(b / (float(np.mean(iso)) * 1e-3) / 1e9 /
                                                HBM_PEAK_GBS, 4)}
    from nvfp4_paged_decode_amd.profiling import read_traffic
    traffic = read_traffic(os.path.join(PROFILES, f"counters_{legs.name}.txt"), legs.name, name)
    if traffic is not None:
        r["counter_traffic_bytes"] = traffic
        r["traffic_over_algorithmic"] = round(traffic / b, 4)
    return r


def roofline_of(legs, kern: dict, leg: str) -> dict:
    """Roofline of one leg: MLA decode against the dense 16-bit MFMA peak (a
    dense contraction of about 820 flop per cache byte), the rest against
    HBM."""
    r = kern[leg]
    traffic = r.get("counter_traffic_bytes")
    if leg == "decode" and legs.name == "mla":
        return {"kernel": leg, "bound": "mfma", "achieved": r["TFLOP/s"],
                "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": r["frac_bf16_mfma_peak"], "traffic": traffic}
    return {"kernel": leg, "bound": "hbm", "achieved": r["GB/s"], "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": r["frac_hbm_peak"], "traffic": traffic}


def isolated_times(torch, stream, legs, evict, n) -> dict:
    """Single calls after an untimed cache eviction, each between its own
    events (the event marker before a call adds a few microseconds)."""
    out = {}
    for name in legs.order:
        evs = []
        for i in range(n):
            evict()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            legs.calls[name][i % SETS]()
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        out[name] = [a.elapsed_time(b) for a, b in evs]
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "sharding of this path is a design note, not a built component.", file=sys.stderr)
        sys.exit(2)

    import torch
    import nvfp4_paged_decode_amd as K

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    K.load_library()
    stream = torch.cuda.current_stream()
    dev = torch.device("cuda")
    # fp32 in and out, so that the sum is one read-only reduction
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
    flush_sink = torch.empty((), dtype=torch.float32, device=dev)

    def evict():
        # read 1 GiB (4x the 256 MiB Infinity Cache); a read leaves no dirty lines
        torch.sum(flush, dim=0, out=flush_sink)

    # the reduction's first launch loads its code object, which held up the
    # first timed block behind it (a decode block measured 74 instead of
    # 61 us per call); launch it once, untimed
    evict()
    torch.cuda.synchronize()

    name = args.workload
    if args.extras_only:
        legs = Legs(K, torch, name, args.gs)
        if legs.wl is None:
            print("--extras-only needs a decode workload", file=sys.stderr)
            sys.exit(2)
        legs.calls["quantize"][0]()  # the packed pool the gathers read
        torch.cuda.synchronize()
        print(json.dumps({"mode": "extras-only", "workload": name,
                          **run_extras(K, torch, legs, stream, evict, args)}), flush=True)
        return

    copy = mixes = None
    if not args.no_copy_yardstick:
        src_c = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst_c = torch.empty_like(src_c)
        ms_c = time_block(torch, stream, [lambda: dst_c.copy_(src_c)], COPY_CALLS, 1)
        copy = {"bytes": 2 * COPY_BYTES, "avg_us": round(ms_c * 1e3, 2),
                "GB/s": round(2 * COPY_BYTES / (ms_c * 1e-3) / 1e9, 1)}
        mixes = stream_yardsticks(torch, src_c, dst_c, stream)
        del src_c, dst_c

    # ---- the headline workload: K timed steps ---------------------------
    legs = Legs(K, torch, name, args.gs)

    # untimed warm-up: each leg in a block of its own, back to back and after
    # the cache flush, as the timed blocks run (interleaved with the codec
    # legs, a decode call instead pays for their write-back: in a kernel
    # trace the warm-up's calls then misstate the timed ones)
    for leg in legs.order:
        evict()
        warm_up(torch, lambda i, leg=leg: legs.calls[leg][i % SETS](), args.warmup,
                WARM_SECONDS / len(legs.order))
    t0 = time.perf_counter()
    evs = {}
    for leg in legs.order:
        # the previous block's dirty lines are written back during this
        # untimed read, not inside the next leg's first calls
        evict()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            legs.calls[leg][i % SETS]()
        e1.record(stream)
        evs[leg] = (e0, e1)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = {k: a.elapsed_time(b) / args.steps for k, (a, b) in evs.items()}
    iso = {} if args.no_isolated else isolated_times(torch, stream, legs, evict,
                                                     min(args.steps, ISOLATED_CALLS))
    kern = {k: leg_report(legs, k, ms[k], iso.get(k), mixes, copy) for k in legs.order}
    step_ms = float(sum(ms.values()))
    step_bytes = sum(legs.leg_bytes.values())
    value = step_bytes / (step_ms * 1e-3) / 1e9
    dom = max(ms, key=ms.get)
    roof = roofline_of(legs, kern, dom)

    extras = {}
    if legs.wl is not None and not args.no_append:
        extras = run_extras(K, torch, legs, stream, evict, args)
    cpu = None
    if legs.wl is not None and not args.no_cpu_baseline:
        try:
            cpu = cpu_baseline(legs.wl, legs.gs, args.cpu_seconds, legs.leg_bytes,
                               legs.db["bytes"] / float(legs.wl.seq_lens.sum()), step_bytes)
        except Exception as e:  # the GPU figure stands on its own
            cpu = {"error": repr(e)}
    wdesc = legs.describe()
    wl = legs.wl
    gen_s = legs.gen_s
    legs.free()
    del legs
    torch.cuda.empty_cache()

    # ---- the other workloads, timed the same way ------------------------
    others = {}
    if not args.only:
        for other in WORKLOADS:
            if other == name:
                continue
            lo = Legs(K, torch, other, args.gs)
            ms_o = {}
            for leg in lo.order:
                evict()
                ms_o[leg] = time_block(torch, stream, lo.calls[leg], args.steps, args.warmup)
            iso_o = {} if args.no_isolated else isolated_times(torch, stream, lo, evict,
                                                               min(args.steps, ISOLATED_CALLS))
            k_o = {k: leg_report(lo, k, ms_o[k], iso_o.get(k), mixes, copy) for k in lo.order}
            d = {"workload": lo.describe(), "legs": k_o,
                 "step_GB/s": round(sum(lo.leg_bytes.values()) /
                                    (sum(ms_o.values()) * 1e-3) / 1e9, 1)}
            if "decode" in k_o:
                d["roofline_decode"] = roofline_of(lo, k_o, "decode")
            d["roofline_quantize"] = roofline_of(lo, k_o, "quantize")
            d["roofline_dequantize"] = roofline_of(lo, k_o, "dequantize")
            others[other] = d
            gen_s += lo.gen_s
            lo.free()
            del lo
            torch.cuda.empty_cache()

    def summary(leg):
        r = kern.get(leg)
        if r is None:
            return None
        return {"avg_us": r["avg_us"], "GB/s": r["GB/s"], "frac_hbm_peak": r["frac_hbm_peak"]}

    line = {
        "metric": "NVFP4-KV decode attn effective HBM GB/s (% peak) + page quant/dequant GB/s",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16<->nvfp4 codec (integer thresholds); attention fp16 MFMA, fp32 accumulate",
        "data": "synthetic (seeded)",
        "config": {"workload": wdesc, "global_scale": args.gs,
                   "value": "the step's algorithmic bytes (encode + decode attention + decode "
                            "of the batch) over the summed steady-state leg times; per-leg "
                            "rates below",
                   "timing": f"steady state: {args.steps} calls per leg back to back over "
                             f"{SETS} buffer copies, one event pair per leg",
                   "global_batch": wl.batch if wl is not None else None,
                   "seq_len": int(wl.seq_lens.max()) if wl is not None else None,
                   "parallelism": "single GPU"},
        "decode_attention": summary("decode"),
        "page_quantize": summary("quantize"),
        "page_dequantize": summary("dequantize"),
        "kernels": kern,
        "roofline": roof,
        "cpu_baseline": cpu,
        "workloads": others,
        "copy_yardstick": copy,
        "stream_yardsticks": mixes,
        **extras,
        "wall_s_timed_region": round(wall, 3),
        "gen_s": round(gen_s, 1),
    }
    print(json.dumps(line), flush=True)


def time_slot_order(K, torch, legs, stream, evict, steps, warmup) -> dict:
    """The step's codec legs (same pages, same pools, steady state) with the
    page list sorted by hot slot, as the step runs them, and with the list
    as given -- the pool's slots in a random order, as a cache's pages would
    lie.  The kernels take pages in list order; the results are the same
    either way, the bandwidth is not."""
    G, gs, n = legs.geometry, legs.gs, legs.pages
    lists = {"as_given": (legs.src, legs.dst), "sorted": (legs.src_sorted, legs.dst_sorted)}
    legs_fn = {
        "quantize": lambda r, s, d: K.kvfp4_quantize_pages(G, legs.hot[r], legs.packed[r], n, gs,
                                                           s, d),
        "dequantize": lambda r, s, d: K.kvfp4_dequantize_pages(G, legs.packed[r], legs.back[r], n,
                                                               gs, d, s),
    }
    out = {}
    for leg, fn in legs_fn.items():
        res = {}
        for tag, (s, d) in lists.items():
            calls = [lambda r=r, s=s, d=d: fn(r, s, d) for r in range(SETS)]
            evict()
            ms = time_block(torch, stream, calls, steps, warmup)
            gbs = legs.leg_bytes[leg] / (ms * 1e6)
            res[tag] = {"avg_us": round(ms * 1e3, 2), "GB/s": round(gbs, 1),
                        "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
        out[leg] = res
    return out


def run_extras(K, torch, legs, stream, evict, args) -> dict:
    """The "next" paths, timed beside the step (never part of it)."""
    wl, G, gs = legs.wl, legs.geometry, legs.gs
    return {
        "codec_slot_order": time_slot_order(K, torch, legs, stream, evict, args.steps,
                                            args.warmup),
        "token_rows": time_append(K, torch, wl, G, gs, legs.hot[0], legs.packed[0], stream,
                                  evict, args.steps, args.warmup),
        "host_offload": time_offload(K, torch, wl, G, gs, legs.hot[0], stream,
                                     min(args.steps, 10), min(args.warmup, 2)),
        "rope_layouts": time_rope_layouts(K, torch, wl, G, gs, legs.hot[0], stream, evict,
                                          min(args.steps, 10), min(args.warmup, 2)),
    }


if __name__ == "__main__":
    main()
