#!/usr/bin/env python3
"""Benchmark of the NVFP4 paged-KV hot path on one MI355X.

One step = the whole hot path over one batch of synthetic input resident in
HBM: encode the batch's bf16 K/V pages into the packed NVFP4 pool
(kvfp4_quantize_pages), run single-token decode attention over the packed
pool (kvfp4_paged_decode_attention, dequantizing in-kernel), and decode the
pages back to bf16 (kvfp4_dequantize_pages).  Default workload: the
Llama-3-8B-shaped layer (batch 32, 32 q / 8 KV heads, head_dim 128, 8192
tokens, 64-token pages in a seeded permutation; 4096 pages).

Timing: HIP events on the stream the kernels run on, around each kernel;
between kernels an untimed 1 GiB read evicts the 256 MiB Infinity Cache so
that bytes come from HBM (a read, so that no dirty lines are left to be
written back inside the next timed kernel).  `value` is the step's algorithmic bytes divided
by its kernel time.  Prints one JSON line.
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


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="llama3_8b",
                   choices=["tiny", "llama3_8b", "qwen3_8b_long", "mla", "cold_pages"])
    p.add_argument("--gs", default="calibrated", choices=["calibrated", "unit"])
    p.add_argument("--no-flush", action="store_true", help="do not evict caches between kernels")
    p.add_argument("--flush-mode", default="read", choices=["read", "write"],
                   help="evict caches by reading (default; leaves no dirty lines to be "
                        "written back inside the next timed kernel) or writing 1 GiB")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=20.0,
                   help="approximate host time budget of the oracle sample")
    p.add_argument("--no-copy-yardstick", action="store_true",
                   help="skip timing a plain 1 GiB device copy (the practical HBM ceiling)")
    p.add_argument("--extras-only", action="store_true",
                   help="time only the paths reported beside the step (no step, no JSON "
                        "metric line); for profiling those kernels on their own")
    p.add_argument("--no-append", action="store_true",
                   help="skip timing the token-row paths (append-quantize, gather-dequantize), "
                        "reported beside the step")
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


# Each leg's traffic mix, for reading its bandwidth against a plain stream of
# the same mix: decode reads (the merge's few writes aside); the encoder reads
# 32 bytes of bf16 for every 9 it writes, the decoder the reverse.
LEG_MIX = {"decode": "read", "quantize": "read4_write1", "dequantize": "read1_write4"}
YARDSTICK_KINDS = {"read": (0, 1.0), "write": (1, 1.0), "read4_write1": (2, 1.25),
                   "read1_write4": (3, 1.25)}


def stream_yardsticks(torch, src, dst, stream, evict, calls=COPY_CALLS):
    """Plain streams of 1 GiB per traffic mix (libkvfp4_yardstick.so), timed
    like the legs: cache eviction before each call, median after the first.
    GB/s counts both directions (read 1 GiB + write 256 MiB for read4_write1)."""
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
        times = []
        for _ in range(calls):
            evict()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            rc = lib.kvfp4_yardstick(kind, src.data_ptr(), dst.data_ptr(), sink.data_ptr(), nbytes,
                                     ctypes.c_void_p(stream.cuda_stream))
            e1.record(stream)
            if rc != 0:
                raise RuntimeError(f"kvfp4_yardstick({name}) failed: {rc}")
            times.append((e0, e1))
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in times[1:]]))
        moved = factor * nbytes
        out[name] = {"bytes": int(moved), "median_us": round(ms * 1e3, 2),
                     "GB/s": round(moved / (ms * 1e-3) / 1e9, 1),
                     "frac_hbm_peak": round(moved / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    return out


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


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "sharding of this path is a design note, not a built component.", file=sys.stderr)
        sys.exit(2)

    import torch
    import nvfp4_paged_decode_amd as K
    from nvfp4_paged_decode_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    K.load_library()

    t_gen = time.perf_counter()
    name = args.workload
    if name == "cold_pages":
        cw = W.cold_pages()
        wl = None
    else:
        wl = W.FULL[name]()
    t_gen = time.perf_counter() - t_gen

    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()

    if wl is not None:
        geometry = wl.geometry
        gs = [float(v) for v in (wl.gs_calibrated if args.gs == "calibrated" else wl.gs_unit)]
        hot = torch.from_numpy(wl.hot_pool.view(np.int16)).to(dev)
        pages = int(wl.used_slots.shape[0])
        slots = torch.from_numpy(wl.used_slots.astype(np.int32)).to(dev)
        num_slots = wl.num_slots
    else:
        geometry = cw.geometry
        gs = [float(v) for v in (cw.gs_calibrated if args.gs == "calibrated" else cw.gs_unit)]
        hot = torch.from_numpy(cw.hot_pool.view(np.int16)).to(dev)
        pages = cw.num_pages
        slots = torch.from_numpy(cw.src_slots).to(dev)
        num_slots = cw.num_pages
    pbytes = K.kvfp4_packed_page_bytes(geometry)
    packed = torch.zeros((num_slots, pbytes), dtype=torch.uint8, device=dev)
    hot_back = torch.empty_like(hot)
    # fp32 in and out, so that the sum is one read-only reduction (an int32
    # sum would first widen the whole buffer to int64 in a 2 GiB write)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
    flush_sink = torch.empty((), dtype=torch.float32, device=dev)

    def evict():
        # touch 1 GiB (4x the 256 MiB Infinity Cache) between timed kernels
        if args.flush_mode == "read":
            torch.sum(flush, dim=0, out=flush_sink)
        else:
            flush.fill_(1)

    if wl is not None:
        q = torch.from_numpy(wl.q.view(np.int16)).to(dev)
        bt = torch.from_numpy(wl.block_table).to(dev)
        sl = torch.from_numpy(wl.seq_lens).to(dev)
        hint = int(wl.seq_lens.max())
        ws_n = K.kvfp4_decode_workspace_bytes(geometry, wl.batch, wl.num_q_heads, wl.v_dim, hint)
        ws = torch.empty(max(ws_n, 4), dtype=torch.uint8, device=dev)
        out = torch.empty((wl.batch, wl.num_q_heads, wl.v_dim), dtype=torch.int16, device=dev)
        lse = torch.empty((wl.batch, wl.num_q_heads), dtype=torch.float32, device=dev)

    def k_quant():
        K.kvfp4_quantize_pages(geometry, hot, packed, pages, gs, slots, slots)

    def k_decode():
        K.kvfp4_paged_decode_attention(geometry, packed, gs, q, bt, sl, hint, wl.softmax_scale,
                                       out, lse, ws, v_dim=wl.v_dim)

    def k_dequant():
        K.kvfp4_dequantize_pages(geometry, packed, hot_back, pages, gs, slots, slots)

    legs = [("quantize", k_quant)]
    if wl is not None:
        legs.append(("decode", k_decode))
    legs.append(("dequantize", k_dequant))

    def run(n_steps, timed):
        ev = {k: [] for k, _ in legs}
        for _ in range(n_steps):
            for k, fn in legs:
                if not args.no_flush:
                    evict()
                if timed:
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    fn()
                    e1.record(stream)
                    ev[k].append((e0, e1))
                else:
                    fn()
        return ev

    def run_extras():
        """The "next" paths, timed beside the step (never part of it)."""
        ev = (lambda: None) if args.no_flush else evict
        return {
            "token_rows": time_append(K, torch, wl, geometry, gs, hot, packed, stream, ev,
                                      args.steps, args.warmup),
            "host_offload": time_offload(K, torch, wl, geometry, gs, hot, stream,
                                         min(args.steps, 10), min(args.warmup, 2)),
            "rope_layouts": time_rope_layouts(K, torch, wl, geometry, gs, hot, stream, ev,
                                              min(args.steps, 10), min(args.warmup, 2)),
        }

    if args.extras_only:
        if wl is None:
            print("--extras-only needs a decode workload", file=sys.stderr)
            sys.exit(2)
        k_quant()  # the packed pool the gathers read
        torch.cuda.synchronize()
        print(json.dumps({"mode": "extras-only", "workload": name, **run_extras()}), flush=True)
        return

    copy = None
    mixes = None
    if not args.no_copy_yardstick:
        # a plain device-to-device copy of 1 GiB: reads 1 GiB and writes 1 GiB
        src_c = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst_c = torch.empty_like(src_c)
        times = []
        for i in range(COPY_CALLS):
            evict()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            dst_c.copy_(src_c)
            e1.record(stream)
            times.append((e0, e1))
        torch.cuda.synchronize()
        ms_c = float(np.median([a.elapsed_time(b) for a, b in times[1:]]))
        copy = {"bytes": 2 * COPY_BYTES, "median_us": round(ms_c * 1e3, 2),
                "GB/s": round(2 * COPY_BYTES / (ms_c * 1e-3) / 1e9, 1)}
        mixes = stream_yardsticks(torch, src_c, dst_c, stream, evict)
        del src_c, dst_c

    run(args.warmup, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev = run(args.steps, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = {k: [a.elapsed_time(b) for a, b in v] for k, v in ev.items()}
    avg = {k: float(np.mean(v)) for k, v in ms.items()}
    med = {k: float(np.median(v)) for k, v in ms.items()}
    mn = {k: float(np.min(v)) for k, v in ms.items()}
    step_ms = float(sum(avg.values()))

    # warm figures (labelled as such, never the reported value): the same
    # calls back to back with no eviction, so inputs may sit in the caches
    warm = {}
    if not args.no_flush:
        ev_w = {k: [] for k, _ in legs}
        for _ in range(min(args.steps, 5)):
            for k, fn in legs:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                ev_w[k].append((e0, e1))
        torch.cuda.synchronize()
        warm = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in ev_w.items()}

    cb = codec_bytes(geometry, pages)
    leg_bytes = {"quantize": cb, "dequantize": cb}
    kern = {}
    if wl is not None:
        db = decode_bytes(wl)
        leg_bytes["decode"] = db["bytes"]
    for k in leg_bytes:
        gbs = leg_bytes[k] / (avg[k] * 1e-3) / 1e9
        kern[k] = {"avg_us": round(avg[k] * 1e3, 2), "median_us": round(med[k] * 1e3, 2),
                   "min_us": round(mn[k] * 1e3, 2),
                   "bytes": leg_bytes[k], "GB/s": round(gbs, 1),
                   "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
        if copy is not None:
            kern[k]["frac_copy_yardstick"] = round(gbs / copy["GB/s"], 4)
        if mixes and LEG_MIX[k] in mixes:
            kern[k]["frac_mix_yardstick"] = round(gbs / mixes[LEG_MIX[k]]["GB/s"], 4)
        if k in warm:
            kern[k]["warm_avg_us_no_eviction"] = round(warm[k] * 1e3, 2)
    if wl is not None:
        t = avg["decode"] * 1e-3
        kern["decode"]["tokens_per_s"] = round(wl.batch / t, 1)
        kern["decode"]["context_tokens_per_s"] = round(float(wl.seq_lens.sum()) / t, 1)
        kern["decode"]["TFLOP/s"] = round(db["flops"] / t / 1e12, 2)
        kern["decode"]["frac_bf16_mfma_peak"] = round(db["flops"] / t / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)
    step_bytes = sum(leg_bytes.values())
    value = step_bytes / (step_ms * 1e-3) / 1e9
    dom = max(avg, key=avg.get)
    from nvfp4_paged_decode_amd.profiling import read_traffic
    traffic = read_traffic(os.path.join(PROFILES, f"counters_{name}.txt"), name, dom)
    if dom == "decode" and name == "mla":
        # 128 query heads over one latent: a dense bf16 contraction (about
        # 820 flop per cache byte), bound by MFMA throughput, not HBM
        roof = {"kernel": dom, "bound": "mfma", "achieved": kern[dom]["TFLOP/s"],
                "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": kern[dom]["frac_bf16_mfma_peak"], "traffic": traffic}
    else:
        roof = {"kernel": dom, "bound": "hbm", "achieved": kern[dom]["GB/s"],
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": kern[dom]["frac_hbm_peak"],
                "traffic": traffic}

    if wl is not None:
        nt, T, H, D = geometry
        wdesc = (f"{name}: batch {wl.batch}, {wl.num_q_heads} q / {H} KV heads, head_dim {D}, "
                 f"v_dim {wl.v_dim}, context {int(wl.seq_lens.min())}-{int(wl.seq_lens.max())} "
                 f"(sum {int(wl.seq_lens.sum())}), page {T}; step = encode {pages} pages + "
                 f"decode attention + decode {pages} pages")
    else:
        wdesc = f"cold_pages: {pages} pages x {geometry}; step = encode + decode of every page"

    extras = run_extras() if wl is not None and not args.no_append else {}
    append = extras.get("token_rows")
    offload = extras.get("host_offload")
    rope = extras.get("rope_layouts")

    cpu = None
    if wl is not None and not args.no_cpu_baseline:
        try:
            cpu = cpu_baseline(wl, gs, args.cpu_seconds, leg_bytes,
                               db["bytes"] / float(wl.seq_lens.sum()), step_bytes)
        except Exception as e:  # the GPU figure stands on its own
            cpu = {"error": repr(e)}

    line = {
        "metric": "NVFP4-KV decode attn effective HBM GB/s (% peak) + page quant/dequant GB/s",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16<->nvfp4 codec (integer thresholds); attention fp16 MFMA, fp32 accumulate",
        "data": "synthetic (seeded)",
        "config": {"workload": wdesc, "global_scale": args.gs, "cache_flush_between_kernels":
                   "none" if args.no_flush else args.flush_mode + " 1 GiB", "global_batch": wl.batch if wl is not None else None,
                   "seq_len": int(wl.seq_lens.max()) if wl is not None else None,
                   "parallelism": "single GPU"},
        "kernels": kern,
        "copy_yardstick": copy,
        "stream_yardsticks": mixes,
        "token_rows": append,
        "host_offload": offload,
        "rope_layouts": rope,
        "roofline": roof,
        "cpu_baseline": cpu,
        "wall_s_timed_region": round(wall, 3),
        "gen_s": round(t_gen, 1),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
