"""Host-side checks of bench.py: the algorithmic byte counts behind its
GB/s figures, and the one-GPU contract (no GPU needed)."""

import os
import subprocess
import sys

import numpy as np

import bench
from nvfp4_paged_decode_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_codec_and_append_bytes():
    # 4096 Llama-3-8B-shaped pages: 1 GiB of bf16 in, 9/16 of the values' count out
    e = 2 * 64 * 8 * 128
    assert bench.codec_bytes((2, 64, 8, 128), 4096) == 4096 * (2 * e + e * 9 // 16)
    assert bench.codec_bytes((2, 64, 8, 128), 4096) == 1375731712
    # a token: 2048 values as bf16 rows, their 1152 packed bytes, 8 bytes of slot and row
    assert bench.append_bytes((2, 64, 8, 128), 1, 2) == 4096 + 1152 + 8
    assert bench.append_bytes((2, 64, 8, 128), 10, 1) == 10 * (2048 + 1152 + 8)


def test_decode_bytes_follow_the_definition():
    wl = W.llama3_8b(seed=3, batch=2, context=200)
    db = bench.decode_bytes(wl)
    L = wl.seq_lens.astype(np.int64)
    kv = int(L.sum()) * 2 * 8 * 128 * 9 // 16
    q = 2 * 32 * 128 * 2
    out = 2 * 32 * 128 * 2 + 2 * 32 * 4
    bt = int(np.sum(-(-L // 64))) * 4 + 2 * 4
    assert db["bytes"] == kv + q + out + bt
    assert db["kv_bytes"] == kv
    assert db["flops"] == 2 * int(L.sum()) * 32 * (128 + 128)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_every_leg_has_a_mix_yardstick():
    """Each streaming leg is read against a stream of its own traffic mix, and
    the mixes' byte factors match the directions they move (1 GiB on the
    reference side, a quarter of it on the other)."""
    assert set(bench.LEG_MIX) == {"decode", "quantize", "dequantize"}
    for leg, mix in bench.LEG_MIX.items():
        assert mix in bench.YARDSTICK_KINDS, (leg, mix)
    kinds = sorted(k for k, _ in bench.YARDSTICK_KINDS.values())
    assert kinds == [0, 1, 2, 3]
    assert bench.YARDSTICK_KINDS["read"][1] == 1.0
    assert bench.YARDSTICK_KINDS["read4_write1"][1] == 1.25
    assert bench.YARDSTICK_KINDS["read1_write4"][1] == 1.25


def test_yardstick_library_rejects_bad_arguments_before_launching():
    """libkvfp4_yardstick.so loads without a GPU and refuses sizes that are
    not whole sweeps, unaligned pointers and unknown kinds on the host
    (hipErrorInvalidValue, 1) before any HIP call."""
    import ctypes
    path = os.path.join(os.path.dirname(bench.__file__), "nvfp4_paged_decode_amd",
                        "libkvfp4_yardstick.so")
    if not os.path.exists(path):
        import pytest
        pytest.skip("libkvfp4_yardstick.so is not built")
    lib = ctypes.CDLL(path)
    f = lib.kvfp4_yardstick
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_size_t, ctypes.c_void_p]
    whole = 1 << 30
    assert f(0, 16, 16, 16, 0, None) == 1                 # empty
    assert f(0, 16, 16, 16, whole + 16, None) == 1        # not a whole sweep
    assert f(1, 16, 8, 16, whole, None) == 1              # unaligned destination
    assert f(7, 16, 16, 16, whole, None) == 1             # unknown kind
    assert f(0, None, 16, 16, whole, None) == 1           # read stream without a source
