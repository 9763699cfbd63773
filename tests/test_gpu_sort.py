"""GPU tests of the page-list sort (kvfp4_sort_page_list): the output is the
input pairs stably sorted by key as unsigned 32-bit values, run by run of
16384 entries, and the codec's results do not depend on the list order."""

import numpy as np
import pytest

import nvfp4_paged_decode_amd as K
from nvfp4_paged_decode_amd import workloads as W
from tests.gpu_common import dev, host, require_gpu, torch

pytestmark = pytest.mark.gpu
RUN = 16384


def expected(key: np.ndarray, other: np.ndarray):
    """Stable sort by unsigned key within consecutive runs of RUN entries."""
    ko, oo = [], []
    for b in range(0, len(key), RUN):
        k, o = key[b:b + RUN], other[b:b + RUN]
        order = np.argsort(k.astype(np.uint32), kind="stable")
        ko.append(k[order])
        oo.append(o[order])
    return np.concatenate(ko), np.concatenate(oo)


@pytest.mark.parametrize("n", [1, 2, 5, 1000, 4096, 4097, RUN, RUN + 3, 2 * RUN + 1000])
def test_sort_matches_stable_sort(n):
    """Random keys with repeats, negative keys and keys past any pool."""
    require_gpu()
    rng = np.random.default_rng(n)
    key = rng.integers(-3, max(8, n // 2), n).astype(np.int32)
    key[rng.random(n) < 0.01] = np.int32(2**31 - 1)
    other = rng.integers(-(2**31), 2**31 - 1, n, dtype=np.int64).astype(np.int32)
    ko = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    oo = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    K.kvfp4_sort_page_list(dev(key), ko, dev(other), oo)
    ek, eo = expected(key, other)
    assert np.array_equal(host(ko), ek)
    assert np.array_equal(host(oo), eo)


@pytest.mark.parametrize("n,span", [(1, 1), (5, 9), (4096, 4160), (RUN, 32768), (RUN + 100, 20000),
                                    (3000, 40000)])
def test_sort_distinct_keys(n, span):
    """Distinct keys drawn from [0, span): the table path while every key
    of a run is below 32768, the network otherwise (span 40000)."""
    require_gpu()
    rng = np.random.default_rng(n + span)
    key = np.concatenate([rng.permutation(span)[:min(RUN, n - b)] for b in range(0, n, RUN)])
    key = key.astype(np.int32)
    other = rng.integers(0, 1 << 30, n).astype(np.int32)
    ko = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    oo = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    K.kvfp4_sort_page_list(dev(key), ko, dev(other), oo)
    ek, eo = expected(key, other)
    assert np.array_equal(host(ko), ek)
    assert np.array_equal(host(oo), eo)


def test_sort_keys_only_and_repeatable():
    """Without the paired list; two calls give the same output."""
    require_gpu()
    rng = np.random.default_rng(5)
    key = rng.permutation(6000).astype(np.int32)
    outs = []
    for _ in range(2):
        ko = torch.empty((6000,), dtype=torch.int32, device="cuda")
        K.kvfp4_sort_page_list(dev(key), ko)
        outs.append(host(ko))
    assert np.array_equal(outs[0], np.arange(6000, dtype=np.int32))
    assert np.array_equal(outs[0], outs[1])


def test_codec_results_do_not_depend_on_list_order():
    """The codec calls with a sorted (src, dst) list write the same bytes as
    with the list as given (a random order of the pool's slots, some of them
    out of range)."""
    require_gpu()
    wl = W.llama3_8b(seed=31, batch=4, context=700)
    G, gs = wl.geometry, [float(v) for v in wl.gs_calibrated]
    n, slots = int(wl.used_slots.shape[0]), wl.num_slots
    rng = np.random.default_rng(7)
    src = wl.used_slots.astype(np.int32)
    dst = rng.permutation(slots)[:n].astype(np.int32)
    src[3] = -1
    dst[5] = slots + 2
    hot = dev(wl.hot_pool.view(np.int16))
    pb = K.kvfp4_packed_page_bytes(G)
    src_s = torch.empty((n,), dtype=torch.int32, device="cuda")
    dst_s = torch.empty((n,), dtype=torch.int32, device="cuda")
    K.kvfp4_sort_page_list(dev(src), src_s, dev(dst), dst_s)
    packed = []
    for s, d in ((dev(src), dev(dst)), (src_s, dst_s)):
        p = torch.zeros((slots, pb), dtype=torch.uint8, device="cuda")
        K.kvfp4_quantize_pages(G, hot, p, n, gs, s, d)
        packed.append(p)
    assert torch.equal(packed[0], packed[1])
    back = []
    for s, d in ((dev(src), dev(dst)), (src_s, dst_s)):
        h = torch.zeros_like(hot)
        K.kvfp4_dequantize_pages(G, packed[0], h, n, gs, d, s)
        back.append(h)
    assert torch.equal(back[0], back[1])
