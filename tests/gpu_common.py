"""Helpers shared by the GPU parity tests: device transfer, the oracle side
of each comparison, poisoning of bytes the kernels must never read, and the
tolerance."""

import numpy as np
import pytest

from oracle import nvfp4 as O
from oracle import attention as A

torch = pytest.importorskip("torch")

# spec tolerance for attention outputs against the fp64 oracle
ATOL, RTOL = 1e-2, 1e-2


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def as_bits16(t):
    """View a GPU tensor of 16-bit values as int16 for transfer."""
    return t.view(torch.int16)


def oracle_packed_pages(hot_pool: np.ndarray, geometry, gs, slots) -> np.ndarray:
    """Oracle-encoded packed bytes for the given hot slots: [len(slots), bytes]."""
    g = O.Geometry(*geometry)
    out = np.zeros((len(slots), O.packed_page_bytes(g)), np.uint8)
    sub = hot_pool[np.asarray(slots)]
    O.quantize_pages(sub, g, len(slots), gs, out)
    return out


def poison_unread(packed: np.ndarray, wl, rng) -> None:
    """Fill every byte no decode may read with garbage whose E4M3 scales are
    NaN: rows past each sequence's length in its last page, and every slot no
    sequence uses (unused block-table entries point at one of them)."""
    g = O.Geometry(*wl.geometry)
    used = np.zeros(wl.num_slots, bool)
    used[wl.used_slots] = True
    for s in np.nonzero(~used)[0]:
        packed[s] = rng.integers(0, 256, packed.shape[1], dtype=np.uint8)
        _, scales = O.split_packed_page(packed[s], g)
        scales[...] = 0x7F
    T = wl.page_size
    for b in range(wl.batch):
        L = int(wl.seq_lens[b])
        if L % T == 0:
            continue
        slot = int(wl.block_table[b, L // T])
        data, scales = O.split_packed_page(packed[slot], g)
        data[:, L % T:] = rng.integers(0, 256, data[:, L % T:].shape, dtype=np.uint8)
        scales[:, L % T:] = 0x7F


def assert_attention_close(out_gpu_bits: np.ndarray, ref: np.ndarray, what: str):
    got = (out_gpu_bits.astype(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = ATOL + RTOL * np.abs(ref)
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside 1e-2 + 1e-2|ref|; "
                           f"max err {err.max():.3g}")


def oracle_attention(packed, wl, gs, batch_indices=None, head_indices=None):
    g = O.Geometry(*wl.geometry)
    return A.decode_attention(packed, g, gs, wl.q, wl.block_table, wl.seq_lens,
                              wl.softmax_scale, wl.v_dim, batch_indices, head_indices)
