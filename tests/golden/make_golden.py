"""Write tests/golden/tiny_page.npz: one small seeded page, its packed NVFP4
bytes and its dequantized bf16 bits, all produced by the CPU oracle.

Run from the repository root:  python tests/golden/make_golden.py
Only ``oracle/`` computes the stored values; the bf16 input is drawn here.
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import nvfp4 as O  # noqa: E402


def main():
    g = O.Geometry(2, 4, 2, 32)
    rng = np.random.default_rng(20260)
    x = rng.standard_normal((1, *g.row_shape)).astype(np.float32)
    x[0, 0, 1, 0, :16] = 0.0              # an all-zero block
    x[0, 1, 2, 1, 16:] *= np.float32(1e4)  # a large block
    x[0, 1, 3, 0, :16] *= np.float32(1e-6)  # a tiny block
    u = x.view(np.uint32)
    hot = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    hot[0, 0, 0, 1, 3] = 0x8000           # a negative zero
    gs = np.array([1.0, np.float32(0.0123456)], dtype=np.float32)
    packed = np.zeros((1, O.packed_page_bytes(g)), np.uint8)
    O.quantize_pages(hot, g, 1, gs, packed)
    back = np.zeros_like(hot)
    O.dequantize_pages(packed, g, 1, gs, back)
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_page.npz")
    np.savez(out, geometry=np.array([2, 4, 2, 32]), hot=hot, gs=gs, packed=packed[0], dequant=back)
    print("wrote", out)


if __name__ == "__main__":
    main()
