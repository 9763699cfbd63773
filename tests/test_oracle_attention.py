"""Pins for the oracle's decode attention."""

import numpy as np
import pytest
import torch

from oracle import nvfp4 as O
from oracle import attention as A
from nvfp4_paged_decode_amd import workloads as W


def _packed(wl, gs):
    g = O.Geometry(*wl.geometry)
    packed = np.zeros((wl.num_slots, O.packed_page_bytes(g)), np.uint8)
    O.quantize_pages(wl.hot_pool, g, wl.num_slots, gs, packed)
    return g, packed


def _dense_kv(wl, g, packed, gs, b):
    L = int(wl.seq_lens[b])
    K = A.gather_rows(packed, g, gs, wl.block_table[b], L, 0)
    V = K if g.num_kv_tensors == 1 else A.gather_rows(packed, g, gs, wl.block_table[b], L, 1)
    return K, V[..., :wl.v_dim]


def _small_gqa(seed=9, B=3, H=2, G=4, D=64, T=16, lens=(37, 16, 1)):
    rng = np.random.default_rng(seed)
    nt = 2
    pages = [-(-l // T) for l in lens]
    slots = sum(pages) + 2
    perm = rng.permutation(slots).astype(np.int32)
    bt = np.full((B, max(pages)), perm[-1], np.int32)
    c = 0
    for b in range(B):
        bt[b, :pages[b]] = perm[c:c + pages[b]]
        c += pages[b]
    hot = W.f32_to_bf16_bits(rng.standard_normal((slots, nt, T, H, D)).astype(np.float32))
    q = W.f32_to_bf16_bits(rng.standard_normal((B, H * G, D)).astype(np.float32))
    return W.DecodeWorkload("small", nt, T, H, D, B, H * G, D, 0.3, hot, bt,
                            np.array(lens, np.int32), q, np.ones(nt, np.float32),
                            W.calibrated_scales(hot), perm[:c], int(perm[-1]))


def _walked_kv(wl, gs, b):
    """K/V of sequence b for the textbook reference, built without the
    oracle's page-table walk or its decode: token j's bf16 row is read from
    the hot pool at slot block_table[b][j // T], row j % T, quantized with
    the oracle's row quantizer (pinned by the brute-force tests), and its
    codes are decoded here from exact E2M1 / E4M3 rationals."""
    from fractions import Fraction
    from tests.exact import E2M1, E4M3
    T, H, D = wl.page_size, wl.num_kv_heads, wl.head_dim
    L = int(wl.seq_lens[b])
    out = []
    for t in range(wl.num_kv_tensors):
        gsf = Fraction(float(np.float32(gs[t])))
        rows = np.empty((L, H, D), np.float64)
        for j in range(L):
            slot = int(wl.block_table[b][j // T])
            bits = wl.hot_pool[slot, t, j % T]           # [H, D] bf16 bits
            data, scales = O.quantize_rows(bits, gs[t])
            for h in range(H):
                for d in range(D):
                    byte = int(data[h, d // 2])
                    nib = byte & 0xF if d % 2 == 0 else byte >> 4
                    v = E2M1[nib & 7] * E4M3[int(scales[h, d // 16])] * gsf
                    rows[j, h, d] = float(-v if nib & 8 else v)
        out.append(rows)
    K = out[0]
    V = K if wl.num_kv_tensors == 1 else out[1]
    return K, V[..., :wl.v_dim]


@pytest.mark.parametrize("gs_kind", ["unit", "calibrated"])
def test_matches_torch_sdpa_in_float64(gs_kind):
    wl = _small_gqa()
    gs = wl.gs_unit if gs_kind == "unit" else wl.gs_calibrated
    g, packed = _packed(wl, gs)
    out, lse = A.decode_attention(packed, g, gs, wl.q, wl.block_table, wl.seq_lens,
                                  wl.softmax_scale, wl.v_dim)
    G = wl.num_q_heads // wl.num_kv_heads
    for b in range(wl.batch):
        K, V = _walked_kv(wl, gs, b)
        q = torch.from_numpy(O.bf16_bits_to_f64(wl.q[b]))[None, :, None, :]  # [1, Hq, 1, D]
        k = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, 0)[None]
        v = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, 0)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=wl.softmax_scale)
        np.testing.assert_allclose(out[b], ref[0, :, 0].numpy(), rtol=1e-12, atol=1e-12)
        s = wl.softmax_scale * torch.einsum("hd,hld->hl", q[0, :, 0], k[0])
        np.testing.assert_allclose(lse[b], torch.logsumexp(s, -1).numpy(), rtol=1e-12)


def test_closed_forms():
    wl = _small_gqa(lens=(1, 20, 33))
    gs = wl.gs_unit
    g, packed = _packed(wl, gs)
    # one token: the output is that token's value row
    out, lse = A.decode_attention(packed, g, gs, wl.q, wl.block_table, wl.seq_lens, 0.3, wl.v_dim)
    G = wl.num_q_heads // wl.num_kv_heads
    K, V = _dense_kv(wl, g, packed, gs, 0)
    for h in range(wl.num_q_heads):
        np.testing.assert_array_equal(out[0, h], V[0, h // G])
    # softmax scale 0: the mean of the value rows
    out0, lse0 = A.decode_attention(packed, g, gs, wl.q, wl.block_table, wl.seq_lens, 0.0, wl.v_dim)
    for b in range(3):
        K, V = _dense_kv(wl, g, packed, gs, b)
        for h in range(wl.num_q_heads):
            np.testing.assert_allclose(out0[b, h], V[:, h // G].mean(0), rtol=1e-13, atol=1e-14)
            assert abs(lse0[b, h] - np.log(wl.seq_lens[b])) < 1e-12


def test_one_dominant_score_selects_its_value():
    wl = _small_gqa(lens=(40, 17, 5))
    gs = wl.gs_unit
    g, packed = _packed(wl, gs)
    G = wl.num_q_heads // wl.num_kv_heads
    b, h = 1, 3
    K, V = _dense_kv(wl, g, packed, gs, b)
    j = 11
    # a query parallel to k_j with a large norm: score j exceeds all others by > 50
    qv = K[j, h // G] / np.linalg.norm(K[j, h // G])
    q = wl.q.copy()
    q[b, h] = W.f32_to_bf16_bits((qv * 400).astype(np.float32))
    s = 1.0 * (K[:, h // G] @ O.bf16_bits_to_f64(q[b, h]))
    assert np.sort(s)[-1] - np.sort(s)[-2] > 50
    out, _ = A.decode_attention(packed, g, gs, q, wl.block_table, wl.seq_lens, 1.0, wl.v_dim,
                                batch_indices=[b], head_indices=[h])
    # every other weight is below e**-50
    np.testing.assert_allclose(out[0, 0], V[j, h // G], rtol=0,
                               atol=1e-13 * np.abs(V).max() + 2 * 40 * np.exp(-50) * np.abs(V).max())


def test_split_invariance_of_lse_merge():
    wl = _small_gqa(lens=(47, 30, 9))
    gs = wl.gs_calibrated
    g, packed = _packed(wl, gs)
    full, lse = A.decode_attention(packed, g, gs, wl.q, wl.block_table, wl.seq_lens, 0.3, wl.v_dim)
    T = wl.page_size
    # attention over the first page only and over the rest, merged
    first = wl.seq_lens.copy(); first[:] = np.minimum(wl.seq_lens, T)
    o1, l1 = A.decode_attention(packed, g, gs, wl.q, wl.block_table, first, 0.3, wl.v_dim)
    rest_bt = wl.block_table[:, 1:]
    rest = np.maximum(wl.seq_lens - T, 0)
    o2, l2 = A.decode_attention(packed, g, gs, wl.q, np.ascontiguousarray(rest_bt), rest, 0.3, wl.v_dim)
    for b in range(wl.batch):
        for h in range(wl.num_q_heads):
            o, l = A.merge_partials([o1[b, h], o2[b, h]], [l1[b, h], l2[b, h]])
            np.testing.assert_allclose(o, full[b, h], rtol=1e-12, atol=1e-13)
            assert abs(l - lse[b, h]) < 1e-12


def test_empty_sequence():
    wl = _small_gqa(lens=(0, 5, 0))
    g, packed = _packed(wl, wl.gs_unit)
    out, lse = A.decode_attention(packed, g, wl.gs_unit, wl.q, wl.block_table, wl.seq_lens, 0.3, wl.v_dim)
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    assert np.all(lse[0] == -np.inf) and np.all(np.isfinite(lse[1]))


def test_mla_value_is_the_latent_prefix():
    # MLA reduces to MQA with one latent head: the value of token j is the
    # first v_dim dims of the same dequantized latent row
    wl = W.mla(seed=21, batch=2, context=70, num_q_heads=8)
    gs = wl.gs_calibrated
    g, packed = _packed(wl, gs)
    out, lse = A.decode_attention(packed, g, gs, wl.q, wl.block_table, wl.seq_lens,
                                  wl.softmax_scale, wl.v_dim)
    for b in range(2):
        K, V = _dense_kv(wl, g, packed, gs, b)
        q = torch.from_numpy(O.bf16_bits_to_f64(wl.q[b]))[None, :, None, :]
        k = torch.from_numpy(K).permute(1, 0, 2).expand(8, -1, -1)[None]
        v = torch.from_numpy(K[..., :512]).permute(1, 0, 2).expand(8, -1, -1)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=wl.softmax_scale)
        np.testing.assert_allclose(out[b], ref[0, :, 0].numpy(), rtol=1e-12, atol=1e-12)
