"""Pins of the fp64 C++ reference (oracle/basa_oracle_ref.cpp) and its agreement
with the numpy oracle.

The C++ reference is pinned to the same independent facts as the numpy
oracle (torch's CPU attention, a brute-force rank count, the merge identity,
torch's average pooling, the planted block of the tiny workload), so a slip in
either implementation shows up against something neither of them computes.
The cross-check against the numpy oracle then covers the ragged, GQA and
invalid-slot cases on the same inputs.  CPU only.
"""
import numpy as np
import pytest
import torch

import oracle as orc
import oracle.cref as cref
import workloads as wl


def _tiny():
    w = wl.WORKLOADS["tiny"]
    x = wl.make_tiny(w.seed)
    return w, {n: x[n].astype(np.float64) for n in ("q", "k", "v")}


def _sdpa(q, k, v, scale, mask=None):
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a)) for a in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
    z = scale * (tq @ tk.transpose(-1, -2))
    if mask is not None:
        z = z.masked_fill(~mask, float("-inf"))
    return o.numpy(), torch.logsumexp(z, dim=-1).numpy()


def test_cref_dense_reduction_equals_library_sdpa():
    # BA-Att Eq. 1: with every key block kept the block-sparse attention is dense attention
    w, x = _tiny()
    nb = w.blocks
    idx = np.broadcast_to(np.arange(nb, dtype=np.int32), (1, w.heads, nb, nb)).copy()
    o, lse = cref.sparse_attention(x["q"], x["k"], x["v"], idx, w.block, w.block, w.scale)
    o_ref, lse_ref = _sdpa(x["q"], x["k"], x["v"], w.scale)
    assert np.abs(o - o_ref).max() < 1e-12
    assert np.abs(lse - lse_ref).max() < 1e-12


def test_cref_block_mask_equals_masked_sdpa_and_planted_block():
    # BA-Att section 3.1: the kept set is the top-kappa by pooled logits; the
    # planted block (key block 12 = 3x the mean of query block 3) ranks first
    w, x = _tiny()
    qb, kb = cref.pool_mean(x["q"], w.block), cref.pool_mean(x["k"], w.block)
    scores = cref.block_logits(qb, kb, w.scale)
    idx = cref.topk_ascending(scores, w.topk)
    g_star, p = wl.TINY_PLANT_QUERY_BLOCK, wl.TINY_PLANT_KEY_BLOCK
    assert all(p in idx[0, h, g_star] for h in range(w.heads))
    assert all(int(np.argmax(scores[0, h, g_star])) == p for h in range(w.heads))
    o, lse = cref.sparse_attention(x["q"], x["k"], x["v"], idx, w.block, w.block, w.scale)
    nb, blk = w.blocks, w.block
    mask = np.zeros((1, w.heads, w.tokens, w.tokens), dtype=bool)
    for h in range(w.heads):
        for t in range(nb):
            for g in idx[0, h, t]:
                mask[0, h, t * blk:(t + 1) * blk, g * blk:(g + 1) * blk] = True
    o_ref, lse_ref = _sdpa(x["q"], x["k"], x["v"], w.scale, torch.from_numpy(mask))
    assert np.abs(o - o_ref).max() < 1e-12
    assert np.abs(lse - lse_ref).max() < 1e-12


def test_cref_topk_matches_brute_force_with_ties():
    # a column is kept iff fewer than k columns beat it under (score desc, index asc)
    g = np.random.default_rng(5)
    s = np.round(g.standard_normal((64, 40)), 1)  # many exact ties
    s[3, :] = 0.0
    s[4, 7] = -0.0
    for k in (1, 5, 17, 40):
        idx = cref.topk_ascending(s, k)
        for r in range(s.shape[0]):
            want = [j for j in range(s.shape[1])
                    if sum(1 for i in range(s.shape[1])
                           if s[r, i] > s[r, j] or (s[r, i] == s[r, j] and i < j)) < k]
            assert list(idx[r]) == want


def test_cref_two_part_merge_equals_one_shot_and_identity():
    # LoSA post: two partials over disjoint key sets merge to the one-shot result
    w, x = _tiny()
    qb, kb = cref.pool_mean(x["q"], w.block), cref.pool_mean(x["k"], w.block)
    idx = cref.topk_ascending(cref.block_logits(qb, kb, w.scale), w.topk)
    o1, l1 = cref.sparse_attention(x["q"], x["k"], x["v"], idx, w.block, w.block, w.scale)
    oa, la = cref.sparse_attention(x["q"], x["k"], x["v"], idx[..., :1], w.block, w.block, w.scale)
    ob, lb = cref.sparse_attention(x["q"], x["k"], x["v"], idx[..., 1:], w.block, w.block, w.scale)
    om, lm = cref.merge(oa, la, ob, lb)
    assert np.abs(om - o1).max() < 1e-12 and np.abs(lm - l1).max() < 1e-12
    empty_o, empty_l = np.zeros_like(oa), np.full(la.shape, -np.inf)
    oi, li = cref.merge(oa, la, empty_o, empty_l)
    assert np.array_equal(oi, oa) and np.array_equal(li, la)
    oe, le = cref.merge(empty_o, empty_l, empty_o, empty_l)
    assert np.all(oe == 0) and np.all(np.isneginf(le))


def test_cref_pooling_against_library_avg_pool():
    g = np.random.default_rng(6)
    x = g.standard_normal((3, 256, 32))
    ref = torch.nn.functional.avg_pool1d(torch.from_numpy(x).transpose(1, 2), 16).transpose(1, 2)
    assert np.abs(cref.pool_mean(x, 16) - ref.numpy()).max() < 1e-14
    with pytest.raises(ValueError):
        cref.pool_mean(x, 7)


def test_cref_constant_values_return_the_value():
    w, x = _tiny()
    v = np.full_like(x["v"], 0.375)
    idx = np.random.default_rng(3).integers(0, w.blocks, (1, w.heads, w.blocks, 3)).astype(np.int32)
    o, _ = cref.sparse_attention(x["q"], x["k"], v, idx, w.block, w.block, w.scale)
    assert np.abs(o - 0.375).max() < 1e-14


@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 2)])
def test_cref_agrees_with_numpy_oracle_gqa_ragged_invalid(hq, hkv):
    # same inputs through both fp64 references: bf16 data, GQA, lists with
    # unused (-1) and out-of-range slots, an empty list
    g = np.random.default_rng(11)
    L, d, blk = 512, 64, 64
    q = wl.f32_to_bf16(g.standard_normal((1, hq, L, d)).astype(np.float32))
    k = wl.f32_to_bf16(g.standard_normal((1, hkv, L, d)).astype(np.float32))
    v = wl.f32_to_bf16(g.standard_normal((1, hkv, L, d)).astype(np.float32))
    nb = L // blk
    qb_c, kb_c = cref.pool_mean(q, blk), cref.pool_mean(k, blk)
    qb_n, kb_n = orc.pool_mean(q, blk), orc.pool_mean(k, blk)
    assert np.abs(qb_c - qb_n).max() < 1e-15 and np.abs(kb_c - kb_n).max() < 1e-15
    s_c = cref.block_logits(qb_c, kb_c, 0.125)
    s_n = orc.block_logits(qb_n, kb_n, 0.125)
    assert np.abs(s_c - s_n).max() < 1e-14
    assert np.array_equal(cref.topk_ascending(s_c, 3), orc.topk_ascending(s_n, 3))
    idx = cref.topk_ascending(s_c, 3)
    idx[0, 0, 1, 2] = -1
    idx[0, -1, 2, 0] = nb + 4
    idx[0, 0, 3, :] = -1
    o_c, l_c = cref.sparse_attention(q, k, v, idx, blk, blk, 0.125)
    o_n, l_n = orc.sparse_attention(q, k, v, np.where(idx >= nb, -1, idx), blk, blk, 0.125)
    fin = np.isfinite(l_n)
    assert np.array_equal(fin, np.isfinite(l_c))
    assert np.abs(o_c - o_n).max() < 1e-12
    assert np.abs(l_c[fin] - l_n[fin]).max() < 1e-12
    assert np.all(o_c[0, 0, 3 * blk:4 * blk] == 0)
