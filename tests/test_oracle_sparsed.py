"""Pins of the oracle's block mass (BA-Att Eq. 3; SparseD's average-pooled
attention scores) and SparseD's isolated top-rho% selection (SparseD section
3.3, Eq. 5-6) to facts it does not compute itself.  CPU only.

* every row of the block mass sums to 1 (each attention row sums to 1);
* all-zero queries attend uniformly: every block holds block / L;
* the block mass equals torch's CPU attention whose values are the key-block
  indicator (output column g = attention on block g), averaged over each
  query block;
* the range top-k matches a brute-force rank count with exact ties;
* keeping every block (rho = 1) gives plain dense attention;
* a key block holding scaled copies of a query block's tokens carries most of
  that query block's mass and is kept.  (The mean-level plant of the tiny
  workload does not: copies of the pooled query score high only after
  pooling, the gap between pre- and post-downsampled maps that BA-Att
  section 3.2 analyses.)
"""
import math

import numpy as np
import torch

import oracle as orc
import workloads as wl


def _x(seed, shape):
    return np.random.default_rng(seed).standard_normal(shape)


def test_block_mass_rows_sum_to_one():
    q, k = _x(61, (1, 3, 256, 16)), _x(62, (1, 3, 256, 16)) * 2.0
    m = orc.block_mass(q, k, 32, 0.5)
    assert np.abs(m.sum(axis=-1) - 1.0).max() < 1e-13


def test_zero_queries_give_uniform_mass():
    k = _x(63, (1, 2, 512, 8))
    m = orc.block_mass(np.zeros((1, 2, 512, 8)), k, 64, 0.3)
    assert np.abs(m - 64 / 512).max() < 1e-15


def test_block_mass_equals_library_attention_on_block_indicators():
    L, d, blk = 384, 16, 32
    q, k = _x(64, (1, 2, L, d)), _x(65, (1, 1, L, d)) * 1.5   # GQA 2:1
    nb = L // blk
    ind = np.zeros((L, nb))
    ind[np.arange(L), np.arange(L) // blk] = 1.0
    tq = torch.from_numpy(q)
    tk = torch.from_numpy(np.repeat(k, 2, axis=1))
    tv = torch.from_numpy(np.broadcast_to(ind, (1, 2, L, nb)).copy())
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=0.25).numpy()
    ref = o.reshape(1, 2, nb, blk, nb).mean(axis=3)
    assert np.abs(orc.block_mass(q, k, blk, 0.25) - ref).max() < 1e-13


def test_topk_in_ranges_brute_force_with_ties():
    g = np.random.default_rng(66)
    s = np.round(g.standard_normal((40, 30)), 1)  # many exact ties
    split, k_lo, k_hi = 11, 4, 7
    got = orc.topk_in_ranges(s, split, k_lo, k_hi)
    for r in range(40):
        want = []
        for lo, hi, k in ((0, split, k_lo), (split, 30, k_hi)):
            for j in range(lo, hi):
                better = sum(1 for i in range(lo, hi) if s[r, i] > s[r, j] or (s[r, i] == s[r, j] and i < j))
                if better < k:
                    want.append(j)
        assert got[r].tolist() == sorted(want)


def test_range_counts_round_up():
    assert orc.range_counts(64, 64, 0.3) == (20, 20)      # 19.2 -> 20
    assert orc.range_counts(10, 90, 0.5) == (5, 45)       # exact halves stay exact
    assert orc.range_counts(3, 0, 0.01) == (1, 0)         # a non-empty range keeps one
    assert orc.range_counts(7, 9, 1.0) == (7, 9)
    assert orc.range_counts(100, 100, 0.07) == (math.ceil(7.0), 7)


def test_rho_one_is_dense_attention():
    w = wl.WORKLOADS["tiny"]
    x = wl.make_tiny(w.seed)
    idx, o, lse = orc.sparsed_forward(x["q"], x["k"], x["v"], w.block, w.scale, prefill=512, rho=1.0)
    assert idx.shape[-1] == w.blocks
    tq, tk, tv = (torch.from_numpy(orc.as_f64(x[n])) for n in "qkv")
    o_ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=w.scale).numpy()
    lse_ref = torch.logsumexp(w.scale * (tq @ tk.transpose(-1, -2)), dim=-1).numpy()
    assert np.abs(o - o_ref).max() < 1e-12
    assert np.abs(lse - lse_ref).max() < 1e-12


def test_pattern_keeps_a_token_level_planted_block():
    # key block 5 holds query block 2's tokens scaled by 3: every query of
    # block 2 meets its own copy with logit 3 |q|^2 scale, far above the rest,
    # so block 5 (a generation block for prefill 96) carries most of the mass
    g = np.random.default_rng(67)
    L, d, blk = 256, 16, 32
    q = g.standard_normal((1, 1, L, d))
    k = g.standard_normal((1, 1, L, d))
    k[0, 0, 5 * blk:6 * blk] = 3.0 * q[0, 0, 2 * blk:3 * blk]
    m = orc.block_mass(q, k, blk, 0.25)
    assert int(np.argmax(m[0, 0, 2])) == 5 and m[0, 0, 2, 5] > 0.5
    idx = orc.sparsed_pattern(q, k, blk, 0.25, prefill=96, rho=0.2)
    assert idx.shape[-1] == 1 + 1                      # ceil(0.2*3), ceil(0.2*5)
    assert 5 in idx[0, 0, 2] and idx[0, 0, 2, 0] < 3   # one prefill block, then block 5
