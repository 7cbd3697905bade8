"""Pins of the oracle's norm ranking (BA-Att section 3.3, Eq. 9-10; Algorithm 1
steps 1, 2 and 12) to facts it does not compute itself.  CPU only.

* closed form: tokens whose only nonzero channel holds a known value have a
  known rank, so the permutation is the inverse of a known shuffle;
* ties: a brute-force rank count under (key ascending, token ascending);
* exactness: the float64 squared norm of bf16 tokens equals the exact
  rational sum of squares;
* the whole ranked method with every block kept equals plain dense attention
  on the unranked tensors (torch's CPU attention): keys and values move
  together and the outputs go back by the inverse permutation, so a wrong
  inverse or a key/value mismatch shows up there;
* a planted mistake (ranking V by its own norms) must break that equality.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as orc
import workloads as wl


def test_rank_closed_form_is_inverse_shuffle():
    g = np.random.default_rng(21)
    L, d = 257, 16
    shuffle = g.permutation(L)
    x = np.zeros((1, 1, L, d))
    x[0, 0, :, 3] = -(shuffle + 1.0)  # norm of token i is shuffle[i] + 1
    perm = orc.norm_rank(x)[0, 0]
    assert perm.dtype == np.int32
    # the token with norm r + 1 is at rank r, and that token is shuffle^-1(r)
    assert all(perm[shuffle[i]] == i for i in range(L))


def test_rank_ties_keep_token_order_brute_force():
    g = np.random.default_rng(22)
    L, d = 96, 8
    base = g.integers(-8, 9, size=(12, d)).astype(np.float64)
    # 8 copies of each of 12 integer rows, each copy sign-flipped and
    # channel-reversed at random: equal squared norms (integers, so exact in
    # any order), positions shuffled
    rows = []
    for r in range(12):
        for _ in range(8):
            v = base[r] * g.choice([-1.0, 1.0], size=d)
            rows.append(v[::-1] if g.random() < 0.5 else v)
    x = np.array(rows)[g.permutation(L)]
    key = orc.norm_key(x)
    assert len(np.unique(key)) <= 12  # every key is shared by 8 tokens
    perm = orc.norm_rank(x)
    for j in range(L):
        pos = sum(1 for i in range(L) if key[i] < key[j] or (key[i] == key[j] and i < j))
        assert perm[pos] == j


def test_squared_norm_of_bf16_tokens_is_exact():
    g = np.random.default_rng(23)
    x = wl.f32_to_bf16(g.standard_normal((40, 128)).astype(np.float32))
    key = orc.norm_key(x)
    vals = orc.as_f64(x)
    for t in range(40):
        exact = sum(Fraction(float(a)) ** 2 for a in vals[t])
        assert Fraction(float(key[t])) == exact


def test_gather_scatter_inverse_and_sorted():
    g = np.random.default_rng(24)
    x = g.standard_normal((2, 3, 64, 8))
    p = orc.norm_rank(x)
    xs = orc.gather_rows(x, p)
    assert np.all(np.diff(orc.norm_key(xs), axis=-1) >= 0)
    assert np.array_equal(orc.scatter_rows(xs, p), x)
    assert np.array_equal(orc.gather_rows(orc.scatter_rows(x, p), p), x)


def _ranked_dense(q, k, v, block, scale, rank_v_by_own_norm=False):
    nb = q.shape[2] // block
    pq, pk, idx, o, lse = orc.ba_forward_ranked(q, k, v, block, nb, scale)
    if rank_v_by_own_norm:  # planted mistake: V ranked apart from K
        qs = orc.gather_rows(orc.as_f64(q), pq)
        ks = orc.gather_rows(orc.as_f64(k), pk)
        vs = orc.gather_rows(orc.as_f64(v), orc.norm_rank(v))
        o_s, lse_s = orc.sparse_attention(qs, ks, vs, idx, block, block, scale)
        o, lse = orc.scatter_rows(o_s, pq), orc.scatter_rows(lse_s[..., None], pq)[..., 0]
    return o, lse


def _sdpa(q, k, v, scale):
    tq, tk, tv = (torch.from_numpy(orc.as_f64(a)) for a in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)
    lse = torch.logsumexp(scale * (tq @ tk.transpose(-1, -2)), dim=-1)
    return o.numpy(), lse.numpy()


def test_ranked_method_with_every_block_kept_is_dense_attention():
    w = wl.WORKLOADS["tiny"]
    x = wl.make_tiny(w.seed)
    o, lse = _ranked_dense(x["q"], x["k"], x["v"], w.block, w.scale)
    o_ref, lse_ref = _sdpa(x["q"], x["k"], x["v"], w.scale)
    assert np.abs(o - o_ref).max() < 1e-12
    assert np.abs(lse - lse_ref).max() < 1e-12


def test_planted_mistake_breaks_the_dense_equality():
    w = wl.WORKLOADS["tiny"]
    x = wl.make_tiny(w.seed)
    o, _ = _ranked_dense(x["q"], x["k"], x["v"], w.block, w.scale, rank_v_by_own_norm=True)
    o_ref, _ = _sdpa(x["q"], x["k"], x["v"], w.scale)
    assert np.abs(o - o_ref).max() > 1e-3


def test_ranked_selection_is_a_valid_mask_over_permutations():
    # ranked lists are ascending, in range, and the rankings are permutations
    w = wl.WORKLOADS["tiny"]
    x = wl.make_tiny(w.seed)
    pq, pk, idx, o, lse = orc.ba_forward_ranked(x["q"], x["k"], x["v"], w.block, w.topk, w.scale)
    assert idx.shape == (1, w.heads, w.blocks, w.topk)
    assert np.all(np.diff(idx, axis=-1) > 0) and idx.min() >= 0 and idx.max() < w.blocks
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    for h in range(w.heads):
        assert sorted(pq[0, h].tolist()) == list(range(w.tokens))
        assert sorted(pk[0, h].tolist()) == list(range(w.tokens))


@pytest.mark.parametrize("hq,hkv", [(4, 2)])
def test_ranked_method_gqa_dense(hq, hkv):
    g = np.random.default_rng(25)
    L, d, blk = 256, 16, 32
    q = g.standard_normal((1, hq, L, d)) * g.uniform(0.2, 3.0, size=(1, hq, L, 1))
    k = g.standard_normal((1, hkv, L, d)) * g.uniform(0.2, 3.0, size=(1, hkv, L, 1))
    v = g.standard_normal((1, hkv, L, d))
    o, lse = _ranked_dense(q, k, v, blk, 0.25)
    kk = np.repeat(k, hq // hkv, axis=1)
    vv = np.repeat(v, hq // hkv, axis=1)
    o_ref, lse_ref = _sdpa(q, kk, vv, 0.25)
    assert np.abs(o - o_ref).max() < 1e-12
    assert np.abs(lse - lse_ref).max() < 1e-12
