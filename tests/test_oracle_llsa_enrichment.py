"""Pins of the oracle's log-linear KV enrichment (llsa_forward's attention
part) to values fixed by the log-linear README, not by the oracle's code.

The README ("Log-linear sparse attention in plain MLX", KV enrichment
paragraph) says: each fine query attends to the surviving fine keys plus the
candidates of every coarser level l, and a level-l token's logit gets
l*ln(block) added so that it counts as block^l tokens.  The candidates of a
level are the children of the tokens its parent query selected one level up
(coarse-to-fine paragraph).  Three constructions make the expected O and LSE
computable by hand:

1. One coarse level with top-k equal to the block: nothing is pruned, so the
   result must equal plain softmax attention (torch's SDPA) over all fine keys
   plus 16 verbatim copies of every level-1 mean (the "counts as 16 tokens").
2. Two levels with all keys zero: every score ties, ties go to the lower
   index, so the candidate sets are the lowest ones; O and LSE are closed
   forms in sums of fine values.
3. Two levels with keys and queries aligned to per-group directions: each
   level-2 group of queries selects its own block first, so the candidate sets
   differ from group to group; O and LSE are closed forms per group, and a
   value shift planted in a coarse token that only one group's candidate set
   holds moves that group's rows by its exact weight.

Every pin runs on both references: the numpy oracle and the C++ one.
"""
import math

import numpy as np
import pytest
import torch

import oracle as orc
import oracle.cref as cref

LN16 = math.log(16.0)


@pytest.fixture(params=["numpy", "cpp"])
def llsa(request):
    """llsa_forward of the numpy oracle or of the C++ reference (same result keys)."""
    return orc.llsa_forward if request.param == "numpy" else cref.llsa_forward


def _sdpa(q, k, v, scale):
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a)) for a in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)
    lse = torch.logsumexp(scale * (tq @ tk.transpose(-1, -2)), dim=-1)
    return o.numpy(), lse.numpy()


def _avgpool16(x):
    """torch's 1-D average pooling over the token axis (an independent mean)."""
    t = torch.from_numpy(np.ascontiguousarray(x)).transpose(-1, -2)   # [H, d, N]
    return torch.nn.functional.avg_pool1d(t, 16, 16).transpose(-1, -2).numpy()


def test_one_level_nothing_pruned_equals_sdpa_over_repeated_means(llsa):
    g = np.random.Generator(np.random.PCG64(101))
    h, n, d, scale = 2, 256, 8, 0.4
    q, k, v = (g.standard_normal((h, n, d)) for _ in range(3))
    res = llsa(q, k, v, 16, 16, scale)
    assert res["levels"] == 1
    assert np.array_equal(res["sel"][1][0, 0], np.arange(16))          # every level-1 token kept
    kc = np.repeat(_avgpool16(k), 16, axis=1)                           # 16 copies of each mean
    vc = np.repeat(_avgpool16(v), 16, axis=1)
    o_ref, lse_ref = _sdpa(q, np.concatenate([k, kc], 1), np.concatenate([v, vc], 1), scale)
    assert np.abs(res["o"] - o_ref).max() < 1e-12
    assert np.abs(res["lse"] - lse_ref).max() < 1e-12


def test_two_levels_all_ties_closed_form(llsa):
    g = np.random.Generator(np.random.PCG64(103))
    n, d = 4096, 8
    q = g.standard_normal((1, n, d))
    k = np.zeros((1, n, d))
    v = g.standard_normal((1, n, d))
    res = llsa(q, k, v, 16, 8, 0.3)
    assert res["levels"] == 2
    # ties go to the lower index: level 2 keeps tokens 0..7 of 16, level 1 keeps
    # 0..7 of its candidates 0..127; fine keys are tokens 0..127
    assert np.all(res["sel"][2][0] == np.arange(8))
    assert np.all(res["sel"][1][0] == np.arange(8))
    # 128 fine keys (weight 1), level-1 tokens 0..127 (16 each), all 16 level-2
    # tokens (256 each), every logit zero before the bias
    total = 128 + 128 * 16 + 16 * 256
    assert np.abs(res["lse"] - math.log(total)).max() < 1e-12
    expect = (v[0, :128].sum(0) + v[0, :2048].sum(0) + v[0, :4096].sum(0)) / total
    assert np.abs(res["o"][0] - expect).max() < 1e-12


def _aligned(seed=107, alpha=2.0, beta=2.0, d=16):
    """Keys of level-2 block c all equal alpha*e_c, queries of level-2 block P
    all equal beta*e_P (e = unit vectors), values random."""
    n = 4096
    blk = np.arange(n) // 256
    e = np.eye(d)
    k = (alpha * e[blk])[None]
    q = (beta * e[blk])[None]
    v = np.random.Generator(np.random.PCG64(seed)).standard_normal((1, n, d))
    return q, k, v


def _others(p):
    """The 7 level-2 tokens a level-2 query of block p keeps besides p: all
    others score 0 and tie, so the lowest 7 indices other than p win."""
    return [c for c in range(16) if c != p][:7]


def test_two_levels_group_candidate_sets_closed_form(llsa):
    scale = 0.25
    q, k, v = _aligned()
    res = llsa(q, k, v, 16, 8, scale)
    assert res["levels"] == 2
    big = math.exp(scale * 2.0 * 2.0)              # e^(scale * alpha * beta)
    vv = v[0]
    for p in range(16):
        # the structure the README's rules give for query group p
        assert res["sel"][2][0, p].tolist() == sorted([p] + _others(p))
        for a in range(16 * p, 16 * p + 16):       # level-1 queries of group p
            assert res["sel"][1][0, a].tolist() == list(range(16 * p, 16 * p + 8))
        rows = slice(256 * p, 256 * (p + 1))
        # fine keys: tokens 256p .. 256p+127, each e^E
        # level 1: the 16 children of p (weight 16 e^E each) and the 112 children of the
        #          other seven picks (weight 16 each); 16 * mean of 16 rows = their sum
        # level 2: token p (256 e^E), the other 15 (256 each); 256 * mean = sum of 256 rows
        z = 128 * big + 256 * big + 112 * 16 + 256 * big + 15 * 256
        assert np.abs(res["lse"][0, rows] - math.log(z)).max() < 1e-12
        blk = lambda c: vv[256 * c:256 * (c + 1)].sum(0)
        num = (big * vv[256 * p:256 * p + 128].sum(0) + big * blk(p) + sum(blk(c) for c in _others(p))
               + big * blk(p) + sum(blk(c) for c in range(16) if c != p))
        assert np.abs(res["o"][0, rows] - num / z).max() < 1e-12, p


def test_coarse_value_shift_moves_only_its_candidate_group(llsa):
    """Level-1 token c = 16*10 + 12 is a candidate only of group 10 (no other
    level-2 query keeps block 10) and is not among the fine keys (group 10
    keeps children 160..167).  Shifting the values of its 16 fine tokens by D
    moves its level-1 mean by D (weight 16 e^E in group 10's rows only) and
    the level-2 mean of block 10 by D/16 (weight 256 in every other group,
    256 e^E in group 10)."""
    scale = 0.25
    q, k, v = _aligned(seed=109)
    base = llsa(q, k, v, 16, 8, scale)
    c, shift = 16 * 10 + 12, np.linspace(-1.0, 1.0, 16)
    v2 = v.copy()
    v2[0, 16 * c:16 * (c + 1)] += shift
    moved = llsa(q, k, v2, 16, 8, scale)
    big = math.exp(scale * 4.0)
    w_lse = np.exp(base["lse"][0])                  # LSE does not depend on values
    assert np.array_equal(moved["lse"], base["lse"])
    for p in range(16):
        rows = slice(256 * p, 256 * (p + 1))
        weight = (16 * big + 256 * big / 16) if p == 10 else 256 / 16
        expect = weight / w_lse[rows][:, None] * shift[None, :]
        got = moved["o"][0, rows] - base["o"][0, rows]
        assert np.abs(got - expect).max() < 1e-12, p
