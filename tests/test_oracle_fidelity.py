"""Pins of the oracle's fidelity diagnostics (BA-Att Eq. 3, Eq. 7-8) to facts
it does not compute itself.  CPU only.

* Eq. 8 is a bound: every token logit lies within U of its block logit (a
  brute-force check over all token pairs, with and without norm ranking);
* radii and max norms of blocks with known geometry, in closed form;
* recall is 1 for the oracle's own selection and 0 for its complement.
"""
import math

import numpy as np

import oracle as orc
import workloads as wl


def test_deviation_bound_holds_for_every_token_pair():
    g = np.random.default_rng(71)
    L, d, blk = 256, 16, 32
    q = g.standard_normal((1, 1, L, d)) * g.uniform(0.2, 3.0, (1, 1, L, 1))
    k = g.standard_normal((1, 1, L, d)) * g.uniform(0.2, 3.0, (1, 1, L, 1))
    for rank in (False, True):
        qq, kk = q, k
        if rank:
            qq, kk = orc.gather_rows(q, orc.norm_rank(q)), orc.gather_rows(k, orc.norm_rank(k))
        rq, mq = orc.block_radius_maxnorm(qq, blk)
        rk, mk = orc.block_radius_maxnorm(kk, blk)
        u = orc.deviation_bound(rq, mq, rk, mk, d)[0, 0]
        tok = (qq[0, 0] @ kk[0, 0].T) / math.sqrt(d)
        blkl = orc.block_logits(orc.pool_mean(qq, blk), orc.pool_mean(kk, blk), 1 / math.sqrt(d))[0, 0]
        dev = np.abs(tok - np.repeat(np.repeat(blkl, blk, axis=0), blk, axis=1))
        bound = np.repeat(np.repeat(u, blk, axis=0), blk, axis=1)
        assert np.all(dev <= bound * (1 + 1e-12))
        assert dev.max() > 0.25 * bound.min()  # the bound is not vacuous


def test_radius_and_max_norm_closed_form():
    # a block of 4 tokens: +-a e_0 and +-b e_1 -> mean 0, radius max(a, b), max norm max(a, b)
    a, b = 3.0, 4.0
    x = np.zeros((1, 4, 8))
    x[0, 0, 0], x[0, 1, 0], x[0, 2, 1], x[0, 3, 1] = a, -a, b, -b
    r, m = orc.block_radius_maxnorm(x, 4)
    assert r[0, 0] == 4.0 and m[0, 0] == 4.0
    # shifted by c e_2: radius unchanged, max norm sqrt(b^2 + c^2)
    x[0, :, 2] = 12.0
    r, m = orc.block_radius_maxnorm(x, 4)
    assert r[0, 0] == 4.0 and m[0, 0] == math.sqrt(16.0 + 144.0)


def test_recall_extremes():
    w = wl.WORKLOADS["tiny"]
    x = wl.make_tiny(w.seed)
    mass = orc.block_mass(x["q"], x["k"], w.block, w.scale)
    best = orc.topk_ascending(mass, w.topk)
    assert orc.selection_recall(best, mass) == 1.0
    worst = orc.topk_ascending(-mass, w.topk)
    assert orc.selection_recall(worst, mass) == 0.0
