"""Pins of the oracle's covariance compensation (BA-Att section 3.4, Eq. 13-14;
Algorithm 1 steps 4-7) to facts it does not compute itself.  CPU only.

* the block variance equals torch's population variance over each block;
* blocks whose tokens are all equal have zero variance, so the compensated
  logit is the plain one (Eq. 2);
* single-channel blocks with known moments give each of Eq. 14's three terms
  in closed form, one term at a time, and a cross-channel case gives zero:
  a dropped term, a missing 1/d, a wrong beta or a mismatched channel fails;
* Algorithm 1 with beta = 0 reduces to the plain (unranked) selection and to
  the ranked forward.
"""
import numpy as np
import pytest
import torch

import oracle as orc
import workloads as wl


def test_block_variance_is_library_population_variance():
    g = np.random.default_rng(31)
    x = g.standard_normal((2, 3, 256, 16)) * 3.0 + 1.5
    ref = torch.from_numpy(x).reshape(2, 3, 8, 32, 16).var(dim=-2, unbiased=False).numpy()
    assert np.abs(orc.block_variance(x, 32) - ref).max() < 1e-13


def test_constant_blocks_have_no_compensation():
    g = np.random.default_rng(32)
    # dyadic values: a block's sum and mean are exact, so its deviations are exactly zero
    q = np.repeat(g.integers(-16, 17, size=(1, 2, 8, 16)) / 4.0, 32, axis=2)
    k = np.repeat(g.integers(-16, 17, size=(1, 2, 8, 16)) / 4.0, 32, axis=2)
    qb, kb = orc.pool_mean(q, 32), orc.pool_mean(k, 32)
    qv, kv = orc.block_variance(q, 32), orc.block_variance(k, 32)
    assert np.all(qv == 0) and np.all(kv == 0)
    got = orc.compensated_logits(qb, kb, qv, kv, 0.25, 1.0)
    assert np.array_equal(got, orc.block_logits(qb, kb, 0.25))


def _one_block(d, ch, values):
    """One block of len(values) tokens whose channel ch holds the values, others zero."""
    x = np.zeros((1, 1, len(values), d))
    x[0, 0, :, ch] = values
    return x


@pytest.mark.parametrize("beta", [1.0, 0.5])
def test_each_term_of_eq14_in_closed_form(beta):
    d, n, a, b, c, e = 16, 8, 3.0, 2.0, 1.25, 0.5
    alt = lambda m: [m if i % 2 == 0 else -m for i in range(n)]  # mean 0, variance m^2
    const = lambda m: [m] * n                                     # mean m, variance 0
    cases = [
        (alt(a), const(b), a * a * b * b / d),   # Var[Q] Kbar^2
        (const(c), alt(e), e * e * c * c / d),   # Var[K] Qbar^2
        (alt(a), alt(e), a * a * e * e / d),     # Var[Q] Var[K]
    ]
    for qv, kv, delta in cases:
        q, k = _one_block(d, 5, qv), _one_block(d, 5, kv)
        got = orc.compensated_logits(orc.pool_mean(q, n), orc.pool_mean(k, n), orc.block_variance(q, n),
                                     orc.block_variance(k, n), 0.25, beta)
        plain = 0.25 * float(np.mean(qv)) * float(np.mean(kv)) * 1.0
        assert abs(float(got[0, 0, 0, 0]) - (plain + beta * delta)) < 1e-14
    # moments in different channels never meet
    q, k = _one_block(d, 1, alt(a)), _one_block(d, 2, const(b))
    got = orc.compensated_logits(orc.pool_mean(q, n), orc.pool_mean(k, n), orc.block_variance(q, n),
                                 orc.block_variance(k, n), 0.25, beta)
    assert got[0, 0, 0, 0] == 0.0


def test_gqa_key_heads_are_shared():
    g = np.random.default_rng(33)
    q = g.standard_normal((1, 4, 128, 8))
    k = g.standard_normal((1, 2, 128, 8)) * 2.0
    args = lambda qq, kk: (orc.pool_mean(qq, 16), orc.pool_mean(kk, 16), orc.block_variance(qq, 16),
                           orc.block_variance(kk, 16))
    got = orc.compensated_logits(*args(q, k), 0.3, 1.0)
    for h in range(4):
        one = orc.compensated_logits(*args(q[:, h:h + 1], k[:, h // 2:h // 2 + 1]), 0.3, 1.0)
        assert np.array_equal(got[:, h:h + 1], one)


def test_algorithm1_with_beta_zero_reduces_to_the_plain_and_ranked_paths():
    w = wl.WORKLOADS["tiny"]
    x = wl.make_tiny(w.seed)
    _, _, idx, o, lse = orc.ba_forward_algorithm1(x["q"], x["k"], x["v"], w.block, w.topk, w.scale,
                                                  beta=0.0, rank=False)
    plain = orc.topk_ascending(orc.block_logits(orc.pool_mean(x["q"], w.block),
                                                orc.pool_mean(x["k"], w.block), w.scale), w.topk)
    assert np.array_equal(idx, plain)
    pq, pk, idx_r, o_r, lse_r = orc.ba_forward_algorithm1(x["q"], x["k"], x["v"], w.block, w.topk,
                                                          w.scale, beta=0.0, rank=True)
    pq2, pk2, idx2, o2, lse2 = orc.ba_forward_ranked(x["q"], x["k"], x["v"], w.block, w.topk, w.scale)
    assert np.array_equal(pq, pq2) and np.array_equal(pk, pk2) and np.array_equal(idx_r, idx2)
    assert np.array_equal(o_r, o2) and np.array_equal(lse_r, lse2)
