"""Covariance-compensated block selection (BA-Att section 3.4, Eq. 13-14;
Algorithm 1 steps 4-7) on the HIP path against the fp64 oracle.

The moment vectors u and w (their dot product is the compensated logit) are
compared with the oracle's block means and variances within 1e-12 relative
(the two sides round in different orders); the selected block indices must
match bit for bit, unranked and after norm ranking (the whole of Algorithm
1); O within 2e-2 and LSE within 1e-3 for bf16 inputs, 1e-5 for float32.
"""
import numpy as np
import pytest
import torch

import oracle as orc
import workloads as wl
from gpu_util import LSE_TOL, O_TOL, dev, host, max_err, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def basa():
    assert torch.cuda.is_available(), "the GPU tests need a visible GPU"
    import block_sparse_attention_mean_amd as mod
    return mod


def rel_err(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


@pytest.mark.parametrize("kind,shape,block", [("bf16", (1, 2, 1024, 128), 128), ("f32", (1, 2, 1024, 64), 64),
                                              ("f64", (2, 1, 256, 16), 32), ("bf16", (1, 1, 512, 168), 16),
                                              ("bf16", (1, 1, 1024, 128), 256)])
def test_moment_vectors_match_oracle(basa, kind, shape, block):
    note(f"moments {kind} {shape} block {block}")
    g = np.random.Generator(np.random.PCG64(shape[-1] + block))
    raw = g.standard_normal(shape) * 1.5 + g.standard_normal(shape[:-2] + (1, shape[-1]))
    x = {"bf16": lambda a: wl.f32_to_bf16(a.astype(np.float32)), "f32": lambda a: a.astype(np.float32),
         "f64": lambda a: a}[kind](raw)
    b, h, length, d = shape
    nb = length // block
    scale, beta = 0.125, 0.75
    xt = dev(x)
    u = torch.empty(b, h, nb, 3 * d, dtype=torch.float64, device="cuda")
    w = torch.empty(b, h, 3 * d, nb, dtype=torch.float64, device="cuda")
    basa.basa_pool_moments(xt, block, u, basa.MOMENTS_QUERY, scale, beta)
    basa.basa_pool_moments(xt, block, w, basa.MOMENTS_KEY, 1.0, beta)
    torch.cuda.synchronize()
    m, var = orc.pool_mean(x, block), orc.block_variance(x, block)
    ref_u = np.concatenate([scale * m, beta / d * var, beta / d * m * m], axis=-1)
    ref_w = np.swapaxes(np.concatenate([m, m * m + var, var], axis=-1), -1, -2)
    assert rel_err(host(u), ref_u) < 1e-12
    assert rel_err(host(w), ref_w) < 1e-12
    # the dot product is the compensated logit of Eq. 13-14
    got = np.einsum("bhqc,bhck->bhqk", host(u), host(w))
    ref = orc.compensated_logits(m, m, var, var, scale, beta)
    assert rel_err(got, ref) < 1e-12


def gpu_compensated_select(basa, q, k, block, topk, scale, beta):
    import block_sparse_attention_mean_amd.pipelines as p
    qt, kt = dev(q), dev(k)
    f = p.BaForward(qt, kt, kt, block, topk, scale, beta=beta)
    f.select()
    torch.cuda.synchronize()
    return host(f.idx)


def oracle_compensated_select(q, k, block, topk, scale, beta):
    return orc.topk_ascending(orc.compensated_logits(orc.pool_mean(q, block), orc.pool_mean(k, block),
                                                     orc.block_variance(q, block),
                                                     orc.block_variance(k, block), scale, beta), topk)


def test_compensated_selection_tiny_and_dlm16k(basa):
    note("compensated selection tiny (beta 1) and dlm16k full (beta 1)")
    for name in ("tiny", "dlm16k"):
        w = wl.WORKLOADS[name]
        x = wl.generate(name)
        got = gpu_compensated_select(basa, x["q"], x["k"], w.block, w.topk, w.scale, 1.0)
        assert np.array_equal(got, oracle_compensated_select(x["q"], x["k"], w.block, w.topk, w.scale, 1.0))


def test_compensated_selection_gqa(basa):
    note("compensated selection GQA 8:2, beta 2")
    g = np.random.Generator(np.random.PCG64(52))
    q = wl.f32_to_bf16((g.standard_normal((1, 8, 4096, 64)) * g.uniform(0.5, 2, (1, 8, 4096, 1))).astype(np.float32))
    k = wl.f32_to_bf16((g.standard_normal((1, 2, 4096, 64)) * g.uniform(0.5, 2, (1, 2, 4096, 1))).astype(np.float32))
    got = gpu_compensated_select(basa, q, k, 64, 12, 0.125, 2.0)
    assert np.array_equal(got, oracle_compensated_select(q, k, 64, 12, 0.125, 2.0))


def test_algorithm1_tiny_fp32_full(basa):
    note("Algorithm 1 (ranking + compensation) tiny fp32 full")
    import block_sparse_attention_mean_amd.pipelines as p
    w = wl.WORKLOADS["tiny"]
    x = wl.generate("tiny")
    f = p.BaRankedForward(dev(x["q"]), dev(x["k"]), dev(x["v"]), w.block, w.topk, w.scale, beta=1.0)
    f.run()
    torch.cuda.synchronize()
    pq, pk, idx, ro, rl = orc.ba_forward_algorithm1(x["q"], x["k"], x["v"], w.block, w.topk, w.scale, 1.0)
    assert np.array_equal(host(f.perm_q), pq) and np.array_equal(host(f.perm_k), pk)
    assert np.array_equal(host(f.idx), idx)
    assert max_err(host(f.o), ro) <= 1e-5
    assert max_err(host(f.lse), rl) <= 1e-5


def test_algorithm1_dlm16k_full_indices_sampled_tiles(basa):
    note("Algorithm 1 dlm16k: perms and indices full, 24 sampled tiles")
    import block_sparse_attention_mean_amd.pipelines as p
    w = wl.WORKLOADS["dlm16k"]
    x = wl.generate("dlm16k")
    f = p.BaRankedForward(dev(x["q"]), dev(x["k"]), dev(x["v"]), w.block, w.topk, w.scale, beta=1.0)
    f.run()
    torch.cuda.synchronize()
    pq, pk = orc.norm_rank(x["q"]), orc.norm_rank(x["k"])
    assert np.array_equal(host(f.perm_q), pq) and np.array_equal(host(f.perm_k), pk)
    qs = orc.gather_rows(orc.as_f64(x["q"]), pq)
    ks = orc.gather_rows(orc.as_f64(x["k"]), pk)
    idx = oracle_compensated_select(qs, ks, w.block, w.topk, w.scale, 1.0)
    assert np.array_equal(host(f.idx), idx)
    vs = orc.gather_rows(x["v"], pk)
    o, lse = host(f.o), host(f.lse)
    g = np.random.Generator(np.random.PCG64(53))
    for h, t in zip(g.integers(0, w.heads, 24), g.integers(0, w.blocks, 24)):
        ranked = np.arange(t * w.block, (t + 1) * w.block)
        ro, rl = orc.attend_rows(qs[0, h, ranked], ks[0, h], vs[0, h], idx[0, h, t], w.block, w.scale)
        rows = pq[0, h, ranked]
        assert max_err(o[0, h, rows], ro) <= O_TOL, (h, t)
        assert max_err(lse[0, h, rows], rl) <= LSE_TOL, (h, t)
