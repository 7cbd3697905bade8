"""Norm-based ranking (BA-Att section 3.3, Eq. 9-10; Algorithm 1 steps 1, 2 and
12) on the HIP path against the fp64 oracle, through the C ABI.

Permutations and gathered/scattered rows must match bit for bit (both sides
form the float64 squared norm with the same additions in the same order;
ties keep token order).  The ranked forward's block indices must match bit
for bit; O within 2e-2 and LSE within 1e-3 for bf16 inputs, 1e-5 for float32.
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


def gpu_rank(basa, x):
    xt = dev(x)
    perm = torch.empty(xt.shape[:-1], dtype=torch.int32, device="cuda")
    basa.basa_rank(xt, perm)
    torch.cuda.synchronize()
    return host(perm)


@pytest.mark.parametrize("shape", [(1, 3, 4096, 128), (2, 2, 1000, 64), (1, 1, 1, 8), (1, 5, 33, 16)])
def test_rank_bf16_matches_oracle(basa, shape):
    note(f"rank bf16 {shape}")
    g = np.random.Generator(np.random.PCG64(sum(shape)))
    x = g.standard_normal(shape).astype(np.float32) * g.uniform(0.1, 4.0, size=shape[:-1] + (1,))
    x = wl.f32_to_bf16(x.astype(np.float32))
    assert np.array_equal(gpu_rank(basa, x), orc.norm_rank(x))


def test_rank_exact_ties_keep_token_order(basa):
    note("rank bf16 exact ties")
    g = np.random.Generator(np.random.PCG64(41))
    seqs, length, d = 4, 2048, 64
    base = g.integers(-6, 7, size=(seqs, 16, d)).astype(np.float32)
    rows = np.empty((seqs, length, d), dtype=np.float32)
    for s in range(seqs):
        pick = g.integers(0, 16, size=length)
        signs = g.choice(np.array([-1.0, 1.0], dtype=np.float32), size=(length, d))
        rows[s] = base[s, pick] * signs
        flip = g.random(length) < 0.5
        rows[s, flip] = rows[s, flip, ::-1]
    x = wl.f32_to_bf16(rows).reshape(2, 2, length, d)
    assert len(np.unique(orc.norm_key(x))) <= 64  # heavy ties
    assert np.array_equal(gpu_rank(basa, x), orc.norm_rank(x))


def test_rank_f32_tiny_and_f64(basa):
    note("rank fp32 tiny workload and float64 tokens")
    x = wl.generate("tiny")
    assert np.array_equal(gpu_rank(basa, x["q"]), orc.norm_rank(x["q"]))
    assert np.array_equal(gpu_rank(basa, x["k"]), orc.norm_rank(x["k"]))
    g = np.random.Generator(np.random.PCG64(42))
    xd = g.standard_normal((1, 2, 512, 16)) * 1e3 ** g.uniform(-1, 1, size=(1, 2, 512, 1))
    assert np.array_equal(gpu_rank(basa, xd), orc.norm_rank(xd))


@pytest.mark.parametrize("dtype,width", [("bf16", 128), ("f32", 1), ("bf16", 3), ("f64", 8), ("f32", 5)])
def test_permute_gather_scatter(basa, dtype, width):
    note(f"permute {dtype} width {width}")
    g = np.random.Generator(np.random.PCG64(43 + width))
    outer, length = 3, 777
    raw = g.standard_normal((outer, length, width))
    x = {"bf16": lambda a: wl.f32_to_bf16(a.astype(np.float32)), "f32": lambda a: a.astype(np.float32),
         "f64": lambda a: a}[dtype](raw)
    if width == 1:
        x = x[..., 0]
    perm = np.stack([g.permutation(length) for _ in range(outer)]).astype(np.int32)
    xt, pt = dev(x), dev(perm)
    out = torch.empty_like(xt)
    basa.basa_permute(xt, pt, out, basa.PERMUTE_GATHER)
    back = torch.empty_like(xt)
    basa.basa_permute(out, pt, back, basa.PERMUTE_SCATTER)
    torch.cuda.synchronize()
    x3 = x[..., None] if width == 1 else x
    ref = orc.gather_rows(x3, perm)
    got = host(out)
    got = got[..., None] if width == 1 else got
    assert np.array_equal(got, orc.as_f64(ref))
    assert np.array_equal(host(back), host(xt))
    # out-of-range entries: a gathered row is zero-filled, a scattered row is not written
    bad = perm.copy()
    bad[0, 5], bad[1, 0] = -1, length
    pb = dev(bad)
    out2 = torch.full_like(xt, 7)
    basa.basa_permute(xt, pb, out2, basa.PERMUTE_GATHER)
    out3 = torch.full_like(xt, 7)
    basa.basa_permute(xt, pb, out3, basa.PERMUTE_SCATTER)
    torch.cuda.synchronize()
    g2, g3 = host(out2), host(out3)
    if width == 1:
        g2, g3 = g2[..., None], g3[..., None]
    assert np.all(g2[0, 5] == 0) and np.all(g2[1, 0] == 0)
    keep = np.ones((outer, length), dtype=bool)
    keep[0, 5] = keep[1, 0] = False
    expect = orc.as_f64(orc.gather_rows(x3, np.where(keep, perm, 0)))
    assert np.array_equal(g2[keep], expect[keep])
    assert np.all(g3[0, perm[0, 5]] == 7) and np.all(g3[1, perm[1, 0]] == 7)
    written = np.zeros((outer, length), dtype=bool)
    for s_, i_ in zip(*np.nonzero(keep)):
        written[s_, perm[s_, i_]] = True
    expect3 = orc.as_f64(orc.scatter_rows(x3, perm))
    assert np.array_equal(g3[written], expect3[written])


def test_ranked_forward_tiny_fp32(basa):
    note("ranked forward tiny fp32 full")
    import block_sparse_attention_mean_amd.pipelines as p
    w = wl.WORKLOADS["tiny"]
    x = wl.generate("tiny")
    f = p.BaRankedForward(dev(x["q"]), dev(x["k"]), dev(x["v"]), w.block, w.topk, w.scale)
    f.run()
    torch.cuda.synchronize()
    pq, pk, idx, ro, rl = orc.ba_forward_ranked(x["q"], x["k"], x["v"], w.block, w.topk, w.scale)
    assert np.array_equal(host(f.perm_q), pq) and np.array_equal(host(f.perm_k), pk)
    assert np.array_equal(host(f.idx), idx)
    assert max_err(host(f.o), ro) <= 1e-5
    assert max_err(host(f.lse), rl) <= 1e-5


def test_ranked_forward_dlm16k_full_indices_sampled_tiles(basa):
    note("ranked forward dlm16k: perms and indices full, 32 sampled tiles")
    import block_sparse_attention_mean_amd.pipelines as p
    w = wl.WORKLOADS["dlm16k"]
    x = wl.generate("dlm16k")
    f = p.BaRankedForward(dev(x["q"]), dev(x["k"]), dev(x["v"]), w.block, w.topk, w.scale)
    f.run()
    torch.cuda.synchronize()
    pq, pk = orc.norm_rank(x["q"]), orc.norm_rank(x["k"])
    assert np.array_equal(host(f.perm_q), pq) and np.array_equal(host(f.perm_k), pk)
    qs = orc.gather_rows(orc.as_f64(x["q"]), pq)
    ks = orc.gather_rows(orc.as_f64(x["k"]), pk)
    vs = orc.gather_rows(orc.as_f64(x["v"]), pk)
    idx = orc.topk_ascending(orc.block_logits(orc.pool_mean(qs, w.block), orc.pool_mean(ks, w.block),
                                              w.scale), w.topk)
    assert np.array_equal(host(f.idx), idx)
    o, lse = host(f.o), host(f.lse)
    g = np.random.Generator(np.random.PCG64(44))
    for h, t in zip(g.integers(0, w.heads, 32), g.integers(0, w.blocks, 32)):
        ranked = np.arange(t * w.block, (t + 1) * w.block)
        ro, rl = orc.attend_rows(qs[0, h, ranked], ks[0, h], vs[0, h], idx[0, h, t], w.block, w.scale)
        rows = pq[0, h, ranked]  # where those ranked rows live in token order
        assert max_err(o[0, h, rows], ro) <= O_TOL, (h, t)
        assert max_err(lse[0, h, rows], rl) <= LSE_TOL, (h, t)


@pytest.mark.parametrize("kind,shape", [("bf16", (1, 2, 300, 512)), ("f64", (2, 1, 257, 128)),
                                        ("bf16", (1, 1, 130, 256))])
def test_rank_wide_rows_match_oracle(basa, kind, shape):
    # rows above 512 bytes take the one-thread-per-row kernel; 512 exactly is staged
    note(f"rank wide rows {kind} {shape}")
    g = np.random.Generator(np.random.PCG64(shape[-1] + shape[-2]))
    raw = g.standard_normal(shape) * g.uniform(0.1, 3.0, shape[:-1] + (1,))
    x = wl.f32_to_bf16(raw.astype(np.float32)) if kind == "bf16" else raw
    assert np.array_equal(gpu_rank(basa, x), orc.norm_rank(x))
