"""Whole workflows through the C ABI against the fp64 oracle, at full size.

* BA-Att forward on the 64K-token workload: every selected index bit-exact,
  attention on sampled query tiles (the oracle computes them one by one).
* Log-linear hierarchical top-k on the 256 x 256 image workload: every level's
  selection bit-exact, O and LSE on all rows.
* LoSA prefix step on the 64K-prefix workload: active tokens and selections
  bit-exact, O / LSE / updated cache rows on all rows.
Tolerances: O 2e-2, LSE 1e-3 (bf16 inputs, float32 accumulation).
"""
import math

import numpy as np
import pytest
import torch

import oracle as orc
import workloads as wl
from gpu_util import (LSE_TOL, O_TOL, check_tiles_against_oracle, dev, host, max_err, note,
                      stratified_tiles)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pipes():
    assert torch.cuda.is_available(), "the GPU tests need a visible GPU"
    import block_sparse_attention_mean_amd.pipelines as p
    return p


def test_ba_forward_dlm64k_indices_full_and_stratified_tiles(pipes):
    note("BA-Att forward dlm64k: H32 L65536 block128 top128; every 8th tile of every head (2048)")
    w = wl.WORKLOADS["dlm64k"]
    x = wl.generate("dlm64k")
    f = pipes.BaForward(dev(x["q"]), dev(x["k"]), dev(x["v"]), w.block, w.topk)
    f.run()
    torch.cuda.synchronize()
    ref_idx = orc.topk_ascending(orc.block_logits(orc.pool_mean(x["q"], w.block),
                                                  orc.pool_mean(x["k"], w.block), w.scale), w.topk)
    assert np.array_equal(host(f.idx), ref_idx)
    o, lse = host(f.o), host(f.lse)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    tiles = stratified_tiles(w.heads, w.blocks)
    assert len(tiles) == 2048
    eo, el = check_tiles_against_oracle(o, lse, x["q"], x["k"], x["v"], ref_idx, tiles, w.block,
                                        w.block, w.scale)
    note(f"dlm64k 2048 tiles: O err {eo:.2e}, LSE err {el:.2e}")
    assert eo <= O_TOL and el <= LSE_TOL


def test_merge_dlm64k_partials_against_oracle(pipes):
    """The split-list merge at full 64K size: each row's 128 kept blocks split
    into two halves, each half's attention as float32 partials, merged on the
    GPU into bf16 O + LSE, compared with the oracle's merge of the same
    partials on every 16th row of every head, and with the oracle's one-shot
    attention on a stratified sample of tiles."""
    import block_sparse_attention_mean_amd as basa
    note("merge dlm64k: halves of every list as float32 partials, merged")
    w = wl.WORKLOADS["dlm64k"]
    x = wl.generate("dlm64k")
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    ref_idx = orc.topk_ascending(orc.block_logits(orc.pool_mean(x["q"], w.block),
                                                  orc.pool_mean(x["k"], w.block), w.scale), w.topk)
    idx = dev(ref_idx)
    half = w.topk // 2
    oa = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    ob = torch.empty_like(oa)
    la = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    lb = torch.empty_like(la)
    kw = dict(tile_q=w.block, block_k=w.block, scale=w.scale)
    basa.basa_attn(q, basa.kv_segment(idx, k, v, count=half), oa, la, **kw)
    basa.basa_attn(q, basa.kv_segment(idx, k, v, offset=half, count=w.topk - half), ob, lb, **kw)
    om = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    lm = torch.empty_like(la)
    basa.basa_merge(oa, la, ob, lb, om, lm)
    torch.cuda.synchronize()
    rows = slice(3, None, 16)
    pa, pla = host(oa[:, :, rows]), host(la[:, :, rows])
    pb, plb = host(ob[:, :, rows]), host(lb[:, :, rows])
    ro, rl = orc.merge(pa, pla, pb, plb)
    got_o, got_l = host(om[:, :, rows]), host(lm[:, :, rows])
    # float32 partials in, bf16 O out: the merge itself adds one bf16 rounding
    assert max_err(got_o, ro) <= 2 ** -8 * np.abs(ro).max() + 1e-6
    assert max_err(got_l, rl) <= 1e-5
    del oa, ob, la, lb
    tiles = stratified_tiles(w.heads, w.blocks, every=64)
    eo, el = check_tiles_against_oracle(host(om), host(lm), x["q"], x["k"], x["v"], ref_idx, tiles,
                                        w.block, w.block, w.scale)
    assert eo <= O_TOL and el <= LSE_TOL


def test_ba_ranked_forward_dlm64k_full_perms_indices_sampled_tiles(pipes):
    note("BA-Att ranked forward dlm64k: perms and indices full, 24 sampled tiles")
    w = wl.WORKLOADS["dlm64k"]
    x = wl.generate("dlm64k")
    f = pipes.BaRankedForward(dev(x["q"]), dev(x["k"]), dev(x["v"]), w.block, w.topk)
    f.run()
    torch.cuda.synchronize()
    pq, pk = orc.norm_rank(x["q"]), orc.norm_rank(x["k"])
    assert np.array_equal(host(f.perm_q), pq)
    assert np.array_equal(host(f.perm_k), pk)
    qs = orc.gather_rows(orc.as_f64(x["q"]), pq)
    ks = orc.gather_rows(orc.as_f64(x["k"]), pk)
    ref_idx = orc.topk_ascending(orc.block_logits(orc.pool_mean(qs, w.block),
                                                  orc.pool_mean(ks, w.block), w.scale), w.topk)
    assert np.array_equal(host(f.idx), ref_idx)
    vs = orc.gather_rows(x["v"], pk)
    o, lse = host(f.o), host(f.lse)
    g = np.random.Generator(np.random.PCG64(37))
    tiles = [(int(h), int(t)) for h, t in zip(g.integers(0, w.heads, 24), g.integers(0, w.blocks, 24))]
    for h, t in tiles + [(0, 0), (w.heads - 1, w.blocks - 1)]:
        ranked = np.arange(t * w.block, (t + 1) * w.block)
        ro, rl = orc.attend_rows(qs[0, h, ranked], ks[0, h], vs[0, h], ref_idx[0, h, t], w.block, w.scale)
        rows = pq[0, h, ranked]
        assert max_err(o[0, h, rows], ro) <= O_TOL, (h, t)
        assert max_err(lse[0, h, rows], rl) <= LSE_TOL, (h, t)


def test_ba_algorithm1_dlm64k_full_perms_indices_sampled_tiles(pipes):
    note("BA-Att Algorithm 1 (ranking + compensation, beta 1) dlm64k: indices full, 16 sampled tiles")
    w = wl.WORKLOADS["dlm64k"]
    x = wl.generate("dlm64k")
    f = pipes.BaRankedForward(dev(x["q"]), dev(x["k"]), dev(x["v"]), w.block, w.topk, beta=1.0)
    f.run()
    torch.cuda.synchronize()
    pq, pk = orc.norm_rank(x["q"]), orc.norm_rank(x["k"])
    assert np.array_equal(host(f.perm_q), pq)
    assert np.array_equal(host(f.perm_k), pk)
    qs = orc.gather_rows(orc.as_f64(x["q"]), pq)
    ks = orc.gather_rows(orc.as_f64(x["k"]), pk)
    scores = orc.compensated_logits(orc.pool_mean(qs, w.block), orc.pool_mean(ks, w.block),
                                    orc.block_variance(qs, w.block), orc.block_variance(ks, w.block),
                                    w.scale, 1.0)
    ref_idx = orc.topk_ascending(scores, w.topk)
    assert np.array_equal(host(f.idx), ref_idx)
    vs = orc.gather_rows(x["v"], pk)
    o, lse = host(f.o), host(f.lse)
    g = np.random.Generator(np.random.PCG64(39))
    for h, t in zip(g.integers(0, w.heads, 16), g.integers(0, w.blocks, 16)):
        ranked = np.arange(t * w.block, (t + 1) * w.block)
        ro, rl = orc.attend_rows(qs[0, h, ranked], ks[0, h], vs[0, h], ref_idx[0, h, t], w.block, w.scale)
        rows = pq[0, h, ranked]
        assert max_err(o[0, h, rows], ro) <= O_TOL, (h, t)
        assert max_err(lse[0, h, rows], rl) <= LSE_TOL, (h, t)


@pytest.mark.parametrize("n,heads,d", [(1024, 2, 64), (4096, 3, 64), (65536, 4, 64)])
def test_llsa_forward_matches_oracle(pipes, n, heads, d):
    note(f"LLSA forward N{n} H{heads} d{d}")
    if n == 65536:
        x = wl.generate("llsa64k")
    else:
        g = np.random.Generator(np.random.PCG64(n))
        x = {k: wl.f32_to_bf16(g.standard_normal((1, heads, n, d)).astype(np.float32)) for k in "qkv"}
    scale = 1.0 / math.sqrt(d)
    f = pipes.LlsaForward(dev(x["q"]), dev(x["k"]), dev(x["v"]), 16, 8, scale)
    f.run()
    torch.cuda.synchronize()
    ref = orc.llsa_forward(x["q"][0], x["k"][0], x["v"][0], 16, 8, scale)
    assert ref["levels"] == f.levels
    for lv in range(1, f.levels + 1):
        assert np.array_equal(host(f.sel[lv])[0], ref["sel"][lv]), lv
    assert max_err(host(f.o)[0], ref["o"]) <= O_TOL
    assert max_err(host(f.lse)[0], ref["lse"]) <= LSE_TOL


@pytest.mark.parametrize("prefix,topk", [(1024, 8), (65536, 128)])
def test_losa_step_matches_oracle(pipes, prefix, topk):
    note(f"LoSA step prefix {prefix} top-{topk}")
    x = wl.make_losa(1004 if prefix == 65536 else 77, prefix=prefix)
    scale = 1.0 / math.sqrt(128)
    co, cl = orc.dense_attention(x["q_prev"], x["k_prefix"], x["v_prefix"], scale)
    co32, cl32 = co.astype(np.float32), cl.astype(np.float32)
    cache_o, cache_lse = dev(co32), dev(cl32)
    s = pipes.LosaStep(dev(x["q_cur"]), dev(x["q_prev"]), dev(x["k_prefix"]), dev(x["v_prefix"]),
                       dev(x["k_block"]), dev(x["v_block"]), cache_o, cache_lse, 5, 16, topk, scale)
    s.prepare()
    s.step()
    torch.cuda.synchronize()
    ref = orc.losa_step(x["q_cur"], x["q_prev"], x["k_prefix"], x["v_prefix"], x["k_block"],
                        x["v_block"], co32, cl32, 5, 16, topk, scale)
    assert np.array_equal(host(s.active), ref["active"])
    assert host(s.active).tolist() == [list(wl.LOSA_PLANTED)]
    assert np.array_equal(host(s.sel), ref["sel"])
    assert max_err(host(cache_o), ref["cache_o"]) <= 1e-3
    assert max_err(host(cache_lse), ref["cache_lse"]) <= LSE_TOL
    assert max_err(host(s.o), ref["o"]) <= O_TOL
    assert max_err(host(s.lse), ref["lse"]) <= LSE_TOL
    stable = [t for t in range(16) if t not in wl.LOSA_PLANTED]
    assert np.array_equal(host(cache_o)[:, :, stable], co32[:, :, stable].astype(np.float64))
