"""Fidelity diagnostics (BA-Att Eq. 3, Eq. 7-8) on the HIP path against the
fp64 oracle, through the C ABI: block radii and max norms within 1e-12
relative; the recall of a selection against the top-k of the block mass,
both taken from GPU results, equal to the oracle's (the indices are exact)."""
import numpy as np
import pytest
import torch

import oracle as orc
import workloads as wl
from gpu_util import dev, host, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def basa():
    assert torch.cuda.is_available(), "the GPU tests need a visible GPU"
    import block_sparse_attention_mean_amd as mod
    return mod


@pytest.mark.parametrize("kind,shape,block", [("bf16", (1, 2, 1024, 128), 128), ("f32", (2, 1, 512, 64), 64),
                                              ("f64", (1, 3, 256, 16), 32), ("bf16", (1, 1, 210, 24), 7)])
def test_block_radius_matches_oracle(basa, kind, shape, block):
    note(f"block radius {kind} {shape} block {block}")
    g = np.random.Generator(np.random.PCG64(shape[-1] * 7 + block))
    raw = g.standard_normal(shape) * g.uniform(0.2, 3.0, shape[:-1] + (1,)) + 0.5
    x = {"bf16": lambda a: wl.f32_to_bf16(a.astype(np.float32)), "f32": lambda a: a.astype(np.float32),
         "f64": lambda a: a}[kind](raw)
    out = torch.empty(*shape[:-2], shape[-2] // block, 2, dtype=torch.float64, device="cuda")
    basa.basa_block_radius(dev(x), block, out)
    torch.cuda.synchronize()
    r, m = orc.block_radius_maxnorm(x, block)
    got = host(out)
    assert np.abs(got[..., 0] - r).max() <= 1e-12 * np.abs(r).max()
    assert np.abs(got[..., 1] - m).max() <= 1e-12 * np.abs(m).max()


def _recall(idx, best):
    k = idx.shape[-1]
    hits = (idx[..., :, None] == best[..., None, :]).any(-1).sum(-1)
    return float(hits.mean()) / k


def test_recall_of_selections_against_block_mass_tiny(basa):
    note("recall of plain / ranked / Algorithm 1 selections against the block mass, tiny fp32")
    import block_sparse_attention_mean_amd.pipelines as p
    w = wl.WORKLOADS["tiny"]
    x = wl.generate("tiny")
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    cases = [
        ("plain", p.BaForward(q, k, v, w.block, w.topk, w.scale), None),
        ("ranked", p.BaRankedForward(q, k, v, w.block, w.topk, w.scale), False),
        ("algorithm1", p.BaRankedForward(q, k, v, w.block, w.topk, w.scale, beta=1.0), True),
    ]
    for name, f, comp in cases:
        if comp is None:
            f.select()
            qp, kp = q, k
            ref_q, ref_k = orc.as_f64(x["q"]), orc.as_f64(x["k"])
        else:
            f.rank()
            f.select()
            qp, kp = f.qs, f.ks
            ref_q = orc.gather_rows(orc.as_f64(x["q"]), orc.norm_rank(x["q"]))
            ref_k = orc.gather_rows(orc.as_f64(x["k"]), orc.norm_rank(x["k"]))
        mass = torch.empty(1, w.heads, w.blocks, w.blocks, dtype=torch.float64, device="cuda")
        basa.basa_block_mass(qp, kp, w.block, mass, w.scale)
        best = torch.empty(1, w.heads, w.blocks, w.topk, dtype=torch.int32, device="cuda")
        basa.basa_select_ranges(mass, w.blocks, w.topk, 0, best)
        torch.cuda.synchronize()
        got = _recall(host(f.idx), host(best))
        ref_mass = orc.block_mass(ref_q, ref_k, w.block, w.scale)
        if comp:
            sc = orc.compensated_logits(orc.pool_mean(ref_q, w.block), orc.pool_mean(ref_k, w.block),
                                        orc.block_variance(ref_q, w.block),
                                        orc.block_variance(ref_k, w.block), w.scale, 1.0)
        else:
            sc = orc.block_logits(orc.pool_mean(ref_q, w.block), orc.pool_mean(ref_k, w.block), w.scale)
        ref = orc.selection_recall(orc.topk_ascending(sc, w.topk), ref_mass)
        assert got == ref, (name, got, ref)
