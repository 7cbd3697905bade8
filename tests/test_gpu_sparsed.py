"""Dense block mass (BA-Att Eq. 3; SparseD's average-pooled attention scores)
and SparseD's isolated top-rho% selection (SparseD section 3.3, Eq. 5-6) on
the HIP path against the fp64 oracle, through the C ABI.

The block mass is float64 on both sides (they add in different orders):
within 1e-12 relative.  Range selections on identical scores and the whole
SparseD pattern must match bit for bit; attention under the pattern within
2e-2 (O) and 1e-3 (LSE) for bf16 inputs, 1e-5 for float32.
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


def gpu_mass(basa, q, k, block, scale, one_pass=False):
    """one_pass: give the call the workspace basa_block_mass_workspace asks for
    (filled with 0x5A, not zeroed); shapes outside the one-pass kernel get none."""
    qt, kt = dev(q), dev(k)
    b, h, lq, _ = qt.shape
    m = torch.empty(b, h, lq // block, kt.shape[2] // block, dtype=torch.float64, device="cuda")
    ws = None
    if one_pass:
        n = basa.basa_block_mass_workspace(qt, kt, block)
        if n > 0:
            ws = torch.full((n,), 0x5A, dtype=torch.uint8, device="cuda")
    basa.basa_block_mass(qt, kt, block, m, scale, workspace=ws)
    torch.cuda.synchronize()
    return host(m)


def rel_err(a, b):
    return float(np.abs(a - b).max() / np.abs(b).max())


@pytest.mark.parametrize("one_pass", [False, True])
@pytest.mark.parametrize("kind,hq,hkv,length,d,block", [
    ("f32", 2, 2, 1024, 64, 64), ("bf16", 3, 3, 2048, 128, 128), ("bf16", 4, 2, 1024, 64, 32),
    ("bf16", 1, 1, 512, 128, 16), ("f32", 1, 1, 256, 8, 4), ("f32", 2, 1, 512, 64, 16),
    ("bf16", 2, 2, 256, 24, 32), ("f32", 1, 1, 128, 8, 16)])
def test_block_mass_matches_oracle(basa, kind, hq, hkv, length, d, block, one_pass):
    note(f"block mass {kind} H{hq}/{hkv} L{length} d{d} block{block} one pass {one_pass}")
    g = np.random.Generator(np.random.PCG64(length + d + block))
    q = g.standard_normal((1, hq, length, d)) * g.uniform(0.5, 2.0, (1, hq, length, 1))
    k = g.standard_normal((1, hkv, length, d))
    conv = (lambda a: wl.f32_to_bf16(a.astype(np.float32))) if kind == "bf16" else (lambda a: a.astype(np.float32))
    q, k = conv(q), conv(k)
    scale = 1.0 / np.sqrt(d)
    got = gpu_mass(basa, q, k, block, scale, one_pass)
    ref = orc.block_mass(q, k, block, scale)
    assert rel_err(got, ref) < 1e-12
    assert np.abs(got.sum(axis=-1) - 1.0).max() < 1e-12


@pytest.mark.parametrize("block", [128, 16])
def test_block_mass_one_pass_large_logits_and_two_pass(basa, block):
    # rows scaled so that logits reach several hundred (each key block's own max
    # keeps the sums finite), keys with one planted block per head: the one-pass
    # form against the oracle and against the two-pass form
    note(f"block mass one pass, large logits, block {block}")
    g = np.random.Generator(np.random.PCG64(77 + block))
    d, length = 128, 2048
    q = g.standard_normal((1, 2, length, d)) * g.uniform(1.0, 60.0, (1, 2, length, 1))
    k = g.standard_normal((1, 2, length, d))
    k[0, :, 5 * block:6 * block] += 3.0 * q[0, :, :block].mean(axis=1, keepdims=True) / 60.0
    q, k = wl.f32_to_bf16(q.astype(np.float32)), wl.f32_to_bf16(k.astype(np.float32))
    scale = 1.0 / np.sqrt(d)
    one = gpu_mass(basa, q, k, block, scale, one_pass=True)
    two = gpu_mass(basa, q, k, block, scale, one_pass=False)
    ref = orc.block_mass(q, k, block, scale)
    assert np.isfinite(one).all()
    assert rel_err(one, ref) < 1e-12 and rel_err(one, two) < 1e-12
    assert np.abs(one.sum(axis=-1) - 1.0).max() < 1e-12


@pytest.mark.parametrize("n,split,k_lo,k_hi", [(37, 10, 3, 5), (128, 64, 20, 20), (512, 0, 0, 100),
                                              (1000, 1000, 7, 0), (64, 63, 63, 1)])
def test_select_ranges_matches_oracle_with_ties(basa, n, split, k_lo, k_hi):
    note(f"select ranges n{n} split{split} k{k_lo}+{k_hi}")
    g = np.random.Generator(np.random.PCG64(n + split))
    s = np.round(g.standard_normal((2, 3, 33, n)), 1)  # many exact ties
    s[0, 0, 0, :] = 0.0
    st = dev(s)
    idx = torch.empty(2, 3, 33, k_lo + k_hi, dtype=torch.int32, device="cuda")
    basa.basa_select_ranges(st, split, k_lo, k_hi, idx)
    torch.cuda.synchronize()
    assert np.array_equal(host(idx), orc.topk_in_ranges(s, split, k_lo, k_hi))


def test_sparsed_pattern_and_attention_tiny_fp32(basa):
    note("SparseD pattern + attention tiny fp32 (prefill 512, rho 0.25)")
    import block_sparse_attention_mean_amd.pipelines as p
    w = wl.WORKLOADS["tiny"]
    x = wl.generate("tiny")
    f = p.SparsedForward(dev(x["q"]), dev(x["k"]), dev(x["v"]), w.block, 512, 0.25, w.scale)
    f.run()
    torch.cuda.synchronize()
    idx, ro, rl = orc.sparsed_forward(x["q"], x["k"], x["v"], w.block, w.scale, 512, 0.25)
    assert np.array_equal(host(f.idx), idx)
    assert max_err(host(f.o), ro) <= 1e-5
    assert max_err(host(f.lse), rl) <= 1e-5


def test_sparsed_pattern_dlm16k_sampled_heads(basa):
    note("SparseD pattern dlm16k (prefill 8192, rho 0.3): 3 heads against the oracle, reuse")
    import block_sparse_attention_mean_amd.pipelines as p
    w = wl.WORKLOADS["dlm16k"]
    x = wl.generate("dlm16k")
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    f = p.SparsedForward(q, k, v, w.block, 8192, 0.3, w.scale)
    f.run()
    torch.cuda.synchronize()
    assert (f.k_lo, f.k_hi) == (20, 20)
    idx, mass, o, lse = host(f.idx), host(f.mass), host(f.o), host(f.lse)
    for h in (0, 17, 31):
        sl = slice(h, h + 1)
        ref_mass = orc.block_mass(x["q"][:, sl], x["k"][:, sl], w.block, w.scale)
        assert rel_err(mass[:, sl], ref_mass) < 1e-12, h
        ref_idx = orc.topk_in_ranges(ref_mass, 64, 20, 20)
        assert np.array_equal(idx[:, sl], ref_idx), h
        for t in (0, 63, 64, 127):
            rows = slice(t * w.block, (t + 1) * w.block)
            ro, rl = orc.attend_rows(x["q"][0, h, rows], x["k"][0, h], x["v"][0, h], ref_idx[0, 0, t],
                                     w.block, w.scale)
            assert max_err(o[0, h, rows], ro) <= O_TOL, (h, t)
            assert max_err(lse[0, h, rows], rl) <= LSE_TOL, (h, t)
    # a later step reuses the pattern with new q, k, v
    v2 = dev(wl.f32_to_bf16(np.full(x["v"].shape, 0.5, dtype=np.float32)))
    f.attend(q, k, v2)
    torch.cuda.synchronize()
    assert np.abs(host(f.o) - 0.5).max() == 0.0
