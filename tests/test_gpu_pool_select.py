"""basa_pool_select (pooling of Q and K plus the block selection in one call)
against the separate basa_pool / basa_select calls and the fp64 oracle's
indices: query and key means bit for bit equal to basa_pool's (the float64
sums of these bf16 blocks are exact), indices equal to the separate calls'
and to the oracle's.  Each case runs twice on the same buffers.

The call enqueues the three launches itself."""
import math

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


def _bf16(g, *shape):
    return wl.f32_to_bf16(g.standard_normal(shape, dtype=np.float32))


def _run(basa, q, k, block, topk, scale, use_ws=True, reps=2):
    qt, kt = dev(q), dev(k)
    b, hq, lq, d = qt.shape
    hkv, lk = kt.shape[1], kt.shape[2]
    qbar = torch.empty(b, hq, lq // block, d, dtype=torch.float64, device="cuda")
    kbt = torch.empty(b, hkv, d, lk // block, dtype=torch.float64, device="cuda")
    idx = torch.empty(b, hq, lq // block, topk, dtype=torch.int32, device="cuda")
    ws = None
    if use_ws:
        n = basa.basa_pool_select_workspace(qt, kt, qbar, kbt, idx, topk, block=block, scale=scale)
        assert n == 0                                  # the call needs no workspace
        ws = torch.full((256,), 0x5A, dtype=torch.uint8, device="cuda")  # accepted, unused
    outs = []
    for _ in range(reps):
        basa.basa_pool_select(qt, kt, qbar, kbt, idx, topk, block=block, scale=scale, workspace=ws)
        torch.cuda.synchronize()
        outs.append((host(qbar), host(kbt), host(idx)))
    if ws is not None:
        assert bool((ws == 0x5A).all())                # left as the caller filled it
    # the separate calls
    qb2 = torch.empty_like(qbar)
    kb2 = torch.empty_like(kbt)
    ix2 = torch.empty_like(idx)
    basa.basa_pool(qt, block, mean_rows=qb2)
    basa.basa_pool(kt, block, mean_cols=kb2)
    basa.basa_select(qb2, kb2, ix2, topk, scale=scale)
    torch.cuda.synchronize()
    return outs, (host(qb2), host(kb2), host(ix2))


def _check(outs, sep, ref_idx):
    for qb, kb, ix in outs:
        assert np.array_equal(qb, sep[0]) and np.array_equal(kb, sep[1])
        assert np.array_equal(ix, sep[2])
        assert np.array_equal(ix, ref_idx)


def test_pool_select_dlm64k(basa):
    note("pool_select dlm64k: H32 L65536 block128 top128")
    w = wl.WORKLOADS["dlm64k"]
    x = wl.generate("dlm64k")
    outs, sep = _run(basa, x["q"], x["k"], w.block, w.topk, w.scale)
    ref = orc.topk_ascending(orc.block_logits(orc.pool_mean(x["q"], w.block),
                                              orc.pool_mean(x["k"], w.block), w.scale), w.topk)
    _check(outs, sep, ref)


def test_pool_select_ragged_groups(basa):
    # 1000 query blocks per head (not a multiple of the selection's 16-row groups), 6 query
    # heads over 3 key heads, blocks of 2 rows
    note("pool_select ragged: Hq6 Hkv3, 1000 query blocks, 512 key blocks of 2, d64 top37")
    g = np.random.Generator(np.random.PCG64(83))
    q, k = _bf16(g, 1, 6, 2000, 64), _bf16(g, 1, 3, 1024, 64)
    outs, sep = _run(basa, q, k, 2, 37, 0.125)
    ref = orc.topk_ascending(orc.block_logits(orc.pool_mean(q, 2), orc.pool_mean(k, 2), 0.125), 37)
    _check(outs, sep, ref)


@pytest.mark.parametrize("b,hq,hkv,tokens,block,d,topk", [
    (2, 4, 2, 16384, 32, 128, 100),   # grouped heads, a batch of two, 512 blocks of 32
    (1, 2, 1, 8192, 16, 64, 128),     # head_dim 64, 512 blocks of 16
    (1, 3, 3, 16384, 128, 128, 64),   # 128 key blocks: the separate launches
    (1, 2, 2, 65536, 128, 128, 1),    # top-1
])
def test_pool_select_shapes(basa, b, hq, hkv, tokens, block, d, topk):
    note(f"pool_select B{b} Hq{hq} Hkv{hkv} L{tokens} block{block} d{d} top{topk}")
    g = np.random.Generator(np.random.PCG64(71 + hq + d))
    q, k = _bf16(g, b, hq, tokens, d), _bf16(g, b, hkv, tokens, d)
    scale = 1 / math.sqrt(d)
    outs, sep = _run(basa, q, k, block, topk, scale)
    ref = orc.topk_ascending(orc.block_logits(orc.pool_mean(q, block), orc.pool_mean(k, block),
                                              scale), topk)
    _check(outs, sep, ref)


def test_pool_select_without_workspace(basa):
    note("pool_select with no workspace argument")
    g = np.random.Generator(np.random.PCG64(79))
    q, k = _bf16(g, 1, 2, 16384, 128), _bf16(g, 1, 2, 16384, 128)
    outs, sep = _run(basa, q, k, 32, 50, 0.1, use_ws=False, reps=1)
    ref = orc.topk_ascending(orc.block_logits(orc.pool_mean(q, 32), orc.pool_mean(k, 32), 0.1), 50)
    _check(outs, sep, ref)
