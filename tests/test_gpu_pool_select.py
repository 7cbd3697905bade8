"""basa_pool_select (pooling of Q and K plus the block selection in one call)
against the separate basa_pool / basa_select calls and the fp64 oracle's
indices: query and key means bit for bit equal to basa_pool's, indices to the
oracle's.  Each case runs twice on the same workspace.

The single-launch form of the call is switched off in the library (its first
GPU run did not finish in 180 s; the cause is not shown), so the call runs the
three separate launches and these cases test that form.  The 64K case, the one
that stalled under the single launch, stays skipped until that form's cause is
found and it is switched back on."""
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


def _run(basa, q, k, block, topk, scale, use_ws=True, reps=2, single_launch=False):
    qt, kt = dev(q), dev(k)
    b, hq, lq, d = qt.shape
    hkv, lk = kt.shape[1], kt.shape[2]
    qbar = torch.empty(b, hq, lq // block, d, dtype=torch.float64, device="cuda")
    kbt = torch.empty(b, hkv, d, lk // block, dtype=torch.float64, device="cuda")
    idx = torch.empty(b, hq, lq // block, topk, dtype=torch.int32, device="cuda")
    ws = None
    if use_ws:
        n = basa.basa_pool_select_workspace(qt, kt, qbar, kbt, idx, topk, block=block, scale=scale)
        ws = torch.full((n,), 0x5A, dtype=torch.uint8, device="cuda")   # not zeroed by the caller
    outs = []
    for _ in range(reps):
        basa.basa_pool_select(qt, kt, qbar, kbt, idx, topk, block=block, scale=scale, workspace=ws)
        torch.cuda.synchronize()
        outs.append((host(qbar), host(kbt), host(idx)))
    # the wait-bound flag exists only in the single launch's workspace; the
    # separate launches leave the workspace as the caller filled it
    flag = int(ws.view(torch.int32)[1].item()) if single_launch else 0
    # the separate calls
    qb2 = torch.empty_like(qbar)
    kb2 = torch.empty_like(kbt)
    ix2 = torch.empty_like(idx)
    basa.basa_pool(qt, block, mean_rows=qb2)
    basa.basa_pool(kt, block, mean_cols=kb2)
    basa.basa_select(qb2, kb2, ix2, topk, scale=scale)
    torch.cuda.synchronize()
    return outs, (host(qb2), host(kb2), host(ix2)), flag


def _check(outs, sep, flag, ref_idx):
    assert flag == 0
    for qb, kb, ix in outs:
        assert np.array_equal(qb, sep[0]) and np.array_equal(kb, sep[1])
        assert np.array_equal(ix, sep[2])
        assert np.array_equal(ix, ref_idx)


@pytest.mark.skip(reason="the single-launch pool+select stalled on this case (no result in 180 s, "
                         "cause not shown); it is switched off and this case waits for its fix")
def test_pool_select_dlm64k(basa):
    note("pool_select dlm64k: H32 L65536 block128 top128, one launch")
    w = wl.WORKLOADS["dlm64k"]
    x = wl.generate("dlm64k")
    outs, sep, flag = _run(basa, x["q"], x["k"], w.block, w.topk, w.scale, single_launch=True)
    ref = orc.topk_ascending(orc.block_logits(orc.pool_mean(x["q"], w.block),
                                              orc.pool_mean(x["k"], w.block), w.scale), w.topk)
    _check(outs, sep, flag, ref)


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
    outs, sep, flag = _run(basa, q, k, block, topk, scale)
    ref = orc.topk_ascending(orc.block_logits(orc.pool_mean(q, block), orc.pool_mean(k, block),
                                              scale), topk)
    _check(outs, sep, flag, ref)


def test_pool_select_without_workspace(basa):
    note("pool_select without a workspace: the separate launches")
    g = np.random.Generator(np.random.PCG64(79))
    q, k = _bf16(g, 1, 2, 16384, 128), _bf16(g, 1, 2, 16384, 128)
    outs, sep, flag = _run(basa, q, k, 32, 50, 0.1, use_ws=False, reps=1)
    ref = orc.topk_ascending(orc.block_logits(orc.pool_mean(q, 32), orc.pool_mean(k, 32), 0.1), 50)
    _check(outs, sep, flag, ref)
