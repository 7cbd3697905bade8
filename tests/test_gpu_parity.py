"""HIP path against the fp64 oracle, element by element, through the C ABI.

Indices must match bit for bit; O within 2e-2 and LSE within 1e-3 (max abs)
for bf16 inputs with float32 accumulation, and tighter where the inputs are
float32.  Attention tests take their key lists from the oracle's selection,
never from the HIP path.
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
def basa():
    assert torch.cuda.is_available(), "the GPU tests need a visible GPU"
    import block_sparse_attention_mean_amd as mod
    return mod


def gpu_pool(basa, x, block, rows=True, cols=False, copy=None):
    xt = dev(x)
    *lead, length, d = xt.shape
    nb = length // block
    out_rows = torch.empty(*lead, nb, d, dtype=torch.float64, device="cuda") if rows else None
    out_cols = torch.empty(*lead, d, nb, dtype=torch.float64, device="cuda") if cols else None
    out_copy = torch.empty(*lead, nb, d, dtype=copy, device="cuda") if copy is not None else None
    basa.basa_pool(xt, block, out_rows, out_cols, out_copy)
    torch.cuda.synchronize()
    return out_rows, out_cols, out_copy


def gpu_select(basa, q, k, block, topk, scale):
    """pool Q (rows) and K (transposed), then select: the BA-Att selection stage."""
    qbar, _, _ = gpu_pool(basa, q, block)
    _, kbt, _ = gpu_pool(basa, k, block, rows=False, cols=True)
    b, h, nq, _ = qbar.shape
    idx = torch.empty(b, h, nq, topk, dtype=torch.int32, device="cuda")
    basa.basa_select(qbar, kbt, idx, topk, scale=scale)
    torch.cuda.synchronize()
    return host(idx)


def oracle_select(q, k, block, topk, scale):
    return orc.topk_ascending(orc.block_logits(orc.pool_mean(q, block), orc.pool_mean(k, block),
                                               scale), topk)


# --------------------------------------------------------------------------- pool

def test_pool_bf16_exact_and_transposed(basa):
    note("pool bf16 H4 L2048 d128 block128")
    x = wl.make_dlm(11, heads=4, tokens=2048, head_dim=128)["q"]
    r, c, _ = gpu_pool(basa, x, 128, rows=True, cols=True)
    ref = orc.pool_mean(x, 128)
    assert np.array_equal(host(r), ref)                 # exact: bf16 sums are exact in float64
    assert np.array_equal(host(c), np.swapaxes(ref, -1, -2))


def test_pool_f32_and_block_one(basa):
    note("pool f32 tiny block64 / block1")
    x = wl.make_tiny(5)["k"]
    r, _, _ = gpu_pool(basa, x, 64)
    ref = orc.pool_mean(x, 64)
    assert max_err(host(r), ref) <= 1e-15 * np.abs(ref).max()
    r1, _, _ = gpu_pool(basa, x, 1)
    assert np.array_equal(host(r1), x.astype(np.float64))


def test_pool_f64_levels_and_copies(basa):
    note("pool f64 level input block16 d64 with f32/bf16 copies")
    g = np.random.Generator(np.random.PCG64(12))
    x = g.standard_normal((1, 3, 4096, 64))
    r, _, c32 = gpu_pool(basa, x, 16, copy=torch.float32)
    ref = orc.pool_mean(x, 16)
    assert max_err(host(r), ref) <= 4e-16 * 16
    assert np.array_equal(host(c32), ref.astype(np.float32).astype(np.float64))
    _, _, c16 = gpu_pool(basa, x, 16, rows=False, copy=torch.bfloat16)
    got = host(c16)
    # nearest bf16: within half a bf16 ulp of the float64 mean
    ulp = 2.0 ** (np.floor(np.log2(np.abs(ref))) - 7)
    assert np.all(np.abs(got - ref) <= 0.5 * ulp * (1 + 1e-12))


def _pyramid_inputs(case):
    g = np.random.Generator(np.random.PCG64(31))
    if case == "bf16_llsa":      # the log-linear shape: Q, K, V, block 16, three levels
        x = wl.make_dlm(31, heads=3, tokens=16 ** 3, head_dim=64)
        return [x["q"], x["k"], x["v"]], 16, 3, torch.float32
    if case == "bf16_copies":    # bf16 copies, two levels, block 8, head_dim 128
        x = wl.make_dlm(32, heads=2, tokens=8 * 8 * 6, head_dim=128)
        return [x["k"], x["v"]], 8, 2, torch.bfloat16
    if case == "bf16_wide":       # block 32 x head_dim 128: 512 items for 256 threads per workgroup
        x = wl.make_dlm(34, heads=2, tokens=32 * 32 * 3, head_dim=128)
        return [x["q"], x["k"]], 32, 2, torch.float32
    if case == "bf16_one_level":  # one level: the plain pooling call per tensor
        x = wl.make_dlm(33, heads=2, tokens=512, head_dim=64)
        return [x["q"], x["k"], x["v"]], 32, 1, torch.float32
    if case == "f32_ragged":     # float32, block 8 (a partial batch of rows in flight), outer 4
        return [g.standard_normal((2, 2, 8 * 8 * 5, 24)).astype(np.float32)], 8, 2, torch.float32
    # float64, block 4, four levels, head_dim 8
    return [g.standard_normal((1, 1, 4 ** 4 * 3, 8)), g.standard_normal((1, 1, 4 ** 4 * 3, 8))], 4, 4, \
        torch.float32


@pytest.mark.parametrize("case", ["bf16_llsa", "bf16_copies", "bf16_wide", "bf16_one_level",
                                  "f32_ragged", "f64_four_levels"])
def test_pool_pyramid_equals_chained_pooling(basa, case):
    """basa_pool_pyramid against basa_pool applied level by level (level l from the float64
    rows of level l - 1): every output identical bit for bit.  For bf16 inputs every level also
    equals the oracle's pooled means exactly (float64 sums of bf16 values are exact)."""
    note(f"pool pyramid {case}")
    xs, block, levels, copy_dt = _pyramid_inputs(case)
    ts = [dev(x) for x in xs]
    *lead, length, d = ts[0].shape
    outs, refs = [], []
    for i, t in enumerate(ts):
        lv_out, lv_ref, src = [], [], t
        for lv in range(1, levels + 1):
            nb = length // block ** lv
            def mk():
                rows = torch.empty(*lead, nb, d, dtype=torch.float64, device="cuda")
                cols = torch.empty(*lead, d, nb, dtype=torch.float64, device="cuda") \
                    if i != 0 or lv == levels else None
                copy = torch.empty(*lead, nb, d, dtype=copy_dt, device="cuda") if i != 0 else None
                return rows, cols, copy
            o, r = mk(), mk()
            for buf in (*o, *r):
                if buf is not None:
                    buf.fill_(float("nan"))
            basa.basa_pool(src, block, *r)
            lv_out.append(o)
            lv_ref.append(r)
            src = r[0]
        outs.append(lv_out)
        refs.append(lv_ref)
    basa.basa_pool_pyramid(ts, block, outs)
    torch.cuda.synchronize()
    for i in range(len(ts)):
        ref_mean = xs[i]
        for lv in range(levels):
            for got, want in zip(outs[i][lv], refs[i][lv]):
                if got is not None:
                    assert torch.equal(got, want), (case, i, lv)
            if case.startswith("bf16"):
                ref_mean = orc.pool_mean(ref_mean, block)
                assert np.array_equal(host(outs[i][lv][0]), ref_mean)


# --------------------------------------------------------------------------- select

def test_select_tiny_planted_block(basa):
    note("select tiny fp32 (planted block)")
    w = wl.WORKLOADS["tiny"]
    x = wl.generate("tiny")
    got = gpu_select(basa, x["q"], x["k"], w.block, w.topk, w.scale)
    ref = oracle_select(x["q"], x["k"], w.block, w.topk, w.scale)
    assert np.array_equal(got, ref)
    for h in range(w.heads):
        assert wl.TINY_PLANT_KEY_BLOCK in got[0, h, wl.TINY_PLANT_QUERY_BLOCK]


def test_select_ragged_rows_and_keys(basa):
    note("select ragged: H3 rows37 keys100 top7 d64")
    g = np.random.Generator(np.random.PCG64(14))
    q = g.standard_normal((1, 3, 37 * 16, 64)).astype(np.float32)
    k = g.standard_normal((1, 3, 100 * 16, 64)).astype(np.float32)
    got = gpu_select(basa, q, k, 16, 7, 0.125)
    assert np.array_equal(got, oracle_select(q, k, 16, 7, 0.125))


def test_select_exact_ties_go_to_lower_index(basa):
    note("select ties: duplicated key blocks and an all-zero query block")
    g = np.random.Generator(np.random.PCG64(15))
    q = g.standard_normal((1, 2, 20 * 16, 64)).astype(np.float32)
    k = g.standard_normal((1, 2, 150 * 16, 64)).astype(np.float32)
    k[:, :, 16 * 90:16 * 91] = k[:, :, 16 * 3:16 * 4]     # identical blocks -> equal scores
    k[:, :, 16 * 120:16 * 121] = k[:, :, 16 * 3:16 * 4]
    q[:, :, 0:16] = 0.0                                    # every score of row 0 ties at zero
    q[:, 1, 16:32] = -0.0
    for topk in (1, 5, 64, 150):
        got = gpu_select(basa, q, k, 16, topk, 0.125)
        ref = oracle_select(q, k, 16, topk, 0.125)
        assert np.array_equal(got, ref), topk
    assert np.array_equal(got[0, 0, 0], np.arange(150))


@pytest.mark.parametrize("ties,keys,workspace", [(False, 4096, False), (True, 4096, False),
                                                  (False, 4096, True), (True, 4096, True),
                                                  (False, 3000, True)])
def test_select_gqa_row_map_and_wide_rows(basa, ties, keys, workspace):
    # more than 1024 candidates: one pass without a workspace, two passes (parts of
    # 512 keys, then a merge) with one; the result must not depend on the path
    note(f"select GQA 8/2 heads, row map, {keys} keys (top-128), ties={ties}, workspace={workspace}")
    g = np.random.Generator(np.random.PCG64(16))
    qf = g.standard_normal((1, 8, 16, 128))
    kbar = g.standard_normal((1, 2, keys, 128))
    if ties:  # 64 distinct key rows repeated: equal scores across quarters and parts
        kbar = np.tile(kbar[:, :, :64], (1, 1, keys // 64, 1))
    rows = np.array([[1, 4, 7, 10, 13]], dtype=np.int32)
    idx = torch.empty(1, 8, 5, 128, dtype=torch.int32, device="cuda")
    qt, kt = dev(qf), dev(np.ascontiguousarray(np.swapaxes(kbar, -1, -2)))
    ws = None
    if workspace:
        n = basa.basa_select_workspace(qt, kt, idx, 128, q_rows=dev(rows))
        assert n == 8 * 5 * ((keys + 511) // 512) * 128 * 12
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    basa.basa_select(qt, kt, idx, 128, scale=1 / math.sqrt(128), q_rows=dev(rows), workspace=ws)
    torch.cuda.synchronize()
    ref = orc.topk_ascending(orc.block_logits(qf[:, :, rows[0]], kbar, 1 / math.sqrt(128)), 128)
    assert np.array_equal(host(idx), ref)


@pytest.mark.parametrize("keys,d,row_map", [(300, 64, False), (512, 128, False), (449, 128, True),
                                             (512, 64, True)])
def test_select_channel_split_rows(basa, keys, d, row_map):
    # 257..511 candidates run the channel-split kernel, exactly 512 the LDS-staged
    # one: 37 rows (ragged last groups), GQA 4/2, duplicated key columns and an
    # all-zero query row
    note(f"select channel-split: {keys} keys, d {d}, row map {row_map}, ties")
    g = np.random.Generator(np.random.PCG64(18 + keys))
    q_len = 40 if row_map else 37
    qf = g.standard_normal((1, 4, q_len, d))
    qf[0, 1, 5] = 0.0
    kbar = g.standard_normal((1, 2, keys, d))
    kbar[:, :, 200] = kbar[:, :, 7]
    kbar[:, :, 250] = kbar[:, :, 7]
    rows = None
    if row_map:
        rows = np.sort(g.choice(q_len, 37, replace=False))[None].astype(np.int32)
        rows[0, 3] = 5
    idx = torch.empty(1, 4, 37, 64, dtype=torch.int32, device="cuda")
    basa.basa_select(dev(qf), dev(np.ascontiguousarray(np.swapaxes(kbar, -1, -2))), idx, 64,
                     scale=1 / math.sqrt(d), q_rows=dev(rows) if row_map else None)
    torch.cuda.synchronize()
    qsel = qf[:, :, rows[0]] if row_map else qf
    ref = orc.topk_ascending(orc.block_logits(qsel, kbar, 1 / math.sqrt(d)), 64)
    assert np.array_equal(host(idx), ref)


@pytest.mark.parametrize("case", ["tiled", "wide_range", "infinite"])
def test_select_512_threshold_search(basa, case):
    # 512 candidates run the matrix-core kernel (scores exchanged through LDS, then
    # the bit search for the threshold): equal scores in groups of 8 on both sides
    # of every threshold, scores spread over hundreds of binades, and rows holding
    # +inf and -inf scores (40 rows: two full 16-row groups and a ragged one)
    note(f"select 512 keys, threshold search: {case}")
    g = np.random.Generator(np.random.PCG64(31))
    qf = g.standard_normal((1, 2, 40, 128))
    kbar = g.standard_normal((1, 2, 512, 128))
    if case == "tiled":
        kbar = np.tile(kbar[:, :, :64], (1, 1, 8, 1))
    elif case == "wide_range":
        kbar *= np.exp(g.uniform(-300.0, 300.0, size=(1, 2, 512, 1)))
    else:
        qf[:, :, :, 0] = 4.0
        kbar[:, :, 5, 0] = 1e308
        kbar[:, :, 9, 0] = -1e308
        kbar[:, :, 300, 0] = 1e308
    qt, kt = dev(qf), dev(np.ascontiguousarray(np.swapaxes(kbar, -1, -2)))
    for topk in (1, 60, 64, 128, 200, 511):
        out = torch.empty(1, 2, 40, topk, dtype=torch.int32, device="cuda")
        basa.basa_select(qt, kt, out, topk, scale=1 / math.sqrt(128))
        torch.cuda.synchronize()
        with np.errstate(over="ignore"):  # the planted scores overflow to +-inf on purpose
            ref = orc.topk_ascending(orc.block_logits(qf, kbar, 1 / math.sqrt(128)), topk)
        assert np.array_equal(host(out), ref), topk
    if case == "infinite":
        with np.errstate(over="ignore"):
            assert np.isinf(orc.block_logits(qf, kbar, 1.0)[..., [5, 9]]).all()


@pytest.mark.parametrize("d,row_map", [(32, True), (64, False), (128, True)])
def test_select_512_batches_groups_and_row_map(basa, d, row_map):
    # the 512-candidate kernel with batch 2, 6 query heads over 3 key heads, 21
    # rows (one full 16-row group and a ragged one) and a row map that repeats
    # and skips query rows; head_dim 32 gives 8 chunks of 4 channels
    note(f"select 512 keys: batch 2, GQA 6/3, 21 rows, d {d}, row map {row_map}")
    g = np.random.Generator(np.random.PCG64(40 + d))
    q_len = 30 if row_map else 21
    qf = g.standard_normal((2, 6, q_len, d))
    kbar = g.standard_normal((2, 3, 512, d))
    rows = None
    if row_map:
        rows = np.stack([np.sort(g.choice(q_len, 21, replace=False)) for _ in range(2)]).astype(np.int32)
        rows[1, 4] = rows[1, 3]
    idx = torch.empty(2, 6, 21, 64, dtype=torch.int32, device="cuda")
    basa.basa_select(dev(qf), dev(np.ascontiguousarray(np.swapaxes(kbar, -1, -2))), idx, 64,
                     scale=1 / math.sqrt(d), q_rows=dev(rows) if row_map else None)
    torch.cuda.synchronize()
    qsel = np.stack([qf[b][:, rows[b]] for b in range(2)]) if row_map else qf
    ref = orc.topk_ascending(orc.block_logits(qsel, kbar, 1 / math.sqrt(d)), 64)
    assert np.array_equal(host(idx), ref)


@pytest.mark.parametrize("seed", range(8))
def test_select_512_random_shapes(basa, seed):
    # seeded shapes for the 512-candidate kernel: head_dim 8..512 (multiples of 8),
    # batch 1-3, 1-4 key heads with 1-3 query heads each, 1-70 rows, top-k 1-512,
    # with and without a row map
    g = np.random.Generator(np.random.PCG64(500 + seed))
    d = int(g.choice([8, 16, 24, 40, 64, 96, 128, 256, 512]))
    batch, hkv, group = int(g.integers(1, 4)), int(g.integers(1, 5)), int(g.integers(1, 4))
    rows, topk, row_map = int(g.integers(1, 71)), int(g.integers(1, 513)), bool(g.integers(0, 2))
    note(f"select 512 keys random shape {seed}: B{batch} Hkv{hkv} g{group} rows {rows} d {d} "
         f"top-{topk} row map {row_map}")
    q_len = rows + 7 if row_map else rows
    qf = g.standard_normal((batch, hkv * group, q_len, d))
    kbar = g.standard_normal((batch, hkv, 512, d))
    rmap = None
    if row_map:
        rmap = np.stack([g.integers(0, q_len, rows) for _ in range(batch)]).astype(np.int32)
    idx = torch.empty(batch, hkv * group, rows, topk, dtype=torch.int32, device="cuda")
    basa.basa_select(dev(qf), dev(np.ascontiguousarray(np.swapaxes(kbar, -1, -2))), idx, topk,
                     scale=1 / math.sqrt(d), q_rows=dev(rmap) if row_map else None)
    torch.cuda.synchronize()
    qsel = np.stack([qf[b][:, rmap[b]] for b in range(batch)]) if row_map else qf
    ref = orc.topk_ascending(orc.block_logits(qsel, kbar, 1 / math.sqrt(d)), topk)
    assert np.array_equal(host(idx), ref)


def test_select_children_of_parent_picks(basa):
    note("select candidate mode: 256 rows, parent top-8 x fanout 16")
    g = np.random.Generator(np.random.PCG64(17))
    nq = nk = 256
    q = g.standard_normal((1, 2, nq, 64))
    kbar = g.standard_normal((1, 2, nk, 64))
    parent = np.sort(np.stack([np.stack([g.choice(16, 8, replace=False) for _ in range(16)])
                               for _ in range(2)])[None], axis=-1).astype(np.int32)
    idx = torch.empty(1, 2, nq, 8, dtype=torch.int32, device="cuda")
    basa.basa_select(dev(q), dev(np.ascontiguousarray(np.swapaxes(kbar, -1, -2))), idx, 8,
                     scale=0.125, parent=dev(parent), fanout=16)
    torch.cuda.synchronize()
    got = host(idx)
    for h in range(2):
        for a in range(nq):
            cands = (parent[0, h, a // 16][:, None] * 16 + np.arange(16)).reshape(-1)
            s = 0.125 * (kbar[0, h, cands] @ q[0, h, a])
            assert np.array_equal(got[0, h, a], cands[orc.topk_ascending(s, 8)])


def test_select_change_mode(basa):
    note("select change mode: LoSA active tokens")
    x = wl.make_losa(4, heads_q=32, heads_kv=8, prefix=256, head_dim=128)
    idx = torch.empty(1, 5, dtype=torch.int32, device="cuda")
    basa.basa_select(dev(x["q_cur"]), dev(x["q_prev"]), idx, 5, mode=basa.SELECT_CHANGE)
    torch.cuda.synchronize()
    ref = orc.active_tokens(x["q_cur"], x["q_prev"], 5)
    assert np.array_equal(host(idx), ref)
    assert host(idx).tolist() == [list(wl.LOSA_PLANTED)]
    idx2 = torch.empty(1, 5, dtype=torch.int32, device="cuda")
    basa.basa_select(dev(x["q_cur"]), dev(x["q_cur"]), idx2, 5, mode=basa.SELECT_CHANGE)
    torch.cuda.synchronize()
    assert host(idx2).tolist() == [[0, 1, 2, 3, 4]]    # all changes tie at zero


def test_select_dlm16k_full(basa):
    note("select dlm16k full: H32 L16384 block128 top64")
    w = wl.WORKLOADS["dlm16k"]
    x = wl.generate("dlm16k")
    got = gpu_select(basa, x["q"], x["k"], w.block, w.topk, w.scale)
    assert np.array_equal(got, oracle_select(x["q"], x["k"], w.block, w.topk, w.scale))


# --------------------------------------------------------------------------- attention

def run_attn(basa, q, segs, tile_q, block_k, scale, o_dtype, q_rows=None, o_init=None, lse_init=None,
             workspace=False):
    """segs: list of (idx np, k np, v np, kwargs).  workspace: pass the one
    basa_attn_workspace asks for (filled with 0x5A, not zeroed)."""
    qt = dev(q)
    segments = [basa.kv_segment(dev(i), dev(k), dev(v), **kw) for i, k, v, kw in segs]
    o = (dev(o_init) if o_init is not None else
         torch.zeros(qt.shape, dtype=o_dtype, device="cuda"))
    lse = (dev(lse_init) if lse_init is not None else
           torch.zeros(qt.shape[:3], dtype=torch.float32, device="cuda"))
    rows = dev(q_rows) if q_rows is not None else None
    ws = None
    if workspace:
        n = basa.basa_attn_workspace(qt, segments, o, lse, tile_q=tile_q, block_k=block_k, scale=scale,
                                     q_rows=rows)
        assert n > 0
        ws = torch.full((n,), 0x5A, dtype=torch.uint8, device="cuda")
    basa.basa_attn(qt, segments, o, lse, tile_q=tile_q, block_k=block_k, scale=scale, q_rows=rows,
                   workspace=ws)
    torch.cuda.synchronize()
    return host(o), host(lse)


@pytest.mark.parametrize("o_dtype", [torch.bfloat16, torch.float32])
def test_attn_mfma_small_with_empty_slots(basa, o_dtype):
    note(f"attn mfma H3 L1152 kept5 with empty slots, out {o_dtype}")
    x = wl.make_dlm(21, heads=3, tokens=1152, head_dim=128)
    g = np.random.Generator(np.random.PCG64(22))
    nb = 9
    idx = np.stack([np.stack([np.sort(g.choice(nb, 5, replace=False)) for _ in range(nb)])
                    for _ in range(3)])[None].astype(np.int32)
    idx[0, 0, 2, 1] = -1
    idx[0, 2, 8, :] = -1                                   # an empty list
    idx[0, 1, 4, 4] = -1
    o, lse = run_attn(basa, x["q"], [(idx, x["k"], x["v"], {})], 128, 128, 1 / math.sqrt(128), o_dtype)
    ro, rl = orc.sparse_attention(x["q"], x["k"], x["v"], idx, 128, 128, 1 / math.sqrt(128))
    empty = np.zeros(ro.shape[:3], dtype=bool)
    empty[0, 2, 8 * 128:] = True
    assert np.all(o[empty] == 0) and np.all(np.isneginf(lse[empty]))
    assert max_err(o[~empty], ro[~empty]) <= O_TOL
    assert max_err(lse[~empty], rl[~empty]) <= LSE_TOL


def test_attn_mfma_batch2_gqa(basa):
    # the MFMA kernel with two batch entries and grouped key heads (4 query heads on
    # 2 key heads), lists of different lengths padded with -1
    note("attn mfma: batch 2, GQA 4/2, L 1024, kept 3 of 8 with padding")
    g = np.random.Generator(np.random.PCG64(29))
    q = wl.f32_to_bf16(g.standard_normal((2, 4, 1024, 128)).astype(np.float32))
    k = wl.f32_to_bf16(g.standard_normal((2, 2, 1024, 128)).astype(np.float32))
    v = wl.f32_to_bf16(g.standard_normal((2, 2, 1024, 128)).astype(np.float32))
    idx = np.sort(np.stack([np.stack([np.stack([g.choice(8, 3, replace=False) for _ in range(8)])
                                      for _ in range(4)]) for _ in range(2)]), axis=-1).astype(np.int32)
    idx[1, 3, 7, 0] = -1
    idx[0, 1, 2, 2] = -1
    o, lse = run_attn(basa, q, [(idx, k, v, {})], 128, 128, 1 / math.sqrt(128), torch.bfloat16)
    ro, rl = orc.sparse_attention(q, k, v, idx, 128, 128, 1 / math.sqrt(128))
    eo, el = max_err(o, ro), max_err(lse, rl)
    assert eo <= O_TOL, eo
    assert el <= LSE_TOL, el


@pytest.mark.parametrize("tokens,heads", [(2048, 2), (65536, 1)])
def test_attn_mfma_all_blocks_is_dense_attention(basa, tokens, heads):
    # keeping every key block is dense bidirectional attention (BA-Att section 2,
    # Eq. 1), checked against the oracle's dense attention; at 65536 tokens the
    # list has 512 entries, the largest the 64K-token shape can have
    note(f"attn mfma: all {tokens // 128} blocks kept == dense attention, {heads} head(s)")
    g = np.random.Generator(np.random.PCG64(30))
    x = wl.make_dlm(31, heads=heads, tokens=tokens, head_dim=128)
    nb = tokens // 128
    idx = np.broadcast_to(np.arange(nb, dtype=np.int32), (1, heads, nb, nb)).copy()
    o, lse = run_attn(basa, x["q"], [(idx, x["k"], x["v"], {})], 128, 128, 1 / math.sqrt(128),
                      torch.float32)
    if tokens > 4096:  # sampled query rows (the oracle's dense attention is O(L^2))
        rows = np.sort(g.choice(tokens, 256, replace=False))
        ro, rl = orc.dense_attention(x["q"][:, :, rows], x["k"], x["v"], 1 / math.sqrt(128))
        o, lse = o[:, :, rows], lse[:, :, rows]
    else:
        ro, rl = orc.dense_attention(x["q"], x["k"], x["v"], 1 / math.sqrt(128))
    eo, el = max_err(o, ro), max_err(lse, rl)
    assert eo <= O_TOL, eo
    assert el <= LSE_TOL, el


@pytest.mark.parametrize("rising", [True, False])
def test_attn_mfma_rising_logits_raise_the_reference_max(basa, rising):
    # key blocks scaled by growing factors: walking a list in ascending order meets
    # logits far above the first block's max, so the kernel must raise its reference
    # max, rescale O and redo stages (several times per row); the descending case
    # starts at the largest logits and never has to
    note(f"attn mfma: key blocks scaled 1..20, rising={rising}")
    g = np.random.Generator(np.random.PCG64(33))
    heads, tokens, nb = 2, 2048, 16
    factor = np.array([1, 1, 2, 3, 5, 8, 12, 16, 20, 4, 1, 6, 2, 9, 14, 18], dtype=np.float32)
    if not rising:
        factor = factor[::-1].copy()
    q = wl.f32_to_bf16(g.standard_normal((1, heads, tokens, 128)).astype(np.float32))
    kf = g.standard_normal((1, heads, tokens, 128)).astype(np.float32)
    k = wl.f32_to_bf16(kf * np.repeat(factor, 128)[None, None, :, None])
    v = wl.f32_to_bf16(g.standard_normal((1, heads, tokens, 128)).astype(np.float32))
    idx = np.sort(np.stack([np.stack([g.choice(nb, 7, replace=False) for _ in range(nb)])
                            for _ in range(heads)]), axis=-1)[None].astype(np.int32)
    idx[0, 0, 3] = np.arange(9, dtype=np.int32)[:7]       # a row walking factors 1, 1, 2, .., 12
    o, lse = run_attn(basa, q, [(idx, k, v, {})], 128, 128, 1 / math.sqrt(128), torch.float32)
    ro, rl = orc.sparse_attention(q, k, v, idx, 128, 128, 1 / math.sqrt(128))
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    eo, el = max_err(o, ro), max_err(lse, rl)
    assert eo <= O_TOL, eo
    assert el <= LSE_TOL, el


def test_attn_mfma_dlm16k_stratified_and_deterministic(basa):
    note("attn mfma dlm16k: oracle lists, every 8th tile of every head (512), repeat-run bitwise")
    w = wl.WORKLOADS["dlm16k"]
    x = wl.generate("dlm16k")
    idx = oracle_select(x["q"], x["k"], w.block, w.topk, w.scale)
    o, lse = run_attn(basa, x["q"], [(idx, x["k"], x["v"], {})], 128, 128, w.scale, torch.bfloat16)
    o2, lse2 = run_attn(basa, x["q"], [(idx, x["k"], x["v"], {})], 128, 128, w.scale, torch.bfloat16)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    tiles = stratified_tiles(w.heads, w.blocks)
    assert len(tiles) == 512
    eo, el = check_tiles_against_oracle(o, lse, x["q"], x["k"], x["v"], idx, tiles, 128, 128, w.scale)
    note(f"dlm16k 512 tiles: O err {eo:.2e}, LSE err {el:.2e}")
    assert eo <= O_TOL and el <= LSE_TOL


@pytest.mark.parametrize("case", ["batch2_gqa_padded", "odd_lists", "dlm16k"])
def test_attn_mfma_tile_order_changes_no_bit(basa, case):
    # With a workspace the MFMA path ranks each head's query tiles by the middle
    # entry of their lists and runs them in that order; each tile is computed
    # the same way wherever it runs, so O and LSE must match the natural order
    # bit for bit (lists with -1 slots, a -1 at the middle slot, an unsorted
    # list, an odd number of tiles per head, and the 16K workload's lists).
    note(f"attn mfma tile order: {case}, with and without the workspace")
    scale = 1 / math.sqrt(128)
    g = np.random.Generator(np.random.PCG64(31))
    if case == "dlm16k":
        w = wl.WORKLOADS["dlm16k"]
        x = wl.generate("dlm16k")
        q, k, v = x["q"], x["k"], x["v"]
        idx = oracle_select(q, k, w.block, w.topk, w.scale)
        scale = w.scale
    else:
        b, hq, hkv, nb, kept = (2, 4, 2, 8, 3) if case == "batch2_gqa_padded" else (1, 3, 3, 9, 5)
        q = wl.f32_to_bf16(g.standard_normal((b, hq, nb * 128, 128)).astype(np.float32))
        k = wl.f32_to_bf16(g.standard_normal((b, hkv, nb * 128, 128)).astype(np.float32))
        v = wl.f32_to_bf16(g.standard_normal((b, hkv, nb * 128, 128)).astype(np.float32))
        idx = np.sort(g.random((b, hq, nb, nb)).argsort(-1)[..., :kept], axis=-1).astype(np.int32)
        idx[0, 1, 2, kept // 2] = -1                        # the ranking key slot is empty
        idx[-1, -1, -1, 0] = -1
        idx[0, 0, 1] = idx[0, 0, 1][::-1]                   # a list in descending order
    o1, l1 = run_attn(basa, q, [(idx, k, v, {})], 128, 128, scale, torch.bfloat16)
    o2, l2 = run_attn(basa, q, [(idx, k, v, {})], 128, 128, scale, torch.bfloat16, workspace=True)
    assert np.isfinite(o1).all() and np.isfinite(l1).all()   # no list is empty here
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)  # host() widens exactly


def test_attn_generic_tiny_fp32(basa):
    note("attn generic tiny fp32 full")
    w = wl.WORKLOADS["tiny"]
    x = wl.generate("tiny")
    idx = oracle_select(x["q"], x["k"], w.block, w.topk, w.scale)
    o, lse = run_attn(basa, x["q"], [(idx, x["k"], x["v"], {})], 64, 64, w.scale, torch.float32)
    ro, rl = orc.sparse_attention(x["q"], x["k"], x["v"], idx, 64, 64, w.scale)
    assert max_err(o, ro) <= 1e-5
    assert max_err(lse, rl) <= 1e-5


@pytest.mark.parametrize("tile_q", [16, 7, 32, 1])
def test_attn_segments_bias_and_f32_tables(basa, tile_q):
    note(f"attn segments: bf16 fine + f32 coarse tables, shifts, level bias, d64 tile {tile_q}")
    g = np.random.Generator(np.random.PCG64(24 + tile_q))
    d, blk = 64, 16
    tiles = 64
    n = tile_q * tiles
    n_keys = 1024
    q = wl.f32_to_bf16(g.standard_normal((1, 2, n, d)).astype(np.float32))
    kf = wl.f32_to_bf16(g.standard_normal((1, 2, n_keys, d)).astype(np.float32))
    vf = wl.f32_to_bf16(g.standard_normal((1, 2, n_keys, d)).astype(np.float32))
    k1 = g.standard_normal((1, 2, 64, d)).astype(np.float32)
    v1 = g.standard_normal((1, 2, 64, d)).astype(np.float32)
    i0 = np.sort(g.integers(0, n_keys // blk, (1, 2, tiles, 8)), axis=-1).astype(np.int32)
    i0[0, 1, 5, 3] = -1                                   # an empty slot
    i1 = np.sort(g.integers(0, 64 // blk, (1, 2, tiles >> 4, 3)), axis=-1).astype(np.int32)
    i2 = np.zeros((1, 2, 1, 1), dtype=np.int32)
    b1, b2 = math.log(16), 2 * math.log(16)
    segs = [(i0, kf, vf, {}), (i1, k1, v1, {"shift": 4, "bias": b1}),
            (i2, k1, v1, {"shift": 10, "bias": b2})]
    o, lse = run_attn(basa, q, segs, tile_q, blk, 0.125, torch.float32)
    # oracle: one table [fine | coarse] with per-entry bias
    kt = np.concatenate([orc.as_f64(kf), k1.astype(np.float64)], axis=2)
    vt = np.concatenate([orc.as_f64(vf), v1.astype(np.float64)], axis=2)
    off = n_keys // blk
    full = np.concatenate([i0, np.where(np.repeat(i1, 16, axis=2) >= 0, np.repeat(i1, 16, axis=2) + off, -1),
                           np.repeat(i2, tiles, axis=2) + off], axis=-1)
    bias = np.concatenate([np.zeros(i0.shape), np.full(i1.shape[:2] + (tiles, 3), b1),
                           np.full(i2.shape[:2] + (tiles, 1), b2)], axis=-1)
    ro, rl = orc.sparse_attention(q, kt, vt, full, tile_q, blk, 0.125, bias=bias)
    # 16-row tiles run on bf16 MFMA (P rounded to bf16): the bf16 bar; the other
    # tile sizes run in float32 throughout
    o_tol, lse_tol = (O_TOL, LSE_TOL) if tile_q == 16 else (1e-4, 1e-4)
    eo, el = max_err(o, ro), max_err(lse, rl)
    assert eo <= o_tol, eo
    assert el <= lse_tol, el


def test_attn_16_row_tiles_workgroup_size_changes_no_bit(basa):
    # 64 lists per head run 8 tiles per workgroup (the float32 lists of shift >= 3 staged
    # once per 8 tiles); the same first 60 tiles as a problem of their own run 4 per
    # workgroup.  Each tile walks the same blocks in the same order either way.
    note("attn 16-row tiles: 8 against 4 tiles per workgroup, d64")
    g = np.random.Generator(np.random.PCG64(29))
    d, tiles, nk = 64, 64, 1024
    q = wl.f32_to_bf16(g.standard_normal((1, 2, tiles * 16, d)).astype(np.float32))
    kb = wl.f32_to_bf16(g.standard_normal((1, 2, nk, d)).astype(np.float32))
    vb = wl.f32_to_bf16(g.standard_normal((1, 2, nk, d)).astype(np.float32))
    kf = g.standard_normal((1, 2, 256, d)).astype(np.float32)
    vf = g.standard_normal((1, 2, 256, d)).astype(np.float32)
    i0 = np.sort(g.integers(0, nk // 16, (1, 2, tiles, 8)), axis=-1).astype(np.int32)
    i0[0, 1, 7, 2] = -1
    i1 = np.sort(g.integers(0, 16, (1, 2, tiles >> 4, 8)), axis=-1).astype(np.int32)
    i2 = np.zeros((1, 2, 1, 1), dtype=np.int32)
    segs = lambda n: [(i0[:, :, :n], kb, vb, {}),
                      (i1[:, :, :(n + 15) // 16], kf, vf, {"shift": 4, "bias": math.log(16)}),
                      (i2, kf, vf, {"shift": 12, "bias": 2 * math.log(16)})]
    o16, l16 = run_attn(basa, q, segs(tiles), 16, 16, 0.125, torch.bfloat16)
    o4, l4 = run_attn(basa, q[:, :, :60 * 16], segs(60), 16, 16, 0.125, torch.bfloat16)
    assert np.array_equal(o16[:, :, :60 * 16], o4)
    assert np.array_equal(l16[:, :, :60 * 16], l4)


@pytest.mark.parametrize("d,row_map", [(128, False), (128, True), (64, True)])
def test_attn_16_row_tiles_f32_tables_row_map(basa, d, row_map):
    # 16-row tiles over 16-key blocks run the tile MFMA kernel: a bf16 segment and a
    # float32 segment with a bias, GQA 4/2, empty slots, optionally a row map, bf16 out
    note(f"attn 16-row tiles: d {d}, row map {row_map}, bf16 + f32 tables")
    g = np.random.Generator(np.random.PCG64(27 + d + row_map))
    n_q, tiles, nk = 320, 12, 512
    q = wl.f32_to_bf16(g.standard_normal((1, 4, n_q, d)).astype(np.float32))
    kb = wl.f32_to_bf16(g.standard_normal((1, 2, nk, d)).astype(np.float32))
    vb = wl.f32_to_bf16(g.standard_normal((1, 2, nk, d)).astype(np.float32))
    kf = g.standard_normal((1, 2, 64, d)).astype(np.float32)
    vf = g.standard_normal((1, 2, 64, d)).astype(np.float32)
    i0 = np.sort(g.integers(0, nk // 16, (1, 4, tiles, 6)), axis=-1).astype(np.int32)
    i0[0, 2, 3, 1] = -1
    i1 = np.sort(g.integers(0, 4, (1, 4, tiles, 3)), axis=-1).astype(np.int32)
    i1[0, 1, 5, :] = -1                                   # a segment list with no block
    rows = None
    if row_map:
        rows = np.stack([np.sort(g.choice(n_q, tiles * 16, replace=False))])[None][0].astype(np.int32)
    else:
        q = q[:, :, :tiles * 16]
    b1 = math.log(16)
    segs = [(i0, kb, vb, {}), (i1, kf, vf, {"bias": b1})]
    o, lse = run_attn(basa, q, segs, 16, 16, 1 / math.sqrt(d), torch.bfloat16, q_rows=rows)
    kt = np.concatenate([orc.as_f64(kb), kf.astype(np.float64)], axis=2)
    vt = np.concatenate([orc.as_f64(vb), vf.astype(np.float64)], axis=2)
    full = np.concatenate([i0, np.where(i1 >= 0, i1 + nk // 16, -1)], axis=-1)
    bias = np.concatenate([np.zeros(i0.shape), np.full(i1.shape, b1)], axis=-1)
    ro, rl = orc.sparse_attention(q, kt, vt, full, 16, 16, 1 / math.sqrt(d), bias=bias, q_rows=rows)
    sel = ~np.isnan(rl)
    assert sel.sum() == 4 * tiles * 16
    eo, el = max_err(o[sel], ro[sel]), max_err(lse[sel], rl[sel])
    assert eo <= O_TOL, eo
    assert el <= LSE_TOL, el


@pytest.mark.parametrize("block_k", [16, 8])
def test_attn_single_rows_row_map_gqa_keeps_other_rows(basa, block_k):
    # block 16 runs the single-row kernel, block 8 the general one
    note(f"attn tile 1, q_rows, GQA 8/2, block {block_k}, top-8, in-place rows")
    g = np.random.Generator(np.random.PCG64(25))
    d = 128
    q = wl.f32_to_bf16(g.standard_normal((1, 8, 16, d)).astype(np.float32))
    k = wl.f32_to_bf16(g.standard_normal((1, 2, 1024, d)).astype(np.float32))
    v = wl.f32_to_bf16(g.standard_normal((1, 2, 1024, d)).astype(np.float32))
    rows = np.array([[1, 4, 7, 10, 13]], dtype=np.int32)
    nblk = 1024 // block_k
    idx = np.sort(np.stack([np.stack([g.choice(nblk, 8, replace=False) for _ in range(5)])
                            for _ in range(8)])[None], axis=-1).astype(np.int32)
    idx[0, 3, 2, 5] = -1                                  # an empty slot
    o0 = g.standard_normal((1, 8, 16, d)).astype(np.float32)
    l0 = g.standard_normal((1, 8, 16)).astype(np.float32)
    o, lse = run_attn(basa, q, [(idx, k, v, {})], 1, block_k, 1 / math.sqrt(d), torch.float32,
                      q_rows=rows, o_init=o0, lse_init=l0)
    ro, rl = orc.sparse_attention(q, k, v, idx, 1, block_k, 1 / math.sqrt(d), q_rows=rows)
    act = np.zeros((1, 8, 16), dtype=bool)
    act[:, :, rows[0]] = True
    assert max_err(o[act], ro[act]) <= 1e-4 and max_err(lse[act], rl[act]) <= 1e-4
    assert np.array_equal(o[~act], o0[~act].astype(np.float64))
    assert np.array_equal(lse[~act], l0[~act].astype(np.float64))


@pytest.mark.parametrize("block_k,d", [(16, 128), (32, 128), (48, 64)])
def test_attn_single_rows_long_lists(basa, block_k, d):
    # lists longer than 64 entries per wave share, several 16-key steps per
    # entry, empty slots and one all-empty list; bf16 out
    note(f"attn tile 1 long lists: block {block_k}, d {d}, 600 entries, GQA 8/2")
    g = np.random.Generator(np.random.PCG64(26 + block_k))
    nblk = 1200
    q = wl.f32_to_bf16(g.standard_normal((1, 8, 3, d)).astype(np.float32))
    k = wl.f32_to_bf16(g.standard_normal((1, 2, nblk * block_k, d)).astype(np.float32))
    v = wl.f32_to_bf16(g.standard_normal((1, 2, nblk * block_k, d)).astype(np.float32))
    idx = np.sort(np.stack([np.stack([g.choice(nblk, 600, replace=False) for _ in range(3)])
                            for _ in range(8)])[None], axis=-1).astype(np.int32)
    idx[0, 1, 0, ::7] = -1
    idx[0, 6, 2, :] = -1
    scale = 1 / math.sqrt(d)
    o, lse = run_attn(basa, q, [(idx, k, v, {})], 1, block_k, scale, torch.bfloat16)
    ro, rl = orc.sparse_attention(q, k, v, idx, 1, block_k, scale)
    empty = np.zeros((1, 8, 3), dtype=bool)
    empty[0, 6, 2] = True
    assert np.all(o[empty] == 0) and np.all(np.isneginf(lse[empty]))
    assert max_err(o[~empty], ro[~empty]) <= O_TOL
    assert max_err(lse[~empty], rl[~empty]) <= LSE_TOL


@pytest.mark.parametrize("case", ["chunked_key_heads", "two_dim_grid"])
def test_attn_single_rows_xcd_chunks(basa, case):
    # The single-row kernel cuts the rows into chunks of up to 64 consecutive rows and
    # runs chunk c on XCD c % 8: 150 rows per key head (chunks that end inside a key
    # head, a padded last round) checked in full; 72,000 rows (a two-dimensional grid)
    # checked on 256 sampled rows.
    note(f"attn tile 1 XCD chunks: {case}")
    g = np.random.Generator(np.random.PCG64(37))
    if case == "chunked_key_heads":
        b, hq, hkv, lq, d, nblk, count = 2, 6, 2, 50, 128, 64, 6
    else:
        b, hq, hkv, lq, d, nblk, count = 1, 2, 1, 36000, 64, 32, 2
    q = wl.f32_to_bf16(g.standard_normal((b, hq, lq, d)).astype(np.float32))
    k = wl.f32_to_bf16(g.standard_normal((b, hkv, nblk * 16, d)).astype(np.float32))
    v = wl.f32_to_bf16(g.standard_normal((b, hkv, nblk * 16, d)).astype(np.float32))
    idx = np.sort(g.random((b, hq, lq, nblk)).argsort(-1)[..., :count], axis=-1).astype(np.int32)
    scale = 1 / math.sqrt(d)
    o, lse = run_attn(basa, q, [(idx, k, v, {})], 1, 16, scale, torch.float32)
    if case == "chunked_key_heads":
        ro, rl = orc.sparse_attention(q, k, v, idx, 1, 16, scale)
        assert max_err(o, ro) <= 1e-4 and max_err(lse, rl) <= 1e-4
    else:
        rows = np.sort(g.choice(lq, 256, replace=False)).astype(np.int32)[None]
        ro, rl = orc.sparse_attention(q, k, v, idx[:, :, rows[0]], 1, 16, scale, q_rows=rows)
        assert max_err(o[:, :, rows[0]], ro[:, :, rows[0]]) <= 1e-4
        assert max_err(lse[:, :, rows[0]], rl[:, :, rows[0]]) <= 1e-4
        assert np.isfinite(lse).all()


# --------------------------------------------------------------------------- merge

@pytest.mark.parametrize("in_dt,out_dt", [(torch.float32, torch.bfloat16), (torch.bfloat16, torch.float32),
                                          (torch.float32, torch.float32)])
def test_merge_matches_oracle(basa, in_dt, out_dt):
    note(f"merge {in_dt}->{out_dt}")
    g = np.random.Generator(np.random.PCG64(26))
    rows, d = 1000, 128
    oa = g.standard_normal((rows, d)).astype(np.float32)
    ob = g.standard_normal((rows, d)).astype(np.float32)
    la = (3 * g.standard_normal(rows)).astype(np.float32)
    lb = (3 * g.standard_normal(rows)).astype(np.float32)
    la[:10] = -np.inf
    lb[5:15] = -np.inf                                  # rows 5..9 are empty on both sides
    if in_dt == torch.bfloat16:
        oa, ob = wl.bf16_to_f32(wl.f32_to_bf16(oa)), wl.bf16_to_f32(wl.f32_to_bf16(ob))
    toa, tob = dev(oa).to(in_dt), dev(ob).to(in_dt)
    o = torch.empty(rows, d, dtype=out_dt, device="cuda")
    lse = torch.empty(rows, dtype=torch.float32, device="cuda")
    basa.basa_merge(toa, dev(la), tob, dev(lb), o, lse)
    torch.cuda.synchronize()
    ro, rl = orc.merge(oa, la, ob, lb)
    tol = 2e-2 if out_dt == torch.bfloat16 else 1e-5
    assert max_err(host(o), ro) <= tol
    assert max_err(host(lse), rl) <= 1e-5
    assert np.all(host(o)[5:10] == 0) and np.all(np.isneginf(host(lse)[5:10]))


def test_merge_in_place(basa):
    note("merge in place f32")
    g = np.random.Generator(np.random.PCG64(27))
    oa = g.standard_normal((300, 64)).astype(np.float32)
    ob = g.standard_normal((300, 64)).astype(np.float32)
    la = g.standard_normal(300).astype(np.float32)
    lb = g.standard_normal(300).astype(np.float32)
    toa, tla = dev(oa), dev(la)
    basa.basa_merge(toa, tla, dev(ob), dev(lb), toa, tla)
    torch.cuda.synchronize()
    ro, rl = orc.merge(oa, la, ob, lb)
    assert max_err(host(toa), ro) <= 1e-5 and max_err(host(tla), rl) <= 1e-5


@pytest.mark.parametrize("kept", [128, 129, 130])
def test_attn_mfma_list_length_boundary(basa, kept):
    """Lists of up to 128 blocks are held in VGPRs, longer ones read from LDS:
    both sides of the boundary, with repeated and unused entries."""
    note(f"attn mfma: kept {kept} of 256 blocks, 1 head, L 32768")
    x = wl.make_dlm(43, heads=1, tokens=32768, head_dim=128)
    nb, scale = 256, 1 / math.sqrt(128)
    g = np.random.Generator(np.random.PCG64(44 + kept))
    idx = np.sort(g.integers(0, nb, (1, 1, nb, kept)), axis=-1).astype(np.int32)  # repeats allowed
    idx[0, 0, 5, 0] = -1
    idx[0, 0, 9, kept - 1] = nb + 1
    o, lse = run_attn(basa, x["q"], [(idx, x["k"], x["v"], {})], 128, 128, scale, torch.bfloat16)
    tiles = [0, 5, 9, 100, 255]
    ro, rl = orc.sparse_attention(x["q"], x["k"], x["v"], np.where(idx >= nb, -1, idx), 128, 128, scale,
                                  lists=[(0, 0, t) for t in tiles])
    sel = ~np.isnan(rl)
    assert max_err(o[sel], ro[sel]) <= O_TOL
    assert max_err(lse[sel], rl[sel]) <= LSE_TOL


# ------------------------------------------------------------- C++ reference

def test_ba_path_matches_cpp_reference(basa):
    """Selection, block-sparse attention and a two-part merge on a DLM-shaped
    case, every row against the fp64 C++ reference (oracle/basa_oracle_ref.cpp)."""
    import oracle.cref as cref
    note("BA path H2 L4096 d128 top-8 against the C++ reference")
    x = wl.make_dlm(41, heads=2, tokens=4096, head_dim=128)
    block, topk, scale = 128, 8, 1 / math.sqrt(128)
    ref_idx = cref.topk_ascending(cref.block_logits(cref.pool_mean(x["q"], block),
                                                    cref.pool_mean(x["k"], block), scale), topk)
    assert np.array_equal(gpu_select(basa, x["q"], x["k"], block, topk, scale), ref_idx)
    o, lse = run_attn(basa, x["q"], [(ref_idx, x["k"], x["v"], {})], 128, 128, scale, torch.bfloat16)
    ro, rl = cref.sparse_attention(x["q"], x["k"], x["v"], ref_idx, 128, 128, scale)
    assert max_err(o, ro) <= O_TOL
    assert max_err(lse, rl) <= LSE_TOL
    # halves of every list as float32 partials, merged on the GPU and by the reference
    oa, la = run_attn(basa, x["q"], [(ref_idx, x["k"], x["v"], {"count": 4})], 128, 128, scale,
                      torch.float32)
    ob, lb = run_attn(basa, x["q"], [(ref_idx, x["k"], x["v"], {"offset": 4, "count": 4})], 128, 128,
                      scale, torch.float32)
    om = torch.empty(o.shape, dtype=torch.bfloat16, device="cuda")
    lm = torch.empty(lse.shape, dtype=torch.float32, device="cuda")
    f32 = lambda a: dev(a.astype(np.float32))  # the partials were float32 (read back widened)
    basa.basa_merge(f32(oa), f32(la), f32(ob), f32(lb), om, lm)
    torch.cuda.synchronize()
    rmo, rml = cref.merge(oa, la, ob, lb)
    assert max_err(host(om), rmo) <= O_TOL and max_err(host(lm), rml) <= 1e-5
    assert max_err(host(om), ro) <= O_TOL and max_err(host(lm), rl) <= LSE_TOL


def test_attn_mfma_longest_list(basa):
    """The largest list the MFMA path takes: 1023 of 1024 key blocks (131072
    keys), every stage's block index read from the LDS copy of the list; one
    head, sampled tiles against the oracle."""
    note("attn mfma: kept 1023 of 1024 blocks, 1 head, L 131072")
    x = wl.make_dlm(45, heads=1, tokens=131072, head_dim=128)
    nb, kept, scale = 1024, 1023, 1 / math.sqrt(128)
    g = np.random.Generator(np.random.PCG64(46))
    idx = np.stack([np.sort(g.permutation(nb)[:kept]) for _ in range(nb)]).astype(np.int32)[None, None]
    o, lse = run_attn(basa, x["q"], [(idx, x["k"], x["v"], {})], 128, 128, scale, torch.bfloat16)
    tiles = [0, 511, 1023]
    ro, rl = orc.sparse_attention(x["q"], x["k"], x["v"], idx, 128, 128, scale,
                                  lists=[(0, 0, t) for t in tiles])
    sel = ~np.isnan(rl)
    assert sel.sum() == 3 * 128
    assert max_err(o[sel], ro[sel]) <= O_TOL
    assert max_err(lse[sel], rl[sel]) <= LSE_TOL
