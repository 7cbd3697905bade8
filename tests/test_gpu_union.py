"""The union walk of basa_attn (LoSA step's active rows, one read of each key
head's union of kept blocks) against the per-row list walk and the fp64 oracle.

Cases cover the LoSA shape (32 query heads over 8 key heads, 5 active rows,
16-key prefix blocks), grouped heads with a batch of two, head_dim 64 and
128, float32 and bf16 queries and outputs, duplicated, empty and
out-of-range list entries, a row-map entry outside q (its row must stay
untouched), and the 32-rows-per-key-head limit (beyond it the request needs no
workspace and takes the list walk).  Tolerances: float32 outputs 1e-4 on O
and LSE (float32 arithmetic on bf16 inputs); bf16 outputs one bf16 rounding."""
import math

import numpy as np
import pytest
import torch

import oracle as orc
import workloads as wl
from gpu_util import dev, host, max_err, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def basa():
    assert torch.cuda.is_available(), "the GPU tests need a visible GPU"
    import block_sparse_attention_mean_amd as mod
    return mod


def _case(seed, b, hq, hkv, t_len, prefix, d, n_rows, kept, q_f32=False):
    g = np.random.Generator(np.random.PCG64(seed))
    bf = lambda *s: wl.f32_to_bf16(g.standard_normal(s, dtype=np.float32))
    q = bf(b, hq, t_len, d)
    if q_f32:
        q = wl.bf16_to_f32(q) + np.float32(1e-3) * g.standard_normal(q.shape, dtype=np.float32)
    k, v = bf(b, hkv, prefix, d), bf(b, hkv, prefix, d)
    nb = prefix // 16
    rows = np.stack([np.sort(g.choice(t_len, n_rows, replace=False)) for _ in range(b)]).astype(np.int32)
    idx = np.sort(g.integers(0, nb, (b, hq, n_rows, kept)), axis=-1).astype(np.int32)
    return q, k, v, rows, idx, nb


def _run(basa, q, k, v, rows, idx, d, o_dtype, use_ws, o_fill=7.0):
    qt, kt, vt = dev(q), dev(k), dev(v)
    seg = basa.kv_segment(dev(idx), kt, vt)
    o = torch.full(qt.shape, o_fill, dtype=o_dtype, device="cuda")
    lse = torch.full(qt.shape[:3], o_fill, dtype=torch.float32, device="cuda")
    kw = dict(tile_q=1, block_k=16, scale=1 / math.sqrt(d), q_rows=dev(rows))
    need = basa.basa_attn_workspace(qt, seg, o, lse, **kw)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda") if (use_ws and need) else None
    basa.basa_attn(qt, seg, o, lse, workspace=ws, **kw)
    torch.cuda.synchronize()
    return host(o), host(lse), need


def _oracle(q, k, v, rows, idx, nb, d):
    ref_idx = np.where((idx >= 0) & (idx < nb), idx, -1)
    return orc.sparse_attention(q, k, v, ref_idx, 1, 16, 1 / math.sqrt(d), q_rows=rows)


CASES = [
    # seed, batch, hq, hkv, tokens, prefix, d, rows, kept, q f32, out dtype
    (1, 1, 32, 8, 16, 8192, 128, 5, 64, False, torch.float32),     # LoSA shape, smaller prefix
    (2, 2, 8, 2, 16, 4096, 64, 6, 37, True, torch.bfloat16),       # 24 rows per key head
    (3, 1, 4, 1, 32, 2048, 128, 8, 50, False, torch.bfloat16),     # 32 rows per key head
    (4, 1, 2, 2, 8, 1040, 128, 3, 9, True, torch.float32),          # a ragged last chunk (65 blocks)
]


@pytest.mark.parametrize("case", CASES)
def test_union_walk_matches_list_walk_and_oracle(basa, case):
    seed, b, hq, hkv, t_len, prefix, d, n_rows, kept, q_f32, o_dtype = case
    note(f"union walk: B{b} Hq{hq} Hkv{hkv} rows{n_rows} prefix{prefix} d{d} kept{kept} {o_dtype}")
    q, k, v, rows, idx, nb = _case(seed, b, hq, hkv, t_len, prefix, d, n_rows, kept, q_f32)
    idx[0, 0, 0, 3] = idx[0, 0, 0, 4]           # a block listed twice by one row
    idx[0, hq - 1, n_rows - 1, 0] = -1          # an empty slot
    idx[-1, 0, 1 % n_rows, kept - 1] = nb + 5   # an entry past the keys (ignored)
    ou, lu, need = _run(basa, q, k, v, rows, idx, d, o_dtype, True)
    assert need > 0
    ol, ll, _ = _run(basa, q, k, v, rows, idx, d, o_dtype, False)
    ro, rl = _oracle(q, k, v, rows, idx, nb, d)
    done = ~np.isnan(rl)
    tol_o = 1e-4 if o_dtype == torch.float32 else 2 ** -8 * np.abs(ro[done]).max() + 1e-6
    for o, lse in ((ou, lu), (ol, ll)):
        assert max_err(o[done], ro[done]) <= tol_o
        assert max_err(lse[done], rl[done]) <= 1e-4
        assert (o[~done] == 7.0).all() and (lse[~done] == 7.0).all()   # other rows untouched
    assert max_err(ou, ol) <= tol_o


def test_union_walk_row_map_entry_outside_q_is_skipped(basa):
    note("union walk: a row-map entry outside q")
    q, k, v, rows, idx, nb = _case(5, 1, 8, 2, 16, 2048, 128, 4, 20)
    rows[0, 2] = 99                              # no such query row: nothing is written for it
    ou, lu, need = _run(basa, q, k, v, rows, idx, 128, torch.float32, True)
    ol, ll, _ = _run(basa, q, k, v, rows, idx, 128, torch.float32, False)
    assert need > 0
    assert np.array_equal(np.isnan(ou), np.isnan(ol))
    assert (ou[0, :, [r for r in range(16) if r not in rows[0, [0, 1, 3]]]] == 7.0).all()
    keep = rows[0, [0, 1, 3]]
    assert max_err(ou[0, :, keep], ol[0, :, keep]) <= 1e-5
    assert max_err(lu[0, :, keep], ll[0, :, keep]) <= 1e-5


def test_union_walk_limits(basa):
    """33 rows per key head, or 32-key blocks: no workspace is asked for (list walk)."""
    q, k, v, rows, idx, nb = _case(6, 1, 33, 1, 2, 1024, 128, 1, 4)
    qt = dev(q)
    o = torch.zeros(qt.shape, dtype=torch.float32, device="cuda")
    lse = torch.zeros(qt.shape[:3], dtype=torch.float32, device="cuda")
    seg = basa.kv_segment(dev(idx), dev(k), dev(v))
    kw = dict(tile_q=1, scale=0.1, q_rows=dev(rows))
    assert basa.basa_attn_workspace(qt, seg, o, lse, block_k=16, **kw) == 0
    q, k, v, rows, idx, nb = _case(7, 1, 4, 1, 16, 1024, 128, 8, 4)
    qt = dev(q)
    o = torch.zeros(qt.shape, dtype=torch.float32, device="cuda")
    lse = torch.zeros(qt.shape[:3], dtype=torch.float32, device="cuda")
    seg = basa.kv_segment(dev(idx), dev(k), dev(v))
    kw["q_rows"] = dev(rows)
    assert basa.basa_attn_workspace(qt, seg, o, lse, block_k=16, **kw) > 0
    assert basa.basa_attn_workspace(qt, seg, o, lse, block_k=32, **kw) == 0
