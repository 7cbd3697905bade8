"""basa_select_static, the selection entry point that allocates nothing,
against basa_select with a caller-owned workspace (through the C ABI).

Both run the two-pass selection of rows with more than 1024 candidates; the
indices must be identical bit for bit.  Two calls in a row, the second with a
smaller request, show that the static scratch's leftover contents from the
first call do not leak into the second.  A request beyond the scratch's 4 MiB
is rejected on the host."""
import numpy as np
import pytest
import torch

import block_sparse_attention_mean_amd as basa
from gpu_util import host, note

pytestmark = pytest.mark.gpu


def _case(seed, hq, hkv, q_len, rows, keys, topk, d=128):
    """float64 query means [1,hq,q_len,d], transposed key means [1,hkv,d,keys]
    and a row map of `rows` query rows; every 7th key column repeats its
    neighbour so that equal scores occur."""
    g = np.random.Generator(np.random.PCG64(seed))
    q = g.standard_normal((1, hq, q_len, d))
    kt = g.standard_normal((1, hkv, d, keys))
    kt[..., 7::7] = kt[..., 6:-1:7][..., :kt[..., 7::7].shape[-1]]
    q_rows = np.sort(g.choice(q_len, rows, replace=False)).astype(np.int32)[None]
    return (torch.from_numpy(q).cuda(), torch.from_numpy(kt).cuda(),
            torch.from_numpy(q_rows).cuda(), topk)


def _both(q, kt, q_rows, topk):
    b, hq = q.shape[:2]
    rows = q_rows.shape[-1]
    ref = torch.full((b, hq, rows, topk), -7, dtype=torch.int32, device="cuda")
    got = torch.full_like(ref, -9)
    need = basa.basa_select_workspace(q, kt, ref, topk, q_rows=q_rows)
    assert need > 0, "the request must take the two-pass path"
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    basa.basa_select(q, kt, ref, topk, scale=0.1, q_rows=q_rows, workspace=ws)
    basa.basa_select_static(q, kt, got, topk, scale=0.1, q_rows=q_rows)
    torch.cuda.synchronize()
    return host(ref), host(got)


def test_static_select_matches_workspace_select_twice():
    # the LoSA prefix shape (32 query heads, 8 key heads, 5 of 16 rows, 4096 keys,
    # top-128), then a smaller request on the same scratch
    for seed, hq, hkv, rows, keys, topk in ((1, 32, 8, 5, 4096, 128), (2, 8, 2, 3, 2048, 64)):
        note(f"static select: Hq {hq} Hkv {hkv} rows {rows} keys {keys} top-{topk}")
        ref, got = _both(*_case(seed, hq, hkv, 16, rows, keys, topk))
        assert (ref >= 0).all() and (np.diff(ref, axis=-1) > 0).all()
        assert np.array_equal(got, ref)


def test_static_select_rejects_oversize_request():
    q, kt, q_rows, _ = _case(3, 32, 8, 16, 16, 4096, 256)
    idx = torch.empty(1, 32, 16, 256, dtype=torch.int32, device="cuda")
    assert basa.basa_select_workspace(q, kt, idx, 256, q_rows=q_rows) > 4 << 20
    with pytest.raises(basa.BasaError) as e:
        basa.basa_select_static(q, kt, idx, 256, scale=0.1, q_rows=q_rows)
    assert e.value.status == 2  # BASA_E_SHAPE, nothing launched
