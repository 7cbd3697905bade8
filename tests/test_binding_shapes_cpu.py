"""The Python binding checks every tensor's shape against the sizes it passes
to the C ABI, before it takes any device pointer (CPU, no GPU needed).

The C functions receive bare pointers: a tensor of the wrong size would make a
kernel read or write out of bounds.  Each case below gives CPU tensors with
one wrong shape and expects the shape error; the control cases give correct
shapes and get as far as the device check ("must live on the GPU"), which
shows the shape checks run first."""
import pytest
import torch

import block_sparse_attention_mean_amd as basa

f32, f64, bf16, i32 = torch.float32, torch.float64, torch.bfloat16, torch.int32
ON_GPU = "must live on the GPU"


def z(*shape, dtype=f32):
    return torch.zeros(*shape, dtype=dtype)


def shape_error(fn, *a, **kw):
    with pytest.raises(ValueError) as e:
        fn(*a, **kw)
    assert ON_GPU not in str(e.value), str(e.value)
    return str(e.value)


def reaches_device_check(fn, *a, **kw):
    with pytest.raises(ValueError, match=ON_GPU):
        fn(*a, **kw)


# ------------------------------------------------------------------ pool

def test_pool_outputs():
    x = z(1, 2, 256, 64, dtype=bf16)
    reaches_device_check(basa.basa_pool, x, 64, mean_rows=z(1, 2, 4, 64, dtype=f64),
                         mean_cols=z(1, 2, 64, 4, dtype=f64))
    shape_error(basa.basa_pool, x, 64, mean_rows=z(1, 2, 8, 64, dtype=f64))
    shape_error(basa.basa_pool, x, 64, mean_cols=z(1, 2, 4, 64, dtype=f64))
    shape_error(basa.basa_pool, x, 64, mean_copy=z(1, 2, 4, 32))


def test_pool_pyramid_outputs():
    xs = [z(1, 2, 4096, 64, dtype=bf16) for _ in range(3)]

    def outs(l1_rows=(1, 2, 256, 64), l2_cols=(1, 2, 64, 16)):
        return [[(z(*l1_rows, dtype=f64), None, z(1, 2, 256, 64)),
                 (z(1, 2, 16, 64, dtype=f64), z(*l2_cols, dtype=f64), None)] for _ in range(3)]
    reaches_device_check(basa.basa_pool_pyramid, xs, 16, outs())
    shape_error(basa.basa_pool_pyramid, xs, 16, outs(l1_rows=(1, 2, 255, 64)))   # level-1 rows
    shape_error(basa.basa_pool_pyramid, xs, 16, outs(l2_cols=(1, 2, 16, 64)))    # level-2 layout
    shape_error(basa.basa_pool_pyramid, [xs[0], z(1, 2, 2048, 64, dtype=bf16)], 16, outs()[:2])
    shape_error(basa.basa_pool_pyramid, xs, 16, [outs()[0], outs()[1][:1], outs()[2]])  # levels
    mixed = outs()
    mixed[1][0] = (mixed[1][0][0], None, z(1, 2, 256, 64, dtype=bf16))             # copy dtypes
    shape_error(basa.basa_pool_pyramid, xs, 16, mixed)
    shape_error(basa.basa_pool_pyramid, xs * 2, 16, outs() * 2)                    # six tensors


# ---------------------------------------------------------------- select

def sel_args(hq=4, hkv=2, nq=8, nk=16, d=64, topk=4):
    return z(1, hq, nq, d, dtype=f64), z(1, hkv, d, nk, dtype=f64), z(1, hq, nq, topk, dtype=i32)


def test_select_blocks_shapes():
    q, k, idx = sel_args()
    reaches_device_check(basa.basa_select, q, k, idx, 4)
    shape_error(basa.basa_select, q, k, idx, 5)                         # topk != idx width
    shape_error(basa.basa_select, q, k, z(1, 4, 7, 4, dtype=i32), 4)    # rows != q_len
    shape_error(basa.basa_select, q, z(1, 2, 32, 16, dtype=f64), idx, 4)  # head_dim
    shape_error(basa.basa_select, q, z(2, 2, 64, 16, dtype=f64), idx, 4)  # batch
    shape_error(basa.basa_select, q, k, idx, 4, keys=32)                # keys beyond k
    shape_error(basa.basa_select, q, k, z(1, 3, 8, 4, dtype=i32), 4)    # heads


def test_select_row_map_and_parent_shapes():
    q, k, _ = sel_args()
    idx = z(1, 4, 3, 4, dtype=i32)
    reaches_device_check(basa.basa_select, q, k, idx, 4, q_rows=z(1, 3, dtype=i32))
    shape_error(basa.basa_select, q, k, idx, 4, q_rows=z(1, 5, dtype=i32))
    q, k, idx = sel_args(nq=32, nk=64)
    reaches_device_check(basa.basa_select, q, k, idx, 4, parent=z(1, 4, 2, 2, dtype=i32), fanout=16)
    shape_error(basa.basa_select, q, k, idx, 4, parent=z(1, 4, 1, 2, dtype=i32), fanout=16)
    shape_error(basa.basa_select, q, k, idx, 4, parent=z(1, 2, 2, 2, dtype=i32), fanout=16)


def test_select_change_shapes():
    q = z(1, 4, 16, 64, dtype=bf16)
    reaches_device_check(basa.basa_select, q, q.clone(), z(1, 5, dtype=i32), 5,
                         mode=basa.SELECT_CHANGE)
    shape_error(basa.basa_select, q, z(1, 4, 15, 64, dtype=bf16), z(1, 5, dtype=i32), 5,
                mode=basa.SELECT_CHANGE)
    shape_error(basa.basa_select, q, q.clone(), z(1, 4, dtype=i32), 5, mode=basa.SELECT_CHANGE)


def test_select_index_dtype():
    q, k, _ = sel_args()
    with pytest.raises(TypeError):
        basa.basa_select(q, k, z(1, 4, 8, 4, dtype=torch.int64), 4)


# ------------------------------------------------------------------ attn

def attn_args(hq=4, hkv=2, lq=512, lk=1024, d=128, kept=3):
    q = z(1, hq, lq, d, dtype=bf16)
    kv = z(1, hkv, lk, d, dtype=bf16)
    idx = z(1, hq, lq // 128, kept, dtype=i32)
    return q, kv, idx, z(1, hq, lq, d, dtype=bf16), z(1, hq, lq)


def test_attn_shapes():
    q, kv, idx, o, lse = attn_args()
    seg = basa.kv_segment(idx, kv, kv.clone())
    kw = dict(tile_q=128, block_k=128, scale=0.1)
    reaches_device_check(basa.basa_attn, q, seg, o, lse, **kw)
    shape_error(basa.basa_attn, q, seg, z(1, 4, 256, 128, dtype=bf16), lse, **kw)
    shape_error(basa.basa_attn, q, seg, o, z(1, 4, 511), **kw)
    shape_error(basa.basa_attn, q, basa.kv_segment(z(1, 4, 3, 3, dtype=i32), kv, kv.clone()),
                o, lse, **kw)                                           # too few index rows
    shape_error(basa.basa_attn, q, basa.kv_segment(z(1, 2, 4, 3, dtype=i32), kv, kv.clone()),
                o, lse, **kw)                                           # index heads
    kv64 = z(1, 2, 1024, 64, dtype=bf16)
    shape_error(basa.basa_attn, q, basa.kv_segment(idx, kv64, kv64.clone()), o, lse, **kw)
    kv3 = z(1, 3, 1024, 128, dtype=bf16)
    shape_error(basa.basa_attn, q, [seg, basa.kv_segment(idx, kv3, kv3.clone())], o, lse, **kw)
    shape_error(basa.basa_attn, q, seg, o, lse, tile_q=100, block_k=128, scale=0.1)


def test_attn_row_map_shapes():
    q, kv, _, o, lse = attn_args(lq=16)
    sel = z(1, 4, 5, 8, dtype=i32)
    seg = basa.kv_segment(sel, kv, kv.clone())
    kw = dict(tile_q=1, block_k=16, scale=0.1)
    reaches_device_check(basa.basa_attn, q, seg, o, lse, q_rows=z(1, 5, dtype=i32), **kw)
    shape_error(basa.basa_attn, q, seg, o, lse, q_rows=z(2, 5, dtype=i32), **kw)
    shape_error(basa.basa_attn, q, seg, o, lse, q_rows=z(1, 6, dtype=i32), **kw)


# ----------------------------------------------------------------- merge

def test_merge_shapes():
    oa, la = z(3, 10, 64), z(3, 10)
    reaches_device_check(basa.basa_merge, oa, la, oa.clone(), la.clone(), oa.clone(), la.clone())
    shape_error(basa.basa_merge, oa, la, z(3, 9, 64), la.clone(), oa.clone(), la.clone())
    shape_error(basa.basa_merge, oa, la, oa.clone(), z(30), oa.clone(), la.clone())
    shape_error(basa.basa_merge, oa, la, oa.clone(), la.clone(), z(3, 10, 32), la.clone())
    shape_error(basa.basa_merge, oa, z(3, 11), oa.clone(), la.clone(), oa.clone(), la.clone())


# ------------------------------------------------- next rows of the path

def test_moments_mass_ranges_radius_shapes():
    x = z(1, 2, 256, 64, dtype=bf16)
    reaches_device_check(basa.basa_pool_moments, x, 64, z(1, 2, 4, 192, dtype=f64), basa.MOMENTS_QUERY)
    shape_error(basa.basa_pool_moments, x, 64, z(1, 2, 192, 4, dtype=f64), basa.MOMENTS_QUERY)
    reaches_device_check(basa.basa_pool_moments, x, 64, z(1, 2, 192, 4, dtype=f64), basa.MOMENTS_KEY)
    shape_error(basa.basa_pool_moments, x, 64, z(1, 2, 4, 192, dtype=f64), basa.MOMENTS_KEY)
    reaches_device_check(basa.basa_block_mass, x, x.clone(), 64, z(1, 2, 4, 4, dtype=f64), 0.1)
    shape_error(basa.basa_block_mass, x, x.clone(), 64, z(1, 2, 4, 8, dtype=f64), 0.1)
    sc = z(8, 16, dtype=f64)
    reaches_device_check(basa.basa_select_ranges, sc, 8, 2, 3, z(8, 5, dtype=i32))
    shape_error(basa.basa_select_ranges, sc, 8, 2, 3, z(8, 4, dtype=i32))
    reaches_device_check(basa.basa_block_radius, x, 64, z(1, 2, 4, 2, dtype=f64))
    shape_error(basa.basa_block_radius, x, 64, z(1, 2, 4, 3, dtype=f64))
