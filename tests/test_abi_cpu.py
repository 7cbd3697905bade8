"""The C ABI without a GPU: the library loads, exports every function that
include/basa.h declares, and rejects invalid arguments with the documented
status codes before any HIP call (so these run on a machine with no GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

import block_sparse_attention_mean_amd as basa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "basa.h")

OK, NULLPTR, SHAPE, DTYPE, ALIGN, UNSUPPORTED = 0, 1, 2, 3, 4, 5


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|const char\*)\s+(basa_\w+)\s*\(", text, re.M)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("basa_pool", "basa_select", "basa_attn", "basa_merge"):
        assert n in names
    assert set(names) == set(basa.EXPORTS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", basa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(basa_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(basa.lib, name)


def test_status_strings_and_version():
    for code in range(7):
        assert basa.lib.basa_status_string(code)
    assert basa.lib.basa_status_string(99) == b"unknown status"
    assert basa.lib.basa_version() >= 100


# a fake, aligned, never-dereferenced device address: validation fails before use
FAKE = 1 << 20
MISALIGNED = FAKE + 4


def pool(x=FAKE, xdt=basa.BF16, outer=2, length=256, d=128, block=64, rows=FAKE, cols=None,
         copy=None, cdt=basa.F32):
    return basa.lib.basa_pool(x, xdt, outer, length, d, block, rows, cols, copy, cdt, None)


def test_pool_validation():
    assert pool(length=250) == SHAPE
    assert pool(block=0) == SHAPE
    assert pool(d=100) == SHAPE
    assert pool(d=1024) == SHAPE
    assert pool(outer=-1) == SHAPE
    assert pool(xdt=7) == DTYPE
    assert pool(copy=FAKE, cdt=basa.F64) == DTYPE
    assert pool(x=None) == NULLPTR
    assert pool(rows=None) == NULLPTR
    assert pool(x=MISALIGNED) == ALIGN
    assert pool(outer=0) == OK          # empty: nothing to do
    assert pool(length=0) == OK


def pyramid(xs=(FAKE,), levels=2, outs=None, xdt=basa.BF16, outer=2, length=4096, d=64, block=16,
            cdt=basa.F32, n=None):
    arr = (basa.PyramidTensor * max(len(xs), 1))()
    for i, x in enumerate(xs):
        arr[i].x = x
        for lv in range(min(levels, basa.PYRAMID_MAX_LEVELS)):
            rows, cols, copy = (outs or {}).get((i, lv), (FAKE, None, None))
            arr[i].level[lv] = basa.PyramidLevel(rows, cols, copy)
    n_t = len(xs) if n is None else n
    return basa.lib.basa_pool_pyramid(arr, n_t, xdt, outer, length, d, block, levels, cdt, None)


def test_pool_pyramid_validation():
    assert pyramid(length=4000) == SHAPE              # not a multiple of block^levels
    assert pyramid(length=16 * 24) == SHAPE           # a multiple of block, not of block^2
    assert pyramid(block=1) == SHAPE
    assert pyramid(block=33, length=33 * 33) == SHAPE
    assert pyramid(d=512) == SHAPE                    # block * head_dim above 4096
    assert pyramid(d=100) == SHAPE
    assert pyramid(outer=-1) == SHAPE
    assert pyramid(levels=0) == SHAPE
    assert pyramid(levels=5, length=16 ** 5) == SHAPE
    assert pyramid(n=0) == SHAPE
    assert pyramid(n=4) == SHAPE
    assert pyramid(xdt=7) == DTYPE
    assert pyramid(outs={(0, 1): (FAKE, None, FAKE)}, cdt=basa.F64) == DTYPE
    assert basa.lib.basa_pool_pyramid(None, 1, basa.BF16, 2, 4096, 64, 16, 2, basa.F32,
                                      None) == NULLPTR
    assert pyramid(xs=(0,)) == NULLPTR
    assert pyramid(outs={(0, 1): (None, None, None)}) == NULLPTR   # a level with no output
    # level 3 is pooled from the rows of level 2 (level 2 from level 1 inside the workgroup)
    assert pyramid(levels=3, outs={(0, 1): (None, FAKE, None)}) == NULLPTR
    assert pyramid(xs=(FAKE, 0)) == NULLPTR
    assert pyramid(xs=(MISALIGNED,)) == ALIGN
    assert pyramid(outs={(0, 1): (FAKE, MISALIGNED, None)}) == ALIGN
    assert pyramid(outer=0) == OK                     # empty: nothing to do
    assert pyramid(length=0) == OK


def sel_desc(**kw):
    d = basa.SelectDesc()
    d.mode, d.topk, d.batch, d.heads_q, d.heads_kv = basa.SELECT_BLOCKS, 4, 1, 2, 2
    d.q_len, d.rows, d.keys, d.head_dim, d.scale = 16, 16, 16, 64, 0.125
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def select(desc, q=FAKE, k=FAKE, dt=basa.F64, idx=FAKE):
    return basa.lib.basa_select(ctypes.byref(desc), q, k, dt, idx, None)


def test_select_workspace_size():
    # host-only: bytes of scratch for the two-pass path over > 1024 candidates
    def ws(**kw):
        n = ctypes.c_int64(-1)
        assert basa.lib.basa_select_workspace(ctypes.byref(sel_desc(**kw)), ctypes.byref(n)) == OK
        return n.value
    assert ws() == 0                                        # 16 keys: one pass
    assert ws(keys=1024, topk=64) == 0
    # 2 x 5 rows, 4096 keys = 8 parts of 512, top-128: (key, candidate) = 12 bytes each
    assert ws(keys=4096, topk=128, rows=5, q_rows=FAKE) == 2 * 5 * 8 * 128 * 12
    assert ws(keys=3000, topk=10) == 2 * 16 * 6 * 10 * 12  # a partial last part
    assert ws(keys=4096, topk=300) == 0                     # top-k beyond the two-pass path
    assert ws(keys=4096, topk=8, parent=FAKE, parent_k=2, fanout=4) == 0
    assert ws(keys=4096, topk=8, mode=basa.SELECT_CHANGE) == 0
    assert basa.lib.basa_select_workspace(None, ctypes.byref(ctypes.c_int64())) == NULLPTR
    assert basa.lib.basa_select_workspace(ctypes.byref(sel_desc()), None) == NULLPTR


def test_select_static_host_checks():
    # host-only rejections of the no-allocation selection: a caller workspace,
    # and a two-pass request beyond the library's 4 MiB scratch
    st = lambda d: basa.lib.basa_select_static(ctypes.byref(d), FAKE, FAKE, basa.F64, FAKE, None)
    assert basa.lib.basa_select_static(None, FAKE, FAKE, basa.F64, FAKE, None) == NULLPTR
    assert st(sel_desc(workspace=FAKE, workspace_bytes=1 << 20)) == UNSUPPORTED
    assert st(sel_desc(workspace_bytes=64)) == UNSUPPORTED
    big = sel_desc(heads_q=32, heads_kv=8, q_len=16, rows=16, keys=4096, topk=256, head_dim=128,
                   q_rows=FAKE)
    assert 32 * 16 * 8 * 256 * 12 > (4 << 20)
    assert st(big) == SHAPE


def test_select_validation():
    assert basa.lib.basa_select(None, FAKE, FAKE, basa.F64, FAKE, None) == NULLPTR
    assert select(sel_desc(topk=0)) == SHAPE
    assert select(sel_desc(topk=17)) == SHAPE
    assert select(sel_desc(heads_kv=3)) == SHAPE
    assert select(sel_desc(keys=5000, topk=4)) == SHAPE
    assert select(sel_desc(scale=0.0)) == SHAPE
    assert select(sel_desc(scale=-1.0)) == SHAPE
    assert select(sel_desc(rows=8)) == SHAPE            # rows != q_len without a row map
    assert select(sel_desc(head_dim=60)) == SHAPE
    assert select(sel_desc(), dt=basa.BF16) == DTYPE
    assert select(sel_desc(mode=7)) == UNSUPPORTED
    assert select(sel_desc(), q=None) == NULLPTR
    assert select(sel_desc(), k=MISALIGNED) == ALIGN
    assert select(sel_desc(batch=0)) == OK
    # candidate restriction
    assert select(sel_desc(parent=FAKE, parent_k=2, fanout=4, topk=9)) == SHAPE   # 9 > 2*4
    assert select(sel_desc(parent=FAKE, parent_k=2, fanout=3)) == SHAPE           # 16 % 3
    assert select(sel_desc(parent=FAKE, parent_k=2, fanout=4, q_rows=FAKE)) == UNSUPPORTED
    # change mode
    ch = sel_desc(mode=basa.SELECT_CHANGE, q_len=16, topk=5)
    assert select(ch, dt=basa.BF16) != DTYPE
    assert select(sel_desc(mode=basa.SELECT_CHANGE, q_len=16, topk=17), dt=basa.BF16) == SHAPE
    assert select(sel_desc(mode=basa.SELECT_CHANGE, q_len=2000, topk=5), dt=basa.BF16) == SHAPE
    assert select(ch, dt=9) == DTYPE


def attn_desc(n_seg=1, **kw):
    d = basa.AttnDesc()
    d.batch, d.heads_q, d.heads_kv, d.len_q, d.head_dim = 1, 4, 2, 256, 128
    d.lists, d.tile_q, d.block_k, d.n_segments, d.scale = 2, 128, 128, n_seg, 0.088
    for i in range(n_seg):
        g = d.seg[i]
        g.idx, g.k, g.v, g.len, g.rows, g.count, g.stride = FAKE, FAKE, FAKE, 256, 2, 2, 2
        g.dtype = basa.BF16
    for k, v in kw.items():
        if k.startswith("seg_"):
            setattr(d.seg[0], k[4:], v)
        else:
            setattr(d, k, v)
    return d


def attn(desc, q=FAKE, qdt=basa.BF16, o=FAKE, odt=basa.BF16, lse=FAKE):
    return basa.lib.basa_attn(ctypes.byref(desc), q, qdt, o, odt, lse, None)


def test_attn_validation():
    assert basa.lib.basa_attn(None, FAKE, 1, FAKE, 1, FAKE, None) == NULLPTR
    assert attn(attn_desc(head_dim=96)) == SHAPE
    assert attn(attn_desc(heads_kv=3)) == SHAPE
    assert attn(attn_desc(lists=3)) == SHAPE            # 3*128 rows != len_q
    assert attn(attn_desc(tile_q=0)) == SHAPE
    assert attn(attn_desc(tile_q=256)) == SHAPE
    assert attn(attn_desc(block_k=0)) == SHAPE
    assert attn(attn_desc(n_seg=0)) == SHAPE
    assert attn(attn_desc(n_seg=1, n_segments=5)) == SHAPE
    assert attn(attn_desc(scale=float("inf"))) == SHAPE
    assert attn(attn_desc(seg_count=-1)) == SHAPE
    assert attn(attn_desc(seg_stride=1)) == SHAPE       # stride < count
    assert attn(attn_desc(seg_rows=1)) == SHAPE         # 2 tiles need 2 index rows
    assert attn(attn_desc(seg_shift=31)) == SHAPE
    assert attn(attn_desc(seg_bias=float("nan"))) == SHAPE
    assert attn(attn_desc(seg_dtype=basa.F64)) == DTYPE
    assert attn(attn_desc(), qdt=basa.F64) == DTYPE
    assert attn(attn_desc(), odt=basa.F64) == DTYPE
    assert attn(attn_desc(), q=None) == NULLPTR
    assert attn(attn_desc(seg_idx=None)) == NULLPTR
    assert attn(attn_desc(), lse=None) == NULLPTR
    assert attn(attn_desc(seg_v=MISALIGNED)) == ALIGN
    assert attn(attn_desc(lists=0, len_q=0)) == OK
    assert attn(attn_desc(batch=0)) == OK


def attn_workspace(desc):
    out = ctypes.c_int64(-1)
    assert basa.lib.basa_attn_workspace(ctypes.byref(desc), ctypes.byref(out)) == OK
    return out.value


def test_attn_workspace_sizes():
    # the MFMA path (bf16, head_dim 128, 128-row tiles of 128-key blocks, one
    # segment) takes one int32 tile rank per query tile, rounded up to 256 bytes
    assert attn_workspace(attn_desc()) == 256                      # 1 x 4 heads x 2 tiles
    assert attn_workspace(attn_desc(batch=3, heads_q=8, heads_kv=8, lists=100, len_q=12800,
                                    seg_rows=100)) == (3 * 8 * 100 * 4 + 255) // 256 * 256
    assert attn_workspace(attn_desc(lists=2049, len_q=2049 * 128, seg_rows=2049)) == 0
    assert attn_workspace(attn_desc(seg_count=0)) == 0
    assert attn_workspace(attn_desc(tile_q=64, lists=4)) == 0       # not the MFMA path
    assert attn_workspace(attn_desc(head_dim=64)) == 0
    assert attn_workspace(attn_desc(n_seg=2)) == 0
    assert basa.lib.basa_attn_workspace(None, ctypes.byref(ctypes.c_int64())) == NULLPTR


def merge(rows=8, d=128, oa=FAKE, la=FAKE, ob=FAKE, lb=FAKE, idt=basa.F32, o=FAKE,
          odt=basa.BF16, lse=FAKE):
    return basa.lib.basa_merge(rows, d, oa, la, ob, lb, idt, o, odt, lse, None)


def test_merge_validation():
    assert merge(rows=-1) == SHAPE
    assert merge(d=96) == SHAPE
    assert merge(d=4) == SHAPE
    assert merge(idt=basa.F64) == DTYPE
    assert merge(odt=basa.F64) == DTYPE
    assert merge(ob=None) == NULLPTR
    assert merge(o=MISALIGNED) == ALIGN
    assert merge(o=FAKE, oa=FAKE, idt=basa.F32, odt=basa.BF16) == UNSUPPORTED   # aliasing, dtype change
    assert merge(rows=0) == OK


def test_binding_needs_gpu_tensors():
    import torch
    x = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        basa.basa_pool(x, 16, mean_rows=torch.zeros(1, 1, 4, 64, dtype=torch.float64))


def rank(x=FAKE, xdt=basa.BF16, outer=2, length=256, d=128, perm=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return basa.lib.basa_rank(x, xdt, outer, length, d, perm, ws, ws_bytes, None)


def test_rank_validation():
    assert rank(outer=-1) == SHAPE
    assert rank(length=-1) == SHAPE
    assert rank(outer=1 << 16, length=1 << 16) == SHAPE  # more than 2^31 - 1 tokens
    assert rank(d=100) == SHAPE
    assert rank(d=4) == SHAPE
    assert rank(d=1024) == SHAPE
    assert rank(xdt=7) == DTYPE
    assert rank(x=None) == NULLPTR
    assert rank(perm=None) == NULLPTR
    assert rank(ws=None) == NULLPTR
    assert rank(x=MISALIGNED) == ALIGN
    assert rank(ws=MISALIGNED) == ALIGN
    assert rank(length=0) == OK
    assert rank(outer=0, x=None, perm=None, ws=None) == OK


def test_rank_workspace_validation():
    out = ctypes.c_int64(-1)
    assert basa.lib.basa_rank_workspace(2, 256, None) == NULLPTR
    assert basa.lib.basa_rank_workspace(-1, 256, ctypes.byref(out)) == SHAPE
    assert basa.lib.basa_rank_workspace(1 << 16, 1 << 16, ctypes.byref(out)) == SHAPE
    assert basa.lib.basa_rank_workspace(0, 256, ctypes.byref(out)) == OK and out.value == 0


def permute(x=FAKE, dt=basa.BF16, outer=2, length=256, width=128, perm=FAKE + (1 << 24), mode=0,
            out=FAKE + (1 << 26)):
    return basa.lib.basa_permute(x, dt, outer, length, width, perm, mode, out, None)


def test_permute_validation():
    assert permute(outer=-1) == SHAPE
    assert permute(width=0) == SHAPE
    assert permute(dt=5) == DTYPE
    assert permute(mode=2) == UNSUPPORTED
    assert permute(x=None) == NULLPTR
    assert permute(perm=None) == NULLPTR
    assert permute(out=None) == NULLPTR
    assert permute(out=MISALIGNED + (1 << 26)) == ALIGN
    assert permute(out=FAKE + 1024) == UNSUPPORTED  # overlaps x
    assert permute(length=0) == OK


def moments(x=FAKE, xdt=basa.BF16, outer=2, length=256, d=128, block=64, role=0, scale=0.1, beta=1.0,
            out=FAKE):
    return basa.lib.basa_pool_moments(x, xdt, outer, length, d, block, role, scale, beta, out, None)


def test_pool_moments_validation():
    assert moments(length=250) == SHAPE
    assert moments(block=0) == SHAPE
    assert moments(d=176) == SHAPE     # 3 d would exceed the selection's 512 channels
    assert moments(d=100) == SHAPE
    assert moments(scale=float("nan")) == SHAPE
    assert moments(beta=float("inf")) == SHAPE
    assert moments(xdt=9) == DTYPE
    assert moments(role=2) == UNSUPPORTED
    assert moments(x=None) == NULLPTR
    assert moments(out=None) == NULLPTR
    assert moments(out=MISALIGNED) == ALIGN
    assert moments(outer=0, x=None, out=None) == OK


def mass(q=FAKE, k=FAKE, dt=basa.BF16, b=1, hq=4, hkv=2, lq=256, lk=256, d=64, block=32, scale=0.1,
         out=FAKE, ws=None, ws_bytes=0):
    return basa.lib.basa_block_mass(q, k, dt, b, hq, hkv, lq, lk, d, block, scale, out, ws, ws_bytes,
                                    None)


def mass_ws(b=1, hq=4, lq=256, lk=256, d=64, block=32):
    out = ctypes.c_int64(-1)
    assert basa.lib.basa_block_mass_workspace(b, hq, lq, lk, d, block, ctypes.byref(out)) == OK
    return out.value


def test_block_mass_validation():
    assert mass(hq=3) == SHAPE
    assert mass(d=136) == SHAPE
    assert mass(block=2) == SHAPE
    assert mass(block=48) == SHAPE
    assert mass(lq=250) == SHAPE
    assert mass(scale=0.0) == SHAPE
    assert mass(dt=basa.F64) == DTYPE
    assert mass(k=None) == NULLPTR
    assert mass(out=MISALIGNED) == ALIGN
    assert mass(b=0, q=None, k=None, out=None) == OK
    assert mass(k=None, ws=FAKE, ws_bytes=1 << 20) == NULLPTR   # the workspace checks nothing else
    assert mass(out=MISALIGNED, ws=FAKE, ws_bytes=1 << 20) == ALIGN


def test_block_mass_workspace_sizes():
    # one (max, sum) pair of float64 per (query row, key block) on the matrix-core shapes
    assert mass_ws() == 1 * 4 * 256 * (256 // 32) * 16
    assert mass_ws(b=2, hq=8, lq=16384, lk=16384, d=128, block=128) == 2 * 8 * 16384 * 128 * 16
    assert mass_ws(block=16) == 4 * 256 * 16 * 16
    assert mass_ws(block=8) == 0          # not a multiple of 16: the one-thread-per-row kernel
    assert mass_ws(block=256) == 0        # above the matrix-core kernel's 128 rows
    assert mass_ws(d=132) == 0
    assert mass_ws(b=0) == 0
    assert basa.lib.basa_block_mass_workspace(1, 4, 256, 256, 64, 32, None) == NULLPTR


def ranges(s=FAKE, rows=4, n=128, split=64, lo=20, hi=20, idx=FAKE):
    return basa.lib.basa_select_ranges(s, rows, n, split, lo, hi, idx, None)


def test_select_ranges_validation():
    assert ranges(n=0) == SHAPE
    assert ranges(n=2000) == SHAPE
    assert ranges(split=129) == SHAPE
    assert ranges(lo=65) == SHAPE
    assert ranges(hi=65) == SHAPE
    assert ranges(lo=0, hi=0) == SHAPE
    assert ranges(s=None) == NULLPTR
    assert ranges(idx=MISALIGNED) == ALIGN
    assert ranges(rows=0, s=None, idx=None) == OK


def radius(x=FAKE, xdt=basa.BF16, outer=2, length=256, d=128, block=64, out=FAKE):
    return basa.lib.basa_block_radius(x, xdt, outer, length, d, block, out, None)


def test_block_radius_validation():
    assert radius(block=0) == SHAPE
    assert radius(block=512, length=512) == SHAPE
    assert radius(length=250) == SHAPE
    assert radius(d=264) == SHAPE
    assert radius(d=12) == SHAPE
    assert radius(xdt=4) == DTYPE
    assert radius(out=None) == NULLPTR
    assert radius(x=MISALIGNED) == ALIGN
    assert radius(outer=0, x=None, out=None) == OK
