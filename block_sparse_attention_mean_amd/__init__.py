"""Python binding of libbasa: argument marshalling only.

Each function takes torch tensors that live on the current GPU, checks their
dtype and layout, and calls the C function of the same name on torch's current
stream.  Every step of the computation runs in the HIP kernels of libbasa.so;
there is no other code path.  Importing this package fails loudly if the
library has not been built (``python block_sparse_attention_mean_amd/build.py``).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbasa.so")

F32, BF16, F64 = 0, 1, 2
SELECT_BLOCKS, SELECT_CHANGE = 0, 1
PERMUTE_GATHER, PERMUTE_SCATTER = 0, 1
MOMENTS_QUERY, MOMENTS_KEY = 0, 1

STATUS = {0: "BASA_OK", 1: "BASA_E_NULLPTR", 2: "BASA_E_SHAPE", 3: "BASA_E_DTYPE",
          4: "BASA_E_ALIGN", 5: "BASA_E_UNSUPPORTED", 6: "BASA_E_LAUNCH"}

EXPORTS = ("basa_status_string", "basa_version", "basa_pool", "basa_select", "basa_select_workspace",
           "basa_select_static", "basa_pool_select", "basa_pool_select_workspace", "basa_attn",
           "basa_attn_workspace",
           "basa_merge", "basa_rank_workspace", "basa_rank", "basa_permute", "basa_pool_moments",
           "basa_block_mass", "basa_block_mass_workspace", "basa_select_ranges", "basa_block_radius",
           "basa_pool_pyramid")


class BasaError(RuntimeError):
    def __init__(self, func: str, status: int, msg: str):
        super().__init__(f"{func} failed: {STATUS.get(status, status)} ({msg})")
        self.status = status


class SelectDesc(ctypes.Structure):
    _fields_ = [
        ("mode", ctypes.c_int32), ("topk", ctypes.c_int32),
        ("batch", ctypes.c_int64), ("heads_q", ctypes.c_int64), ("heads_kv", ctypes.c_int64),
        ("q_len", ctypes.c_int64), ("rows", ctypes.c_int64), ("keys", ctypes.c_int64),
        ("head_dim", ctypes.c_int64), ("scale", ctypes.c_double),
        ("q_rows", ctypes.c_void_p), ("parent", ctypes.c_void_p),
        ("parent_k", ctypes.c_int32), ("fanout", ctypes.c_int32),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_int64),
    ]


MAX_SEGMENTS = 4
PYRAMID_MAX_LEVELS, PYRAMID_MAX_TENSORS = 4, 3


class PyramidLevel(ctypes.Structure):
    _fields_ = [("mean_rows", ctypes.c_void_p), ("mean_cols", ctypes.c_void_p),
                ("mean_copy", ctypes.c_void_p)]


class PyramidTensor(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("level", PyramidLevel * PYRAMID_MAX_LEVELS)]


class KvSegment(ctypes.Structure):
    _fields_ = [
        ("idx", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("len", ctypes.c_int64), ("rows", ctypes.c_int64), ("count", ctypes.c_int32),
        ("stride", ctypes.c_int32), ("shift", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("bias", ctypes.c_float), ("reserved", ctypes.c_int32),
    ]


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("heads_q", ctypes.c_int64), ("heads_kv", ctypes.c_int64),
        ("len_q", ctypes.c_int64), ("head_dim", ctypes.c_int64), ("lists", ctypes.c_int64),
        ("tile_q", ctypes.c_int32), ("block_k", ctypes.c_int32), ("n_segments", ctypes.c_int32),
        ("reserved", ctypes.c_int32), ("seg", KvSegment * MAX_SEGMENTS),
        ("q_rows", ctypes.c_void_p), ("scale", ctypes.c_double),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_int64),
    ]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python block_sparse_attention_mean_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.basa_status_string.restype = ctypes.c_char_p
    lib.basa_status_string.argtypes = [i32]
    lib.basa_version.restype = i32
    lib.basa_version.argtypes = []
    lib.basa_pool.restype = i32
    lib.basa_pool.argtypes = [vp, i32, i64, i64, i64, i64, vp, vp, vp, i32, vp]
    lib.basa_pool_pyramid.restype = i32
    lib.basa_pool_pyramid.argtypes = [ctypes.POINTER(PyramidTensor), i32, i32, i64, i64, i64, i64,
                                      i32, i32, vp]
    lib.basa_select.restype = i32
    lib.basa_select.argtypes = [ctypes.POINTER(SelectDesc), vp, vp, i32, vp, vp]
    lib.basa_pool_select.restype = i32
    lib.basa_pool_select.argtypes = [ctypes.POINTER(SelectDesc), vp, vp, i32, i64, vp, vp, vp, vp]
    lib.basa_pool_select_workspace.restype = i32
    lib.basa_pool_select_workspace.argtypes = [ctypes.POINTER(SelectDesc), ctypes.POINTER(i64)]
    lib.basa_select_static.restype = i32
    lib.basa_select_static.argtypes = [ctypes.POINTER(SelectDesc), vp, vp, i32, vp, vp]
    lib.basa_select_workspace.restype = i32
    lib.basa_select_workspace.argtypes = [ctypes.POINTER(SelectDesc), ctypes.POINTER(i64)]
    lib.basa_attn_workspace.restype = i32
    lib.basa_attn_workspace.argtypes = [ctypes.POINTER(AttnDesc), ctypes.POINTER(i64)]
    lib.basa_attn.restype = i32
    lib.basa_attn.argtypes = [ctypes.POINTER(AttnDesc), vp, i32, vp, i32, vp, vp]
    lib.basa_merge.restype = i32
    lib.basa_merge.argtypes = [i64, i64, vp, vp, vp, vp, i32, vp, i32, vp, vp]
    lib.basa_pool_moments.restype = i32
    lib.basa_pool_moments.argtypes = [vp, i32, i64, i64, i64, i64, i32, ctypes.c_double,
                                      ctypes.c_double, vp, vp]
    lib.basa_block_mass.restype = i32
    lib.basa_block_mass.argtypes = [vp, vp, i32, i64, i64, i64, i64, i64, i64, i64, ctypes.c_double,
                                    vp, vp, i64, vp]
    lib.basa_block_mass_workspace.restype = i32
    lib.basa_block_mass_workspace.argtypes = [i64, i64, i64, i64, i64, i64, ctypes.POINTER(i64)]
    lib.basa_select_ranges.restype = i32
    lib.basa_select_ranges.argtypes = [vp, i64, i64, i64, ctypes.c_int32, ctypes.c_int32, vp, vp]
    lib.basa_block_radius.restype = i32
    lib.basa_block_radius.argtypes = [vp, i32, i64, i64, i64, i64, vp, vp]
    lib.basa_rank_workspace.restype = i32
    lib.basa_rank_workspace.argtypes = [i64, i64, ctypes.POINTER(i64)]
    lib.basa_rank.restype = i32
    lib.basa_rank.argtypes = [vp, i32, i64, i64, i64, vp, vp, i64, vp]
    lib.basa_permute.restype = i32
    lib.basa_permute.argtypes = [vp, i32, i64, i64, i64, vp, i32, vp, vp]
    return lib


lib = _load()


def _check(func: str, status: int) -> None:
    if status != 0:
        raise BasaError(func, status, lib.basa_status_string(status).decode())


_DT = {torch.float32: F32, torch.bfloat16: BF16, torch.float64: F64}


def _dt(t: torch.Tensor) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _shape(name: str, t, want) -> None:
    """Raise ValueError unless tensor t (when given) has exactly the shape `want`.
    The C functions receive bare pointers and cannot see sizes, so every
    tensor is checked here against the sizes passed with it."""
    if t is not None and tuple(t.shape) != tuple(int(w) for w in want):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(want)}")


def _int32(name: str, t) -> None:
    if t is not None and t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def basa_pool(x: torch.Tensor, block: int, mean_rows: torch.Tensor | None = None,
              mean_cols: torch.Tensor | None = None, mean_copy: torch.Tensor | None = None) -> None:
    """Block means of x [..., len, head_dim] into the given float64/float32/bf16 outputs."""
    prepare_pool(x, block, mean_rows, mean_cols, mean_copy)()


def prepare_pool(x: torch.Tensor, block: int, mean_rows: torch.Tensor | None = None,
                 mean_cols: torch.Tensor | None = None, mean_copy: torch.Tensor | None = None):
    """basa_pool validated once; the returned function issues it on torch's current stream."""
    *lead, length, d = x.shape
    outer = 1
    for s in lead:
        outer *= s
    if block > 0 and length % block == 0:     # otherwise the C call reports BASA_E_SHAPE
        nb = length // block
        _shape("mean_rows", mean_rows, (*lead, nb, d))
        _shape("mean_cols", mean_cols, (*lead, d, nb))
        _shape("mean_copy", mean_copy, (*lead, nb, d))
    copy_dt = _dt(mean_copy) if mean_copy is not None else F32
    args = (_ptr(x), _dt(x), outer, length, d, block, _ptr(mean_rows), _ptr(mean_cols),
            _ptr(mean_copy), copy_dt)
    return _prepared("basa_pool", lib.basa_pool, args, (x, mean_rows, mean_cols, mean_copy))


def basa_pool_pyramid(xs, block: int, outputs) -> None:
    """The log-linear pooling pyramid of up to three tensors (see prepare_pool_pyramid)."""
    prepare_pool_pyramid(xs, block, outputs)()


def prepare_pool_pyramid(xs, block: int, outputs):
    """basa_pool_pyramid validated once.  xs: 1-3 tensors [..., len, head_dim] of one shape and
    dtype; outputs[i][l] = (mean_rows, mean_cols, mean_copy) of level l + 1 of xs[i], None where
    absent (mean_rows [..., n_l, head_dim] float64, mean_cols [..., head_dim, n_l] float64,
    mean_copy [..., n_l, head_dim] float32 or bf16, n_l = len / block^(l+1))."""
    n = len(xs)
    if not 1 <= n <= PYRAMID_MAX_TENSORS or len(outputs) != n:
        raise ValueError(f"1 to {PYRAMID_MAX_TENSORS} tensors, one output list each")
    levels = len(outputs[0])
    if not 1 <= levels <= PYRAMID_MAX_LEVELS:
        raise ValueError(f"1 to {PYRAMID_MAX_LEVELS} levels")
    *lead, length, d = xs[0].shape
    outer = 1
    for s in lead:
        outer *= s
    # every shape first, then the device pointers
    copy_dts = set()
    for i, x in enumerate(xs):
        if x.shape != xs[0].shape or x.dtype != xs[0].dtype:
            raise ValueError("pyramid inputs must share shape and dtype")
        if len(outputs[i]) != levels:
            raise ValueError("every tensor needs the same number of levels")
        span = 1
        for rows, cols, copy in outputs[i]:
            span *= block
            if block > 0 and length % span == 0:   # otherwise the C call reports BASA_E_SHAPE
                nb = length // span
                _shape("mean_rows", rows, (*lead, nb, d))
                _shape("mean_cols", cols, (*lead, d, nb))
                _shape("mean_copy", copy, (*lead, nb, d))
            if copy is not None:
                copy_dts.add(_dt(copy))
    if len(copy_dts) > 1:
        raise ValueError("every mean_copy of one pyramid call must have the same dtype")
    copy_dt = copy_dts.pop() if copy_dts else F32
    arr = (PyramidTensor * n)()
    for i, x in enumerate(xs):
        arr[i].x = _ptr(x)
        for lv, (rows, cols, copy) in enumerate(outputs[i]):
            arr[i].level[lv] = PyramidLevel(_ptr(rows), _ptr(cols), _ptr(copy))
    args = (arr, n, _dt(xs[0]), outer, length, d, block, levels, copy_dt)
    return _prepared("basa_pool_pyramid", lib.basa_pool_pyramid, args, (xs, outputs, arr))


def _prepared(name, fn, args, keep):
    """A function that calls fn(*args, stream) on torch's current stream and checks the status;
    `keep` holds the objects the pointers in args belong to."""
    def call():
        _check(name, fn(*args, torch.cuda.current_stream().cuda_stream))
    call.keep = keep
    return call


def _select_desc(q, k, idx, topk, mode, scale, heads_kv, keys, q_rows, parent, fanout):
    if q.dim() != 4:
        raise ValueError("q must be [batch, heads, len, head_dim]")
    b, hq, lq, d = q.shape
    _int32("idx", idx)
    _int32("q_rows", q_rows)
    _int32("parent", parent)
    desc = SelectDesc()
    desc.mode = mode
    desc.topk = topk
    desc.batch, desc.heads_q, desc.q_len, desc.head_dim = b, hq, lq, d
    if mode == SELECT_CHANGE:
        _shape("k", k, q.shape)
        _shape("idx", idx, (b, topk))
        desc.heads_kv, desc.rows, desc.keys, desc.scale = hq, lq, lq, 1.0
    else:
        if k.dim() != 4 or idx.dim() != 4:
            raise ValueError("k must be [batch, heads_kv, head_dim, keys] and idx "
                             "[batch, heads_q, rows, topk]")
        desc.heads_kv = k.shape[1] if heads_kv is None else heads_kv
        desc.keys = k.shape[-1] if keys is None else keys
        desc.rows = idx.shape[2]
        desc.scale = scale
        _shape("k", k, (b, desc.heads_kv, d, desc.keys))
        _shape("idx", idx, (b, hq, desc.rows, topk))
        if q_rows is None and desc.rows != lq:
            raise ValueError(f"idx has {desc.rows} rows per head but q has {lq} (no q_rows map)")
        _shape("q_rows", q_rows, (b, desc.rows))
        if parent is not None:
            if fanout < 1:
                raise ValueError("fanout must be >= 1")
            _shape("parent", parent, (b, hq, (desc.rows + fanout - 1) // fanout, parent.shape[-1]))
    desc.q_rows = _ptr(q_rows)
    desc.parent = _ptr(parent)
    desc.parent_k = parent.shape[-1] if parent is not None else 0
    desc.fanout = fanout
    return desc


def basa_select(q: torch.Tensor, k: torch.Tensor, idx: torch.Tensor, topk: int, *,
                mode: int = SELECT_BLOCKS, scale: float = 1.0, heads_kv: int | None = None,
                keys: int | None = None, q_rows: torch.Tensor | None = None,
                parent: torch.Tensor | None = None, fanout: int = 1,
                workspace: torch.Tensor | None = None) -> None:
    """BLOCKS: q [B,Hq,Lq,d] float64 means, k [B,Hkv,d,keys] float64 transposed means,
    idx [B,Hq,rows,topk] int32.  CHANGE: q, k [B,H,T,d] current/previous queries,
    idx [B,topk] int32.  workspace: optional device scratch (uint8), see
    basa_select_workspace."""
    prepare_select(q, k, idx, topk, mode=mode, scale=scale, heads_kv=heads_kv, keys=keys,
                   q_rows=q_rows, parent=parent, fanout=fanout, workspace=workspace)()


def prepare_select(q: torch.Tensor, k: torch.Tensor, idx: torch.Tensor, topk: int, *,
                   mode: int = SELECT_BLOCKS, scale: float = 1.0, heads_kv: int | None = None,
                   keys: int | None = None, q_rows: torch.Tensor | None = None,
                   parent: torch.Tensor | None = None, fanout: int = 1,
                   workspace: torch.Tensor | None = None):
    """basa_select validated once; the returned function issues it on torch's current stream."""
    desc = _select_desc(q, k, idx, topk, mode, scale, heads_kv, keys, q_rows, parent, fanout)
    if workspace is not None:
        desc.workspace = _ptr(workspace)
        desc.workspace_bytes = workspace.numel() * workspace.element_size()
    args = (ctypes.byref(desc), _ptr(q), _ptr(k), _dt(q), _ptr(idx))
    return _prepared("basa_select", lib.basa_select, args,
                     (desc, q, k, idx, q_rows, parent, workspace))


def _pool_select_desc(q, k, qbar, kbar_t, idx, topk, block, scale):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [batch, heads, len, head_dim]")
    b, hq, lq, d = q.shape
    if k.shape[0] != b or k.shape[3] != d or k.dtype != q.dtype:
        raise ValueError("k must share batch, head_dim and dtype with q")
    hkv, lk = k.shape[1], k.shape[2]
    if block < 1 or lq % block or lk % block:
        raise ValueError(f"lengths {lq}, {lk} are not multiples of block {block}")
    nq, nk = lq // block, lk // block
    _int32("idx", idx)
    _shape("qbar", qbar, (b, hq, nq, d))
    _shape("kbar_t", kbar_t, (b, hkv, d, nk))
    _shape("idx", idx, (b, hq, nq, topk))
    if qbar.dtype != torch.float64 or kbar_t.dtype != torch.float64:
        raise TypeError("qbar and kbar_t are float64")
    desc = SelectDesc()
    desc.mode, desc.topk = SELECT_BLOCKS, topk
    desc.batch, desc.heads_q, desc.heads_kv = b, hq, hkv
    desc.q_len, desc.rows, desc.keys, desc.head_dim, desc.scale = nq, nq, nk, d, scale
    return desc


def basa_pool_select_workspace(q: torch.Tensor, k: torch.Tensor, qbar: torch.Tensor,
                               kbar_t: torch.Tensor, idx: torch.Tensor, topk: int, *, block: int,
                               scale: float = 1.0) -> int:
    """Bytes of workspace (counters) basa_pool_select uses for its single-launch form."""
    desc = _pool_select_desc(q, k, qbar, kbar_t, idx, topk, block, scale)
    out = ctypes.c_int64(0)
    _check("basa_pool_select_workspace", lib.basa_pool_select_workspace(ctypes.byref(desc),
                                                                        ctypes.byref(out)))
    return out.value


def prepare_pool_select(q: torch.Tensor, k: torch.Tensor, qbar: torch.Tensor, kbar_t: torch.Tensor,
                        idx: torch.Tensor, topk: int, *, block: int, scale: float = 1.0,
                        workspace: torch.Tensor | None = None):
    """basa_pool_select validated once: q [B,Hq,Lq,d], k [B,Hkv,Lk,d] -> qbar [B,Hq,Lq/block,d],
    kbar_t [B,Hkv,d,Lk/block] (float64), idx [B,Hq,Lq/block,topk] (int32)."""
    desc = _pool_select_desc(q, k, qbar, kbar_t, idx, topk, block, scale)
    if workspace is not None:
        desc.workspace = _ptr(workspace)
        desc.workspace_bytes = workspace.numel() * workspace.element_size()
    args = (ctypes.byref(desc), _ptr(q), _ptr(k), _dt(q), block, _ptr(qbar), _ptr(kbar_t), _ptr(idx))
    return _prepared("basa_pool_select", lib.basa_pool_select, args,
                     (desc, q, k, qbar, kbar_t, idx, workspace))


def basa_pool_select(q: torch.Tensor, k: torch.Tensor, qbar: torch.Tensor, kbar_t: torch.Tensor,
                     idx: torch.Tensor, topk: int, *, block: int, scale: float = 1.0,
                     workspace: torch.Tensor | None = None) -> None:
    """Pool q (rows) and k (transposed) by `block` and select each query block's top-k key
    blocks, as basa_pool + basa_pool + basa_select (the library enqueues those three launches)."""
    prepare_pool_select(q, k, qbar, kbar_t, idx, topk, block=block, scale=scale,
                        workspace=workspace)()


def basa_select_static(q: torch.Tensor, k: torch.Tensor, idx: torch.Tensor, topk: int, *,
                       mode: int = SELECT_BLOCKS, scale: float = 1.0, heads_kv: int | None = None,
                       keys: int | None = None, q_rows: torch.Tensor | None = None,
                       parent: torch.Tensor | None = None, fanout: int = 1) -> None:
    """basa_select with the library's own device scratch for the two-pass path
    (no workspace argument, nothing allocated): same tensors and result."""
    desc = _select_desc(q, k, idx, topk, mode, scale, heads_kv, keys, q_rows, parent, fanout)
    _check("basa_select_static", lib.basa_select_static(ctypes.byref(desc), _ptr(q), _ptr(k), _dt(q),
                                                        _ptr(idx), _stream()))


def basa_select_workspace(q: torch.Tensor, k: torch.Tensor, idx: torch.Tensor, topk: int, *,
                          mode: int = SELECT_BLOCKS, heads_kv: int | None = None,
                          keys: int | None = None, q_rows: torch.Tensor | None = None,
                          parent: torch.Tensor | None = None, fanout: int = 1) -> int:
    """Bytes of workspace basa_select can use for this request (0: none)."""
    desc = _select_desc(q, k, idx, topk, mode, 1.0, heads_kv, keys, q_rows, parent, fanout)
    out = ctypes.c_int64(0)
    _check("basa_select_workspace", lib.basa_select_workspace(ctypes.byref(desc), ctypes.byref(out)))
    return out.value


def kv_segment(idx: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, count: int | None = None,
               offset: int = 0, shift: int = 0, bias: float = 0.0) -> dict:
    """One key source for basa_attn.  idx [B,Hq,rows,stride] int32 block indices
    (entries offset .. offset+count-1 of each row are used); k/v [B,Hkv,len,d]."""
    if idx.dtype != torch.int32:
        raise TypeError("segment index must be int32")
    if k.dtype != v.dtype or k.shape != v.shape:
        raise TypeError("segment k and v must match")
    stride = idx.shape[-1]
    count = stride - offset if count is None else count
    if not 0 <= offset <= stride - count:
        raise ValueError("segment column range out of bounds")
    return {"idx": idx, "k": k, "v": v, "count": count, "offset": offset, "stride": stride,
            "shift": shift, "bias": bias}


def _attn_desc(q, segments, o, lse, tile_q, block_k, scale, q_rows, workspace):
    """Validated AttnDesc for basa_attn (every shape checked before any pointer is taken)."""
    if q.dim() != 4:
        raise ValueError("q must be [batch, heads, len, head_dim]")
    b, hq, lq, d = q.shape
    if isinstance(segments, dict):
        segments = [segments]
    if not 1 <= len(segments) <= MAX_SEGMENTS:
        raise ValueError("1 to 4 segments")
    if lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    if tile_q < 1 or block_k < 1:
        raise ValueError("tile_q and block_k must be positive")
    _shape("o", o, q.shape)
    _shape("lse", lse, (b, hq, lq))
    _int32("q_rows", q_rows)
    n_rows = q_rows.shape[-1] if q_rows is not None else lq
    if n_rows % tile_q:
        raise ValueError(f"{n_rows} query rows are not a whole number of {tile_q}-row tiles")
    _shape("q_rows", q_rows, (b, n_rows))
    if workspace is not None and workspace.dtype != torch.uint8:
        raise TypeError("workspace must be a uint8 tensor")
    desc = AttnDesc()
    desc.batch, desc.heads_q, desc.len_q, desc.head_dim = b, hq, lq, d
    desc.heads_kv = segments[0]["k"].shape[1]
    desc.lists = n_rows // tile_q
    desc.tile_q, desc.block_k, desc.n_segments = tile_q, block_k, len(segments)
    for i, sg in enumerate(segments):
        kk, ix = sg["k"], sg["idx"]
        if kk.dim() != 4 or kk.shape[0] != b or kk.shape[1] != desc.heads_kv or kk.shape[3] != d:
            raise ValueError(f"segment {i}: k/v {tuple(kk.shape)} must be [{b}, {desc.heads_kv}, "
                             f"len, {d}] (all segments share the key heads)")
        if ix.dim() != 4 or ix.shape[0] != b or ix.shape[1] != hq:
            raise ValueError(f"segment {i}: idx {tuple(ix.shape)} must be [{b}, {hq}, rows, stride]")
        if desc.lists and ix.shape[2] <= (desc.lists - 1) >> sg["shift"]:
            raise ValueError(f"segment {i}: idx has {ix.shape[2]} rows, tile {desc.lists - 1} "
                             f"reads row {(desc.lists - 1) >> sg['shift']}")
    for i, sg in enumerate(segments):
        kk, ix = sg["k"], sg["idx"]
        t = desc.seg[i]
        t.idx = _ptr(ix) + 4 * sg["offset"]
        t.k, t.v = _ptr(kk), _ptr(sg["v"])
        t.len, t.rows = kk.shape[2], ix.shape[2]
        t.count, t.stride, t.shift = sg["count"], sg["stride"], sg["shift"]
        t.dtype, t.bias = _dt(kk), sg["bias"]
    desc.q_rows = _ptr(q_rows)
    desc.scale = scale
    if workspace is not None:
        desc.workspace = _ptr(workspace)
        desc.workspace_bytes = workspace.numel()
    return desc


def basa_attn(q: torch.Tensor, segments, o: torch.Tensor, lse: torch.Tensor, *, tile_q: int,
              block_k: int, scale: float, q_rows: torch.Tensor | None = None,
              workspace: torch.Tensor | None = None) -> None:
    """q [B,Hq,Lq,d]; segments from kv_segment(); o [B,Hq,Lq,d]; lse [B,Hq,Lq] float32.
    q_rows [B, lists*tile_q] int32 selects the query rows of each tile.  workspace:
    optional uint8 device scratch (see basa_attn_workspace)."""
    prepare_attn(q, segments, o, lse, tile_q=tile_q, block_k=block_k, scale=scale, q_rows=q_rows,
                 workspace=workspace)()


def basa_attn_workspace(q: torch.Tensor, segments, o: torch.Tensor, lse: torch.Tensor, *,
                        tile_q: int, block_k: int, scale: float,
                        q_rows: torch.Tensor | None = None) -> int:
    """Bytes of workspace basa_attn can use for this request (0: none): the union walk of
    row-mapped 16-key rows, or the query-tile order of the bf16 128-row MFMA path."""
    desc = _attn_desc(q, segments, o, lse, tile_q, block_k, scale, q_rows, None)
    out = ctypes.c_int64(0)
    _check("basa_attn_workspace", lib.basa_attn_workspace(ctypes.byref(desc), ctypes.byref(out)))
    return out.value


def prepare_attn(q: torch.Tensor, segments, o: torch.Tensor, lse: torch.Tensor, *, tile_q: int,
                 block_k: int, scale: float, q_rows: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None):
    """Validate a basa_attn call once and return a function that issues it on
    torch's current stream (for loops that repeat the same call on the same
    buffers: the descriptor and pointers are built here, not per call).  The
    tensors must stay alive and keep their storage while the function is used."""
    desc = _attn_desc(q, segments, o, lse, tile_q, block_k, scale, q_rows, workspace)
    args = (ctypes.byref(desc), _ptr(q), _dt(q), _ptr(o), _dt(o), _ptr(lse))
    return _prepared("basa_attn", lib.basa_attn, args, (desc, q, segments, o, lse, q_rows, workspace))


def basa_merge(o_a: torch.Tensor, lse_a: torch.Tensor, o_b: torch.Tensor, lse_b: torch.Tensor,
               o: torch.Tensor, lse: torch.Tensor) -> None:
    """Merge two partials [..., d] + [...] into o, lse (o may be o_a)."""
    prepare_merge(o_a, lse_a, o_b, lse_b, o, lse)()


def prepare_merge(o_a: torch.Tensor, lse_a: torch.Tensor, o_b: torch.Tensor, lse_b: torch.Tensor,
                  o: torch.Tensor, lse: torch.Tensor):
    """basa_merge validated once; the returned function issues it on torch's current stream."""
    d = o_a.shape[-1]
    rows = o_a.numel() // d if d else 0
    if o_a.dtype != o_b.dtype:
        raise TypeError("partials must share a dtype")
    for t in (lse_a, lse_b, lse):
        if t.dtype != torch.float32:
            raise TypeError("LSE tensors must be float32")
    _shape("o_b", o_b, o_a.shape)
    _shape("o", o, o_a.shape)
    for name, t in (("lse_a", lse_a), ("lse_b", lse_b), ("lse", lse)):
        _shape(name, t, o_a.shape[:-1])
    args = (rows, d, _ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _dt(o_a), _ptr(o), _dt(o),
            _ptr(lse))
    return _prepared("basa_merge", lib.basa_merge, args, (o_a, lse_a, o_b, lse_b, o, lse))


def basa_pool_moments(x: torch.Tensor, block: int, out: torch.Tensor, role: int,
                      scale: float = 1.0, beta: float = 1.0) -> None:
    """Block moments of x [..., len, d] arranged for compensated scoring: QUERY
    out [..., len/block, 3d] = [scale*mean, beta/d*var, beta/d*mean^2]; KEY out
    [..., 3d, len/block] = [mean, mean^2+var, var] (float64)."""
    *lead, length, d = x.shape
    outer = 1
    for s in lead:
        outer *= s
    if out.dtype != torch.float64:
        raise TypeError("moments are float64")
    if block > 0 and length % block == 0:
        nb = length // block
        _shape("out", out, (*lead, nb, 3 * d) if role == MOMENTS_QUERY else (*lead, 3 * d, nb))
    _check("basa_pool_moments", lib.basa_pool_moments(_ptr(x), _dt(x), outer, length, d, block, role,
                                                      float(scale), float(beta), _ptr(out), _stream()))


def basa_block_mass_workspace(q: torch.Tensor, k: torch.Tensor, block: int) -> int:
    """Bytes of workspace that let basa_block_mass run in one pass (0: this shape never does)."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [batch, heads, len, head_dim]")
    b, hq, lq, d = q.shape
    out = ctypes.c_int64(0)
    _check("basa_block_mass_workspace",
           lib.basa_block_mass_workspace(b, hq, lq, k.shape[2], d, block, ctypes.byref(out)))
    return out.value


def basa_block_mass(q: torch.Tensor, k: torch.Tensor, block: int, mass: torch.Tensor,
                    scale: float, workspace: torch.Tensor | None = None) -> None:
    """mass [B, Hq, Lq/block, Lk/block] float64 <- the dense attention map's
    block mass (rows sum to 1) for q [B, Hq, Lq, d], k [B, Hkv, Lk, d].
    workspace: optional uint8 device scratch (see basa_block_mass_workspace)."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [batch, heads, len, head_dim]")
    b, hq, lq, d = q.shape
    if k.dtype != q.dtype or k.shape[0] != b or k.shape[3] != d:
        raise TypeError("q and k must share batch, head_dim and dtype")
    if mass.dtype != torch.float64:
        raise TypeError("mass is float64")
    if block > 0 and lq % block == 0 and k.shape[2] % block == 0:
        _shape("mass", mass, (b, hq, lq // block, k.shape[2] // block))
    if workspace is not None and workspace.dtype != torch.uint8:
        raise TypeError("workspace must be a uint8 tensor")
    ws, n_ws = (_ptr(workspace), workspace.numel()) if workspace is not None else (None, 0)
    _check("basa_block_mass", lib.basa_block_mass(_ptr(q), _ptr(k), _dt(q), b, hq, k.shape[1], lq,
                                                  k.shape[2], d, block, float(scale), _ptr(mass),
                                                  ws, n_ws, _stream()))


def basa_select_ranges(scores: torch.Tensor, split: int, k_lo: int, k_hi: int,
                       idx: torch.Tensor) -> None:
    """idx [..., k_lo + k_hi] int32 <- per row of scores [..., n] (float64), the k_lo
    best of columns [0, split) and the k_hi best of [split, n), ascending."""
    if scores.dtype != torch.float64 or idx.dtype != torch.int32:
        raise TypeError("scores are float64 and idx int32")
    n = scores.shape[-1]
    rows = scores.numel() // max(n, 1)
    _shape("idx", idx, (*scores.shape[:-1], k_lo + k_hi))
    _check("basa_select_ranges", lib.basa_select_ranges(_ptr(scores), rows, n, split, k_lo, k_hi,
                                                        _ptr(idx), _stream()))


def basa_block_radius(x: torch.Tensor, block: int, out: torch.Tensor) -> None:
    """out [..., len/block, 2] float64 <- per block of x [..., len, d]: (max distance of a
    token from the block mean, max token norm)."""
    *lead, length, d = x.shape
    outer = 1
    for s in lead:
        outer *= s
    if out.dtype != torch.float64:
        raise TypeError("out is float64")
    if block > 0 and length % block == 0:
        _shape("out", out, (*lead, length // block, 2))
    _check("basa_block_radius", lib.basa_block_radius(_ptr(x), _dt(x), outer, length, d, block,
                                                      _ptr(out), _stream()))


def _outer_len(x: torch.Tensor, lead_dims: int) -> tuple[int, int]:
    outer = 1
    for s in x.shape[:lead_dims]:
        outer *= s
    return outer, x.shape[lead_dims]


def basa_rank_workspace(outer: int, length: int) -> int:
    """Bytes of device workspace basa_rank needs for `outer` sequences of `length` tokens."""
    out = ctypes.c_int64(0)
    _check("basa_rank_workspace", lib.basa_rank_workspace(outer, length, ctypes.byref(out)))
    return out.value


def basa_rank(x: torch.Tensor, perm: torch.Tensor, workspace: torch.Tensor | None = None) -> None:
    """perm [..., L] int32 <- the order of x [..., L, d]'s tokens by non-decreasing l2 norm
    (stable), per sequence.  workspace: uint8 device tensor of basa_rank_workspace bytes
    (allocated here when not given)."""
    if perm.dtype != torch.int32 or perm.shape != x.shape[:-1]:
        raise TypeError("perm must be int32 with x's shape minus the channel dimension")
    outer, length = _outer_len(x, x.dim() - 2)
    need = basa_rank_workspace(outer, length)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _check("basa_rank", lib.basa_rank(_ptr(x), _dt(x), outer, length, x.shape[-1], _ptr(perm),
                                      _ptr(workspace), workspace.numel(), _stream()))


def basa_permute(x: torch.Tensor, perm: torch.Tensor, out: torch.Tensor,
                 mode: int = PERMUTE_GATHER) -> None:
    """Rows of x moved by perm [..., L]: GATHER out[i] = x[perm[i]], SCATTER out[perm[i]] = x[i].
    x and out are [..., L, width] or, for width 1, [..., L] (e.g. an LSE)."""
    if perm.dtype != torch.int32:
        raise TypeError("perm must be int32")
    if out.shape != x.shape or out.dtype != x.dtype:
        raise TypeError("out must match x in shape and dtype")
    if x.shape == perm.shape:
        width = 1
    elif x.shape[:-1] == perm.shape:
        width = x.shape[-1]
    else:
        raise TypeError("perm must be x's shape, or x's shape minus the last dimension")
    outer, length = _outer_len(perm, perm.dim() - 1)
    _check("basa_permute", lib.basa_permute(_ptr(x), _dt(x), outer, length, width, _ptr(perm),
                                            mode, _ptr(out), _stream()))


__all__ = ["basa_pool", "basa_pool_pyramid", "prepare_pool_pyramid", "PyramidLevel", "PyramidTensor",
           "PYRAMID_MAX_LEVELS", "PYRAMID_MAX_TENSORS", "basa_select", "basa_select_workspace", "basa_select_static", "basa_attn",
           "basa_pool_select", "basa_pool_select_workspace", "prepare_pool_select",
           "basa_attn_workspace", "prepare_attn", "prepare_pool", "prepare_select", "prepare_merge", "basa_merge", "kv_segment", "BasaError", "lib",
           "LIB_PATH", "EXPORTS", "SelectDesc", "AttnDesc", "KvSegment", "MAX_SEGMENTS", "F32", "BF16", "F64", "SELECT_BLOCKS",
           "SELECT_CHANGE", "basa_rank_workspace", "basa_rank", "basa_permute", "PERMUTE_GATHER",
           "PERMUTE_SCATTER", "basa_pool_moments", "MOMENTS_QUERY", "MOMENTS_KEY", "basa_block_mass", "basa_block_mass_workspace",
           "basa_select_ranges", "basa_block_radius"]
