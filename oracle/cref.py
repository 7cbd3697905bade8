"""ctypes wrapper of the fp64 C++ reference (basa_oracle_ref.cpp).

TEST INFRASTRUCTURE ONLY (see the package docstring).  The shared library is
built in-tree with g++ by build() (and here, when it is missing).  Inputs are
widened exactly to float64 before the call; bf16 inputs are uint16 bit
patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "basa_oracle_ref.cpp")
LIB = os.path.join(HERE, "liboracle_ref.so")
GXX_FLAGS = ["-O2", "-std=c++17", "-fopenmp", "-shared", "-fPIC"]


def build() -> str:
    """Compile the reference with g++ (plain -O2, no fast-math, OpenMP) into oracle/liboracle_ref.so."""
    tmp = LIB + ".tmp"
    subprocess.run(["g++", *GXX_FLAGS, SRC, "-o", tmp], check=True)
    os.replace(tmp, LIB)
    return LIB


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB):
        build()
    lib = ctypes.CDLL(LIB)
    i64, f64, p = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    lib.oracle_pool_mean.argtypes = [p, i64, i64, i64, i64, p]
    lib.oracle_block_logits.argtypes = [p, p, i64, i64, i64, i64, i64, i64, f64, p]
    lib.oracle_topk.argtypes = [p, i64, i64, i64, p]
    lib.oracle_sparse_attention.argtypes = [p, p, p, i64, i64, i64, i64, i64, i64, p, i64, i64, i64,
                                            f64, p, p]
    lib.oracle_merge.argtypes = [p, p, p, p, i64, i64, p, p]
    lib.oracle_llsa_num_levels.argtypes = [i64, i64]
    lib.oracle_llsa_num_levels.restype = i64
    lib.oracle_llsa_forward.argtypes = [p, p, p, i64, i64, i64, i64, i64, f64, i64, p, p, p]
    lib.oracle_losa_step.argtypes = [p, p, p, p, p, p, p, p, i64, i64, i64, i64, i64, i64, i64, i64,
                                     i64, f64, p, p, p, p, p, p, p, p]
    lib.oracle_threads.argtypes = []
    for f in (lib.oracle_pool_mean, lib.oracle_block_logits, lib.oracle_topk,
              lib.oracle_sparse_attention, lib.oracle_merge, lib.oracle_llsa_forward,
              lib.oracle_losa_step, lib.oracle_threads):
        f.restype = ctypes.c_int
    return lib


_lib = None


def _l() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = _load()
    return _lib


def _f64(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.uint16:  # bf16 bit patterns
        x = (x.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _ok(status: int, name: str) -> None:
    if status != 0:
        raise ValueError(f"{name}: invalid arguments")


def pool_mean(x, block: int) -> np.ndarray:
    x = _f64(x)
    *lead, length, d = x.shape
    outer = int(np.prod(lead)) if lead else 1
    out = np.empty((*lead, length // block, d))
    _ok(_l().oracle_pool_mean(_ptr(x), outer, length, d, block, _ptr(out)), "pool_mean")
    return out


def block_logits(qbar, kbar, scale: float) -> np.ndarray:
    qbar, kbar = _f64(qbar), _f64(kbar)
    b, hq, nq, d = qbar.shape
    hkv, nk = kbar.shape[1], kbar.shape[2]
    out = np.empty((b, hq, nq, nk))
    _ok(_l().oracle_block_logits(_ptr(qbar), _ptr(kbar), b, hq, hkv, nq, nk, d, scale, _ptr(out)),
        "block_logits")
    return out


def topk_ascending(scores, k: int) -> np.ndarray:
    scores = _f64(scores)
    n = scores.shape[-1]
    rows = scores.size // n
    idx = np.empty((*scores.shape[:-1], k), dtype=np.int32)
    _ok(_l().oracle_topk(_ptr(scores), rows, n, k, _ptr(idx)), "topk")
    return idx


def sparse_attention(q, k, v, kv_idx, tile_q: int, block_k: int, scale: float):
    q, k, v = _f64(q), _f64(k), _f64(v)
    idx = np.ascontiguousarray(kv_idx, dtype=np.int32)
    b, hq, lq, d = q.shape
    hkv, lk = k.shape[1], k.shape[2]
    o = np.empty(q.shape)
    lse = np.empty((b, hq, lq))
    _ok(_l().oracle_sparse_attention(_ptr(q), _ptr(k), _ptr(v), b, hq, hkv, lq, lk, d, _ptr(idx),
                                     idx.shape[-1], tile_q, block_k, scale, _ptr(o), _ptr(lse)),
        "sparse_attention")
    return o, lse


def merge(o_a, lse_a, o_b, lse_b):
    o_a, o_b = _f64(o_a), _f64(o_b)
    lse_a, lse_b = _f64(lse_a), _f64(lse_b)
    d = o_a.shape[-1]
    rows = o_a.size // d
    o = np.empty(o_a.shape)
    lse = np.empty(lse_a.shape)
    _ok(_l().oracle_merge(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), rows, d, _ptr(o), _ptr(lse)),
        "merge")
    return o, lse


def threads() -> int:
    """Threads the reference's OpenMP loops use."""
    return int(_l().oracle_threads())


def llsa_num_levels(n: int, block: int) -> int:
    lv = int(_l().oracle_llsa_num_levels(n, block))
    if lv < 0:
        raise ValueError(f"sequence length {n} is not a multiple of block {block}")
    return lv


def llsa_forward(q, k, v, block: int, topk: int, scale: float, levels: int | None = None):
    """q, k, v [H, N, d] -> {"sel": {l: [H, N/block^l, topk]}, "o", "lse", "levels"}."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    h, n, d = q.shape
    if levels is None:
        levels = llsa_num_levels(n, block)
    sizes = [n // block ** lv for lv in range(levels + 1)]
    sel = np.empty(sum(h * sizes[lv] * topk for lv in range(1, levels + 1)), dtype=np.int32)
    o = np.empty((h, n, v.shape[-1]))
    lse = np.empty((h, n))
    _ok(_l().oracle_llsa_forward(_ptr(q), _ptr(k), _ptr(v), h, n, d, block, topk, scale, levels,
                                 _ptr(sel), _ptr(o), _ptr(lse)), "llsa_forward")
    out, off = {}, 0
    for lv in range(1, levels + 1):
        m = h * sizes[lv] * topk
        out[lv] = sel[off:off + m].reshape(h, sizes[lv], topk)
        off += m
    return {"sel": out, "o": o, "lse": lse, "levels": levels, "sizes": sizes}


def losa_step(q_cur, q_prev, k_prefix, v_prefix, k_block, v_block, cache_o, cache_lse,
              n_active: int, block: int, topk: int, scale: float):
    """The LoSA denoising step; same inputs and result keys as the numpy oracle's losa_step."""
    qc, qp = _f64(q_cur), _f64(q_prev)
    kp, vp = _f64(k_prefix), _f64(v_prefix)
    kb, vb = _f64(k_block), _f64(v_block)
    co, cl = _f64(cache_o), _f64(cache_lse)
    b, hq, t, d = qc.shape
    hkv, p = kp.shape[1], kp.shape[2]
    act = np.empty((b, n_active), dtype=np.int32)
    sel = np.empty((b, hq, n_active, topk), dtype=np.int32)
    nco, ncl = np.empty(co.shape), np.empty(cl.shape)
    o_in, lse_in = np.empty(co.shape), np.empty(cl.shape)
    o, lse = np.empty(co.shape), np.empty(cl.shape)
    _ok(_l().oracle_losa_step(_ptr(qc), _ptr(qp), _ptr(kp), _ptr(vp), _ptr(kb), _ptr(vb), _ptr(co),
                              _ptr(cl), b, hq, hkv, t, p, d, n_active, block, topk, scale, _ptr(act),
                              _ptr(sel), _ptr(nco), _ptr(ncl), _ptr(o_in), _ptr(lse_in), _ptr(o),
                              _ptr(lse)), "losa_step")
    return {"active": act, "sel": sel, "o": o, "lse": lse, "cache_o": nco, "cache_lse": ncl,
            "o_in": o_in, "lse_in": lse_in}
