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


def build() -> str:
    """Compile the reference with g++ (plain -O2, no fast-math) into oracle/liboracle_ref.so."""
    tmp = LIB + ".tmp"
    subprocess.run(["g++", "-O2", "-std=c++17", "-shared", "-fPIC", SRC, "-o", tmp], check=True)
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
    for f in (lib.oracle_pool_mean, lib.oracle_block_logits, lib.oracle_topk,
              lib.oracle_sparse_attention, lib.oracle_merge):
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
