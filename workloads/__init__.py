"""Seeded synthetic inputs for the five block-sparse attention workloads.

This module only draws random tensors and lays them out; it holds none of the
method's arithmetic (no pooling, scoring, selection, attention or merging).
Both the fp64 oracle tests and the HIP path read their inputs from here, so
the two sides always see the same bytes.

Conventions
-----------
* RNG: ``numpy.random.Generator(PCG64(seed))``; normals are drawn as float32.
* bf16 tensors are returned as ``uint16`` bit patterns, rounded from float32
  with round-to-nearest-even.  ``bf16_to_f32`` widens them exactly.
* Layout is ``[batch, heads, tokens, head_dim]``, row-major.

Workloads (shapes follow the pages' settings; the recipes are this
repository's own and are listed in the design notes):

* ``tiny``  - batch 1, 2 heads, 1024 tokens, d=64, block 64, top-4, fp32
  N(0,1) plus one planted key block (block 12 of every head is set to three
  times the mean of query block 3, computed in float64 from the unplanted Q).
* ``dlm16k`` / ``dlm64k`` - 32 heads, d=128, block 128, bf16.  Each tensor
  X in {Q, K, V} is ``Z_X + 2.0 * c_X(t) @ U_h`` where Z is N(0,1), ``U_h`` is a
  per-head 4 x d basis with unit-length rows shared by Q, K and V, and the
  coefficients ``c_X(t)`` interpolate linearly between N(0,1) anchors placed
  every 512 tokens (smooth along the sequence so block means keep them).
* ``llsa64k`` - 4 heads, 65536 tokens of a 256 x 256 image in Z-order, d=64,
  bf16 N(0,1) with a field of 8 Gaussian blobs per head added to Q and K.
* ``losa64k`` - 32 query heads / 8 KV heads, d=128, a 65536-token prefix,
  a 16-token block; previous-step queries differ from the current ones by
  N(0, 0.1^2) noise except 5 planted tokens that change by N(0, 1).
"""
from __future__ import annotations

import dataclasses
import numpy as np

__all__ = [
    "f32_to_bf16", "bf16_to_f32", "Workload", "WORKLOADS", "make_tiny",
    "make_dlm", "make_llsa", "make_losa", "zorder_index", "generate",
]


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32, exact."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    tokens: int
    head_dim: int
    block: int
    topk: int
    dtype: str          # "f32" or "bf16"
    seed: int
    heads_kv: int = 0   # 0 -> same as heads

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))

    @property
    def blocks(self) -> int:
        return self.tokens // self.block


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 1024, 64, 64, 4, "f32", 1000),
    "dlm16k": Workload("dlm16k", 1, 32, 16384, 128, 128, 64, "bf16", 1001),
    "dlm64k": Workload("dlm64k", 1, 32, 65536, 128, 128, 128, "bf16", 1002),
    "llsa64k": Workload("llsa64k", 1, 4, 65536, 64, 16, 8, "bf16", 1003),
    "losa64k": Workload("losa64k", 1, 32, 65536, 128, 16, 128, "bf16", 1004, heads_kv=8),
}

# Planted-block geometry of the tiny workload.
TINY_PLANT_QUERY_BLOCK = 3
TINY_PLANT_KEY_BLOCK = 12
TINY_PLANT_GAIN = 3.0

# Planted changing tokens of the LoSA step workload.
LOSA_BLOCK_TOKENS = 16
LOSA_ACTIVE = 5
LOSA_PLANTED = (1, 4, 7, 10, 13)


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def make_tiny(seed: int = 1000, heads: int = 2, tokens: int = 1024, head_dim: int = 64,
              block: int = 64, plant: bool = True) -> dict:
    """fp32 N(0,1) Q, K, V with one planted key block per head."""
    g = _rng(seed)
    shape = (1, heads, tokens, head_dim)
    q = g.standard_normal(shape, dtype=np.float32)
    k = g.standard_normal(shape, dtype=np.float32)
    v = g.standard_normal(shape, dtype=np.float32)
    if plant:
        qs = slice(TINY_PLANT_QUERY_BLOCK * block, (TINY_PLANT_QUERY_BLOCK + 1) * block)
        ks = slice(TINY_PLANT_KEY_BLOCK * block, (TINY_PLANT_KEY_BLOCK + 1) * block)
        # the planted rows copy a scaled average of one query block (input recipe)
        target = q[:, :, qs, :].astype(np.float64).sum(axis=2) / block
        k[:, :, ks, :] = (TINY_PLANT_GAIN * target)[:, :, None, :].astype(np.float32)
    return {"q": q, "k": k, "v": v}


def _structured(g: np.random.Generator, z: np.ndarray, basis: np.ndarray, anchor_every: int,
                gain: float) -> np.ndarray:
    """z[b,h,t,:] + gain * c(t) @ basis[h], with c interpolated from N(0,1) anchors."""
    b, h, t, d = z.shape
    rank = basis.shape[1]
    n_anchor = t // anchor_every + 1
    anchors = g.standard_normal((b, h, n_anchor, rank), dtype=np.float32)
    pos = np.arange(t, dtype=np.float64) / anchor_every
    i0 = np.floor(pos).astype(np.int64)
    w = (pos - i0).astype(np.float32)[:, None]
    out = np.empty_like(z)
    for bi in range(b):
        for hi in range(h):
            a = anchors[bi, hi]
            c = (1.0 - w) * a[i0] + w * a[np.minimum(i0 + 1, n_anchor - 1)]
            out[bi, hi] = z[bi, hi] + gain * (c @ basis[hi])
    return out


def make_dlm(seed: int, heads: int, tokens: int, head_dim: int, batch: int = 1,
             rank: int = 4, gain: float = 2.0, anchor_every: int = 512) -> dict:
    """bf16 Q, K, V: N(0,1) plus a smooth per-head rank-4 component."""
    g = _rng(seed)
    shape = (batch, heads, tokens, head_dim)
    zs = [g.standard_normal(shape, dtype=np.float32) for _ in range(3)]
    basis = g.standard_normal((heads, rank, head_dim), dtype=np.float32)
    basis /= np.linalg.norm(basis, axis=-1, keepdims=True)
    out = {}
    for name, z in zip(("q", "k", "v"), zs):
        out[name] = f32_to_bf16(_structured(g, z, basis, anchor_every, gain))
        del z
    return out


def zorder_index(side: int) -> np.ndarray:
    """pixel (y, x) -> token index with x bit b at bit 2b and y bit b at bit 2b+1."""
    bits = int(side).bit_length() - 1
    assert (1 << bits) == side
    x = np.arange(side, dtype=np.int64)[None, :].repeat(side, 0)
    y = np.arange(side, dtype=np.int64)[:, None].repeat(side, 1)
    t = np.zeros_like(x)
    for bit in range(bits):
        t |= ((x >> bit) & 1) << (2 * bit)
        t |= ((y >> bit) & 1) << (2 * bit + 1)
    return t


def make_llsa(seed: int = 1003, heads: int = 4, side: int = 256, head_dim: int = 64,
              blobs: int = 8, gain: float = 2.0) -> dict:
    """bf16 tokens of a side x side grid in Z-order; a Gaussian-blob field is added to Q and K."""
    g = _rng(seed)
    n = side * side
    shape = (1, heads, n, head_dim)
    zq = g.standard_normal(shape, dtype=np.float32)
    zk = g.standard_normal(shape, dtype=np.float32)
    zv = g.standard_normal(shape, dtype=np.float32)
    tok = zorder_index(side)                       # [y, x] -> token
    yy, xx = np.meshgrid(np.arange(side, dtype=np.float64), np.arange(side, dtype=np.float64),
                         indexing="ij")
    for h in range(heads):
        centres = g.uniform(0.0, float(side), size=(blobs, 2))
        sigmas = g.uniform(8.0, 32.0, size=blobs)
        amps = gain * g.standard_normal((blobs, head_dim))
        field = np.zeros((side, side, head_dim), dtype=np.float64)
        for b in range(blobs):
            r2 = (yy - centres[b, 0]) ** 2 + (xx - centres[b, 1]) ** 2
            field += np.exp(-r2 / (2.0 * sigmas[b] ** 2))[:, :, None] * amps[b][None, None, :]
        per_token = np.empty((n, head_dim), dtype=np.float32)
        per_token[tok.reshape(-1)] = field.reshape(n, head_dim).astype(np.float32)
        zq[0, h] += per_token
        zk[0, h] += per_token
    return {"q": f32_to_bf16(zq), "k": f32_to_bf16(zk), "v": f32_to_bf16(zv)}


def make_losa(seed: int = 1004, heads_q: int = 32, heads_kv: int = 8, prefix: int = 65536,
              head_dim: int = 128, block_tokens: int = LOSA_BLOCK_TOKENS,
              planted=LOSA_PLANTED, noise: float = 0.1) -> dict:
    """Prefix K/V cache, one block of K/V, current and previous-step queries (bf16)."""
    g = _rng(seed)
    kp = f32_to_bf16(g.standard_normal((1, heads_kv, prefix, head_dim), dtype=np.float32))
    vp = f32_to_bf16(g.standard_normal((1, heads_kv, prefix, head_dim), dtype=np.float32))
    kb = f32_to_bf16(g.standard_normal((1, heads_kv, block_tokens, head_dim), dtype=np.float32))
    vb = f32_to_bf16(g.standard_normal((1, heads_kv, block_tokens, head_dim), dtype=np.float32))
    q_cur = f32_to_bf16(g.standard_normal((1, heads_q, block_tokens, head_dim), dtype=np.float32))
    step = noise * g.standard_normal((1, heads_q, block_tokens, head_dim), dtype=np.float32)
    big = g.standard_normal((1, heads_q, len(planted), head_dim), dtype=np.float32)
    step[:, :, list(planted), :] = big
    q_prev = f32_to_bf16(bf16_to_f32(q_cur) + step)
    return {"k_prefix": kp, "v_prefix": vp, "k_block": kb, "v_block": vb,
            "q_cur": q_cur, "q_prev": q_prev}


def generate(name: str, seed: int | None = None) -> dict:
    """Inputs of a named workload at its full size."""
    w = WORKLOADS[name]
    s = w.seed if seed is None else seed
    if name == "tiny":
        return make_tiny(s, w.heads, w.tokens, w.head_dim, w.block)
    if name in ("dlm16k", "dlm64k"):
        return make_dlm(s, w.heads, w.tokens, w.head_dim)
    if name == "llsa64k":
        return make_llsa(s)
    if name == "losa64k":
        return make_losa(s)
    raise KeyError(name)
