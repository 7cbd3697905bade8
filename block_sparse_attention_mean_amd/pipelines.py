"""The three workflows of the method as sequences of libbasa calls.

Every arithmetic step runs in the HIP kernels; this module only allocates
intermediate device buffers (torch) and chains the four C calls.

* ba_forward       - BA-Att paper, section 3.1 / Algorithm 1 without sorting
                     or compensation: pool Q and K per block, score the blocks,
                     keep the top-k key blocks per query block, attend.
* ba_forward_ranked - the same with the norm-based ranking of section 3.3
                     (Algorithm 1 steps 1, 2 and 12): tokens reordered by l2
                     norm before the blocks are formed, outputs mapped back.
* SparsedForward   - SparseD section 3.3: block pattern from the dense
                     attention map's block mass, top-rho% of prefill and of
                     generation key blocks per query block, reused.
* llsa_forward     - log-linear sparse attention (loglinear-sparse-dit
                     README): levels of 16-token means, coarse-to-fine per-token
                     top-k, attention over fine survivors plus every coarse
                     candidate with a level bias l*ln(block).
* losa_step        - LoSA post: active tokens by query change, sparse prefix
                     attention for active rows written into the cached
                     (O, LSE), dense in-block attention, online-softmax merge.
"""
from __future__ import annotations

import math

import torch

from . import (MOMENTS_KEY, MOMENTS_QUERY, PERMUTE_GATHER, PERMUTE_SCATTER, SELECT_BLOCKS,
               SELECT_CHANGE, basa_attn, basa_attn_workspace, basa_block_mass,
               basa_block_mass_workspace, basa_merge,
               basa_permute, basa_pool, basa_pool_moments, basa_pool_pyramid, basa_rank,
               basa_rank_workspace,
               basa_select, basa_select_ranges, basa_select_workspace, kv_segment, prepare_attn,
               prepare_merge, prepare_pool, prepare_pool_select, prepare_select)


def _empty(*shape, dtype, like):
    return torch.empty(*shape, dtype=dtype, device=like.device)


# ---------------------------------------------------------------------------
# BA-Att selection + block-sparse attention
# ---------------------------------------------------------------------------

class BaForward:
    """Buffers and calls of one BA-Att forward for fixed shapes.

    q, k, v [B, H, L, d] bf16 (or float32); block = query/key block size;
    topk = kept key blocks per query block.  run() fills self.idx (int32
    [B, H, L/block, topk], ascending), self.o and self.lse.

    beta: when given, blocks are ranked by the covariance-compensated logit
    of BA-Att Eq. 13-14 (section 3.4) with that weight: the block moments go
    into 3d-long vectors whose dot product is the compensated logit, and the
    same selection kernels rank them.
    """

    def __init__(self, q, k, v, block: int, topk: int, scale: float | None = None,
                 o_dtype=None, beta: float | None = None):
        b, h, length, d = q.shape
        self.q, self.k, self.v = q, k, v
        self.block, self.topk = block, topk
        self.scale = 1.0 / math.sqrt(d) if scale is None else scale
        self.beta = beta
        nb = length // block
        width = d if beta is None else 3 * d
        self.qbar = _empty(b, h, nb, width, dtype=torch.float64, like=q)
        self.kbt = _empty(b, k.shape[1], width, k.shape[2] // block, dtype=torch.float64, like=q)
        self.idx = _empty(b, h, nb, topk, dtype=torch.int32, like=q)
        self.o = torch.empty(q.shape, dtype=o_dtype or q.dtype, device=q.device)
        self.lse = _empty(b, h, length, dtype=torch.float32, like=q)
        self._select = None
        if beta is None:
            # the selection stage (pool Q and K, score, top-k) as one call, validated once:
            # the library overlaps the query pooling with the selection where it can
            self._select = [prepare_pool_select(q, k, self.qbar, self.kbt, self.idx, topk, block=block,
                                                scale=self.scale)]
        # the attention call, validated once, with the workspace in which the
        # library orders the query tiles (the same output without it)
        seg = kv_segment(self.idx, k, v)
        kw = dict(tile_q=block, block_k=block, scale=self.scale)
        n_ws = basa_attn_workspace(q, seg, self.o, self.lse, **kw)
        self.attn_ws = _empty(n_ws, dtype=torch.uint8, like=q) if n_ws > 0 else None
        self._attend = prepare_attn(q, seg, self.o, self.lse, workspace=self.attn_ws, **kw)

    def select(self):
        if self.beta is None:
            for call in self._select:
                call()
            return
        basa_pool_moments(self.q, self.block, self.qbar, MOMENTS_QUERY, self.scale, self.beta)
        basa_pool_moments(self.k, self.block, self.kbt, MOMENTS_KEY, 1.0, self.beta)
        basa_select(self.qbar, self.kbt, self.idx, self.topk, scale=1.0)

    def attend(self):
        self._attend()

    def run(self):
        self.select()
        self.attend()
        return self.o, self.lse


def ba_forward(q, k, v, block: int, topk: int, scale: float | None = None):
    f = BaForward(q, k, v, block, topk, scale)
    f.run()
    return f.idx, f.o, f.lse


class BaRankedForward:
    """BA-Att Algorithm 1 with norm-based ranking (section 3.3), for fixed
    shapes; with beta given, also the covariance compensation of section 3.4
    (the whole of Algorithm 1), else none (beta = 0).

    rank(): perm_q orders each query head's tokens by non-decreasing l2 norm,
    perm_k each key head's (Eq. 10, stable); Q' = Q[perm_q], K' = K[perm_k],
    V' = V[perm_k] (steps 1 and 2).  select() and attend() run the plain
    forward on the ranked tensors (idx indexes ranked key blocks); attend()
    then maps O and LSE back to token order by the inverse of perm_q (step 12).
    run() does all three and returns (o, lse).
    """

    def __init__(self, q, k, v, block: int, topk: int, scale: float | None = None,
                 o_dtype=None, beta: float | None = None):
        b, h, length, _ = q.shape
        hkv = k.shape[1]
        self.q, self.k, self.v = q, k, v
        self.perm_q = _empty(b, h, length, dtype=torch.int32, like=q)
        self.perm_k = _empty(b, hkv, length, dtype=torch.int32, like=q)
        need = max(basa_rank_workspace(b * h, length), basa_rank_workspace(b * hkv, length), 1)
        self.workspace = _empty(need, dtype=torch.uint8, like=q)
        self.qs, self.ks, self.vs = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        self.inner = BaForward(self.qs, self.ks, self.vs, block, topk, scale, o_dtype, beta)
        self.o = torch.empty_like(self.inner.o)
        self.lse = torch.empty_like(self.inner.lse)

    @property
    def idx(self):
        return self.inner.idx

    def rank(self):
        basa_rank(self.q, self.perm_q, self.workspace)
        basa_rank(self.k, self.perm_k, self.workspace)
        basa_permute(self.q, self.perm_q, self.qs, PERMUTE_GATHER)
        basa_permute(self.k, self.perm_k, self.ks, PERMUTE_GATHER)
        basa_permute(self.v, self.perm_k, self.vs, PERMUTE_GATHER)

    def select(self):
        self.inner.select()

    def attend(self):
        self.inner.attend()
        basa_permute(self.inner.o, self.perm_q, self.o, PERMUTE_SCATTER)
        basa_permute(self.inner.lse, self.perm_q, self.lse, PERMUTE_SCATTER)

    def run(self):
        self.rank()
        self.select()
        self.attend()
        return self.o, self.lse


# ---------------------------------------------------------------------------
# SparseD isolated selection and pattern reuse
# ---------------------------------------------------------------------------

def range_counts(n_pre: int, n_gen: int, rho: float) -> tuple[int, int]:
    """Blocks kept per key range: ceil(rho * n), at least one of a non-empty range."""
    f = lambda n: 0 if n == 0 else min(n, max(1, math.ceil(rho * n - 1e-12)))
    return f(n_pre), f(n_gen)


class SparsedForward:
    """SparseD (section 3.3) for fixed shapes.

    pattern(): the dense attention map's block mass (BA-Att Eq. 3; SparseD's
    avgpool(A, block) ranks the same way), then per query block the top
    rho of the prefill key blocks (tokens before `prefill`) and, separately,
    of the generation key blocks, united (Eq. 5-6).  attend(q, k, v): block-
    sparse attention under that pattern; later denoising steps reuse it by
    calling attend with their own q, k, v.
    """

    def __init__(self, q, k, v, block: int, prefill: int, rho: float, scale: float | None = None,
                 o_dtype=None):
        b, h, length, d = q.shape
        if prefill % block:
            raise ValueError("the prefill length must be a multiple of the block")
        self.q, self.k, self.v = q, k, v
        self.block = block
        self.scale = 1.0 / math.sqrt(d) if scale is None else scale
        nq, nk = length // block, k.shape[2] // block
        self.split = prefill // block
        self.k_lo, self.k_hi = range_counts(self.split, nk - self.split, rho)
        self.mass = _empty(b, h, nq, nk, dtype=torch.float64, like=q)
        self.idx = _empty(b, h, nq, self.k_lo + self.k_hi, dtype=torch.int32, like=q)
        self.o = torch.empty(q.shape, dtype=o_dtype or q.dtype, device=q.device)
        self.lse = _empty(b, h, length, dtype=torch.float32, like=q)
        self.attn_ws = None  # tile-order workspace of the attention, sized at the first attend()
        # the block mass in one pass over the keys: one (max, sum) pair per (query row, key block)
        n_mws = basa_block_mass_workspace(q, k, block)
        self.mass_ws = _empty(n_mws, dtype=torch.uint8, like=q) if n_mws > 0 else None

    def pattern(self):
        basa_block_mass(self.q, self.k, self.block, self.mass, self.scale, workspace=self.mass_ws)
        basa_select_ranges(self.mass, self.split, self.k_lo, self.k_hi, self.idx)

    def attend(self, q=None, k=None, v=None):
        q = self.q if q is None else q
        k = self.k if k is None else k
        v = self.v if v is None else v
        seg = kv_segment(self.idx, k, v)
        kw = dict(tile_q=self.block, block_k=self.block, scale=self.scale)
        if self.attn_ws is None:
            n_ws = basa_attn_workspace(q, seg, self.o, self.lse, **kw)
            self.attn_ws = _empty(max(n_ws, 1), dtype=torch.uint8, like=q)
        basa_attn(q, seg, self.o, self.lse, workspace=self.attn_ws, **kw)

    def run(self):
        self.pattern()
        self.attend()
        return self.o, self.lse


# ---------------------------------------------------------------------------
# Log-linear hierarchical top-k
# ---------------------------------------------------------------------------

def llsa_levels(n: int, block: int) -> int:
    """Coarse levels used for n tokens: the largest L with block^(L+1) | n."""
    if n % block:
        raise ValueError(f"{n} tokens is not a multiple of block {block}")
    lv = 0
    while n % (block ** (lv + 2)) == 0:
        lv += 1
    return lv


class LlsaForward:
    """Buffers and calls of one log-linear sparse attention forward.

    q, k, v [B, H, N, d] bf16; block (pooling factor and fine key block),
    topk per query token.  At most three coarse levels (four key segments).
    run() fills self.sel[l] for l = 1..L (int32 [B, H, N/block^l, topk]),
    self.o and self.lse.
    """

    def __init__(self, q, k, v, block: int = 16, topk: int = 8, scale: float | None = None):
        b, h, n, d = q.shape
        self.q, self.k, self.v = q, k, v
        self.block, self.topk = block, topk
        self.scale = 1.0 / math.sqrt(d) if scale is None else scale
        self.levels = llsa_levels(n, block)
        if not 1 <= self.levels <= 3:
            raise ValueError(f"{self.levels} coarse levels: this path supports 1 to 3")
        f64, f32 = torch.float64, torch.float32
        self.qm, self.km, self.kt, self.vm, self.kf, self.vf, self.sel = {}, {}, {}, {}, {}, {}, {}
        for lv in range(1, self.levels + 1):
            nl = n // block ** lv
            self.qm[lv] = _empty(b, h, nl, d, dtype=f64, like=q)
            self.kt[lv] = _empty(b, h, d, nl, dtype=f64, like=q)
            # float64 K and V rows only where the next level is pooled from them
            self.km[lv] = _empty(b, h, nl, d, dtype=f64, like=q) if 2 <= lv < self.levels else None
            self.vm[lv] = _empty(b, h, nl, d, dtype=f64, like=q) if 2 <= lv < self.levels else None
            self.kf[lv] = _empty(b, h, nl, d, dtype=f32, like=q)
            self.vf[lv] = _empty(b, h, nl, d, dtype=f32, like=q)
            self.sel[lv] = _empty(b, h, nl, topk, dtype=torch.int32, like=q)
        # every token of the top level is a candidate: all of its 16-token blocks
        n_top_blocks = (n // block ** self.levels) // block
        self.top_all = torch.arange(n_top_blocks, dtype=torch.int32, device=q.device).expand(
            b, h, 1, n_top_blocks).contiguous()
        self.o = torch.empty_like(q)
        self.lse = _empty(b, h, n, dtype=f32, like=q)

    def pool(self):
        # every level of Q, K and V in one call (levels 1-2 in one launch, each further
        # level in one more); the same means as pooling level by level
        lv = range(1, self.levels + 1)
        basa_pool_pyramid([self.q, self.k, self.v], self.block,
                          [[(self.qm[i], None, None) for i in lv],
                           [(self.km[i], self.kt[i], self.kf[i]) for i in lv],
                           [(self.vm[i], None, self.vf[i]) for i in lv]])

    def select(self):
        top = self.levels
        basa_select(self.qm[top], self.kt[top], self.sel[top], self.topk, scale=self.scale)
        for lv in range(top - 1, 0, -1):
            basa_select(self.qm[lv], self.kt[lv], self.sel[lv], self.topk, scale=self.scale,
                        parent=self.sel[lv + 1], fanout=self.block)

    def attend(self):
        bl, lb = self.block, math.log(self.block)
        segs = [kv_segment(self.sel[1], self.k, self.v)]          # fine keys: children of level-1 picks
        for lv in range(1, self.levels):                          # level-lv candidates
            segs.append(kv_segment(self.sel[lv + 1], self.kf[lv], self.vf[lv],
                                   shift=4 * lv, bias=lv * lb))
        top = self.levels                                          # every top-level token
        segs.append(kv_segment(self.top_all, self.kf[top], self.vf[top], shift=30,
                               bias=top * lb))
        basa_attn(self.q, segs, self.o, self.lse, tile_q=bl, block_k=bl, scale=self.scale)

    def run(self):
        self.pool()
        self.select()
        self.attend()
        return self.o, self.lse


# ---------------------------------------------------------------------------
# LoSA denoising step
# ---------------------------------------------------------------------------

class LosaStep:
    """Buffers and calls of one LoSA denoising step of a block.

    q_cur, q_prev [B, Hq, T, d] bf16; k_prefix, v_prefix [B, Hkv, P, d] bf16;
    k_block, v_block [B, Hkv, T, d]; cache_o [B, Hq, T, d] float32 and
    cache_lse [B, Hq, T] float32 are updated in place for the active rows.
    prepare() pools the prefix keys (once per generation block); step() runs
    the per-step work and fills self.active, self.sel, self.o (bf16), self.lse.
    The step's six calls are validated once, here; step() only issues them.
    union_walk: give the prefix attention its workspace, so that each key
    head's union of kept blocks is read once.  The default (False) lets every
    row walk its own list: on the 64K-prefix workload that takes 27 us against
    45 us for the union walk (the rows of a key head run on one XCD, whose L2
    serves the blocks several of them keep; the union walk is bound by the
    latency of its block chains and needs a second launch for its partials).
    """

    def __init__(self, q_cur, q_prev, k_prefix, v_prefix, k_block, v_block, cache_o, cache_lse,
                 n_active: int = 5, block: int = 16, topk: int = 128, scale: float | None = None,
                 union_walk: bool = False):
        b, hq, t, d = q_cur.shape
        self.q_cur, self.q_prev = q_cur, q_prev
        self.k_prefix, self.v_prefix = k_prefix, v_prefix
        self.k_block, self.v_block = k_block, v_block
        self.cache_o, self.cache_lse = cache_o, cache_lse
        self.n_active, self.block, self.topk = n_active, block, topk
        self.scale = 1.0 / math.sqrt(d) if scale is None else scale
        hkv, p = k_prefix.shape[1], k_prefix.shape[2]
        self.active = _empty(b, n_active, dtype=torch.int32, like=q_cur)
        self.q64 = _empty(b, hq, t, d, dtype=torch.float64, like=q_cur)
        self.kbt = _empty(b, hkv, d, p // block, dtype=torch.float64, like=q_cur)
        self.sel = _empty(b, hq, n_active, topk, dtype=torch.int32, like=q_cur)
        self.inblock = torch.zeros(b, hq, 1, 1, dtype=torch.int32, device=q_cur.device)
        self.o_in = _empty(b, hq, t, d, dtype=torch.float32, like=q_cur)
        self.lse_in = _empty(b, hq, t, dtype=torch.float32, like=q_cur)
        self.o = torch.empty_like(q_cur)
        self.lse = _empty(b, hq, t, dtype=torch.float32, like=q_cur)
        # scratch of the prefix selection (lets it run in two passes over 512-key parts)
        n_ws = basa_select_workspace(self.q64, self.kbt, self.sel, topk, q_rows=self.active)
        self.ws = torch.empty(max(n_ws, 1), dtype=torch.uint8, device=q_cur.device) if n_ws else None
        # scratch of the prefix attention (lets it walk each key head's union of kept blocks once)
        prefix = kv_segment(self.sel, self.k_prefix, self.v_prefix)
        kw = dict(tile_q=1, block_k=self.block, scale=self.scale, q_rows=self.active)
        n_aws = basa_attn_workspace(self.q_cur, prefix, self.cache_o, self.cache_lse, **kw)
        self.attn_ws = (torch.empty(n_aws, dtype=torch.uint8, device=q_cur.device)
                        if n_aws and union_walk else None)
        # the step's calls, validated once (their buffers never change)
        self.calls = [
            prepare_select(self.q_cur, self.q_prev, self.active, self.n_active, mode=SELECT_CHANGE),
            prepare_pool(self.q_cur, 1, mean_rows=self.q64),
            prepare_select(self.q64, self.kbt, self.sel, self.topk, scale=self.scale,
                           q_rows=self.active, workspace=self.ws),
            prepare_attn(self.q_cur, prefix, self.cache_o, self.cache_lse, workspace=self.attn_ws,
                         **kw),
            prepare_attn(self.q_cur, kv_segment(self.inblock, self.k_block, self.v_block), self.o_in,
                         self.lse_in, tile_q=t, block_k=t, scale=self.scale),
            prepare_merge(self.cache_o, self.cache_lse, self.o_in, self.lse_in, self.o, self.lse),
        ]

    def prepare(self):
        basa_pool(self.k_prefix, self.block, mean_cols=self.kbt)

    def step(self):
        for call in self.calls:
            call()
        return self.o, self.lse
