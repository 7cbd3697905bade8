"""fp64 definitions of every step of the block-sparse attention path.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Inputs may be float32
arrays, float64 arrays or bf16 bit patterns (uint16); they are widened to
float64 exactly before any arithmetic.
"""
from __future__ import annotations

import math
import numpy as np

__all__ = [
    "as_f64", "pool_mean", "block_logits", "topk_ascending", "attend_rows",
    "sparse_attention", "dense_attention", "merge", "llsa_num_levels", "llsa_forward",
    "llsa_keys_per_query", "token_change", "active_tokens", "losa_step",
    "norm_key", "norm_rank", "gather_rows", "scatter_rows", "ba_forward_ranked",
    "block_variance", "compensated_logits", "ba_forward_algorithm1",
    "block_mass", "range_counts", "topk_in_ranges", "sparsed_pattern", "sparsed_forward",
    "block_radius_maxnorm", "deviation_bound", "selection_recall",
]


def as_f64(x: np.ndarray) -> np.ndarray:
    """Exact widening to float64; uint16 arrays are read as bf16 bit patterns.
    A float64 array is returned as it is (not copied)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64, copy=False)


# ---------------------------------------------------------------------------
# BA-Att, section 3.1: pooled block representatives and block logits
# ---------------------------------------------------------------------------

def pool_mean(x: np.ndarray, block: int) -> np.ndarray:
    """Mean of each run of `block` consecutive tokens: [..., L, d] -> [..., L/block, d].

    BA-Att section 3.1: the block embeddings Qbar_gq, Kbar_gk are obtained by
    mean pooling over the tokens of each block (Algorithm 1, block partition and
    block statistics).  The LLSA README pools the same way, level by level.
    A length that is not a multiple of the block is rejected, as the LLSA
    README says its implementation raises for such inputs.
    """
    x = as_f64(x)
    length, d = x.shape[-2], x.shape[-1]
    if block <= 0 or length % block:
        raise ValueError(f"length {length} is not a multiple of block {block}")
    return x.reshape(*x.shape[:-2], length // block, block, d).mean(axis=-2)


def block_logits(qbar: np.ndarray, kbar: np.ndarray, scale: float) -> np.ndarray:
    """l[gq, gk] = scale * (Qbar_gq . Kbar_gk), BA-Att section 3.1, Eq. 2.

    qbar [B, Hq, Nq, d], kbar [B, Hkv, Nk, d] with Hq a multiple of Hkv
    (query head h reads key head h // (Hq/Hkv)); result [B, Hq, Nq, Nk].
    """
    qbar = as_f64(qbar)
    kbar = as_f64(kbar)
    group = qbar.shape[1] // kbar.shape[1]
    if group * kbar.shape[1] != qbar.shape[1]:
        raise ValueError("query heads must be a multiple of key heads")
    kb = np.repeat(kbar, group, axis=1) if group > 1 else kbar
    return scale * np.matmul(qbar, np.swapaxes(kb, -1, -2))


def topk_ascending(scores: np.ndarray, k: int) -> np.ndarray:
    """Per row, the k best columns under (score descending, column ascending),
    returned in ascending column order (int32).

    BA-Att Algorithm 1 takes a softmax over each query-block row and keeps the
    top-kappa key blocks.  Softmax is strictly increasing in the logit, so the
    kept set is the top-kappa by logit; ranking the logits directly avoids ties
    that rounding inside exp could create.  Equal scores go to the lower column
    (a stable sort of the negated scores keeps equal keys in column order).
    """
    scores = np.asarray(scores, dtype=np.float64)
    n = scores.shape[-1]
    if not 0 < k <= n:
        raise ValueError(f"top-k {k} out of range for {n} columns")
    order = np.argsort(-scores, axis=-1, kind="stable")
    return np.sort(order[..., :k], axis=-1).astype(np.int32)


# ---------------------------------------------------------------------------
# Attention restricted to the kept key blocks (BA-Att section 2, Eq. 1)
# ---------------------------------------------------------------------------

def attend_rows(q_rows: np.ndarray, k_head: np.ndarray, v_head: np.ndarray, blocks,
                block_k: int, scale: float, bias=None):
    """Softmax attention of some query rows over a listed set of key blocks.

    q_rows [r, d]; k_head, v_head [Lk, d]; blocks: key-block indices (negative
    entries are unused slots); bias: per listed block, added to every logit of
    that block.  Logits z_ij = scale * q_i . k_j (+ bias); with M the row max,
    LSE_i = M + ln(sum_j exp(z_ij - M)) and O_i = sum_j exp(z_ij - LSE_i) v_j.
    This is Eq. 1 of the BA-Att paper evaluated only on the key blocks that
    the block mask M keeps for this query block.  A row with no keys returns
    O = 0, LSE = -inf.
    """
    q_rows = as_f64(q_rows)
    k_head = as_f64(k_head)
    v_head = as_f64(v_head)
    blocks = np.asarray(blocks).reshape(-1)
    use = [i for i in range(blocks.size) if blocks[i] >= 0]
    r, d = q_rows.shape
    if not use:
        return np.zeros((r, v_head.shape[-1])), np.full(r, -np.inf)
    key_idx = np.concatenate([np.arange(blocks[i] * block_k, (blocks[i] + 1) * block_k) for i in use])
    z = scale * (q_rows @ k_head[key_idx].T)
    if bias is not None:
        bias = np.asarray(bias, dtype=np.float64).reshape(-1)
        z = z + np.repeat(bias[use], block_k)[None, :]
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    s = e.sum(axis=1, keepdims=True)
    lse = (m + np.log(s))[:, 0]
    o = (e @ v_head[key_idx]) / s
    return o, lse


def sparse_attention(q, k, v, kv_idx, tile_q: int, block_k: int, scale: float,
                     bias=None, q_rows=None, lists=None):
    """Block-sparse attention over whole tensors.

    q [B, Hq, Lq, d]; k, v [B, Hkv, Lk, d]; kv_idx [B, Hq, T, kept] key-block
    indices per list; list t covers query rows t*tile_q .. t*tile_q+tile_q-1,
    or the rows q_rows[b, t*tile_q + r] when a row map is given.  bias has the
    shape of kv_idx.  `lists` restricts the work to the given (b, h, t)
    triples.  Returns O [B, Hq, Lq, d] and LSE [B, Hq, Lq] in float64; rows
    that no computed list covers hold NaN.
    """
    q = as_f64(q)
    kv_idx = np.asarray(kv_idx)
    nb, hq, lq, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    n_lists = kv_idx.shape[2]
    o = np.full((nb, hq, lq, v.shape[-1]), np.nan)
    lse = np.full((nb, hq, lq), np.nan)
    if lists is None:
        lists = [(b, h, t) for b in range(nb) for h in range(hq) for t in range(n_lists)]
    kf = {}
    for b, h, t in lists:
        key = (b, h // group)
        if key not in kf:
            kf[key] = (as_f64(k[b, h // group]), as_f64(v[b, h // group]))
        kh, vh = kf[key]
        if q_rows is None:
            rows = np.arange(t * tile_q, (t + 1) * tile_q)
        else:
            rows = np.asarray(q_rows)[b, t * tile_q:(t + 1) * tile_q]
        bb = None if bias is None else np.asarray(bias)[b, h, t]
        o_t, lse_t = attend_rows(q[b, h, rows], kh, vh, kv_idx[b, h, t], block_k, scale, bb)
        o[b, h, rows] = o_t
        lse[b, h, rows] = lse_t
    return o, lse


def dense_attention(q, k, v, scale: float):
    """Full softmax attention (BA-Att section 2, Eq. 1), bidirectional.

    q [B, Hq, Lq, d], k/v [B, Hkv, Lk, d] (query head h reads key head
    h // (Hq/Hkv)); returns O and natural-log LSE.
    """
    q = as_f64(q)
    nb, hq = q.shape[:2]
    group = hq // np.asarray(k).shape[1]
    o = np.empty(q.shape[:3] + (np.asarray(v).shape[-1],))
    lse = np.empty(q.shape[:3])
    for b in range(nb):
        for hk in range(np.asarray(k).shape[1]):
            kh, vh = as_f64(k[b, hk]), as_f64(v[b, hk])
            for h in range(hk * group, (hk + 1) * group):
                z = scale * (q[b, h] @ kh.T)
                m = z.max(axis=-1, keepdims=True)
                e = np.exp(z - m)
                s = e.sum(axis=-1, keepdims=True)
                o[b, h] = (e @ vh) / s
                lse[b, h] = (m + np.log(s))[:, 0]
    return o, lse


def merge(o_a, lse_a, o_b, lse_b):
    """Combine two partial softmax results over disjoint key sets.

    The LoSA post merges the cached prefix attention with the in-block
    (suffix) attention by online softmax: with m = max(LSE_a, LSE_b),
    LSE = m + ln(e^(LSE_a - m) + e^(LSE_b - m)) and
    O = e^(LSE_a - LSE) O_a + e^(LSE_b - LSE) O_b.  (0, -inf) is the empty
    partial; two empty partials give (0, -inf).
    """
    o_a = as_f64(o_a)
    o_b = as_f64(o_b)
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    m = np.maximum(lse_a, lse_b)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    s = np.exp(lse_a - m_safe) + np.exp(lse_b - m_safe)
    lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, s)))
    lse_safe = np.where(empty, 0.0, lse)
    wa = np.where(empty, 0.0, np.exp(lse_a - lse_safe))[..., None]
    wb = np.where(empty, 0.0, np.exp(lse_b - lse_safe))[..., None]
    return wa * o_a + wb * o_b, lse


# ---------------------------------------------------------------------------
# BA-Att, section 3.3 (Eq. 9-10) and Algorithm 1 steps 1, 2 and 12:
# norm-based ranking of the tokens before the blocks are formed
# ---------------------------------------------------------------------------

def norm_key(x) -> np.ndarray:
    """Squared l2 norm of every token, float64: [..., L, d] -> [..., L].

    BA-Att section 3.3, Eq. 9 scores a token by its l2 norm.  The square
    orders the tokens the same way in exact arithmetic and needs no square
    root (whose rounding could merge two distinct norms).  The channels are
    added one after another, c = 0, 1, ..., d-1.  For bf16 inputs every square
    and every partial sum is exact unless one token's squares span more than
    about 2^37 in magnitude.
    """
    x = as_f64(x)
    s = np.zeros(x.shape[:-1])
    for c in range(x.shape[-1]):
        s = s + x[..., c] * x[..., c]
    return s


def norm_rank(x) -> np.ndarray:
    """The permutation of BA-Att Eq. 10, per sequence: int32 [..., L].

    Position i of the ranked sequence holds token perm[i]; the norms are
    non-decreasing along the ranked sequence.  Tokens with equal norms keep
    their order (a stable sort: the pages do not say how ties go).  Every
    leading index (batch, head) is ranked on its own, over the whole sequence
    (Algorithm 1 mentions a "(windowed)" sort without giving a window).
    """
    return np.argsort(norm_key(x), axis=-1, kind="stable").astype(np.int32)


def gather_rows(x, perm) -> np.ndarray:
    """X'[..., i, :] = X[..., perm[i], :] (Algorithm 1 steps 1 and 2)."""
    x = np.asarray(x)
    return np.take_along_axis(x, np.asarray(perm, dtype=np.int64)[..., None], axis=-2)


def scatter_rows(x, perm) -> np.ndarray:
    """Out[..., perm[i], :] = X[..., i, :]: the inverse of gather_rows
    (Algorithm 1 step 12 remaps the outputs to the original order by pi_q^-1)."""
    x = np.asarray(x)
    out = np.empty_like(x)
    np.put_along_axis(out, np.asarray(perm, dtype=np.int64)[..., None], x, axis=-2)
    return out


def ba_forward_ranked(q, k, v, block: int, topk: int, scale: float):
    """BA-Att Algorithm 1 with norm ranking and without covariance compensation
    (beta = 0): rank Q by its token norms and K (with V) by theirs, pool, score
    and select on the ranked sequences, attend there, and return O and LSE in
    the original query order.  Returns (perm_q, perm_k, idx, O, LSE); idx
    indexes ranked key blocks.
    """
    pq, pk = norm_rank(q), norm_rank(k)
    qs = gather_rows(as_f64(q), pq)
    ks = gather_rows(as_f64(k), pk)
    vs = gather_rows(as_f64(v), pk)
    idx = topk_ascending(block_logits(pool_mean(qs, block), pool_mean(ks, block), scale), topk)
    o_s, lse_s = sparse_attention(qs, ks, vs, idx, block, block, scale)
    o = scatter_rows(o_s, pq)
    lse = scatter_rows(lse_s[..., None], pq)[..., 0]
    return pq, pk, idx, o, lse


# ---------------------------------------------------------------------------
# BA-Att, section 3.4 (Eq. 13-14) and Algorithm 1 steps 4, 6 and 7:
# covariance compensation of the block logits
# ---------------------------------------------------------------------------

def block_variance(x: np.ndarray, block: int) -> np.ndarray:
    """Population variance of every channel over each run of `block` tokens:
    [..., L, d] -> [..., L/block, d], the mean of (x - block mean)^2.

    The diagonal of the block covariance Sigma = E[dX dX^T] of BA-Att section
    3.4 (dX the deviation from the block mean, E over the block's tokens);
    Algorithm 1 step 4 computes it with the block means.
    """
    x = as_f64(x)
    length, d = x.shape[-2], x.shape[-1]
    xb = x.reshape(*x.shape[:-2], length // block, block, d)
    dev = xb - xb.mean(axis=-2, keepdims=True)
    return (dev * dev).mean(axis=-2)


def compensated_logits(qbar, kbar, qvar, kvar, scale: float, beta: float) -> np.ndarray:
    """BA-Att Eq. 13 with the diagonal approximation of Eq. 14, taken as printed:

        l~[gq, gk] = scale * Qbar_gq . Kbar_gk + beta * Delta[gq, gk],
        Delta = (1/d) sum_t (Var[Q_t]_gq Kbar_gk,t^2 + Var[K_t]_gk Qbar_gq,t^2
                             + Var[Q_t]_gq Var[K_t]_gk).

    qbar, qvar [B, Hq, Nq, d]; kbar, kvar [B, Hkv, Nk, d] (query head h reads
    key head h // (Hq/Hkv)); result [B, Hq, Nq, Nk].
    """
    qbar, kbar, qvar, kvar = (as_f64(a) for a in (qbar, kbar, qvar, kvar))
    group = qbar.shape[1] // kbar.shape[1]
    if group > 1:
        kbar = np.repeat(kbar, group, axis=1)
        kvar = np.repeat(kvar, group, axis=1)
    d = qbar.shape[-1]
    t = lambda a: np.swapaxes(a, -1, -2)
    delta = (qvar @ t(kbar * kbar) + (qbar * qbar) @ t(kvar) + qvar @ t(kvar)) / d
    return scale * (qbar @ t(kbar)) + beta * delta


def ba_forward_algorithm1(q, k, v, block: int, topk: int, scale: float, beta: float = 1.0,
                          rank: bool = True):
    """BA-Att Algorithm 1: norm ranking (steps 1-2, when rank), block means and
    variances (step 4), compensated logits (steps 5-7), per-row top-kappa
    (steps 8-11), block-sparse attention and the remap to token order (step
    12).  Returns (perm_q, perm_k, idx, O, LSE); the permutations are None
    without ranking.
    """
    pq = pk = None
    qs, ks, vs = as_f64(q), as_f64(k), as_f64(v)
    if rank:
        pq, pk = norm_rank(q), norm_rank(k)
        qs, ks, vs = gather_rows(qs, pq), gather_rows(ks, pk), gather_rows(vs, pk)
    scores = compensated_logits(pool_mean(qs, block), pool_mean(ks, block),
                                block_variance(qs, block), block_variance(ks, block), scale, beta)
    idx = topk_ascending(scores, topk)
    o, lse = sparse_attention(qs, ks, vs, idx, block, block, scale)
    if rank:
        o = scatter_rows(o, pq)
        lse = scatter_rows(lse[..., None], pq)[..., 0]
    return pq, pk, idx, o, lse


# ---------------------------------------------------------------------------
# Block mass of the dense attention map: BA-Att Eq. 3 (oracle block
# distribution) and SparseD section 3.3 (average-pooled attention scores,
# isolated top-rho% selection over prefill and generation keys, Eq. 5-6)
# ---------------------------------------------------------------------------

def block_mass(q, k, block: int, scale: float) -> np.ndarray:
    """m^[gq, gk] = (1/|I(gq)|) sum_{i in I(gq)} sum_{j in J(gk)} A_ij, BA-Att Eq. 3,
    with A = softmax(scale * Q K^T) the dense attention map of Eq. 1, row by
    row over all keys.  q [B, Hq, L, d], k [B, Hkv, L, d]; result
    [B, Hq, L/block, L/block].  SparseD's avgpool(A, block) is m^ / block.
    """
    q, k = as_f64(q), as_f64(k)
    nb_, hq, length, d = q.shape
    group = hq // k.shape[1]
    nq, nk = length // block, k.shape[2] // block
    out = np.empty((nb_, hq, nq, nk))
    for b in range(nb_):
        for h in range(hq):
            z = scale * (q[b, h] @ k[b, h // group].T)
            m = z.max(axis=-1, keepdims=True)
            e = np.exp(z - m)
            a = e / e.sum(axis=-1, keepdims=True)
            out[b, h] = a.reshape(nq, block, nk, block).sum(axis=(1, 3)) / block
    return out


def range_counts(n_pre: int, n_gen: int, rho: float) -> tuple[int, int]:
    """Blocks kept in each key range: ceil(rho * n) (at least rho of the range;
    the pages give the fraction, not the rounding), none for an empty range."""
    f = lambda n: 0 if n == 0 else min(n, max(1, math.ceil(rho * n - 1e-12)))
    return f(n_pre), f(n_gen)


def topk_in_ranges(scores, split: int, k_lo: int, k_hi: int) -> np.ndarray:
    """Per row, the k_lo best columns of [0, split) and the k_hi best of
    [split, n), each under (score descending, column ascending), returned
    together in ascending column order (int32 [..., k_lo + k_hi])."""
    scores = np.asarray(scores, dtype=np.float64)
    lo = topk_ascending(scores[..., :split], k_lo) if k_lo else np.zeros(scores.shape[:-1] + (0,), np.int32)
    hi = (topk_ascending(scores[..., split:], k_hi) + split) if k_hi else np.zeros(scores.shape[:-1] + (0,), np.int32)
    return np.concatenate([lo, hi], axis=-1).astype(np.int32)


def sparsed_pattern(q, k, block: int, scale: float, prefill: int, rho: float) -> np.ndarray:
    """SparseD isolated selection (section 3.3, Eq. 5-6) on query/key blocks:
    per query block, the top-rho% key blocks by average-pooled attention score
    among the prefill keys (tokens before `prefill`) and, separately, among the
    generation keys (the rest), united.  `prefill` must be a multiple of the
    block (the text of Eq. 6 ends inside the generation range's bounds; they
    are read as the complement of the prefill range)."""
    if prefill % block:
        raise ValueError("the prefill length must be a multiple of the block")
    m = block_mass(q, k, block, scale)
    split = prefill // block
    k_lo, k_hi = range_counts(split, m.shape[-1] - split, rho)
    return topk_in_ranges(m, split, k_lo, k_hi)


def sparsed_forward(q, k, v, block: int, scale: float, prefill: int, rho: float):
    """SparseD's sparse step: the pattern of sparsed_pattern (computed once from
    a dense step and reused) applied as the block mask of Eq. 3-4.  Returns
    (idx, O, LSE)."""
    idx = sparsed_pattern(q, k, block, scale, prefill, rho)
    o, lse = sparse_attention(q, k, v, idx, block, block, scale)
    return idx, o, lse


# ---------------------------------------------------------------------------
# Fidelity diagnostics: BA-Att Eq. 7-8 (block radii, max norms and the bound
# on the token/block logit deviation) and recall against the oracle block
# distribution of Eq. 3
# ---------------------------------------------------------------------------

def block_radius_maxnorm(x, block: int):
    """BA-Att Eq. 7: per block, R = max_i ||x_i - xbar||_2 (radius around the
    block mean) and M = max_i ||x_i||_2 (largest token norm).  [..., L, d] ->
    two [..., L/block] arrays."""
    x = as_f64(x)
    length, d = x.shape[-2], x.shape[-1]
    xb = x.reshape(*x.shape[:-2], length // block, block, d)
    dev = xb - xb.mean(axis=-2, keepdims=True)
    r = np.sqrt((dev * dev).sum(axis=-1)).max(axis=-1)
    m = np.sqrt((xb * xb).sum(axis=-1)).max(axis=-1)
    return r, m


def deviation_bound(rq, mq, rk, mk, d: int) -> np.ndarray:
    """BA-Att Eq. 8: U[gq, gk] = (R^Q M^K + M^Q R^K + R^Q R^K) / sqrt(d), the
    bound on |token logit - block logit| inside block pair (gq, gk) (scale
    1/sqrt(d)).  rq, mq [..., Nq]; rk, mk [..., Nk] (same leading shape)."""
    rq, mq, rk, mk = (np.asarray(a, dtype=np.float64)[..., :, None] if i < 2 else
                      np.asarray(a, dtype=np.float64)[..., None, :] for i, a in enumerate((rq, mq, rk, mk)))
    return (rq * mk + mq * rk + rq * rk) / math.sqrt(d)


def selection_recall(idx, mass) -> float:
    """Mean over rows of |S ∩ S*| / k: S the selected blocks idx [..., k], S*
    the k blocks of largest oracle block mass (BA-Att Eq. 3) in the same row
    (ties to the lower index)."""
    idx = np.asarray(idx)
    k = idx.shape[-1]
    best = topk_ascending(mass, k)
    hits = [len(set(a.tolist()) & set(b.tolist())) for a, b in
            zip(idx.reshape(-1, k), best.reshape(-1, k))]
    return float(np.mean(hits)) / k


# ---------------------------------------------------------------------------
# Log-linear (hierarchical) top-k, from the loglinear-sparse-dit README
# ---------------------------------------------------------------------------

def llsa_num_levels(n: int, block: int) -> int:
    """Number of coarse levels L: the largest L with block^(L+1) dividing n.

    The README supports only n that is a multiple of block^(L+1) and raises
    otherwise; we take the deepest L that the length allows.
    """
    if n % block:
        raise ValueError(f"sequence length {n} is not a multiple of block {block}")
    levels = 0
    while n % (block ** (levels + 2)) == 0:
        levels += 1
    return levels


def llsa_forward(q, k, v, block: int, topk: int, scale: float, levels: int | None = None,
                 with_attention: bool = True):
    """Coarse-to-fine per-token top-k and enriched attention for one batch.

    q, k, v [H, N, d].  Level l holds N / block^l tokens, each the mean of
    `block` tokens of level l-1 (queries, keys and values alike).  At the
    coarsest level L every token is a candidate; at every level each query
    keeps its own top-k among the candidates that its group of `block`
    consecutive queries shares, and the children of a kept token become the
    candidates of its children one level down.  Level 0 does no selection: its
    candidates are the surviving fine keys.  Attention runs over the fine keys
    plus every candidate at each coarser level l, with l*ln(block) added to
    their logits.

    Returns a dict: sel[l] int32 [H, N_l, topk] (ascending) for l = 1..L,
    cand[l] int32 [H, N_l / block, C_l] (ascending; the top level holds all
    tokens) for l = 0..L, levels, and O / LSE [H, N, d] / [H, N] when asked.
    """
    qs = [as_f64(q)]
    ks = [as_f64(k)]
    vs = [as_f64(v)]
    n_heads, n, d = qs[0].shape
    if levels is None:
        levels = llsa_num_levels(n, block)
    for _ in range(levels):
        qs.append(pool_mean(qs[-1], block))
        ks.append(pool_mean(ks[-1], block))
        vs.append(pool_mean(vs[-1], block))
    sizes = [x.shape[1] for x in qs]
    sel = {}
    cand = {}
    # coarsest level: one group holding every token
    cand[levels] = np.broadcast_to(np.arange(sizes[levels], dtype=np.int32),
                                   (n_heads, 1, sizes[levels])).copy()
    for lvl in range(levels, 0, -1):
        n_l = sizes[lvl]
        c = cand[lvl]
        group = n_l // c.shape[1]
        s_l = np.empty((n_heads, n_l, topk), dtype=np.int32)
        for h in range(n_heads):
            for a in range(n_l):
                cands = c[h, a // group]
                scores = scale * (ks[lvl][h, cands] @ qs[lvl][h, a])
                s_l[h, a] = cands[topk_ascending(scores, topk)]
        sel[lvl] = s_l
        # children of each selected token become the next level's candidates
        child = (s_l[..., :, None] * block + np.arange(block, dtype=np.int32)).reshape(
            n_heads, n_l, topk * block)
        cand[lvl - 1] = child
    out = {"sel": sel, "cand": cand, "levels": levels, "sizes": sizes}
    if not with_attention:
        return out
    o = np.empty((n_heads, n, vs[0].shape[-1]))
    lse = np.empty((n_heads, n))
    log_b = math.log(block)
    fine_group = n // cand[0].shape[1]
    for h in range(n_heads):
        for g in range(cand[0].shape[1]):
            rows = np.arange(g * fine_group, (g + 1) * fine_group)
            parts_k, parts_v, parts_b = [], [], []
            for lvl in range(levels + 1):
                c_l = cand[lvl]
                grp_l = sizes[lvl] // c_l.shape[1]
                a_l = (g * fine_group) // (block ** lvl)   # ancestor of the rows at level l
                idx = c_l[h, a_l // grp_l]
                parts_k.append(ks[lvl][h, idx])
                parts_v.append(vs[lvl][h, idx])
                parts_b.append(np.full(idx.size, lvl * log_b))
            kk = np.concatenate(parts_k)
            vv = np.concatenate(parts_v)
            bb = np.concatenate(parts_b)
            z = scale * (qs[0][h, rows] @ kk.T) + bb[None, :]
            m = z.max(axis=1, keepdims=True)
            e = np.exp(z - m)
            s = e.sum(axis=1, keepdims=True)
            o[h, rows] = (e @ vv) / s
            lse[h, rows] = (m + np.log(s))[:, 0]
    out["o"] = o
    out["lse"] = lse
    return out


def llsa_keys_per_query(n: int, block: int, topk: int) -> int:
    """Keys each fine query attends to, counted from the candidate structure
    that llsa_forward builds (selection run on random data of width 1)."""
    g = np.random.Generator(np.random.PCG64(0))
    x = g.standard_normal((1, n, 1))
    res = llsa_forward(x, x, x, block, topk, 1.0, with_attention=False)
    return int(sum(res["cand"][lvl].shape[-1] for lvl in range(res["levels"] + 1)))


# ---------------------------------------------------------------------------
# LoSA denoising step (Locality-aware Sparse Attention blog post)
# ---------------------------------------------------------------------------

def token_change(q_cur, q_prev) -> np.ndarray:
    """Per-token mean squared change of the query between two denoising steps,
    averaged over every head and channel: [B, H, T, d] x2 -> [B, T]."""
    diff = as_f64(q_cur) - as_f64(q_prev)
    return (diff * diff).mean(axis=(1, 3))


def active_tokens(q_cur, q_prev, n_active: int) -> np.ndarray:
    """The n_active tokens with the largest query change (ties: lower token),
    in ascending token order: [B, n_active] int32 (LoSA locality pruning)."""
    return topk_ascending(token_change(q_cur, q_prev), n_active)


def losa_step(q_cur, q_prev, k_prefix, v_prefix, k_block, v_block, cache_o, cache_lse,
              n_active: int, block: int, topk: int, scale: float):
    """One denoising step of a block with locality-aware prefix reuse.

    q_* [B, Hq, T, d]; k/v_prefix [B, Hkv, P, d]; k/v_block [B, Hkv, T, d];
    cache_o [B, Hq, T, d], cache_lse [B, Hq, T]: prefix attention results of
    the previous step.  Steps, in the post's order:
      1. active tokens = top n_active by query MSE; the rest are stable;
      2. every (active token, query head) scores the mean-pooled prefix key
         blocks with its own query and keeps its top-`topk` blocks;
      3. active rows get fresh sparse prefix attention, written into the
         cache (this is the cache update); stable rows keep the cached values;
      4. every token attends densely to the block's own keys (in-block);
      5. prefix and in-block results are merged by online softmax.
    Returns active, sel [B, Hq, n_active, topk], O, LSE, new cache O/LSE,
    and the in-block partials.
    """
    nb, hq, t_len, d = np.asarray(q_cur).shape
    hkv = np.asarray(k_prefix).shape[1]
    group = hq // hkv
    act = active_tokens(q_cur, q_prev, n_active)
    qc = as_f64(q_cur)
    kbar = pool_mean(k_prefix, block)                      # [B, Hkv, P/block, d]
    sel = np.empty((nb, hq, n_active, topk), dtype=np.int32)
    new_o = as_f64(cache_o).copy()
    new_lse = np.asarray(cache_lse, dtype=np.float64).copy()
    for b in range(nb):
        for h in range(hq):
            if h % group == 0:
                kh = as_f64(k_prefix[b, h // group])
                vh = as_f64(v_prefix[b, h // group])
            for j, t in enumerate(act[b]):
                scores = scale * (kbar[b, h // group] @ qc[b, h, t])
                sel[b, h, j] = topk_ascending(scores, topk)
                o_t, lse_t = attend_rows(qc[b, h, t][None, :], kh, vh, sel[b, h, j], block, scale)
                new_o[b, h, t] = o_t[0]
                new_lse[b, h, t] = lse_t[0]
    o_in, lse_in = dense_attention(qc, k_block, v_block, scale)
    o, lse = merge(new_o, new_lse, o_in, lse_in)
    return {"active": act, "sel": sel, "o": o, "lse": lse, "cache_o": new_o,
            "cache_lse": new_lse, "o_in": o_in, "lse_in": lse_in}
