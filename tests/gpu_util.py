"""Helpers for the GPU tests: move seeded numpy inputs to the device and read
results back, and measure the largest difference between two results.  Only
marshalling and comparison; no arithmetic of the method."""
import math

import numpy as np
import torch


def dev(x: np.ndarray) -> torch.Tensor:
    """numpy -> contiguous tensor on cuda:0 (uint16 arrays become bf16)."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    """device tensor -> float64/int numpy (bf16 widened exactly)."""
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float32):
        return t.to(torch.float64).numpy()
    return t.numpy()


def max_err(a, b) -> float:
    """Largest |a - b| over all elements, strict about non-finite values.

    A NaN on either side is an infinite error: a kernel that writes NaN fails,
    and rows the oracle did not compute (it marks them NaN) must be masked out
    by the caller before the comparison.  Infinities count as equal only when
    both sides hold the same one (an empty row's LSE of -inf); any other
    infinity is an infinite error.  Shapes must match exactly."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.shape != b.shape:
        raise ValueError(f"shapes differ: {a.shape} vs {b.shape}")
    if a.size == 0:
        return 0.0
    if np.isnan(a).any() or np.isnan(b).any():
        return math.inf
    inf_a, inf_b = np.isinf(a), np.isinf(b)
    if (inf_a != inf_b).any() or (a[inf_a] != b[inf_a]).any():
        return math.inf
    fin = ~inf_a
    return float(np.abs(a[fin] - b[fin]).max()) if fin.any() else 0.0


# Parity bar for bf16 inputs with float32 accumulation
O_TOL = 2e-2
LSE_TOL = 1e-3


def note(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)


def scale_of(d: int) -> float:
    return 1.0 / math.sqrt(d)


def stratified_tiles(heads: int, blocks: int, every: int = 8, batch: int = 0):
    """Every `every`-th query tile of every head, the residue turning with the
    head (tile t of head h when (t - h) % every == 0), so that the sample spans
    all tile positions across heads."""
    return [(batch, h, t) for h in range(heads) for t in range(h % every, blocks, every)]


def check_tiles_against_oracle(o, lse, q, k, v, idx, tiles, tile_q: int, block_k: int,
                               scale: float, workers: int = 8):
    """Compare the rows of each listed (b, h, t) query tile of a GPU result
    (o [B,Hq,L,d], lse [B,Hq,L] on the host) with the oracle's attention over
    the same key list (oracle.attend_rows, one tile at a time; query head h
    reads key head h // (Hq/Hkv)).  Tiles of one head run in one worker
    thread, its K and V widened once.  Returns (max O error, max LSE error)."""
    import concurrent.futures

    import oracle as orc

    group = q.shape[1] // k.shape[1]
    by_head = {}
    for b, h, t in tiles:
        by_head.setdefault((b, h), []).append(t)

    def one_head(key):
        b, h = key
        kh, vh = orc.as_f64(k[b, h // group]), orc.as_f64(v[b, h // group])
        eo = el = 0.0
        for t in by_head[key]:
            rows = slice(t * tile_q, (t + 1) * tile_q)
            ro, rl = orc.attend_rows(q[b, h, rows], kh, vh, idx[b, h, t], block_k, scale)
            eo = max(eo, max_err(o[b, h, rows], ro))
            el = max(el, max_err(lse[b, h, rows], rl))
        return eo, el

    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=2), \
            concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        errs = list(ex.map(one_head, sorted(by_head)))
    return max(e[0] for e in errs), max(e[1] for e in errs)
