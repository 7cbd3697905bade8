"""Throughput of the block-sparse attention path on one MI355X.

A step is one pass of the selection + attention path over the 64K-token
workload (batch 1, 32 heads, 65536 tokens, head_dim 128, block 128, top-128
of 512 key blocks per query block, bf16): pool Q, pool K, block scores +
top-k, block-sparse attention emitting O (bf16) and LSE (float32).  Inputs are
seeded synthetic tensors already resident in HBM when timing starts.

The headline value is kept-block attention TFLOP/s of the whole step
(4 * 128^3 flops per kept (query block, key block) pair, nothing else
counted).  Also reported: per-kernel times from HIP events on the launch
stream, the roofline of the attention kernel, the two-way LSE merge on
64K-shaped partials, and the fp64 CPU oracle on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA (256 CUs x 2.4 GHz x 4096 flop/clk)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E

# HBM traffic of one attention-kernel launch on this workload, from rocprofv3 --pmc
# FETCH_SIZE and WRITE_SIZE (separate runs), each scaled by the same counter on a 1 GiB
# device copy (factors 2.0 and 1.0); see profiles/attn_mfma_dlm64k.md.  Valid only for
# the kernel source it was measured on (first 16 hex digits of its sha256).
MEASURED_ATTN_TRAFFIC = {"source_sha256": "444d31f91ea40271", "fetch_bytes": 27.525e9, "write_bytes": 0.547e9}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="dlm64k", choices=["dlm64k", "dlm16k"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-stages", action="store_true", help="skip the merge stage measurement")
    p.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                   help="only run a device-to-device copy of BYTES bytes 5 times (calibrates the "
                        "HBM byte counters of a profiler run) and exit")
    return p.parse_args()


def copy_probe(nbytes: int) -> None:
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "reps": 5}))


def attn_traffic(workload: str):
    """Counter-measured HBM bytes of one attention launch, or None when the kernel source
    changed since the counters were taken (or for another workload)."""
    import hashlib
    src = os.path.join(ROOT, "block_sparse_attention_mean_amd", "csrc", "attn_mfma.hip")
    h = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    m = MEASURED_ATTN_TRAFFIC
    if workload != "dlm64k" or h != m["source_sha256"]:
        return None
    return m["fetch_bytes"] + m["write_bytes"]


def wl_bf16_to_f64(a) -> "np.ndarray":
    """bf16 bit patterns (uint16) or floats -> float64, exactly."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(x, w, budget_s: float = 15.0) -> dict:
    """The fp64 C++ oracle (oracle/basa_oracle_ref.cpp, OpenMP over query
    tiles), as it stands, on a bounded sample of the same workload: pooling +
    block logits + top-k of head 0, then batches of head 0's query tiles (one
    tile per thread) until the time budget is used.  Extrapolated linearly to
    the whole step (all heads, all tiles) and expressed in the GPU value's unit."""
    import oracle.cref as cref
    threads = cref.threads()
    h = 0
    t0 = time.perf_counter()
    qb = cref.pool_mean(x["q"][:, h:h + 1], w.block)
    kb = cref.pool_mean(x["k"][:, h:h + 1], w.block)
    idx = cref.topk_ascending(cref.block_logits(qb, kb, w.scale), w.topk)
    t_sel_head = time.perf_counter() - t0
    # the head's keys and values widened to float64 once (exact), outside the timed loop
    kh, vh = (np.ascontiguousarray(wl_bf16_to_f64(x[n][:, h:h + 1])) for n in ("k", "v"))
    tiles = 0
    t1 = time.perf_counter()
    while tiles < w.blocks and (tiles == 0 or time.perf_counter() - t1 < budget_s):
        n = min(threads, w.blocks - tiles)
        cref.sparse_attention(x["q"][:, h:h + 1, tiles * w.block:(tiles + n) * w.block], kh, vh,
                              idx[:, :, tiles:tiles + n], w.block, w.block, w.scale)
        tiles += n
    t_tile = (time.perf_counter() - t1) / tiles
    est = t_sel_head * w.heads + t_tile * w.heads * w.blocks
    flops = 4.0 * w.block ** 3 * w.heads * w.blocks * w.topk
    return {"value": flops / est / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "nproc": os.cpu_count(), "cpu": _cpu_model(),
            "sample": f"fp64 C++ oracle, {threads} OpenMP threads: head 0 pool+score+top-k "
                      f"({t_sel_head:.2f} s) and {tiles} of {w.blocks} query tiles of attention "
                      f"({t_tile * threads:.2f} s per batch of {threads}); scaled linearly to "
                      f"{w.heads} heads (est. {est:.0f} s for the whole step)"}


def measured_peaks(torch) -> dict:
    """Peaks measured on this GPU by the probe kernels of libbasa_peak.so: a
    bf16 matrix-core loop (8 independent 32x32x16 MFMA chains per wave, two
    4-wave workgroups per CU: the attention kernel's occupancy, all resident,
    about 0.15 s per call) and streaming HBM kernels (a 4 GiB read, a 2 GiB
    copy).  Each figure is the median of three timed calls after one warm-up."""
    import ctypes
    import statistics
    here = os.path.join(ROOT, "block_sparse_attention_mean_amd")
    lib = ctypes.CDLL(os.path.join(here, "libbasa_peak.so"))
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.peak_mfma_flops.restype = ctypes.c_double
    lib.peak_mfma_flops.argtypes = [i64, ctypes.c_int]
    lib.peak_mfma_bf16.argtypes = [vp, vp, i64, ctypes.c_int, vp]
    lib.peak_hbm_read.argtypes = [vp, i64, vp, i64, vp]
    lib.peak_hbm_copy.argtypes = [vp, vp, i64, i64, vp]
    stream = torch.cuda.current_stream().cuda_stream
    g = torch.Generator(device="cuda").manual_seed(5)
    seed = torch.randn(4160 * 8, device="cuda", generator=g).to(torch.bfloat16)
    wgs, iters = 512, 500
    out = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")

    def timed(fn, reps=3):
        fn()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return statistics.median(ts)

    def mfma():
        assert lib.peak_mfma_bf16(seed.data_ptr(), out.data_ptr(), wgs, iters, stream) == 0
    t_mfma = timed(mfma)
    nread = 4 << 30
    src = torch.empty(nread, dtype=torch.uint8, device="cuda").fill_(7)
    sums = torch.empty(8192 * 256, dtype=torch.int32, device="cuda")

    def rd():
        assert lib.peak_hbm_read(src.data_ptr(), nread, sums.data_ptr(), 8192, stream) == 0
    t_read = timed(rd)
    ncopy = 2 << 30
    dst = torch.empty(ncopy, dtype=torch.uint8, device="cuda")

    def cp():
        assert lib.peak_hbm_copy(src.data_ptr(), dst.data_ptr(), ncopy, 8192, stream) == 0
    t_copy = timed(cp)
    del src, dst, sums, out
    return {"bf16_mfma_TFLOP/s": lib.peak_mfma_flops(wgs, iters) / t_mfma / 1e12,
            "hbm_read_GB/s": nread / t_read / 1e9, "hbm_copy_GB/s": 2 * ncopy / t_copy / 1e9,
            "note": "bf16 MFMA loop at the attention kernel's occupancy; streaming 4 GiB read and "
                    "2 GiB copy (read + write bytes); medians of 3 calls after a warm-up"}


def _time(torch, fn, reps=10):
    """Average wall time of fn() over reps calls, bracketed by HIP events on the launch stream."""
    fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def ranked_stage(torch, basa, q, k, v, w) -> dict:
    """BA-Att with norm-based ranking (section 3.3) on the same 64K inputs:
    ranking of Q and K (squared norms + stable radix sorts), the gathers of
    Q, K, V into ranked order, the whole ranked forward (rank, pool, select,
    attend, scatter of O and LSE back to token order), and the same with the
    covariance compensation of section 3.4 (beta = 1): its moments + selection
    stage and the whole Algorithm 1 forward."""
    from block_sparse_attention_mean_amd.pipelines import BaRankedForward
    f = BaRankedForward(q, k, v, w.block, w.topk, w.scale)
    t_rank = _time(torch, lambda: (basa.basa_rank(q, f.perm_q, f.workspace),
                                   basa.basa_rank(k, f.perm_k, f.workspace)))
    t_gather = _time(torch, lambda: (basa.basa_permute(q, f.perm_q, f.qs),
                                     basa.basa_permute(k, f.perm_k, f.ks),
                                     basa.basa_permute(v, f.perm_k, f.vs)))
    t_fwd = _time(torch, f.run, reps=5)
    del f
    # the whole of Algorithm 1: ranking plus covariance compensation (beta = 1)
    g = BaRankedForward(q, k, v, w.block, w.topk, w.scale, beta=1.0)
    g.rank()
    t_comp_sel = _time(torch, g.select)
    t_alg1 = _time(torch, g.run, reps=5)
    tensor = q.numel() * q.element_size()
    flops = 4.0 * w.block ** 3 * w.heads * w.blocks * w.topk
    out = {
        "rank_q_k": {"ms": t_rank, "read_GB/s": 2 * tensor / (t_rank * 1e-3) / 1e9},
        "gather_q_k_v": {"ms": t_gather, "GB/s": 6 * tensor / (t_gather * 1e-3) / 1e9,
                         "frac_hbm": 6 * tensor / (t_gather * 1e-3) / 1e9 / PEAK_HBM_GBS},
        "forward_ms": t_fwd, "forward_TFLOP/s": flops / (t_fwd * 1e-3) / 1e12,
        "compensated_pool_select_ms": t_comp_sel,
        "algorithm1_forward_ms": t_alg1, "algorithm1_TFLOP/s": flops / (t_alg1 * 1e-3) / 1e12,
    }
    del g
    return out


def sparsed_stage(torch, wl, basa) -> dict:
    """SparseD (section 3.3) on the 16K DLM-shaped workload, prefill 8192,
    rho 0.3: the dense float64 block mass of the attention map (computed once
    per pattern), the isolated range selection, and the block-sparse attention
    that reuses the pattern."""
    from block_sparse_attention_mean_amd.pipelines import SparsedForward

    def dev(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()

    w = wl.WORKLOADS["dlm16k"]
    x = wl.generate("dlm16k")
    f = SparsedForward(dev(x["q"]), dev(x["k"]), dev(x["v"]), w.block, w.tokens // 2, 0.3, w.scale)
    t_mass = _time(torch, lambda: basa.basa_block_mass(f.q, f.k, w.block, f.mass, f.scale,
                                                       workspace=f.mass_ws), reps=2)
    t_mass2 = _time(torch, lambda: basa.basa_block_mass(f.q, f.k, w.block, f.mass, f.scale), reps=2)
    t_sel = _time(torch, lambda: basa.basa_select_ranges(f.mass, f.split, f.k_lo, f.k_hi, f.idx))
    f.pattern()
    t_attn = _time(torch, f.attend)
    dense_fp64 = 2.0 * w.heads * w.tokens * w.tokens * w.head_dim  # one Q K^T product
    kept = f.k_lo + f.k_hi
    out = {"block_mass_ms": t_mass, "block_mass_fp64_TFLOP/s": dense_fp64 / (t_mass * 1e-3) / 1e12,
           "block_mass_frac_fp64": dense_fp64 / (t_mass * 1e-3) / 1e12 / 78.6,
           "block_mass_two_pass_ms": t_mass2,
           "block_mass_note": "algorithmic flops: one float64 scale*Q*K^T product; the one-pass form "
                              "(workspace) computes it once, the two-pass form twice",
           "select_ranges_ms": t_sel, "kept_blocks": kept, "attn_ms": t_attn,
           "attn_TFLOP/s": 4.0 * w.block ** 3 * w.heads * w.blocks * kept / (t_attn * 1e-3) / 1e12}
    del f
    return out


def fidelity_stage(torch, wl, basa) -> dict:
    """Fidelity diagnostics on the 16K DLM-shaped workload (BA-Att Eq. 3 and
    Eq. 7-8): for the plain, norm-ranked and Algorithm 1 (ranked and
    compensated, beta 1) selections, the recall of each query block's kept
    set against the top-k of the dense block mass of its own block partition,
    and the mean over block pairs of the logit-deviation bound U of Eq. 8.
    Kernels compute the selections, masses, top-k and block radii; the host
    only counts set overlaps and averages."""
    import math
    import block_sparse_attention_mean_amd.pipelines as pl

    def dev(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()

    w = wl.WORKLOADS["dlm16k"]
    x = wl.generate("dlm16k")
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    nb, kk = w.blocks, w.topk
    mass = torch.empty(1, w.heads, nb, nb, dtype=torch.float64, device="cuda")
    best = torch.empty(1, w.heads, nb, kk, dtype=torch.int32, device="cuda")
    rad_q = torch.empty(1, w.heads, nb, 2, dtype=torch.float64, device="cuda")
    rad_k = torch.empty_like(rad_q)
    out = {}
    for name, beta, ranked in (("plain", None, False), ("ranked", None, True), ("algorithm1", 1.0, True)):
        if ranked:
            f = pl.BaRankedForward(q, k, v, w.block, kk, w.scale, beta=beta)
            f.rank()
            qp, kp = f.qs, f.ks
        else:
            f = pl.BaForward(q, k, v, w.block, kk, w.scale)
            qp, kp = q, k
        f.select()
        basa.basa_block_mass(qp, kp, w.block, mass, w.scale)
        basa.basa_select_ranges(mass, nb, kk, 0, best)
        basa.basa_block_radius(qp, w.block, rad_q)
        basa.basa_block_radius(kp, w.block, rad_k)
        torch.cuda.synchronize()
        idx, top = f.idx.cpu().numpy(), best.cpu().numpy()
        hits = (idx[..., :, None] == top[..., None, :]).any(-1).sum(-1)
        rq, mq = rad_q[..., 0].mean(-1).cpu().numpy(), rad_q[..., 1].mean(-1).cpu().numpy()
        rk, mk = rad_k[..., 0].mean(-1).cpu().numpy(), rad_k[..., 1].mean(-1).cpu().numpy()
        u = (rq * mk + mq * rk + rq * rk) / math.sqrt(w.head_dim)  # mean over pairs, per head
        out[name] = {"recall_vs_block_mass_topk": float(hits.mean()) / kk, "mean_U": float(u.mean())}
        del f
    return out


def llsa_and_losa_stages(torch, wl, basa) -> dict:
    """The hierarchical (log-linear) forward on the 256x256-image workload and the
    LoSA prefix step on the 64K-prefix workload, each with its fraction of the
    HBM peak on algorithmic bytes (the bytes the step cannot avoid moving)."""
    import math
    import block_sparse_attention_mean_amd.pipelines as pl

    def dev(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()

    out = {}
    x = wl.generate("llsa64k")
    f = pl.LlsaForward(dev(x["q"]), dev(x["k"]), dev(x["v"]), 16, 8, 1.0 / 8)
    t_pool, t_sel, t_attn = _time(torch, f.pool), _time(torch, f.select), _time(torch, f.attend)
    n, h, d = 65536, 4, 64
    keys = 400
    flops = 4.0 * h * n * keys * d
    tensor = h * n * d * 2
    # Q, K, V read once, O (bf16) and LSE (float32) written once
    llsa_bytes = 3 * tensor + tensor + h * n * 4
    t_all = t_pool + t_sel + t_attn
    out["llsa64k"] = {"ms": t_all, "pool_ms": t_pool, "select_ms": t_sel,
                      "attn_ms": t_attn, "attn_TFLOP/s": flops / (t_attn * 1e-3) / 1e12,
                      "attn_frac_mfma": flops / (t_attn * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                      "algorithmic_bytes": llsa_bytes,
                      "frac_hbm": llsa_bytes / (t_all * 1e-3) / 1e9 / PEAK_HBM_GBS,
                      "keys_per_query": keys,
                      "bound": "latency of the gathered 16-key blocks (400 keys per query, "
                               "16 queries per tile); neither HBM nor the matrix core is near its peak"}
    y = wl.make_losa(1004)
    hq, t, dd = 32, 16, 128
    cache_o = torch.zeros(1, hq, t, dd, dtype=torch.float32, device="cuda")
    cache_lse = torch.zeros(1, hq, t, dtype=torch.float32, device="cuda")
    s = pl.LosaStep(dev(y["q_cur"]), dev(y["q_prev"]), dev(y["k_prefix"]), dev(y["v_prefix"]),
                    dev(y["k_block"]), dev(y["v_block"]), cache_o, cache_lse, 5, 16, 128,
                    1.0 / math.sqrt(128))
    t_prep = _time(torch, s.prepare)
    t_step = _time(torch, s.step)
    torch.cuda.synchronize()
    # algorithmic bytes of a step: the union over each key head's active rows of the kept
    # prefix blocks (K and V, bf16), the pooled prefix keys read by the selection (float64),
    # the queries, the block's K/V, and the cache rows and outputs
    sel = s.sel.cpu().numpy()[0]                      # [Hq, n_active, topk]
    hkv = y["k_prefix"].shape[1]
    grp = hq // hkv
    union = sum(len(np.unique(sel[g * grp:(g + 1) * grp])) for g in range(hkv))
    union_bytes = union * 16 * dd * 2 * 2
    kbar_bytes = hkv * (y["k_prefix"].shape[2] // 16) * dd * 8
    small = 2 * hq * t * dd * 2 + 2 * hkv * t * dd * 2 + 2 * hq * t * (dd * 4 + 4) + hq * t * (dd * 2 + 4)
    step_bytes = union_bytes + kbar_bytes + small
    seg = basa.kv_segment(s.sel, s.k_prefix, s.v_prefix)
    kw = dict(tile_q=1, block_k=16, scale=s.scale, q_rows=s.active)
    t_prefix = _time(torch, basa.prepare_attn(s.q_cur, seg, s.cache_o, s.cache_lse, **kw))
    # the same prefix attention as one walk over each key head's union of kept blocks
    ws = torch.empty(basa.basa_attn_workspace(s.q_cur, seg, s.cache_o, s.cache_lse, **kw),
                     dtype=torch.uint8, device="cuda")
    t_union = _time(torch, basa.prepare_attn(s.q_cur, seg, s.cache_o, s.cache_lse, workspace=ws, **kw))
    out["losa64k_step"] = {"ms": t_step, "prefix_pool_ms": t_prep,
                           "union_blocks": int(union), "union_kv_bytes": union_bytes,
                           "algorithmic_bytes": step_bytes,
                           "frac_hbm": step_bytes / (t_step * 1e-3) / 1e9 / PEAK_HBM_GBS,
                           "prefix_attn_ms": t_prefix,
                           "prefix_attn_frac_hbm": union_bytes / (t_prefix * 1e-3) / 1e9 / PEAK_HBM_GBS,
                           "prefix_attn_union_walk_ms": t_union,
                           "prefix_attn_union_walk_frac_hbm": union_bytes / (t_union * 1e-3) / 1e9
                           / PEAK_HBM_GBS,
                           "note": "per denoising step: active-token pick, selection, sparse prefix "
                                   "attention for 5 tokens x 32 heads, in-block attention, merge"}
    return out


def main():
    args = parse()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the path shards by "
              "(batch, head) with no exchange, so N GPUs run N independent copies.", file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads as wl
    import block_sparse_attention_mean_amd as basa
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    w = wl.WORKLOADS[args.workload]
    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    x = wl.generate(w.name)

    def dev(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()

    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    nb = w.blocks
    from block_sparse_attention_mean_amd.pipelines import BaForward
    fw = BaForward(q, k, v, w.block, w.topk, w.scale)
    qbar, kbt, idx, o, lse = fw.qbar, fw.kbt, fw.idx, fw.o, fw.lse

    ev = {name: [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps)]
          for name in ("select", "attn")}

    def step(i=None):
        # one pass of the hot path: pool Q and K, score and select, block-sparse attention
        if i is not None:
            ev["select"][2 * i].record()
        fw.select()
        if i is not None:
            ev["select"][2 * i + 1].record()
            ev["attn"][2 * i].record()
        fw.attend()
        if i is not None:
            ev["attn"][2 * i + 1].record()

    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("[bench] timing", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps

    def avg_ms(name):
        e = ev[name]
        return sum(e[2 * i].elapsed_time(e[2 * i + 1]) for i in range(args.steps)) / args.steps

    t_ps, t_attn = avg_ms("select"), avg_ms("attn")

    # the pooling and the selection alone (per-kernel figures)
    t_pool = _time(torch, lambda: (basa.basa_pool(q, w.block, mean_rows=qbar),
                                   basa.basa_pool(k, w.block, mean_cols=kbt)))
    t_sel = _time(torch, lambda: basa.basa_select(qbar, kbt, idx, w.topk, scale=w.scale))
    kept_pairs = w.heads * nb * w.topk
    flops = 4.0 * w.block ** 3 * kept_pairs
    tflops = flops / (ms_step * 1e-3) / 1e12
    attn_tflops = flops / (t_attn * 1e-3) / 1e12
    pool_bytes = 2 * (w.heads * w.tokens * w.head_dim * 2) + 2 * (w.heads * nb * w.head_dim * 8)
    sel_bytes = 2 * (w.heads * nb * w.head_dim * 8) + w.heads * nb * w.topk * 4
    # pool+select, algorithmic: Q and K read once (bf16) + the int32 kept indices written
    ps_bytes = 2 * (w.heads * w.tokens * w.head_dim * 2) + w.heads * nb * w.topk * 4

    stages = {
        "pool_q_k": {"ms": t_pool, "GB/s": pool_bytes / (t_pool * 1e-3) / 1e9,
                     "frac_hbm": pool_bytes / (t_pool * 1e-3) / 1e9 / PEAK_HBM_GBS},
        "select": {"ms": t_sel, "GB/s": sel_bytes / (t_sel * 1e-3) / 1e9,
                   "fp64_GFLOP/s": 2.0 * w.heads * nb * nb * w.head_dim / (t_sel * 1e-3) / 1e9},
        "pool+select": {"ms": t_ps, "algorithmic_bytes": ps_bytes,
                        "GB/s": ps_bytes / (t_ps * 1e-3) / 1e9,
                        "frac_hbm": ps_bytes / (t_ps * 1e-3) / 1e9 / PEAK_HBM_GBS,
                        "intermediate_bytes": 2 * 2 * (w.heads * nb * w.head_dim * 8),
                        "note": "algorithmic bytes: Q and K read once, kept indices written; the "
                                "float64 block means (written by the pooling, read by the "
                                "selection) are listed apart as intermediate_bytes"},
        "attn": {"ms": t_attn, "TFLOP/s": attn_tflops},
    }

    if not args.no_stages:
        # two-way LSE merge on 64K-shaped partials: each row's kept list split in
        # two halves, each half's attention written as float32 O + LSE, merged to bf16
        half = w.topk // 2
        oa = torch.empty(q.shape, dtype=torch.float32, device="cuda")
        ob = torch.empty_like(oa)
        la = torch.empty_like(lse)
        lb = torch.empty_like(lse)
        sa = basa.kv_segment(idx, k, v, count=half, offset=0)
        sb = basa.kv_segment(idx, k, v, count=w.topk - half, offset=half)
        basa.basa_attn(q, sa, oa, la, tile_q=w.block, block_k=w.block, scale=w.scale)
        basa.basa_attn(q, sb, ob, lb, tile_q=w.block, block_k=w.block, scale=w.scale)
        om = torch.empty_like(o)
        lm = torch.empty_like(lse)
        reps = 10
        basa.basa_merge(oa, la, ob, lb, om, lm)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            basa.basa_merge(oa, la, ob, lb, om, lm)
        e1.record()
        torch.cuda.synchronize()
        t_merge = e0.elapsed_time(e1) / reps
        merge_bytes = 2 * (oa.numel() * 4 + la.numel() * 4) + om.numel() * 2 + lm.numel() * 4
        stages["merge"] = {"ms": t_merge, "GB/s": merge_bytes / (t_merge * 1e-3) / 1e9,
                           "frac_hbm": merge_bytes / (t_merge * 1e-3) / 1e9 / PEAK_HBM_GBS,
                           "max_abs_vs_one_shot": float((om.float() - o.float()).abs().max())}
        del oa, ob, la, lb, om, lm
        stages["ranked64k"] = ranked_stage(torch, basa, q, k, v, w)
        stages["sparsed16k"] = sparsed_stage(torch, wl, basa)
        stages["fidelity16k"] = fidelity_stage(torch, wl, basa)
        stages.update(llsa_and_losa_stages(torch, wl, basa))

    result = {
        "metric": "block-sparse attn TFLOP/s (kept blocks) + % MFMA peak at L=64K, d=128",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: batch 1, {w.heads} heads, L={w.tokens}, d={w.head_dim}, "
                               f"block {w.block}, top-{w.topk} of {nb} key blocks, bidirectional",
                   "global_batch": 1, "seq_len": w.tokens, "parallelism": "none"},
        "roofline": {"bound": "mfma", "achieved": attn_tflops, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": attn_tflops / PEAK_BF16_TFLOPS,
                     "traffic": attn_traffic(w.name)},
        "pct_mfma_peak_step": 100.0 * tflops / PEAK_BF16_TFLOPS,
        "stages": stages,
    }
    if not args.no_stages:
        peaks = measured_peaks(torch)
        result["measured_peaks"] = peaks
        result["roofline"]["peak_measured"] = peaks["bf16_mfma_TFLOP/s"]
        result["roofline"]["frac_of_measured"] = attn_tflops / peaks["bf16_mfma_TFLOP/s"]
        for name in ("pool_q_k", "merge"):
            if name in stages and "GB/s" in stages[name]:
                stages[name]["frac_of_measured_read"] = stages[name]["GB/s"] / peaks["hbm_read_GB/s"]
        stages["pool+select"]["frac_of_measured_read"] = (stages["pool+select"]["GB/s"]
                                                          / peaks["hbm_read_GB/s"])
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (fp64 C++ oracle, bounded sample)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(x, w)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
