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
MEASURED_ATTN_TRAFFIC = {"source_sha256": "789418d3b06499cb", "fetch_bytes": 53.010e9, "write_bytes": 0.546e9}


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


def cpu_baseline(x, w, budget_s: float = 12.0) -> dict:
    """The fp64 oracle, as it stands, on a bounded sample of the same workload:
    pooling + scoring + top-k of one head, then whole query tiles of that head's
    attention until the time budget is used.  Extrapolated linearly to the whole
    step and expressed in the same unit as the GPU value."""
    import oracle as orc
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = 1
    h = 0
    t0 = time.perf_counter()
    qb = orc.pool_mean(x["q"][:, h:h + 1], w.block)
    kb = orc.pool_mean(x["k"][:, h:h + 1], w.block)
    idx = orc.topk_ascending(orc.block_logits(qb, kb, w.scale), w.topk)
    t_sel_head = time.perf_counter() - t0
    kh, vh = orc.as_f64(x["k"][0, h]), orc.as_f64(x["v"][0, h])
    tiles = 0
    t1 = time.perf_counter()
    while tiles < 2 or (time.perf_counter() - t1 < budget_s and tiles < w.blocks):
        rows = x["q"][0, h, tiles * w.block:(tiles + 1) * w.block]
        orc.attend_rows(rows, kh, vh, idx[0, 0, tiles], w.block, w.scale)
        tiles += 1
    t_tile = (time.perf_counter() - t1) / tiles
    est = t_sel_head * w.heads + t_tile * w.heads * w.blocks
    flops = 4.0 * w.block ** 3 * w.heads * w.blocks * w.topk
    return {"value": flops / est / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"head 0: pool+score+top-k ({t_sel_head:.2f} s) and {tiles} of {w.blocks} "
                      f"query tiles of attention ({t_tile:.3f} s each); scaled linearly to "
                      f"{w.heads} heads (est. {est:.0f} s for the whole step)"}


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
    t_mass = _time(torch, lambda: basa.basa_block_mass(f.q, f.k, w.block, f.mass, f.scale), reps=2)
    t_sel = _time(torch, lambda: basa.basa_select_ranges(f.mass, f.split, f.k_lo, f.k_hi, f.idx))
    f.pattern()
    t_attn = _time(torch, f.attend)
    dense_fp64 = 2 * 2.0 * w.heads * w.tokens * w.tokens * w.head_dim  # two Q K^T passes
    kept = f.k_lo + f.k_hi
    out = {"block_mass_ms": t_mass, "block_mass_fp64_TFLOP/s": dense_fp64 / (t_mass * 1e-3) / 1e12,
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
    LoSA prefix step on the 64K-prefix workload."""
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
    out["llsa64k"] = {"ms": t_pool + t_sel + t_attn, "pool_ms": t_pool, "select_ms": t_sel,
                      "attn_ms": t_attn, "attn_TFLOP/s": flops / (t_attn * 1e-3) / 1e12,
                      "keys_per_query": keys}
    y = wl.make_losa(1004)
    hq, t, dd = 32, 16, 128
    cache_o = torch.zeros(1, hq, t, dd, dtype=torch.float32, device="cuda")
    cache_lse = torch.zeros(1, hq, t, dtype=torch.float32, device="cuda")
    s = pl.LosaStep(dev(y["q_cur"]), dev(y["q_prev"]), dev(y["k_prefix"]), dev(y["v_prefix"]),
                    dev(y["k_block"]), dev(y["v_block"]), cache_o, cache_lse, 5, 16, 128,
                    1.0 / math.sqrt(128))
    t_prep = _time(torch, s.prepare)
    t_step = _time(torch, s.step)
    out["losa64k_step"] = {"ms": t_step, "prefix_pool_ms": t_prep,
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

    stages = {
        "pool_q_k": {"ms": t_pool, "GB/s": pool_bytes / (t_pool * 1e-3) / 1e9,
                     "frac_hbm": pool_bytes / (t_pool * 1e-3) / 1e9 / PEAK_HBM_GBS},
        "select": {"ms": t_sel, "GB/s": sel_bytes / (t_sel * 1e-3) / 1e9,
                   "fp64_GFLOP/s": 2.0 * w.heads * nb * nb * w.head_dim / (t_sel * 1e-3) / 1e9},
        "pool+select": {"ms": t_ps,
                        "frac_hbm": (pool_bytes + w.heads * nb * w.topk * 4) / (t_ps * 1e-3)
                        / 1e9 / PEAK_HBM_GBS},
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
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (fp64 oracle, bounded sample)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(x, w)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
