"""The fp64 C++ reference's log-linear forward and LoSA step (CPU).

Both are checked against the numpy oracle on small cases (selections
identical, O and LSE to 1e-12) and against the facts that pin the numpy
oracle: the LLSA README's degenerate single-level case (full attention) and
constant values, and the LoSA identities (unchanged queries give dense
attention over prefix and block, keeping every block gives dense attention,
the active set is the planted tokens).  The closed-form enrichment pins run on
both references in test_oracle_llsa_enrichment.py."""
import math

import numpy as np
import torch

import oracle as orc
import oracle.cref as cref
import workloads as wl


def _sdpa(q, k, v, scale):
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a)) for a in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)
    return o.numpy(), torch.logsumexp(scale * (tq @ tk.transpose(-1, -2)), dim=-1).numpy()


def test_llsa_matches_numpy_oracle():
    g = np.random.Generator(np.random.PCG64(201))
    q, k, v = (g.standard_normal((2, 4096, 16)) for _ in range(3))
    a = orc.llsa_forward(q, k, v, 16, 8, 0.3)
    b = cref.llsa_forward(q, k, v, 16, 8, 0.3)
    assert a["levels"] == b["levels"] == 2
    for lv in (1, 2):
        assert np.array_equal(a["sel"][lv], b["sel"][lv])
    assert np.abs(a["o"] - b["o"]).max() < 1e-12
    assert np.abs(a["lse"] - b["lse"]).max() < 1e-12


def test_llsa_bf16_image_slice_matches_numpy_oracle():
    x = wl.make_llsa(1003, heads=1, side=64, head_dim=64)   # 4096 tokens in Z-order
    a = orc.llsa_forward(x["q"][0], x["k"][0], x["v"][0], 16, 8, 0.125)
    b = cref.llsa_forward(x["q"][0], x["k"][0], x["v"][0], 16, 8, 0.125)
    for lv in a["sel"]:
        assert np.array_equal(a["sel"][lv], b["sel"][lv])
    assert np.abs(a["o"] - b["o"]).max() < 1e-12 and np.abs(a["lse"] - b["lse"]).max() < 1e-12


def test_llsa_single_level_full_attention_and_constant_values():
    g = np.random.Generator(np.random.PCG64(203))
    q, k, v = (g.standard_normal((2, 48, 8)) for _ in range(3))
    res = cref.llsa_forward(q, k, v, 16, 8, 0.35)
    assert res["levels"] == 0
    o_ref, l_ref = _sdpa(q, k, v, 0.35)
    assert np.abs(res["o"] - o_ref).max() < 1e-12 and np.abs(res["lse"] - l_ref).max() < 1e-12
    q, k = (g.standard_normal((1, 4096, 8)) for _ in range(2))
    c = g.standard_normal(8)
    res = cref.llsa_forward(q, k, np.broadcast_to(c, q.shape).copy(), 16, 8, 0.35)
    assert np.abs(res["o"] - c).max() < 1e-12


def _small_losa(seed=29, same=False):
    x = wl.make_losa(seed, heads_q=8, heads_kv=2, prefix=1024, head_dim=32)
    if same:
        x["q_prev"] = x["q_cur"].copy()
    scale = 1.0 / math.sqrt(32)
    co, cl = orc.dense_attention(x["q_prev"], x["k_prefix"], x["v_prefix"], scale)
    return x, scale, co, cl


def _step(impl, x, scale, co, cl, topk):
    return impl.losa_step(x["q_cur"], x["q_prev"], x["k_prefix"], x["v_prefix"], x["k_block"],
                          x["v_block"], co, cl, wl.LOSA_ACTIVE, 16, topk, scale)


def test_losa_matches_numpy_oracle():
    x, scale, co, cl = _small_losa()
    a, b = _step(orc, x, scale, co, cl, 8), _step(cref, x, scale, co, cl, 8)
    assert np.array_equal(a["active"], b["active"]) and np.array_equal(a["sel"], b["sel"])
    for key in ("o", "lse", "cache_o", "cache_lse", "o_in", "lse_in"):
        assert np.abs(a[key] - b[key]).max() < 1e-12, key


def _dense_full(x, scale):
    k = np.concatenate([orc.as_f64(x["k_prefix"]), orc.as_f64(x["k_block"])], axis=2)
    v = np.concatenate([orc.as_f64(x["v_prefix"]), orc.as_f64(x["v_block"])], axis=2)
    q = orc.as_f64(x["q_cur"])
    hq, hkv = q.shape[1], k.shape[1]
    k, v = np.repeat(k, hq // hkv, axis=1), np.repeat(v, hq // hkv, axis=1)
    return _sdpa(q, k, v, scale)


def test_losa_identities():
    # unchanged queries: the stable rows keep the dense cache, so the step gives them
    # dense attention over prefix and block
    x, scale, co, cl = _small_losa(same=True)
    res = _step(cref, x, scale, co, cl, 8)
    stable = [t for t in range(16) if t not in res["active"][0].tolist()]
    assert len(stable) == 16 - wl.LOSA_ACTIVE
    o_ref, l_ref = _dense_full(x, scale)
    assert np.abs(res["o"][:, :, stable] - o_ref[:, :, stable]).max() < 1e-12
    assert np.abs(res["lse"][:, :, stable] - l_ref[:, :, stable]).max() < 1e-12
    # every prefix block kept: the active rows are dense attention of the current
    # queries (stable rows keep the previous step's cache), and the active set is the plant
    x, scale, co, cl = _small_losa()
    res = _step(cref, x, scale, co, cl, 1024 // 16)
    assert res["active"].tolist() == [list(wl.LOSA_PLANTED)]
    act = list(wl.LOSA_PLANTED)
    o_ref, l_ref = _dense_full(x, scale)
    assert np.abs(res["o"][:, :, act] - o_ref[:, :, act]).max() < 1e-12
    assert np.abs(res["lse"][:, :, act] - l_ref[:, :, act]).max() < 1e-12


def test_threads_reported():
    assert cref.threads() >= 1
