"""Pins of the fp64 oracle to facts it does not compute itself.

Each test checks the oracle against a library routine (torch's CPU attention,
logsumexp, avg-pooling), a closed form, a brute-force count, or numbers the
pages print.  None of them calls the HIP library.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle as orc
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _sdpa(q, k, v, scale, mask=None):
    """torch's CPU attention in float64 (an independent implementation)."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
    z = scale * (tq @ tk.transpose(-1, -2))
    if mask is not None:
        z = z.masked_fill(~mask, float("-inf"))
    return o.numpy(), torch.logsumexp(z, dim=-1).numpy()


def _tiny():
    w = wl.WORKLOADS["tiny"]
    x = wl.make_tiny(w.seed)
    return w, {n: x[n].astype(np.float64) for n in ("q", "k", "v")}


def _tiny_select(w, x):
    qb = orc.pool_mean(x["q"], w.block)
    kb = orc.pool_mean(x["k"], w.block)
    return orc.topk_ascending(orc.block_logits(qb, kb, w.scale), w.topk)


# --- P1: every block kept -> dense attention -------------------------------

def test_dense_reduction_equals_library_sdpa():
    w, x = _tiny()
    nb = w.blocks
    idx = np.broadcast_to(np.arange(nb, dtype=np.int32), (1, w.heads, nb, nb)).copy()
    o, lse = orc.sparse_attention(x["q"], x["k"], x["v"], idx, w.block, w.block, w.scale)
    o_ref, lse_ref = _sdpa(x["q"], x["k"], x["v"], w.scale)
    assert np.abs(o - o_ref).max() < 1e-12
    assert np.abs(lse - lse_ref).max() < 1e-12
    od, lsed = orc.dense_attention(x["q"], x["k"], x["v"], w.scale)
    assert np.abs(od - o_ref).max() < 1e-12 and np.abs(lsed - lse_ref).max() < 1e-12


# --- P2: block mask == token-level additive mask ---------------------------

def test_block_sparse_equals_masked_sdpa():
    w, x = _tiny()
    idx = _tiny_select(w, x)
    o, lse = orc.sparse_attention(x["q"], x["k"], x["v"], idx, w.block, w.block, w.scale)
    nb = w.blocks
    blockmask = np.zeros((1, w.heads, nb, nb), dtype=bool)
    for h in range(w.heads):
        for g in range(nb):
            blockmask[0, h, g, idx[0, h, g]] = True
    tokmask = torch.from_numpy(np.repeat(np.repeat(blockmask, w.block, axis=2), w.block, axis=3))
    o_ref, lse_ref = _sdpa(x["q"], x["k"], x["v"], w.scale, tokmask)
    assert np.abs(o - o_ref).max() < 1e-12
    assert np.abs(lse - lse_ref).max() < 1e-12


def test_gqa_and_ragged_lists_match_masked_sdpa():
    g = np.random.Generator(np.random.PCG64(7))
    hq, hkv, lq, lk, d, bq, bk = 6, 2, 96, 160, 16, 32, 16
    q = g.standard_normal((1, hq, lq, d))
    k = g.standard_normal((1, hkv, lk, d))
    v = g.standard_normal((1, hkv, lk, d))
    kept = 4
    idx = np.full((1, hq, lq // bq, kept), -1, dtype=np.int32)
    for h in range(hq):
        for t in range(lq // bq):
            n_use = 1 + (h + t) % kept           # ragged: 1..4 valid entries
            idx[0, h, t, :n_use] = np.sort(g.choice(lk // bk, n_use, replace=False))
    o, lse = orc.sparse_attention(q, k, v, idx, bq, bk, 0.3)
    mask = np.zeros((1, hq, lq, lk), dtype=bool)
    for h in range(hq):
        for t in range(lq // bq):
            for e in idx[0, h, t]:
                if e >= 0:
                    mask[0, h, t * bq:(t + 1) * bq, e * bk:(e + 1) * bk] = True
    kk = np.repeat(k, hq // hkv, axis=1)
    vv = np.repeat(v, hq // hkv, axis=1)
    o_ref, lse_ref = _sdpa(q, kk, vv, 0.3, torch.from_numpy(mask))
    assert np.abs(o - o_ref).max() < 1e-12
    assert np.abs(lse - lse_ref).max() < 1e-12


# --- P3: constant V ---------------------------------------------------------

def test_constant_values_return_the_value():
    w, x = _tiny()
    c = np.random.Generator(np.random.PCG64(3)).standard_normal(w.head_dim)
    v = np.broadcast_to(c, x["v"].shape).copy()
    idx = _tiny_select(w, x)
    bias = np.random.Generator(np.random.PCG64(4)).standard_normal(idx.shape)
    o, _ = orc.sparse_attention(x["q"], x["k"], v, idx, w.block, w.block, w.scale, bias=bias)
    assert np.abs(o - c).max() < 1e-12


# --- P4: the planted distant block is selected and attended ---------------

def test_planted_block_selected_first_and_attended():
    w, x = _tiny()
    qb = orc.pool_mean(x["q"], w.block)
    kb = orc.pool_mean(x["k"], w.block)
    logits = orc.block_logits(qb, kb, w.scale)
    g_star, p = wl.TINY_PLANT_QUERY_BLOCK, wl.TINY_PLANT_KEY_BLOCK
    idx = orc.topk_ascending(logits, w.topk)
    for h in range(w.heads):
        assert int(np.argmax(logits[0, h, g_star])) == p
        assert p in idx[0, h, g_star]
    # attended: the planted block carries mass, and O is linear in its values
    h = 0
    rows = x["q"][0, h, g_star * w.block:(g_star + 1) * w.block]
    o, lse = orc.attend_rows(rows, x["k"][0, h], x["v"][0, h], idx[0, h, g_star], w.block, w.scale)
    _, lse_p = orc.attend_rows(rows, x["k"][0, h], x["v"][0, h], [p], w.block, w.scale)
    mass = np.exp(lse_p - lse)
    assert mass.min() > 0.05
    delta = np.random.Generator(np.random.PCG64(5)).standard_normal(w.head_dim)
    v2 = x["v"][0, h].copy()
    v2[p * w.block:(p + 1) * w.block] += delta
    o2, _ = orc.attend_rows(rows, x["k"][0, h], v2, idx[0, h, g_star], w.block, w.scale)
    assert np.abs((o2 - o) - mass[:, None] * delta[None, :]).max() < 1e-12
    # dropping the planted block from the list moves O far beyond the O tolerance
    others = [j for j in np.argsort(-logits[0, h, g_star], kind="stable") if j != p][:w.topk]
    o3, _ = orc.attend_rows(rows, x["k"][0, h], x["v"][0, h], sorted(others), w.block, w.scale)
    assert np.abs(o3 - o).max() > 2e-2


# --- P5: two-part merge == one-shot attention; merge algebra --------------

def test_two_part_merge_equals_one_shot():
    w, x = _tiny()
    idx = _tiny_select(w, x)
    o, lse = orc.sparse_attention(x["q"], x["k"], x["v"], idx, w.block, w.block, w.scale)
    half = w.topk // 2
    a = orc.sparse_attention(x["q"], x["k"], x["v"], idx[..., :half], w.block, w.block, w.scale)
    b = orc.sparse_attention(x["q"], x["k"], x["v"], idx[..., half:], w.block, w.block, w.scale)
    om, lsem = orc.merge(a[0], a[1], b[0], b[1])
    assert np.abs(om - o).max() < 1e-12 and np.abs(lsem - lse).max() < 1e-12
    om2, lsem2 = orc.merge(b[0], b[1], a[0], a[1])
    assert np.abs(om2 - om).max() < 1e-14 and np.abs(lsem2 - lsem).max() < 1e-14


def test_merge_associative_and_identity():
    g = np.random.Generator(np.random.PCG64(11))
    parts = [(g.standard_normal((5, 8)), 3.0 * g.standard_normal(5)) for _ in range(3)]
    (oa, la), (ob, lb), (oc, lc) = parts
    left = orc.merge(*orc.merge(oa, la, ob, lb), oc, lc)
    right = orc.merge(oa, la, *orc.merge(ob, lb, oc, lc))
    assert np.abs(left[0] - right[0]).max() < 1e-13 and np.abs(left[1] - right[1]).max() < 1e-13
    zero, ninf = np.zeros((5, 8)), np.full(5, -np.inf)
    o, lse = orc.merge(oa, la, zero, ninf)
    assert np.abs(o - oa).max() == 0 and np.abs(lse - la).max() == 0
    o, lse = orc.merge(zero, ninf, zero, ninf)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    # merge weights against the library logsumexp of the two normalisers
    ref = torch.logsumexp(torch.stack([torch.from_numpy(la), torch.from_numpy(lb)]), dim=0).numpy()
    o, lse = orc.merge(oa, la, ob, lb)
    assert np.abs(lse - ref).max() < 1e-14
    assert np.abs(o - (np.exp(la - ref)[:, None] * oa + np.exp(lb - ref)[:, None] * ob)).max() < 1e-14


# --- P6: BA-Att Eq. 8 bound on the logit deviation --------------------------

@pytest.mark.parametrize("which", ["tiny", "dlm-slice"])
def test_eq8_deviation_bound_holds(which):
    if which == "tiny":
        w, x = _tiny()
        q, k, block, scale = x["q"][0], x["k"][0], w.block, w.scale
    else:
        xs = wl.make_dlm(5, heads=2, tokens=1024, head_dim=128)
        q, k = orc.as_f64(xs["q"])[0], orc.as_f64(xs["k"])[0]
        block, scale = 128, 1.0 / math.sqrt(128)
    qb, kb = orc.pool_mean(q, block), orc.pool_mean(k, block)
    ell = orc.block_logits(qb[None], kb[None], scale)[0]
    for h in range(q.shape[0]):
        nb = qb.shape[1]
        qr = q[h].reshape(nb, block, -1)
        kr = k[h].reshape(nb, block, -1)
        rq = np.linalg.norm(qr - qb[h][:, None], axis=-1).max(axis=1)
        mq = np.linalg.norm(qr, axis=-1).max(axis=1)
        rk = np.linalg.norm(kr - kb[h][:, None], axis=-1).max(axis=1)
        mk = np.linalg.norm(kr, axis=-1).max(axis=1)
        u = scale * (rq[:, None] * mk[None] + mq[:, None] * rk[None] + rq[:, None] * rk[None])
        tok = scale * (q[h] @ k[h].T)
        dev = np.abs(tok.reshape(nb, block, nb, block) - ell[h][:, None, :, None]).max(axis=(1, 3))
        assert np.all(dev <= u * (1 + 1e-12))
        assert dev.max() > 0.1 * u.max()        # the bound is not vacuous


# --- P7: top-k against a brute-force rank count ---------------------------

def test_topk_matches_brute_force_with_ties():
    g = np.random.Generator(np.random.PCG64(13))
    s = np.round(g.standard_normal((40, 37)) * 2) / 2     # many exact ties
    s[3, :] = 0.0
    s[4, ::2] = -0.0                                        # signed zeros tie
    for k in (1, 5, 17, 37):
        got = orc.topk_ascending(s, k)
        for r in range(s.shape[0]):
            better = (s[r][None, :] > s[r][:, None]) | (
                (s[r][None, :] == s[r][:, None]) & (np.arange(37)[None, :] < np.arange(37)[:, None]))
            want = np.nonzero(better.sum(axis=1) < k)[0]
            assert np.array_equal(got[r], want)
    with pytest.raises(ValueError):
        orc.topk_ascending(s, 38)


# --- P8: LLSA keys per query (printed in the README) -----------------------

def _golden_keys():
    rows = []
    with open(os.path.join(GOLDEN, "llsa_keys_per_query.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                n, kq = line.split()
                rows.append((int(n), int(kq)))
    return rows


@pytest.mark.parametrize("n,keys", _golden_keys())
def test_llsa_keys_per_query_match_readme(n, keys):
    assert orc.llsa_keys_per_query(n, 16, 8) == keys


def test_llsa_keys_grow_slowly_and_workload_count():
    assert orc.llsa_keys_per_query(65536, 16, 8) == 400
    assert orc.llsa_num_levels(1 << 20, 16) == 4
    # 1M tokens: 16 top-level tokens + 4 levels x top-k 8 x 16 children
    k_1m = 16 + 4 * 8 * 16
    assert k_1m / orc.llsa_keys_per_query(4096, 16, 8) < 2.0
    with pytest.raises(ValueError):
        orc.llsa_num_levels(1000, 16)


# --- P9: LLSA degenerate cases ----------------------------------------------

def test_llsa_single_level_is_full_attention():
    g = np.random.Generator(np.random.PCG64(17))
    q, k, v = (g.standard_normal((2, 48, 8)) for _ in range(3))    # 48 = 16*3: no coarse level
    res = orc.llsa_forward(q, k, v, 16, 8, 0.35)
    assert res["levels"] == 0
    o_ref, lse_ref = _sdpa(q[None], k[None], v[None], 0.35)
    assert np.abs(res["o"] - o_ref[0]).max() < 1e-12
    assert np.abs(res["lse"] - lse_ref[0]).max() < 1e-12


def test_llsa_constant_values_and_selection_structure():
    g = np.random.Generator(np.random.PCG64(19))
    q, k = (g.standard_normal((1, 4096, 8)) for _ in range(2))
    c = g.standard_normal(8)
    v = np.broadcast_to(c, q.shape).copy()
    res = orc.llsa_forward(q, k, v, 16, 8, 0.35)
    assert res["levels"] == 2
    assert np.abs(res["o"] - c).max() < 1e-12
    # each level-l selection lies inside its group's candidates and is ascending
    for lvl, s in res["sel"].items():
        assert np.all(np.diff(s, axis=-1) > 0)
        cand = res["cand"][lvl]
        grp = res["sizes"][lvl] // cand.shape[1]
        for a in range(s.shape[1]):
            assert np.all(np.isin(s[0, a], cand[0, a // grp]))


# --- P10: the level bias counts a coarse token as block^l fine tokens -------

@pytest.mark.parametrize("level", [1, 2])
def test_level_bias_equals_repeated_tokens(level):
    g = np.random.Generator(np.random.PCG64(23))
    d, blk = 8, 16
    q = g.standard_normal((3, d))
    kc, vc = g.standard_normal((1, d)), g.standard_normal((1, d))
    kf, vf = g.standard_normal((16, d)), g.standard_normal((16, d))
    # coarse entry: a block of 16 identical rows would over-count, so use block_k=1 lists
    k_tab = np.concatenate([kf, kc])
    v_tab = np.concatenate([vf, vc])
    o1, l1 = orc.attend_rows(q, k_tab, v_tab, list(range(17)), 1, 0.4,
                             bias=[0.0] * 16 + [level * math.log(blk)])
    rep = blk ** level
    k_rep = np.concatenate([kf, np.repeat(kc, rep, axis=0)])
    v_rep = np.concatenate([vf, np.repeat(vc, rep, axis=0)])
    o2, l2 = orc.attend_rows(q, k_rep, v_rep, list(range(16 + rep)), 1, 0.4)
    assert np.abs(o1 - o2).max() < 1e-12 and np.abs(l1 - l2).max() < 1e-12


# --- P11: LoSA step identities ------------------------------------------------

def _small_losa(seed=29, prefix=1024, hq=8, hkv=2, d=32, same=False):
    x = wl.make_losa(seed, heads_q=hq, heads_kv=hkv, prefix=prefix, head_dim=d)
    if same:
        x["q_prev"] = x["q_cur"].copy()
    scale = 1.0 / math.sqrt(d)
    cache_o, cache_lse = orc.dense_attention(x["q_prev"], x["k_prefix"], x["v_prefix"], scale)
    return x, scale, cache_o, cache_lse


def _dense_full(x, scale):
    k = np.concatenate([orc.as_f64(x["k_prefix"]), orc.as_f64(x["k_block"])], axis=2)
    v = np.concatenate([orc.as_f64(x["v_prefix"]), orc.as_f64(x["v_block"])], axis=2)
    return orc.dense_attention(x["q_cur"], k, v, scale)


def test_losa_active_set_is_the_planted_tokens():
    x, scale, co, cl = _small_losa()
    act = orc.active_tokens(x["q_cur"], x["q_prev"], wl.LOSA_ACTIVE)
    assert act.tolist() == [list(wl.LOSA_PLANTED)]


def test_losa_unchanged_queries_give_dense_attention():
    x, scale, co, cl = _small_losa(same=True)
    res = orc.losa_step(x["q_cur"], x["q_prev"], x["k_prefix"], x["v_prefix"], x["k_block"],
                        x["v_block"], co, cl, wl.LOSA_ACTIVE, 16, 8, scale)
    o_ref, lse_ref = _dense_full(x, scale)
    stable = [t for t in range(16) if t not in res["active"][0]]
    assert res["active"][0].tolist() == [0, 1, 2, 3, 4]      # all changes tie at 0
    assert np.abs(res["o"][:, :, stable] - o_ref[:, :, stable]).max() < 1e-12
    assert np.abs(res["lse"][:, :, stable] - lse_ref[:, :, stable]).max() < 1e-12


def test_losa_all_blocks_kept_gives_dense_attention():
    x, scale, co, cl = _small_losa()
    res = orc.losa_step(x["q_cur"], x["q_prev"], x["k_prefix"], x["v_prefix"], x["k_block"],
                        x["v_block"], co, cl, wl.LOSA_ACTIVE, 16, 1024 // 16, scale)
    o_ref, lse_ref = _dense_full(x, scale)
    act = res["active"][0]
    assert np.abs(res["o"][:, :, act] - o_ref[:, :, act]).max() < 1e-12
    assert np.abs(res["lse"][:, :, act] - lse_ref[:, :, act]).max() < 1e-12
    # stable rows: merge of the cached prefix with the in-block part
    stable = [t for t in range(16) if t not in act]
    o_s, lse_s = orc.merge(co, cl, res["o_in"], res["lse_in"])
    assert np.abs(res["o"][:, :, stable] - o_s[:, :, stable]).max() < 1e-14


# --- P12: ranking does not depend on the positive scale --------------------

def test_selection_scale_invariant():
    xs = wl.make_dlm(9, heads=4, tokens=2048, head_dim=128)
    qb, kb = orc.pool_mean(xs["q"], 128), orc.pool_mean(xs["k"], 128)
    a = orc.topk_ascending(orc.block_logits(qb, kb, 1.0), 5)
    b = orc.topk_ascending(orc.block_logits(qb, kb, 1.0 / math.sqrt(128)), 5)
    assert np.array_equal(a, b)


# --- P13: pooling ---------------------------------------------------------------

def test_pooling_against_library_and_mean_of_means():
    g = np.random.Generator(np.random.PCG64(31))
    x = g.standard_normal((2, 3, 4096, 8))
    p = orc.pool_mean(x, 16)
    t = torch.from_numpy(x).reshape(6, 4096, 8).transpose(1, 2)
    ref = torch.nn.functional.avg_pool1d(t, 16).transpose(1, 2).reshape(2, 3, 256, 8).numpy()
    assert np.abs(p - ref).max() < 1e-14
    assert np.abs(orc.pool_mean(p, 16) - orc.pool_mean(x, 256)).max() < 1e-14
    with pytest.raises(ValueError):
        orc.pool_mean(x[:, :, :100], 16)


# --- inputs ---------------------------------------------------------------------

def test_bf16_rounding_matches_torch():
    g = np.random.Generator(np.random.PCG64(37))
    x = (g.standard_normal(100000) * np.exp(g.uniform(-20, 20, 100000))).astype(np.float32)
    ours = wl.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(wl.bf16_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generators_are_deterministic():
    a = wl.make_dlm(3, heads=2, tokens=1024, head_dim=64)
    b = wl.make_dlm(3, heads=2, tokens=1024, head_dim=64)
    assert all(np.array_equal(a[n], b[n]) for n in a)
    t = wl.zorder_index(4)
    assert sorted(t.reshape(-1).tolist()) == list(range(16))
    assert set(t[:2, :2].reshape(-1).tolist()) == {0, 1, 2, 3}      # aligned 4 = 2x2 patch


# --- planted targets for the hierarchical descent and the LoSA selector ------

def test_llsa_descent_finds_planted_distant_block():
    """README test: a planted distant matching block is found and attended to."""
    g = np.random.Generator(np.random.PCG64(41))
    n, d = 4096, 16
    q, k, v = (g.standard_normal((1, n, d)) for _ in range(3))
    u = g.standard_normal(d)
    q[0, 256:512] += 2.0 * u            # one level-2 query group shares a direction
    p = 200                              # distant fine block of 16 keys
    k[0, p * 16:(p + 1) * 16] = 3.0 * u
    res = orc.llsa_forward(q, k, v, 16, 8, 0.25)
    for tile in range(16, 32):           # fine tiles inside the planted query group
        assert np.any(res["cand"][0][0, tile] // 16 == p)
    # attended: dropping the planted values changes those rows by a visible amount
    v2 = v.copy()
    v2[0, p * 16:(p + 1) * 16] += 1.0
    res2 = orc.llsa_forward(q, k, v2, 16, 8, 0.25)
    assert np.abs(res2["o"][0, 256:512] - res["o"][0, 256:512]).min() > 1e-3


def test_losa_selection_uses_the_query_heads_kv_group():
    x, scale, co, cl = _small_losa()
    t, h, p = wl.LOSA_PLANTED[0], 4, 7          # head 4 reads kv head 1 (group of 4)
    kp = orc.as_f64(x["k_prefix"])
    kp[0, 1, p * 16:(p + 1) * 16] = 3.0 * orc.as_f64(x["q_cur"])[0, h, t]
    x["k_prefix"] = wl.f32_to_bf16(kp.astype(np.float32))
    res = orc.losa_step(x["q_cur"], x["q_prev"], x["k_prefix"], x["v_prefix"], x["k_block"],
                        x["v_block"], co, cl, wl.LOSA_ACTIVE, 16, 8, scale)
    j = list(res["active"][0]).index(t)
    assert p in res["sel"][0, h, j]
    kbar = orc.pool_mean(x["k_prefix"], 16)
    assert int(np.argmax(kbar[0, 1] @ orc.as_f64(x["q_cur"])[0, h, t])) == p
