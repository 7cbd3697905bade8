// fp64 C++ reference of the block-sparse attention path (BA-Att).
//
// TEST INFRASTRUCTURE ONLY, like the rest of this directory: only the tests,
// the smoke check and the benchmark's CPU baseline may load it.  It shares no
// code, header or helper with the HIP library and never calls it.
//
// Plain loops in double precision, one definition per step, in the order the
// pages give them.  Inputs are float64 arrays (the caller widens bf16 or
// float32 exactly); outputs are float64 (indices int32).  Layouts: tensors
// [B][H][L][d] row-major; block index lists [B][Hq][rows][kept].
//
// Pages (cited by title and section):
//   "Efficient Long-Context Modeling in Diffusion Language Models via Block
//   Approximate Sparse Attention" (BA-Att): section 2 (Eq. 1, block-sparse
//   attention), section 3.1 (mean pooling, Eq. 2, top-kappa selection),
//   Algorithm 1.
//   LoSA blog post, "LoSA method" section: locality pruning by query change,
//   per-token prefix block selection, cached (O, LSE) of stable tokens,
//   in-block attention and the merge of two partial (O, LSE).
//   "Log-linear sparse attention in plain MLX" (README of loglinear-sparse-dit):
//   repeated mean pooling, coarse-to-fine per-token top-k, KV enrichment with
//   a level logit bias.
//
// Independent outputs (rows, heads, tiles) are spread over threads with
// OpenMP; every value is computed by one thread in the order written here,
// so the result does not depend on the thread count.
#include <omp.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <limits>
#include <numeric>
#include <vector>

extern "C" {

// BA-Att section 3.1: block representatives are the means of the rows of each
// block of `block` consecutive tokens.  x [outer][len][d] -> out [outer][len/block][d].
int oracle_pool_mean(const double* x, int64_t outer, int64_t len, int64_t d, int64_t block,
                     double* out) {
  if (block <= 0 || len % block != 0) return 1;
  const int64_t nb = len / block;
  for (int64_t o = 0; o < outer; ++o)
    for (int64_t g = 0; g < nb; ++g)
      for (int64_t c = 0; c < d; ++c) {
        double s = 0.0;
        for (int64_t i = 0; i < block; ++i) s += x[(o * len + g * block + i) * d + c];
        out[(o * nb + g) * d + c] = s / (double)block;
      }
  return 0;
}

// BA-Att section 3.1, Eq. 2: l[gq][gk] = scale * (Qbar_gq . Kbar_gk); query
// head h reads key head h / (hq / hkv).  qbar [b][hq][nq][d], kbar [b][hkv][nk][d]
// -> out [b][hq][nq][nk].
int oracle_block_logits(const double* qbar, const double* kbar, int64_t b, int64_t hq, int64_t hkv,
                        int64_t nq, int64_t nk, int64_t d, double scale, double* out) {
  if (hkv <= 0 || hq % hkv != 0) return 1;
  const int64_t group = hq / hkv;
  for (int64_t bi = 0; bi < b; ++bi)
    for (int64_t h = 0; h < hq; ++h) {
      const double* q = qbar + (bi * hq + h) * nq * d;
      const double* k = kbar + (bi * hkv + h / group) * nk * d;
      for (int64_t i = 0; i < nq; ++i)
        for (int64_t j = 0; j < nk; ++j) {
          double s = 0.0;
          for (int64_t c = 0; c < d; ++c) s += q[i * d + c] * k[j * d + c];
          out[((bi * hq + h) * nq + i) * nk + j] = scale * s;
        }
    }
  return 0;
}

// BA-Att section 3.1 / Algorithm 1: each query-block row keeps its top-kappa
// key blocks.  The softmax Algorithm 1 applies first is strictly increasing,
// so the kept set is the top-kappa by logit.  Order: score descending, equal
// scores to the lower column; the kept columns are written in ascending order.
// scores [rows][n] -> idx [rows][k].
int oracle_topk(const double* scores, int64_t rows, int64_t n, int64_t k, int32_t* idx) {
  if (k <= 0 || k > n) return 1;
  std::vector<int64_t> order(n);
  for (int64_t r = 0; r < rows; ++r) {
    const double* s = scores + r * n;
    std::iota(order.begin(), order.end(), 0);
    std::sort(order.begin(), order.end(), [s](int64_t a, int64_t b) {
      if (s[a] != s[b]) return s[a] > s[b];
      return a < b;
    });
    std::vector<int64_t> kept(order.begin(), order.begin() + k);
    std::sort(kept.begin(), kept.end());
    for (int64_t j = 0; j < k; ++j) idx[r * k + j] = (int32_t)kept[j];
  }
  return 0;
}

// BA-Att section 2, Eq. 1, evaluated only on the key blocks the block mask
// keeps: for query row i of list t, z_ij = scale * q_i . k_j over the keys of
// the listed blocks (entries outside [0, Lk/block_k) are unused slots),
// LSE_i = max_j z_ij + ln sum_j exp(z_ij - max), O_i = sum_j exp(z_ij - LSE_i) v_j.
// A row without keys gets O = 0, LSE = -inf.
// q [b][hq][lq][d], k/v [b][hkv][lk][d], idx [b][hq][lq/tile_q][kept].
int oracle_sparse_attention(const double* q, const double* k, const double* v, int64_t b, int64_t hq,
                            int64_t hkv, int64_t lq, int64_t lk, int64_t d, const int32_t* idx,
                            int64_t kept, int64_t tile_q, int64_t block_k, double scale, double* o,
                            double* lse) {
  if (hkv <= 0 || hq % hkv != 0 || tile_q <= 0 || lq % tile_q != 0 || block_k <= 0) return 1;
  const int64_t group = hq / hkv, lists = lq / tile_q, nblk = lk / block_k;
#pragma omp parallel for schedule(dynamic)
  for (int64_t unit = 0; unit < b * hq * lists; ++unit) {
    const int64_t bi = unit / (hq * lists), h = (unit / lists) % hq, t = unit % lists;
    std::vector<int64_t> keys;
    std::vector<double> z;
    {
      const double* kh = k + (bi * hkv + h / group) * lk * d;
      const double* vh = v + (bi * hkv + h / group) * lk * d;
      {
        const int32_t* lst = idx + ((bi * hq + h) * lists + t) * kept;
        keys.clear();
        for (int64_t e = 0; e < kept; ++e)
          if (lst[e] >= 0 && lst[e] < nblk)
            for (int64_t j = 0; j < block_k; ++j) keys.push_back((int64_t)lst[e] * block_k + j);
        for (int64_t r = 0; r < tile_q; ++r) {
          const int64_t row = (bi * hq + h) * lq + t * tile_q + r;
          const double* qi = q + row * d;
          double* oi = o + row * d;
          for (int64_t c = 0; c < d; ++c) oi[c] = 0.0;
          if (keys.empty()) {
            lse[row] = -std::numeric_limits<double>::infinity();
            continue;
          }
          z.assign(keys.size(), 0.0);
          double mx = -std::numeric_limits<double>::infinity();
          for (size_t j = 0; j < keys.size(); ++j) {
            double s = 0.0;
            for (int64_t c = 0; c < d; ++c) s += qi[c] * kh[keys[j] * d + c];
            z[j] = scale * s;
            mx = std::max(mx, z[j]);
          }
          double sum = 0.0;
          for (size_t j = 0; j < keys.size(); ++j) sum += std::exp(z[j] - mx);
          const double l = mx + std::log(sum);
          lse[row] = l;
          for (size_t j = 0; j < keys.size(); ++j) {
            const double p = std::exp(z[j] - l);
            for (int64_t c = 0; c < d; ++c) oi[c] += p * vh[keys[j] * d + c];
          }
        }
      }
    }
  }
  return 0;
}

// LoSA post, "LoSA method": two partial results over disjoint key sets merge
// by online softmax: m = max(LSE_a, LSE_b), LSE = m + ln(e^(LSE_a - m) +
// e^(LSE_b - m)), O = e^(LSE_a - LSE) O_a + e^(LSE_b - LSE) O_b; (0, -inf) is
// the empty partial.  o_a/o_b/o [rows][d], lse_* [rows].
int oracle_merge(const double* o_a, const double* lse_a, const double* o_b, const double* lse_b,
                 int64_t rows, int64_t d, double* o, double* lse) {
  for (int64_t r = 0; r < rows; ++r) {
    const double m = std::max(lse_a[r], lse_b[r]);
    if (std::isinf(m) && m < 0) {
      lse[r] = m;
      for (int64_t c = 0; c < d; ++c) o[r * d + c] = 0.0;
      continue;
    }
    const double l = m + std::log(std::exp(lse_a[r] - m) + std::exp(lse_b[r] - m));
    const double wa = std::exp(lse_a[r] - l), wb = std::exp(lse_b[r] - l);
    lse[r] = l;
    for (int64_t c = 0; c < d; ++c) o[r * d + c] = wa * o_a[r * d + c] + wb * o_b[r * d + c];
  }
  return 0;
}

// Number of threads OpenMP uses for the parallel loops above and below.
int oracle_threads(void) { return omp_get_max_threads(); }

// ---------------------------------------------------------------------------
// Log-linear sparse attention (README of loglinear-sparse-dit)
// ---------------------------------------------------------------------------

namespace {

// Top-k of a candidate list under (score descending, candidate ascending),
// written in ascending candidate order.  Scores belong to the candidates in
// the order given.
void topk_of(const std::vector<int32_t>& cand, const std::vector<double>& score, int64_t k,
             int32_t* out) {
  std::vector<size_t> order(cand.size());
  std::iota(order.begin(), order.end(), (size_t)0);
  std::sort(order.begin(), order.end(), [&](size_t a, size_t b) {
    if (score[a] != score[b]) return score[a] > score[b];
    return cand[a] < cand[b];
  });
  std::vector<int32_t> kept;
  for (int64_t j = 0; j < k; ++j) kept.push_back(cand[order[j]]);
  std::sort(kept.begin(), kept.end());
  for (int64_t j = 0; j < k; ++j) out[j] = kept[j];
}

// Two-pass softmax of one query row over explicit keys: z_j = scale * q . k_j
// + bias_j, LSE = max + ln sum exp(z - max), O = sum exp(z - LSE) v_j.
void attend_keys(const double* qi, const std::vector<const double*>& kr,
                 const std::vector<const double*>& vr, const std::vector<double>& bias, int64_t d,
                 double scale, double* oi, double* lse) {
  for (int64_t c = 0; c < d; ++c) oi[c] = 0.0;
  if (kr.empty()) {
    *lse = -std::numeric_limits<double>::infinity();
    return;
  }
  std::vector<double> z(kr.size());
  double mx = -std::numeric_limits<double>::infinity();
  for (size_t j = 0; j < kr.size(); ++j) {
    double s = 0.0;
    for (int64_t c = 0; c < d; ++c) s += qi[c] * kr[j][c];
    z[j] = scale * s + bias[j];
    mx = std::max(mx, z[j]);
  }
  double sum = 0.0;
  for (size_t j = 0; j < z.size(); ++j) sum += std::exp(z[j] - mx);
  const double l = mx + std::log(sum);
  *lse = l;
  for (size_t j = 0; j < z.size(); ++j) {
    const double p = std::exp(z[j] - l);
    for (int64_t c = 0; c < d; ++c) oi[c] += p * vr[j][c];
  }
}

}  // namespace

// The README supports lengths that are a multiple of block^(L+1) for L coarse
// levels; the deepest L the length allows is taken.  -1 if n is not a
// multiple of block.
int64_t oracle_llsa_num_levels(int64_t n, int64_t block) {
  if (block < 2 || n % block != 0) return -1;
  int64_t levels = 0, p = block * block;
  while (n % p == 0) {
    ++levels;
    p *= block;
  }
  return levels;
}

// Coarse-to-fine selection and enriched attention of one batch, from the
// README's method paragraphs:
//  - level l holds n / block^l tokens, each the mean of `block` consecutive
//    level l-1 tokens (queries, keys and values alike);
//  - at the coarsest level every token is a candidate of every query; at each
//    level a query keeps its own top-k (score scale * q . k, ties to the lower
//    token) among the candidates its group shares, and the children of each
//    kept token are the candidates of its children one level down (the group
//    of a level-(l-1) query is its parent);
//  - level 0 does no selection: a fine query attends to the candidates its
//    group received (the fine keys) and to the candidates of its ancestor's
//    group at every coarser level l, whose logits get l * ln(block) added.
// q, k, v [H][n][d]; sel: for l = 1 .. levels, [H][n/block^l][topk] int32,
// level 1 first; o [H][n][d], lse [H][n].  Non-zero for unsupported sizes.
int oracle_llsa_forward(const double* q, const double* k, const double* v, int64_t H, int64_t n,
                        int64_t d, int64_t block, int64_t topk, double scale, int64_t levels,
                        int32_t* sel, double* o, double* lse) {
  if (H < 1 || d < 1 || levels < 0 || levels > oracle_llsa_num_levels(n, block) || topk < 1)
    return 1;
  // level tables
  std::vector<int64_t> size(levels + 1);
  std::vector<std::vector<double>> qs(levels + 1), ks(levels + 1), vs(levels + 1);
  size[0] = n;
  qs[0].assign(q, q + H * n * d);
  ks[0].assign(k, k + H * n * d);
  vs[0].assign(v, v + H * n * d);
  for (int64_t l = 1; l <= levels; ++l) {
    size[l] = size[l - 1] / block;
    for (auto* t : {&qs, &ks, &vs}) {
      (*t)[l].assign(H * size[l] * d, 0.0);
      oracle_pool_mean((*t)[l - 1].data(), H, size[l - 1], d, block, (*t)[l].data());
    }
  }
  const int64_t top_n = size[levels];
  if (levels > 0 && topk > top_n) return 1;
  // candidates: cand[l][h][g] for group g of level l (level `levels`: one group
  // of every token; below: one group per level-(l+1) token, its picks' children)
  std::vector<std::vector<std::vector<std::vector<int32_t>>>> cand(levels + 1);
  cand[levels].assign(H, std::vector<std::vector<int32_t>>(1));
  for (int64_t h = 0; h < H; ++h)
    for (int64_t t = 0; t < top_n; ++t) cand[levels][h][0].push_back((int32_t)t);
  int64_t sel_off = 0;
  std::vector<int64_t> sel_at(levels + 1, 0);
  for (int64_t l = 1; l <= levels; ++l) {
    sel_at[l] = sel_off;
    sel_off += H * size[l] * topk;
  }
  for (int64_t l = levels; l >= 1; --l) {
    cand[l - 1].assign(H, std::vector<std::vector<int32_t>>(size[l]));
    const int64_t groups = (int64_t)cand[l][0].size();
    const int64_t per_group = size[l] / groups;
#pragma omp parallel for schedule(dynamic)
    for (int64_t u = 0; u < H * size[l]; ++u) {
      const int64_t h = u / size[l], a = u % size[l];
      const std::vector<int32_t>& c = cand[l][h][a / per_group];
      if ((int64_t)c.size() < topk) continue;  // not reached for supported sizes
      std::vector<double> sc(c.size());
      const double* qa = &qs[l][(h * size[l] + a) * d];
      for (size_t j = 0; j < c.size(); ++j) {
        const double* kc = &ks[l][(h * size[l] + c[j]) * d];
        double s = 0.0;
        for (int64_t x = 0; x < d; ++x) s += kc[x] * qa[x];
        sc[j] = scale * s;
      }
      int32_t* out = sel + sel_at[l] + (h * size[l] + a) * topk;
      topk_of(c, sc, topk, out);
      std::vector<int32_t>& child = cand[l - 1][h][a];
      for (int64_t j = 0; j < topk; ++j)
        for (int64_t u2 = 0; u2 < block; ++u2) child.push_back((int32_t)(out[j] * block + u2));
    }
  }
  // enriched attention of every fine query
  const double ln_b = std::log((double)block);
#pragma omp parallel for schedule(dynamic)
  for (int64_t u = 0; u < H * n; ++u) {
    const int64_t h = u / n, i = u % n;
    std::vector<const double*> kr, vr;
    std::vector<double> bias;
    int64_t anc = i;  // ancestor of query i at level l
    for (int64_t l = 0; l <= levels; ++l) {
      const int64_t g = (l == levels) ? 0 : anc / block;  // its group at level l
      for (int32_t c : cand[l][h][g]) {
        kr.push_back(&ks[l][(h * size[l] + c) * d]);
        vr.push_back(&vs[l][(h * size[l] + c) * d]);
        bias.push_back((double)l * ln_b);
      }
      anc /= block;
    }
    attend_keys(&qs[0][(h * n + i) * d], kr, vr, bias, d, scale, o + (h * n + i) * d, lse + h * n + i);
  }
  return 0;
}

// ---------------------------------------------------------------------------
// LoSA denoising step (blog post, "LoSA method" section)
// ---------------------------------------------------------------------------

// One denoising step of a block of T tokens with a cached prefix, in the
// post's order:
//  1. locality pruning: per token the mean over heads and channels of the
//     squared query change; the n_active largest are active (ties to the
//     lower token), listed ascending in active[b][n_active];
//  2. every (active token, query head) scores the mean-pooled prefix key
//     blocks with its own query (scale * q . Kbar) and keeps its top-k blocks
//     (ascending, ties to the lower block) in sel[b][hq][n_active][topk];
//  3. active rows get sparse prefix attention over their kept blocks, written
//     over the cached rows (new_cache = cache with those rows replaced);
//     stable rows keep the cached (O, LSE);
//  4. every token attends densely to the block's own keys (o_in, lse_in);
//  5. prefix and in-block partials merge by online softmax into (o, lse).
// Query head h reads key head h / (hq / hkv).  Layouts: q_* [b][hq][T][d],
// k/v_prefix [b][hkv][P][d], k/v_block [b][hkv][T][d], cache and outputs
// [b][hq][T][d] and [b][hq][T].
int oracle_losa_step(const double* q_cur, const double* q_prev, const double* k_prefix,
                     const double* v_prefix, const double* k_block, const double* v_block,
                     const double* cache_o, const double* cache_lse, int64_t b, int64_t hq,
                     int64_t hkv, int64_t T, int64_t P, int64_t d, int64_t n_active, int64_t block,
                     int64_t topk, double scale, int32_t* active, int32_t* sel,
                     double* new_cache_o, double* new_cache_lse, double* o_in, double* lse_in,
                     double* o, double* lse) {
  if (hkv < 1 || hq % hkv != 0 || n_active < 1 || n_active > T || block < 1 || P % block != 0 ||
      topk < 1 || topk > P / block)
    return 1;
  const int64_t group = hq / hkv, nb = P / block;
  std::vector<double> kbar(b * hkv * nb * d);
  oracle_pool_mean(k_prefix, b * hkv, P, d, block, kbar.data());
  std::copy(cache_o, cache_o + b * hq * T * d, new_cache_o);
  std::copy(cache_lse, cache_lse + b * hq * T, new_cache_lse);
  for (int64_t bi = 0; bi < b; ++bi) {
    // 1. active tokens
    std::vector<double> mse(T, 0.0);
    for (int64_t t = 0; t < T; ++t) {
      double s = 0.0;
      for (int64_t h = 0; h < hq; ++h)
        for (int64_t c = 0; c < d; ++c) {
          const int64_t at = ((bi * hq + h) * T + t) * d + c;
          const double diff = q_cur[at] - q_prev[at];
          s += diff * diff;
        }
      mse[t] = s / (double)(hq * d);
    }
    std::vector<int32_t> tok(T);
    std::iota(tok.begin(), tok.end(), 0);
    topk_of(tok, mse, n_active, active + bi * n_active);
    // 2-3. per (query head, active token): prefix blocks and sparse attention
#pragma omp parallel for schedule(dynamic)
    for (int64_t u = 0; u < hq * n_active; ++u) {
      const int64_t h = u / n_active, j = u % n_active;
      const int64_t t = active[bi * n_active + j];
      const int64_t hk = h / group;
      const double* qi = q_cur + ((bi * hq + h) * T + t) * d;
      std::vector<int32_t> blocks(nb);
      std::iota(blocks.begin(), blocks.end(), 0);
      std::vector<double> sc(nb);
      for (int64_t g = 0; g < nb; ++g) {
        const double* kb = &kbar[((bi * hkv + hk) * nb + g) * d];
        double s = 0.0;
        for (int64_t c = 0; c < d; ++c) s += kb[c] * qi[c];
        sc[g] = scale * s;
      }
      int32_t* out = sel + ((bi * hq + h) * n_active + j) * topk;
      topk_of(blocks, sc, topk, out);
      std::vector<const double*> kr, vr;
      for (int64_t e = 0; e < topk; ++e)
        for (int64_t r = 0; r < block; ++r) {
          const int64_t key = (int64_t)out[e] * block + r;
          kr.push_back(k_prefix + ((bi * hkv + hk) * P + key) * d);
          vr.push_back(v_prefix + ((bi * hkv + hk) * P + key) * d);
        }
      std::vector<double> bias(kr.size(), 0.0);
      const int64_t row = (bi * hq + h) * T + t;
      attend_keys(qi, kr, vr, bias, d, scale, new_cache_o + row * d, new_cache_lse + row);
    }
    // 4. dense in-block attention of every token
    for (int64_t h = 0; h < hq; ++h)
      for (int64_t t = 0; t < T; ++t) {
        const int64_t hk = h / group;
        std::vector<const double*> kr, vr;
        for (int64_t r = 0; r < T; ++r) {
          kr.push_back(k_block + ((bi * hkv + hk) * T + r) * d);
          vr.push_back(v_block + ((bi * hkv + hk) * T + r) * d);
        }
        std::vector<double> bias(T, 0.0);
        const int64_t row = (bi * hq + h) * T + t;
        attend_keys(q_cur + row * d, kr, vr, bias, d, scale, o_in + row * d, lse_in + row);
      }
  }
  // 5. merge of the (updated) prefix cache with the in-block partials
  return oracle_merge(new_cache_o, new_cache_lse, o_in, lse_in, b * hq * T, d, o, lse);
}

}  // extern "C"
