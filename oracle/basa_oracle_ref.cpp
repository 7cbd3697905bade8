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
//   LoSA blog post, "LoSA method" section: merge of two partial (O, LSE).
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
  std::vector<int64_t> keys;
  std::vector<double> z;
  for (int64_t bi = 0; bi < b; ++bi)
    for (int64_t h = 0; h < hq; ++h) {
      const double* kh = k + (bi * hkv + h / group) * lk * d;
      const double* vh = v + (bi * hkv + h / group) * lk * d;
      for (int64_t t = 0; t < lists; ++t) {
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

}  // extern "C"
