// Block selection: block scores and a per-row top-k (BA-Att section 3.1, Eq. 2
// and Algorithm 1), optionally restricted to the children of a parent's picks
// (log-linear README, coarse-to-fine descent); and the LoSA active-token pick
// by query change.
//
// BLOCKS mode.  One wavefront owns RW query rows of one head; lane l owns the
// candidates l, l+64, l+128, ... so a row's scores sit in registers, KPL per
// lane.  Scores are float64 dot products.  Keys are read from the transposed
// means [head_dim][keys], so at each channel the lanes read consecutive keys
// (one coalesced load per 64 candidates); the query values are wave-uniform
// and come through the scalar cache.  The four waves of a workgroup work on
// neighbouring rows of the same head and share the key loads in L1.
//
// Top-k per row, in registers: scores become order-preserving 64-bit keys; a
// bitwise search from the top bit finds the largest threshold T with at least
// k keys >= T (ballot + popcount per step), stopping as soon as exactly k keys
// clear it.  If it never does, T is the k-th largest key, and the keys equal to
// T are taken in candidate order until k are kept (ties to the lower index).
// The kept candidates are written in candidate order, which is ascending key
// order, with ballot prefix counts.
#include "common.h"

namespace basa {
namespace {

struct SelArgs {
  const double* q;      // [B][Hq][q_len][d]
  const double* kt;     // [B][Hkv][d][keys]
  int32_t* idx;         // [B][Hq][rows][topk]
  const int32_t* q_rows;
  const int32_t* parent;
  int64_t q_len, rows, keys;
  int d, topk, group, heads_q, heads_kv, parent_k, fanout, n_cand;
};

__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }

typedef uint32_t u32x4_sel __attribute__((ext_vector_type(4)));
typedef double f64x4_sel __attribute__((ext_vector_type(4)));

// A wave-uniform element of read-only input through the constant address space,
// so it is fetched with a scalar load.  (A vector load would share the in-order
// vector-memory counter with the key means streamed into LDS, and waiting for
// it would wait for them.)
typedef __attribute__((address_space(4))) const double const_f64;
__device__ __forceinline__ double uniform_ld(const double* p) {
  return *(const_f64*)p;
}

// Largest / smallest 32-bit value over the wave (every lane active): DPP
// exchanges inside each row of 16 lanes (pairs, quad halves, half-row mirror,
// row mirror), then the four rows' results read into scalars.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_ext_u32(uint32_t v) {
  auto pick = [](uint32_t a, uint32_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
  v = pick(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false));
  v = pick(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false));
  v = pick(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xF, 0xF, false));
  v = pick(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xF, 0xF, false));
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return pick(pick(r0, r1), pick(r2, r3));
}

// Largest and smallest valid key of the wave (at least one valid key), as
// wave-uniform values: the high halves first, then the low halves among the
// lanes whose high half is the extreme one.
template <int KPL>
__device__ __forceinline__ void wave_key_range(const uint64_t* key, const bool* valid,
                                               uint64_t& hi, uint64_t& lo) {
  uint64_t lmax = 0, lmin = ~0ull;
#pragma unroll
  for (int j = 0; j < KPL; ++j)
    if (valid[j]) {
      lmax = key[j] > lmax ? key[j] : lmax;
      lmin = key[j] < lmin ? key[j] : lmin;
    }
  const uint32_t hh = wave_ext_u32<true>((uint32_t)(lmax >> 32));
  const uint32_t hl = wave_ext_u32<true>((uint32_t)(lmax >> 32) == hh ? (uint32_t)lmax : 0u);
  const uint32_t lh = wave_ext_u32<false>((uint32_t)(lmin >> 32));
  const uint32_t ll = wave_ext_u32<false>((uint32_t)(lmin >> 32) == lh ? (uint32_t)lmin : ~0u);
  hi = ((uint64_t)hh << 32) | hl;
  lo = ((uint64_t)lh << 32) | ll;
}

// Marks the keys of a wave-level top-k once its threshold T (the k-th largest
// key) is known: every valid key above T, then the keys equal to T in candidate
// order until k are taken.  With exact set, exactly k keys are at or above T and
// those are taken.
template <int KPL>
__device__ __forceinline__ void select_at(const uint64_t* key, const bool* valid, int k,
                                          uint64_t below, uint64_t thr, bool exact, bool* sel) {
  if (exact) {
#pragma unroll
    for (int j = 0; j < KPL; ++j) sel[j] = valid[j] && key[j] >= thr;
    return;
  }
  int gt = 0;
#pragma unroll
  for (int j = 0; j < KPL; ++j) gt += popc64(__ballot(valid[j] && key[j] > thr));
  const int need_eq = k - gt;
  int eq_seen = 0;
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const bool eq = valid[j] && key[j] == thr;
    const uint64_t em = __ballot(eq);
    const int eq_rank = eq_seen + popc64(em & below);
    eq_seen += popc64(em);
    sel[j] = (valid[j] && key[j] > thr) || (eq && eq_rank < need_eq);
  }
}

// Wave-level top-k over KPL keys per lane in candidate order (lane + 64 j).
// Marks sel[j] for the min(k, #valid) best under (key desc, candidate asc):
// bitwise search from the top for the largest threshold T with at least k
// keys >= T, stopping early when exactly k clear it; otherwise T is the k-th
// largest key and keys equal to T are taken in candidate order.
template <int KPL>
__device__ __forceinline__ void wave_topk(const uint64_t* key, const bool* valid, int k,
                                          uint64_t below, bool* sel) {
  int n_valid = 0;
#pragma unroll
  for (int j = 0; j < KPL; ++j) n_valid += popc64(__ballot(valid[j]));
  if (n_valid <= k) {
#pragma unroll
    for (int j = 0; j < KPL; ++j) sel[j] = valid[j];
    return;
  }
  // Every valid key lies in [lo, hi], so all share the bits above the highest
  // bit where lo and hi differ: T has those bits, and the search starts below.
  uint64_t hi, lo;
  wave_key_range<KPL>(key, valid, hi, lo);
  // diff == 0: all valid keys are equal, T = hi and the tie rule below takes the first k
  const uint64_t diff = hi ^ lo;
  const int top = diff ? 63 - __clzll(diff) : -1;
  uint64_t thr = top >= 63 ? 0 : (hi >> (top + 1)) << (top + 1);
  // The loop leaves with bit >= 0 exactly when a count hit k, so no flag is
  // carried through it (a flag set before a break costs the loop a round trip
  // through the vector unit per bit).
  int bit = top;
  for (; bit >= 0; --bit) {
    const uint64_t t = thr | (1ull << bit);
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) cnt += popc64(__ballot(valid[j] && key[j] >= t));
    if (cnt >= k) thr = t;
    if (cnt == k) break;
  }
  select_at<KPL>(key, valid, k, below, thr, bit >= 0, sel);
}

template <int KPL, int RW>
__global__ __launch_bounds__(256) void select_blocks_kernel(SelArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + wave) * RW;
  if (row0 >= a.rows) return;
  const int hk = h / a.group;
  const double* kt = a.kt + ((int64_t)b * a.heads_kv + hk) * a.d * a.keys;

  // candidate key index per lane slot (-1 = no candidate)
  int cand[KPL];
  if (a.parent) {
    const int32_t* par = a.parent + (((int64_t)b * a.heads_q + h) * (a.rows / a.fanout) + row0 / a.fanout) * a.parent_k;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const int c = lane + 64 * j;
      cand[j] = -1;
      if (c < a.n_cand) {
        const int32_t pv = par[c / a.fanout];
        const int64_t key = (int64_t)pv * a.fanout + (c % a.fanout);
        if (pv >= 0 && key < a.keys) cand[j] = (int)key;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const int c = lane + 64 * j;
      cand[j] = c < a.n_cand ? c : -1;
    }
  }

  // query row pointers (wave-uniform)
  const double* qp[RW];
  bool rvalid[RW];
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    const int64_t r = row0 + i;
    rvalid[i] = r < a.rows;
    int64_t qr = rvalid[i] ? r : row0;
    if (a.q_rows) qr = a.q_rows[(int64_t)b * a.rows + qr];
    if (qr < 0 || qr >= a.q_len) qr = 0;  // a row map entry outside q reads row 0
    qr = __builtin_amdgcn_readfirstlane((int)qr);
    qp[i] = a.q + (((int64_t)b * a.heads_q + h) * a.q_len + qr) * a.d;
  }

  double acc[RW][KPL];
#pragma unroll
  for (int i = 0; i < RW; ++i)
#pragma unroll
    for (int j = 0; j < KPL; ++j) acc[i][j] = 0.0;

  // empty slots read key 0 (always present) and their scores are never used
  int safe[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) safe[j] = cand[j] >= 0 ? cand[j] : 0;
  // The key loads come from L2; unrolling 8 channels keeps 8 of them in flight
  // per slot (the rows of the 16K and log-linear selections wait on them, not
  // on the multiply-adds: 37 -> 22 us at 16K).  Wider rows keep 2, for registers.
  constexpr int UNR = KPL <= 8 ? 8 : 2;
#pragma unroll UNR
  for (int c = 0; c < a.d; ++c) {
    double kv[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) kv[j] = kt[(int64_t)c * a.keys + safe[j]];
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const double qv = qp[i][c];
#pragma unroll
      for (int j = 0; j < KPL; ++j) acc[i][j] = __builtin_fma(qv, kv[j], acc[i][j]);
    }
  }

  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    if (!rvalid[i]) continue;
    // order-preserving keys, kept in the score registers
    uint64_t* key = reinterpret_cast<uint64_t*>(acc[i]);
    bool valid[KPL], sel[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      valid[j] = cand[j] >= 0;
      key[j] = valid[j] ? ordered_key(acc[i][j]) : 0ull;
    }
    wave_topk<KPL>(key, valid, a.topk, below, sel);
    int32_t* out = a.idx + (((int64_t)b * a.heads_q + h) * a.rows + row0 + i) * a.topk;
    int base = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const uint64_t m = __ballot(sel[j]);
      if (sel[j]) out[base + popc64(m & below)] = cand[j];
      base += popc64(m);
    }
  }
}

// ---------------------------------------------------------------------------
// Wide rows (more than 1024 candidates, top-k <= 256): a workgroup per row.
// Wave w scores the contiguous quarter [w*Q, (w+1)*Q) of the candidates and
// keeps its own top-k; wave 0 then takes the top-k of the (at most 4k)
// survivors, which are in ascending candidate order.  Anything in the row's
// top-k is in its quarter's top-k under the same order, so the result is exact.
// ---------------------------------------------------------------------------
constexpr int WIDE_MAX_K = 256;

template <int KPL>
__global__ __launch_bounds__(256) void select_wide_kernel(SelArgs a) {
  __shared__ uint64_t s_key[4][WIDE_MAX_K];
  __shared__ int32_t s_cand[4][WIDE_MAX_K];
  __shared__ int s_n[4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int hk = h / a.group;
  const double* kt = a.kt + ((int64_t)b * a.heads_kv + hk) * a.d * a.keys;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int qtr = (a.n_cand + 3) / 4;
  const int c_lo = wave * qtr;
  const int c_hi = min(a.n_cand, c_lo + qtr);

  int cand[KPL];
  if (a.parent) {
    const int32_t* par = a.parent + (((int64_t)b * a.heads_q + h) * (a.rows / a.fanout) + row / a.fanout) * a.parent_k;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const int c = c_lo + lane + 64 * j;
      cand[j] = -1;
      if (c < c_hi) {
        const int32_t pv = par[c / a.fanout];
        const int64_t key = (int64_t)pv * a.fanout + (c % a.fanout);
        if (pv >= 0 && key < a.keys) cand[j] = (int)key;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const int c = c_lo + lane + 64 * j;
      cand[j] = c < c_hi ? c : -1;
    }
  }
  int64_t qr = row;
  if (a.q_rows) qr = a.q_rows[(int64_t)b * a.rows + row];
  if (qr < 0 || qr >= a.q_len) qr = 0;
  qr = __builtin_amdgcn_readfirstlane((int)qr);
  const double* qp = a.q + (((int64_t)b * a.heads_q + h) * a.q_len + qr) * a.d;

  double acc[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) acc[j] = 0.0;
  // empty slots read key 0 (always present) and their scores are never used
  int safe[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) safe[j] = cand[j] >= 0 ? cand[j] : 0;
#pragma unroll 2
  for (int c = 0; c < a.d; ++c) {
    const double qv = qp[c];
    double kv[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) kv[j] = kt[(int64_t)c * a.keys + safe[j]];
#pragma unroll
    for (int j = 0; j < KPL; ++j) acc[j] = __builtin_fma(qv, kv[j], acc[j]);
  }
  uint64_t* key = reinterpret_cast<uint64_t*>(acc);
  bool valid[KPL], sel[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    valid[j] = cand[j] >= 0;
    key[j] = valid[j] ? ordered_key(acc[j]) : 0ull;
  }
  wave_topk<KPL>(key, valid, a.topk, below, sel);
  int base = 0;
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const uint64_t m = __ballot(sel[j]);
    if (sel[j]) {
      const int pos = base + popc64(m & below);
      s_key[wave][pos] = key[j];
      s_cand[wave][pos] = cand[j];
    }
    base += popc64(m);
  }
  if (lane == 0) s_n[wave] = base;
  __syncthreads();
  if (wave != 0) return;

  // survivors of the four quarters, in ascending candidate order: at most 4 x 256
  constexpr int KPL2 = 4 * WIDE_MAX_K / 64;
  int off[5];
  off[0] = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) off[w + 1] = off[w] + s_n[w];
  uint64_t key2[KPL2];
  bool valid2[KPL2], sel2[KPL2];
  int cand2[KPL2];
#pragma unroll
  for (int j = 0; j < KPL2; ++j) {
    const int e = lane + 64 * j;
    valid2[j] = e < off[4];
    key2[j] = 0ull;
    cand2[j] = -1;
    if (valid2[j]) {
      int w = 0;
      while (e >= off[w + 1]) ++w;
      key2[j] = s_key[w][e - off[w]];
      cand2[j] = s_cand[w][e - off[w]];
    }
  }
  wave_topk<KPL2>(key2, valid2, a.topk, below, sel2);
  int32_t* out = a.idx + (((int64_t)b * a.heads_q + h) * a.rows + row) * a.topk;
  base = 0;
#pragma unroll
  for (int j = 0; j < KPL2; ++j) {
    const uint64_t m = __ballot(sel2[j]);
    if (sel2[j]) out[base + popc64(m & below)] = cand2[j];
    base += popc64(m);
  }
}

// ---------------------------------------------------------------------------
// Channel-split rows (257..512 candidates, no parent list): a workgroup per
// four rows of one head.  Wave w forms the partial scores of all four rows over
// its quarter of the channels (a short chain of dependent loads instead of a
// long one), the partials meet in LDS, and wave w completes row w - adding the
// four quarters in the fixed order 0, 1, 2, 3 - and takes its top-k.
// ---------------------------------------------------------------------------
// Workgroups go to the 8 XCDs round-robin; numbering them so that XCD x takes
// the x-th contiguous eighth of the (batch, head, row group) space keeps each
// head's key means in one XCD's L2.
__device__ __forceinline__ int64_t xcd_major(int64_t id, int64_t n) {
  const int64_t per = n / 8;
  if (id >= 8 * per) return id;  // the last n % 8 workgroups keep their number
  return (id % 8) * per + id / 8;
}

template <int KPL>
__global__ __launch_bounds__(256) void select_split_kernel(SelArgs a, int64_t groups) {
  __shared__ double part[4][3][KPL * 64];  // [writer wave][other row][slot]: 3 rows per writer
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // (b, h, row group) from the XCD-major workgroup number
  const int64_t unit = xcd_major(blockIdx.x, gridDim.x);
  const int64_t rg = unit % groups;
  const int h = (int)((unit / groups) % a.heads_q);
  const int b = (int)(unit / (groups * a.heads_q));
  const int64_t row0 = rg * 4;
  const int hk = h / a.group;
  const double* kt = a.kt + ((int64_t)b * a.heads_kv + hk) * a.d * a.keys;

  int cand[KPL], safe[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const int c = lane + 64 * j;
    cand[j] = c < a.n_cand ? c : -1;
    safe[j] = c < a.n_cand ? c : 0;  // empty slots read key 0; their scores are never used
  }
  const double* qp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int64_t qr = row0 + i < a.rows ? row0 + i : row0;
    if (a.q_rows) qr = a.q_rows[(int64_t)b * a.rows + qr];
    if (qr < 0 || qr >= a.q_len) qr = 0;  // a row map entry outside q reads row 0
    qr = __builtin_amdgcn_readfirstlane((int)qr);
    qp[i] = a.q + (((int64_t)b * a.heads_q + h) * a.q_len + qr) * a.d;
  }

  double acc[4][KPL];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < KPL; ++j) acc[i][j] = 0.0;
  const int cq = a.d / 4;
  const int c0 = wave * cq;
#pragma unroll 4
  for (int c = c0; c < c0 + cq; ++c) {
    double kv[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) kv[j] = kt[(int64_t)c * a.keys + safe[j]];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double qv = qp[i][c];
#pragma unroll
      for (int j = 0; j < KPL; ++j) acc[i][j] = __builtin_fma(qv, kv[j], acc[i][j]);
    }
  }
  // hand the other rows' partials over
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i == wave) continue;
    const int slot = i < wave ? i : i - 1;
#pragma unroll
    for (int j = 0; j < KPL; ++j) part[wave][slot][j * 64 + lane] = acc[i][j];
  }
  __syncthreads();
  const int64_t row = row0 + wave;
  if (row >= a.rows) return;
  double sc[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    double tot = 0.0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      double pv;
      if (v == wave) {
        // own partial: the registers of row `wave` (a wave-uniform choice among four)
        pv = wave == 0 ? acc[0][j] : wave == 1 ? acc[1][j] : wave == 2 ? acc[2][j] : acc[3][j];
      } else {
        pv = part[v][wave < v ? wave : wave - 1][j * 64 + lane];
      }
      tot = v == 0 ? pv : tot + pv;
    }
    sc[j] = tot;
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint64_t key[KPL];
  bool valid[KPL], sel[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    valid[j] = cand[j] >= 0;
    key[j] = valid[j] ? ordered_key(sc[j]) : 0ull;
  }
  wave_topk<KPL>(key, valid, a.topk, below, sel);
  int32_t* out = a.idx + (((int64_t)b * a.heads_q + h) * a.rows + row) * a.topk;
  int base = 0;
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const uint64_t m = __ballot(sel[j]);
    if (sel[j]) out[base + popc64(m & below)] = cand[j];
    base += popc64(m);
  }
}

// ---------------------------------------------------------------------------
// Top-k in two column ranges of given float64 scores (SparseD section 3.3,
// Eq. 5-6: the prefill keys [0, split) and the generation keys [split, n)
// are selected separately, k_lo and k_hi of them).  One wave per row, the
// same wave top-k as above, once per range; the kept columns of both ranges
// are written together in ascending order.
// ---------------------------------------------------------------------------
template <int KPL>
__global__ __launch_bounds__(256) void select_ranges_kernel(const double* scores, int64_t rows, int n,
                                                            int split, int k_lo, int k_hi,
                                                            int32_t* idx) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // wave-uniform
  const double* s = scores + row * n;
  uint64_t key[KPL];
  bool lo[KPL], hi[KPL], sel_lo[KPL], sel_hi[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const int c = lane + 64 * j;
    key[j] = c < n ? ordered_key(s[c]) : 0ull;
    lo[j] = c < split;
    hi[j] = c >= split && c < n;
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  if (k_lo > 0) {
    wave_topk<KPL>(key, lo, k_lo, below, sel_lo);
  } else {
#pragma unroll
    for (int j = 0; j < KPL; ++j) sel_lo[j] = false;
  }
  if (k_hi > 0) {
    wave_topk<KPL>(key, hi, k_hi, below, sel_hi);
  } else {
#pragma unroll
    for (int j = 0; j < KPL; ++j) sel_hi[j] = false;
  }
  int32_t* out = idx + row * (k_lo + k_hi);
  int base = 0;
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const bool keep = sel_lo[j] || sel_hi[j];
    const uint64_t m = __ballot(keep);
    if (keep) out[base + popc64(m & below)] = lane + 64 * j;
    base += popc64(m);
  }
}

// ---------------------------------------------------------------------------
// Key means staged in LDS.  The two-pass kernel below streams chunks of
// SEL_CH channels x PART keys.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;
constexpr int SEL_CH = 8;  // channels per staged chunk

constexpr int SEL_BYTES = SEL_CH * 8 * 64 * 8;  // 8 channels x 512 keys of float64
__shared__ __attribute__((aligned(16))) uint8_t s_sel0[SEL_BYTES];
__shared__ __attribute__((aligned(16))) uint8_t s_sel1[SEL_BYTES];

// ---------------------------------------------------------------------------
// 512 candidates (no parent list) on the float64 matrix core
// (v_mfma_f64_16x16x4f64: C[16x16] += A[16x4] B[4x16]).  A workgroup of 4 waves
// takes 16 rows of one (batch, query head); wave w owns the keys
// [128w, 128w + 128) as 8 tiles of 16 and copies exactly its own quarter of each
// chunk of 4 channels into LDS (16-byte copies straight to LDS, two buffers),
// so the walk over the channels needs no workgroup barrier: a wave waits only
// for its own copies.  Each 4 KB channel row of a chunk is followed by 128
// bytes of padding, which puts the two channel rows that a half-wave reads on
// different banks.  For matrix step s the A operand of lane l is
// q[row l%16][4s + l/16] (a vector load issued a chunk ahead), the B operand
// K^T[4s + l/16][key 16u + l%16], and lane l receives the scores of rows
// l/16 + 4r (r = 0..3) at key 16u + l%16.  After the walk the scores go through
// LDS, 8 rows at a time, and each wave takes the top-k of 2 of them, with the
// candidates in the order wave_topk expects (lane + 64j).  The float64 products
// are those of a plain dot product; only the order of the additions differs.
// Against scoring with vector FMAs (64 FMAs per 8 doubles read from LDS, four
// rows sharing each key value) the matrix core reads a quarter of the LDS bytes
// per product and leaves the vector and scalar units free.
// ---------------------------------------------------------------------------
constexpr int MS_CH = 4;                                  // channels per chunk (one step)
constexpr int MS_ROW = 4096 + 128;                        // bytes per padded channel row
constexpr int MS_BUF = MS_CH * MS_ROW;                    // one chunk
constexpr int MS_SC = 512 + 8;                            // doubles per score row in the exchange
constexpr int MS_LDS = 2 * MS_BUF > 8 * MS_SC * 8 ? 2 * MS_BUF : 8 * MS_SC * 8;
__shared__ __attribute__((aligned(16))) uint8_t s_ms[MS_LDS];

// this wave's quarter of chunk `src` (4 channel rows of 512 keys) into buffer P
template <int P>
__device__ __forceinline__ void ms_dma(const double* src, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < MS_CH; ++i)
    __builtin_amdgcn_global_load_lds(src + i * 512 + wave * 128 + lane * 2,
                                     (lds_void*)(s_ms + P * MS_BUF + i * MS_ROW + wave * 1024), 16, 0, 0);
}

// the 8 B operands of this wave for the chunk in buffer P
template <int P>
__device__ __forceinline__ void ms_read_b(double (&bv)[8], int wave, int lane) {
  const double* kc = reinterpret_cast<const double*>(s_ms + P * MS_BUF + (lane >> 4) * MS_ROW) +
                     wave * 128 + (lane & 15);
#pragma unroll
  for (int u = 0; u < 8; ++u) bv[u] = kc[16 * u];
}

__global__ __launch_bounds__(256, 4) void select_mfma_kernel(SelArgs a, int64_t groups) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t unit = xcd_major(blockIdx.x, gridDim.x);
  const int64_t rg = unit % groups;
  const int h = (int)((unit / groups) % a.heads_q);
  const int b = (int)(unit / (groups * a.heads_q));
  const int64_t row0 = rg * 16;
  const int hk = h / a.group;
  const double* kt = a.kt + ((int64_t)b * a.heads_kv + hk) * a.d * 512;

  // A operand row (a row past the end, or a row map entry outside q, reads row 0)
  int64_t qr = row0 + (lane & 15);
  qr = qr < a.rows ? qr : 0;
  if (a.q_rows) qr = a.q_rows[(int64_t)b * a.rows + qr];
  if (qr < 0 || qr >= a.q_len) qr = 0;
  const double* qa = a.q + (((int64_t)b * a.heads_q + h) * a.q_len + qr) * a.d + (lane >> 4);
  f64x4_sel acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = f64x4_sel{0.0, 0.0, 0.0, 0.0};

  // chunks of 4 channels, head_dim / 4 even (checked at launch); chunk c + 1 is
  // copied while chunk c is multiplied
  const int n_chunk = a.d / MS_CH;
  double bv[8];
  ms_dma<0>(kt, wave, lane);
  double av = qa[0];
  __builtin_amdgcn_s_waitcnt(0x0F70);
  for (int c = 0; c < n_chunk; c += 2) {
    ms_dma<1>(kt + (c + 1) * MS_CH * 512, wave, lane);
    const double an = qa[(c + 1) * MS_CH];
    ms_read_b<0>(bv, wave, lane);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv[u], acc[u], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);  // the products stay ahead of the wait for the copies
    __builtin_amdgcn_s_waitcnt(0x0F70);
    if (c + 2 < n_chunk) {
      ms_dma<0>(kt + (c + 2) * MS_CH * 512, wave, lane);
      av = qa[(c + 2) * MS_CH];
    }
    ms_read_b<1>(bv, wave, lane);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] = __builtin_amdgcn_mfma_f64_16x16x4f64(an, bv[u], acc[u], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
  }
  __syncthreads();  // every wave is done with the chunk buffers, which now hold scores

  double* sc = reinterpret_cast<double*>(s_ms);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    // rows 8half .. 8half + 7: lane l holds rows l/16 + 4r for r = 2half, 2half + 1
#pragma unroll
    for (int rr = 0; rr < 2; ++rr)
#pragma unroll
      for (int u = 0; u < 8; ++u)
        sc[((lane >> 4) + 4 * rr) * MS_SC + wave * 128 + 16 * u + (lane & 15)] = acc[u][2 * half + rr];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r8 = 2 * wave + i;  // row within the 8
      const int64_t row = row0 + 8 * half + r8;
      if (row < a.rows) {  // wave-uniform
        uint64_t key[8];
        bool valid[8], sel[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          valid[j] = true;
          key[j] = ordered_key(sc[r8 * MS_SC + lane + 64 * j]);
        }
        wave_topk<8>(key, valid, a.topk, below, sel);
        int32_t* out = a.idx + (((int64_t)b * a.heads_q + h) * a.rows + row) * a.topk;
        int base = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint64_t m = __ballot(sel[j]);
          if (sel[j]) out[base + popc64(m & below)] = lane + 64 * j;
          base += popc64(m);
        }
      }
    }
    __syncthreads();  // the next 8 rows overwrite the exchange
  }
}

// ---------------------------------------------------------------------------
// Wide rows in two passes (workspace given; more than 1024 candidates, no
// parent list, top-k <= 256).  The candidates are cut into parts of PART keys.
// Pass 1: a workgroup takes one part for up to 4*PRW rows that read the same key
// head (the rows of the query heads of one group, head-major), streams the
// part's transposed means through LDS in 8-channel chunks (every wave reads
// every key of a chunk), and writes each row's top-k of the part, in ascending key
// order, to the workspace (empty slots: candidate -1).  Pass 2: a workgroup
// per row takes the top-k of the parts' survivors, which are in ascending key
// order part after part (in two steps, below).  A key in the row's top-k is in
// its part's top-k under the same order, so the result equals the one-pass
// selection.
// ---------------------------------------------------------------------------
constexpr int PART = 512;        // keys per part (KPL 8)
constexpr int PRW = 1;           // rows per wave in pass 1 (one: a shorter chain per wave; 2 rows cost the LoSA step 5 us)
constexpr int PMAX_K = 256;      // largest top-k of the two-pass path

__host__ __device__ inline int64_t part_count(int64_t n_cand) { return (n_cand + PART - 1) / PART; }

// chunk of 8 channels x PART keys of one part into LDS buffer P: channel row
// c0+i lands at 4 KB * i; a lane whose key pair lies past the candidates reads
// the last pair of the channel row instead (never used)
template <int P>
__device__ __forceinline__ void part_dma(const double* kt, int c0, int k0, int64_t keys, int n_cand) {
  uint8_t* dst = P ? s_sel1 : s_sel0;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int kp = k0 + (wave * 1024 + lane * 16) / 8;  // first key of this lane's pair
  kp = kp + 1 < n_cand ? kp : ((n_cand - 2) & ~1);
#pragma unroll
  for (int i = 0; i < SEL_CH; ++i)
    __builtin_amdgcn_global_load_lds(kt + (int64_t)(c0 + i) * keys + kp,
                                     (lds_void*)(dst + i * 4096 + wave * 1024), 16, 0, 0);
}

template <int P>
__device__ __forceinline__ void part_chunk(const double* const* qp, int c0, double (*acc)[PART / 64]) {
  constexpr int KPL = PART / 64;
  const double* kc = reinterpret_cast<const double*>(P ? s_sel1 : s_sel0);
  const int lane = threadIdx.x & 63;
#pragma unroll 2
  for (int cc = 0; cc < SEL_CH; ++cc) {
    double kv[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) kv[j] = kc[cc * PART + lane + 64 * j];
#pragma unroll
    for (int i = 0; i < PRW; ++i) {
      const double qv = uniform_ld(qp[i] + c0 + cc);
#pragma unroll
      for (int j = 0; j < KPL; ++j) acc[i][j] = __builtin_fma(qv, kv[j], acc[i][j]);
    }
  }
}

__global__ __launch_bounds__(256, 2) void select_part_kernel(SelArgs a, int n_parts, int64_t groups,
                                                            uint64_t* __restrict__ ws_key,
                                                            int32_t* __restrict__ ws_cand) {
  constexpr int KPL = PART / 64;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // (b, kv head, part, row group), row group fastest: neighbouring workgroups
  // read the same part of the same key head
  const int64_t unit = xcd_major(blockIdx.x, gridDim.x);
  const int64_t rg = unit % groups;
  const int p = (int)((unit / groups) % n_parts);
  const int hk = (int)((unit / (groups * n_parts)) % a.heads_kv);
  const int b = (int)(unit / (groups * n_parts * a.heads_kv));
  const int64_t rows_kv = (int64_t)a.group * a.rows;  // rows that read key head hk
  const double* kt = a.kt + ((int64_t)b * a.heads_kv + hk) * a.d * a.keys;
  const int k0 = p * PART;

  // this wave's rows: kv-head row r -> query head hk*group + r/rows, row r%rows
  const double* qp[PRW];
  int64_t orow[PRW];
#pragma unroll
  for (int i = 0; i < PRW; ++i) {
    const int64_t r = rg * 4 * PRW + wave * PRW + i;
    const int64_t rr = r < rows_kv ? r : 0;
    const int h = hk * a.group + (int)(rr / a.rows);
    const int64_t row = rr % a.rows;
    int64_t qr = row;
    if (a.q_rows) qr = a.q_rows[(int64_t)b * a.rows + row];
    if (qr < 0 || qr >= a.q_len) qr = 0;  // a row map entry outside q reads row 0
    qr = __builtin_amdgcn_readfirstlane((int)qr);
    qp[i] = a.q + (((int64_t)b * a.heads_q + h) * a.q_len + qr) * a.d;
    orow[i] = r < rows_kv ? (((int64_t)b * a.heads_q + h) * a.rows + row) : -1;
  }
  double acc[PRW][KPL];
#pragma unroll
  for (int i = 0; i < PRW; ++i)
#pragma unroll
    for (int j = 0; j < KPL; ++j) acc[i][j] = 0.0;

  const int n_chunk = a.d / SEL_CH;  // even (checked at launch)
  part_dma<0>(kt, 0, k0, a.keys, a.n_cand);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  for (int c = 0; c < n_chunk; c += 2) {
    part_dma<1>(kt, (c + 1) * SEL_CH, k0, a.keys, a.n_cand);
    part_chunk<0>(qp, c * SEL_CH, acc);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (c + 2 < n_chunk) part_dma<0>(kt, (c + 2) * SEL_CH, k0, a.keys, a.n_cand);
    part_chunk<1>(qp, (c + 1) * SEL_CH, acc);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  }

  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int i = 0; i < PRW; ++i) {
    if (orow[i] < 0) continue;
    uint64_t key[KPL];
    bool valid[KPL], sel[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      valid[j] = k0 + lane + 64 * j < a.n_cand;
      key[j] = valid[j] ? ordered_key(acc[i][j]) : 0ull;
    }
    wave_topk<KPL>(key, valid, a.topk, below, sel);
    uint64_t* wk = ws_key + (orow[i] * n_parts + p) * a.topk;
    int32_t* wc = ws_cand + (orow[i] * n_parts + p) * a.topk;
    int base = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const uint64_t m = __ballot(sel[j]);
      if (sel[j]) {
        const int pos = base + popc64(m & below);
        wk[pos] = key[j];
        wc[pos] = k0 + lane + 64 * j;
      }
      base += popc64(m);
    }
    for (int e = base + lane; e < a.topk; e += 64) wc[e] = -1;  // fewer than k candidates
  }
}

// Pass 2, a workgroup per row: wave w takes the top-k of the quarter
// [w*Q, (w+1)*Q) of the row's n_parts*topk survivors (KPL per lane), and wave 0
// the top-k of the quarters' survivors (KPL2 per lane), which stay in
// workspace order, i.e. ascending candidate order.  An entry of the row's top-k
// is in its quarter's top-k under the same order, so this is exact.  (One wave
// per row over all survivors took 19 us for the 160 LoSA rows; the four
// shorter chains take the LoSA step 6 us lower.)
template <int KPL, int KPL2>
__global__ __launch_bounds__(256) void select_merge4_kernel(SelArgs a, int n_parts,
                                                            const uint64_t* __restrict__ ws_key,
                                                            const int32_t* __restrict__ ws_cand) {
  __shared__ uint64_t s_key[4][WIDE_MAX_K];
  __shared__ int32_t s_cand[4][WIDE_MAX_K];
  __shared__ int s_n[4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t r = blockIdx.x;  // (b, h, row) flattened
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int n_e = n_parts * a.topk;
  const int qtr = (n_e + 3) / 4;
  const int e_lo = wave * qtr, e_hi = min(n_e, e_lo + qtr);
  uint64_t key[KPL];
  bool valid[KPL], sel[KPL];
  int cand[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const int e = e_lo + lane + 64 * j;
    cand[j] = e < e_hi ? ws_cand[r * n_e + e] : -1;
    valid[j] = cand[j] >= 0;
    key[j] = valid[j] ? ws_key[r * n_e + e] : 0ull;
  }
  wave_topk<KPL>(key, valid, a.topk, below, sel);
  int base = 0;
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const uint64_t m = __ballot(sel[j]);
    if (sel[j]) {
      const int pos = base + popc64(m & below);
      s_key[wave][pos] = key[j];
      s_cand[wave][pos] = cand[j];
    }
    base += popc64(m);
  }
  if (lane == 0) s_n[wave] = base;
  __syncthreads();
  if (wave != 0) return;
  int off[5];
  off[0] = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) off[w + 1] = off[w] + s_n[w];
  uint64_t key2[KPL2];
  bool valid2[KPL2], sel2[KPL2];
  int cand2[KPL2];
#pragma unroll
  for (int j = 0; j < KPL2; ++j) {
    const int e = lane + 64 * j;
    valid2[j] = e < off[4];
    key2[j] = 0ull;
    cand2[j] = -1;
    if (valid2[j]) {
      int w = 0;
      while (e >= off[w + 1]) ++w;
      key2[j] = s_key[w][e - off[w]];
      cand2[j] = s_cand[w][e - off[w]];
    }
  }
  wave_topk<KPL2>(key2, valid2, a.topk, below, sel2);
  int32_t* out = a.idx + r * a.topk;
  base = 0;
#pragma unroll
  for (int j = 0; j < KPL2; ++j) {
    const uint64_t m = __ballot(sel2[j]);
    if (sel2[j]) out[base + popc64(m & below)] = cand2[j];
    base += popc64(m);
  }
}

template <int KPL, int RW>
hipError_t launch_kr(const SelArgs& a, int64_t batch, hipStream_t s) {
  const int64_t rows_per_wg = 4 * RW;
  dim3 grid((unsigned)((a.rows + rows_per_wg - 1) / rows_per_wg), (unsigned)a.heads_q, (unsigned)batch);
  select_blocks_kernel<KPL, RW><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// CHANGE mode: per token, mean over heads and channels of (cur - prev)^2 in
// float64; the topk largest (ties to the lower token), ascending.  One
// workgroup per batch entry; wave w sums tokens w, w+4, ...
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ double sq_diff_row(const T* cur, const T* prev, int d) {
  double s = 0.0;
#pragma unroll 8  // the loads of 8 channel groups in flight; the sum keeps its order
  for (int c = 0; c < d; c += 8) {
    float x[8], y[8];
    if constexpr (sizeof(T) == 8) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const double df = (double)cur[c + i] - (double)prev[c + i];
        s = __builtin_fma(df, df, s);
      }
      continue;
    } else {
      Vec8<T>::load(cur + c, x);
      Vec8<T>::load(prev + c, y);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double df = (double)x[i] - (double)y[i];
      s = __builtin_fma(df, df, s);
    }
  }
  return s;
}

// Sixteen threads per token: thread g of a token sums the squared change of
// heads g, g+16, ... over all channels; the sixteen partials are then added in
// a fixed order, so the result does not depend on scheduling.
template <typename T>
__global__ __launch_bounds__(256) void select_change_kernel(const T* __restrict__ cur,
                                                            const T* __restrict__ prev, int heads,
                                                            int tokens, int d, int topk,
                                                            int32_t* __restrict__ idx) {
  __shared__ double part[256];
  __shared__ double mse[1024];
  __shared__ int keep[1024];
  const int b = blockIdx.x;
  const int g = threadIdx.x & 15;
  for (int t0 = 0; t0 < tokens; t0 += 16) {
    const int t = t0 + (threadIdx.x >> 4);
    double s = 0.0;
    if (t < tokens) {
      for (int h = g; h < heads; h += 16) {
        const int64_t base = (((int64_t)b * heads + h) * tokens + t) * d;
        s += sq_diff_row<T>(cur + base, prev + base, d);
      }
    }
    part[threadIdx.x] = s;
    __syncthreads();
    if (g == 0 && t < tokens) {
      double tot = 0.0;
      for (int i = 0; i < 16; ++i) tot += part[threadIdx.x + i];
      mse[t] = tot / ((double)heads * (double)d);
    }
    __syncthreads();
  }
  for (int t = threadIdx.x; t < tokens; t += 256) {
    const double v = mse[t];
    int rank = 0;
    for (int u = 0; u < tokens; ++u) {
      const double w = mse[u];
      rank += (w > v || (w == v && u < t)) ? 1 : 0;
    }
    keep[t] = rank < topk ? 1 : 0;
  }
  __syncthreads();
  for (int t = threadIdx.x; t < tokens; t += 256) {
    if (!keep[t]) continue;
    int pos = 0;
    for (int u = 0; u < t; ++u) pos += keep[u];
    idx[(int64_t)b * topk + pos] = t;
  }
}

}  // namespace

int64_t select_workspace_bytes(const basa_select_desc* d) {
  // (an even key count keeps the 16-byte loads of key pairs aligned)
  if (d->mode != BASA_SELECT_BLOCKS || d->parent || d->keys <= 1024 || d->keys > 4096 ||
      d->keys % 2 != 0 || d->topk > PMAX_K || d->topk < 1 || d->batch < 1 || d->rows < 1 ||
      d->heads_q < 1 || d->head_dim % (2 * SEL_CH) != 0)
    return 0;
  const int64_t n_rows = d->batch * d->heads_q * d->rows;
  return n_rows * part_count(d->keys) * d->topk * (int64_t)(sizeof(uint64_t) + sizeof(int32_t));
}

hipError_t launch_select_blocks(const basa_select_desc* d, const double* q, const double* kt,
                                int32_t* idx, hipStream_t s) {
  SelArgs a;
  a.q = q;
  a.kt = kt;
  a.idx = idx;
  a.q_rows = d->q_rows;
  a.parent = d->parent;
  a.q_len = d->q_len;
  a.rows = d->rows;
  a.keys = d->keys;
  a.d = (int)d->head_dim;
  a.topk = d->topk;
  a.heads_q = (int)d->heads_q;
  a.heads_kv = (int)d->heads_kv;
  a.group = (int)(d->heads_q / d->heads_kv);
  a.parent_k = d->parent ? d->parent_k : 0;
  a.fanout = d->parent ? d->fanout : 1;
  a.n_cand = d->parent ? d->parent_k * d->fanout : (int)d->keys;
  if (a.rows == 0 || d->batch == 0 || d->heads_q == 0) return hipSuccess;
  // rows per wave: share each key load across rows while RW*KPL stays <= 32
  // doubles; with a parent list all rows of a wave must share one parent
  const int kpl = (a.n_cand + 63) / 64;
  const bool one_row = d->parent && (a.fanout % 4) != 0;
  if (kpl <= 1) return one_row ? launch_kr<1, 1>(a, d->batch, s) : launch_kr<1, 4>(a, d->batch, s);
  if (kpl <= 2) return one_row ? launch_kr<2, 1>(a, d->batch, s) : launch_kr<2, 4>(a, d->batch, s);
  if (kpl <= 4) return one_row ? launch_kr<4, 1>(a, d->batch, s) : launch_kr<4, 4>(a, d->batch, s);
  if (!d->parent && a.keys == 512 && a.d % (2 * MS_CH) == 0) {  // float64 matrix core
    const int64_t groups = (a.rows + 15) / 16;
    dim3 grid((unsigned)(groups * a.heads_q * d->batch), 1);
    select_mfma_kernel<<<grid, 256, 0, s>>>(a, groups);
    return hipGetLastError();
  }
  if (kpl > 4 && kpl <= 8 && !d->parent && a.d % 4 == 0) {  // channel-split rows
    const int64_t groups = (a.rows + 3) / 4;
    dim3 grid((unsigned)(groups * a.heads_q * d->batch), 1);
    select_split_kernel<8><<<grid, 256, 0, s>>>(a, groups);
    return hipGetLastError();
  }
  if (kpl <= 8) return one_row ? launch_kr<8, 1>(a, d->batch, s) : launch_kr<8, 4>(a, d->batch, s);
  if (kpl <= 16) return launch_kr<16, 1>(a, d->batch, s);
  const int64_t ws_need = select_workspace_bytes(d);
  if (ws_need > 0 && d->workspace && d->workspace_bytes >= ws_need &&
      (reinterpret_cast<uintptr_t>(d->workspace) & 7) == 0) {
    // two passes: parts of PART keys, then the merge
    const int n_parts = (int)part_count(a.n_cand);
    const int64_t n_rows = d->batch * a.heads_q * a.rows;
    uint64_t* ws_key = static_cast<uint64_t*>(d->workspace);
    int32_t* ws_cand = reinterpret_cast<int32_t*>(ws_key + n_rows * n_parts * a.topk);
    const int64_t groups = ((int64_t)a.group * a.rows + 4 * PRW - 1) / (4 * PRW);
    dim3 g1((unsigned)(groups * n_parts * a.heads_kv * d->batch), 1);
    select_part_kernel<<<g1, 256, 0, s>>>(a, n_parts, groups, ws_key, ws_cand);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // pass 2: a workgroup per row, quarters of at most 4*64 (or 8*64) survivors
    dim3 g2((unsigned)n_rows, 1);
    const int qtr = (n_parts * a.topk + 3) / 4;
    if (qtr <= 4 * 64 && a.topk <= 128)
      select_merge4_kernel<4, 8><<<g2, 256, 0, s>>>(a, n_parts, ws_key, ws_cand);
    else if (qtr <= 4 * 64)
      select_merge4_kernel<4, 16><<<g2, 256, 0, s>>>(a, n_parts, ws_key, ws_cand);
    else if (a.topk <= 128)
      select_merge4_kernel<8, 8><<<g2, 256, 0, s>>>(a, n_parts, ws_key, ws_cand);
    else
      select_merge4_kernel<8, 16><<<g2, 256, 0, s>>>(a, n_parts, ws_key, ws_cand);
    return hipGetLastError();
  }
  if (a.topk <= WIDE_MAX_K) {  // a workgroup per row, four quarters of at most 1024
    dim3 grid((unsigned)a.rows, (unsigned)a.heads_q, (unsigned)d->batch);
    select_wide_kernel<16><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
  }
  if (kpl <= 32) return launch_kr<32, 1>(a, d->batch, s);
  return launch_kr<64, 1>(a, d->batch, s);
}

int64_t pool_select_workspace_bytes(const basa_select_desc*) { return 0; }

hipError_t launch_select_change(const basa_select_desc* d, const void* q, const void* k, int dtype,
                                int32_t* idx, hipStream_t s) {
  if (d->batch == 0) return hipSuccess;
  dim3 grid((unsigned)d->batch);
  const int H = (int)d->heads_q, T = (int)d->q_len, D = (int)d->head_dim;
  if (dtype == BASA_BF16)
    select_change_kernel<uint16_t><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(q),
                                                        static_cast<const uint16_t*>(k), H, T, D,
                                                        d->topk, idx);
  else if (dtype == BASA_F32)
    select_change_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float*>(q),
                                                     static_cast<const float*>(k), H, T, D,
                                                     d->topk, idx);
  else
    select_change_kernel<double><<<grid, 256, 0, s>>>(static_cast<const double*>(q),
                                                      static_cast<const double*>(k), H, T, D,
                                                      d->topk, idx);
  return hipGetLastError();
}

hipError_t launch_select_ranges(const double* scores, int64_t rows, int64_t n, int64_t split,
                                int k_lo, int k_hi, int32_t* idx, hipStream_t s) {
  const dim3 grid((unsigned)((rows + 3) / 4));
  const int nn = (int)n, sp = (int)split;
  if (n <= 64)
    select_ranges_kernel<1><<<grid, 256, 0, s>>>(scores, rows, nn, sp, k_lo, k_hi, idx);
  else if (n <= 128)
    select_ranges_kernel<2><<<grid, 256, 0, s>>>(scores, rows, nn, sp, k_lo, k_hi, idx);
  else if (n <= 256)
    select_ranges_kernel<4><<<grid, 256, 0, s>>>(scores, rows, nn, sp, k_lo, k_hi, idx);
  else if (n <= 512)
    select_ranges_kernel<8><<<grid, 256, 0, s>>>(scores, rows, nn, sp, k_lo, k_hi, idx);
  else
    select_ranges_kernel<16><<<grid, 256, 0, s>>>(scores, rows, nn, sp, k_lo, k_hi, idx);
  return hipGetLastError();
}

}  // namespace basa
