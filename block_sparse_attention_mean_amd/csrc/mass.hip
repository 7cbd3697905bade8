// Dense block mass of the attention map (BA-Att Eq. 3, the oracle block
// distribution; SparseD section 3.3, whose average-pooled attention scores
// are this mass divided by the block size):
//   m[gq][gk] = (1/block) sum_{i in gq} sum_{j in gk} A_ij,
//   A_ij = exp(s_ij - LSE_i),  s_ij = scale * q_i . k_j,  LSE_i over all keys.
//
// Everything is float64: the logits (products of exact float64 widenings of
// the bf16/float32 inputs), the row LSE and the block sums, so that a top-k
// over the mass is decided as an exact float64 reference would decide it.
// One workgroup per query block; each of its rows is owned by 256/block
// consecutive threads that split every staged key chunk between them.  Pass 1
// forms each row's LSE (online max and sum); pass 2 adds exp(s - LSE) per key
// block, and the workgroup adds its threads' partial sums in a fixed tree.
// This is a dense pass (the pattern it feeds is computed once and reused).
// Blocks of 16..128 rows (multiples of 16) take the float64 MFMA kernel
// below; other blocks take this one-thread-per-row kernel.
#include "common.h"

#include <type_traits>

namespace basa {
namespace {

constexpr int MASS_NT = 256;
constexpr int MASS_MAX_D = 128;
constexpr int MASS_KC = 32;  // keys per staged chunk

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<uint16_t>(uint16_t v) { return bf16_bits_to_f32(v); }
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }

struct MassArgs {
  const void* q;
  const void* k;
  double* mass;
  int64_t len_q, len_k;
  int heads_q, heads_kv, d, block;
  double scale;
};

// keys [j0, j0 + MASS_KC) of the head into LDS as float64 (rows past len_k: zero)
template <typename T>
__device__ __forceinline__ void stage_keys(const T* kh, int64_t len_k, int d, int64_t j0, double* kc) {
  for (int e = threadIdx.x; e < MASS_KC * d; e += MASS_NT) {
    const int64_t j = j0 + e / d;
    kc[e] = j < len_k ? (double)to_f32<T>(kh[j * d + e % d]) : 0.0;
  }
}

// channels past d hold zero in both operands' staging (q) or are never read (k)
__device__ __forceinline__ double dot_row(const float* qr, const double* kr, int d) {
  double s = 0.0;
#pragma unroll
  for (int c = 0; c < MASS_MAX_D; ++c)
    if (c < d) s = __builtin_fma((double)qr[c], kr[c], s);
  return s;
}

template <typename T>
__global__ __launch_bounds__(MASS_NT) void block_mass_kernel(MassArgs a) {
  __shared__ double kc[MASS_KC * MASS_MAX_D];
  __shared__ double red[MASS_NT];
  const int64_t nq = a.len_q / a.block, nk = a.len_k / a.block;
  const int64_t gq = blockIdx.x % nq;
  const int64_t bh = blockIdx.x / nq;
  const int h = (int)(bh % a.heads_q);
  const int64_t b = bh / a.heads_q;
  const int hk = h / (a.heads_q / a.heads_kv);
  const int d = a.d;
  const int tpr = MASS_NT / a.block;  // threads per row (block divides 256)
  const int row = threadIdx.x / tpr, sub = threadIdx.x % tpr;
  const T* qh = static_cast<const T*>(a.q) + ((b * a.heads_q + h) * a.len_q + gq * a.block) * d;
  const T* kh = static_cast<const T*>(a.k) + (b * a.heads_kv + hk) * a.len_k * d;
  float qr[MASS_MAX_D];
#pragma unroll
  for (int c = 0; c < MASS_MAX_D; ++c) qr[c] = c < d ? to_f32<T>(qh[(int64_t)row * d + c]) : 0.f;

  // pass 1: LSE of the row over all keys (online max and sum, float64)
  double m = -INFINITY, l = 0.0;
  for (int64_t j0 = 0; j0 < a.len_k; j0 += MASS_KC) {
    __syncthreads();
    stage_keys<T>(kh, a.len_k, d, j0, kc);
    __syncthreads();
    for (int jj = sub; jj < MASS_KC && j0 + jj < a.len_k; jj += tpr) {
      const double s = a.scale * dot_row(qr, kc + jj * d, d);
      if (s > m) {
        l = l * exp(m - s) + 1.0;
        m = s;
      } else {
        l += exp(s - m);
      }
    }
  }
  // the row's tpr threads are consecutive lanes: combine their (m, l)
  for (int off = 1; off < tpr; off <<= 1) {
    const double mo = __shfl_xor(m, off), lo = __shfl_xor(l, off);
    const double mn = fmax(m, mo);
    l = (m == -INFINITY ? 0.0 : l * exp(m - mn)) + (mo == -INFINITY ? 0.0 : lo * exp(mo - mn));
    m = mn;
  }
  const double lse = m + log(l);

  // pass 2: per key block, the sum of exp(s - LSE) over the block's rows and keys
  double* out = a.mass + (bh * nq + gq) * nk;
  for (int64_t gk = 0; gk < nk; ++gk) {
    double part = 0.0;
    for (int64_t j0 = gk * a.block; j0 < (gk + 1) * a.block; j0 += MASS_KC) {
      __syncthreads();
      stage_keys<T>(kh, a.len_k, d, j0, kc);
      __syncthreads();
      const int64_t jend = (gk + 1) * a.block;
      for (int jj = sub; jj < MASS_KC && j0 + jj < jend; jj += tpr)
        part += exp(a.scale * dot_row(qr, kc + jj * d, d) - lse);
    }
    red[threadIdx.x] = part;
    __syncthreads();
    for (int w = MASS_NT / 2; w > 0; w >>= 1) {
      if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
      __syncthreads();
    }
    if (threadIdx.x == 0) out[gk] = red[0] / a.block;
  }
}

// ---------------------------------------------------------------------------
// The same mass on the float64 matrix core (v_mfma_f64_16x16x4f64), for
// blocks of 16..128 rows that are multiples of 16 and head_dim <= 128.  Each
// wave owns 16-row query tiles (tile w, w+4, ...); for channel step s the
// A operand of lane l is Q[row0 + l%16][4s + l/16] (kept in registers), the
// B operand K[j0 + l%16][4s + l/16] (from LDS), and lane l receives the
// logits of rows row0 + l/16 + 4r (r = 0..3) at key j0 + l%16.  Keys are
// staged in LDS as float64 with a row stride of head_dim + 2 doubles, which
// spreads the 16 keys x 2 channel groups a half-wave reads over all banks,
// in two buffers: the loads of chunk c + 1 are in flight while chunk c is
// multiplied, and one barrier per chunk separates them.
// ---------------------------------------------------------------------------
typedef double f64x4 __attribute__((ext_vector_type(4)));
constexpr int MM_TILES = 2;              // 16-row tiles per wave (blocks up to 128 rows)
constexpr int MM_STEPS = MASS_MAX_D / 4;  // channel steps of 4

// One chunk of KC keys in flight: thread t holds the 8-channel groups t,
// t + 256, ... of the chunk (16-byte loads of bf16, 32 of float32), issued a
// chunk ahead and written to LDS as float64 (row stride head_dim + 2) once the
// current chunk is done, so the matrix core does not wait on the loads.
template <typename T, int KC>
struct KeyStage {
  static constexpr int NG = KC / 16;            // groups per thread (head_dim <= 128)
  static constexpr int W = sizeof(T) / 2;       // 16-byte words per group of 8 values
  uint4 raw[NG][W];
  __device__ __forceinline__ void load(const T* kh, int d, int64_t j0) {
    const int gpr = d >> 3;  // groups per key
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const int g = threadIdx.x + i * MASS_NT;
      if (g < KC * gpr) {
        const uint4* src = reinterpret_cast<const uint4*>(kh + (j0 + g / gpr) * d + (g % gpr) * 8);
#pragma unroll
        for (int w = 0; w < W; ++w) raw[i][w] = src[w];
      }
    }
  }
  __device__ __forceinline__ void store(double* kc, int d) const {
    const int gpr = d >> 3, str = d + 2;
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const int g = threadIdx.x + i * MASS_NT;
      if (g < KC * gpr) {
        double v[8];
        if constexpr (sizeof(T) == 2) {
          const uint32_t wd[4] = {raw[i][0].x, raw[i][0].y, raw[i][0].z, raw[i][0].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[2 * e] = (double)bf16_bits_to_f32(wd[e] & 0xFFFFu);
            v[2 * e + 1] = (double)bf16_bits_to_f32(wd[e] >> 16);
          }
        } else {
#pragma unroll
          for (int w = 0; w < 2; ++w) {
            v[4 * w] = (double)__uint_as_float(raw[i][w].x);
            v[4 * w + 1] = (double)__uint_as_float(raw[i][w].y);
            v[4 * w + 2] = (double)__uint_as_float(raw[i][w].z);
            v[4 * w + 3] = (double)__uint_as_float(raw[i][w].w);
          }
        }
        double2* dst = reinterpret_cast<double2*>(kc + (g / gpr) * str + (g % gpr) * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[e] = double2{v[2 * e], v[2 * e + 1]};
      }
    }
  }
};

// Online (max, sum of exp(s - max)) update with one exponential and no branch:
// with d = v - m, a new maximum (d > 0) rescales the sum by exp(-d) and adds 1,
// otherwise exp(d) is added; both are exp(-|d|), so lanes that disagree do not
// make the wave evaluate the (software, float64) exponential twice.  The same
// exponentials as the two-branch form; the sums can round differently only in
// how the compiler fuses the multiply-add.
__device__ __forceinline__ void online_add(double v, double& m, double& l) {
  const double d = v - m;  // m = -inf at the start: d = +inf, e = 0, l = 0 * 0 + 1
  const double e = exp(-fabs(d));
  l = d > 0.0 ? l * e + 1.0 : l + e;
  m = d > 0.0 ? v : m;
}

// The 16x16 logits of tile t against every 16-key sub-tile of the staged chunk:
// the KC/16 accumulation chains advance together, so the matrix core always has
// an independent product to start.  NS > 0: head_dim = 4*NS is a compile-time
// constant, so every key read has a fixed offset and none waits behind a branch;
// NS = 0: any head_dim that is a multiple of 4 (steps past it are skipped).
template <int KC, int NS>
__device__ __forceinline__ void chunk_logits(const double (*aq)[MM_STEPS], int t, const double* kc,
                                             int d, int lane, f64x4 (&sv)[KC / 16]) {
  constexpr int NU = KC / 16;
  const int str = NS > 0 ? 4 * NS + 2 : d + 2;
  const double* kb = kc + (lane & 15) * str + (lane >> 4);
#pragma unroll
  for (int u = 0; u < NU; ++u) sv[u] = f64x4{0.0, 0.0, 0.0, 0.0};
  if constexpr (NS > 0) {
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int u = 0; u < NU; ++u)
        sv[u] = __builtin_amdgcn_mfma_f64_16x16x4f64(aq[t][s], kb[u * 16 * str + 4 * s], sv[u], 0, 0, 0);
  } else {
#pragma unroll
    for (int s = 0; s < MM_STEPS; ++s)
      if (4 * s < d)
#pragma unroll
        for (int u = 0; u < NU; ++u)
          sv[u] = __builtin_amdgcn_mfma_f64_16x16x4f64(aq[t][s], kb[u * 16 * str + 4 * s], sv[u], 0, 0, 0);
  }
}

template <typename T, int KC, int NS>
__global__ __launch_bounds__(MASS_NT, 2) void block_mass_mfma_kernel(MassArgs a) {
  __shared__ double kc0[KC * (MASS_MAX_D + 2)];
  __shared__ double kc1[KC * (MASS_MAX_D + 2)];
  __shared__ double red[2][MASS_NT / 64];
  const int64_t nq = a.len_q / a.block, nk = a.len_k / a.block;
  const int64_t gq = blockIdx.x % nq;
  const int64_t bh = blockIdx.x / nq;
  const int h = (int)(bh % a.heads_q);
  const int64_t b = bh / a.heads_q;
  const int hk = h / (a.heads_q / a.heads_kv);
  const int d = a.d, lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_tiles = a.block / 16;
  const T* qh = static_cast<const T*>(a.q) + ((b * a.heads_q + h) * a.len_q + gq * a.block) * d;
  const T* kh = static_cast<const T*>(a.k) + (b * a.heads_kv + hk) * a.len_k * d;
  double aq[MM_TILES][MM_STEPS];
#pragma unroll
  for (int t = 0; t < MM_TILES; ++t) {
    const int tile = wave + 4 * t;
#pragma unroll
    for (int s = 0; s < MM_STEPS; ++s)
      aq[t][s] = (tile < n_tiles && 4 * s < d)
                     ? (double)to_f32<T>(qh[(int64_t)(tile * 16 + (lane & 15)) * d + 4 * s + (lane >> 4)])
                     : 0.0;
  }

  // pass 1: per row, online max and sum of exp over all keys (lane: rows lane/16 + 4r)
  double m[MM_TILES][4], l[MM_TILES][4];
#pragma unroll
  for (int t = 0; t < MM_TILES; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      m[t][r] = -INFINITY;
      l[t][r] = 0.0;
    }
  const int64_t n_chunks = a.len_k / KC;  // len_k is a multiple of block, block of KC
  KeyStage<T, KC> st;
  st.load(kh, d, 0);
  st.store(kc0, d);
  __syncthreads();
  for (int64_t c = 0; c < n_chunks; ++c) {
    const double* kc = (c & 1) ? kc1 : kc0;
    if (c + 1 < n_chunks) st.load(kh, d, (c + 1) * KC);
#pragma unroll
    for (int t = 0; t < MM_TILES; ++t) {
      if (wave + 4 * t >= n_tiles) continue;  // wave-uniform
      f64x4 sv[KC / 16];
      chunk_logits<KC, NS>(aq, t, kc, d, lane, sv);
#pragma unroll
      for (int u = 0; u < KC / 16; ++u) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const double v = a.scale * sv[u][r];
          online_add(v, m[t][r], l[t][r]);
        }
      }
    }
    if (c + 1 < n_chunks) st.store((c & 1) ? kc0 : kc1, d);
    __syncthreads();
  }
  // the 16 lanes of a group hold one row's keys: combine their (m, l)
  double lse[MM_TILES][4];
#pragma unroll
  for (int t = 0; t < MM_TILES; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      double mm = m[t][r], ll = l[t][r];
      for (int off = 1; off < 16; off <<= 1) {
        const double mo = __shfl_xor(mm, off), lo = __shfl_xor(ll, off);
        const double mn = fmax(mm, mo);
        ll = (mm == -INFINITY ? 0.0 : ll * exp(mm - mn)) + (mo == -INFINITY ? 0.0 : lo * exp(mo - mn));
        mm = mn;
      }
      lse[t][r] = mm + log(ll);
    }

  // pass 2: per key block, the sum of exp(s - LSE) over the query block; the
  // chunks run in key order and each key block's sum is closed after its last
  double* out = a.mass + (bh * nq + gq) * nk;
  const int64_t cpb = a.block / KC;  // chunks per key block
  st.load(kh, d, 0);
  st.store(kc0, d);
  __syncthreads();
  double part = 0.0;
  for (int64_t c = 0; c < n_chunks; ++c) {
    const double* kc = (c & 1) ? kc1 : kc0;
    if (c + 1 < n_chunks) st.load(kh, d, (c + 1) * KC);
#pragma unroll
    for (int t = 0; t < MM_TILES; ++t) {
      if (wave + 4 * t >= n_tiles) continue;
      f64x4 sv[KC / 16];
      chunk_logits<KC, NS>(aq, t, kc, d, lane, sv);
#pragma unroll
      for (int u = 0; u < KC / 16; ++u) {
#pragma unroll
        for (int r = 0; r < 4; ++r) part += exp(a.scale * sv[u][r] - lse[t][r]);
      }
    }
    const bool closes = (c + 1) % cpb == 0;
    const int64_t gk = c / cpb;
    if (closes) {
      for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
      if (lane == 0) red[gk & 1][wave] = part;
      part = 0.0;
    }
    if (c + 1 < n_chunks) st.store((c & 1) ? kc0 : kc1, d);
    __syncthreads();
    // red[gk & 1] is written again two key blocks later, after another barrier
    if (closes && threadIdx.x == 0)
      out[gk] = (red[gk & 1][0] + red[gk & 1][1] + red[gk & 1][2] + red[gk & 1][3]) / a.block;
  }
}

// ---------------------------------------------------------------------------
// One pass over the keys (with a workspace).  The two passes above compute
// every logit twice: once for the row LSE, once for exp(s - LSE).  Here, for
// each (row, key block), the walk keeps the block's own running max and sum of
// exp(s - max) (online inside the block, so nothing overflows), and when the
// block closes the 16 lanes of the row combine theirs and write (max, sum) to
// the workspace.  After the walk each row's LSE is formed from its (max, sum)
// pairs, and mass[gq][gk] = (1/block) sum_i sum_gk,i exp(max_gk,i - LSE_i).
// The same sums, one exponential per logit instead of two; the result differs
// from the two-pass kernel only in float64 rounding order.
// ---------------------------------------------------------------------------
template <typename T, int KC, int NS>
__global__ __launch_bounds__(MASS_NT, 2) void block_mass_onepass_kernel(MassArgs a, double2* ws) {
  __shared__ double kc0[KC * (MASS_MAX_D + 2)];
  __shared__ double kc1[KC * (MASS_MAX_D + 2)];
  __shared__ double s_lse[16 * 4 * MM_TILES];
  const int64_t nq = a.len_q / a.block, nk = a.len_k / a.block;
  const int64_t gq = blockIdx.x % nq;
  const int64_t bh = blockIdx.x / nq;
  const int h = (int)(bh % a.heads_q);
  const int64_t b = bh / a.heads_q;
  const int hk = h / (a.heads_q / a.heads_kv);
  const int d = a.d, lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_tiles = a.block / 16;
  const T* qh = static_cast<const T*>(a.q) + ((b * a.heads_q + h) * a.len_q + gq * a.block) * d;
  const T* kh = static_cast<const T*>(a.k) + (b * a.heads_kv + hk) * a.len_k * d;
  double2* wsb = ws + (bh * nq + gq) * nk * a.block;  // [key block][row]: (max, sum)
  double aq[MM_TILES][MM_STEPS];
#pragma unroll
  for (int t = 0; t < MM_TILES; ++t) {
    const int tile = wave + 4 * t;
#pragma unroll
    for (int s = 0; s < MM_STEPS; ++s)
      aq[t][s] = (tile < n_tiles && 4 * s < d)
                     ? (double)to_f32<T>(qh[(int64_t)(tile * 16 + (lane & 15)) * d + 4 * s + (lane >> 4)])
                     : 0.0;
  }
  // block-local online state of this lane's keys (rows lane/16 + 4r of each tile)
  double mb[MM_TILES][4], bb[MM_TILES][4];
#pragma unroll
  for (int t = 0; t < MM_TILES; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      mb[t][r] = -INFINITY;
      bb[t][r] = 0.0;
    }
  const int64_t n_chunks = a.len_k / KC;
  const int64_t cpb = a.block / KC;  // chunks per key block
  KeyStage<T, KC> st;
  st.load(kh, d, 0);
  st.store(kc0, d);
  __syncthreads();
  for (int64_t c = 0; c < n_chunks; ++c) {
    const double* kc = (c & 1) ? kc1 : kc0;
    if (c + 1 < n_chunks) st.load(kh, d, (c + 1) * KC);
#pragma unroll
    for (int t = 0; t < MM_TILES; ++t) {
      if (wave + 4 * t >= n_tiles) continue;  // wave-uniform
      f64x4 sv[KC / 16];
      chunk_logits<KC, NS>(aq, t, kc, d, lane, sv);
#pragma unroll
      for (int u = 0; u < KC / 16; ++u) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const double v = a.scale * sv[u][r];
          online_add(v, mb[t][r], bb[t][r]);
        }
      }
    }
    if ((c + 1) % cpb == 0) {  // key block gk closes: each row's (max, sum) to the workspace
      const int64_t gk = c / cpb;
#pragma unroll
      for (int t = 0; t < MM_TILES; ++t) {
        if (wave + 4 * t >= n_tiles) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          double mx = mb[t][r];
          for (int off = 1; off < 16; off <<= 1) mx = fmax(mx, __shfl_xor(mx, off));
          double sm = mb[t][r] == -INFINITY ? 0.0 : bb[t][r] * exp(mb[t][r] - mx);
          for (int off = 1; off < 16; off <<= 1) sm += __shfl_xor(sm, off);
          if ((lane & 15) == 0)
            wsb[gk * a.block + (wave + 4 * t) * 16 + (lane >> 4) + 4 * r] = double2{mx, sm};
          mb[t][r] = -INFINITY;
          bb[t][r] = 0.0;
        }
      }
    }
    if (c + 1 < n_chunks) st.store((c & 1) ? kc0 : kc1, d);
    __syncthreads();
  }
  // the workspace writes of every wave are visible to the workgroup after this barrier
  __syncthreads();
  // LSE of each row from its per-block (max, sum)
  for (int i = threadIdx.x; i < a.block; i += MASS_NT) {
    double mx = -INFINITY;
    for (int64_t gk = 0; gk < nk; ++gk) mx = fmax(mx, wsb[gk * a.block + i].x);
    double sm = 0.0;
    for (int64_t gk = 0; gk < nk; ++gk) {
      const double2 e = wsb[gk * a.block + i];
      if (e.x != -INFINITY) sm += e.y * exp(e.x - mx);
    }
    s_lse[i] = mx + log(sm);
  }
  __syncthreads();
  // mass of each key block: its rows' sums rescaled to their LSE, in row order
  double* out = a.mass + (bh * nq + gq) * nk;
  for (int64_t gk = threadIdx.x; gk < nk; gk += MASS_NT) {
    double sum = 0.0;
    for (int i = 0; i < a.block; ++i) {
      const double2 e = wsb[gk * a.block + i];
      if (e.x != -INFINITY) sum += e.y * exp(e.x - s_lse[i]);
    }
    out[gk] = sum / a.block;
  }
}

template <typename T> struct TypeTag { using type = T; };

}  // namespace

int64_t block_mass_workspace_bytes(int64_t batch, int64_t heads_q, int64_t len_q, int64_t len_k,
                                   int64_t head_dim, int64_t block) {
  // the one-pass kernel serves the float64 matrix-core shapes
  if (batch < 1 || heads_q < 1 || block < 16 || block % 16 != 0 || block > 16 * 4 * MM_TILES ||
      head_dim % 4 != 0 || head_dim > MASS_MAX_D || len_q < block || len_k < block)
    return 0;
  return batch * heads_q * len_q * (len_k / block) * (int64_t)sizeof(double2);
}

hipError_t launch_block_mass(const void* q, const void* k, int dtype, int64_t batch, int64_t heads_q,
                             int64_t heads_kv, int64_t len_q, int64_t len_k, int64_t head_dim,
                             int64_t block, double scale, double* mass, void* workspace, hipStream_t s) {
  MassArgs a;
  a.q = q;
  a.k = k;
  a.mass = mass;
  a.len_q = len_q;
  a.len_k = len_k;
  a.heads_q = (int)heads_q;
  a.heads_kv = (int)heads_kv;
  a.d = (int)head_dim;
  a.block = (int)block;
  a.scale = scale;
  const dim3 grid((unsigned)(batch * heads_q * (len_q / block)));
  const bool mfma = block % 16 == 0 && block <= 16 * 4 * MM_TILES && head_dim % 4 == 0;
  if (mfma) {
    // head_dim 64 or 128 at compile time; other multiples of 4 through the general steps
    const int ns = head_dim == 128 ? 32 : head_dim == 64 ? 16 : 0;
    double2* ws = static_cast<double2*>(workspace);  // the caller checked its size
    auto go = [&](auto tt, auto kc, auto nsc) {
      using T = typename decltype(tt)::type;
      constexpr int KC = decltype(kc)::value, NS = decltype(nsc)::value;
      if (ws)
        block_mass_onepass_kernel<T, KC, NS><<<grid, MASS_NT, 0, s>>>(a, ws);
      else
        block_mass_mfma_kernel<T, KC, NS><<<grid, MASS_NT, 0, s>>>(a);
    };
    auto by_ns = [&](auto tt, auto kc) {
      if (ns == 32)
        go(tt, kc, std::integral_constant<int, 32>());
      else if (ns == 16)
        go(tt, kc, std::integral_constant<int, 16>());
      else
        go(tt, kc, std::integral_constant<int, 0>());
    };
    auto by_kc = [&](auto tt) {
      if (block % 32 == 0)
        by_ns(tt, std::integral_constant<int, 32>());
      else
        by_ns(tt, std::integral_constant<int, 16>());
    };
    if (dtype == BASA_BF16)
      by_kc(TypeTag<uint16_t>());
    else
      by_kc(TypeTag<float>());
  } else if (dtype == BASA_BF16) {
    block_mass_kernel<uint16_t><<<grid, MASS_NT, 0, s>>>(a);
  } else {
    block_mass_kernel<float><<<grid, MASS_NT, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace basa
