// Norm-based token ranking and row permutation (BA-Att section 3.3, Eq. 9-10;
// Algorithm 1 steps 1, 2 and 12).
//
// Ranking.  Every token gets a sort key: its squared l2 norm in float64, the
// channels added one after another (c = 0, 1, ..., d-1), each square and each
// addition rounded separately (no fused multiply-add), one token per thread
// (rows of up to 512 bytes are first copied to LDS with coalesced loads).
// The squared norm orders tokens as the norm does in exact arithmetic and
// needs no square root.  For bf16 tokens every step is exact.  A nonnegative
// double's bit pattern orders like its value, so the key is the raw 64 bits.
// The permutation comes from two stable device-wide radix sorts (rocPRIM, a
// library primitive): all tokens of all sequences by key, then by sequence.
// The second sort keeps the first one's order inside each sequence, so every
// sequence ends up in key order with equal keys in token order.  (One
// segmented sort would give each sequence to a single workgroup, which is
// slow for the few long sequences of this path.)
//
// Permutation.  Rows of any width move as 16-, 4- or 2-byte units, one unit
// per thread: GATHER out[i] = x[perm[i]], SCATTER out[perm[i]] = x[i].
#include <cstring>

#include <rocprim/device/device_radix_sort.hpp>

#include "common.h"

namespace basa {
namespace {

constexpr int RANK_NT = 256;

__host__ __device__ inline int64_t align256(int64_t b) { return (b + 255) & ~int64_t(255); }

template <typename T> struct Row16;  // sixteen bytes of a row as float64 values, in order
template <> struct Row16<uint16_t> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void load(const uint16_t* p, double* v) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = (double)bf16_bits_to_f32(w[i] & 0xFFFFu);
      v[2 * i + 1] = (double)bf16_bits_to_f32(w[i] >> 16);
    }
  }
};
template <> struct Row16<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void load(const float* p, double* v) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  }
};
template <> struct Row16<double> {
  static constexpr int N = 2;
  static __device__ __forceinline__ void load(const double* p, double* v) {
    const double2 a = *reinterpret_cast<const double2*>(p);
    v[0] = a.x; v[1] = a.y;
  }
};

// keys[r] = squared norm of row r (bits), vals[r] = r
template <typename T>
__global__ __launch_bounds__(RANK_NT) void norm_key_kernel(const T* x, int64_t rows, int d,
                                                           uint64_t* keys, int32_t* vals) {
  const int64_t r = (int64_t)blockIdx.x * RANK_NT + threadIdx.x;
  if (r >= rows) return;
  const T* p = x + r * d;
  double s = 0.0;
  for (int c = 0; c < d; c += Row16<T>::N) {
    double v[Row16<T>::N];
    Row16<T>::load(p + c, v);
#pragma unroll
    for (int i = 0; i < Row16<T>::N; ++i) s = __dadd_rn(s, __dmul_rn(v[i], v[i]));
  }
  keys[r] = (uint64_t)__double_as_longlong(s);
  vals[r] = (int32_t)r;
}

// The same keys with coalesced reads: a workgroup copies 64 whole rows (at
// most 512 bytes each) into LDS with consecutive 16-byte loads, then one
// thread per row adds its squares from LDS in the same channel order.
constexpr int NK_ROWS = 64;
constexpr int NK_MAX_ROW = 512;  // bytes

template <typename T>
__global__ __launch_bounds__(RANK_NT) void norm_key_staged_kernel(const T* x, int64_t rows, int d,
                                                                  uint64_t* keys, int32_t* vals) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[NK_ROWS * (NK_MAX_ROW + 16)];
  const int row_bytes = d * (int)sizeof(T), stride = row_bytes + 16, upr = row_bytes / 16;
  const int64_t r0 = (int64_t)blockIdx.x * NK_ROWS;
  const int n_rows = rows - r0 < NK_ROWS ? (int)(rows - r0) : NK_ROWS;
  const uint4* src = reinterpret_cast<const uint4*>(x + r0 * d);
  for (int u = threadIdx.x; u < n_rows * upr; u += RANK_NT)
    *reinterpret_cast<uint4*>(tile + (u / upr) * stride + (u % upr) * 16) = src[u];
  __syncthreads();
  if ((int)threadIdx.x >= n_rows) return;
  const T* p = reinterpret_cast<const T*>(tile + threadIdx.x * stride);
  double s = 0.0;
  for (int c = 0; c < d; c += Row16<T>::N) {
    double v[Row16<T>::N];
    Row16<T>::load(p + c, v);
#pragma unroll
    for (int i = 0; i < Row16<T>::N; ++i) s = __dadd_rn(s, __dmul_rn(v[i], v[i]));
  }
  const int64_t r = r0 + threadIdx.x;
  keys[r] = (uint64_t)__double_as_longlong(s);
  vals[r] = (int32_t)r;
}

// seg[i] = sequence of row vals[i]
__global__ __launch_bounds__(RANK_NT) void seq_of_kernel(const int32_t* vals, int64_t rows,
                                                         int64_t len, uint32_t* seg) {
  const int64_t i = (int64_t)blockIdx.x * RANK_NT + threadIdx.x;
  if (i < rows) seg[i] = (uint32_t)(vals[i] / len);
}

// perm[i] = position of row vals[i] inside its sequence
__global__ __launch_bounds__(RANK_NT) void local_index_kernel(const int32_t* vals, int64_t rows,
                                                              int64_t len, int32_t* perm) {
  const int64_t i = (int64_t)blockIdx.x * RANK_NT + threadIdx.x;
  if (i < rows) perm[i] = (int32_t)(vals[i] % len);
}

template <typename U>
__global__ __launch_bounds__(RANK_NT) void permute_kernel(const U* x, int64_t len, int64_t upr,
                                                          int64_t units, const int32_t* perm,
                                                          int scatter, U* out) {
  const int64_t t = (int64_t)blockIdx.x * RANK_NT + threadIdx.x;
  if (t >= units) return;
  const int64_t row = t / upr, u = t - row * upr;
  const int64_t seg0 = row - row % len;  // first row of this sequence
  const int32_t p = perm[row];
  const bool ok = p >= 0 && p < len;
  if (scatter) {
    if (ok) out[(seg0 + p) * upr + u] = x[t];
  } else {
    out[t] = ok ? x[(seg0 + p) * upr + u] : U{};
  }
}

// workspace: keys in | keys out | rows | rows by key | sequences in | out |
// rows by (sequence, key) | rocPRIM temp (the larger of the two sorts')
struct RankLayout {
  int64_t keys_in, keys_out, vals_a, vals_b, seg_in, seg_out, vals_c, temp, temp_bytes, total;
  hipError_t status;  // of rocPRIM's size queries
};

int seq_bits(int64_t outer) {
  int b = 0;
  while (b < 31 && (int64_t(1) << b) < outer) ++b;
  return b;
}

RankLayout rank_layout(int64_t outer, int64_t len) {
  const int64_t n = outer * len;
  RankLayout l;
  l.keys_in = 0;
  l.keys_out = align256(l.keys_in + n * 8);
  l.vals_a = align256(l.keys_out + n * 8);
  l.vals_b = align256(l.vals_a + n * 4);
  l.seg_in = align256(l.vals_b + n * 4);
  l.seg_out = align256(l.seg_in + n * 4);
  l.vals_c = align256(l.seg_out + n * 4);
  l.temp = align256(l.vals_c + n * 4);
  // size queries: nothing is launched and no pointer is read
  size_t t1 = 0, t2 = 0;
  l.status = rocprim::radix_sort_pairs(nullptr, t1, (const uint64_t*)nullptr, (uint64_t*)nullptr,
                                       (const int32_t*)nullptr, (int32_t*)nullptr, (unsigned int)n,
                                       0u, 64u);
  if (l.status == hipSuccess && seq_bits(outer) > 0)
    l.status = rocprim::radix_sort_pairs(nullptr, t2, (const uint32_t*)nullptr, (uint32_t*)nullptr,
                                         (const int32_t*)nullptr, (int32_t*)nullptr, (unsigned int)n,
                                         0u, (unsigned int)seq_bits(outer));
  l.temp_bytes = (int64_t)(t1 > t2 ? t1 : t2);
  l.total = align256(l.temp + l.temp_bytes);
  return l;
}

}  // namespace

int64_t rank_workspace_bytes(int64_t outer, int64_t len) {
  if (outer * len == 0) return 0;
  const RankLayout l = rank_layout(outer, len);
  return l.status == hipSuccess ? l.total : -1;
}

hipError_t launch_rank(const void* x, int x_dtype, int64_t outer, int64_t len, int64_t head_dim,
                       int32_t* perm, void* workspace, int64_t workspace_bytes, hipStream_t s) {
  const RankLayout l = rank_layout(outer, len);
  if (l.status != hipSuccess) return l.status;
  if (workspace_bytes < l.total) return hipErrorInvalidValue;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint64_t* keys_in = reinterpret_cast<uint64_t*>(ws + l.keys_in);
  uint64_t* keys_out = reinterpret_cast<uint64_t*>(ws + l.keys_out);
  int32_t* vals_a = reinterpret_cast<int32_t*>(ws + l.vals_a);
  int32_t* vals_b = reinterpret_cast<int32_t*>(ws + l.vals_b);
  uint32_t* seg_in = reinterpret_cast<uint32_t*>(ws + l.seg_in);
  uint32_t* seg_out = reinterpret_cast<uint32_t*>(ws + l.seg_out);
  int32_t* vals_c = reinterpret_cast<int32_t*>(ws + l.vals_c);
  const int64_t rows = outer * len;
  const unsigned n = (unsigned)rows;
  const dim3 grid((unsigned)((rows + RANK_NT - 1) / RANK_NT));
  const int d = (int)head_dim;
  const int esize = x_dtype == BASA_BF16 ? 2 : (x_dtype == BASA_F32 ? 4 : 8);
  if (d * esize <= NK_MAX_ROW) {
    const dim3 sgrid((unsigned)((rows + NK_ROWS - 1) / NK_ROWS));
    if (x_dtype == BASA_BF16)
      norm_key_staged_kernel<uint16_t><<<sgrid, RANK_NT, 0, s>>>(static_cast<const uint16_t*>(x), rows,
                                                                 d, keys_in, vals_a);
    else if (x_dtype == BASA_F32)
      norm_key_staged_kernel<float><<<sgrid, RANK_NT, 0, s>>>(static_cast<const float*>(x), rows, d,
                                                              keys_in, vals_a);
    else
      norm_key_staged_kernel<double><<<sgrid, RANK_NT, 0, s>>>(static_cast<const double*>(x), rows, d,
                                                               keys_in, vals_a);
  } else if (x_dtype == BASA_BF16) {
    norm_key_kernel<uint16_t><<<grid, RANK_NT, 0, s>>>(static_cast<const uint16_t*>(x), rows, d,
                                                       keys_in, vals_a);
  } else if (x_dtype == BASA_F32) {
    norm_key_kernel<float><<<grid, RANK_NT, 0, s>>>(static_cast<const float*>(x), rows, d, keys_in,
                                                    vals_a);
  } else {
    norm_key_kernel<double><<<grid, RANK_NT, 0, s>>>(static_cast<const double*>(x), rows, d,
                                                     keys_in, vals_a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  size_t tb = (size_t)l.temp_bytes;
  e = rocprim::radix_sort_pairs(ws + l.temp, tb, (const uint64_t*)keys_in, keys_out,
                                (const int32_t*)vals_a, vals_b, n, 0u, 64u, s);
  if (e != hipSuccess) return e;
  const int bits = seq_bits(outer);
  const int32_t* by_seq = vals_b;
  if (bits > 0) {
    seq_of_kernel<<<grid, RANK_NT, 0, s>>>(vals_b, rows, len, seg_in);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    tb = (size_t)l.temp_bytes;
    e = rocprim::radix_sort_pairs(ws + l.temp, tb, (const uint32_t*)seg_in, seg_out,
                                  (const int32_t*)vals_b, vals_c, n, 0u, (unsigned)bits, s);
    if (e != hipSuccess) return e;
    by_seq = vals_c;
  }
  local_index_kernel<<<grid, RANK_NT, 0, s>>>(by_seq, rows, len, perm);
  return hipGetLastError();
}

hipError_t launch_permute(const void* x, int64_t outer, int64_t len, int64_t row_bytes,
                          const int32_t* perm, int mode, void* out, hipStream_t s) {
  const int scatter = mode == BASA_PERMUTE_SCATTER;
  const int64_t rows = outer * len;
  if (row_bytes % 16 == 0) {
    const int64_t upr = row_bytes / 16, units = rows * upr;
    permute_kernel<uint4><<<dim3((unsigned)((units + RANK_NT - 1) / RANK_NT)), RANK_NT, 0, s>>>(
        static_cast<const uint4*>(x), len, upr, units, perm, scatter, static_cast<uint4*>(out));
  } else if (row_bytes % 4 == 0) {
    const int64_t upr = row_bytes / 4, units = rows * upr;
    permute_kernel<uint32_t><<<dim3((unsigned)((units + RANK_NT - 1) / RANK_NT)), RANK_NT, 0, s>>>(
        static_cast<const uint32_t*>(x), len, upr, units, perm, scatter, static_cast<uint32_t*>(out));
  } else {
    const int64_t upr = row_bytes / 2, units = rows * upr;
    permute_kernel<uint16_t><<<dim3((unsigned)((units + RANK_NT - 1) / RANK_NT)), RANK_NT, 0, s>>>(
        static_cast<const uint16_t*>(x), len, upr, units, perm, scatter, static_cast<uint16_t*>(out));
  }
  return hipGetLastError();
}

}  // namespace basa
