// Block mean pooling (BA-Att section 3.1: block representatives are the means
// of their rows; the log-linear README pools level by level the same way).
//
// One workgroup per (outer, pair of consecutive blocks), or per block when the
// block count is odd.  Each thread reads 8 consecutive channels of a row with
// one 16/32/64-byte load, walking down each block in steps of
// (256 / (head_dim/8)) rows, and keeps float64 partial sums.  The partial sums
// of the row groups are combined through LDS in a fixed order, so the result
// does not depend on scheduling.  For bf16 inputs and power-of-two blocks the
// float64 sums and the division are exact.
#include "common.h"

namespace basa {
namespace {

// The input is read once: nontemporal loads keep it from displacing other
// data in the caches (measured ~6% faster on the 64K-token workload).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Load8<T>: one row's 8 channels.  load() issues the read, add() widens the
// values and adds them to the float64 partial sums; the main loop issues all
// of a step's reads before the first add so that they are in flight together.
template <typename T> struct Load8;
template <> struct Load8<uint16_t> {
  struct Raw { u32x4 a; };
  static __device__ __forceinline__ Raw load(const uint16_t* p) {
    return {__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p))};
  }
  static __device__ __forceinline__ void add(const Raw& r, double* acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += (double)bf16_bits_to_f32(r.a[i] & 0xFFFFu);
      acc[2 * i + 1] += (double)bf16_bits_to_f32(r.a[i] >> 16);
    }
  }
};
template <> struct Load8<float> {
  struct Raw { u32x4 a, b; };
  static __device__ __forceinline__ Raw load(const float* p) {
    return {__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)),
            __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + 4))};
  }
  static __device__ __forceinline__ void add(const Raw& r, double* acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[i] += (double)__uint_as_float(r.a[i]);
      acc[4 + i] += (double)__uint_as_float(r.b[i]);
    }
  }
};
template <> struct Load8<double> {
  struct Raw { double2 a[4]; };
  static __device__ __forceinline__ Raw load(const double* p) {
    Raw r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.a[i] = *reinterpret_cast<const double2*>(p + 2 * i);
    return r;
  }
  static __device__ __forceinline__ void add(const Raw& r, double* acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += r.a[i].x;
      acc[2 * i + 1] += r.a[i].y;
    }
  }
};

// Workgroups go to the 8 XCDs round-robin; numbering them so that XCD x takes
// the x-th contiguous eighth of the blocks keeps neighbouring blocks, whose
// transposed means share cache lines, in one L2.
__device__ __forceinline__ int64_t xcd_major(int64_t id, int64_t n) {
  const int64_t per = n / 8;
  if (id >= 8 * per) return id;  // the last n % 8 workgroups keep their number
  return (id % 8) * per + id / 8;
}

template <typename T, int BPW>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ x, int64_t len, int d,
                                                   int block, int64_t nb, int64_t n_wg,
                                                   double* __restrict__ mean_rows,
                                                   double* __restrict__ mean_cols,
                                                   void* __restrict__ mean_copy, int copy_dtype) {
  __shared__ double red[BPW][2048];  // [block of the workgroup][row groups][head_dim]
  const int64_t lin = (int64_t)blockIdx.x + (int64_t)blockIdx.y * gridDim.x;
  if (lin >= n_wg) return;
  const int64_t wg = xcd_major(lin, n_wg);
  const int64_t per_outer = nb / BPW;
  const int64_t o = wg / per_outer;
  const int64_t g0 = (wg - o * per_outer) * BPW;
  const int cols8 = d >> 3;
  const int groups = 256 / cols8;
  const int t = threadIdx.x;
  const int rg = t / cols8;
  const int c8 = t - rg * cols8;
  double acc[BPW][8];
#pragma unroll
  for (int s2 = 0; s2 < BPW; ++s2)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[s2][i] = 0.0;
  if (rg < groups) {
    const T* src = x + (o * len + g0 * (int64_t)block) * d + c8 * 8;
    int r = rg;
    // eight rows of each of the BPW blocks in flight per step
    for (; r + 7 * groups < block; r += 8 * groups) {
      typename Load8<T>::Raw raw[BPW][8];
#pragma unroll
      for (int s2 = 0; s2 < BPW; ++s2)
#pragma unroll
        for (int u = 0; u < 8; ++u) raw[s2][u] = Load8<T>::load(src + ((int64_t)s2 * block + r + u * groups) * d);
#pragma unroll
      for (int s2 = 0; s2 < BPW; ++s2)
#pragma unroll
        for (int u = 0; u < 8; ++u) Load8<T>::add(raw[s2][u], acc[s2]);
    }
    for (; r < block; r += groups) {
#pragma unroll
      for (int s2 = 0; s2 < BPW; ++s2)
        Load8<T>::add(Load8<T>::load(src + ((int64_t)s2 * block + r) * d), acc[s2]);
    }
#pragma unroll
    for (int s2 = 0; s2 < BPW; ++s2)
#pragma unroll
      for (int i = 0; i < 8; ++i) red[s2][rg * d + c8 * 8 + i] = acc[s2][i];
  }
  __syncthreads();
  const int used = groups < block ? groups : block;
  const double inv_n = (double)block;
  for (int e = t; e < BPW * d; e += 256) {
    const int s2 = e / d, c = e - s2 * d;
    const int64_t g = g0 + s2;
    double s = 0.0;
    for (int r = 0; r < used; ++r) s += red[s2][r * d + c];
    const double mean = s / inv_n;
    if (mean_rows) mean_rows[(o * nb + g) * d + c] = mean;
    if (mean_cols) mean_cols[(o * d + c) * nb + g] = mean;
    if (mean_copy) {
      if (copy_dtype == BASA_F32)
        reinterpret_cast<float*>(mean_copy)[(o * nb + g) * d + c] = (float)mean;
      else
        reinterpret_cast<uint16_t*>(mean_copy)[(o * nb + g) * d + c] = f64_to_bf16_bits(mean);
    }
  }
}

// Short blocks (up to 32 rows): one thread per (block, 8-channel group) adds
// the block's rows itself, so a workgroup covers 256 / (head_dim/8) blocks
// and no partial sums go through LDS.  Consecutive threads read consecutive
// 16-byte pieces of the same row.
template <typename T>
__global__ __launch_bounds__(256) void pool_short_kernel(const T* __restrict__ x, int64_t len, int d,
                                                         int block, int64_t nb, int64_t n_items,
                                                         double* __restrict__ mean_rows,
                                                         double* __restrict__ mean_cols,
                                                         void* __restrict__ mean_copy,
                                                         int copy_dtype) {
  const int64_t item = ((int64_t)blockIdx.x + (int64_t)blockIdx.y * gridDim.x) * 256 + threadIdx.x;
  if (item >= n_items) return;
  const int cols8 = d >> 3;
  const int c8 = (int)(item % cols8);
  const int64_t gb = item / cols8;  // block over all sequences
  const int64_t o = gb / nb, g = gb - o * nb;
  const T* src = x + (o * len + g * (int64_t)block) * d + c8 * 8;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int r = 0;
  for (; r + 8 <= block; r += 8) {  // eight row loads in flight, then their adds in row order
    typename Load8<T>::Raw raw[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) raw[u] = Load8<T>::load(src + (int64_t)(r + u) * d);
#pragma unroll
    for (int u = 0; u < 8; ++u) Load8<T>::add(raw[u], acc);
  }
  for (; r < block; ++r) Load8<T>::add(Load8<T>::load(src + (int64_t)r * d), acc);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = c8 * 8 + i;
    const double mean = acc[i] / (double)block;
    if (mean_rows) mean_rows[(o * nb + g) * d + c] = mean;
    if (mean_cols) mean_cols[(o * d + c) * nb + g] = mean;
    if (mean_copy) {
      if (copy_dtype == BASA_F32)
        reinterpret_cast<float*>(mean_copy)[(o * nb + g) * d + c] = (float)mean;
      else
        reinterpret_cast<uint16_t*>(mean_copy)[(o * nb + g) * d + c] = f64_to_bf16_bits(mean);
    }
  }
}

// ---------------------------------------------------------------------------
// The log-linear pyramid (log-linear README: each level pools the level below
// by `block`).  Levels 1 and 2 of every tensor in one launch: a workgroup
// takes one level-2 block of one tensor (blockIdx.y), one thread per (level-1
// block, 8-channel group) adds that block's rows in row order with all of
// them in flight, keeps the mean in LDS, and then one thread per channel adds
// the `block` level-1 means in block order.  Further levels: one thread per
// (block, 8-channel group) of every tensor, from the level below's float64
// means.  The sums run in the order pool_short_kernel uses, so every level
// equals a chain of single-level pooling calls bit for bit.
// ---------------------------------------------------------------------------
struct PyrLevel {
  double* rows;
  double* cols;
  void* copy;
};
struct PyrArgs {
  const void* x[BASA_PYRAMID_MAX_TENSORS];
  PyrLevel lv[BASA_PYRAMID_MAX_TENSORS][BASA_PYRAMID_MAX_LEVELS];
  int64_t outer, len;
  int d, block, copy_dtype;
};
constexpr int PYR_RED = 4096;  // doubles of level-1 means per workgroup (block * head_dim)

__device__ __forceinline__ void pyr_put(const PyrLevel& out, int64_t o, int64_t nb, int64_t g, int d,
                                        int c, double mean, int copy_dtype) {
  if (out.rows) out.rows[(o * nb + g) * d + c] = mean;
  if (out.cols) out.cols[(o * d + c) * nb + g] = mean;
  if (out.copy) {
    if (copy_dtype == BASA_F32)
      reinterpret_cast<float*>(out.copy)[(o * nb + g) * d + c] = (float)mean;
    else
      reinterpret_cast<uint16_t*>(out.copy)[(o * nb + g) * d + c] = f64_to_bf16_bits(mean);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void pyramid12_kernel(PyrArgs a) {
  __shared__ double red[PYR_RED];
  const int tn = blockIdx.y;
  const int d = a.d, block = a.block, cols8 = d >> 3;
  const int64_t nb1 = a.len / block, nb2 = nb1 / block;
  const int64_t o = blockIdx.x / nb2, g2 = blockIdx.x - o * nb2;
  const T* x = static_cast<const T*>(a.x[tn]);
  for (int item = threadIdx.x; item < block * cols8; item += blockDim.x) {
    const int b1 = item / cols8, c8 = item - b1 * cols8;
    const int64_t g1 = g2 * block + b1;
    const T* src = x + (o * a.len + g1 * block) * d + c8 * 8;
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int r = 0;
    // NB rows in flight (64 registers of raw data), then their adds in row order
    constexpr int NB = sizeof(T) == 2 ? 16 : (sizeof(T) == 4 ? 8 : 4);
    for (; r + NB <= block; r += NB) {
      typename Load8<T>::Raw raw[NB];
#pragma unroll
      for (int u = 0; u < NB; ++u) raw[u] = Load8<T>::load(src + (int64_t)(r + u) * d);
#pragma unroll
      for (int u = 0; u < NB; ++u) Load8<T>::add(raw[u], acc);
    }
    for (; r < block; ++r) Load8<T>::add(Load8<T>::load(src + (int64_t)r * d), acc);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double mean = acc[i] / (double)block;
      pyr_put(a.lv[tn][0], o, nb1, g1, d, c8 * 8 + i, mean, a.copy_dtype);
      red[b1 * d + c8 * 8 + i] = mean;
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    double sum = 0.0;
    for (int r = 0; r < block; ++r) sum += red[r * d + c];
    pyr_put(a.lv[tn][1], o, nb2, g2, d, c, sum / (double)block, a.copy_dtype);
  }
}

// level lv (0-based index, >= 2) from the float64 rows of level lv - 1
__global__ __launch_bounds__(256) void pyramid_next_kernel(PyrArgs a, int lv, int64_t nb_in, int64_t nb,
                                                           int64_t n_items) {
  const int64_t item = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (item >= n_items) return;
  const int tn = blockIdx.y;
  const int d = a.d, block = a.block, cols8 = d >> 3;
  const int c8 = (int)(item % cols8);
  const int64_t gb = item / cols8;
  const int64_t o = gb / nb, g = gb - o * nb;
  const double* src = a.lv[tn][lv - 1].rows + (o * nb_in + g * (int64_t)block) * d + c8 * 8;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int r = 0;
  for (; r + 8 <= block; r += 8) {
    typename Load8<double>::Raw raw[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) raw[u] = Load8<double>::load(src + (int64_t)(r + u) * d);
#pragma unroll
    for (int u = 0; u < 8; ++u) Load8<double>::add(raw[u], acc);
  }
  for (; r < block; ++r) Load8<double>::add(Load8<double>::load(src + (int64_t)r * d), acc);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    pyr_put(a.lv[tn][lv], o, nb, g, d, c8 * 8 + i, acc[i] / (double)block, a.copy_dtype);
}

template <typename T>
hipError_t launch_typed(const T* x, int64_t outer, int64_t len, int d, int block, double* mean_rows,
                        double* mean_cols, void* mean_copy, int copy_dtype, hipStream_t s) {
  const int64_t nb = len / block;
  if (block <= 32) {
    const int64_t n_items = outer * nb * (d / 8);
    const int64_t n_wg = (n_items + 255) / 256;
    const int64_t gx = n_wg < 65536 ? n_wg : 65536;
    dim3 grid((unsigned)gx, (unsigned)((n_wg + gx - 1) / gx));
    pool_short_kernel<T><<<grid, 256, 0, s>>>(x, len, d, block, nb, n_items, mean_rows, mean_cols,
                                              mean_copy, copy_dtype);
    return hipGetLastError();
  }
  // two consecutive blocks per workgroup when the count allows (bf16 and
  // float32 inputs): twice the loads in flight per thread (the 64K pooling:
  // 194 -> 178 us); four blocks need 64 KB of LDS per workgroup and measured
  // no better than one
  const bool two = nb % 2 == 0 && sizeof(T) < 8;
  const int64_t n_wg = outer * (two ? nb / 2 : nb);
  const int64_t gx = n_wg < 65536 ? n_wg : 65536;
  const int64_t gy = (n_wg + gx - 1) / gx;
  dim3 grid((unsigned)gx, (unsigned)gy);
  if (two)
    pool_kernel<T, 2><<<grid, 256, 0, s>>>(x, len, d, block, nb, n_wg, mean_rows, mean_cols, mean_copy,
                                           copy_dtype);
  else
    pool_kernel<T, 1><<<grid, 256, 0, s>>>(x, len, d, block, nb, n_wg, mean_rows, mean_cols, mean_copy,
                                           copy_dtype);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pool(const void* x, int x_dtype, int64_t outer, int64_t len, int64_t head_dim,
                       int64_t block, double* mean_rows, double* mean_cols, void* mean_copy,
                       int copy_dtype, hipStream_t s) {
  if (outer * (len / block) == 0) return hipSuccess;
  const int d = (int)head_dim, b = (int)block;
  switch (x_dtype) {
    case BASA_BF16:
      return launch_typed(static_cast<const uint16_t*>(x), outer, len, d, b, mean_rows, mean_cols,
                          mean_copy, copy_dtype, s);
    case BASA_F32:
      return launch_typed(static_cast<const float*>(x), outer, len, d, b, mean_rows, mean_cols,
                          mean_copy, copy_dtype, s);
    default:
      return launch_typed(static_cast<const double*>(x), outer, len, d, b, mean_rows, mean_cols,
                          mean_copy, copy_dtype, s);
  }
}

hipError_t launch_pool_pyramid(const basa_pyramid_tensor* t, int n_t, int x_dtype, int64_t outer,
                               int64_t len, int64_t head_dim, int64_t block, int levels,
                               int copy_dtype, hipStream_t s) {
  if (outer * len == 0) return hipSuccess;
  if (levels == 1) {  // one level: the plain pooling call per tensor
    for (int i = 0; i < n_t; ++i) {
      const hipError_t e = launch_pool(t[i].x, x_dtype, outer, len, head_dim, block,
                                       t[i].level[0].mean_rows, t[i].level[0].mean_cols,
                                       t[i].level[0].mean_copy, copy_dtype, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  PyrArgs a{};
  for (int i = 0; i < n_t; ++i) {
    a.x[i] = t[i].x;
    for (int l = 0; l < levels; ++l)
      a.lv[i][l] = PyrLevel{t[i].level[l].mean_rows, t[i].level[l].mean_cols, t[i].level[l].mean_copy};
  }
  a.outer = outer;
  a.len = len;
  a.d = (int)head_dim;
  a.block = (int)block;
  a.copy_dtype = copy_dtype;
  const int64_t nb2 = len / block / block;
  const int items = (int)(block * (head_dim / 8));
  const int threads = items >= 256 ? 256 : (items + 63) / 64 * 64;
  dim3 g12((unsigned)(outer * nb2), (unsigned)n_t);
  switch (x_dtype) {
    case BASA_BF16: pyramid12_kernel<uint16_t><<<g12, threads, 0, s>>>(a); break;
    case BASA_F32: pyramid12_kernel<float><<<g12, threads, 0, s>>>(a); break;
    default: pyramid12_kernel<double><<<g12, threads, 0, s>>>(a); break;
  }
  hipError_t e = hipGetLastError();
  int64_t nb_in = nb2;
  for (int l = 2; l < levels && e == hipSuccess; ++l) {
    const int64_t nb = nb_in / block;
    const int64_t n_items = outer * nb * (head_dim / 8);
    dim3 g((unsigned)((n_items + 255) / 256), (unsigned)n_t);
    pyramid_next_kernel<<<g, 256, 0, s>>>(a, l, nb_in, nb, n_items);
    e = hipGetLastError();
    nb_in = nb;
  }
  return e;
}

}  // namespace basa
