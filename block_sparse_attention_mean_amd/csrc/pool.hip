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

}  // namespace basa
