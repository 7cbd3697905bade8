// Block mean pooling (BA-Att section 3.1: block representatives are the means
// of their rows; the log-linear README pools level by level the same way).
//
// One workgroup per (outer, block).  Each thread reads 8 consecutive channels
// of a row with one 16/32/64-byte load, walking down the block in steps of
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

template <typename T> struct Load8;
template <> struct Load8<uint16_t> {
  static __device__ __forceinline__ void add(const uint16_t* p, double* acc) {
    const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += (double)bf16_bits_to_f32(a[i] & 0xFFFFu);
      acc[2 * i + 1] += (double)bf16_bits_to_f32(a[i] >> 16);
    }
  }
};
template <> struct Load8<float> {
  static __device__ __forceinline__ void add(const float* p, double* acc) {
    const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    const u32x4 b = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + 4));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[i] += (double)__uint_as_float(a[i]);
      acc[4 + i] += (double)__uint_as_float(b[i]);
    }
  }
};
template <> struct Load8<double> {
  static __device__ __forceinline__ void add(const double* p, double* acc) {
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      double2 a = *reinterpret_cast<const double2*>(p + i);
      acc[i] += a.x;
      acc[i + 1] += a.y;
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

template <typename T>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ x, int64_t len, int d,
                                                   int block, int64_t nb, int64_t n_wg,
                                                   double* __restrict__ mean_rows,
                                                   double* __restrict__ mean_cols,
                                                   void* __restrict__ mean_copy, int copy_dtype) {
  __shared__ double red[2048];  // [row groups][head_dim], row groups * head_dim == 2048
  const int64_t lin = (int64_t)blockIdx.x + (int64_t)blockIdx.y * gridDim.x;
  if (lin >= n_wg) return;
  const int64_t wg = xcd_major(lin, n_wg);
  const int64_t o = wg / nb;
  const int64_t g = wg - o * nb;
  const int cols8 = d >> 3;
  const int groups = 256 / cols8;
  const int t = threadIdx.x;
  const int rg = t / cols8;
  const int c8 = t - rg * cols8;
  const T* src = x + (o * len + g * (int64_t)block) * d + c8 * 8;
  double acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0;
  if (rg < groups) {
    int r = rg;
    // eight independent rows in flight per iteration
    for (; r + 7 * groups < block; r += 8 * groups) {
#pragma unroll
      for (int u = 0; u < 8; ++u) Load8<T>::add(src + (int64_t)(r + u * groups) * d, acc);
    }
    for (; r < block; r += groups) Load8<T>::add(src + (int64_t)r * d, acc);
#pragma unroll
    for (int i = 0; i < 8; ++i) red[rg * d + c8 * 8 + i] = acc[i];
  }
  __syncthreads();
  const int used = groups < block ? groups : block;
  const double inv_n = (double)block;
  for (int c = t; c < d; c += 256) {
    double s = 0.0;
    for (int r = 0; r < used; ++r) s += red[r * d + c];
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

}  // namespace

hipError_t launch_pool(const void* x, int x_dtype, int64_t outer, int64_t len, int64_t head_dim,
                       int64_t block, double* mean_rows, double* mean_cols, void* mean_copy,
                       int copy_dtype, hipStream_t s) {
  const int64_t nb = len / block;
  const int64_t n_wg = outer * nb;
  if (n_wg == 0) return hipSuccess;
  const int64_t gx = n_wg < 65536 ? n_wg : 65536;
  const int64_t gy = (n_wg + gx - 1) / gx;
  dim3 grid((unsigned)gx, (unsigned)gy);
  const int d = (int)head_dim, b = (int)block;
  switch (x_dtype) {
    case BASA_BF16:
      pool_kernel<uint16_t><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(x), len, d, b, nb,
                                                  n_wg, mean_rows, mean_cols, mean_copy, copy_dtype);
      break;
    case BASA_F32:
      pool_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float*>(x), len, d, b, nb, n_wg,
                                               mean_rows, mean_cols, mean_copy, copy_dtype);
      break;
    default:
      pool_kernel<double><<<grid, 256, 0, s>>>(static_cast<const double*>(x), len, d, b, nb, n_wg,
                                                mean_rows, mean_cols, mean_copy, copy_dtype);
      break;
  }
  return hipGetLastError();
}

}  // namespace basa
