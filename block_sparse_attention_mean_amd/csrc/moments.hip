// Block moments for covariance-compensated block scores (BA-Att section 3.4,
// Eq. 13-14; Algorithm 1 steps 4-7).
//
// With per-block means Xbar and population variances Var[X] (channel-wise,
// over the block's tokens), the compensated logit
//   l~ = s Qbar.Kbar + beta (1/d) sum_t (Var[Q_t] Kbar_t^2 + Var[K_t] Qbar_t^2
//                                         + Var[Q_t] Var[K_t])
// is exactly the dot product of two 3d-long vectors,
//   u = [s Qbar, (beta/d) Var[Q], (beta/d) Qbar^2]   (query blocks, rows)
//   w = [Kbar, Kbar^2 + Var[K], Var[K]]              (key blocks, transposed)
// so the float64 selection kernels rank blocks by l~ unchanged (head_dim 3d,
// scale 1).
//
// One workgroup per block.  Thread (rg, cg) owns 8 channels (16-byte loads)
// of the rows rg, rg + RG, ...; partial sums meet in LDS and are added in row
// group order.  The variance is the mean of squared deviations from the block
// mean, in a second pass over the block's rows (served by the cache).
#include "common.h"

namespace basa {
namespace {

constexpr int MOM_NT = 256;
constexpr int MOM_MAX_D = 168;  // 3 d <= 512, the selection's largest head_dim
constexpr int MOM_MAX_D_R = 256;  // block radii: one thread per channel for the mean

template <typename T> struct Chunk8;
template <> struct Chunk8<uint16_t> {
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
template <> struct Chunk8<float> {
  static __device__ __forceinline__ void load(const float* p, double* v) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};
template <> struct Chunk8<double> {
  static __device__ __forceinline__ void load(const double* p, double* v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double2 a = *reinterpret_cast<const double2*>(p + 2 * i);
      v[2 * i] = a.x;
      v[2 * i + 1] = a.y;
    }
  }
};

// sum over the block's rows of f(x) for this thread's 8 channels, then the
// per-channel total over row groups into tot[c] (LDS)
template <typename T, typename F>
__device__ __forceinline__ void block_sum(const T* xb, int d, int block, int cg, int rg, int n_cg,
                                          int n_rg, bool active, F f, double* part, double* tot) {
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (active) {
    for (int r = rg; r < block; r += n_rg) {
      double v[8];
      Chunk8<T>::load(xb + (int64_t)r * d + 8 * cg, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += f(v[i], 8 * cg + i);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) part[rg * d + 8 * cg + i] = acc[i];
  }
  __syncthreads();
  if ((int)threadIdx.x < d) {
    double s = 0.0;
    for (int g = 0; g < n_rg; ++g) s += part[g * d + threadIdx.x];
    tot[threadIdx.x] = s;
  }
  __syncthreads();
}

// bf16 blocks whose rows fit MOM_ROWS per thread: the rows are read once into
// registers (16 bytes per row and thread) and both sums run over them, in the
// same order as block_sum, so the moments equal the two-read form bit for bit.
constexpr int MOM_ROWS = 8;

__device__ __forceinline__ void bf16x8_to_f64(uint4 a, double* v) {
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = (double)bf16_bits_to_f32(w[i] & 0xFFFFu);
    v[2 * i + 1] = (double)bf16_bits_to_f32(w[i] >> 16);
  }
}

template <typename F>
__device__ __forceinline__ void cached_sum(const uint4* raw, int n_rows, int d, int cg, int rg,
                                           int n_rg, bool active, F f, double* part, double* tot) {
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (active) {
#pragma unroll
    for (int i = 0; i < MOM_ROWS; ++i) {
      if (i < n_rows) {
        double v[8];
        bf16x8_to_f64(raw[i], v);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += f(v[e], 8 * cg + e);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[rg * d + 8 * cg + e] = acc[e];
  }
  __syncthreads();
  if ((int)threadIdx.x < d) {
    double s = 0.0;
    for (int g = 0; g < n_rg; ++g) s += part[g * d + threadIdx.x];
    tot[threadIdx.x] = s;
  }
  __syncthreads();
}

template <typename T>
__global__ __launch_bounds__(MOM_NT) void moments_kernel(const T* x, int64_t len, int d, int block,
                                                         int key_role, double scale, double beta,
                                                         double* out) {
  __shared__ double part[MOM_NT * 8];
  __shared__ double mean[MOM_MAX_D];
  __shared__ double var[MOM_MAX_D];
  const int64_t nb = len / block;
  const int64_t o = blockIdx.x / nb, g = blockIdx.x % nb;
  const int n_cg = d / 8, n_rg = MOM_NT / n_cg;
  const int cg = threadIdx.x % n_cg, rg = threadIdx.x / n_cg;
  const bool active = rg < n_rg;
  const T* xb = x + (o * len + g * block) * d;
  const int my_rows = active && rg < block ? (block - rg + n_rg - 1) / n_rg : 0;
  const int rows_max = (block + n_rg - 1) / n_rg;  // the same for every thread
  if constexpr (sizeof(T) == 2) {
    if (rows_max <= MOM_ROWS) {
      uint4 raw[MOM_ROWS];
#pragma unroll
      for (int i = 0; i < MOM_ROWS; ++i)
        if (i < my_rows) raw[i] = *reinterpret_cast<const uint4*>(xb + (int64_t)(rg + i * n_rg) * d + 8 * cg);
      cached_sum(raw, my_rows, d, cg, rg, n_rg, active, [](double v, int) { return v; }, part, mean);
      if ((int)threadIdx.x < d) mean[threadIdx.x] = mean[threadIdx.x] / block;
      __syncthreads();
      cached_sum(raw, my_rows, d, cg, rg, n_rg, active,
                 [&](double v, int c) { const double e = v - mean[c]; return e * e; }, part, var);
    }
  }
  if (sizeof(T) != 2 || rows_max > MOM_ROWS) {
    block_sum<T>(xb, d, block, cg, rg, n_cg, n_rg, active, [](double v, int) { return v; }, part, mean);
    if ((int)threadIdx.x < d) mean[threadIdx.x] = mean[threadIdx.x] / block;
    __syncthreads();
    block_sum<T>(xb, d, block, cg, rg, n_cg, n_rg, active,
                 [&](double v, int c) { const double e = v - mean[c]; return e * e; }, part, var);
  }
  const int c = threadIdx.x;
  if (c >= d) return;
  const double m = mean[c], s2 = var[c] / block;
  if (!key_role) {  // u rows [outer][nb][3d]
    double* u = out + (o * nb + g) * 3 * d;
    u[c] = scale * m;
    u[d + c] = beta / d * s2;
    u[2 * d + c] = beta / d * (m * m);
  } else {          // w transposed [outer][3d][nb]
    double* w = out + o * 3 * d * nb + g;
    w[(int64_t)c * nb] = m;
    w[(int64_t)(d + c) * nb] = m * m + s2;
    w[(int64_t)(2 * d + c) * nb] = s2;
  }
}

// BA-Att Eq. 7 per block: R = max_i ||x_i - xbar|| and M = max_i ||x_i||.
// The mean as in moments_kernel; then one thread per token forms its two
// squared norms (channels in order) and the workgroup takes their maxima.
template <typename T>
__global__ __launch_bounds__(MOM_NT) void radius_kernel(const T* x, int64_t len, int d, int block,
                                                        double* out) {
  __shared__ double part[MOM_NT * 8];
  __shared__ double mean[MOM_MAX_D_R];
  __shared__ double r2[MOM_NT], n2[MOM_NT];
  const int64_t nb = len / block;
  const int64_t o = blockIdx.x / nb, g = blockIdx.x % nb;
  const int n_cg = d / 8, n_rg = MOM_NT / n_cg;
  const int cg = threadIdx.x % n_cg, rg = threadIdx.x / n_cg;
  const T* xb = x + (o * len + g * block) * d;
  block_sum<T>(xb, d, block, cg, rg, n_cg, n_rg, rg < n_rg, [](double v, int) { return v; }, part, mean);
  if ((int)threadIdx.x < d) mean[threadIdx.x] = mean[threadIdx.x] / block;
  __syncthreads();
  double a = 0.0, b = 0.0;
  if ((int)threadIdx.x < block) {
    const T* xr = xb + (int64_t)threadIdx.x * d;
    for (int c = 0; c < d; c += 8) {
      double v[8];
      Chunk8<T>::load(xr + c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const double e = v[i] - mean[c + i];
        a += e * e;
        b += v[i] * v[i];
      }
    }
  }
  r2[threadIdx.x] = a;
  n2[threadIdx.x] = b;
  __syncthreads();
  for (int w = MOM_NT / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      r2[threadIdx.x] = fmax(r2[threadIdx.x], r2[threadIdx.x + w]);
      n2[threadIdx.x] = fmax(n2[threadIdx.x], n2[threadIdx.x + w]);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    out[(o * nb + g) * 2] = sqrt(r2[0]);
    out[(o * nb + g) * 2 + 1] = sqrt(n2[0]);
  }
}

}  // namespace

hipError_t launch_radius(const void* x, int x_dtype, int64_t outer, int64_t len, int64_t head_dim,
                         int64_t block, double* out, hipStream_t s) {
  const dim3 grid((unsigned)(outer * (len / block)));
  const int d = (int)head_dim, b = (int)block;
  if (x_dtype == BASA_BF16)
    radius_kernel<uint16_t><<<grid, MOM_NT, 0, s>>>(static_cast<const uint16_t*>(x), len, d, b, out);
  else if (x_dtype == BASA_F32)
    radius_kernel<float><<<grid, MOM_NT, 0, s>>>(static_cast<const float*>(x), len, d, b, out);
  else
    radius_kernel<double><<<grid, MOM_NT, 0, s>>>(static_cast<const double*>(x), len, d, b, out);
  return hipGetLastError();
}

hipError_t launch_moments(const void* x, int x_dtype, int64_t outer, int64_t len, int64_t head_dim,
                          int64_t block, int role, double scale, double beta, double* out,
                          hipStream_t s) {
  const dim3 grid((unsigned)(outer * (len / block)));
  const int d = (int)head_dim, b = (int)block, key = role == BASA_MOMENTS_KEY;
  if (x_dtype == BASA_BF16)
    moments_kernel<uint16_t><<<grid, MOM_NT, 0, s>>>(static_cast<const uint16_t*>(x), len, d, b, key,
                                                     scale, beta, out);
  else if (x_dtype == BASA_F32)
    moments_kernel<float><<<grid, MOM_NT, 0, s>>>(static_cast<const float*>(x), len, d, b, key, scale,
                                                  beta, out);
  else
    moments_kernel<double><<<grid, MOM_NT, 0, s>>>(static_cast<const double*>(x), len, d, b, key,
                                                   scale, beta, out);
  return hipGetLastError();
}

}  // namespace basa
