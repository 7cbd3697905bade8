// Two-way merge of partial attention results (LoSA post: the prefix result and
// the in-block result are combined by online softmax; the merged LSE is
// max-shifted log-sum-exp of the two, and each O is weighted by
// exp(its LSE - merged LSE)).
//
// Streaming kernel: each thread handles 8 consecutive channels of one row
// (one 16- or 32-byte load per input), so a 256-thread workgroup covers
// 256*8/head_dim rows.  The row's two LSE values are read by every thread of
// the row (they hit in cache); the thread owning channel 0 writes the LSE.
#include "common.h"

namespace basa {
namespace {

// The partials are read once and the result written once: nontemporal
// accesses keep them from displacing other data in the caches.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
template <typename TIN> struct Load8NT;
template <> struct Load8NT<float> {
  static __device__ __forceinline__ void load(const float* p, float* out) {
    const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    const u32x4 b = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + 4));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[i] = __uint_as_float(a[i]);
      out[4 + i] = __uint_as_float(b[i]);
    }
  }
};
template <> struct Load8NT<uint16_t> {
  static __device__ __forceinline__ void load(const uint16_t* p, float* out) {
    const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = bf16_bits_to_f32(a[i] & 0xFFFFu);
      out[2 * i + 1] = bf16_bits_to_f32(a[i] >> 16);
    }
  }
};
template <typename TIN>
__device__ __forceinline__ void load8(const void* p, int64_t i, float* out) {
  Load8NT<TIN>::load(static_cast<const TIN*>(p) + i, out);
}

template <typename TIN, typename TOUT>
__global__ __launch_bounds__(256) void merge_kernel(int64_t rows, int d, const void* o_a,
                                                    const float* lse_a, const void* o_b,
                                                    const float* lse_b, void* o, float* lse) {
  const int cols8 = d >> 3;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / cols8;
  if (row >= rows) return;
  const int c = (int)(gid - row * cols8) * 8;
  const float la = lse_a[row], lb = lse_b[row];
  const float mx = fmaxf(la, lb);
  float wa = 0.f, wb = 0.f, lm = -INFINITY;
  if (mx != -INFINITY) {
    const float ea = __expf(la - mx), eb = __expf(lb - mx);
    const float s = ea + eb;
    lm = mx + __logf(s);
    const float inv = 1.f / s;
    wa = ea * inv;
    wb = eb * inv;
  }
  float xa[8], xb[8];
  load8<TIN>(o_a, row * d + c, xa);
  load8<TIN>(o_b, row * d + c, xb);
  float r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = wa * xa[i] + wb * xb[i];
  if constexpr (sizeof(TOUT) == 2) {
    uint4 pk;
    pk.x = (uint32_t)f32_to_bf16_bits(r[0]) | ((uint32_t)f32_to_bf16_bits(r[1]) << 16);
    pk.y = (uint32_t)f32_to_bf16_bits(r[2]) | ((uint32_t)f32_to_bf16_bits(r[3]) << 16);
    pk.z = (uint32_t)f32_to_bf16_bits(r[4]) | ((uint32_t)f32_to_bf16_bits(r[5]) << 16);
    pk.w = (uint32_t)f32_to_bf16_bits(r[6]) | ((uint32_t)f32_to_bf16_bits(r[7]) << 16);
    __builtin_nontemporal_store(u32x4{pk.x, pk.y, pk.z, pk.w},
                                reinterpret_cast<u32x4*>(static_cast<uint16_t*>(o) + row * d + c));
  } else {
    float* op = static_cast<float*>(o) + row * d + c;
    __builtin_nontemporal_store(u32x4{__float_as_uint(r[0]), __float_as_uint(r[1]), __float_as_uint(r[2]),
                                      __float_as_uint(r[3])}, reinterpret_cast<u32x4*>(op));
    __builtin_nontemporal_store(u32x4{__float_as_uint(r[4]), __float_as_uint(r[5]), __float_as_uint(r[6]),
                                      __float_as_uint(r[7])}, reinterpret_cast<u32x4*>(op + 4));
  }
  if (c == 0) lse[row] = lm;
}

template <typename TIN>
hipError_t launch_in(int64_t rows, int d, const void* o_a, const float* lse_a, const void* o_b,
                     const float* lse_b, void* o, int o_dtype, float* lse, hipStream_t s) {
  const int64_t threads = rows * (d / 8);
  const unsigned grid = (unsigned)((threads + 255) / 256);
  if (o_dtype == BASA_BF16)
    merge_kernel<TIN, uint16_t><<<grid, 256, 0, s>>>(rows, d, o_a, lse_a, o_b, lse_b, o, lse);
  else
    merge_kernel<TIN, float><<<grid, 256, 0, s>>>(rows, d, o_a, lse_a, o_b, lse_b, o, lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(int64_t rows, int64_t head_dim, const void* o_a, const float* lse_a,
                        const void* o_b, const float* lse_b, int in_dtype, void* o, int o_dtype,
                        float* lse, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int d = (int)head_dim;
  if (in_dtype == BASA_BF16)
    return launch_in<uint16_t>(rows, d, o_a, lse_a, o_b, lse_b, o, o_dtype, lse, s);
  return launch_in<float>(rows, d, o_a, lse_a, o_b, lse_b, o, o_dtype, lse, s);
}

}  // namespace basa
