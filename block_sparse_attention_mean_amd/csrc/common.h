// Internal helpers shared by the HIP sources of libbasa.  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/basa.h"

namespace basa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

// float64 -> bf16 with a single round-to-nearest-even step (no double rounding
// through float32).  Values below the bf16 normal range flush to signed zero.
__device__ __forceinline__ uint16_t f64_to_bf16_bits(double x) {
  uint64_t u = __double_as_longlong(x);
  uint64_t sign = u >> 63;
  uint64_t mag = u & 0x7FFFFFFFFFFFFFFFull;
  if (mag >= 0x7FF0000000000000ull) {  // inf or nan
    return (uint16_t)((sign << 15) | (mag > 0x7FF0000000000000ull ? 0x7FC0 : 0x7F80));
  }
  // keep 7 of the 52 fraction bits: drop bits 0..44, ties to an even bit 45
  uint64_t r = mag + 0x00000FFFFFFFFFFFull + ((mag >> 45) & 1ull);
  r &= ~0x00001FFFFFFFFFFFull;
  double rd = __longlong_as_double((long long)r);
  float f = (float)rd;  // exact: at most 8 significant bits, in range or overflowing to inf
  uint32_t fb = __float_as_uint(f);
  if ((fb & 0x7F800000u) == 0) fb = 0;  // flush float32 subnormals
  return (uint16_t)((sign << 15) | (fb >> 16));
}

// Order-preserving map of a double to an unsigned key: a > b <=> key(a) > key(b);
// -0.0 and +0.0 map to the same key.
__device__ __forceinline__ uint64_t ordered_key(double x) {
  uint64_t u = __double_as_longlong(x + 0.0);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

template <typename T> struct Vec8;
template <> struct Vec8<float> {
  static __device__ __forceinline__ void load(const float* p, float* out) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  }
};
template <> struct Vec8<uint16_t> {
  static __device__ __forceinline__ void load(const uint16_t* p, float* out) {
    uint4 a = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
      out[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    }
  }
};

// Launchers (defined in the .hip files).  All return the hipGetLastError() of
// the launch; arguments have been validated by the ABI layer.
hipError_t launch_pool(const void* x, int x_dtype, int64_t outer, int64_t len, int64_t head_dim,
                       int64_t block, double* mean_rows, double* mean_cols, void* mean_copy,
                       int copy_dtype, hipStream_t s);
hipError_t launch_pool_pyramid(const basa_pyramid_tensor* t, int n_t, int x_dtype, int64_t outer,
                               int64_t len, int64_t head_dim, int64_t block, int levels,
                               int copy_dtype, hipStream_t s);
hipError_t launch_select_blocks(const basa_select_desc* d, const double* q, const double* kt,
                                int32_t* idx, hipStream_t s);
int64_t select_workspace_bytes(const basa_select_desc* d);
int64_t pool_select_workspace_bytes(const basa_select_desc* d);
hipError_t launch_select_change(const basa_select_desc* d, const void* q, const void* k,
                                int dtype, int32_t* idx, hipStream_t s);
bool attn_mfma_supported(const basa_attn_desc* d, int q_dtype, int o_dtype);
// order: attn_mfma_workspace_bytes() of device scratch for the tile ranks, or null
int64_t attn_mfma_workspace_bytes(const basa_attn_desc* d);
hipError_t launch_attn_mfma(const basa_attn_desc* d, const void* q, void* o, int o_dtype,
                            float* lse, int32_t* order, hipStream_t s);
int64_t attn_union_workspace_bytes(const basa_attn_desc* d);
bool attn_union_supported(const basa_attn_desc* d, int64_t workspace_bytes);
hipError_t launch_attn_union(const basa_attn_desc* d, const void* q, int q_dtype, void* o,
                             int o_dtype, float* lse, void* workspace, hipStream_t s);
bool attn_row_supported(const basa_attn_desc* d);
hipError_t launch_attn_row(const basa_attn_desc* d, const void* q, int q_dtype, void* o,
                           int o_dtype, float* lse, hipStream_t s);
bool attn_t16_supported(const basa_attn_desc* d, int q_dtype);
hipError_t launch_attn_t16(const basa_attn_desc* d, const void* q, void* o, int o_dtype, float* lse,
                           hipStream_t s);
bool attn_tile_supported(const basa_attn_desc* d);
hipError_t launch_attn_tile(const basa_attn_desc* d, const void* q, int q_dtype, void* o,
                            int o_dtype, float* lse, hipStream_t s);
hipError_t launch_attn_generic(const basa_attn_desc* d, const void* q, int q_dtype, void* o,
                               int o_dtype, float* lse, hipStream_t s);
hipError_t launch_merge(int64_t rows, int64_t head_dim, const void* o_a, const float* lse_a,
                        const void* o_b, const float* lse_b, int in_dtype, void* o, int o_dtype,
                        float* lse, hipStream_t s);
hipError_t launch_moments(const void* x, int x_dtype, int64_t outer, int64_t len, int64_t head_dim,
                          int64_t block, int role, double scale, double beta, double* out,
                          hipStream_t s);
// workspace: block_mass_workspace_bytes() of device scratch (the one-pass kernel), or null
int64_t block_mass_workspace_bytes(int64_t batch, int64_t heads_q, int64_t len_q, int64_t len_k,
                                   int64_t head_dim, int64_t block);
hipError_t launch_block_mass(const void* q, const void* k, int dtype, int64_t batch, int64_t heads_q,
                             int64_t heads_kv, int64_t len_q, int64_t len_k, int64_t head_dim,
                             int64_t block, double scale, double* mass, void* workspace, hipStream_t s);
hipError_t launch_select_ranges(const double* scores, int64_t rows, int64_t n, int64_t split,
                                int k_lo, int k_hi, int32_t* idx, hipStream_t s);
hipError_t launch_radius(const void* x, int x_dtype, int64_t outer, int64_t len, int64_t head_dim,
                         int64_t block, double* out, hipStream_t s);
int64_t rank_workspace_bytes(int64_t outer, int64_t len);
hipError_t launch_rank(const void* x, int x_dtype, int64_t outer, int64_t len, int64_t head_dim,
                       int32_t* perm, void* workspace, int64_t workspace_bytes, hipStream_t s);
hipError_t launch_permute(const void* x, int64_t outer, int64_t len, int64_t row_bytes,
                          const int32_t* perm, int mode, void* out, hipStream_t s);

}  // namespace basa
