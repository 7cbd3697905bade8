// Measured machine peaks for the roofline fractions: a bf16 matrix-core loop
// and two streaming kernels (read-only and copy) over HBM.  Not part of the
// attention library; bench.py loads this file's library to report each
// kernel's fraction of a peak measured on the same GPU next to its fraction
// of the datasheet figure.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 8;  // independent accumulators per wave: back-to-back MFMAs never wait

// Each wave runs `iters` rounds of kChains independent 32x32x16 bf16 MFMAs
// (32768 flops each) on operands loaded once from `seed`; two workgroups of
// four waves per CU, the occupancy of the attention kernel.  The accumulators
// are summed into out[] so that nothing is optimised away.
__global__ __launch_bounds__(256, 2) void mfma_loop_kernel(const uint4* __restrict__ seed,
                                                           float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  const uint4 ra = seed[(blockIdx.x * 4 + (threadIdx.x >> 6)) % 64 * 64 + lane];
  const uint4 rb = seed[4096 + lane];
  const bf16x8 a = __builtin_bit_cast(bf16x8, ra);
  const bf16x8 b = __builtin_bit_cast(bf16x8, rb);
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Streaming read: every 16-byte word of src once (grid-stride), summed per
// thread, sixteen nontemporal loads in flight per thread (the fastest of the
// shapes tried on the box: 4 and 8 loads in flight, one contiguous 64 KB chunk
// per workgroup, cached loads, 1024-65536 workgroups).
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src, int64_t n,
                                                   uint32_t* __restrict__ out) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 15 * stride < n; i += 16 * stride) {
    u32x4 v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = __builtin_nontemporal_load(src + i + j * stride);
#pragma unroll
    for (int j = 0; j < 16; ++j) acc += v[j].x ^ v[j].z;
  }
  for (; i < n; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc += v.x ^ v.y ^ v.z ^ v.w;
  }
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// Streaming copy of n 16-byte words.
__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                   int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace

extern "C" {

// flops of one peak_mfma_bf16 call with these sizes
double peak_mfma_flops(int64_t workgroups, int iters) {
  return (double)workgroups * 4.0 * iters * kChains * 32768.0;
}

// seed: device, >= 4096 + 64 uint4 words (66,560 bytes) of bf16 data;
// out: device float [workgroups * 256].  0 on success, -1 on bad sizes.
int peak_mfma_bf16(const void* seed, float* out, int64_t workgroups, int iters, void* stream) {
  if (!seed || !out || workgroups < 1 || workgroups > (1 << 20) || iters < 1) return -1;
  mfma_loop_kernel<<<dim3((unsigned)workgroups), 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint4*>(seed), out, iters);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// src: device, bytes a multiple of 16; out: device uint32 [workgroups * 256].
int peak_hbm_read(const void* src, int64_t bytes, uint32_t* out, int64_t workgroups, void* stream) {
  if (!src || !out || bytes < 16 || bytes % 16 || workgroups < 1 || workgroups > (1 << 20)) return -1;
  read_kernel<<<dim3((unsigned)workgroups), 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const u32x4*>(src), bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// src, dst: device, non-overlapping, bytes a multiple of 16.
int peak_hbm_copy(const void* src, void* dst, int64_t bytes, int64_t workgroups, void* stream) {
  if (!src || !dst || bytes < 16 || bytes % 16 || workgroups < 1 || workgroups > (1 << 20)) return -1;
  copy_kernel<<<dim3((unsigned)workgroups), 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // extern "C"
