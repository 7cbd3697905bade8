// Attention over listed key blocks, general form: float32 or bf16 queries and
// key/value tables, head_dim 64 or 128, any tile and block size, up to four
// key segments (each with its own table, index rows and logit bias), a query
// row map and grouped key heads.
//
// BA-Att section 2: each query block attends only to the key/value blocks its
// mask keeps; Eq. 1's softmax runs over those keys only.  The online softmax
// keeps a running max m, a running sum l and an unnormalised output per row;
// a new chunk of logits with max m' rescales them by exp(m - m').
//
// One workgroup computes one query row.  Its four waves take four contiguous
// shares of every segment's entries; within a share, keys go 64 at a time,
// lane j taking key j: the lane forms its logit from the query row (broadcast
// from LDS) and its key row, then the wave updates the row state, each lane
// owning head_dim/64 output channels.  At the end the four partial states are
// merged through LDS with the max-shifted rule of basa_merge.
//
// This is the general path; bf16 / head_dim 128 / 128-row tiles / 128-key
// blocks with one segment run on the MFMA kernel instead.
#include "common.h"

namespace basa {
namespace {

struct Seg {
  const int32_t* idx;
  const void* k;
  const void* v;
  int64_t len, rows;
  int count, stride, shift, bf16;
  float bias_log2;
};

struct GenArgs {
  Seg seg[BASA_MAX_SEGMENTS];
  int n_seg;
  const void* q;
  void* o;
  float* lse;
  const int32_t* q_rows;
  int64_t len_q, lists, rows_total;
  int heads_q, heads_kv, group, tile_q, block_k;
  float scale_log2;
};

__device__ __forceinline__ float ld1(const void* base, int64_t i, bool bf16) {
  return bf16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(base)[i])
              : static_cast<const float*>(base)[i];
}

template <int D>
__device__ __forceinline__ float dot_row(const float* qs, const void* kt, int64_t row, bool bf16) {
  float dot = 0.f;
  if (bf16) {
    const uint16_t* kp = static_cast<const uint16_t*>(kt) + row * D;
#pragma unroll
    for (int c = 0; c < D; c += 8) {
      float kv8[8];
      Vec8<uint16_t>::load(kp + c, kv8);
#pragma unroll
      for (int i = 0; i < 8; ++i) dot = __builtin_fmaf(qs[c + i], kv8[i], dot);
    }
  } else {
    const float* kp = static_cast<const float*>(kt) + row * D;
#pragma unroll
    for (int c = 0; c < D; c += 8) {
      float kv8[8];
      Vec8<float>::load(kp + c, kv8);
#pragma unroll
      for (int i = 0; i < 8; ++i) dot = __builtin_fmaf(qs[c + i], kv8[i], dot);
    }
  }
  return dot;
}

template <bool Q_BF16, bool O_BF16, int D>
__global__ __launch_bounds__(256) void attn_generic_kernel(GenArgs a) {
  constexpr int CPL = D / 64;  // output channels per lane
  __shared__ float qs[D];
  __shared__ float p_s[4][64];
  __shared__ int64_t krow_s[4][64];
  __shared__ float part_m[4], part_l[4];
  __shared__ float part_o[4][D];

  const int64_t unit = (int64_t)blockIdx.x + (int64_t)blockIdx.y * gridDim.x;
  if (unit >= a.rows_total) return;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = (int)(unit % a.tile_q);
  const int64_t rest = unit / a.tile_q;
  const int64_t t = rest % a.lists;
  const int64_t bh = rest / a.lists;
  const int h = (int)(bh % a.heads_q);
  const int64_t b = bh / a.heads_q;
  const int hk = h / a.group;
  int64_t row = t * a.tile_q + r;
  if (a.q_rows) row = a.q_rows[b * a.lists * a.tile_q + t * a.tile_q + r];
  if (row < 0 || row >= a.len_q) return;  // a row map entry outside q: nothing to write
  const int64_t qoff = ((b * a.heads_q + h) * a.len_q + row) * D;

  for (int c = threadIdx.x; c < D; c += 256) qs[c] = ld1(a.q, qoff + c, Q_BF16);
  __syncthreads();

  float m = -INFINITY;  // running max, log2 units
  float l = 0.f;        // this lane's share of the running sum
  float acc[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) acc[i] = 0.f;

  for (int si = 0; si < a.n_seg; ++si) {
    const Seg sg = a.seg[si];
    const bool kbf = sg.bf16 != 0;
    const int32_t* lst = sg.idx + ((b * a.heads_q + h) * sg.rows + (t >> sg.shift)) * sg.stride;
    const int64_t head_row = (b * a.heads_kv + hk) * sg.len;
    const int e0 = (int)(((int64_t)sg.count * wave) / 4);
    const int e1 = (int)(((int64_t)sg.count * (wave + 1)) / 4);
    const int64_t n_keys = (int64_t)(e1 - e0) * a.block_k;
    for (int64_t k0 = 0; k0 < n_keys; k0 += 64) {
      const int64_t f = k0 + lane;
      float z = -INFINITY;
      int64_t krow = -1;
      if (f < n_keys) {
        const int ent = e0 + (int)(f / a.block_k);
        const int off = (int)(f % a.block_k);
        const int32_t blk = lst[ent];
        const int64_t key = (int64_t)blk * a.block_k + off;
        if (blk >= 0 && key < sg.len) {
          krow = head_row + key;
          z = dot_row<D>(qs, sg.k, krow, kbf) * a.scale_log2 + sg.bias_log2;
        }
      }
      float cm = z;
#pragma unroll
      for (int sh = 32; sh >= 1; sh >>= 1) cm = fmaxf(cm, __shfl_xor(cm, sh));
      const float m_new = fmaxf(m, cm);
      if (m_new == -INFINITY) continue;  // nothing valid yet (wave-uniform)
      const float alpha = exp2f(m - m_new);
      const float p = (z == -INFINITY) ? 0.f : exp2f(z - m_new);
      l = l * alpha + p;
      m = m_new;
#pragma unroll
      for (int i = 0; i < CPL; ++i) acc[i] *= alpha;
      // empty slots carry p = 0 and a valid row of this head (some key of the chunk is valid)
      p_s[wave][lane] = p;
      krow_s[wave][lane] = krow >= 0 ? krow : head_row;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // fixed trip count and no data-dependent exits, so the V loads of several keys are in flight
#pragma unroll 8
      for (int j = 0; j < 64; ++j) {
        const float pj = p_s[wave][j];
        const int64_t kr = krow_s[wave][j];
#pragma unroll
        for (int i = 0; i < CPL; ++i)
          acc[i] = __builtin_fmaf(pj, ld1(sg.v, kr * D + lane + 64 * i, kbf), acc[i]);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) l += __shfl_xor(l, sh);
  if (lane == 0) {
    part_m[wave] = m;
    part_l[wave] = l;
  }
#pragma unroll
  for (int i = 0; i < CPL; ++i) part_o[wave][lane + 64 * i] = acc[i];
  __syncthreads();

  float mm = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) mm = fmaxf(mm, part_m[w]);
  float wsc[4];
  float ltot = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    wsc[w] = (part_m[w] == -INFINITY) ? 0.f : exp2f(part_m[w] - mm);
    ltot += part_l[w] * wsc[w];
  }
  const int64_t ooff = (b * a.heads_q + h) * a.len_q + row;
  for (int c = threadIdx.x; c < D; c += 256) {
    float val = 0.f;
    if (ltot > 0.f) {
#pragma unroll
      for (int w = 0; w < 4; ++w) val += part_o[w][c] * wsc[w];
      val /= ltot;
    }
    if constexpr (O_BF16)
      static_cast<uint16_t*>(a.o)[ooff * D + c] = f32_to_bf16_bits(val);
    else
      static_cast<float*>(a.o)[ooff * D + c] = val;
  }
  if (threadIdx.x == 0) a.lse[ooff] = (ltot > 0.f) ? (mm + log2f(ltot)) * kLn2 : -INFINITY;
}

template <bool QB, bool OB>
hipError_t launch_d(const GenArgs& a, int d, dim3 grid, hipStream_t s) {
  if (d == 64)
    attn_generic_kernel<QB, OB, 64><<<grid, 256, 0, s>>>(a);
  else
    attn_generic_kernel<QB, OB, 128><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_generic(const basa_attn_desc* d, const void* q, int q_dtype, void* o,
                               int o_dtype, float* lse, hipStream_t s) {
  GenArgs a = {};
  a.n_seg = d->n_segments;
  for (int i = 0; i < d->n_segments; ++i) {
    const basa_kv_segment& g = d->seg[i];
    a.seg[i].idx = g.idx;
    a.seg[i].k = g.k;
    a.seg[i].v = g.v;
    a.seg[i].len = g.len;
    a.seg[i].rows = g.rows;
    a.seg[i].count = g.count;
    a.seg[i].stride = g.stride;
    a.seg[i].shift = g.shift;
    a.seg[i].bf16 = g.dtype == BASA_BF16;
    a.seg[i].bias_log2 = g.bias * kLog2e;
  }
  a.q = q;
  a.o = o;
  a.lse = lse;
  a.q_rows = d->q_rows;
  a.len_q = d->len_q;
  a.lists = d->lists;
  a.heads_q = (int)d->heads_q;
  a.heads_kv = (int)d->heads_kv;
  a.group = (int)(d->heads_q / d->heads_kv);
  a.tile_q = d->tile_q;
  a.block_k = d->block_k;
  a.scale_log2 = (float)(d->scale * 1.4426950408889634);
  a.rows_total = d->batch * d->heads_q * d->lists * d->tile_q;
  if (a.rows_total == 0) return hipSuccess;
  const int64_t gx = a.rows_total < 65536 ? a.rows_total : 65536;
  const int64_t gy = (a.rows_total + gx - 1) / gx;
  dim3 grid((unsigned)gx, (unsigned)gy);
  const int dd = (int)d->head_dim;
  const bool qb = q_dtype == BASA_BF16, ob = o_dtype == BASA_BF16;
  if (qb) return ob ? launch_d<true, true>(a, dd, grid, s) : launch_d<true, false>(a, dd, grid, s);
  return ob ? launch_d<false, true>(a, dd, grid, s) : launch_d<false, false>(a, dd, grid, s);
}

}  // namespace basa
