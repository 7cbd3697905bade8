// Block-sparse flash attention on bf16 MFMA for gfx950: head_dim 128, query
// tiles of 128 rows (one query block), key blocks of 128 keys.
//
// BA-Att section 2 / section 3.1: attention is computed only for the kept
// (query block, key block) pairs; within them it is the softmax attention of
// Eq. 1, bidirectional.  The online softmax carries (m, l, O) per row across
// the kept blocks, and the kernel emits O and the natural-log LSE.
//
// Work decomposition
//   one workgroup = one query tile (b, h, 128 rows), 4 waves x 32 rows.
//   For each kept key block: K (128 x 128) and V (transposed, 128 x 128) are
//   staged in LDS; every wave computes S^T = K Q^T for its 32 rows with
//   v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = the wave's Q rows held
//   in registers for the whole walk), so each lane holds 64 logits of ONE
//   query row: the row max and row sum need only one cross-lane step (lane
//   l and l^32).  Then O^T += V^T P^T with the same instruction (A = V^T from
//   LDS, B = P straight from the S accumulators after a bf16 conversion).
//
// Key permutation.  The 32x32 accumulator puts row rho of S^T at register
// r = 4*(rho/8) + rho%4 of lane-half (rho/4)%2.  Loading key kappa into MFMA
// row rho = kappa with bits 2 and 3 swapped makes registers 8c..8c+7 of lane
// half h hold keys 16c + 8h .. 16c + 8h + 7, which is exactly the B-operand
// layout of a 16-key P chunk.  The V^T operand reads the same keys, so the
// contraction pairs each P value with its own V row.
//
// LDS rows are padded to 272 bytes so that the 16-byte reads of 16 lanes fall
// in distinct banks.  Two workgroups fit per CU (2 x 68 KB of 160 KB), which
// gives each SIMD two waves to overlap one wave's softmax with the other's MFMA.
//
// Workgroups are numbered so that each XCD (dispatch round-robins workgroups
// over the 8 XCDs) receives a contiguous run of tiles: neighbouring query
// tiles of the same head, whose kept key blocks overlap, share that XCD's L2.
#include "common.h"

namespace basa {
namespace {

constexpr int D = 128;
constexpr int BQ = 128;
constexpr int BK = 128;
constexpr int KSTR = D * 2 + 16;   // bytes per K row in LDS
constexpr int VSTR = BK * 2 + 16;  // bytes per V^T row (one channel) in LDS
constexpr int LDS_BYTES = BK * KSTR + D * VSTR;

struct MfmaArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* o;
  float* lse;
  const int32_t* kv_idx;
  int64_t len_q, len_k, lists, tiles, idx_rows;
  int heads_q, heads_kv, group, kept, idx_stride;
  float scale_log2;
};

__device__ __forceinline__ int swap_bits_2_3(int x) {
  return (x & ~0xC) | ((x >> 1) & 0x4) | ((x << 1) & 0x8);
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256, 2) void attn_mfma_kernel(MfmaArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];
  uint8_t* ks = smem;
  uint8_t* vts = smem + BK * KSTR;

  // XCD-aware tile numbering (bijective: the tail beyond a multiple of 8 keeps its id)
  const int64_t w = blockIdx.x;
  const int64_t full = (a.tiles / 8) * 8;
  const int64_t tile = (w < full) ? (w % 8) * (a.tiles / 8) + w / 8 : w;
  const int64_t t = tile % a.lists;
  const int64_t bh = tile / a.lists;
  const int h = (int)(bh % a.heads_q);
  const int64_t b = bh / a.heads_q;
  const int hk = h / a.group;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 31;
  const int hi = lane >> 5;

  // this lane's query row and its 128 channels as 8 B-operand fragments
  const int64_t qrow = t * BQ + wave * 32 + li;
  const uint16_t* qp = a.q + ((b * a.heads_q + h) * a.len_q + qrow) * D;
  bf16x8 qf[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) qf[c] = *reinterpret_cast<const bf16x8*>(qp + 16 * c + 8 * hi);

  f32x16 oacc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[u][r] = 0.f;
  float m = -INFINITY;  // running row max of scale*log2(e)*logit
  float l = 0.f;        // this lane's half of the running row sum

  const int32_t* lst = a.kv_idx + ((b * a.heads_q + h) * a.idx_rows + t) * a.idx_stride;
  const uint16_t* kbase = a.k + (b * a.heads_kv + hk) * a.len_k * D;
  const uint16_t* vbase = a.v + (b * a.heads_kv + hk) * a.len_k * D;
  const int krow_lds = swap_bits_2_3(li);

  for (int e = 0; e < a.kept; ++e) {
    const int blk = lst[e];
    if (blk < 0 || (int64_t)blk * BK + BK > a.len_k) continue;  // empty slot (or out of range)
    const uint16_t* kg = kbase + (int64_t)blk * BK * D;
    const uint16_t* vg = vbase + (int64_t)blk * BK * D;

    // global -> registers (K: 8 x 16 B per thread; V: 2 x 4 rows x 16 B per thread)
    uint4 kr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int ch = tid + 256 * i;
      kr[i] = *reinterpret_cast<const uint4*>(kg + (ch >> 4) * D + (ch & 15) * 8);
    }
    const int kgrp = tid & 31;
    uint4 vr[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int dg = (tid >> 5) + 8 * i;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        vr[i][r] = *reinterpret_cast<const uint4*>(vg + (4 * kgrp + r) * D + dg * 8);
    }
    __syncthreads();  // previous block's LDS reads are done
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int ch = tid + 256 * i;
      *reinterpret_cast<uint4*>(ks + (ch >> 4) * KSTR + (ch & 15) * 16) = kr[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int dg = (tid >> 5) + 8 * i;
      const uint32_t w0[4] = {vr[i][0].x, vr[i][0].y, vr[i][0].z, vr[i][0].w};
      const uint32_t w1[4] = {vr[i][1].x, vr[i][1].y, vr[i][1].z, vr[i][1].w};
      const uint32_t w2[4] = {vr[i][2].x, vr[i][2].y, vr[i][2].z, vr[i][2].w};
      const uint32_t w3[4] = {vr[i][3].x, vr[i][3].y, vr[i][3].z, vr[i][3].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // channel 8*dg + 2j (low halves) and 8*dg + 2j + 1 (high halves)
        uint2 lo, hv;
        lo.x = (w0[j] & 0xFFFFu) | (w1[j] << 16);
        lo.y = (w2[j] & 0xFFFFu) | (w3[j] << 16);
        hv.x = (w0[j] >> 16) | (w1[j] & 0xFFFF0000u);
        hv.y = (w2[j] >> 16) | (w3[j] & 0xFFFF0000u);
        *reinterpret_cast<uint2*>(vts + (8 * dg + 2 * j) * VSTR + 8 * kgrp) = lo;
        *reinterpret_cast<uint2*>(vts + (8 * dg + 2 * j + 1) * VSTR + 8 * kgrp) = hv;
      }
    }
    __syncthreads();

    // S^T = K Q^T for 4 sub-tiles of 32 keys
    f32x16 s[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[st][r] = 0.f;
      const uint8_t* krow = ks + (32 * st + krow_lds) * KSTR + 16 * hi;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const bf16x8 af = *reinterpret_cast<const bf16x8*>(krow + 32 * c);
        s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[c], s[st], 0, 0, 0);
      }
    }

    // online softmax (log2 domain); lane halves l and l^32 share a row
    float mx = s[0][0];
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[st][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx * a.scale_log2);
    const float alpha = exp2f(m - m_new);
    float psum = 0.f;
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f(__builtin_fmaf(s[st][r], a.scale_log2, -m_new));
        s[st][r] = p;
        psum += p;
      }
    l = l * alpha + psum;
    m = m_new;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[u][r] *= alpha;

    // O^T += V^T P^T, 16 keys per step
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        bf16x8 pf;
#pragma unroll
        for (int j = 0; j < 8; ++j) pf[j] = (__bf16)s[st][8 * cc + j];
        const int key0 = 32 * st + 16 * cc + 8 * hi;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vts + (32 * u + li) * VSTR + 2 * key0);
          oacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, oacc[u], 0, 0, 0);
        }
      }
    }
  }

  // epilogue: O = O^T / l, LSE = (m + log2 l) ln 2
  const float l_tot = l + __shfl_xor(l, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int64_t orow = (b * a.heads_q + h) * a.len_q + qrow;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int ch = 32 * u + 8 * rq + 4 * hi;
      const float v0 = oacc[u][4 * rq + 0] * inv, v1 = oacc[u][4 * rq + 1] * inv;
      const float v2 = oacc[u][4 * rq + 2] * inv, v3 = oacc[u][4 * rq + 3] * inv;
      if constexpr (OUT_BF16) {
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16_bits(v0) | ((uint32_t)f32_to_bf16_bits(v1) << 16);
        pk.y = (uint32_t)f32_to_bf16_bits(v2) | ((uint32_t)f32_to_bf16_bits(v3) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.o) + orow * D + ch) = pk;
      } else {
        *reinterpret_cast<float4*>(static_cast<float*>(a.o) + orow * D + ch) = make_float4(v0, v1, v2, v3);
      }
    }
  }
  if (hi == 0) a.lse[orow] = l_tot > 0.f ? (m + log2f(l_tot)) * kLn2 : -INFINITY;
}

}  // namespace

bool attn_mfma_supported(const basa_attn_desc* d, int q_dtype, int o_dtype) {
  const basa_kv_segment& g = d->seg[0];
  return q_dtype == BASA_BF16 && d->n_segments == 1 && g.dtype == BASA_BF16 && g.shift == 0 &&
         g.bias == 0.f && d->head_dim == D && d->tile_q == BQ && d->block_k == BK &&
         d->q_rows == nullptr && d->lists * BQ == d->len_q && d->scale > 0.0 &&
         (o_dtype == BASA_BF16 || o_dtype == BASA_F32);
}

hipError_t launch_attn_mfma(const basa_attn_desc* d, const void* q, void* o, int o_dtype,
                            float* lse, hipStream_t s) {
  const basa_kv_segment& g = d->seg[0];
  MfmaArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(g.k);
  a.v = static_cast<const uint16_t*>(g.v);
  a.o = o;
  a.lse = lse;
  a.kv_idx = g.idx;
  a.len_q = d->len_q;
  a.len_k = g.len;
  a.lists = d->lists;
  a.idx_rows = g.rows;
  a.idx_stride = g.stride;
  a.tiles = d->batch * d->heads_q * d->lists;
  a.heads_q = (int)d->heads_q;
  a.heads_kv = (int)d->heads_kv;
  a.group = (int)(d->heads_q / d->heads_kv);
  a.kept = g.count;
  a.scale_log2 = (float)(d->scale * 1.4426950408889634);
  if (a.tiles == 0) return hipSuccess;
  dim3 grid((unsigned)a.tiles);
  if (o_dtype == BASA_BF16)
    attn_mfma_kernel<true><<<grid, 256, 0, s>>>(a);
  else
    attn_mfma_kernel<false><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace basa
