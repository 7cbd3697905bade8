// Block-sparse flash attention on bf16 MFMA for gfx950: head_dim 128, query
// tiles of 128 rows (one query block), key blocks of 128 keys.
//
// BA-Att section 2 / section 3.1: attention is computed only for the kept
// (query block, key block) pairs; within them it is the softmax attention of
// Eq. 1, bidirectional.  The online softmax carries (m, l, O) per row across
// the kept blocks, and the kernel emits O and the natural-log LSE.
//
// Work decomposition
//   One workgroup (4 waves) computes one query tile of 128 rows; wave w owns
//   rows 32w .. 32w+31.  Kept key blocks are streamed in stages of 64 keys
//   (two stages per block).  Two workgroups share a CU (72 KB of LDS each),
//   and as they synchronise only internally, one workgroup's softmax runs
//   while the other's MFMAs do.
//   Per stage a wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16
//   (A = K rows from LDS, B = the wave's Q rows, held in registers for the
//   whole walk), so each lane holds 32 logits of ONE query row: the row max and
//   row sum need one cross-lane step (lane l and l^32).  Then O^T += V^T P^T
//   with the same instruction (A = V^T from LDS, B = P taken straight from the
//   S accumulators after a bf16 conversion).
//
// Key permutation.  The 32x32 accumulator puts row rho of S^T in register
// r = 4*(rho/8) + rho%4 of lane-half (rho/4)%2.  Loading key kappa into MFMA
// row rho = kappa with bits 2 and 3 swapped makes registers 8c..8c+7 of lane
// half h hold keys 16c + 8h .. 16c + 8h + 7, which is exactly the B-operand
// layout of a 16-key P chunk; the V^T operand reads the same keys.
//
// Data movement (double-buffered, one barrier per stage)
//   K and V of the next stage are loaded into registers at the top of a stage
//   and written to the other LDS buffer after the current stage's softmax, so
//   the loads overlap the current stage's MFMA and softmax work.  (Direct
//   global->LDS loads were tried: the compiler cannot prove that the DMA into
//   one buffer does not alias reads of the other, and waits for the loads
//   before every LDS read.)  K rows are 256 bytes whose 16-byte chunks are
//   XOR-swizzled by the row number, so the 16 lanes reading one MFMA operand
//   hit distinct banks; V is stored transposed, channel-major, in rows padded
//   to 144 bytes (again conflict-free for the operand reads).
//
// Softmax: log2 domain with the scale folded in; the running max is only
// raised when a stage's max exceeds it by more than 8 (a factor 256), so the
// O rescale is usually skipped; O/l and LSE = m + log2(l) do not depend on the
// choice of m.
//
// Workgroup numbering: dispatch hands workgroups to the 8 XCDs round-robin.
// Tiles are numbered so that in every round of 8 x 64 resident workgroups all
// XCDs work on one contiguous run of tiles (the same head), each XCD on its
// own contiguous sub-run: the head's K/V stays in the shared last-level cache
// and neighbouring query tiles, whose kept blocks overlap, share an L2.
#include "common.h"

namespace basa {
namespace {

constexpr int D = 128;
constexpr int BQ = 128;
constexpr int BK = 128;
constexpr int SK = 64;                        // keys per stage
constexpr int NT = 256;                       // threads per workgroup (4 waves)
constexpr int KBUF = SK * D * 2;              // 16 KB, swizzled rows of 256 B
constexpr int VSTR = SK * 2 + 16;             // bytes per V^T row (one channel)
constexpr int VBUF = D * VSTR;                // 18 KB
constexpr int MAX_KEPT = 1024;                // list slots staged in LDS (the last holds the count)
constexpr int LDS_BYTES = 2 * KBUF + 2 * VBUF + MAX_KEPT * 4;
constexpr int RESIDENT_PER_XCD = 64;          // two workgroups per CU, 32 CUs per XCD
constexpr float kLazy = 8.0f;                 // log2 of the allowed growth before a rescale

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

__device__ __forceinline__ int64_t tile_of(int64_t w, int64_t tiles) {
  const int64_t round_sz = 8 * RESIDENT_PER_XCD;
  const int64_t full = (tiles / round_sz) * round_sz;
  if (w >= full) return w;
  const int64_t xcd = w % 8, k = w / 8;
  const int64_t r = k / RESIDENT_PER_XCD, s = k % RESIDENT_PER_XCD;
  return r * round_sz + xcd * RESIDENT_PER_XCD + s;
}

struct Stage {
  uint4 k0, k1, k2, k3;  // K: 16-byte chunks tid + 256 i of the 64 x 256-byte stage
  uint4 v0, v1, v2, v3;  // V: keys 4*(tid%16) .. +3, channels 8*(tid/16) .. +7
};

__device__ __forceinline__ Stage load_stage(const uint16_t* kg, const uint16_t* vg, int tid) {
  Stage s;
  const uint16_t* kp = kg + (tid >> 4) * D + (tid & 15) * 8;
  s.k0 = *reinterpret_cast<const uint4*>(kp);
  s.k1 = *reinterpret_cast<const uint4*>(kp + 16 * D);
  s.k2 = *reinterpret_cast<const uint4*>(kp + 32 * D);
  s.k3 = *reinterpret_cast<const uint4*>(kp + 48 * D);
  const uint16_t* vp = vg + (4 * (tid & 15)) * D + (tid >> 4) * 8;
  s.v0 = *reinterpret_cast<const uint4*>(vp);
  s.v1 = *reinterpret_cast<const uint4*>(vp + D);
  s.v2 = *reinterpret_cast<const uint4*>(vp + 2 * D);
  s.v3 = *reinterpret_cast<const uint4*>(vp + 3 * D);
  return s;
}

__device__ __forceinline__ void store_stage(uint8_t* kbuf, uint8_t* vbuf, const Stage& s, int tid) {
  // K: logical chunk c of row r sits at physical chunk c ^ (r & 15); rows r + 16 i share r & 15
  const int r = tid >> 4, c = tid & 15;
  const int off = r * 256 + ((c ^ (r & 15)) * 16);
  *reinterpret_cast<uint4*>(kbuf + off) = s.k0;
  *reinterpret_cast<uint4*>(kbuf + off + 16 * 256) = s.k1;
  *reinterpret_cast<uint4*>(kbuf + off + 32 * 256) = s.k2;
  *reinterpret_cast<uint4*>(kbuf + off + 48 * 256) = s.k3;
  // V^T: channel 8*dg + 2j from the low halves, 8*dg + 2j + 1 from the high halves.
  // v_perm_b32 selects bytes of {a:b}: 0x05040100 = low halves (b, a), 0x07060302 = high halves.
  const int kgrp = tid & 15, dg = tid >> 4;
  const uint32_t w0[4] = {s.v0.x, s.v0.y, s.v0.z, s.v0.w};
  const uint32_t w1[4] = {s.v1.x, s.v1.y, s.v1.z, s.v1.w};
  const uint32_t w2[4] = {s.v2.x, s.v2.y, s.v2.z, s.v2.w};
  const uint32_t w3[4] = {s.v3.x, s.v3.y, s.v3.z, s.v3.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint2 lo, hv;
    lo.x = __builtin_amdgcn_perm(w1[j], w0[j], 0x05040100u);
    lo.y = __builtin_amdgcn_perm(w3[j], w2[j], 0x05040100u);
    hv.x = __builtin_amdgcn_perm(w1[j], w0[j], 0x07060302u);
    hv.y = __builtin_amdgcn_perm(w3[j], w2[j], 0x07060302u);
    *reinterpret_cast<uint2*>(vbuf + (8 * dg + 2 * j) * VSTR + 8 * kgrp) = lo;
    *reinterpret_cast<uint2*>(vbuf + (8 * dg + 2 * j + 1) * VSTR + 8 * kgrp) = hv;
  }
}

template <bool OUT_BF16>
__global__ __launch_bounds__(NT, 2) void attn_mfma_kernel(MfmaArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // K buffer i at smem + i*KBUF, V^T buffer i at smem + 2*KBUF + i*VBUF, list after them
  int32_t* lst = reinterpret_cast<int32_t*>(smem + 2 * KBUF + 2 * VBUF);

  const int64_t tile = tile_of(blockIdx.x, a.tiles);
  const int64_t t = tile % a.lists;
  const int64_t bh = tile / a.lists;
  const int h = (int)(bh % a.heads_q);
  const int64_t b = bh / a.heads_q;
  const int hk = h / a.group;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31;
  const int hi = lane >> 5;

  const int64_t qrow = t * BQ + wave * 32 + li;
  const uint16_t* qp = a.q + ((b * a.heads_q + h) * a.len_q + qrow) * D;
  bf16x8 qf[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) qf[c] = *reinterpret_cast<const bf16x8*>(qp + 16 * c + 8 * hi);

  // compact the tile's list into LDS (valid blocks only, order kept): wave 0, 64 entries a step
  const int nblk_k = (int)(a.len_k / BK);
  if (wave == 0) {
    const int32_t* g = a.kv_idx + ((b * a.heads_q + h) * a.idx_rows + t) * a.idx_stride;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int n = 0;
    for (int base = 0; base < a.kept; base += 64) {
      const int e = base + lane;
      const int32_t blk = e < a.kept ? g[e] : -1;
      const bool ok = blk >= 0 && blk < nblk_k;
      const uint64_t m = __ballot(ok);
      if (ok) lst[n + __popcll(m & below)] = blk;
      n += __popcll(m);
    }
    if (lane == 0) lst[MAX_KEPT - 1] = n;  // kept < MAX_KEPT, so the count slot is never an entry
  }
  // settle the Q loads with a compiler-visible vmcnt(0): otherwise the wait-count
  // bookkeeping at the loop head cannot tell them from the in-loop prefetches
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  const int n_valid = lst[MAX_KEPT - 1];
  const int n_stage = 2 * n_valid;

  f32x16 oacc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[u][r] = 0.f;
  float m = -INFINITY;  // running row max of scale*log2(e)*logit (lazily raised)
  float l = 0.f;        // this lane's share of the running row sum

  const uint16_t* kbase = a.k + (b * a.heads_kv + hk) * a.len_k * D;
  const uint16_t* vbase = a.v + (b * a.heads_kv + hk) * a.len_k * D;
  const int krow_l = swap_bits_2_3(li);

  if (n_stage > 0) {
    const int64_t off = (int64_t)lst[0] * BK * D;
    const Stage s0 = load_stage(kbase + off, vbase + off, tid);
    store_stage(smem, smem + 2 * KBUF, s0, tid);
  }
  __syncthreads();

  for (int st_i = 0; st_i < n_stage; ++st_i) {
    const int buf = st_i & 1;
    const bool has_next = st_i + 1 < n_stage;
    Stage nx;
    if (has_next) {
      const int sn = st_i + 1;
      const int64_t off = (int64_t)lst[sn >> 1] * BK * D + (int64_t)(sn & 1) * SK * D;
      nx = load_stage(kbase + off, vbase + off, tid);
    }

    // S^T = K Q^T for the stage's two 32-key sub-tiles
    const uint8_t* kcur = smem + buf * KBUF;
    f32x16 s[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[st][r] = 0.f;
      const int krow = 32 * st + krow_l;
      const uint8_t* rowp = kcur + krow * 256;
      bf16x8 af[8];
#pragma unroll
      for (int c = 0; c < 8; ++c)
        af[c] = *reinterpret_cast<const bf16x8*>(rowp + (((2 * c + hi) ^ (krow & 15)) * 16));
      __builtin_amdgcn_sched_barrier(0);  // all 8 operand reads in flight before the chain
#pragma unroll
      for (int c = 0; c < 8; ++c)
        s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[c], qf[c], s[st], 0, 0, 0);
    }

    // online softmax in the log2 domain; lanes l and l^32 hold the same row
    float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[st][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * a.scale_log2;
    if (__ballot(mx > m + kLazy) != 0) {  // some row outgrew its max: rescale (wave-uniform)
      const float m_new = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
      l *= alpha;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[u][r] *= alpha;
      m = m_new;
    }
    float psum = 0.f;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][r], a.scale_log2, -m));
        s[st][r] = p;
        psum += p;
      }
    l += psum;

    if (has_next)  // the other buffers were last read before the previous barrier
      store_stage(smem + (buf ^ 1) * KBUF, smem + 2 * KBUF + (buf ^ 1) * VBUF, nx, tid);

    // O^T += V^T P^T over the stage's 64 keys, 16 at a time
    const uint8_t* vcur = smem + 2 * KBUF + buf * VBUF;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        bf16x8 pf;
#pragma unroll
        for (int j = 0; j < 8; ++j) pf[j] = (__bf16)s[st][8 * cc + j];
        const int key0 = 32 * st + 16 * cc + 8 * hi;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vcur + (32 * u + li) * VSTR + 2 * key0);
          oacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, oacc[u], 0, 0, 0);
        }
      }
    }
    __syncthreads();  // the current buffers are free; the next ones are complete
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
  // the list is compacted into the first MAX_KEPT-1 LDS slots; the last holds the count
  return q_dtype == BASA_BF16 && d->n_segments == 1 && g.dtype == BASA_BF16 && g.shift == 0 &&
         g.bias == 0.f && d->head_dim == D && d->tile_q == BQ && d->block_k == BK &&
         d->q_rows == nullptr && d->lists * BQ == d->len_q && d->scale > 0.0 &&
         g.count < MAX_KEPT && (o_dtype == BASA_BF16 || o_dtype == BASA_F32);
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
  const void* fn = o_dtype == BASA_BF16 ? (const void*)attn_mfma_kernel<true>
                                        : (const void*)attn_mfma_kernel<false>;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)a.tiles);
  if (o_dtype == BASA_BF16)
    attn_mfma_kernel<true><<<grid, NT, LDS_BYTES, s>>>(a);
  else
    attn_mfma_kernel<false><<<grid, NT, LDS_BYTES, s>>>(a);
  return hipGetLastError();
}

}  // namespace basa
