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
//   (two stages per block).  Two workgroups share a CU (68 KB of LDS each).
//   Per stage a wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16
//   (A = K rows from LDS, B = the wave's Q rows, held in registers for the
//   whole walk), so each lane holds 32 logits of ONE query row: the row max
//   needs one cross-lane step (lane l and l^32, v_permlane32_swap).  Then
//   O^T += V^T P^T with the same instruction (A = V^T read from LDS with the
//   transposing ds_read_b64_tr_b16, B = P taken straight from the S
//   accumulators after a bf16 conversion).
//
// Software pipeline.  Stage i issues the MFMAs of S(i+1) and, in the same
// instruction stream, the exponentials of S(i) (exp2, row sum, bf16
// packing), so the vector ALU works while the matrix core does; then the
// MFMAs of O += P(i) V(i).
//
// Key permutation.  The 32x32 accumulator puts row rho of S^T in register
// r = 4*(rho/8) + rho%4 of lane-half (rho/4)%2.  Loading key kappa into MFMA
// row rho = kappa with bits 2 and 3 swapped makes registers 8c..8c+7 of lane
// half h hold keys 16c + 8h .. 16c + 8h + 7, which is exactly the B-operand
// layout of a 16-key P chunk; the V^T operand reads the same keys.
//
// Data movement.  K and V stages go from global memory straight into LDS
// (global_load_lds_dwordx4, 16 bytes per lane, no registers): K(i+2) and
// V(i+1) are requested at the top of stage i into the buffers that stage i-1
// finished with, and one barrier per stage publishes them.  The four buffers
// are separate LDS objects, so the compiler can tell the DMA targets from
// the buffers being read and does not wait for the loads before each read.
// Both layouts are permuted on the global side (each lane fetches the chunk
// that belongs at its LDS slot):
//   K: rows of 256 bytes, 16-byte chunk c of row r at chunk c ^ (r & 15), so
//      the 16 lanes reading one MFMA operand hit distinct banks;
//   V: rows of 256 bytes, chunk c of row r at chunk (c + 4 (r & 3)) & 15, so
//      the four rows of one transposing read cover all banks once.
//
// Softmax: log2 domain with the scale folded in.  The exponentials of every
// stage are taken against a fixed reference m, the first stage's row max; no
// row max is tracked per stage and O is never rescaled inside the walk.  When
// a lane's share of a stage's row sum exceeds 2^32 (a logit above m + 27),
// the stage's row max is recorded and, after the walk, the whole workgroup
// walks the tile again from that larger m (rare: the logits of a tile rise
// that far above its first stage only for adversarial inputs).  O/l and
// LSE = m + log2(l) do not depend on the choice of m.
//
// Workgroup numbering: dispatch hands workgroups to the 8 XCDs round-robin.
// Tiles are numbered so that in every round of 8 x 64 resident workgroups all
// XCDs work on one contiguous run of tiles (the same head), each XCD on its
// own contiguous sub-run: the head's K/V stays in the shared last-level cache
// and query tiles whose kept blocks overlap share an L2.  With a workspace,
// the tiles of each (batch, head) are first ranked by the middle entry of
// their lists (tile_order_kernel) and a sub-run takes consecutive ranks: the
// 64 tiles that walk their ascending lists side by side on one XCD then sit
// near the same key blocks at the same time, and fewer blocks leave the L2
// before their last reader.  Each tile is computed the same way wherever it
// runs, so the order changes no output bit.
#include "common.h"

namespace basa {
namespace {

constexpr int D = 128;
constexpr int BQ = 128;
constexpr int BK = 128;
constexpr int SK = 64;                        // keys per stage
constexpr int NT = 256;                       // threads per workgroup (4 waves)
constexpr int SBYTES = SK * D * 2;            // 16 KB per K or V stage
constexpr int MAX_KEPT = 1024;                // list slots staged in LDS (the last holds the count)
constexpr int REG_KEPT = 128;                 // lists up to this long are also held in two VGPRs
constexpr int RESIDENT_PER_XCD = 64;          // two workgroups per CU, 32 CUs per XCD
constexpr float kBound = 4294967296.0f;       // 2^32: largest lane share of a row sum taken as is

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;

__shared__ __attribute__((aligned(16))) uint8_t s_k0[SBYTES];
__shared__ __attribute__((aligned(16))) uint8_t s_k1[SBYTES];
__shared__ __attribute__((aligned(16))) uint8_t s_v0[SBYTES];
__shared__ __attribute__((aligned(16))) uint8_t s_v1[SBYTES];
__shared__ int32_t s_lst[MAX_KEPT];
__shared__ int32_t s_flag;  // set when the walk needs a second pass

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
  const int32_t* order;  // [batch*heads_q][lists] tile ranks, or null (natural order)
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

template <int P> __device__ __forceinline__ uint8_t* kbuf() { return P ? s_k1 : s_k0; }
template <int P> __device__ __forceinline__ uint8_t* vbuf() { return P ? s_v1 : s_v0; }

// Per-thread state of the walk.
struct Walk {
  const uint16_t* kbase;   // this head's K rows
  const uint16_t* vbase;
  int koff[4], voff[4];    // element offsets of this lane's DMA chunks within a stage
  int vrd[4];              // byte offsets of this lane's V^T operand reads (per 32-channel group)
  int lst0, lst1;          // short lists: entry e in lane e % 64 of lst0 (e < 64) or lst1
  int wave, krow_l, hi, n_stage;
};

// first element of stage j (64 keys) of the head's K or V.  A short list is
// read from the VGPRs (wave-uniform lane select, no LDS access); a long one
// from LDS.
template <bool REG>
__device__ __forceinline__ int64_t stage_elem(const Walk& w, int j) {
  const int e = j >> 1;
  const int blk = REG ? __builtin_amdgcn_readlane(e < 64 ? w.lst0 : w.lst1, e & 63) : s_lst[e];
  return ((int64_t)blk * BK + (j & 1) * SK) * D;
}

template <int P, bool REG>
__device__ __forceinline__ void dma_k(const Walk& w, int j) {
  const uint16_t* g = w.kbase + stage_elem<REG>(w, j);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    __builtin_amdgcn_global_load_lds(g + w.koff[i], (lds_void*)(kbuf<P>() + (16 * w.wave + 4 * i) * 256),
                                     16, 0, 0);
}

template <int P, bool REG>
__device__ __forceinline__ void dma_v(const Walk& w, int j) {
  const uint16_t* g = w.vbase + stage_elem<REG>(w, j);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    __builtin_amdgcn_global_load_lds(g + w.voff[i], (lds_void*)(vbuf<P>() + (16 * w.wave + 4 * i) * 256),
                                     16, 0, 0);
}

// S^T = K Q^T for the 64 keys in K buffer P: two 32-key sub-tiles whose
// accumulation chains alternate, so consecutive MFMAs are independent
template <int P>
__device__ __forceinline__ void qk(const Walk& w, const bf16x8* qf, f32x16* s) {
  const uint8_t* kc = kbuf<P>();
#pragma unroll
  for (int c = 0; c < 8; ++c) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int krow = 32 * st + w.krow_l;
      const bf16x8 af =
          *reinterpret_cast<const bf16x8*>(kc + krow * 256 + (((2 * c + w.hi) ^ (krow & 15)) * 16));
      if (c == 0) {
        const f32x16 zero = {};
        s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[c], zero, 0, 0, 0);
      } else {
        s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[c], s[st], 0, 0, 0);
      }
    }
  }
}

// Row max of the first stage's logits (log2 units), the starting m.
__device__ __forceinline__ float max_stage(const f32x16* s, float scale_log2) {
  float mx = s[0][0];
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[st][r]);
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * scale_log2;
}

// P = exp2(scale*S - m) as bf16 MFMA operands; returns the lane's share of the row sum.
__device__ __forceinline__ float exp_stage(const f32x16* s, float scale_log2, float m, bf16x8* pf) {
  float psum = 0.f;
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][8 * cc + j], scale_log2, -m));
        psum += p;
        pf[2 * st + cc][j] = (__bf16)p;
      }
  return psum;
}

// Row state of the walk.  The exponentials are taken against a fixed
// reference m (log2 units), the first stage's row max.  A lane share of a
// stage's row sum above 2^32 means a logit exceeds m by more than 27: the
// stage's row max is then recorded in m_seen and the walk is marked for a
// second pass, which starts from m = m_seen and cannot overflow (every logit
// of the tile is at most m_seen + 32).  Values below the bound keep O, l and
// P far inside the float range.
struct Rows {
  float m, m_seen, l;
  bool over;
};

// O^T += V^T P^T over the 64 keys in V buffer P, 16 keys at a time
template <int P>
__device__ __forceinline__ void pv(const Walk& w, const bf16x8* pf, f32x16* oacc) {
  const uint8_t* vc = vbuf<P>();
#pragma unroll
  for (int ch = 0; ch < 4; ++ch) {  // 16-key chunk: keys 16 ch .. 16 ch + 15
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint8_t* p0 = vc + 16 * ch * 256 + w.vrd[u];
      const v4i16 k03 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p0);
      const v4i16 k47 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0 + 4 * 256));
      const bf16x8 vf =
          __builtin_bit_cast(bf16x8, __builtin_shufflevector(k03, k47, 0, 1, 2, 3, 4, 5, 6, 7));
      oacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ch], oacc[u], 0, 0, 0);
    }
  }
}

// One stage i with buffer parity P = i & 1.  On entry S(i) is in s_cur,
// K(i+1) sits in K buffer P^1 and V(i) in V buffer P; S(i+1) goes to s_next.
// NEXT: stage i+1 exists.
template <int P, bool NEXT, bool REG>
__device__ __forceinline__ void stage(const Walk& w, int i, const bf16x8* qf, const f32x16* s_cur,
                                      f32x16* s_next, f32x16* oacc, Rows& r, float scale_log2) {
  if (NEXT) {
    // K(i) and V(i-1) were consumed by stage i-1; past the end, K(n-1) is fetched again
    dma_k<P, REG>(w, min(i + 2, w.n_stage - 1));
    dma_v<P ^ 1, REG>(w, i + 1);
  }
  bf16x8 pf[4];
  if (NEXT) qk<P ^ 1>(w, qf, s_next);  // S(i+1) on the matrix core while P(i) is formed
  const float psum = exp_stage(s_cur, scale_log2, r.m, pf);
  r.l += psum;
  pv<P>(w, pf, oacc);
  if (__ballot(!(psum <= kBound)) != 0) {  // rare, wave-uniform: the walk is redone
    r.over = true;
    r.m_seen = fmaxf(r.m_seen, max_stage(s_cur, scale_log2));
  }
  if (NEXT) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // this wave's loads of stage i+1 have landed
    __syncthreads();                     // ... and everyone's; buffers of stage i are free
  }
}

template <bool OUT_BF16, bool REG>
__global__ __launch_bounds__(NT, 2) void attn_mfma_kernel(MfmaArgs a) {
  int64_t tile = tile_of(blockIdx.x, a.tiles);
  if (a.order) tile = tile / a.lists * a.lists + a.order[tile];
  const int64_t t = tile % a.lists;
  const int64_t bh = tile / a.lists;
  const int h = (int)(bh % a.heads_q);
  const int64_t b = bh / a.heads_q;
  const int hk = h / a.group;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int li = lane & 31;

  Walk w;
  w.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  w.hi = lane >> 5;
  w.krow_l = swap_bits_2_3(li);
  w.kbase = a.k + (b * a.heads_kv + hk) * a.len_k * D;
  w.vbase = a.v + (b * a.heads_kv + hk) * a.len_k * D;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // DMA: lane lands at byte 16*lane of rows 16w+4i .. +3: row r, physical chunk p = lane & 15
    const int r = 16 * w.wave + 4 * i + (lane >> 4);
    const int p = lane & 15;
    w.koff[i] = r * D + (p ^ (r & 15)) * 8;
    w.voff[i] = r * D + ((p - 4 * (r & 3)) & 15) * 8;
  }
  {
    // V^T operand: 16-lane group G, lane g: rows 8(G/2) + g/4 (+4), channels
    // 32u + 16(G%2) + 4(g%4) .. +3 (bytes 8*(g&1) of logical chunk 4u + 2(G%2) + (g%4)/2)
    const int G = lane >> 4, g = lane & 15;
    const int row = 8 * (G >> 1) + (g >> 2);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int cl = 4 * u + 2 * (G & 1) + ((g & 3) >> 1);
      w.vrd[u] = row * 256 + ((cl + 4 * (row & 3)) & 15) * 16 + 8 * (g & 1);
    }
  }

  const int64_t qrow = t * BQ + w.wave * 32 + li;
  const uint16_t* qp = a.q + ((b * a.heads_q + h) * a.len_q + qrow) * D;
  bf16x8 qf[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) qf[c] = *reinterpret_cast<const bf16x8*>(qp + 16 * c + 8 * w.hi);

  // compact the tile's list into LDS (valid blocks only, order kept): wave 0, 64 entries a step
  const int nblk_k = (int)(a.len_k / BK);
  if (w.wave == 0) {
    const int32_t* g = a.kv_idx + ((b * a.heads_q + h) * a.idx_rows + t) * a.idx_stride;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int n = 0;
    for (int base = 0; base < a.kept; base += 64) {
      const int e = base + lane;
      const int32_t blk = e < a.kept ? g[e] : -1;
      const bool ok = blk >= 0 && blk < nblk_k;
      const uint64_t msk = __ballot(ok);
      if (ok) s_lst[n + __popcll(msk & below)] = blk;
      n += __popcll(msk);
    }
    if (lane == 0) {
      s_lst[MAX_KEPT - 1] = n;  // kept < MAX_KEPT, so the count slot is never an entry
      s_flag = 0;
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // Q loads settled (compiler-visible vmcnt(0))
  __syncthreads();
  w.n_stage = 2 * s_lst[MAX_KEPT - 1];
  if (REG) {
    w.lst0 = s_lst[lane];
    w.lst1 = s_lst[64 + lane];
  }

  f32x16 oacc[4];
  Rows r;
  r.over = false;
  r.m_seen = -INFINITY;
  // At most two passes over the kept blocks: the second only when a logit
  // exceeded the first stage's row max by more than 27 (log2 units).
  for (int pass = 0;; ++pass) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[u][e] = 0.f;
    r.l = 0.f;
    r.m = -INFINITY;
    if (w.n_stage > 0) {
      // prologue: K(0), K(1), V(0); then S(0)
      dma_k<0, REG>(w, 0);
      dma_k<1, REG>(w, 1);
      dma_v<0, REG>(w, 0);
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      f32x16 s_a[2], s_b[2];  // logits of even / odd stages
      qk<0>(w, qf, s_a);
      r.m = pass == 0 ? max_stage(s_a, a.scale_log2) : r.m_seen;
      r.m_seen = r.m;
      __syncthreads();  // every wave has read K(0) before stage 0 refills its buffer with K(2)
      // n_stage is even: stages go in pairs (even, odd); the last pair ends the walk
      int i = 0;
      for (; i + 2 < w.n_stage; i += 2) {
        stage<0, true, REG>(w, i, qf, s_a, s_b, oacc, r, a.scale_log2);
        stage<1, true, REG>(w, i + 1, qf, s_b, s_a, oacc, r, a.scale_log2);
      }
      stage<0, true, REG>(w, i, qf, s_a, s_b, oacc, r, a.scale_log2);
      stage<1, false, REG>(w, i + 1, qf, s_b, s_a, oacc, r, a.scale_log2);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // no load into this workgroup's LDS outlives the walk
    if (pass == 0 && r.over) s_flag = 1;
    __syncthreads();  // every wave is done with the stage buffers; the flag is settled
    if (pass != 0 || s_flag == 0) break;  // workgroup-uniform
  }
  const float m = r.m, l = r.l;

  // epilogue: O = O^T / l, LSE = (m + log2 l) ln 2
  const float l_tot = l + __shfl_xor(l, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int64_t orow = (b * a.heads_q + h) * a.len_q + qrow;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int ch = 32 * u + 8 * rq + 4 * w.hi;
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
  if (w.hi == 0) a.lse[orow] = l_tot > 0.f ? (m + log2f(l_tot)) * kLn2 : -INFINITY;
}

constexpr int ORDER_MAX = 2048;  // lists per head that tile_order_kernel ranks (keys in LDS)
constexpr int ORDER_KEYS = 1 << 20;  // key blocks per head it handles (key * ORDER_MAX + tile < 2^31)

// order[bh][r] = the tile of (batch, head) bh with rank r by the middle entry
// of its list (ties by tile index); entries outside the key range rank as 0.
// One workgroup per (batch, head).  Each tile's rank is the count of packed
// keys (middle entry * ORDER_MAX + tile, all distinct) below its own, read
// four at a time from LDS.
__global__ __launch_bounds__(256) void tile_order_kernel(MfmaArgs a, int nblk_k, int32_t* order) {
  __shared__ __attribute__((aligned(16))) int32_t key[ORDER_MAX];
  const int64_t bh = blockIdx.x;
  const int n = (int)a.lists;
  const int n4 = (n + 3) >> 2;
  for (int t = threadIdx.x; t < 4 * n4; t += 256) {
    int32_t packed = INT32_MAX;  // padding to a multiple of 4 ranks above every tile
    if (t < n) {
      const int32_t k = a.kv_idx[(bh * a.idx_rows + t) * a.idx_stride + a.kept / 2];
      packed = ((k >= 0 && k < nblk_k) ? k : 0) * ORDER_MAX + t;
    }
    key[t] = packed;
  }
  __syncthreads();
  const int4* key4 = reinterpret_cast<const int4*>(key);
  for (int t = threadIdx.x; t < n; t += 256) {
    const int kt = key[t];
    int r = 0;
#pragma unroll 4
    for (int u = 0; u < n4; ++u) {
      const int4 k4 = key4[u];
      r += (k4.x < kt) + (k4.y < kt) + (k4.z < kt) + (k4.w < kt);
    }
    order[bh * n + r] = t;
  }
}

}  // namespace

int64_t attn_mfma_workspace_bytes(const basa_attn_desc* d) {
  const basa_kv_segment& g = d->seg[0];
  if (d->lists < 1 || d->lists > ORDER_MAX || g.count < 1 || d->batch < 1 || g.len / BK > ORDER_KEYS)
    return 0;
  return (d->batch * d->heads_q * d->lists * (int64_t)sizeof(int32_t) + 255) / 256 * 256;
}

bool attn_mfma_supported(const basa_attn_desc* d, int q_dtype, int o_dtype) {
  const basa_kv_segment& g = d->seg[0];
  // the list is compacted into the first MAX_KEPT-1 LDS slots; the last holds the count
  return q_dtype == BASA_BF16 && d->n_segments == 1 && g.dtype == BASA_BF16 && g.shift == 0 &&
         g.bias == 0.f && d->head_dim == D && d->tile_q == BQ && d->block_k == BK &&
         d->q_rows == nullptr && d->lists * BQ == d->len_q && d->scale > 0.0 &&
         g.count < MAX_KEPT && (o_dtype == BASA_BF16 || o_dtype == BASA_F32);
}

hipError_t launch_attn_mfma(const basa_attn_desc* d, const void* q, void* o, int o_dtype,
                            float* lse, int32_t* order, hipStream_t s) {
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
  a.order = nullptr;
  if (a.tiles == 0) return hipSuccess;
  if (order) {  // the caller checked the workspace against attn_mfma_workspace_bytes
    tile_order_kernel<<<dim3((unsigned)(a.tiles / a.lists)), 256, 0, s>>>(a, (int)(a.len_k / BK), order);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.order = order;
  }
  dim3 grid((unsigned)a.tiles);
  const bool reg = g.count <= REG_KEPT;
  if (o_dtype == BASA_BF16) {
    if (reg)
      attn_mfma_kernel<true, true><<<grid, NT, 0, s>>>(a);
    else
      attn_mfma_kernel<true, false><<<grid, NT, 0, s>>>(a);
  } else {
    if (reg)
      attn_mfma_kernel<false, true><<<grid, NT, 0, s>>>(a);
    else
      attn_mfma_kernel<false, false><<<grid, NT, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace basa
