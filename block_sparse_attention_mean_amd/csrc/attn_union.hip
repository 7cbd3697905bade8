// Sparse prefix attention of a few query rows per key head as one walk over
// the union of their kept key blocks (the LoSA step's active rows).
//
// LoSA post, "KV inflation" and method steps 2-4: every active (token, query
// head) row keeps its own prefix blocks, so the key heads' data that the step
// must read is the union of the rows' selections, not the sum.  Here each key
// block of that union is read from memory once and used by every row that
// kept it; the result per row is the softmax attention of Eq. 1 over exactly
// its own listed blocks, as the row-at-a-time kernel computes it.
//
// Work decomposition.  The prefix blocks of a key head are cut into chunks of
// UCB consecutive blocks.  Workgroup (batch, key head, chunk) first counts,
// in LDS, how often each row of the key head lists each block of its chunk
// (a block listed twice by a row counts twice, as in the list walk).  Its
// waves then take work items (query head of the group, share): an item walks
// the chunk's blocks that any row of its query head kept, every P-th of them,
// so the P items of a head split its blocks and the heads of a group walk the
// same blocks at about the same time (a block kept by several heads is read
// from memory once and found in the cache by the others).  A wave holds a
// block's 16 key rows (four lanes per key, a quarter of the channels each: one
// contiguous 4 KB read) and 16 value rows (two channels per lane) in
// registers, loads the next block while it reduces the current one, and for
// every row of its head that kept the block computes 16 logits from the row's
// query (LDS), updates the row's online-softmax state (lazy max, as in the
// row kernel) and adds the value product with each key's probability
// broadcast from its lanes.  Row states live in LDS per (share, row); at the
// end the shares of each row are combined and written to the workspace as the
// chunk's partial (unnormalised O, max, sum).  A second kernel combines each
// row's chunk partials in chunk order and writes O and the LSE into the row's
// place, like the list walk (the cache update of the LoSA step).  Both
// kernels are deterministic: every sum runs in a fixed order.
#include "common.h"

namespace basa {
namespace {

constexpr int UCB = 64;        // key blocks per chunk
constexpr int UW = 8;          // waves per workgroup
constexpr int UMAX_R = 32;     // rows per key head (group * lists)
constexpr float kULazy = 8.0f; // log2 headroom before a row's max is raised
constexpr int UMAX_STATES = 64; // row states per workgroup (rows x shares)
static_assert(UCB == 64, "one lane of a wave per block of a chunk");

// waves (shares) per query head: enough to occupy the workgroup's waves, at
// most UMAX_STATES row states in all
__host__ __device__ inline int share_count(int group, int rows) {
  int p = group < UW ? UW / group : 1;
  while (p > 1 && p * rows > UMAX_STATES) --p;
  return p;
}

struct UnionArgs {
  const void* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* idx;
  const int32_t* q_rows;
  void* o;
  float* lse;
  float* ws_o;   // [B][Hkv][chunks][R][D] unnormalised partial outputs
  float* ws_ml;  // [B][Hkv][chunks][R][2] (max in log2 units, sum)
  int64_t len_q, len_k, idx_rows;
  int idx_stride, count, lists, heads_q, heads_kv, group, rows, chunks, nblk;
  float scale_log2;
};

__device__ __forceinline__ float dpp_swap1(float x) {  // quad_perm [1,0,3,2]
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_swap2(float x) {  // quad_perm [2,3,0,1]
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) x = fmaxf(x, __shfl_xor(x, sh));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) x += __shfl_xor(x, sh);
  return x;
}

// query row of key-head row r (query head g*group + r/lists, list r%lists)
__device__ __forceinline__ int64_t row_token(const UnionArgs& a, int64_t b, int r) {
  const int t = r % a.lists;
  const int64_t tok = a.q_rows[b * a.lists + t];
  return (tok < 0 || tok >= a.len_q) ? -1 : tok;
}

// a key block's 16 key rows (lane: key `slot`, channels kq..kq+CPL-1, raw
// bf16 words) and 16 value rows (lane: channels VPL*lane.., raw bf16 words)
template <int D>
struct BlockRegs {
  static constexpr int CPL = D / 4;
  static constexpr int VW = D / 128;  // 32-bit value words per lane and key (1 or 0.5)
  uint4 k[CPL / 8];
  uint32_t v[16];
  __device__ __forceinline__ void load(const uint16_t* kb, const uint16_t* vb, int slot, int kq,
                                       int lane) {
    const uint4* kp = reinterpret_cast<const uint4*>(kb + slot * D + kq);
#pragma unroll
    for (int w = 0; w < CPL / 8; ++w) k[w] = kp[w];
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      if constexpr (D == 128)
        v[s] = *reinterpret_cast<const uint32_t*>(vb + s * D + 2 * lane);
      else
        v[s] = vb[s * D + lane];
    }
  }
};

template <int D, bool QBF>
__global__ __launch_bounds__(UW * 64) void union_walk_kernel(UnionArgs a) {
  constexpr int CPL = D / 4;           // channels per lane in the key layout
  constexpr int VPL = D / 64;          // channels per lane in the value layout
  // dynamic LDS: the rows' queries [R][D], then the row states' outputs [P*R][D]
  extern __shared__ float s_dyn[];
  __shared__ int32_t s_cnt[UCB][UMAX_R];
  __shared__ float s_m[UMAX_STATES];
  __shared__ float s_l[UMAX_STATES];
  __shared__ int64_t s_tok[UMAX_R];        // query row of each key-head row, or -1

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t unit = blockIdx.x;
  const int c = (int)(unit % a.chunks);
  const int g = (int)((unit / a.chunks) % a.heads_kv);
  const int64_t b = unit / ((int64_t)a.chunks * a.heads_kv);
  const int R = a.rows, L = a.lists;
  const int blk0 = c * UCB;
  const int P = share_count(a.group, R);   // waves per query head
  float* s_q = s_dyn;                      // s_q[r * D + ch]
  float* s_o = s_dyn + R * D;              // s_o[(p * R + r) * D + ch]: state of row r, share p

  // how often each row lists each block of this chunk.  Every list entry and
  // query value a thread needs is requested before the first one is used.
  for (int e = threadIdx.x; e < UCB * UMAX_R; e += UW * 64) s_cnt[e / UMAX_R][e % UMAX_R] = 0;
  if ((int)threadIdx.x < R) s_tok[threadIdx.x] = row_token(a, b, threadIdx.x);
  __syncthreads();
  constexpr int NT = UW * 64;
  for (int e0 = 0; e0 < R * a.count; e0 += 8 * NT) {
    int32_t blk[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = e0 + i * NT + threadIdx.x;
      blk[i] = -1;
      if (e < R * a.count) {
        const int r = e / a.count, j = e % a.count;
        const int h = g * a.group + r / L;
        if (s_tok[r] >= 0)
          blk[i] = a.idx[((b * a.heads_q + h) * a.idx_rows + r % L) * a.idx_stride + j];
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = e0 + i * NT + threadIdx.x;
      if (blk[i] >= blk0 && blk[i] < blk0 + UCB && blk[i] < a.nblk)
        atomicAdd(&s_cnt[blk[i] - blk0][e / a.count], 1);
    }
  }
  // the key head's query rows (float32 in LDS), zeroed states
  for (int e0 = 0; e0 < R * D; e0 += 8 * NT) {
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = e0 + i * NT + threadIdx.x;
      x[i] = 0.f;
      if (e < R * D) {
        const int r = e / D, ch = e % D;
        const int64_t tok = s_tok[r];
        if (tok >= 0) {
          const int h = g * a.group + r / L;
          const int64_t off = ((b * a.heads_q + h) * a.len_q + tok) * D + ch;
          x[i] = QBF ? bf16_bits_to_f32(static_cast<const uint16_t*>(a.q)[off])
                     : static_cast<const float*>(a.q)[off];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = e0 + i * NT + threadIdx.x;
      if (e < R * D) s_q[e] = x[i];
    }
  }
  for (int e = threadIdx.x; e < P * R * D; e += UW * 64) s_o[e] = 0.f;
  for (int e = threadIdx.x; e < UMAX_STATES; e += UW * 64) {
    s_m[e] = -INFINITY;
    s_l[e] = 0.f;
  }
  __syncthreads();

  // Work items: (query head j of the group, share p of its blocks); a wave
  // takes items w, w + UW, ...  The P items of a query head split the head's
  // blocks by position (p, p + P, ...); each item has its own row states.
  const int slot = lane >> 2;            // key of the block this lane holds (key layout)
  const int kq = (lane & 3) * CPL;       // first channel of this lane's quarter
  const int64_t head = (b * a.heads_kv + g) * a.len_k;
  for (int item = wave; item < a.group * P; item += UW) {
    const int j = item / P, p = item % P;
    // blocks of the chunk kept by any row of query head j: bit u of `mine`
    uint32_t rows_u = 0;                 // lane u: the rows of head j that keep block u (bit t)
    for (int t = 0; t < L; ++t) rows_u |= (s_cnt[lane][j * L + t] > 0 ? 1u : 0u) << t;
    uint64_t mine = __ballot(rows_u != 0);
    // this wave's share: every P-th of those blocks, starting at the p-th
    for (int skip = 0; skip < p && mine; ++skip) mine &= mine - 1;
    auto next_of = [&](uint64_t m) {     // drop P-1 blocks after the lowest
      m &= m - 1;
      for (int skip = 1; skip < P && m; ++skip) m &= m - 1;
      return m;
    };
    BlockRegs<D> cur, nxt;
    if (mine) {
      const int u0 = __builtin_ctzll(mine);
      const int64_t key0 = (int64_t)(blk0 + u0) * 16;
      cur.load(a.k + (head + key0) * D, a.v + (head + key0) * D, slot, kq, lane);
    }
    while (mine) {
      const int u = __builtin_ctzll(mine);
      const uint64_t rest = next_of(mine);
      {  // the next block's rows are in flight while this one is reduced (past the
         // last block the current one is requested again: an unconditional load
         // keeps the wait for the current rows exact)
        const int u1 = rest ? __builtin_ctzll(rest) : u;
        const int64_t key1 = (int64_t)(blk0 + u1) * 16;
        nxt.load(a.k + (head + key1) * D, a.v + (head + key1) * D, slot, kq, lane);
      }
      float kf[CPL];
#pragma unroll
      for (int w = 0; w < CPL / 8; ++w) {
        const uint32_t x[4] = {cur.k[w].x, cur.k[w].y, cur.k[w].z, cur.k[w].w};
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
          kf[8 * w + 2 * q2] = bf16_bits_to_f32(x[q2] & 0xFFFFu);
          kf[8 * w + 2 * q2 + 1] = bf16_bits_to_f32(x[q2] >> 16);
        }
      }
      float vv[16][VPL];
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        if constexpr (VPL == 2) {
          vv[s][0] = bf16_bits_to_f32(cur.v[s] & 0xFFFFu);
          vv[s][1] = bf16_bits_to_f32(cur.v[s] >> 16);
        } else {
          vv[s][0] = bf16_bits_to_f32(cur.v[s] & 0xFFFFu);
        }
      }
      uint32_t rows = __builtin_amdgcn_readlane(rows_u, u);
      while (rows) {
        const int t = __builtin_ctz(rows);
        rows &= rows - 1;
        const int r = j * L + t;
        const float cnt = (float)s_cnt[u][r];
        float dot = 0.f;
#pragma unroll
        for (int ch = 0; ch < CPL; ++ch) dot = __builtin_fmaf(s_q[r * D + kq + ch], kf[ch], dot);
        dot += dpp_swap1(dot);
        dot += dpp_swap2(dot);
        const float z = dot * a.scale_log2;
        // the row's state in this item; every lane keeps (and writes) the same m and l
        const int st = p * R + r;
        float m = s_m[st];
        float l = s_l[st];
        float* orow = s_o + st * D + VPL * lane;
        float acc[VPL];
#pragma unroll
        for (int q2 = 0; q2 < VPL; ++q2) acc[q2] = orow[q2];
        if (__ballot(z > m + kULazy) != 0) {  // raise the row's max (wave-uniform)
          const float mn = fmaxf(m, wave_max(z));
          const float sc = m == -INFINITY ? 0.f : exp2f(m - mn);
#pragma unroll
          for (int q2 = 0; q2 < VPL; ++q2) acc[q2] *= sc;
          l *= sc;
          m = mn;
        }
        const float pk = cnt * exp2f(z - m);
#pragma unroll
        for (int s = 0; s < 16; ++s) {
          const float ps = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pk), 4 * s));
          l += ps;
#pragma unroll
          for (int q2 = 0; q2 < VPL; ++q2) acc[q2] = __builtin_fmaf(ps, vv[s][q2], acc[q2]);
        }
#pragma unroll
        for (int q2 = 0; q2 < VPL; ++q2) orow[q2] = acc[q2];
        s_m[st] = m;
        s_l[st] = l;
      }
      mine = rest;
      cur = nxt;
    }
  }
  __syncthreads();

  // combine, per row, the states of its P shares (in share order)
  const int64_t base = (b * a.heads_kv + g) * a.chunks + c;
  for (int e = threadIdx.x; e < R * D; e += UW * 64) {
    const int r = e / D, ch = e % D;
    float mm = -INFINITY;
    for (int q2 = 0; q2 < P; ++q2) mm = fmaxf(mm, s_m[q2 * R + r]);
    float o = 0.f, l = 0.f;
    if (mm != -INFINITY) {
      for (int q2 = 0; q2 < P; ++q2) {
        const float m2 = s_m[q2 * R + r];
        const float sc = m2 == -INFINITY ? 0.f : exp2f(m2 - mm);
        o += s_o[(q2 * R + r) * D + ch] * sc;
        l += s_l[q2 * R + r] * sc;
      }
    }
    a.ws_o[(base * R + r) * D + ch] = o;
    if (ch == 0) {
      a.ws_ml[(base * R + r) * 2] = mm;
      a.ws_ml[(base * R + r) * 2 + 1] = l;
    }
  }
}

// One wave per row: the row's chunk partials combined in chunk order, then
// O = o / l and LSE = (m + log2 l) ln 2 written at the row's place.  Lane c
// reads the max and sum of chunk c (64 chunks at a time), so the scale of
// every chunk is known before the outputs are read; the output loop then has
// no branch on loaded values and its loads overlap.
template <int D, bool OBF>
__global__ __launch_bounds__(64) void union_merge_kernel(UnionArgs a) {
  constexpr int VPL = D / 64;
  const int lane = threadIdx.x;
  const int64_t unit = blockIdx.x;            // (b, key head, row)
  const int r = (int)(unit % a.rows);
  const int g = (int)((unit / a.rows) % a.heads_kv);
  const int64_t b = unit / ((int64_t)a.rows * a.heads_kv);
  const int64_t tok = row_token(a, b, r);
  if (tok < 0) return;  // a row map entry outside q: nothing to write
  const int h = g * a.group + r / a.lists;
  const int64_t base = (b * a.heads_kv + g) * a.chunks;
  float mm = -INFINITY;
  for (int c0 = 0; c0 < a.chunks; c0 += 64) {
    const int c = c0 + lane;
    if (c < a.chunks) mm = fmaxf(mm, a.ws_ml[((base + c) * a.rows + r) * 2]);
  }
  mm = wave_max(mm);
  float o[VPL] = {}, l = 0.f;
  for (int c0 = 0; c0 < a.chunks; c0 += 64) {
    const int c = c0 + lane;
    float sc = 0.f, lc = 0.f;
    if (c < a.chunks && mm != -INFINITY) {
      const float m = a.ws_ml[((base + c) * a.rows + r) * 2];
      lc = a.ws_ml[((base + c) * a.rows + r) * 2 + 1];
      sc = m == -INFINITY ? 0.f : exp2f(m - mm);
    }
    l += wave_sum(lc * sc);
    const int n = min(64, a.chunks - c0);
    // chunk order; partials without keys hold zeros.  Eight chunks' outputs are
    // requested before the first is added.
    for (int i0 = 0; i0 < n; i0 += 8) {
      float pv[8][VPL];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t pr = (base + c0 + min(i0 + i, n - 1)) * a.rows + r;
#pragma unroll
        for (int u = 0; u < VPL; ++u) pv[i][u] = a.ws_o[pr * D + VPL * lane + u];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float si = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc), min(i0 + i, 63)));
        if (i0 + i < n) {
#pragma unroll
          for (int u = 0; u < VPL; ++u) o[u] = __builtin_fmaf(pv[i][u], si, o[u]);
        }
      }
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int64_t orow = (b * a.heads_q + h) * a.len_q + tok;
#pragma unroll
  for (int u = 0; u < VPL; ++u) {
    const float val = o[u] * inv;
    if constexpr (OBF)
      static_cast<uint16_t*>(a.o)[orow * D + VPL * lane + u] = f32_to_bf16_bits(val);
    else
      static_cast<float*>(a.o)[orow * D + VPL * lane + u] = val;
  }
  if (lane == 0) a.lse[orow] = l > 0.f ? (mm + log2f(l)) * kLn2 : -INFINITY;
}

}  // namespace

int64_t attn_union_workspace_bytes(const basa_attn_desc* d) {
  const basa_kv_segment& g = d->seg[0];
  if (!(d->q_rows && d->tile_q == 1 && d->n_segments == 1 && d->block_k == 16 &&
        (d->head_dim == 64 || d->head_dim == 128) && g.dtype == BASA_BF16 && g.shift == 0 &&
        g.bias == 0.f && d->batch >= 1 && d->lists >= 1 && g.len >= 16 && g.len % 16 == 0 &&
        (d->heads_q / d->heads_kv) * d->lists <= UMAX_R && g.count >= 1))
    return 0;
  const int64_t rows = (d->heads_q / d->heads_kv) * d->lists;
  const int64_t chunks = (g.len / 16 + UCB - 1) / UCB;
  return d->batch * d->heads_kv * chunks * rows * (d->head_dim + 2) * (int64_t)sizeof(float);
}

bool attn_union_supported(const basa_attn_desc* d, int64_t workspace_bytes) {
  const int64_t need = attn_union_workspace_bytes(d);
  return need > 0 && workspace_bytes >= need;
}

hipError_t launch_attn_union(const basa_attn_desc* d, const void* q, int q_dtype, void* o,
                             int o_dtype, float* lse, void* workspace, hipStream_t s) {
  const basa_kv_segment& g = d->seg[0];
  UnionArgs a;
  a.q = q;
  a.k = static_cast<const uint16_t*>(g.k);
  a.v = static_cast<const uint16_t*>(g.v);
  a.idx = g.idx;
  a.q_rows = d->q_rows;
  a.o = o;
  a.lse = lse;
  a.len_q = d->len_q;
  a.len_k = g.len;
  a.idx_rows = g.rows;
  a.idx_stride = g.stride;
  a.count = g.count;
  a.lists = (int)d->lists;
  a.heads_q = (int)d->heads_q;
  a.heads_kv = (int)d->heads_kv;
  a.group = (int)(d->heads_q / d->heads_kv);
  a.rows = a.group * a.lists;
  a.nblk = (int)(g.len / 16);
  a.chunks = (a.nblk + UCB - 1) / UCB;
  a.scale_log2 = (float)(d->scale * 1.4426950408889634);
  const int64_t parts = d->batch * d->heads_kv * a.chunks * (int64_t)a.rows;
  a.ws_o = static_cast<float*>(workspace);
  a.ws_ml = a.ws_o + parts * d->head_dim;
  const dim3 g1((unsigned)(d->batch * d->heads_kv * a.chunks));
  const dim3 g2((unsigned)(d->batch * d->heads_kv * a.rows));
  const bool qb = q_dtype == BASA_BF16, ob = o_dtype == BASA_BF16;
  const size_t lds = (size_t)(1 + share_count(a.group, a.rows)) * a.rows * d->head_dim * sizeof(float);
  if (d->head_dim == 128) {
    if (qb) union_walk_kernel<128, true><<<g1, UW * 64, lds, s>>>(a);
    else union_walk_kernel<128, false><<<g1, UW * 64, lds, s>>>(a);
  } else {
    if (qb) union_walk_kernel<64, true><<<g1, UW * 64, lds, s>>>(a);
    else union_walk_kernel<64, false><<<g1, UW * 64, lds, s>>>(a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (d->head_dim == 128) {
    if (ob) union_merge_kernel<128, true><<<g2, 64, 0, s>>>(a);
    else union_merge_kernel<128, false><<<g2, 64, 0, s>>>(a);
  } else {
    if (ob) union_merge_kernel<64, true><<<g2, 64, 0, s>>>(a);
    else union_merge_kernel<64, false><<<g2, 64, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace basa
