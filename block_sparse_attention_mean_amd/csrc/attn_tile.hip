// Attention for small query tiles (2..16 rows sharing one key list): the
// log-linear forward's 16-row tiles over fine and coarse key segments, and the
// LoSA in-block attention.
//
// BA-Att section 2: attention restricted to the listed key blocks, Eq. 1's
// softmax over them; the log-linear README's level bias enters as a per-segment
// additive logit term.  Online softmax over chunks of 64 keys.
//
// One workgroup (256 threads) computes one tile.  Each chunk of up to 64 keys
// of one segment is staged in LDS as float32 (from bf16 or float32 tables);
// thread t owns query row r = t/16 and
//   - for the logits, keys (t%16) + 16 i, i < 4 (dot products from LDS, the
//     key rows padded so the 16 threads of a row hit distinct banks),
//   - for the output, channels CPT*(t%16) .. +CPT-1 (CPT = head_dim/16).
// The 16 threads of a row are 16 consecutive lanes, so the row max and sum are
// 16-lane shuffles.  All arithmetic is float32.
#include "common.h"

namespace basa {
namespace {

constexpr int NT = 256;
constexpr int CK = 64;    // keys per chunk
constexpr int MAXR = 16;  // rows per tile

struct TSeg {
  const int32_t* idx;
  const void* k;
  const void* v;
  int64_t len, rows;
  int count, stride, shift, bf16;
  float bias_log2;
};

struct TileArgs {
  TSeg seg[BASA_MAX_SEGMENTS];
  int n_seg;
  const void* q;
  void* o;
  float* lse;
  const int32_t* q_rows;
  int64_t len_q, lists, tiles;
  int heads_q, heads_kv, group, tile_q, block_k;
  float scale_log2;
};

template <int D>
struct TileSmem {
  float k[CK][D + 4];  // padded rows: 16 threads reading 16 rows at one channel hit distinct banks
  float v[CK][D];
  float q[MAXR][D];
  float p[MAXR][CK];
  int64_t row[CK];     // key row of each chunk slot in its table (-1: empty)
};

__device__ __forceinline__ void load4(const void* base, int64_t elem, bool bf16, float* out) {
  if (bf16) {
    const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + elem);
    out[0] = bf16_bits_to_f32(w.x & 0xFFFFu);
    out[1] = bf16_bits_to_f32(w.x >> 16);
    out[2] = bf16_bits_to_f32(w.y & 0xFFFFu);
    out[3] = bf16_bits_to_f32(w.y >> 16);
  } else {
    const float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
    out[0] = f.x; out[1] = f.y; out[2] = f.z; out[3] = f.w;
  }
}

template <bool Q_BF16, bool O_BF16, int D>
__global__ __launch_bounds__(NT) void attn_tile_kernel(TileArgs a) {
  constexpr int CPT = D / 16;  // output channels per thread
  __shared__ TileSmem<D> sm;
  const int64_t tile = blockIdx.x;
  if (tile >= a.tiles) return;
  const int64_t t = tile % a.lists;
  const int64_t bh = tile / a.lists;
  const int h = (int)(bh % a.heads_q);
  const int64_t b = bh / a.heads_q;
  const int hk = h / a.group;
  const int tid = threadIdx.x;
  const int r = tid >> 4;   // query row of this thread
  const int kk = tid & 15;  // key column group / channel group
  const bool row_ok = r < a.tile_q;

  // query rows -> LDS (float32); rows beyond the tile are zero
  for (int e = tid; e < MAXR * D / 4; e += NT) {
    const int rr = (e * 4) / D, c = (e * 4) % D;
    float v4[4] = {0.f, 0.f, 0.f, 0.f};
    if (rr < a.tile_q) {
      int64_t row = t * a.tile_q + rr;
      if (a.q_rows) row = a.q_rows[b * a.lists * a.tile_q + row];
      if (row >= 0 && row < a.len_q) load4(a.q, ((b * a.heads_q + h) * a.len_q + row) * D + c, Q_BF16, v4);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.q[rr][c + i] = v4[i];
  }

  float m = -INFINITY, l = 0.f;
  float acc[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) acc[i] = 0.f;

  for (int si = 0; si < a.n_seg; ++si) {
    const TSeg sg = a.seg[si];
    const bool kbf = sg.bf16 != 0;
    const int32_t* lst = sg.idx + ((b * a.heads_q + h) * sg.rows + (t >> sg.shift)) * sg.stride;
    const int64_t head_row = (b * a.heads_kv + hk) * sg.len;
    const int64_t n_keys = (int64_t)sg.count * a.block_k;
    for (int64_t k0 = 0; k0 < n_keys; k0 += CK) {
      __syncthreads();  // previous chunk's LDS reads are done
      if (tid < CK) {
        int64_t row = -1;
        const int64_t f = k0 + tid;
        if (f < n_keys) {
          const int32_t blk = lst[f / a.block_k];
          const int64_t key = (int64_t)blk * a.block_k + (f % a.block_k);
          if (blk >= 0 && key < sg.len) row = head_row + key;
        }
        sm.row[tid] = row;
      }
      __syncthreads();
      // K and V rows of the chunk -> LDS float32 (4 channels per step; empty slots are zero)
      for (int e = tid; e < CK * D / 4; e += NT) {
        const int j = (e * 4) / D, c = (e * 4) % D;
        const int64_t row = sm.row[j];
        float kv[4] = {0.f, 0.f, 0.f, 0.f}, vv[4] = {0.f, 0.f, 0.f, 0.f};
        if (row >= 0) {
          load4(sg.k, row * D + c, kbf, kv);
          load4(sg.v, row * D + c, kbf, vv);
        }
        *reinterpret_cast<float4*>(&sm.k[j][c]) = make_float4(kv[0], kv[1], kv[2], kv[3]);
        *reinterpret_cast<float4*>(&sm.v[j][c]) = make_float4(vv[0], vv[1], vv[2], vv[3]);
      }
      __syncthreads();

      // logits of row r for keys kk + 16 i
      float z[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) z[i] = 0.f;
#pragma unroll 4
      for (int c = 0; c < D; c += 4) {
        const float4 qv = *reinterpret_cast<const float4*>(&sm.q[r][c]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 kv = *reinterpret_cast<const float4*>(&sm.k[kk + 16 * i][c]);
          z[i] = __builtin_fmaf(qv.x, kv.x, z[i]);
          z[i] = __builtin_fmaf(qv.y, kv.y, z[i]);
          z[i] = __builtin_fmaf(qv.z, kv.z, z[i]);
          z[i] = __builtin_fmaf(qv.w, kv.w, z[i]);
        }
      }
      float cm = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        z[i] = sm.row[kk + 16 * i] >= 0 ? z[i] * a.scale_log2 + sg.bias_log2 : -INFINITY;
        cm = fmaxf(cm, z[i]);
      }
#pragma unroll
      for (int sh = 8; sh >= 1; sh >>= 1) cm = fmaxf(cm, __shfl_xor(cm, sh, 16));
      const float m_new = fmaxf(m, cm);
      float p[4];
      if (m_new == -INFINITY) {  // nothing valid for this row yet
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = 0.f;
      } else {
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);
        l *= alpha;
#pragma unroll
        for (int i = 0; i < CPT; ++i) acc[i] *= alpha;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[i] = z[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(z[i] - m_new);
          l += p[i];
        }
        m = m_new;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.p[r][kk + 16 * i] = p[i];
      __syncthreads();

      // O[r][CPT*kk .. +CPT-1] += sum_j p[r][j] v[j][...]
#pragma unroll 4
      for (int j = 0; j < CK; ++j) {
        const float pj = sm.p[r][j];
#pragma unroll
        for (int i = 0; i < CPT; i += 4) {
          const float4 vv = *reinterpret_cast<const float4*>(&sm.v[j][CPT * kk + i]);
          acc[i] = __builtin_fmaf(pj, vv.x, acc[i]);
          acc[i + 1] = __builtin_fmaf(pj, vv.y, acc[i + 1]);
          acc[i + 2] = __builtin_fmaf(pj, vv.z, acc[i + 2]);
          acc[i + 3] = __builtin_fmaf(pj, vv.w, acc[i + 3]);
        }
      }
    }
  }

  // row sum over the 16 threads of the row, then write
#pragma unroll
  for (int sh = 8; sh >= 1; sh >>= 1) l += __shfl_xor(l, sh, 16);
  if (!row_ok) return;
  int64_t row = t * a.tile_q + r;
  if (a.q_rows) row = a.q_rows[b * a.lists * a.tile_q + row];
  if (row < 0 || row >= a.len_q) return;
  const int64_t orow = (b * a.heads_q + h) * a.len_q + row;
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const float val = acc[i] * inv;
    if constexpr (O_BF16)
      static_cast<uint16_t*>(a.o)[orow * D + CPT * kk + i] = f32_to_bf16_bits(val);
    else
      static_cast<float*>(a.o)[orow * D + CPT * kk + i] = val;
  }
  if (kk == 0) a.lse[orow] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
}

template <bool QB, bool OB>
hipError_t launch_d(const TileArgs& a, int d, hipStream_t s) {
  dim3 grid((unsigned)a.tiles);
  if (d == 64)
    attn_tile_kernel<QB, OB, 64><<<grid, NT, 0, s>>>(a);
  else
    attn_tile_kernel<QB, OB, 128><<<grid, NT, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

bool attn_tile_supported(const basa_attn_desc* d) {
  return d->tile_q >= 2 && d->tile_q <= MAXR && d->batch * d->heads_q * d->lists < (1ll << 31);
}

hipError_t launch_attn_tile(const basa_attn_desc* d, const void* q, int q_dtype, void* o,
                            int o_dtype, float* lse, hipStream_t s) {
  TileArgs a = {};
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
  a.tiles = d->batch * d->heads_q * d->lists;
  a.heads_q = (int)d->heads_q;
  a.heads_kv = (int)d->heads_kv;
  a.group = (int)(d->heads_q / d->heads_kv);
  a.tile_q = d->tile_q;
  a.block_k = d->block_k;
  a.scale_log2 = (float)(d->scale * 1.4426950408889634);
  if (a.tiles == 0) return hipSuccess;
  const int dd = (int)d->head_dim;
  const bool qb = q_dtype == BASA_BF16, ob = o_dtype == BASA_BF16;
  if (qb) return ob ? launch_d<true, true>(a, dd, s) : launch_d<true, false>(a, dd, s);
  return ob ? launch_d<false, true>(a, dd, s) : launch_d<false, false>(a, dd, s);
}

}  // namespace basa
