// Attention of single query rows over listed key blocks (decode-shaped:
// one query row per list, many keys), for key blocks that are a multiple of
// 16 keys, head_dim 64 or 128, float32 or bf16 queries and key/value tables,
// up to four key segments with their own logit bias, a query row map and
// grouped key heads.  This is the LoSA step's sparse prefix attention: each
// active query token attends to the 16-token prefix blocks it selected and its
// (O, LSE) pair replaces the cached one (LoSA post, the cache of outputs and
// log-sum-exps per token).
//
// One workgroup of NW waves computes one row.  The waves split every segment's
// entries into NW contiguous shares.  A wave walks its share 16 keys at a
// time: four lanes own one key, each lane a quarter of the channels, so the
// 16 key rows of a step are read as 16 contiguous row segments (fully
// coalesced), the dot product is finished with two quad DPP swaps, and the
// value row is read with the same layout.  Each group of four lanes keeps its
// own online-softmax state (max m, sum l, unnormalised output of its channel
// quarter) over the keys it owns; the max is raised lazily, only when a logit
// exceeds it by more than 2^8 in linear scale, so most steps need no rescale.
// The next step's key and value rows are loaded while the current one is being
// reduced.  At the end the 16 states of a wave are merged with a butterfly and
// the NW wave states through LDS, with the max-shifted rule of basa_merge.
//
// Workgroup numbering: dispatch hands workgroups to the 8 XCDs round-robin, and
// the rows of one key head (query heads of a group x lists) are consecutive.
// Rows are cut into chunks of up to 64 consecutive rows and chunk c runs on XCD
// c % 8, so the rows of one key head share one L2 and a block that several of
// them keep is fetched once (the LoSA step: 20 rows per key head, 8 key heads,
// one XCD each).
#include "common.h"

namespace basa {
namespace {

constexpr int NW = 8;                 // waves per row (16: registers spill, 3x slower)
constexpr float kLazy = 8.0f;         // log2 headroom before the max is raised

struct RowSeg {
  const int32_t* idx;
  const void* k;
  const void* v;
  int64_t len, rows;
  int count, stride, shift, bf16;
  float bias_log2;
};

struct RowArgs {
  RowSeg seg[BASA_MAX_SEGMENTS];
  int n_seg;
  const void* q;
  void* o;
  float* lse;
  const int32_t* q_rows;
  int64_t len_q, lists, rows_total, chunk;
  int heads_q, heads_kv, group, block_k;
  float scale_log2;
};

// lane value of the partner in its quad: CTRL = 0xB1 swaps lanes 0<->1, 2<->3
// (quad_perm [1,0,3,2]); 0x4E swaps 0<->2, 1<->3 (quad_perm [2,3,0,1])
template <int CTRL>
__device__ __forceinline__ float dpp_quad(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// CPL consecutive channels of one key row, as raw 16-byte words
template <int CPL, bool BF>
struct RowPart {
  static constexpr int W = BF ? CPL / 8 : CPL / 4;  // uint4 words
  uint4 w[W];
  __device__ __forceinline__ void load(const void* base, int64_t elem) {
    const uint4* p = reinterpret_cast<const uint4*>(
        BF ? (const void*)(static_cast<const uint16_t*>(base) + elem)
           : (const void*)(static_cast<const float*>(base) + elem));
#pragma unroll
    for (int i = 0; i < W; ++i) w[i] = p[i];
  }
  __device__ __forceinline__ float get(int c) const {
    if constexpr (BF) {
      const uint4& u = w[c / 8];
      const int j = c % 8;
      const uint32_t x = j < 2 ? u.x : j < 4 ? u.y : j < 6 ? u.z : u.w;
      return (j & 1) ? __uint_as_float(x & 0xFFFF0000u) : __uint_as_float(x << 16);
    } else {
      const uint4& u = w[c / 4];
      const int j = c % 4;
      return __uint_as_float(j == 0 ? u.x : j == 1 ? u.y : j == 2 ? u.z : u.w);
    }
  }
};

template <int CPL>
struct RowState {
  float m, l;
  float o[CPL];
};

// One segment's share for this wave: entries [e0, e1) of the row's list.
template <int D, bool BF>
__device__ __forceinline__ void row_segment(const RowArgs& a, const RowSeg& sg, const int32_t* lst,
                                            int64_t head_row, int e0, int e1, const float* qv,
                                            RowState<D / 4>& st) {
  constexpr int CPL = D / 4;
  const int lane = threadIdx.x & 63;
  const int slot = lane >> 2;             // key of the 16-key step
  const int ch0 = (lane & 3) * CPL;       // first channel of this lane
  const int cpe = a.block_k / 16;         // steps per entry
  for (int eb = e0; eb < e1; eb += 64) {  // entries in passes of 64, one index per lane
    const int n_e = min(64, e1 - eb);
    const int my_blk = lane < n_e ? lst[eb + lane] : -1;
    const int n_steps = n_e * cpe;

    // key row of step s for this lane, or -1
    auto key_row = [&](int s) -> int64_t {
      const int blk = __builtin_amdgcn_readlane(my_blk, s / cpe);
      if (blk < 0) return -1;
      const int64_t key = (int64_t)blk * a.block_k + (s % cpe) * 16 + slot;
      return key < sg.len ? head_row + key : -1;
    };

    auto step = [&](const RowPart<CPL, BF>& kc, const RowPart<CPL, BF>& vc, int64_t row_c) {
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) dot = __builtin_fmaf(qv[c], kc.get(c), dot);
      dot += dpp_quad<0xB1>(dot);
      dot += dpp_quad<0x4E>(dot);
      const float z = row_c >= 0 ? dot * a.scale_log2 + sg.bias_log2 : -INFINITY;
      if (__builtin_expect(__ballot(z > st.m + kLazy) != 0, 0)) {
        const float m_new = z > st.m + kLazy ? z : st.m;
        const float alpha = st.m == -INFINITY ? 0.f : exp2f(st.m - m_new);
        st.l *= alpha;
#pragma unroll
        for (int c = 0; c < CPL; ++c) st.o[c] *= alpha;
        st.m = m_new;
      }
      const float p = z == -INFINITY ? 0.f : exp2f(z - st.m);
      st.l += p;
#pragma unroll
      for (int c = 0; c < CPL; ++c) st.o[c] = __builtin_fmaf(p, vc.get(c), st.o[c]);
    };

    if constexpr (BF) {
      // bf16 rows: the next step's rows are loaded before this step is reduced
      RowPart<CPL, BF> kc, vc, kn, vn;
      int64_t row_c = key_row(0);
      {
        const int64_t r = row_c >= 0 ? row_c : head_row;
        kc.load(sg.k, r * D + ch0);
        vc.load(sg.v, r * D + ch0);
      }
      for (int s = 0; s < n_steps; ++s) {
        int64_t row_n = -1;
        if (s + 1 < n_steps) {
          row_n = key_row(s + 1);
          const int64_t r = row_n >= 0 ? row_n : head_row;
          kn.load(sg.k, r * D + ch0);
          vn.load(sg.v, r * D + ch0);
        }
        step(kc, vc, row_c);
        if (s + 1 < n_steps) {
          kc = kn;
          vc = vn;
          row_c = row_n;
        }
      }
    } else {
      // float32 rows hold twice the registers: one step at a time
      for (int s = 0; s < n_steps; ++s) {
        RowPart<CPL, BF> kc, vc;
        const int64_t row_c = key_row(s);
        const int64_t r = row_c >= 0 ? row_c : head_row;
        kc.load(sg.k, r * D + ch0);
        vc.load(sg.v, r * D + ch0);
        step(kc, vc, row_c);
      }
    }
  }
}

template <bool Q_BF16, bool O_BF16, int D>
__global__ __launch_bounds__(NW * 64) void attn_row_kernel(RowArgs a) {
  constexpr int CPL = D / 4;
  __shared__ float part_m[NW], part_l[NW];
  __shared__ float part_o[NW][D];

  const int64_t w = (int64_t)blockIdx.x + (int64_t)blockIdx.y * gridDim.x;
  const int64_t unit = (w % 8 + 8 * (w / 8 / a.chunk)) * a.chunk + (w / 8) % a.chunk;
  if (unit >= a.rows_total) return;  // the last round of chunks is padded to all 8 XCDs
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t t = unit % a.lists;
  const int64_t bh = unit / a.lists;
  const int h = (int)(bh % a.heads_q);
  const int64_t b = bh / a.heads_q;
  const int hk = h / a.group;
  int64_t row = t;
  if (a.q_rows) row = a.q_rows[b * a.lists + t];
  if (row < 0 || row >= a.len_q) return;  // a row map entry outside q: nothing to write
  const int64_t qoff = ((b * a.heads_q + h) * a.len_q + row) * D;
  const int ch0 = (lane & 3) * CPL;

  float qv[CPL];
#pragma unroll
  for (int c = 0; c < CPL; c += 8) {
    if constexpr (Q_BF16)
      Vec8<uint16_t>::load(static_cast<const uint16_t*>(a.q) + qoff + ch0 + c, qv + c);
    else
      Vec8<float>::load(static_cast<const float*>(a.q) + qoff + ch0 + c, qv + c);
  }

  RowState<CPL> st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) st.o[c] = 0.f;

  for (int si = 0; si < a.n_seg; ++si) {
    const RowSeg& sg = a.seg[si];
    if (sg.count == 0 || sg.len == 0) continue;
    const int32_t* lst = sg.idx + ((b * a.heads_q + h) * sg.rows + (t >> sg.shift)) * sg.stride;
    const int64_t head_row = (b * a.heads_kv + hk) * sg.len;
    const int e0 = (int)(((int64_t)sg.count * wave) / NW);
    const int e1 = (int)(((int64_t)sg.count * (wave + 1)) / NW);
    if (sg.bf16)
      row_segment<D, true>(a, sg, lst, head_row, e0, e1, qv, st);
    else
      row_segment<D, false>(a, sg, lst, head_row, e0, e1, qv, st);
  }

  // merge the 16 key-slot states of the wave (lanes that share lane & 3)
#pragma unroll
  for (int sh = 4; sh <= 32; sh <<= 1) {
    const float m_o = __shfl_xor(st.m, sh);
    const float l_o = __shfl_xor(st.l, sh);
    const float mm = fmaxf(st.m, m_o);
    const float sa = st.m == -INFINITY ? 0.f : exp2f(st.m - mm);
    const float sb = m_o == -INFINITY ? 0.f : exp2f(m_o - mm);
    st.l = st.l * sa + l_o * sb;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const float o_o = __shfl_xor(st.o[c], sh);
      st.o[c] = st.o[c] * sa + o_o * sb;
    }
    st.m = mm;
  }
  if (lane < 4) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) part_o[wave][ch0 + c] = st.o[c];
  }
  if (lane == 0) {
    part_m[wave] = st.m;
    part_l[wave] = st.l;
  }
  __syncthreads();

  float mm = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) mm = fmaxf(mm, part_m[w]);
  float wsc[NW];
  float ltot = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    wsc[w] = part_m[w] == -INFINITY ? 0.f : exp2f(part_m[w] - mm);
    ltot += part_l[w] * wsc[w];
  }
  const int64_t ooff = (b * a.heads_q + h) * a.len_q + row;
  for (int c = threadIdx.x; c < D; c += NW * 64) {
    float val = 0.f;
    if (ltot > 0.f) {
#pragma unroll
      for (int w = 0; w < NW; ++w) val += part_o[w][c] * wsc[w];
      val /= ltot;
    }
    if constexpr (O_BF16)
      static_cast<uint16_t*>(a.o)[ooff * D + c] = f32_to_bf16_bits(val);
    else
      static_cast<float*>(a.o)[ooff * D + c] = val;
  }
  if (threadIdx.x == 0) a.lse[ooff] = ltot > 0.f ? (mm + log2f(ltot)) * kLn2 : -INFINITY;
}

template <bool QB, bool OB>
hipError_t launch_rd(const RowArgs& a, int d, dim3 grid, hipStream_t s) {
  if (d == 64)
    attn_row_kernel<QB, OB, 64><<<grid, NW * 64, 0, s>>>(a);
  else
    attn_row_kernel<QB, OB, 128><<<grid, NW * 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

bool attn_row_supported(const basa_attn_desc* d) {
  return d->tile_q == 1 && d->block_k % 16 == 0 && (d->head_dim == 64 || d->head_dim == 128);
}

hipError_t launch_attn_row(const basa_attn_desc* d, const void* q, int q_dtype, void* o,
                           int o_dtype, float* lse, hipStream_t s) {
  RowArgs a = {};
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
  a.block_k = d->block_k;
  a.scale_log2 = (float)(d->scale * 1.4426950408889634);
  a.rows_total = d->batch * d->heads_q * d->lists;
  if (a.rows_total == 0) return hipSuccess;
  const int64_t per_kv = a.group * a.lists;  // consecutive rows of one key head
  a.chunk = per_kv < 64 ? per_kv : 64;
  const int64_t n_chunks = (a.rows_total + a.chunk - 1) / a.chunk;
  const int64_t wgs = (n_chunks + 7) / 8 * 8 * a.chunk;  // chunk c on XCD c % 8
  const int64_t gx = wgs < 65536 ? wgs : 65536;
  const int64_t gy = (wgs + gx - 1) / gx;
  dim3 grid((unsigned)gx, (unsigned)gy);
  const int dd = (int)d->head_dim;
  const bool qb = q_dtype == BASA_BF16, ob = o_dtype == BASA_BF16;
  if (qb) return ob ? launch_rd<true, true>(a, dd, grid, s) : launch_rd<true, false>(a, dd, grid, s);
  return ob ? launch_rd<false, true>(a, dd, grid, s) : launch_rd<false, false>(a, dd, grid, s);
}

}  // namespace basa
