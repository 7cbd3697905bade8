// Attention of 16-row query tiles over listed 16-key blocks on bf16 MFMA: the
// log-linear forward (16-token query tiles, 16-token fine blocks plus float32
// coarse tables with a level bias) and the LoSA in-block attention.
//
// BA-Att section 2: attention restricted to the listed key blocks, Eq. 1's
// softmax over them; the log-linear README's coarse levels enter as more key
// segments with an additive logit bias per level.  Online softmax per 16-key
// block.
//
// One wave computes one tile; a workgroup holds four waves (eight for the
// log-linear levels).  Float32 segments whose list row is shared by the
// workgroup's tiles are staged once per
// workgroup (barrier-synchronised); everything else each wave walks alone.  Per 16-key block the wave forms S^T = K Q^T with
// v_mfma_f32_16x16x16bf16_1k: lane l holds the logits of query row l%16 for
// keys 4(l/16) .. +3, which is exactly the B operand (P^T) of the next
// O^T += V^T P^T; V^T comes from the wave's LDS area through the transposing
// ds_read_b64_tr_b16.  The channel order inside each MFMA k-step is permuted
// so that every lane reads one contiguous run of head_dim/4 channels of its
// key (and of its query row): the dot product is a sum over channels, so any
// permutation applied to both operands gives the same logits.
//
// float32 tables (the coarse means) are split into bf16 pairs, x = hi + lo
// with hi = bf16(x), lo = bf16(x - hi): two MFMAs per product, relative error
// about 2^-16 (the queries are bf16 and exact).  P is rounded to bf16 for the
// P.V product, as in the other MFMA kernel; the row sums use the float32 P.
// The next block's key and value rows are loaded while the current one is
// reduced.
#include "common.h"

namespace basa {
namespace {

constexpr int NW = 4;          // waves (tiles) per workgroup (8 for the log-linear coarse levels)
constexpr float kLazy = 8.0f;  // log2 headroom before the max is raised

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

struct T16Seg {
  const int32_t* idx;
  const void* k;
  const void* v;
  int64_t len, rows;
  int count, stride, shift, bf16;
  float bias_log2;
};

struct T16Args {
  T16Seg seg[BASA_MAX_SEGMENTS];
  int n_seg;
  const uint16_t* q;
  void* o;
  float* lse;
  const int32_t* q_rows;
  int64_t len_q, lists, tiles;
  int heads_q, heads_kv, group;
  int share;  // the workgroup's tiles are consecutive tiles of one (batch, head) (lists % tiles per workgroup == 0)
  float scale_log2;
};

// head_dim/4 channels of one key row as raw 32-bit words (bf16 pairs or
// float32), held as one vector value so it stays in registers
template <int D, bool BF>
struct Raw {
  static constexpr int CPL = D / 4;
  static constexpr int N = BF ? CPL / 2 : CPL;  // 32-bit words
  typedef uint32_t vec __attribute__((ext_vector_type(N)));
  vec v;
  __device__ __forceinline__ void load(const void* base, int64_t elem) {
    v = *reinterpret_cast<const vec*>(BF ? (const void*)(static_cast<const uint16_t*>(base) + elem)
                                         : (const void*)(static_cast<const float*>(base) + elem));
  }
  __device__ __forceinline__ float f(int c) const { return __uint_as_float(v[c]); }  // float32 tables
  // bf16 tables: channels 4s .. 4s+3 of the run as an MFMA operand
  __device__ __forceinline__ v4i16 b4(int s) const {
    return __builtin_bit_cast(v4i16, make_uint2(v[2 * s], v[2 * s + 1]));
  }
  __device__ __forceinline__ uint4 word4(int i) const {  // 16 bytes i
    return make_uint4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  }
};

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return (uint32_t)f32_to_bf16_bits(a) | ((uint32_t)f32_to_bf16_bits(b) << 16);
}

// float32 -> (hi, lo) bf16 pair of 4 channels
__device__ __forceinline__ void split4(float x0, float x1, float x2, float x3, uint2& hi, uint2& lo) {
  const uint16_t h0 = f32_to_bf16_bits(x0), h1 = f32_to_bf16_bits(x1);
  const uint16_t h2 = f32_to_bf16_bits(x2), h3 = f32_to_bf16_bits(x3);
  hi = make_uint2((uint32_t)h0 | ((uint32_t)h1 << 16), (uint32_t)h2 | ((uint32_t)h3 << 16));
  lo = make_uint2(pack2(x0 - bf16_bits_to_f32(h0), x1 - bf16_bits_to_f32(h1)),
                  pack2(x2 - bf16_bits_to_f32(h2), x3 - bf16_bits_to_f32(h3)));
}

template <int D>
struct T16State {
  f32x4 o[D / 16];  // O^T: channel block cb, lane l: channels 16cb + 4(l/16) .. +3 of row l%16
  float m, l;
};

// LDS area of one wave: the value rows of one block, key-major, hi and lo
// halves, rows padded by 16 bytes (row stride D*2+16)
template <int D>
struct T16Lds {
  static constexpr int STRIDE = D * 2 + 16;
  static constexpr int HALF = 16 * STRIDE;
  static constexpr int BYTES = 2 * HALF;
};

// Online softmax of one block's logits (lane l: query row l%16, keys
// 4(l/16)+i) and O^T += V^T P^T with V^T from an LDS value area (the hi half,
// and with LO the lo half at +HALF).  kvalid: this lane's key (l%16) exists.
template <int D, bool LO>
__device__ __forceinline__ void t16_softmax_pv(const f32x4& s, bool kvalid, float scale_log2,
                                               float bias_log2, const uint8_t* varea,
                                               T16State<D>& st) {
  const int lane = threadIdx.x & 63;
  const int G = lane >> 4;
  // keys 4G+i of this lane's query row; a key that does not exist has logit -inf
  // (the lane's own kvalid flag is for key l%16: fetch the flags of keys 4G+i)
  float z[4];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool ok = __shfl(kvalid ? 1 : 0, 4 * G + i) != 0;
    z[i] = ok ? s[i] * scale_log2 + bias_log2 : -INFINITY;
    mx = fmaxf(mx, z[i]);
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  if (__ballot(mx > st.m + kLazy) != 0) {  // some row raised its max (wave-uniform branch)
    const float m_new = mx > st.m + kLazy ? mx : st.m;
    const float alpha = st.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st.m - m_new);
    st.l *= alpha;
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) st.o[cb] *= alpha;
    st.m = m_new;
  }
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p[i] = z[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(z[i] - st.m);
    st.l += p[i];
  }
  const v4i16 pb = __builtin_bit_cast(v4i16, make_uint2(pack2(p[0], p[1]), pack2(p[2], p[3])));
  // lane r of group G reads value row 4G + r/4, channels 16cb + 4(r%4) .. +3
  const int g = lane & 15;
  const uint8_t* vb = varea + (4 * G + (g >> 2)) * T16Lds<D>::STRIDE + 8 * (g & 3);
#pragma unroll
  for (int cb = 0; cb < D / 16; ++cb) {
    const v4i16 vhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vb + 32 * cb));
    st.o[cb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vhi, pb, st.o[cb], 0, 0, 0);
    if constexpr (LO) {
      const v4i16 vlo =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vb + T16Lds<D>::HALF + 32 * cb));
      st.o[cb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vlo, pb, st.o[cb], 0, 0, 0);
    }
  }
}

// Key or value rows of one block (this lane: row l%16, its channel run) into an
// LDS area, as bf16 (hi half; float32 rows also get the lo half at +HALF).
template <int D, bool BF>
__device__ __forceinline__ void t16_store_rows(const Raw<D, BF>& raw, uint8_t* area) {
  constexpr int CPL = D / 4;
  const int lane = threadIdx.x & 63;
  uint8_t* rowp = area + (lane & 15) * T16Lds<D>::STRIDE + CPL * (lane >> 4) * 2;
  if constexpr (BF) {
#pragma unroll
    for (int i = 0; i < Raw<D, BF>::N / 4; ++i) *reinterpret_cast<uint4*>(rowp + 16 * i) = raw.word4(i);
  } else {
#pragma unroll
    for (int s = 0; s < CPL / 4; ++s) {
      uint2 hi, lo;
      split4(raw.f(4 * s), raw.f(4 * s + 1), raw.f(4 * s + 2), raw.f(4 * s + 3), hi, lo);
      *reinterpret_cast<uint2*>(rowp + 8 * s) = hi;
      *reinterpret_cast<uint2*>(rowp + T16Lds<D>::HALF + 8 * s) = lo;
    }
  }
}

// One 16-key block of this wave's own list: logits from the key rows in
// registers, values through the wave's LDS area.
template <int D, bool BF>
__device__ __forceinline__ void t16_block(const Raw<D, BF>& kraw, const Raw<D, BF>& vraw, bool kvalid,
                                          const v4i16* qb, float scale_log2, float bias_log2,
                                          uint8_t* lds, T16State<D>& st) {
  constexpr int STEPS = D / 16;
  t16_store_rows<D, BF>(vraw, lds);
  // S^T = K Q^T (16 keys x 16 query rows)
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st_ = 0; st_ < STEPS; ++st_) {
    if constexpr (BF) {
      s = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kraw.b4(st_), qb[st_], s, 0, 0, 0);
    } else {
      uint2 hi, lo;
      split4(kraw.f(4 * st_), kraw.f(4 * st_ + 1), kraw.f(4 * st_ + 2), kraw.f(4 * st_ + 3), hi, lo);
      s = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(v4i16, hi), qb[st_], s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(v4i16, lo), qb[st_], s, 0, 0, 0);
    }
  }
  t16_softmax_pv<D, !BF>(s, kvalid, scale_log2, bias_log2, lds, st);
}

// This lane's key (l%16 of list entry j) relative to the head, or -1.
__device__ __forceinline__ int64_t t16_row(const int32_t* lst, int j, int64_t len) {
  const int32_t blk = lst[j];
  if (blk < 0) return -1;
  const int64_t key = (int64_t)blk * 16 + (threadIdx.x & 15);
  return key < len ? key : -1;
}

// All blocks of one segment for this wave's tile (16-key blocks).  The next
// block's rows are loaded before the current block is reduced; the loop is
// unrolled by two so the two register sets swap roles without copies.
template <int D, bool BF>
__device__ __forceinline__ void t16_segment(float scale_log2, const T16Seg& sg, const int32_t* lst,
                                            int64_t head_row, const v4i16* qb, uint8_t* lds,
                                            T16State<D>& st) {
  constexpr int CPL = D / 4;
  const int ch0 = CPL * ((threadIdx.x & 63) >> 4);
  const int n = sg.count;
  if (n == 0) return;
  Raw<D, BF> k0, v0, k1, v1;
  int64_t r0 = t16_row(lst, 0, sg.len);
  {
    const int64_t r = head_row + (r0 >= 0 ? r0 : 0);
    k0.load(sg.k, r * D + ch0);
    v0.load(sg.v, r * D + ch0);
  }
  for (int j = 0; j < n; j += 2) {
    int64_t r1 = -1;
    if (j + 1 < n) {
      r1 = t16_row(lst, j + 1, sg.len);
      const int64_t r = head_row + (r1 >= 0 ? r1 : 0);
      k1.load(sg.k, r * D + ch0);
      v1.load(sg.v, r * D + ch0);
    }
    if (__ballot(r0 >= 0) != 0)  // blocks with no key at all (unused list slots) are skipped
      t16_block<D, BF>(k0, v0, r0 >= 0, qb, scale_log2, sg.bias_log2, lds, st);
    if (j + 1 >= n) break;
    if (j + 2 < n) {
      r0 = t16_row(lst, j + 2, sg.len);
      const int64_t r = head_row + (r0 >= 0 ? r0 : 0);
      k0.load(sg.k, r * D + ch0);
      v0.load(sg.v, r * D + ch0);
    }
    if (__ballot(r1 >= 0) != 0)
      t16_block<D, BF>(k1, v1, r1 >= 0, qb, scale_log2, sg.bias_log2, lds, st);
  }
}

// A float32 segment whose list row is the same for all NWT tiles of the
// workgroup (the log-linear coarse levels): the workgroup walks it together,
// NWT blocks per chunk.  Wave w loads block w of the chunk, splits it into bf16
// hi/lo and stores keys and values in slot w of the shared LDS area; after a
// barrier every wave reduces all NWT slots for its own rows.  Each coarse block
// is thus read and split once per workgroup instead of once per tile.  The
// next chunk's rows are loaded while the current chunk is reduced.
template <int D, int NWT>
struct T16Shared {
  static constexpr int SLOT = 4 * T16Lds<D>::HALF;  // keys hi, keys lo, values hi, values lo
  static constexpr int BYTES = NWT * SLOT;
};

template <int D, int NWT>
__device__ __forceinline__ void t16_shared_segment(float scale_log2, const T16Seg& sg,
                                                   const int32_t* lst, int64_t head_row,
                                                   const v4i16* qb, uint8_t* shared,
                                                   T16State<D>& st) {
  constexpr int CPL = D / 4;
  constexpr int HALF = T16Lds<D>::HALF;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ch0 = CPL * (lane >> 4);
  const int n = sg.count;
  Raw<D, false> kr, vr;
  {
    const int64_t rr = wave < n ? t16_row(lst, wave, sg.len) : -1;
    const int64_t r = head_row + (rr >= 0 ? rr : 0);
    kr.load(sg.k, r * D + ch0);
    vr.load(sg.v, r * D + ch0);
  }
  for (int c0 = 0; c0 < n; c0 += NWT) {
    uint8_t* slot = shared + wave * T16Shared<D, NWT>::SLOT;
    t16_store_rows<D, false>(kr, slot);
    t16_store_rows<D, false>(vr, slot + 2 * HALF);
    __syncthreads();
    if (c0 + NWT < n) {  // next chunk's rows
      const int j = c0 + NWT + wave;
      const int64_t rr = j < n ? t16_row(lst, j, sg.len) : -1;
      const int64_t r = head_row + (rr >= 0 ? rr : 0);
      kr.load(sg.k, r * D + ch0);
      vr.load(sg.v, r * D + ch0);
    }
    for (int b = 0; b < NWT; ++b) {
      const int j = c0 + b;
      if (j >= n) break;
      const int32_t blk = lst[j];
      if (blk < 0) continue;  // an unused list slot (wave-uniform)
      const bool kvalid = (int64_t)blk * 16 + (lane & 15) < sg.len;
      const uint8_t* ks = shared + b * T16Shared<D, NWT>::SLOT + (lane & 15) * T16Lds<D>::STRIDE + ch0 * 2;
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st_ = 0; st_ < CPL / 4; ++st_) {
        const v4i16 hi = *reinterpret_cast<const v4i16*>(ks + 8 * st_);
        const v4i16 lo = *reinterpret_cast<const v4i16*>(ks + HALF + 8 * st_);
        s = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(hi, qb[st_], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lo, qb[st_], s, 0, 0, 0);
      }
      t16_softmax_pv<D, true>(s, kvalid, scale_log2, sg.bias_log2,
                              shared + b * T16Shared<D, NWT>::SLOT + 2 * HALF, st);
    }
    __syncthreads();  // the slots are rewritten by the next chunk
  }
}

// F32: some segment has a float32 table (without it the float32 path, and its
// registers, are not compiled in).  NWT tiles (waves) per workgroup: 4, or 8
// when the float32 lists repeat over 8 consecutive tiles (the log-linear
// levels above the first: a level-2 block's 16 tiles share their level-1
// candidates), so that each coarse block is read and split once per 8 tiles;
// two such workgroups share a CU (74 KB of LDS each), so one waits on its
// loads while the other computes.  (The second launch bound is the minimum
// number of waves per SIMD: 4, i.e. at most 128 registers.)
template <bool O_BF16, int D, bool F32, int NWT>
__global__ __launch_bounds__(NWT * 64, (D == 64 || NWT == 8) ? 4 : 3) void attn_t16_kernel(T16Args a) {
  constexpr int CPL = D / 4;
  constexpr int SHARE_SHIFT = NWT == 8 ? 3 : 2;  // list rows with this shift repeat over the workgroup
  // per-wave areas; with float32 segments also the shared area, which they alias
  // (the shared segments are done, behind a barrier, before any per-wave area is used)
  constexpr int SMEM = (F32 && T16Shared<D, NWT>::BYTES > NWT * T16Lds<D>::BYTES)
                           ? T16Shared<D, NWT>::BYTES
                           : NWT * T16Lds<D>::BYTES;
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t tile = (int64_t)blockIdx.x * NWT + wave;
  // with a.share the tile count is a multiple of NWT, so no wave of a workgroup that
  // meets a barrier leaves here
  if (tile >= a.tiles) return;
  uint8_t* lds = smem + wave * T16Lds<D>::BYTES;
  const int64_t t = tile % a.lists;
  const int64_t bh = tile / a.lists;
  const int h = (int)(bh % a.heads_q);
  const int64_t b = bh / a.heads_q;
  const int hk = h / a.group;
  const int G = lane >> 4;

  // this lane's query row (l%16) and its channel run CPL*G .. +CPL-1, as MFMA B operands
  int64_t qrow = t * 16 + (lane & 15);
  if (a.q_rows) qrow = a.q_rows[b * a.lists * 16 + t * 16 + (lane & 15)];
  const bool q_ok = qrow >= 0 && qrow < a.len_q;
  v4i16 qb[CPL / 4];
  {
    Raw<D, true> qr;
    if (q_ok)
      qr.load(a.q, ((b * a.heads_q + h) * a.len_q + qrow) * D + CPL * G);
    else
      qr.v = 0;
#pragma unroll
    for (int s = 0; s < CPL / 4; ++s) qb[s] = qr.b4(s);
  }

  T16State<D> st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int cb = 0; cb < D / 16; ++cb) st.o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // float32 segments shared by the workgroup's tiles first (every wave takes part:
  // a.share guarantees that the workgroup holds NWT tiles of one (batch, head))
  if constexpr (F32) {
    if (a.share) {
      for (int si = 0; si < a.n_seg; ++si) {
        const T16Seg& sg = a.seg[si];
        if (sg.bf16 || sg.shift < SHARE_SHIFT || sg.count == 0 || sg.len == 0) continue;
        const int32_t* lst = sg.idx + ((b * a.heads_q + h) * sg.rows + (t >> sg.shift)) * sg.stride;
        t16_shared_segment<D, NWT>(a.scale_log2, sg, lst, (b * a.heads_kv + hk) * sg.len, qb, smem, st);
      }
    }
  }

  for (int si = 0; si < a.n_seg; ++si) {
    const T16Seg& sg = a.seg[si];
    if (sg.count == 0 || sg.len == 0) continue;
    if (F32 && a.share && !sg.bf16 && sg.shift >= SHARE_SHIFT) continue;  // done above
    const int32_t* lst = sg.idx + ((b * a.heads_q + h) * sg.rows + (t >> sg.shift)) * sg.stride;
    const int64_t head_row = (b * a.heads_kv + hk) * sg.len;
    if (!F32 || sg.bf16)
      t16_segment<D, true>(a.scale_log2, sg, lst, head_row, qb, lds, st);
    else if constexpr (F32)
      t16_segment<D, false>(a.scale_log2, sg, lst, head_row, qb, lds, st);
  }

  // row sums: the four lanes of a query row hold disjoint key subsets
  float l = st.l;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (!q_ok) return;
  const int64_t orow = (b * a.heads_q + h) * a.len_q + qrow;
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int cb = 0; cb < D / 16; ++cb) {
    const int ch = 16 * cb + 4 * G;
    const float v0 = st.o[cb][0] * inv, v1 = st.o[cb][1] * inv;
    const float v2 = st.o[cb][2] * inv, v3 = st.o[cb][3] * inv;
    if constexpr (O_BF16) {
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.o) + orow * D + ch) =
          make_uint2(pack2(v0, v1), pack2(v2, v3));
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(a.o) + orow * D + ch) = make_float4(v0, v1, v2, v3);
    }
  }
  if (G == 0) a.lse[orow] = l > 0.f ? (st.m + log2f(l)) * kLn2 : -INFINITY;
}

template <bool OB, bool F32>
hipError_t launch_t16(T16Args a, int d, hipStream_t s) {
  if constexpr (F32) {
    if (d == 64 && a.lists % 8 == 0) {  // 8 tiles per workgroup share the coarse lists
      a.share = 1;
      dim3 grid((unsigned)(a.tiles / 8));
      attn_t16_kernel<OB, 64, true, 8><<<grid, 8 * 64, 0, s>>>(a);
      return hipGetLastError();
    }
  }
  dim3 grid((unsigned)((a.tiles + NW - 1) / NW));
  if (d == 64)
    attn_t16_kernel<OB, 64, F32, NW><<<grid, NW * 64, 0, s>>>(a);
  else
    attn_t16_kernel<OB, 128, F32, NW><<<grid, NW * 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

bool attn_t16_supported(const basa_attn_desc* d, int q_dtype) {
  return q_dtype == BASA_BF16 && d->tile_q == 16 && d->block_k == 16 &&
         (d->head_dim == 64 || d->head_dim == 128) &&
         (d->batch * d->heads_q * d->lists + NW - 1) / NW < (1ll << 31);
}

hipError_t launch_attn_t16(const basa_attn_desc* d, const void* q, void* o, int o_dtype, float* lse,
                           hipStream_t s) {
  T16Args a = {};
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
  a.q = static_cast<const uint16_t*>(q);
  a.o = o;
  a.lse = lse;
  a.q_rows = d->q_rows;
  a.len_q = d->len_q;
  a.lists = d->lists;
  a.tiles = d->batch * d->heads_q * d->lists;
  a.heads_q = (int)d->heads_q;
  a.heads_kv = (int)d->heads_kv;
  a.group = (int)(d->heads_q / d->heads_kv);
  a.scale_log2 = (float)(d->scale * 1.4426950408889634);
  a.share = d->lists % NW == 0;
  if (a.tiles == 0) return hipSuccess;
  bool f32 = false;
  for (int i = 0; i < a.n_seg; ++i) f32 = f32 || !a.seg[i].bf16;
  const int dd = (int)d->head_dim;
  if (o_dtype == BASA_BF16)
    return f32 ? launch_t16<true, true>(a, dd, s) : launch_t16<true, false>(a, dd, s);
  return f32 ? launch_t16<false, true>(a, dd, s) : launch_t16<false, false>(a, dd, s);
}

}  // namespace basa
