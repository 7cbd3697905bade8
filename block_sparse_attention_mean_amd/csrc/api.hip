// C ABI of libbasa: host-side argument checks, then dispatch to the kernels.
// Every check runs before any HIP call, so an invalid request enqueues nothing
// and touches no device state.
#include <climits>
#include <cmath>

#include "common.h"

namespace {

constexpr int kVersion = 100;  // 0.1.0

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool is_pow2_dim(int64_t d, int64_t lo, int64_t hi) {
  return d >= lo && d <= hi && (d & (d - 1)) == 0;
}

int from_hip(hipError_t e) { return e == hipSuccess ? BASA_OK : BASA_E_LAUNCH; }

}  // namespace

extern "C" {

const char* basa_status_string(int status) {
  switch (status) {
    case BASA_OK: return "ok";
    case BASA_E_NULLPTR: return "required pointer is NULL";
    case BASA_E_SHAPE: return "inconsistent or out-of-range sizes";
    case BASA_E_DTYPE: return "unsupported element type";
    case BASA_E_ALIGN: return "pointer not 16-byte aligned";
    case BASA_E_UNSUPPORTED: return "request not implemented by the kernels";
    case BASA_E_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int basa_version(void) { return kVersion; }

int basa_pool(const void* x, int x_dtype, int64_t outer, int64_t len, int64_t head_dim,
              int64_t block, double* mean_rows, double* mean_cols, void* mean_copy,
              int copy_dtype, void* stream) {
  try {
    if (outer < 0 || len < 0 || block < 1 || head_dim < 8 || head_dim > 512 || head_dim % 8 != 0)
      return BASA_E_SHAPE;
    if (len % block != 0) return BASA_E_SHAPE;
    if (x_dtype != BASA_F32 && x_dtype != BASA_BF16 && x_dtype != BASA_F64) return BASA_E_DTYPE;
    if (mean_copy && copy_dtype != BASA_F32 && copy_dtype != BASA_BF16) return BASA_E_DTYPE;
    if (outer * len == 0) return BASA_OK;
    if (!x || (!mean_rows && !mean_cols && !mean_copy)) return BASA_E_NULLPTR;
    if (!aligned16(x) || !aligned16(mean_rows) || !aligned16(mean_cols) || !aligned16(mean_copy))
      return BASA_E_ALIGN;
    return from_hip(basa::launch_pool(x, x_dtype, outer, len, head_dim, block, mean_rows,
                                      mean_cols, mean_copy, copy_dtype,
                                      static_cast<hipStream_t>(stream)));
  } catch (...) {
    return BASA_E_LAUNCH;
  }
}

int basa_pool_pyramid(const basa_pyramid_tensor* tensors, int n_tensors, int x_dtype,
                      int64_t outer, int64_t len, int64_t head_dim, int64_t block, int levels,
                      int copy_dtype, void* stream) {
  try {
    if (!tensors) return BASA_E_NULLPTR;
    if (n_tensors < 1 || n_tensors > BASA_PYRAMID_MAX_TENSORS) return BASA_E_SHAPE;
    if (levels < 1 || levels > BASA_PYRAMID_MAX_LEVELS) return BASA_E_SHAPE;
    if (outer < 0 || len < 0 || block < 2 || block > 32) return BASA_E_SHAPE;
    if (head_dim < 8 || head_dim > 512 || head_dim % 8 != 0 || block * head_dim > 4096)
      return BASA_E_SHAPE;
    int64_t span = 1;
    for (int l = 0; l < levels; ++l) span *= block;
    if (len % span != 0) return BASA_E_SHAPE;
    if (x_dtype != BASA_F32 && x_dtype != BASA_BF16 && x_dtype != BASA_F64) return BASA_E_DTYPE;
    bool any_copy = false;
    for (int i = 0; i < n_tensors; ++i)
      for (int l = 0; l < levels; ++l) any_copy = any_copy || tensors[i].level[l].mean_copy;
    if (any_copy && copy_dtype != BASA_F32 && copy_dtype != BASA_BF16) return BASA_E_DTYPE;
    if (outer * len == 0) return BASA_OK;
    for (int i = 0; i < n_tensors; ++i) {
      const basa_pyramid_tensor& t = tensors[i];
      if (!t.x) return BASA_E_NULLPTR;
      if (!aligned16(t.x)) return BASA_E_ALIGN;
      for (int l = 0; l < levels; ++l) {
        const basa_pyramid_level& v = t.level[l];
        if (!v.mean_rows && !v.mean_cols && !v.mean_copy) return BASA_E_NULLPTR;
        if (l >= 1 && l + 1 < levels && !v.mean_rows) return BASA_E_NULLPTR;  // read by level l+2
        if (!aligned16(v.mean_rows) || !aligned16(v.mean_cols) || !aligned16(v.mean_copy))
          return BASA_E_ALIGN;
      }
    }
    return from_hip(basa::launch_pool_pyramid(tensors, n_tensors, x_dtype, outer, len, head_dim,
                                              block, levels, copy_dtype,
                                              static_cast<hipStream_t>(stream)));
  } catch (...) {
    return BASA_E_LAUNCH;
  }
}

int basa_pool_moments(const void* x, int x_dtype, int64_t outer, int64_t len, int64_t head_dim,
                      int64_t block, int role, double scale, double beta, double* out,
                      void* stream) {
  try {
    if (outer < 0 || len < 0 || block < 1 || len % block != 0) return BASA_E_SHAPE;
    if (head_dim < 8 || head_dim > 168 || head_dim % 8 != 0) return BASA_E_SHAPE;
    if (!std::isfinite(scale) || !std::isfinite(beta)) return BASA_E_SHAPE;
    if (x_dtype != BASA_F32 && x_dtype != BASA_BF16 && x_dtype != BASA_F64) return BASA_E_DTYPE;
    if (role != BASA_MOMENTS_QUERY && role != BASA_MOMENTS_KEY) return BASA_E_UNSUPPORTED;
    if (outer * len == 0) return BASA_OK;
    if (!x || !out) return BASA_E_NULLPTR;
    if (!aligned16(x) || !aligned16(out)) return BASA_E_ALIGN;
    return from_hip(basa::launch_moments(x, x_dtype, outer, len, head_dim, block, role, scale, beta,
                                         out, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return BASA_E_LAUNCH;
  }
}

int basa_select(const basa_select_desc* d, const void* q, const void* k, int dtype, int32_t* idx,
                void* stream) {
  try {
    if (!d) return BASA_E_NULLPTR;
    if (d->batch < 0 || d->heads_q < 1 || d->q_len < 0 || d->topk < 1) return BASA_E_SHAPE;
    if (d->head_dim < 8 || d->head_dim > 512 || d->head_dim % 8 != 0) return BASA_E_SHAPE;
    if (d->mode == BASA_SELECT_CHANGE) {
      if (dtype != BASA_F32 && dtype != BASA_BF16 && dtype != BASA_F64) return BASA_E_DTYPE;
      if (d->q_len > 1024 || d->topk > d->q_len) return BASA_E_SHAPE;
      if (d->batch == 0) return BASA_OK;
      if (!q || !k || !idx) return BASA_E_NULLPTR;
      if (!aligned16(q) || !aligned16(k)) return BASA_E_ALIGN;
      return from_hip(basa::launch_select_change(d, q, k, dtype, idx,
                                                 static_cast<hipStream_t>(stream)));
    }
    if (d->mode != BASA_SELECT_BLOCKS) return BASA_E_UNSUPPORTED;
    if (dtype != BASA_F64) return BASA_E_DTYPE;
    if (d->heads_kv < 1 || d->heads_q % d->heads_kv != 0) return BASA_E_SHAPE;
    if (d->rows < 0 || d->keys < 1 || d->keys > 4096) return BASA_E_SHAPE;
    if (!(d->scale > 0.0) || !std::isfinite(d->scale)) return BASA_E_SHAPE;
    if (!d->q_rows && d->rows != d->q_len) return BASA_E_SHAPE;
    int64_t n_cand = d->keys;
    if (d->parent) {
      if (d->q_rows) return BASA_E_UNSUPPORTED;
      if (d->parent_k < 1 || d->fanout < 1) return BASA_E_SHAPE;
      n_cand = (int64_t)d->parent_k * d->fanout;
      if (n_cand > 4096 || d->rows % d->fanout != 0 || d->keys % d->fanout != 0)
        return BASA_E_SHAPE;
    }
    if (d->topk > n_cand) return BASA_E_SHAPE;
    if (d->batch == 0 || d->rows == 0) return BASA_OK;
    if (!q || !k || !idx) return BASA_E_NULLPTR;
    if (!aligned16(q) || !aligned16(k)) return BASA_E_ALIGN;
    return from_hip(basa::launch_select_blocks(d, static_cast<const double*>(q),
                                               static_cast<const double*>(k), idx,
                                               static_cast<hipStream_t>(stream)));
  } catch (...) {
    return BASA_E_LAUNCH;
  }
}

int basa_pool_select(const basa_select_desc* d, const void* q, const void* k, int dtype,
                     int64_t block, double* qbar, double* kbar_t, int32_t* idx, void* stream) {
  try {
    if (!d) return BASA_E_NULLPTR;
    if (d->mode != BASA_SELECT_BLOCKS || d->q_rows || d->parent) return BASA_E_UNSUPPORTED;
    if (dtype != BASA_F32 && dtype != BASA_BF16 && dtype != BASA_F64) return BASA_E_DTYPE;
    if (block < 1 || d->batch < 0 || d->heads_q < 1 || d->q_len < 0 || d->topk < 1)
      return BASA_E_SHAPE;
    if (d->head_dim < 8 || d->head_dim > 512 || d->head_dim % 8 != 0) return BASA_E_SHAPE;
    if (d->heads_kv < 1 || d->heads_q % d->heads_kv != 0) return BASA_E_SHAPE;
    if (d->rows != d->q_len || d->keys < 1 || d->keys > 4096 || d->topk > d->keys) return BASA_E_SHAPE;
    if (!(d->scale > 0.0) || !std::isfinite(d->scale)) return BASA_E_SHAPE;
    if (d->q_len > INT64_MAX / block || d->keys > INT64_MAX / block) return BASA_E_SHAPE;
    if (d->batch == 0 || d->q_len == 0) return BASA_OK;
    if (!q || !k || !qbar || !kbar_t || !idx) return BASA_E_NULLPTR;
    if (!aligned16(q) || !aligned16(k) || !aligned16(qbar) || !aligned16(kbar_t)) return BASA_E_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // the three steps as separate launches on the stream
    hipError_t e = basa::launch_pool(q, dtype, d->batch * d->heads_q, d->q_len * block, d->head_dim,
                                     block, qbar, nullptr, nullptr, BASA_F32, s);
    if (e != hipSuccess) return BASA_E_LAUNCH;
    e = basa::launch_pool(k, dtype, d->batch * d->heads_kv, d->keys * block, d->head_dim, block,
                          nullptr, kbar_t, nullptr, BASA_F32, s);
    if (e != hipSuccess) return BASA_E_LAUNCH;
    return from_hip(basa::launch_select_blocks(d, qbar, kbar_t, idx, s));
  } catch (...) {
    return BASA_E_LAUNCH;
  }
}

int basa_pool_select_workspace(const basa_select_desc* d, int64_t* bytes) {
  try {
    if (!d || !bytes) return BASA_E_NULLPTR;
    *bytes = basa::pool_select_workspace_bytes(d);
    return BASA_OK;
  } catch (...) {
    return BASA_E_LAUNCH;
  }
}

int basa_select_workspace(const basa_select_desc* d, int64_t* bytes) {
  try {
    if (!d || !bytes) return BASA_E_NULLPTR;
    *bytes = basa::select_workspace_bytes(d);
    return BASA_OK;
  } catch (...) {
    return BASA_E_LAUNCH;
  }
}

int basa_attn(const basa_attn_desc* d, const void* q, int q_dtype, void* o, int o_dtype,
              float* lse, void* stream) {
  try {
    if (!d) return BASA_E_NULLPTR;
    if (q_dtype != BASA_F32 && q_dtype != BASA_BF16) return BASA_E_DTYPE;
    if (o_dtype != BASA_F32 && o_dtype != BASA_BF16) return BASA_E_DTYPE;
    if (d->batch < 0 || d->heads_q < 1 || d->heads_kv < 1 || d->heads_q % d->heads_kv != 0)
      return BASA_E_SHAPE;
    if (d->head_dim != 64 && d->head_dim != 128) return BASA_E_SHAPE;
    if (d->len_q < 0 || d->lists < 0) return BASA_E_SHAPE;
    if (d->tile_q < 1 || d->tile_q > 128 || d->block_k < 1 || d->block_k > 4096) return BASA_E_SHAPE;
    if (d->n_segments < 1 || d->n_segments > BASA_MAX_SEGMENTS) return BASA_E_SHAPE;
    if (!std::isfinite(d->scale)) return BASA_E_SHAPE;
    if (!d->q_rows && d->lists * d->tile_q != d->len_q) return BASA_E_SHAPE;
    for (int i = 0; i < d->n_segments; ++i) {
      const basa_kv_segment& g = d->seg[i];
      if (g.dtype != BASA_F32 && g.dtype != BASA_BF16) return BASA_E_DTYPE;
      if (g.count < 0 || g.count > 65536 || g.stride < g.count || g.len < 0) return BASA_E_SHAPE;
      if (g.shift < 0 || g.shift > 30 || !std::isfinite(g.bias)) return BASA_E_SHAPE;
      if (d->lists > 0 && g.count > 0 && g.rows < ((d->lists - 1) >> g.shift) + 1) return BASA_E_SHAPE;
    }
    if (d->batch == 0 || d->lists == 0) return BASA_OK;
    if (!q || !o || !lse) return BASA_E_NULLPTR;
    if (!aligned16(q) || !aligned16(o)) return BASA_E_ALIGN;
    for (int i = 0; i < d->n_segments; ++i) {
      const basa_kv_segment& g = d->seg[i];
      if (g.count == 0) continue;
      if (!g.idx || !g.k || !g.v) return BASA_E_NULLPTR;
      if (!aligned16(g.k) || !aligned16(g.v)) return BASA_E_ALIGN;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (basa::attn_mfma_supported(d, q_dtype, o_dtype)) {
      const int64_t need = basa::attn_mfma_workspace_bytes(d);
      int32_t* order = need > 0 && d->workspace && aligned16(d->workspace) && d->workspace_bytes >= need
                           ? static_cast<int32_t*>(d->workspace)
                           : nullptr;
      return from_hip(basa::launch_attn_mfma(d, q, o, o_dtype, lse, order, s));
    }
    if (d->workspace && aligned16(d->workspace) && basa::attn_union_supported(d, d->workspace_bytes))
      return from_hip(basa::launch_attn_union(d, q, q_dtype, o, o_dtype, lse, d->workspace, s));
    if (basa::attn_row_supported(d))
      return from_hip(basa::launch_attn_row(d, q, q_dtype, o, o_dtype, lse, s));
    if (basa::attn_t16_supported(d, q_dtype))
      return from_hip(basa::launch_attn_t16(d, q, o, o_dtype, lse, s));
    if (basa::attn_tile_supported(d))
      return from_hip(basa::launch_attn_tile(d, q, q_dtype, o, o_dtype, lse, s));
    return from_hip(basa::launch_attn_generic(d, q, q_dtype, o, o_dtype, lse, s));
  } catch (...) {
    return BASA_E_LAUNCH;
  }
}

int basa_attn_workspace(const basa_attn_desc* d, int64_t* bytes) {
  try {
    if (!d || !bytes) return BASA_E_NULLPTR;
    *bytes = basa::attn_union_workspace_bytes(d);
    if (*bytes == 0 && d->n_segments >= 1 && d->n_segments <= BASA_MAX_SEGMENTS &&
        basa::attn_mfma_supported(d, BASA_BF16, BASA_BF16))
      *bytes = basa::attn_mfma_workspace_bytes(d);
    return BASA_OK;
  } catch (...) {
    return BASA_E_LAUNCH;
  }
}

int basa_merge(int64_t rows, int64_t head_dim, const void* o_a, const float* lse_a,
               const void* o_b, const float* lse_b, int in_dtype, void* o, int o_dtype,
               float* lse, void* stream) {
  try {
    if (rows < 0 || !is_pow2_dim(head_dim, 8, 512)) return BASA_E_SHAPE;
    if (in_dtype != BASA_F32 && in_dtype != BASA_BF16) return BASA_E_DTYPE;
    if (o_dtype != BASA_F32 && o_dtype != BASA_BF16) return BASA_E_DTYPE;
    if (rows == 0) return BASA_OK;
    if (!o_a || !lse_a || !o_b || !lse_b || !o || !lse) return BASA_E_NULLPTR;
    if (!aligned16(o_a) || !aligned16(o_b) || !aligned16(o)) return BASA_E_ALIGN;
    if (o == o_a && o_dtype != in_dtype) return BASA_E_UNSUPPORTED;
    if (o == o_b && o_dtype != in_dtype) return BASA_E_UNSUPPORTED;
    return from_hip(basa::launch_merge(rows, head_dim, o_a, lse_a, o_b, lse_b, in_dtype, o,
                                       o_dtype, lse, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return BASA_E_LAUNCH;
  }
}

int basa_block_mass(const void* q, const void* k, int dtype, int64_t batch, int64_t heads_q,
                    int64_t heads_kv, int64_t len_q, int64_t len_k, int64_t head_dim, int64_t block,
                    double scale, double* mass, void* workspace, int64_t workspace_bytes,
                    void* stream) {
  try {
    if (batch < 0 || heads_q < 1 || heads_kv < 1 || heads_q % heads_kv != 0) return BASA_E_SHAPE;
    if (head_dim < 8 || head_dim > 128 || head_dim % 8 != 0) return BASA_E_SHAPE;
    if (block < 4 || block > 256 || (block & (block - 1)) != 0) return BASA_E_SHAPE;
    if (len_q < 0 || len_k < 0 || len_q % block != 0 || len_k % block != 0) return BASA_E_SHAPE;
    if (!(scale > 0.0) || !std::isfinite(scale)) return BASA_E_SHAPE;
    if (dtype != BASA_F32 && dtype != BASA_BF16) return BASA_E_DTYPE;
    if (batch == 0 || len_q == 0 || len_k == 0) return BASA_OK;
    if (!q || !k || !mass) return BASA_E_NULLPTR;
    if (!aligned16(q) || !aligned16(k) || !aligned16(mass)) return BASA_E_ALIGN;
    const int64_t need = basa::block_mass_workspace_bytes(batch, heads_q, len_q, len_k, head_dim, block);
    void* ws = need > 0 && workspace && aligned16(workspace) && workspace_bytes >= need ? workspace : nullptr;
    return from_hip(basa::launch_block_mass(q, k, dtype, batch, heads_q, heads_kv, len_q, len_k,
                                            head_dim, block, scale, mass, ws,
                                            static_cast<hipStream_t>(stream)));
  } catch (...) {
    return BASA_E_LAUNCH;
  }
}

int basa_block_mass_workspace(int64_t batch, int64_t heads_q, int64_t len_q, int64_t len_k,
                              int64_t head_dim, int64_t block, int64_t* bytes) {
  try {
    if (!bytes) return BASA_E_NULLPTR;
    *bytes = basa::block_mass_workspace_bytes(batch, heads_q, len_q, len_k, head_dim, block);
    return BASA_OK;
  } catch (...) {
    return BASA_E_LAUNCH;
  }
}

int basa_select_ranges(const double* scores, int64_t rows, int64_t n, int64_t split, int32_t k_lo,
                       int32_t k_hi, int32_t* idx, void* stream) {
  try {
    if (rows < 0 || n < 1 || n > 1024 || split < 0 || split > n) return BASA_E_SHAPE;
    if (k_lo < 0 || k_lo > split || k_hi < 0 || k_hi > n - split || k_lo + k_hi == 0)
      return BASA_E_SHAPE;
    if (rows == 0) return BASA_OK;
    if (!scores || !idx) return BASA_E_NULLPTR;
    if (!aligned16(scores) || !aligned16(idx)) return BASA_E_ALIGN;
    return from_hip(basa::launch_select_ranges(scores, rows, n, split, k_lo, k_hi, idx,
                                               static_cast<hipStream_t>(stream)));
  } catch (...) {
    return BASA_E_LAUNCH;
  }
}

int basa_block_radius(const void* x, int x_dtype, int64_t outer, int64_t len, int64_t head_dim,
                      int64_t block, double* out, void* stream) {
  try {
    if (outer < 0 || len < 0 || block < 1 || block > 256 || len % block != 0) return BASA_E_SHAPE;
    if (head_dim < 8 || head_dim > 256 || head_dim % 8 != 0) return BASA_E_SHAPE;
    if (x_dtype != BASA_F32 && x_dtype != BASA_BF16 && x_dtype != BASA_F64) return BASA_E_DTYPE;
    if (outer * len == 0) return BASA_OK;
    if (!x || !out) return BASA_E_NULLPTR;
    if (!aligned16(x) || !aligned16(out)) return BASA_E_ALIGN;
    return from_hip(basa::launch_radius(x, x_dtype, outer, len, head_dim, block, out,
                                        static_cast<hipStream_t>(stream)));
  } catch (...) {
    return BASA_E_LAUNCH;
  }
}

int basa_rank_workspace(int64_t outer, int64_t len, int64_t* bytes) {
  try {
    if (!bytes) return BASA_E_NULLPTR;
    if (outer < 0 || len < 0 || (len > 0 && outer > INT32_MAX / len)) return BASA_E_SHAPE;
    const int64_t need = basa::rank_workspace_bytes(outer, len);
    if (need < 0) return BASA_E_LAUNCH;  // the sort library could not size its storage
    *bytes = need;
    return BASA_OK;
  } catch (...) {
    return BASA_E_LAUNCH;
  }
}

int basa_rank(const void* x, int x_dtype, int64_t outer, int64_t len, int64_t head_dim,
              int32_t* perm, void* workspace, int64_t workspace_bytes, void* stream) {
  try {
    if (outer < 0 || len < 0 || (len > 0 && outer > INT32_MAX / len)) return BASA_E_SHAPE;
    if (head_dim < 8 || head_dim > 512 || head_dim % 8 != 0) return BASA_E_SHAPE;
    if (x_dtype != BASA_F32 && x_dtype != BASA_BF16 && x_dtype != BASA_F64) return BASA_E_DTYPE;
    if (outer * len == 0) return BASA_OK;
    if (!x || !perm || !workspace) return BASA_E_NULLPTR;
    if (!aligned16(x) || !aligned16(perm) || !aligned16(workspace)) return BASA_E_ALIGN;
    const int64_t need = basa::rank_workspace_bytes(outer, len);
    if (need < 0) return BASA_E_LAUNCH;
    if (workspace_bytes < need) return BASA_E_SHAPE;
    return from_hip(basa::launch_rank(x, x_dtype, outer, len, head_dim, perm, workspace,
                                      workspace_bytes, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return BASA_E_LAUNCH;
  }
}

int basa_permute(const void* x, int dtype, int64_t outer, int64_t len, int64_t width,
                 const int32_t* perm, int mode, void* out, void* stream) {
  try {
    if (outer < 0 || len < 0 || width < 1) return BASA_E_SHAPE;
    if (dtype != BASA_F32 && dtype != BASA_BF16 && dtype != BASA_F64) return BASA_E_DTYPE;
    if (mode != BASA_PERMUTE_GATHER && mode != BASA_PERMUTE_SCATTER) return BASA_E_UNSUPPORTED;
    if (outer * len == 0) return BASA_OK;
    if (!x || !perm || !out) return BASA_E_NULLPTR;
    if (!aligned16(x) || !aligned16(perm) || !aligned16(out)) return BASA_E_ALIGN;
    const int64_t esize = dtype == BASA_BF16 ? 2 : (dtype == BASA_F32 ? 4 : 8);
    const int64_t row_bytes = width * esize;
    const int64_t bytes = outer * len * row_bytes;
    const uintptr_t xa = reinterpret_cast<uintptr_t>(x), oa = reinterpret_cast<uintptr_t>(out);
    if (xa < oa + (uintptr_t)bytes && oa < xa + (uintptr_t)bytes) return BASA_E_UNSUPPORTED;
    return from_hip(basa::launch_permute(x, outer, len, row_bytes, perm, mode, out,
                                         static_cast<hipStream_t>(stream)));
  } catch (...) {
    return BASA_E_LAUNCH;
  }
}

}  // extern "C"
