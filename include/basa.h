/*
 * basa.h - block-sparse bidirectional attention with mean-pooled block
 * selection, for AMD Instinct MI355X (gfx950).
 *
 * The library exposes the four steps of the path as plain C calls:
 *
 *   basa_pool    mean of each run of `block` consecutive rows
 *   basa_select  block scores (pooled Q times pooled K transposed) and a
 *                per-row top-k, or the top-k tokens by query change
 *   basa_attn    flash-style attention with an online softmax over the key
 *                blocks listed for each query tile; emits O and the LSE
 *   basa_merge   combines two partial (O, LSE) results of one row
 *   basa_select_static  basa_select without a caller workspace (no allocation)
 *   basa_pool_pyramid  basa_pool repeated level by level (each level pools
 *                the previous one) for up to three tensors in two launches
 *   basa_pool_moments  block means and variances arranged so that the
 *                covariance-compensated block score is one dot product
 *   basa_block_mass    block mass of the dense attention map
 *   basa_select_ranges top-k of given scores in two column ranges
 *   basa_block_radius  per-block radius and largest token norm
 *   basa_rank    orders each sequence's tokens by their l2 norm
 *   basa_permute moves rows by such an order (gather) or back (scatter)
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every pointer named as device memory must be device memory of the
 *   current HIP device, 16-byte aligned, and stay valid until the work on
 *   `stream` has finished.  The caller owns every buffer; the library never
 *   allocates or frees device memory.  Its only device memory of its own is
 *   the fixed scratch array of basa_select_static (one per GPU).
 * - Tensors are dense and row-major in the order their shapes are written.
 * - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *   enqueues work and returns; nothing synchronises the host.
 * - Arguments are checked on the host before anything is enqueued; a
 *   non-zero basa_status means nothing was launched.  BASA_E_LAUNCH reports a
 *   failed kernel launch (hipGetLastError after the launch).
 * - Inputs are never written.  Results are deterministic run to run (no
 *   floating-point atomics).
 * - No C++ exception crosses this interface.
 */
#ifndef BASA_H
#define BASA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum basa_status {
  BASA_OK = 0,
  BASA_E_NULLPTR = 1,     /* a required pointer is NULL */
  BASA_E_SHAPE = 2,       /* inconsistent or out-of-range sizes */
  BASA_E_DTYPE = 3,       /* unsupported element type for this argument */
  BASA_E_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  BASA_E_UNSUPPORTED = 5, /* valid request the kernels do not implement */
  BASA_E_LAUNCH = 6       /* the HIP runtime rejected a kernel launch */
} basa_status;

typedef enum basa_dtype {
  BASA_F32 = 0,  /* IEEE binary32 */
  BASA_BF16 = 1, /* bfloat16 (upper half of a binary32) */
  BASA_F64 = 2   /* IEEE binary64 */
} basa_dtype;

/* Human-readable name of a status code (static storage, never NULL). */
const char* basa_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int basa_version(void);

/*
 * basa_pool - block mean pooling.
 *
 * Follows the BA-Att paper (section 3.1 and Algorithm 1, "block statistics"):
 * the representative of a block is the mean of its rows.  The log-linear
 * README pools the same way, repeatedly, one level from the previous one.
 *
 *   x         device, [outer][len][head_dim] of x_dtype (F32, BF16 or F64)
 *   mean_rows device or NULL, [outer][len/block][head_dim] float64
 *   mean_cols device or NULL, [outer][head_dim][len/block] float64
 *             (the same means, transposed; basa_select reads keys this way)
 *   mean_copy device or NULL, [outer][len/block][head_dim] of copy_dtype
 *             (F32 or BF16), the float64 mean rounded to nearest even
 *
 * Sums are accumulated in float64.  At least one output must be non-NULL.
 * Errors: BASA_E_SHAPE if outer < 0, len < 0, block < 1, len % block != 0,
 * head_dim not a multiple of 8 or above 512.  outer*len == 0 enqueues nothing.
 */
int basa_pool(const void* x, int x_dtype, int64_t outer, int64_t len, int64_t head_dim,
              int64_t block, double* mean_rows, double* mean_cols, void* mean_copy,
              int copy_dtype, void* stream);

/* Outputs of one pyramid level of one tensor (any of them may be NULL). */
typedef struct basa_pyramid_level {
  double* mean_rows;  /* device, [outer][len/block^l][head_dim] float64 */
  double* mean_cols;  /* device, [outer][head_dim][len/block^l] float64 */
  void* mean_copy;    /* device, [outer][len/block^l][head_dim] of copy_dtype */
} basa_pyramid_level;

#define BASA_PYRAMID_MAX_LEVELS 4
#define BASA_PYRAMID_MAX_TENSORS 3

/* One input of basa_pool_pyramid and its outputs; level[l-1] is level l. */
typedef struct basa_pyramid_tensor {
  const void* x;      /* device, [outer][len][head_dim] of x_dtype */
  basa_pyramid_level level[BASA_PYRAMID_MAX_LEVELS];
} basa_pyramid_tensor;

/*
 * basa_pool_pyramid - the log-linear pooling pyramid.
 *
 * Follows the log-linear README (method paragraphs on the hierarchy): level
 * 1 holds the means of `block` consecutive tokens, and every further level
 * the means of `block` consecutive entries of the level below.  For each of
 * the n_tensors inputs and each level l = 1..levels the call writes what
 * basa_pool(level l-1 -> level l) would write into that level's outputs, bit
 * for bit: every sum is taken in float64 in the same order (the rows of a
 * block in ascending order), and level l >= 2 is pooled from the float64
 * means of level l-1.  Levels 1 and 2 of all tensors take one launch (a
 * workgroup pools `block` level-1 blocks and then their level-2 block from
 * LDS), every further level one launch.
 *
 *   tensors    host array of n_tensors (1..BASA_PYRAMID_MAX_TENSORS)
 *              descriptors; all share x_dtype (F32, BF16 or F64), outer,
 *              len and head_dim
 *   levels     1..BASA_PYRAMID_MAX_LEVELS; len must be a multiple of
 *              block^levels
 *   block      2..32, with block * head_dim <= 4096
 *   copy_dtype F32 or BF16 (read only where a mean_copy is given)
 *
 * Every level of every tensor needs at least one output, and every level
 * from 2 up to the one below the top its mean_rows (the next level is pooled
 * from them; level 2 is pooled from level 1 inside the workgroup, so level
 * 1 needs no float64 rows unless the caller wants them).
 * Errors: BASA_E_SHAPE for sizes outside the above (head_dim a multiple of 8,
 * at most 512), BASA_E_NULLPTR for a missing input or required output,
 * BASA_E_DTYPE, BASA_E_ALIGN.  outer*len == 0 enqueues nothing.
 */
int basa_pool_pyramid(const basa_pyramid_tensor* tensors, int n_tensors, int x_dtype,
                      int64_t outer, int64_t len, int64_t head_dim, int64_t block, int levels,
                      int copy_dtype, void* stream);

/* Roles of basa_pool_moments. */
enum {
  BASA_MOMENTS_QUERY = 0, /* query blocks: rows u */
  BASA_MOMENTS_KEY = 1    /* key blocks: transposed w */
};

/*
 * basa_pool_moments - block statistics for covariance-compensated scores.
 *
 * Follows the BA-Att paper, section 3.4 (Eq. 13 adds beta * Delta to the
 * block logit; Eq. 14 approximates Delta from per-channel block variances)
 * and Algorithm 1 steps 4-7.  With block means Xbar and population variances
 * Var[X] (per channel, the mean of squared deviations over the block's
 * tokens, both in float64),
 *   l~ = scale * Qbar.Kbar + beta * (1/d) sum_t (Var[Q_t] Kbar_t^2
 *        + Var[K_t] Qbar_t^2 + Var[Q_t] Var[K_t])
 * is the dot product of
 *   u = [scale * Qbar, (beta/d) * Var[Q], (beta/d) * Qbar^2]   (QUERY role)
 *   w = [Kbar, Kbar^2 + Var[K], Var[K]]                        (KEY role)
 * so basa_select with head_dim 3*head_dim, scale 1 and these vectors ranks
 * key blocks by the compensated logit.
 *   x     device [outer][len][head_dim] of x_dtype (F32, BF16 or F64)
 *   out   device float64: QUERY [outer][len/block][3*head_dim],
 *         KEY [outer][3*head_dim][len/block]
 * Errors: BASA_E_SHAPE for negative sizes, block < 1, len % block != 0,
 * head_dim not a multiple of 8 or above 168 (3*head_dim <= 512), or a
 * non-finite scale or beta; BASA_E_UNSUPPORTED for another role.
 */
int basa_pool_moments(const void* x, int x_dtype, int64_t outer, int64_t len, int64_t head_dim,
                      int64_t block, int role, double scale, double beta, double* out,
                      void* stream);

/* Selection modes of basa_select. */
enum {
  BASA_SELECT_BLOCKS = 0, /* top-k key rows per query row by q . k */
  BASA_SELECT_CHANGE = 1  /* top-k tokens by mean squared query change */
};

typedef struct basa_select_desc {
  int32_t mode;      /* BASA_SELECT_BLOCKS or BASA_SELECT_CHANGE */
  int32_t topk;      /* entries kept per output row, >= 1 */
  int64_t batch;
  int64_t heads_q;   /* query heads */
  int64_t heads_kv;  /* key heads; query head h reads key head h / (heads_q/heads_kv) */
  int64_t q_len;     /* rows per query head in q */
  int64_t rows;      /* output rows per query head (== q_len unless q_rows is set) */
  int64_t keys;      /* key rows per key head */
  int64_t head_dim;
  double scale;      /* positive factor applied to the scores; the ranking does not depend on it */
  /* optional row map: output row r of batch b reads query row q_rows[b*rows + r] */
  const int32_t* q_rows;
  /* optional candidate restriction (coarse-to-fine descent): output row r may
     only pick among keys fanout*s + u, s in parent[b][h][r / fanout][0..parent_k),
     u in [0, fanout).  parent rows must be ascending and lie in [0, keys/fanout). */
  const int32_t* parent;
  int32_t parent_k;
  int32_t fanout;
  /* optional device scratch, owned by the caller (NULL: none).  Rows with
     more than 1024 candidates and no parent list are selected in two passes
     when it holds at least basa_select_workspace() bytes (otherwise in one,
     slower, pass; the result is the same).  The call overwrites it; calls
     that overlap in time must not share it. */
  void* workspace;
  int64_t workspace_bytes;
} basa_select_desc;
/* (parent entries outside [0, keys/fanout) are treated as no candidate.) */

/*
 * basa_select - which keys each query row keeps.
 *
 * BASA_SELECT_BLOCKS follows BA-Att section 3.1, Eq. 2 and Algorithm 1: the
 * block logit is the scaled dot product of the pooled query and pooled key,
 * the block distribution is its softmax over key blocks, and each query block
 * keeps the top-k key blocks.  Softmax is strictly increasing, so the kept set
 * is the top-k by logit.  Order: larger score first, equal scores to the lower
 * key index.  Scores are formed in float64.  With `parent` set this is the
 * per-token candidate selection of the log-linear README (a selected coarse
 * token's children become the candidates one level down).
 *   q    device, float64 [batch][heads_q][q_len][head_dim]  (dtype must be F64)
 *   k    device, float64 [batch][heads_kv][head_dim][keys]  (transposed means)
 *   idx  device, int32 [batch][heads_q][rows][topk], each row ascending
 *
 * BASA_SELECT_CHANGE follows the LoSA post's locality pruning: per token, the
 * mean over heads and channels of (q - k)^2, where q is the current and k the
 * previous step's queries; the topk tokens with the largest change are active
 * (ties to the lower token).
 *   q, k device, [batch][heads_q][q_len][head_dim] of dtype (F32, BF16 or F64)
 *   idx  device, int32 [batch][topk], ascending token numbers
 *   (heads_kv, keys, rows, scale, q_rows and parent are ignored; q_len <= 1024)
 *
 * Errors: BASA_E_SHAPE for topk < 1 or topk above the candidate count,
 * heads_q % heads_kv != 0, head_dim not a multiple of 8 or above 512,
 * keys > 4096 (BLOCKS), parent_k*fanout > 4096, or non-positive scale.
 */
int basa_select(const basa_select_desc* desc, const void* q, const void* k, int dtype,
                int32_t* idx, void* stream);

/*
 * basa_pool_select - the selection stage in one call: the block means of q
 * (rows, as basa_pool's mean_rows), of k (transposed, as mean_cols) and the
 * BLOCKS-mode selection of basa_select on them (BA-Att section 3.1, Eq. 2
 * and Algorithm 1 steps 3-5), with the same results as those three calls.
 *   desc    BLOCKS mode, no q_rows, no parent; q_len = query blocks per head,
 *           keys = key blocks per key head, rows = q_len
 *   q       device [batch][heads_q][q_len*block][head_dim] of dtype
 *   k       device [batch][heads_kv][keys*block][head_dim] of dtype
 *   qbar    device float64 [batch][heads_q][q_len][head_dim] (written)
 *   kbar_t  device float64 [batch][heads_kv][head_dim][keys] (written)
 *   idx     device int32 [batch][heads_q][q_len][topk] (written)
 * It enqueues the three launches (query means, key means, selection) on the
 * stream.  desc->workspace is accepted and unused.
 * Errors: as basa_pool and basa_select, plus BASA_E_UNSUPPORTED for another
 * mode, a row map or a parent list, and BASA_E_NULLPTR for a NULL output.
 */
int basa_pool_select(const basa_select_desc* desc, const void* q, const void* k, int dtype,
                     int64_t block, double* qbar, double* kbar_t, int32_t* idx, void* stream);

/* basa_pool_select_workspace - bytes of workspace basa_pool_select uses: 0
 * (kept so that callers written against a workspace-taking form still work).
 * Errors: BASA_E_NULLPTR. */
int basa_pool_select_workspace(const basa_select_desc* desc, int64_t* bytes);

/*
 * basa_select_workspace - bytes of workspace that lets basa_select take the
 * two-pass path for this request (0: the request never uses one).  Reads
 * only the sizes in desc (mode, batch, heads_q, rows, keys, topk, parent).
 * The two passes compute the same selection as one (BA-Att section 3.1): the
 * candidates are split into parts of 512 keys, each part keeps its own top-k,
 * and the top-k of the union of the parts' top-k is the row's top-k.
 * Errors: BASA_E_NULLPTR for a NULL desc or bytes.
 */
int basa_select_workspace(const basa_select_desc* desc, int64_t* bytes);

/* Size of the device scratch array basa_select_static uses (4 MiB). */
#define BASA_STATIC_SCRATCH_BYTES (4 << 20)

/*
 * basa_select_static - basa_select for callers that cannot allocate device
 * memory (code under stream capture, tight serving loops, harnesses that
 * forbid allocation): the two-pass path uses a 4 MiB device array of this
 * library instead of a caller-owned workspace.  It calls no allocator.
 *
 * Same arguments, results and errors as basa_select, except:
 *   - desc->workspace must be NULL and desc->workspace_bytes 0
 *     (BASA_E_UNSUPPORTED otherwise);
 *   - a request whose two-pass workspace (basa_select_workspace) exceeds
 *     BASA_STATIC_SCRATCH_BYTES is rejected with BASA_E_SHAPE and nothing is
 *     launched (e.g. 160 LoSA rows x 4096 keys, top-128, need 1.97 MB);
 *   - BASA_E_LAUNCH also reports a failure to find the array's device address.
 * The array exists once per GPU, for the life of the process, and keeps the
 * last call's contents (every entry a call reads is written earlier in the
 * same call).  Calls that overlap in time on one GPU (different streams or
 * host threads) share it and race: serialise them.  The device address is
 * looked up on the first call on each device, under a lock.
 */
int basa_select_static(const basa_select_desc* desc, const void* q, const void* k, int dtype,
                       int32_t* idx, void* stream);

/* One source of keys for basa_attn.  The key list of query tile t is the
 * concatenation, over the descriptor's segments, of `count` entries of row
 * (t >> shift) of the segment's index array; entry value e >= 0 names keys
 * e*block_k .. e*block_k+block_k-1 of the segment's own key/value table, and
 * a negative entry is an empty slot. */
typedef struct basa_kv_segment {
  const int32_t* idx; /* device int32; entry j of index row r of (b, h) is
                         idx[((b*heads_q + h)*rows + r)*stride + j] */
  const void* k;      /* device [batch][heads_kv][len][head_dim] of dtype */
  const void* v;      /* device [batch][heads_kv][len][head_dim] of dtype */
  int64_t len;        /* key rows per key head in k and v */
  int64_t rows;       /* index rows per query head, >= ((lists-1) >> shift) + 1 */
  int32_t count;      /* entries taken from each index row */
  int32_t stride;     /* distance between index rows, in entries (>= count) */
  int32_t shift;      /* query tile t reads index row t >> shift (0..30) */
  int32_t dtype;      /* F32 or BF16 */
  float bias;         /* added to every logit of this segment's keys */
  int32_t reserved;
} basa_kv_segment;

#define BASA_MAX_SEGMENTS 4

typedef struct basa_attn_desc {
  int64_t batch;
  int64_t heads_q;    /* query heads */
  int64_t heads_kv;   /* key/value heads; query head h reads head h / (heads_q/heads_kv) */
  int64_t len_q;      /* rows per query head in q, o and lse */
  int64_t head_dim;   /* 64 or 128 */
  int64_t lists;      /* query tiles (key lists) per query head */
  int32_t tile_q;     /* query rows per tile (1..128) */
  int32_t block_k;    /* keys per list entry (1..4096) */
  int32_t n_segments; /* 1..BASA_MAX_SEGMENTS */
  int32_t reserved;
  basa_kv_segment seg[BASA_MAX_SEGMENTS];
  /* q_rows: device int32 [batch][lists*tile_q] or NULL.  NULL: tile t holds
     query rows t*tile_q .. t*tile_q+tile_q-1.  Otherwise its rows are
     q_rows[b][t*tile_q + r]; they are read from q and written to o and lse,
     and other rows of o and lse are left untouched (the LoSA cache update). */
  const int32_t* q_rows;
  double scale;       /* logit scale, normally 1/sqrt(head_dim) */
  /* optional device scratch, owned by the caller (NULL: none), 16-byte
     aligned.  With at least basa_attn_workspace() bytes:
     - rows given by a row map (tile_q 1, one bf16 segment of 16-key blocks,
       at most 32 rows per key head) are computed as one walk over the union
       of each key head's kept blocks: every block of the union is read once
       (the LoSA step's active rows).  Without it each row walks its own
       list; the result is the same up to float32 rounding.
     - on the MFMA path (see basa_attn) the query tiles of each (batch,
       head) are ranked by the middle entry of their lists and run in that
       order, so that tiles running side by side on one XCD keep nearby key
       blocks and share its L2.  The output is bit-identical without it.
     The call overwrites it; calls that overlap in time must not share it. */
  void* workspace;
  int64_t workspace_bytes;
} basa_attn_desc;

/*
 * basa_attn - attention confined to listed key blocks, with online softmax.
 *
 * Follows BA-Att section 2 (block-sparse attention: each query block attends
 * only to the key/value blocks its mask keeps) with the softmax of Eq. 1
 * restricted to those keys; bidirectional, no causal mask.  Segments express
 * the log-linear README's KV enrichment (fine keys plus coarse candidates of
 * every level, each level with logit bias l*ln(block)) and the LoSA prefix /
 * in-block split.  For query row i: z_j = scale * q_i . k_j + bias(seg(j))
 * over the listed keys j, LSE_i = ln sum_j exp(z_j),
 * O_i = sum_j exp(z_j - LSE_i) v_j.  A row with no valid entry gets O = 0 and
 * LSE = -inf.
 *   q     device [batch][heads_q][len_q][head_dim] of q_dtype (F32 or BF16)
 *   o     device [batch][heads_q][len_q][head_dim] of o_dtype (F32 or BF16)
 *   lse   device float32 [batch][heads_q][len_q], natural logarithm
 * Accumulation is float32.  On the MFMA path (bf16 q/k/v, head_dim 128,
 * 128-row tiles, 128-key blocks, one segment) the probabilities are rounded
 * to bf16 before the value product.  Entries must name existing keys:
 * e*block_k + block_k <= len (not checked on the device).
 * Errors: BASA_E_SHAPE for inconsistent sizes (including len_q not equal to
 * lists*tile_q when q_rows is NULL), head_dim not 64/128, or a segment whose
 * rows/count/stride/shift do not cover the tiles.
 */
int basa_attn(const basa_attn_desc* desc, const void* q, int q_dtype, void* o, int o_dtype,
              float* lse, void* stream);

/*
 * basa_attn_workspace - bytes of workspace basa_attn can use for this request
 * (0: the request never uses one).  Reads only the sizes and types in desc.
 * MFMA-path requests (bf16, head_dim 128, 128-row tiles of 128-key blocks,
 * one segment, at most 2048 tiles per head) take one int32 rank per query
 * tile (batch * heads_q * lists * 4 bytes, rounded up to 256) for the tile
 * order described at basa_attn_desc.workspace.  Row-map requests of 16-key
 * blocks take the union walk's partials, below.  The union walk follows the LoSA post
 * ("KV inflation" and method steps 2-4): the active rows of one key head
 * each keep their own prefix blocks, and the data the step must move is the
 * union of those selections.  The prefix blocks of a key head are cut into
 * chunks of 64 blocks; each chunk's union is read once and every row that
 * kept a block attends to it, giving per-(chunk, row) partial results
 * (unnormalised O, max, sum: (head_dim + 2) floats each) in the workspace,
 * which a second kernel combines per row by the online-softmax merge rule.
 * Errors: BASA_E_NULLPTR for a NULL desc or bytes.
 */
int basa_attn_workspace(const basa_attn_desc* desc, int64_t* bytes);

/*
 * basa_merge - combine two partial attention results of the same rows.
 *
 * Follows the LoSA post's prefix/suffix merge by online softmax: with
 * m = max(lse_a, lse_b), LSE = m + ln(exp(lse_a - m) + exp(lse_b - m)) and
 * O = exp(lse_a - LSE) o_a + exp(lse_b - LSE) o_b.  (anything, -inf) is the
 * empty partial; two empty partials give O = 0, LSE = -inf.
 *   o_a, o_b  device [rows][head_dim] of in_dtype (F32 or BF16)
 *   lse_a/b   device float32 [rows]
 *   o         device [rows][head_dim] of o_dtype (F32 or BF16); may be o_a
 *             when o_dtype == in_dtype (in place)
 *   lse       device float32 [rows]; may be lse_a
 * Errors: BASA_E_SHAPE for rows < 0 or head_dim not a power of two in
 * [8, 512]; BASA_E_UNSUPPORTED when o aliases an input of another dtype.
 */
int basa_merge(int64_t rows, int64_t head_dim, const void* o_a, const float* lse_a,
               const void* o_b, const float* lse_b, int in_dtype, void* o, int o_dtype,
               float* lse, void* stream);

/*
 * basa_block_mass - how much attention each query block puts on each key
 * block, from the dense attention map.
 *
 * Follows the BA-Att paper, section 3.1, Eq. 3 (the oracle block
 * distribution): m[gq][gk] = (1/block) sum over the block's query rows i and
 * key columns j of A_ij, with A = softmax(scale * Q K^T) row by row over all
 * keys (Eq. 1).  SparseD section 3.3 ranks blocks by the average-pooled
 * attention scores, which are m / block.  Logits, row LSE and sums are float64
 * (exact widenings of the inputs); each row of m sums to 1.
 *   q     device [batch][heads_q][len_q][head_dim] of dtype (BF16 or F32)
 *   k     device [batch][heads_kv][len_k][head_dim] of dtype; query head h
 *         reads key head h / (heads_q / heads_kv)
 *   mass  device float64 [batch][heads_q][len_q/block][len_k/block]
 *   workspace  optional device scratch owned by the caller (NULL: none), 16-byte
 *         aligned, of workspace_bytes.  With at least basa_block_mass_workspace()
 *         bytes the mass is formed in one pass over the keys: per (row, key
 *         block) the block's own max and sum of exp(s - max) go to the
 *         workspace, the row LSE follows from them, and the mass from both
 *         (one float64 scale*Q*K^T product).  Without it, two passes (the row
 *         LSE first, then the sums of exp(s - LSE)).  The two differ only in
 *         float64 rounding order.  The call overwrites the workspace; calls
 *         that overlap in time must not share it.
 * Errors: BASA_E_SHAPE for non-positive heads, heads_q not a multiple of
 * heads_kv, head_dim not a multiple of 8 or above 128, block not a power of
 * two in [4, 256], lengths not multiples of block, or a scale that is not
 * finite and positive.
 */
int basa_block_mass(const void* q, const void* k, int dtype, int64_t batch, int64_t heads_q,
                    int64_t heads_kv, int64_t len_q, int64_t len_k, int64_t head_dim, int64_t block,
                    double scale, double* mass, void* workspace, int64_t workspace_bytes,
                    void* stream);

/*
 * basa_block_mass_workspace - bytes of workspace that let basa_block_mass take
 * its one-pass form (0: this shape never does: blocks of 16..128 rows that are
 * multiples of 16, head_dim a multiple of 4 and at most 128):
 * batch * heads_q * len_q * (len_k / block) * 16 bytes.
 * Errors: BASA_E_NULLPTR for a NULL bytes.
 */
int basa_block_mass_workspace(int64_t batch, int64_t heads_q, int64_t len_q, int64_t len_k,
                              int64_t head_dim, int64_t block, int64_t* bytes);

/*
 * basa_select_ranges - per row, the best columns of two column ranges.
 *
 * Follows SparseD section 3.3 (Eq. 5-6, isolated selection): the top
 * entries among the prefill keys and among the generation keys are taken
 * separately and united.  For each row r of scores [rows][n] (float64): the
 * k_lo best columns of [0, split) and the k_hi best of [split, n), each under
 * (score descending, column ascending), written together in ascending column
 * order to idx [rows][k_lo + k_hi] (int32).
 * Errors: BASA_E_SHAPE for rows < 0, n outside [1, 1024], split outside
 * [0, n], k_lo outside [0, split], k_hi outside [0, n - split] or
 * k_lo + k_hi == 0.
 */
int basa_select_ranges(const double* scores, int64_t rows, int64_t n, int64_t split, int32_t k_lo,
                       int32_t k_hi, int32_t* idx, void* stream);

/*
 * basa_block_radius - block geometry of the deviation bound.
 *
 * Follows the BA-Att paper, section 3.2, Eq. 7: for each block of `block`
 * consecutive tokens, R = max_i ||x_i - xbar||_2 (the radius around the block
 * mean) and M = max_i ||x_i||_2 (the largest token norm), in float64.  Eq. 8
 * bounds the gap between a token logit and its block logit by
 * (R^Q M^K + M^Q R^K + R^Q R^K) / sqrt(d).
 *   x    device [outer][len][head_dim] of x_dtype (F32, BF16 or F64)
 *   out  device float64 [outer][len/block][2] = (R, M)
 * Errors: BASA_E_SHAPE for negative sizes, block outside [1, 256], len not a
 * multiple of block, head_dim not a multiple of 8 or above 256.
 */
int basa_block_radius(const void* x, int x_dtype, int64_t outer, int64_t len, int64_t head_dim,
                      int64_t block, double* out, void* stream);

/*
 * basa_rank_workspace - bytes of device workspace basa_rank needs to rank
 * `outer` sequences of `len` tokens (0 when outer*len == 0).
 * Errors: BASA_E_NULLPTR for bytes == NULL; BASA_E_SHAPE as in basa_rank;
 * BASA_E_LAUNCH if the HIP runtime cannot size the sort's storage.
 */
int basa_rank_workspace(int64_t outer, int64_t len, int64_t* bytes);

/*
 * basa_rank - norm-based token ranking.
 *
 * Follows the BA-Att paper, section 3.3 (Eq. 9 scores a token by its l2 norm,
 * Eq. 10 orders the tokens by non-decreasing score) and Algorithm 1 steps 1
 * and 2 (queries and keys are ranked before the blocks are formed).  Each of
 * the `outer` sequences is ranked on its own, over all its tokens.  The key
 * of a token is its squared norm in float64, channels added in order with
 * every square and sum rounded separately (exact for bf16 tokens); tokens
 * with equal keys keep their order (a stable sort).
 *   x          device [outer][len][head_dim] of x_dtype (F32, BF16 or F64)
 *   perm       device int32 [outer][len]: position i of sequence s holds
 *              token perm[s][i] (an index into that sequence)
 *   workspace  device scratch of at least basa_rank_workspace(outer, len)
 *              bytes, caller-owned; its contents are not kept
 * Errors: BASA_E_SHAPE for outer < 0, len < 0, outer*len above 2^31 - 1,
 * head_dim not a multiple of 8 or above 512; BASA_E_NULLPTR for a missing
 * pointer; BASA_E_SHAPE when workspace_bytes is too small.
 */
int basa_rank(const void* x, int x_dtype, int64_t outer, int64_t len, int64_t head_dim,
              int32_t* perm, void* workspace, int64_t workspace_bytes, void* stream);

/* Directions of basa_permute. */
enum {
  BASA_PERMUTE_GATHER = 0, /* out[s][i] = x[s][perm[s][i]] (into ranked order) */
  BASA_PERMUTE_SCATTER = 1 /* out[s][perm[s][i]] = x[s][i] (back to token order) */
};

/*
 * basa_permute - move whole rows of each sequence by a permutation.
 *
 * BA-Att Algorithm 1: GATHER forms the ranked sequences Q', K', V' (steps 1
 * and 2; V moves with K's order); SCATTER maps outputs of ranked query rows
 * back to the original order by the inverse permutation (step 12).
 *   x     device [outer][len][width] of dtype (F32, BF16 or F64)
 *   perm  device int32 [outer][len], each sequence a permutation of 0..len-1
 *         (a GATHER row whose entry is out of range is zero-filled; a
 *         SCATTER entry out of range writes nothing)
 *   out   device [outer][len][width] of dtype; must not overlap x
 * Errors: BASA_E_SHAPE for negative sizes or width < 1; BASA_E_UNSUPPORTED
 * for a mode other than the two above or overlapping x and out.
 */
int basa_permute(const void* x, int dtype, int64_t outer, int64_t len, int64_t width,
                 const int32_t* perm, int mode, void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BASA_H */
