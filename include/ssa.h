/*
 * ssa.h - C ABI of the MI355X (gfx950) Spatial Sparse Attention library.
 *
 * Spatial Sparse Attention (SSA) is the attention of Direct3D-S2's sparse
 * diffusion transformer over the variable-length tokens of a sparse voxel grid
 * (hyper.ai summary of arXiv 2505.17412, "Method", second paragraph):
 *   - tokens are grouped by their 3D coordinate into m_cmp^3 blocks (not by
 *     their 1D index) and into non-overlapping m_win^3 windows;
 *   - compression: keys and values are mean-pooled per block, and every query
 *     attends to all compressed blocks of its sequence;
 *   - selection: the query-to-block attention scores pick the top-k blocks and
 *     the query attends to every token inside them;
 *   - window: the query attends to every token of its own window;
 *   - the three results are summed with per-token, per-head gates.
 * Grouped-query attention (several query heads sharing one key/value head,
 * LSRM article, "Stage 1": 32 query heads over 2 key/value heads) shares the
 * selection across the heads of a group: the block score is the softmax
 * probability summed over the group's query heads.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers, caller-allocated and
 *     caller-owned; the library allocates nothing and keeps no state between
 *     calls.  Tensors are dense row-major, 16-byte aligned.
 *   - Work is enqueued on `hip_stream` (a hipStream_t, NULL = default
 *     stream).  SSA_OK means "validated and enqueued"; only ssa_build_blocks
 *     with sync_counts != 0 blocks the host.
 *   - Arguments are validated before anything is enqueued; on an error no
 *     output is touched and ssa_last_error() describes the problem.
 *   - Calls are re-entrant; ssa_last_error() is thread-local.
 */
#ifndef SSA_H
#define SSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SSA_OK = 0,
  SSA_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative size, bad geometry, out-of-range coords (when synced) */
  SSA_ERR_UNSUPPORTED = 2,      /* valid request the library does not implement (head_dim, top-k, key width) */
  SSA_ERR_WORKSPACE = 3,        /* workspace pointer null or smaller than the *_workspace() query */
  SSA_ERR_DEVICE = 4            /* a HIP runtime call or kernel launch failed */
} ssa_status;

typedef enum { SSA_F32 = 0, SSA_BF16 = 1 } ssa_dtype;

/* Grid and block geometry.  grid_res (R), m_cmp and m_win are powers of two
 * with m_cmp <= m_win <= R <= 1024.  Blocks are the m_cmp^3 cells and windows
 * the m_win^3 cells of the grid, both aligned to the origin
 * (Direct3D-S2 page, "Method": non-overlapping windows).  win_shift = 0
 * keeps them so; a win_shift that is a multiple of m_cmp in (0, m_win) moves
 * the window origin to -win_shift on every axis (the shifted windows of the
 * same page's sparse VAE; m_win / 2 is the usual choice).  Blocks do not
 * move, since the shift is a whole number of blocks. */
typedef struct {
  int32_t grid_res;
  int32_t m_cmp;
  int32_t m_win;
  int32_t win_shift;
} ssa_geometry;

/* Device-side counters written by ssa_build_blocks (int32 each). */
enum {
  SSA_COUNT_NB = 0,          /* number of blocks                       */
  SSA_COUNT_NW = 1,          /* number of windows                      */
  SSA_COUNT_INVALID = 2,     /* tokens with a coordinate outside [0,R) */
  SSA_COUNT_MAX_BLK = 3,     /* most tokens in one block               */
  SSA_COUNT_MAX_WIN = 4,     /* most tokens in one window              */
  SSA_COUNT_KEY_BITS = 5,    /* bits of the block key                  */
  SSA_COUNTS = 8             /* length of the counts array             */
};

/* Result of the block build: the tokens' stable sort by block key and the CSR
 * segments over the sorted order.  The block key of a token of sequence b at
 * coordinate c is ((b * Rw^3 + lin(c / m_win)) * r^3 + lin((c / m_cmp) mod r))
 * with Rw = R / m_win, r = m_win / m_cmp, lin(x,y,z) = (x*n + y)*n + z; block
 * ids and window ids count up in that key order.  All arrays are DEVICE
 * int32 buffers owned by the caller, with the capacities given. */
typedef struct {
  int32_t *perm;        /* [N]     sorted position -> input token index (stable: ties keep input order) */
  int32_t *blk_off;     /* [N + 1] first sorted position of block j; blk_off[nb] = N                    */
  int32_t *win_off;     /* [N + 1] first sorted position of window w; win_off[nw] = N                   */
  int32_t *win_blk_off; /* [N + 1] first block id of window w; win_blk_off[nw] = nb                     */
  int32_t *seq_blk_off; /* [B + 1] first block id of sequence b; seq_blk_off[B] = nb                    */
  int32_t *seq_win_off; /* [B + 1] first window id of sequence b; seq_win_off[B] = nw                   */
  int32_t *counts;      /* [SSA_COUNTS] device counters (see enum above)                                */
  int64_t n_tokens;     /* N, filled by ssa_build_blocks                                               */
  int32_t batch;        /* B, filled by ssa_build_blocks                                               */
  int32_t nb, nw;       /* host copies of the counts when synced, else -1                              */
  int32_t max_blk_tokens, max_win_tokens; /* host copies when synced, else -1                          */
  ssa_geometry geo;     /* filled by ssa_build_blocks                                                  */
  const int32_t *coords;/* the [N, 3] coordinates given to ssa_build_blocks (set by it); read by the   */
                        /* forward with geometric routing, so they must stay valid for such calls      */
} ssa_blocks;

/* Block selection rule (ssa_attn.routing). */
typedef enum {
  /* top-k blocks by compressed-attention probability, summed over the
   * group's query heads (Direct3D-S2 page, "Method"; LSRM article) */
  SSA_ROUTE_SCORE = 0,
  /* top-k blocks by geometric distance (LSRM article, "3D-aware block
   * routing"): the smallest squared distance between the query's voxel
   * centre and the centres of the block's voxels, ties to the lower block id;
   * the same for every key/value group.  bfloat16 layouts of the MFMA path
   * only (D = 32 or 64 with 1 to 16 query heads per key/value head) */
  SSA_ROUTE_GEOMETRIC = 1
} ssa_routing;

/* Attention layout.  h_q query heads over h_kv key/value heads (h_q % h_kv
 * == 0; query head h uses key/value head h / (h_q / h_kv)).  head_dim D in
 * {32, 64}.  1 <= topk <= 32.  scale <= 0 selects 1/sqrt(D).  q, k, v, gates
 * and out all have `dtype`; accumulation is float32. */
typedef struct {
  int32_t h_q;
  int32_t h_kv;
  int32_t head_dim;
  int32_t topk;
  float scale;
  ssa_dtype dtype;
  int32_t routing;      /* ssa_routing; 0 = by score */
} ssa_attn;

/* Workspace bytes ssa_build_blocks needs for N tokens in B sequences. */
size_t ssa_build_blocks_workspace(int64_t n_tokens, int32_t batch, const ssa_geometry *geo);

/* Group tokens into blocks and windows (Direct3D-S2 page, "Method": blocking
 * by 3D coordinate; non-overlapping windows).
 *   coords     [N, 3] int32 device, (x, y, z) per token in input order.
 *   cu_seqlens [B + 1] int32 device, cu_seqlens[0] = 0, non-decreasing,
 *              cu_seqlens[B] = N; sequence b owns tokens [cu[b], cu[b+1]).
 *              Empty sequences are allowed.  Duplicate coordinates are
 *              distinct tokens.
 *   out        caller struct whose device pointers are set (capacities
 *              above); the library fills n_tokens, batch, geo and, when
 *              sync_counts != 0, nb / nw / max_*.
 *   sync_counts  != 0: copy the counts to the host and wait; then a token
 *              outside [0, R) gives SSA_ERR_INVALID_ARGUMENT.  == 0: fully
 *              asynchronous; out-of-range tokens are clamped for memory
 *              safety and counted in counts[SSA_COUNT_INVALID].
 *   workspace  device scratch of at least ssa_build_blocks_workspace() bytes.
 * Errors: INVALID_ARGUMENT (null pointers, N < 0, B < 1, bad geometry),
 * UNSUPPORTED (block key wider than 32 bits), WORKSPACE, DEVICE. */
ssa_status ssa_build_blocks(const int32_t *coords, const int32_t *cu_seqlens, int64_t n_tokens,
                            int32_t batch, const ssa_geometry *geo, ssa_blocks *out,
                            int sync_counts, void *workspace, size_t ws_bytes, void *hip_stream);

/* Workspace bytes ssa_forward needs for these blocks and this layout.  Uses
 * blocks->nb when known (synced), else the worst case nb = N. */
size_t ssa_forward_workspace(const ssa_blocks *blocks, const ssa_attn *attn);

/* SSA forward pass (Direct3D-S2 page, "Method", second paragraph).
 *   q      [N, h_q, D]  query per token (input order)
 *   k, v   [N, h_kv, D] key / value per token
 *   gates  [N, h_q, 3]  per-token, per-head gates in the order
 *                       (compressed, selected, window); used as given
 *   out    [N, h_q, D]  G0 * o_cmp + G1 * o_sel + G2 * o_win, rounded once
 *   k_cmp, v_cmp  optional [nb, h_kv, D] mean-pooled keys / values (NULL = skip)
 *   topk_idx      optional [N, h_kv, topk] int32 selected block ids per token
 *                 and key/value group, highest score first, ties to the lower
 *                 block id, -1 padded when the sequence has fewer blocks
 *                 (NULL = skip).  A block's score is its compressed-attention
 *                 probability summed over the group's query heads (LSRM
 *                 article, sparse-attention section: the query heads of a
 *                 group share one selection).
 *   workspace     device scratch of at least ssa_forward_workspace() bytes.
 * Attention never crosses sequences; the selection is non-causal and forces
 * no block.  Errors: INVALID_ARGUMENT, UNSUPPORTED (head_dim, topk, dtype
 * combination), WORKSPACE, DEVICE. */
ssa_status ssa_forward(const ssa_blocks *blocks, const ssa_attn *attn, const void *q,
                       const void *k, const void *v, const void *gates, void *out,
                       void *k_cmp, void *v_cmp, int32_t *topk_idx, void *workspace,
                       size_t ws_bytes, void *hip_stream);

/* Largest workspace ssa_forward_noalloc can serve (64 MiB). */
#define SSA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* ssa_forward without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The scratch is a
 * file-scope device array of SSA_NOALLOC_SCRATCH_BYTES inside the library;
 * every GPU it runs on holds its own copy until the process ends.  Arguments,
 * outputs and results are those of ssa_forward (q, k, v, gates, out and the
 * optional k_cmp, v_cmp, topk_idx stay caller-owned).  The device current on
 * the calling thread must be the one hip_stream and the pointers belong to.
 * Every call on one GPU uses that GPU's one array: calls that overlap in time
 * on the same GPU (other streams, other threads) race and must be ordered by
 * the caller.  Each kernel reads only scratch bytes written earlier in the
 * same call, so what a previous call left there does not matter.
 * Errors: as ssa_forward; WORKSPACE when ssa_forward_workspace() for these
 * blocks and this layout exceeds SSA_NOALLOC_SCRATCH_BYTES (nothing is
 * launched); DEVICE when the array's address cannot be obtained. */
ssa_status ssa_forward_noalloc(const ssa_blocks *blocks, const ssa_attn *attn, const void *q,
                               const void *k, const void *v, const void *gates, void *out,
                               void *k_cmp, void *v_cmp, int32_t *topk_idx, void *hip_stream);

/* Stages of ssa_forward, in launch order (indices into stage_ms below). */
enum {
  SSA_STAGE_POOL = 0,        /* mean pooling of keys / values                      */
  SSA_STAGE_ATTN = 1,        /* attention branches (compressed + top-k, selected,   */
                             /* window) and the gated sum                          */
  SSA_STAGE_ATTN2 = 2,       /* a second attention kernel, when the plan has one    */
  SSA_STAGE_ATTN3 = 3,       /* a third attention kernel, when the plan has one     */
  SSA_STAGES = 12
};

/* Same as ssa_forward, but records a hipEvent on hip_stream around every
 * kernel it launches, waits for the stream, and writes each stage's duration
 * in milliseconds to stage_ms[0 .. SSA_STAGES) (0 for stages the plan does
 * not launch).  For profiling and benchmarking; results are identical to
 * ssa_forward.  *n_stages receives the number of stages launched. */
ssa_status ssa_forward_timed(const ssa_blocks *blocks, const ssa_attn *attn, const void *q,
                             const void *k, const void *v, const void *gates, void *out,
                             void *k_cmp, void *v_cmp, int32_t *topk_idx, void *workspace,
                             size_t ws_bytes, void *hip_stream, float *stage_ms, int32_t *n_stages);

/* Name of the kernel that runs stage `stage` for this layout ("" if none). */
const char *ssa_stage_name(const ssa_attn *attn, int32_t stage);

/* ---------------------------------------------------------------- training */

/* SSA forward that also saves what ssa_backward reads.  Same computation and
 * output as ssa_forward (Direct3D-S2 page, "Method"), plus:
 *   topk_idx  required [N, h_kv, topk] int32 (as in ssa_forward).
 *   lse       required [3, N, h_q] float32: for branch x (0 compressed,
 *             1 selected, 2 window) and query (t, h), the natural log of the
 *             softmax denominator, log sum_j exp(scale * q . k_j) over the
 *             branch's keys.
 * Workspace: ssa_forward_workspace() bytes.  Errors as ssa_forward. */
ssa_status ssa_forward_train(const ssa_blocks *blocks, const ssa_attn *attn, const void *q,
                             const void *k, const void *v, const void *gates, void *out,
                             int32_t *topk_idx, float *lse, void *workspace, size_t ws_bytes,
                             void *hip_stream);

/* Workspace bytes ssa_backward needs for these blocks and this layout. */
size_t ssa_backward_workspace(const ssa_blocks *blocks, const ssa_attn *attn);

/* Gradients of L = sum(dout * out), out being the ssa_forward output of the
 * same inputs (Direct3D-S2 page, "Method": out = G0 o_cmp + G1 o_sel + G2
 * o_win, three softmax attentions of the query over the sequence's pooled
 * blocks, the tokens of its top-k blocks and the tokens of its window).
 * The top-k choice is held fixed: it is piecewise constant in q and k, so it
 * has no gradient.  The pooled rows are block means, so each token of block
 * j receives 1 / n_j of its pooled row's gradient; their one rounding to the
 * dtype counts as the identity.
 *   q, k, v, gates  the forward's inputs (layouts as in ssa_forward)
 *   dout      [N, h_q, D]  gradient of the output
 *   topk_idx, lse  as written by ssa_forward_train for these inputs
 *   dq        [N, h_q, D]  out
 *   dk, dv    [N, h_kv, D] out
 *   dgates    optional [N, h_q, 3] out: dout . o_x per branch (NULL = skip)
 *   workspace device scratch of at least ssa_backward_workspace() bytes.
 * All tensors in dtype except lse (float32).  Sums run in float32 in a
 * fixed order, so repeated calls give identical results.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED (as ssa_forward), WORKSPACE, DEVICE. */
ssa_status ssa_backward(const ssa_blocks *blocks, const ssa_attn *attn, const void *q, const void *k,
                        const void *v, const void *gates, const void *dout, const int32_t *topk_idx,
                        const float *lse, void *dq, void *dk, void *dv, void *dgates,
                        void *workspace, size_t ws_bytes, void *hip_stream);

/* Same as ssa_backward, with per-stage times as in ssa_forward_timed. */
ssa_status ssa_backward_timed(const ssa_blocks *blocks, const ssa_attn *attn, const void *q,
                              const void *k, const void *v, const void *gates, const void *dout,
                              const int32_t *topk_idx, const float *lse, void *dq, void *dk,
                              void *dv, void *dgates, void *workspace, size_t ws_bytes,
                              void *hip_stream, float *stage_ms, int32_t *n_stages);

/* Name of backward stage `stage` for this layout ("" if none). */
const char *ssa_backward_stage_name(const ssa_attn *attn, int32_t stage);

/* Static text for a status code. */
const char *ssa_status_string(ssa_status status);

/* Message for the last error on the calling thread ("" if none). */
const char *ssa_last_error(void);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int32_t ssa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSA_H */
