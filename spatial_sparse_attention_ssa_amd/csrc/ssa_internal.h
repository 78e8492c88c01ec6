// Internal declarations shared by the HIP translation units of libssa.
// gfx950 (CDNA4) only: wave64, MFMA, 160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssa.h"

namespace ssa {

constexpr int kWave = 64;

// ---------------------------------------------------------------- numerics

// Orders LDS traffic of one wave around a point where lanes exchange data
// through LDS (a wave issues its LDS operations in order; this keeps the
// compiler from moving memory operations across it).
__device__ __forceinline__ void wave_lds_sync() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_wave_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Instruction-scheduling pattern for the region that ends here: kMfma times
// (one MFMA, then up to kValu vector ALU instructions).  An MFMA runs for many
// cycles after issue, and the same wave can issue independent VALU work
// meanwhile; the compiler otherwise tends to cluster the MFMAs.
template <int kMfma, int kValu>
__device__ __forceinline__ void interleave_mfma_valu() {
  if constexpr (kMfma > 0) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);
    interleave_mfma_valu<kMfma - 1, kValu>();
  }
}

typedef short tr_s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) tr_s16x4 lds_tr_s16x4;
typedef __bf16 tr_bf16x8 __attribute__((ext_vector_type(8)));

// One v_mfma_f32_32x32x16_bf16 A operand (32 dims x 16 rows; lane half h
// holds rows {0-3, 8-11} + 4 h of the 16, the k order in which a 32x32
// accumulator feeds the next MFMA as its B operand) of a tile of rows stored
// row-major in LDS (row stride kRowP elements), read with gfx950's
// transposing LDS load (ds_read_b64_tr_b16): within each 16-lane
// group, output lane 4a + b receives element b of the 4-element chunks that
// source lanes a, a + 4, a + 8 and a + 12 address.  So source lane
// (g, a, i) = (lane / 16, lane % 4, lane % 16 / 4) addresses row
// 16 ks + 4 (g / 2) + i (plus 8 for the operand's upper four k slots) at dims
// 32 x + 16 (g % 2) + 4 a, and lane l receives dim 32 x + l % 32 of rows
// 16 ks + 4 (l / 32) + {0..3} and 16 ks + 8 + 4 (l / 32) + {0..3}: the rows
// that k slots 8 (l / 32) + {0..7} hold.
template <int kRowP>
__device__ __forceinline__ tr_bf16x8 lds_tr_operand(const uint16_t* tile, int lane, int x, int ks) {
  const int g = lane >> 4;
  const int row = 16 * ks + 4 * (g >> 1) + ((lane & 15) >> 2);
  const int dim = 32 * x + 16 * (g & 1) + 4 * (lane & 3);
  const uint16_t* p0 = tile + row * kRowP + dim;
  const tr_s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_tr_s16x4*)(p0));
  const tr_s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_tr_s16x4*)(p0 + 8 * kRowP));
  const tr_s16x4 v[2] = {lo, hi};
  return __builtin_bit_cast(tr_bf16x8, v);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float32 -> bfloat16 bits (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

constexpr float kLn2 = 0.69314718055994531f;

// Four float32 values rounded to bfloat16 and stored as 8 bytes.
__device__ __forceinline__ void store_bf16x4(uint16_t* dst, float a, float b, float c, float d) {
  uint2 w;
  w.x = static_cast<uint32_t>(f32_to_bf16_bits(a)) | (static_cast<uint32_t>(f32_to_bf16_bits(b)) << 16);
  w.y = static_cast<uint32_t>(f32_to_bf16_bits(c)) | (static_cast<uint32_t>(f32_to_bf16_bits(d)) << 16);
  *reinterpret_cast<uint2*>(dst) = w;
}

// Element access for the two storage types: float, or bfloat16 carried as
// its 16-bit pattern.
template <typename T> struct Elt;
template <> struct Elt<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
};
template <> struct Elt<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p) { return bf16_bits_to_f32(*p); }
  static __device__ __forceinline__ void store(uint16_t* p, float v) { *p = f32_to_bf16_bits(v); }
};

// ---------------------------------------------------------------- block build

// Bit layout of the block key (all fields are powers of two).
struct KeyLayout {
  int l_rw;      // log2(R / m_win): bits per axis of the window cell
  int l_r;       // log2(m_win / m_cmp): bits per axis of the block cell inside a window
  int l_win;     // log2(m_win)
  int l_cmp;     // log2(m_cmp)
  int seq_bits;  // ceil(log2(B))
  int key_bits;  // seq_bits + 3 * (l_rw + l_r)
  int grid_res;
  int shift;     // window origin at -shift per axis (a multiple of m_cmp), 0 = unshifted
};

constexpr int kSortTile = 4096;   // keys per workgroup tile (256 threads x 16)
constexpr int kRadixBits = 8;
constexpr int kMaxPasses = 4;     // 8-bit digits of a 32-bit key

struct BuildWorkspace {
  uint32_t* keys_a;      // [N]
  uint32_t* keys_b;      // [N]
  int32_t* vals_b;       // [N]
  // one-sweep sort (small builds; null otherwise)
  uint32_t* glob_hist;   // [kMaxPasses][256] keys of each digit, per pass
  int32_t* tile_ctr;     // [kMaxPasses] next tile of each pass
  uint64_t* tile_state;  // [kMaxPasses][ntiles][256] look-back words
  // reduce-then-scan passes (large builds; null otherwise)
  uint32_t* tile_hist;   // [256 * ntiles] plus the scan's chunk sums
  // segment pass: one look-back kernel (smaller builds) or count / scan /
  // write kernels (larger builds); the other path's pointers are null
  uint64_t* seg_state;   // [ntiles] look-back words
  int32_t* seg_ctr;      // next tile
  int32_t* tile_cnt;     // [2 * ntiles]
  int32_t* tile_base;    // [2 * ntiles]
};

size_t build_workspace_bytes(int64_t n, int32_t batch);
void carve_build_workspace(void* ws, int64_t n, BuildWorkspace* out);

hipError_t launch_build(const int32_t* coords, const int32_t* cu_seqlens, int32_t n, int32_t batch,
                        const KeyLayout& kl, const ssa_blocks& out, const BuildWorkspace& ws,
                        hipStream_t stream);

// Stable LSD radix sort of (key, value) pairs by the low `key_bits` bits of
// the keys, 8 bits per pass, ping-ponging between (keys, vals) and the tmp
// pair: the result lands in the tmp pair when the pass count is odd.
bool sort_pairs_lands_in_tmp(int key_bits);
size_t sort_pairs_hist_bytes(int64_t n);
hipError_t launch_sort_pairs(uint32_t* keys, int32_t* vals, uint32_t* keys_tmp, int32_t* vals_tmp, int32_t n,
                             int key_bits, uint32_t* tile_hist, hipStream_t stream);

// ---------------------------------------------------------------- forward

struct FwdParams {
  // blocks
  const int32_t* perm;
  const int32_t* blk_off;
  const int32_t* win_off;
  const int32_t* seq_blk_off;
  const int32_t* seq_win_off;
  const int32_t* counts;
  int32_t n;         // tokens
  int32_t batch;
  int32_t nb_cap;    // row capacity of the internal pooled arrays
  // layout
  int32_t h_q, h_kv, d, topk;
  float scale;
  // tensors (input order)
  const void* q;
  const void* k;
  const void* v;
  const void* gates;
  void* out;
  // pooled keys / values, internal layout [h_kv][nb_cap][D] in the input dtype
  // (nb_cap is a multiple of 32; rows nb..nb_cap are zero)
  void* kbar;
  void* vbar;
  // pooled values for the MFMA path: [h_kv][nb_cap/32][D][32], keys of each
  // 32-block tile in the order the MFMA B operand of P^T expects (null = skip)
  void* vbar_t;
  // keys / values in sorted token order, head-major [h_kv][N][D] (MFMA path;
  // written by the pooling kernel; null = skip)
  void* k_s;
  void* v_s;
  // MFMA path scratch
  int32_t* tile_pre;  // [batch + 1] prefix of query tiles per sequence
  int32_t* fix;       // [1 + n * h_kv] overflow counter, then (token * h_kv + group) entries
  float* acc;         // [n][h_q][D] partial sum of the gated branches (input token order)
  int32_t max_tiles;  // upper bound of query tiles
  // probe set of the one-head-per-group compressed kernel (bf16, D = 64): for
  // every sequence with more than kProbeBlocks blocks, per head, the
  // kProbeBlocks pooled keys of largest norm (null = no probes)
  float* knorm2;         // [h_kv][nb_cap] squared norm of each pooled key row (written by pooling)
  int32_t* probe_slot;   // [batch + 1] probe slot of each sequence or -1; [batch] = slots used
  int32_t* probe_seq;    // [max_probe_slots] sequence of each slot
  float* probe_maxn2;    // [h_kv][max_probe_slots] largest squared key norm of the slot's sequence
  void* probe;           // [h_kv][max_probe_slots][kProbeBlocks][D] the probe keys, in block order (or null)
  int32_t* probe_ids;    // [h_kv][max_probe_slots][kProbeBlocks] their block ids (or null)
  int32_t max_probe_slots;
  // grouped-head path: log2 softmax normaliser per (token, query head), and
  // the prefix of 16-token tiles per sequence
  float* norm;        // [n][h_q]
  int32_t* tile_pre2; // [batch + 1]
  int32_t max_tiles2;
  float* seq_kmax2;   // [h_kv][batch] largest squared pooled-key norm of each sequence (knorm2 above)
  // optional public outputs
  void* k_cmp;       // [nb][h_kv][D] or null
  void* v_cmp;
  int32_t* topk_idx; // [N][h_kv][topk]  (always valid: library workspace when the caller passes null)
  // training: the state the backward reads (null = plain forward)
  float* lse;        // [3][n][h_q] natural-log softmax denominators of the
                     // (compressed, selected, window) branches, input token order
  // geometric routing
  const int32_t* coords;   // [n][3] token coordinates (input order)
  int4* blk_cell;          // [nb_cap] the m_cmp^3 cell of each block
  int32_t l_cmp;           // log2(m_cmp)
};

// Backward pass: the forward's parameters plus the gradients and scratch.
struct BwdParams {
  FwdParams f;          // blocks, layout, inputs, pooled rows, sorted K / V copies
  const void* dout;     // [n][h_q][D] gradient of the output
  const float* lse;     // [3][n][h_q] natural-log softmax denominators (saved by the forward)
  void* dq;             // [n][h_q][D] out
  void* dk;             // [n][h_kv][D] out
  void* dv;
  void* dgates;         // [n][h_q][3] out, or null
  float* delta;         // [3][n][h_q] Delta_x = sum_j P_j (dout . v_j), i.e. dout . o_x
  float* dq_acc;        // [n][h_q][D]
  float* dk_acc;        // [h_kv][n][D], sorted token order
  float* dv_acc;
  float* dkbar;         // [h_kv][nb_cap][D] gradients of the pooled rows
  float* dvbar;
  // inverted top-k lists: every (token, group, rank) entry keyed by
  // group * nb_cap + block, stably sorted, so that each list holds its
  // selecting tokens in increasing order
  uint32_t* sel_keys;   // [n * h_kv * topk] keys (input of the sort)
  int32_t* sel_vals;    // [n * h_kv * topk] selecting token (input of the sort)
  uint32_t* sel_keys_tmp;
  int32_t* sel_vals_tmp;
  uint32_t* sel_hist;   // radix sort tile histograms
  int32_t sel_key_bits;
  int32_t* sel_off;     // [h_kv * nb_cap + 1] start of each list in sel_list
  int32_t* sel_list;    // the sorted tokens (one of the two value buffers)
  const uint32_t* sel_sorted_keys;   // the sorted keys (one of the two key buffers)
  // MFMA kernels of the compressed branch (bf16)
  int32_t* qtile_pre;   // [batch + 1] prefix of 128-query tiles per sequence
  int32_t* btile_pre;   // [batch + 1] prefix of 128-block chunks per sequence, in seq_order
  int32_t* seq_order;   // [batch] sequences by decreasing token count (ties: lower index first)
  int32_t max_qtiles;   // grid bounds of the two
  int32_t max_btiles;
  // (query, head) rows of each group in sorted order: row R = i * G + hh is
  // query head g * G + hh of the token at sorted position i
  int32_t rows_cap;     // n * G rounded up to 32
  void* q_rows;         // [h_kv][rows_cap][D] Q rows (bf16)
  void* do_rows;        // [h_kv][rows_cap][D] dO rows
  float4* st_rows;      // [2][h_kv][rows_cap] (log2 lse, Delta, gate) of the compressed / window branch
  int32_t row_splits;   // the pooled-row gradients are summed over this many row ranges
  float* dkbar_part;    // [row_splits][h_kv][nb_cap][D] partial sums (row_splits > 1)
  float* dvbar_part;
};

constexpr int kKeyTile = 32;     // pooled blocks per MFMA key tile
constexpr int kQueryTile = 256;  // queries per workgroup of the compressed MFMA kernel (4 waves x 64)
constexpr int kProbeBlocks = 512;  // pooled keys per probe set (16 key tiles)

hipError_t launch_pool(const FwdParams& p, ssa_dtype dtype, hipStream_t stream);
void tile_prefix_kernel_launch(const FwdParams& p, hipStream_t stream);
// probe sets (needs the pooled-key norms and the probe slots of tile_prefix_kernel)
void probe_select_launch(const FwdParams& p, hipStream_t stream);
hipError_t launch_gqa_cmp(const FwdParams& p, ssa_dtype dtype, hipStream_t stream);
hipError_t launch_gqa_topk(const FwdParams& p, ssa_dtype dtype, hipStream_t stream);
hipError_t launch_geo_topk(const FwdParams& p, ssa_dtype dtype, hipStream_t stream);

// backward stages (ssa_bwd.hip, ssa_bwd_mfma.hip)
hipError_t launch_bwd_pool(const BwdParams& p, ssa_dtype dtype, hipStream_t stream);
hipError_t launch_bwd_sel_index(const BwdParams& p, ssa_dtype dtype, hipStream_t stream);
hipError_t launch_bwd_cmp_dq(const BwdParams& p, ssa_dtype dtype, hipStream_t stream);
hipError_t launch_bwd_cmp_dkv(const BwdParams& p, ssa_dtype dtype, hipStream_t stream);
hipError_t launch_bwd_win_dq(const BwdParams& p, ssa_dtype dtype, hipStream_t stream);
hipError_t launch_bwd_win_dkv(const BwdParams& p, ssa_dtype dtype, hipStream_t stream);
hipError_t launch_bwd_sel_dkv(const BwdParams& p, ssa_dtype dtype, hipStream_t stream);
hipError_t launch_bwd_sel_dq(const BwdParams& p, ssa_dtype dtype, hipStream_t stream);
hipError_t launch_bwd_finalize(const BwdParams& p, ssa_dtype dtype, hipStream_t stream);
hipError_t launch_bwd_cmp_dq_mfma(const BwdParams& p, ssa_dtype dtype, hipStream_t stream);
hipError_t launch_bwd_cmp_dkv_mfma(const BwdParams& p, ssa_dtype dtype, hipStream_t stream);
hipError_t launch_bwd_win_dq_mfma(const BwdParams& p, ssa_dtype dtype, hipStream_t stream);
hipError_t launch_bwd_kv_sel_mfma(const BwdParams& p, ssa_dtype dtype, hipStream_t stream);
hipError_t launch_bwd_kv_win_mfma(const BwdParams& p, ssa_dtype dtype, hipStream_t stream);
hipError_t launch_bwd_rows_prep(const BwdParams& p, ssa_dtype dtype, hipStream_t stream);
hipError_t launch_cmp_probe(const FwdParams& p, ssa_dtype dtype, hipStream_t stream);
hipError_t launch_cmp_mfma(const FwdParams& p, ssa_dtype dtype, hipStream_t stream);
hipError_t launch_topk_fixup(const FwdParams& p, ssa_dtype dtype, hipStream_t stream);
hipError_t launch_win_mfma(const FwdParams& p, ssa_dtype dtype, hipStream_t stream);
hipError_t launch_vt_transpose(const FwdParams& p, ssa_dtype dtype, hipStream_t stream);
hipError_t launch_sel_combine(const FwdParams& p, ssa_dtype dtype, hipStream_t stream);
hipError_t launch_generic(const FwdParams& p, ssa_dtype dtype, hipStream_t stream);

}  // namespace ssa
