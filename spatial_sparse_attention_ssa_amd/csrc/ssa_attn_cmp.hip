// Compressed-block attention with top-k block selection, on MFMA (bf16, D = 32
// or 64, one query head per key/value head).
//
// Direct3D-S2 page, "Method": every query attends to the mean-pooled blocks of
// its sequence, and the same query-to-block scores choose the top-k blocks
// for the selection branch.  With one query head per key/value group the
// score order is the logit order (softmax is monotone), so the ranking uses
// float32 logits; ties go to the lower block id.
//
// Work split: a workgroup owns 256 consecutive sorted queries of one sequence
// and one head; each of its 4 waves owns 64 queries as two 32-query blocks A
// and B.  The sequence's pooled keys and values stream through a two-slot LDS
// ring in tiles of 32 blocks (one barrier per tile, global loads one tile
// ahead).  A wave reads each tile's MFMA operands from LDS once into registers
// and uses them for both query blocks, which halves the LDS traffic per MFMA
// against one block per wave.  Each product is a v_mfma_f32_32x32x16_bf16
// S^T = Kbar Q^T; lane l then holds 16 block logits of query l % 32 of a block
// (lanes l and l ^ 32 split the row between them).  The two blocks form a
// software pipeline inside the wave: the MFMAs of one block are issued next to
// the VALU work of the other (MFMA and VALU overlap only within one wave's
// instruction stream on this hardware).
//
// Two passes over the keys:
//  1. scan: per lane and block, the maximum of a group of the lane's logits
//     (4 to 32 of them, chosen per sequence) is merged into a sorted list of
//     the KMAX largest group maxima with v_med3 (for a descending list L, inserting x gives
//     L'[i] = med3(L[i-1], x, L[i])).  The row maximum is max(L0 of both
//     lanes).  For every split a + b = KMAX the two lanes hold a + b distinct
//     elements no smaller than min(L_A[a-1], L_B[b-1]); the largest such value,
//     tau, bounds the KMAX-th (so also the k-th, k <= KMAX) largest logit from
//     below.
//  2. attend: x = (s - tau') * scale * log2 e with tau' = tau lowered by a
//     small relative slack (rounding differences between the passes); the
//     sign bit of x says whether the logit can be in the top-k, and p = 2^x is
//     the softmax numerator shifted by tau' instead of the row maximum (the
//     shift cancels in the normalisation; a row whose maximum lies so far above
//     tau' that 2^x could overflow uses the maximum and takes the fallback).
//     O^T += Vbar^T P^T on MFMA with P truncated to bf16 (one v_perm_b32 per
//     pair; the mean truncation loss is compensated by a constant factor), the
//     row sum over the float32 p, and one v_alignbit per logit packs the 16
//     sign bits of a tile; a tile with any candidate appends one word (tile,
//     bit mask) to the lane's LDS list.
//     There is no per-logit branch.
// Afterwards each lane recomputes its candidates' logits in float32 from the
// pooled keys, and each candidate's rank among the query's candidates (value
// descending, block ascending) places it in the output.  A query whose lists
// overflow goes to the exact fallback kernel below.
#include <float.h>

#include <type_traits>

#include "ssa_internal.h"

namespace ssa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kVRow = kKeyTile + 8;    // LDS row of a transposed value tile (bf16)
// tile shapes for head dim D (32 or 64)
template <int D>
struct CmpDims {
  static constexpr int kKRow = D + 8;            // LDS row of a key tile (bf16), padded against bank conflicts
  static constexpr int kKTileElems = kKeyTile * kKRow;
  static constexpr int kVTileElems = D * kVRow;
  static constexpr int KS = D / 16;              // MFMA k steps over the dims
  static constexpr int VB = D / 32;              // 32-dim row blocks of O^T
  static constexpr int kKStagers = kKeyTile * (D / 8);   // threads that stage a key tile (16 bytes each)
  static constexpr int kVStagers = D * 4;                // threads that stage a value tile
};
constexpr int kBlockQ = 32;            // queries per MFMA column block
// bf16 P by truncation: the mean relative loss of truncating a float32 with
// a log-uniform mantissa to 8 significant bits is 2^-8 * (1/ln 2) * (1/2);
// p is scaled up by the inverse factor (an exponent offset of log2 of it) and
// the row sum divided by it again, so P V and the row sum agree on average
constexpr float kTruncLog2 = 0.0040711f;   // log2(1 / (1 - 2^-8 * 0.5 / ln 2))
constexpr float kTruncInv = 0.99718215f;   // 1 - 2^-8 * 0.5 / ln 2

// float -> uint32 with the same order (finite values; -0 and +0 both map to
// the image of +0)
__device__ __forceinline__ uint32_t ordered_bits(float v) {
  const uint32_t b = __float_as_uint(v + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// inverse of ordered_bits
__device__ __forceinline__ float ordered_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// the larger 64-bit key of this lane and the lane that the DPP control CTRL
// selects (the two 32-bit halves moved by two DPP moves)
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max_key(uint64_t k) {
  const uint32_t hi = static_cast<uint32_t>(k >> 32), lo = static_cast<uint32_t>(k);
  const uint32_t ohi = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(hi), static_cast<int>(hi), CTRL, 0xF, 0xF, false));
  const uint32_t olo = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(lo), static_cast<int>(lo), CTRL, 0xF, 0xF, false));
  const uint64_t o = (static_cast<uint64_t>(ohi) << 32) | olo;
  return o > k ? o : k;
}

// the largest 64-bit key of the wave, on every lane: DPP butterflies within
// 16-lane rows (lane ^ 1, lane ^ 2, then the mirrors of 8 and 16 lanes), a
// lane shuffle across rows, and v_permlane32_swap across the halves
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k) {
  k = dpp_max_key<0xB1>(k);    // quad_perm [1,0,3,2]
  k = dpp_max_key<0x4E>(k);    // quad_perm [2,3,0,1]
  k = dpp_max_key<0x141>(k);   // row_half_mirror
  k = dpp_max_key<0x140>(k);   // row_mirror
  {
    const uint32_t hi = static_cast<uint32_t>(k >> 32), lo = static_cast<uint32_t>(k);
    const uint64_t o = (static_cast<uint64_t>(static_cast<uint32_t>(__shfl_xor(static_cast<int>(hi), 16))) << 32) |
                       static_cast<uint32_t>(__shfl_xor(static_cast<int>(lo), 16));
    k = o > k ? o : k;
  }
  {
    const uint32_t hi = static_cast<uint32_t>(k >> 32), lo = static_cast<uint32_t>(k);
    const auto rh = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    const auto rl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const uint64_t a = (static_cast<uint64_t>(rh[0]) << 32) | rl[0];
    const uint64_t b = (static_cast<uint64_t>(rh[1]) << 32) | rl[1];
    k = a > b ? a : b;
  }
  return k;
}

// maxima of logits (never NaN here) as explicit three-operand trees, which
// become v_maximum3_f32
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmax3(float a, float b, float c) { return vmax(vmax(a, b), c); }

__device__ __forceinline__ bf16x8 lds_b128(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// sorted position of sequence b's first token and one past its last
__device__ __forceinline__ void seq_token_range(const FwdParams& p, int b, int* s0, int* s1) {
  *s0 = p.win_off[p.seq_win_off[b]];
  *s1 = p.win_off[p.seq_win_off[b + 1]];
}

// tile_pre[b] = number of query tiles of sequences before b; with probes,
// also the probe slot of every sequence with more than kProbeBlocks blocks
__global__ void tile_prefix_kernel(FwdParams p) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int run = 0, slots = 0;
  for (int b = 0; b < p.batch; ++b) {
    p.tile_pre[b] = run;
    int s0, s1;
    seq_token_range(p, b, &s0, &s1);
    run += (s1 - s0 + kQueryTile - 1) / kQueryTile;
    if (p.probe_slot) {
      int slot = -1;
      if (p.seq_blk_off[b + 1] - p.seq_blk_off[b] > kProbeBlocks && slots < p.max_probe_slots) {
        slot = slots++;
        p.probe_seq[slot] = b;
      }
      p.probe_slot[b] = slot;
    }
  }
  p.tile_pre[p.batch] = run;
  if (p.probe_slot) p.probe_slot[p.batch] = slots;
  p.fix[0] = 0;
}

// Probe set of one (sequence, head): the kProbeBlocks pooled keys of largest
// squared norm, copied in block order (when p.probe is set), their block ids
// (when p.probe_ids is set), and the largest squared norm.  Any
// set of the sequence's blocks gives a valid lower bound on its k-th largest
// logit (the compressed kernel's first pass); blocks of large key norm give
// a tight one, since a logit is at most |q| |Kbar_j|.  The selection is a
// 1024-bin histogram of the norms' top bits: every block of a bin above the
// threshold bin, then the lowest-numbered blocks of the threshold bin until
// kProbeBlocks are chosen.
__global__ void __launch_bounds__(256)
probe_select_kernel(FwdParams p) {
  constexpr int kBins = 1024;
  __shared__ int hist[kBins];
  __shared__ int wcnt[2][4];
  __shared__ float wmax[4];
  __shared__ int sh_bin, sh_need;
  const int s = blockIdx.x, g = blockIdx.y;
  if (s >= p.probe_slot[p.batch]) return;   // uniform over the workgroup
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int b = p.probe_seq[s];
  const int j0 = p.seq_blk_off[b], nbs = p.seq_blk_off[b + 1] - j0;   // nbs > kProbeBlocks
  const float* n2 = p.knorm2 + static_cast<int64_t>(g) * p.nb_cap + j0;
  for (int i = tid; i < kBins; i += 256) hist[i] = 0;
  __syncthreads();
  float mx = 0.f;
  for (int j = tid; j < nbs; j += 256) {
    const float v = n2[j];   // >= 0: the bits order like the values
    mx = fmaxf(mx, v);
    atomicAdd(&hist[__float_as_uint(v) >> 21], 1);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (lane == 0) wmax[wv] = mx;
  __syncthreads();
  if (wv == 0) {
    // lane l counts bins 1023 - 16 l - (0..15); an inclusive scan over the
    // lanes runs from the top bin down, and the lane where it reaches
    // kProbeBlocks finds the threshold bin in its range
    int c = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) c += hist[kBins - 1 - 16 * lane - i];
    int incl = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off);
      if (lane >= off) incl += t;
    }
    const int excl = incl - c;
    if (excl < kProbeBlocks && incl >= kProbeBlocks) {
      int cum = excl;
      for (int i = 0; i < 16; ++i) {
        const int bin = kBins - 1 - 16 * lane - i;
        if (cum + hist[bin] >= kProbeBlocks) {
          sh_bin = bin;
          sh_need = kProbeBlocks - cum;
          break;
        }
        cum += hist[bin];
      }
    }
    if (lane == 0)
      p.probe_maxn2[g * p.max_probe_slots + s] = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  }
  __syncthreads();
  const int tbin = sh_bin, need = sh_need;
  const int dh = p.d;   // 32 or 64
  const uint16_t* src = static_cast<const uint16_t*>(p.kbar) + (static_cast<int64_t>(g) * p.nb_cap + j0) * dh;
  const int64_t set = static_cast<int64_t>(g) * p.max_probe_slots + s;
  uint16_t* dst = p.probe ? static_cast<uint16_t*>(p.probe) + set * kProbeBlocks * dh : nullptr;
  int32_t* ids = p.probe_ids ? p.probe_ids + set * kProbeBlocks : nullptr;
  const uint64_t below = (uint64_t(1) << lane) - 1;
  int base_gt = 0, base_eq = 0;   // chosen blocks above / in the threshold bin before this chunk
  for (int c0 = 0; c0 < nbs; c0 += 256) {
    const int j = c0 + tid;
    const int bin = j < nbs ? static_cast<int>(__float_as_uint(n2[j]) >> 21) : -1;
    const bool gt = bin > tbin, eq = bin == tbin;
    const uint64_t bg = __ballot(gt), be = __ballot(eq);
    if (lane == 0) {
      wcnt[0][wv] = __popcll(bg);
      wcnt[1][wv] = __popcll(be);
    }
    __syncthreads();
    int pgt = base_gt + __popcll(bg & below), peq = base_eq + __popcll(be & below);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (w < wv) {
        pgt += wcnt[0][w];
        peq += wcnt[1][w];
      }
      base_gt += wcnt[0][w];
      base_eq += wcnt[1][w];
    }
    __syncthreads();   // wcnt is rewritten by the next chunk
    if (gt || (eq && peq < need)) {
      // position among the chosen blocks, in block order
      const int pos = pgt + min(peq, need);
      if (ids) ids[pos] = j0 + j;
      if (dst) {
        const u32x4* from = reinterpret_cast<const u32x4*>(src + static_cast<int64_t>(j) * dh);
        u32x4* to = reinterpret_cast<u32x4*>(dst + static_cast<int64_t>(pos) * dh);
        for (int c = 0; c < dh / 8; ++c) to[c] = from[c];
      }
    }
  }
}

template <int KMAX, int D>
struct CmpShape {
  // candidate slots per query, shared by its two lanes (with the bound above
  // a query rarely has more than KMAX + 6; overflow goes to the fallback)
  static constexpr int kCap = KMAX + KMAX / 2 + 2;
  // hit-tile words per lane and block (a lane typically has about KMAX / 2
  // candidates)
  static constexpr int kEnt = KMAX <= 16 ? 20 : 36;
  static constexpr int kRingBytes = 2 * (CmpDims<D>::kKTileElems + CmpDims<D>::kVTileElems) * 2;
  // candidate lists of one query block of every wave (the blocks take turns):
  // per query kSlots 64-bit keys (kSlots even, so a query's keys start on a
  // 16-byte boundary)
  static constexpr int kSlots = kCap + 2;
  static_assert(kSlots % 2 == 0, "a query's key row must be whole 16-byte words");
  static constexpr int kCandSlots = 4 * kBlockQ * kSlots;
  static constexpr int kCandBytes = kCandSlots * 8;
  static constexpr int kSmem = kRingBytes > kCandBytes ? kRingBytes : kCandBytes;
};

// Per-lane state of one 32-query block.
template <int KMAX, int D>
struct QBlock {
  bf16x8 qb[D / 16];  // Q^T B operand: query (l % 32), d = 16 ks + 8 half + 0..7
  const uint16_t* q_row;
  int qi;             // sorted position
  int t;              // token (input order)
  bool valid;
  float L[KMAX];      // pass 1: descending list of group maxima
  float g;            // pass 1: running maximum of the open group
  f32x16 s;           // logits of the tile in flight
  f32x16 o[D / 32];    // O^T, dims 32 vb .. 32 vb + 31
  float l0, l1;       // row-sum partials
  float k0;           // exponent offset: x = s * c2 + k0
  uint32_t f_or, f_and;
  bool to_fix;        // the fallback computes this query's top-k
  int ecnt;           // hit-tile words written
};

template <int KMAX, int D>
__global__ void __launch_bounds__(256, 2)
cmp_mfma_kernel(FwdParams p) {
  using Shape = CmpShape<KMAX, D>;
  using Dims = CmpDims<D>;
  constexpr int kD = D;
  constexpr int kKRow = Dims::kKRow;
  constexpr int kKTileElems = Dims::kKTileElems;
  constexpr int kVTileElems = Dims::kVTileElems;
  constexpr int KS = Dims::KS;
  constexpr int VB = Dims::VB;
  constexpr int kCap = Shape::kCap;
  constexpr int kEnt = Shape::kEnt;
  // the key/value ring while the passes run; afterwards the same bytes hold
  // the candidate lists of one query block: per query kCap data slots
  // 1..kCap plus a sink slot at each end that absorbs writes past the
  // capacity.  A slot is one 64-bit key whose unsigned order is the ranking
  // order: the high word is the logit mapped to an order-preserving integer,
  // the low word the complement of the block id relative to the sequence's
  // first key tile (sequences with 65536 or more blocks take the fallback);
  // an unused slot is 0, below every key.
  __shared__ __align__(16) uint8_t smem[Shape::kSmem];
  // hit-tile words: word e of block x of thread t at [(2 e + x) * 256 + t];
  // word kEnt is a sink
  __shared__ uint32_t ent[(kEnt + 1) * 2 * 256];
  uint16_t* const k_lds = reinterpret_cast<uint16_t*>(smem);
  uint16_t* const v_lds = k_lds + 2 * kKTileElems;
  uint64_t* const cand_key = reinterpret_cast<uint64_t*>(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int half = lane >> 5;          // which 8-wide k slice / which half of the keys
  const int h = blockIdx.y;            // query head == key/value head
  const int tile = blockIdx.x;
  if (tile >= p.tile_pre[p.batch]) return;  // uniform over the workgroup

  // tile -> sequence b and its query range
  int lo = 0, hi = p.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.tile_pre[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  int s0, s1;
  seq_token_range(p, b, &s0, &s1);
  const int q_begin = s0 + (tile - p.tile_pre[b]) * kQueryTile;
  const int q_end = min(q_begin + kQueryTile, s1);
  const int j0 = p.seq_blk_off[b], j1 = p.seq_blk_off[b + 1];
  const int nbs = j1 - j0;

  const uint16_t* Q = static_cast<const uint16_t*>(p.q);
  QBlock<KMAX, D> blk[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    QBlock<KMAX, D>& B = blk[x];
    B.qi = q_begin + wv * 64 + x * kBlockQ + (lane & 31);
    B.valid = B.qi < q_end;
    B.t = B.valid ? p.perm[B.qi] : 0;
    B.q_row = Q + (static_cast<int64_t>(B.t) * p.h_q + h) * kD;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 u = {0u, 0u, 0u, 0u};
      if (B.valid) u = *reinterpret_cast<const u32x4*>(B.q_row + 16 * ks + 8 * half);
      B.qb[ks] = __builtin_bit_cast(bf16x8, u);
    }
  }

  const uint16_t* KB = static_cast<const uint16_t*>(p.kbar) + static_cast<int64_t>(h) * p.nb_cap * kD;
  const uint16_t* VT = static_cast<const uint16_t*>(p.vbar_t) + static_cast<int64_t>(h) * p.nb_cap * kD;
  const int kt0 = j0 / kKeyTile, kt1 = (j1 + kKeyTile - 1) / kKeyTile;
  const int n_kt = kt1 - kt0;

  // cooperative tile staging: thread -> 16 bytes of the key tile / value tile
  // (D = 32: the first 128 threads stage each tile)
  const int k_row = tid / (kD / 8), k_chunk = tid % (kD / 8);   // key tile: 32 rows x D / 8 chunks
  const int v_row = tid >> 2, v_chunk = tid & 3;                // value tile: D rows x 4 chunks
  // (compile-time true when every thread stages)
  const bool k_stager = Dims::kKStagers >= 256 || tid < Dims::kKStagers;
  const bool v_stager = Dims::kVStagers >= 256 || tid < Dims::kVStagers;
  const uint16_t* kg = KB + (static_cast<int64_t>(kt0) * kKeyTile + k_row) * kD + 8 * k_chunk;
  const uint16_t* vg = VT + (static_cast<int64_t>(kt0) * kD + v_row) * kKeyTile + 8 * v_chunk;
  auto load_k = [&](int rel) {
    u32x4 u = {0u, 0u, 0u, 0u};
    if (k_stager) u = *reinterpret_cast<const u32x4*>(kg + static_cast<int64_t>(rel) * kKeyTile * kD);
    return u;
  };
  auto load_v = [&](int rel) {
    u32x4 u = {0u, 0u, 0u, 0u};
    if (v_stager) u = *reinterpret_cast<const u32x4*>(vg + static_cast<int64_t>(rel) * kKeyTile * kD);
    return u;
  };
  const int ks_dst = k_row * kKRow + 8 * k_chunk;
  const int vs_dst = v_row * kVRow + 8 * v_chunk;
  const int ka = (lane & 31) * kKRow + 8 * half;
  const int va = (lane & 31) * kVRow + 8 * half;
  auto store_k = [&](int slot, const u32x4& u) {
    if (k_stager) *reinterpret_cast<u32x4*>(k_lds + slot * kKTileElems + ks_dst) = u;
  };
  auto store_v = [&](int slot, const u32x4& u) {
    if (v_stager) *reinterpret_cast<u32x4*>(v_lds + slot * kVTileElems + vs_dst) = u;
  };

  // MFMA A operands of key tile rel (slot rel & 1): rows = blocks, k = dims
  auto read_k = [&](int rel, bf16x8 (&a)[KS]) {
    const uint16_t* kl = k_lds + (rel & 1) * kKTileElems + ka;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) a[ks] = lds_b128(kl + 16 * ks);
  };
  // MFMA A operands of value tile rel: rows = dims (0..31, 32..63), k = blocks
  auto read_v = [&](int rel, bf16x8 (&a)[2 * VB]) {
    const uint16_t* vl = v_lds + (rel & 1) * kVTileElems + va;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) a[ks * VB + vb] = lds_b128(vl + vb * 32 * kVRow + 16 * ks);
  };
  auto qk = [&](const bf16x8 (&a)[KS], const bf16x8 (&qb)[KS]) {
    f32x16 s = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], qb[ks], s, 0, 0, 0);
    return s;
  };
  // keys of tile rel outside [j0, j1) get -FLT_MAX; returns the in-range mask
  // (bit 15 - r for accumulator entry r)
  auto mask = [&](int rel, f32x16& s) {
    const int kt = kt0 + rel;
    uint32_t valid = 0u;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = kt * kKeyTile + 8 * (r >> 2) + 4 * half + (r & 3);
      const bool ok = j >= j0 && j < j1;
      if (!ok) s[r] = -FLT_MAX;
      valid = (valid << 1) | (ok ? 1u : 0u);
    }
    return valid;
  };

  // Tile order of both passes: the first and the last tile are the only ones
  // that can hold keys outside [j0, j1); they run in peeled steps with the
  // masking code, the steps in between without it.
  using kT = std::true_type;
  using kF = std::false_type;
  auto run_tiles = [&](auto step) {
    step(0, kT{}, kF{}, kF{});
    if (n_kt == 2) {
      step(1, kT{}, kT{}, kT{});
    } else if (n_kt > 2) {
      step(1, kF{}, kT{}, kT{});
      for (int rel = 2; rel < n_kt - 1; ++rel) step(rel, kF{}, kT{}, kF{});
      step(n_kt - 1, kT{}, kT{}, kF{});
    }
  };

  // ---------------- pass 1: sorted lists of the KMAX largest group maxima
  // A sequence with a probe set (its kProbeBlocks keys of largest norm) runs
  // pass 1 over those 16 tiles instead of all of its tiles, when every query
  // of the workgroup has |q| max_j |Kbar_j| scale log2 e <= 60: every logit s
  // then satisfies |s| c2 <= 60, so x = (s - tau') c2 stays within +-120 and
  // 2^x neither overflows nor flushes the row to zero (the shift by tau' is
  // always safe; the pass never needs the row maximum).
  const float c2 = p.scale * kLog2e;
  const int pslot = p.probe_slot ? p.probe_slot[b] : -1;
  bool probe_ok = true;
  if (pslot >= 0) {
    const float maxn2 = p.probe_maxn2[h * p.max_probe_slots + pslot];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      float qn2 = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float qv = static_cast<float>(blk[x].qb[ks][e]);
          qn2 = fmaf(qv, qv, qn2);
        }
      qn2 += __shfl_xor(qn2, 32);
      // 1 % covers the float32 rounding of the products' sum
      probe_ok = probe_ok && sqrtf(qn2 * maxn2) * 1.01f * c2 <= 60.f;
    }
  }
  const bool use_probe = pslot >= 0 && __syncthreads_and(probe_ok ? 1 : 0);
  const int n1 = use_probe ? kProbeBlocks / kKeyTile : n_kt;
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int i = 0; i < KMAX; ++i) blk[x].L[i] = -FLT_MAX;
  // Group size, per sequence: a group is a run of one lane's logits whose
  // maximum goes into the list.  Larger groups cost fewer list updates but
  // give a looser bound; each lane keeps at least ~48 groups:
  //   glog 32: two tiles (16 logits each), glog 16: one tile,
  //   glog 8: half a tile, glog 4: a quarter tile.
  const int glog = n1 >= 96 ? 32 : n1 >= 48 ? 16 : n1 >= 24 ? 8 : 4;
  auto list_insert = [&](QBlock<KMAX, D>& B, float m) {
#pragma unroll
    for (int i = KMAX - 1; i >= 1; --i) B.L[i] = __builtin_amdgcn_fmed3f(B.L[i - 1], m, B.L[i]);
    B.L[0] = fmaxf(B.L[0], m);
  };
  // the logits of tile rel of block B into its list (glog 32: into the open
  // two-tile group, inserted after the odd tile)
  auto group_update = [&](QBlock<KMAX, D>& B, int rel, auto masked) {
    if (decltype(masked)::value) mask(rel, B.s);
    const f32x16& s = B.s;
    if (glog >= 16) {
      const float m = vmax3(vmax3(vmax3(s[0], s[1], s[2]), vmax3(s[3], s[4], s[5]), vmax3(s[6], s[7], s[8])),
                            vmax3(s[9], s[10], s[11]), vmax3(vmax3(s[12], s[13], s[14]), s[15], B.g));
      if (glog == 16 || (rel & 1)) {
        list_insert(B, m);
        B.g = -FLT_MAX;
      } else {
        B.g = m;
      }
    } else if (glog == 8) {
#pragma unroll
      for (int q8 = 0; q8 < 2; ++q8) {
        const int o = 8 * q8;
        list_insert(B, vmax3(vmax3(s[o], s[o + 1], s[o + 2]), vmax3(s[o + 3], s[o + 4], s[o + 5]), vmax(s[o + 6], s[o + 7])));
      }
    } else {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        list_insert(B, vmax3(vmax(s[4 * q4], s[4 * q4 + 1]), s[4 * q4 + 2], s[4 * q4 + 3]));
    }
  };
  {
    blk[0].g = blk[1].g = -FLT_MAX;
    // pass 1 reads the probe tiles (every row a real key) or the sequence's
    // own tiles
    const uint16_t* kg1 = kg;
    if (use_probe)
      kg1 = static_cast<const uint16_t*>(p.probe) +
            (static_cast<int64_t>(h * p.max_probe_slots + pslot) * kProbeBlocks + k_row) * kD + 8 * k_chunk;
    auto load_k1 = [&](int rel) {
      u32x4 u = {0u, 0u, 0u, 0u};
      if (k_stager) u = *reinterpret_cast<const u32x4*>(kg1 + static_cast<int64_t>(rel) * kKeyTile * kD);
      return u;
    };
    u32x4 kr = {0u, 0u, 0u, 0u};
    store_k(0, load_k1(0));
    if (n1 > 1) kr = load_k1(1);
    // step rel: S of block A for tile rel next to block B's update for tile
    // rel - 1, then S of block B next to block A's update
    auto step = [&](int rel, auto mask_a, auto has_b, auto mask_b) {
      __syncthreads();  // key tile rel stored; everyone is done with tile rel - 1
      if (rel + 1 < n1) store_k((rel + 1) & 1, kr);
      if (rel + 2 < n1) kr = load_k1(rel + 2);
      bf16x8 a[KS];
      read_k(rel, a);
      const f32x16 sa = qk(a, blk[0].qb);
      if (decltype(has_b)::value) group_update(blk[1], rel - 1, mask_b);
      blk[1].s = qk(a, blk[1].qb);
      blk[0].s = sa;
      group_update(blk[0], rel, mask_a);
    };
    if (use_probe) {
      step(0, kF{}, kF{}, kF{});
      for (int rel = 1; rel < n1; ++rel) step(rel, kF{}, kT{}, kF{});
      group_update(blk[1], n1 - 1, kF{});
    } else {
      run_tiles(step);
      group_update(blk[1], n_kt - 1, kT{});
    }
    // an open two-tile group (odd tile count)
    if (glog == 32 && (n1 & 1)) {
      list_insert(blk[0], blk[0].g);
      list_insert(blk[1], blk[1].g);
    }
  }

  // ---------------- per-query constants for pass 2
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    QBlock<KMAX, D>& B = blk[x];
    // row maximum, and the best lower bound on the KMAX-th largest logit
    // (hence on the k-th, k <= KMAX): for any split a + b = KMAX the two
    // lanes hold a and b distinct elements >= min(L_this[a-1], L_other[b-1])
    float Lo[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) Lo[i] = __shfl_xor(B.L[i], 32);
    const float row_max = fmaxf(B.L[0], Lo[0]);
    float tau = fmaxf(B.L[KMAX - 1], Lo[KMAX - 1]);
#pragma unroll
    for (int a = 1; a < KMAX; ++a) tau = fmaxf(tau, fminf(B.L[a - 1], Lo[KMAX - 1 - a]));
    // x = s * c2 + k0: shifted by tau' (sign bit = candidate), or by the row
    // maximum when fewer than KMAX group maxima exist (every real key is a
    // candidate) or when 2^x could overflow (the fallback ranks the query)
    B.k0 = 0.f;
    B.f_or = 0u;
    B.f_and = 0u;
    B.to_fix = false;
    if (B.valid) {
      B.f_and = 0xFFFFu;
      if (tau > -FLT_MAX) {
        const float tp = tau - (fabsf(tau) + fabsf(row_max)) * (1.0f / 4096.0f);
        // with the probe, row_max is only the probe's maximum, but every
        // exponent is bounded (see pass 1)
        if (use_probe || (row_max - tp) * c2 <= 64.f) {
          B.k0 = -tp * c2;
        } else {
          B.k0 = -row_max * c2;
          B.f_and = 0u;
          B.to_fix = true;
        }
      } else {
        B.k0 = -row_max * c2;
        B.f_or = 0xFFFFu;
      }
    }
    B.k0 += kTruncLog2;  // after the sign decisions: the shift is a factor of p only
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) B.o[vb] = f32x16{};
    B.l0 = 0.f;
    B.l1 = 0.f;
    B.ecnt = 0;
  }

  // ---------------- pass 2: probabilities, P V, candidate tiles
  // probabilities, row sums and the candidate word of block x's tile rel;
  // returns P^T as two bf16 B operands (truncated: v_perm_b32 takes the high
  // halves of two float32 values)
  auto softmax_tile = [&](QBlock<KMAX, D>& B, int x, int rel, bf16x8 (&pb)[2], auto masked) {
    uint32_t valid = 0xFFFFu;
    if (decltype(masked)::value) valid = mask(rel, B.s);
    float pr[16];
    uint32_t bits = 0u;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float xr = fmaf(B.s[r], c2, B.k0);
      pr[r] = __builtin_amdgcn_exp2f(xr);
      bits = __builtin_amdgcn_alignbit(bits, __float_as_uint(xr), 31);
    }
    // bit 15 - r set: logit r is >= tau' (a clear sign bit; the truncation
    // offset in k0 lowers tau' a little further, which keeps it a lower bound)
    const uint32_t hit = (~bits | B.f_or) & valid & B.f_and;
    ent[(2 * B.ecnt + x) * 256 + tid] = (static_cast<uint32_t>(rel) << 16) | hit;
    B.ecnt = min(B.ecnt + (hit != 0u ? 1 : 0), kEnt);
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      B.l0 += pr[r];
      B.l1 += pr[r + 1];
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 u;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        u[e] = __builtin_amdgcn_perm(__float_as_uint(pr[8 * ks + 2 * e + 1]), __float_as_uint(pr[8 * ks + 2 * e]),
                                     0x07060302u);
      pb[ks] = __builtin_bit_cast(bf16x8, u);
    }
  };
  auto pv = [&](QBlock<KMAX, D>& B, const bf16x8 (&a)[2 * VB], const bf16x8 (&pb)[2]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int vb = 0; vb < VB; ++vb)
        B.o[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks * VB + vb], pb[ks], B.o[vb], 0, 0, 0);
  };
  {
    u32x4 kr = {0u, 0u, 0u, 0u}, vr = {0u, 0u, 0u, 0u};
    __syncthreads();  // every wave is done with pass 1's ring
    store_k(0, load_k(0));
    store_v(0, load_v(0));
    if (n_kt > 1) {
      kr = load_k(1);
      vr = load_v(1);
    }
    bf16x8 va_prev[2 * VB];   // value tile rel - 1 (MFMA A operands)
    // MFMAs of a step (two blocks' S and P V), and the VALU instructions
    // placed after each (about 160 per step for the two softmaxes)
    constexpr int kStepMfma = 2 * (KS + 2 * VB);
    constexpr int kStepValu = 160 / kStepMfma;
    bf16x8 pa[2];        // P^T of block A for tile rel - 1
    // step rel: block A's P V for tile rel - 1 and its S for tile rel issue
    // next to block B's softmax for tile rel - 1; block B's P V for tile
    // rel - 1 and its S for tile rel issue next to block A's softmax for tile
    // rel.  No MFMA of a step waits for the VALU work of the same step, so the
    // two kinds can interleave.
    auto step = [&](int rel, auto mask_a, auto has_b, auto mask_b) {
      __syncthreads();  // tiles rel stored; everyone is done with the tiles of rel - 1
      if (rel + 1 < n_kt) {
        store_k((rel + 1) & 1, kr);
        store_v((rel + 1) & 1, vr);
      }
      if (rel + 2 < n_kt) {
        kr = load_k(rel + 2);
        vr = load_v(rel + 2);
      }
      bf16x8 a[KS];
      read_k(rel, a);
      if (decltype(has_b)::value) pv(blk[0], va_prev, pa);
      const f32x16 sa = qk(a, blk[0].qb);
      if (decltype(has_b)::value) {
        bf16x8 pb[2];
        softmax_tile(blk[1], 1, rel - 1, pb, mask_b);
        pv(blk[1], va_prev, pb);
      }
      blk[1].s = qk(a, blk[1].qb);
      blk[0].s = sa;
      read_v(rel, va_prev);
      softmax_tile(blk[0], 0, rel, pa, mask_a);
      if (decltype(has_b)::value) interleave_mfma_valu<kStepMfma, kStepValu>();
    };
    run_tiles(step);
    pv(blk[0], va_prev, pa);
    bf16x8 pb[2];
    softmax_tile(blk[1], 1, n_kt - 1, pb, kT{});
    pv(blk[1], va_prev, pb);
  }

  // ---------------- o_cmp (times its gate) added to the branch accumulator (the
  // window kernel, which runs first, wrote it)
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    QBlock<KMAX, D>& B = blk[x];
    const float lsum = B.l0 + B.l1;
    const float lsum_q = lsum + __shfl_xor(lsum, 32);
    const float l_q = lsum_q * kTruncInv;
    if (B.valid) {
      const int64_t row = static_cast<int64_t>(B.t) * p.h_q + h;
      const uint16_t* gt = static_cast<const uint16_t*>(p.gates) + row * 3;
      const float f = bf16_bits_to_f32(gt[0]) / l_q;
      float* dst = p.acc + row * kD;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const int d = 8 * rb + 4 * half;
        float4 a[VB];
#pragma unroll
        for (int vb = 0; vb < VB; ++vb) a[vb] = *reinterpret_cast<float4*>(dst + 32 * vb + d);
#pragma unroll
        for (int vb = 0; vb < VB; ++vb) {
          const f32x16& o = B.o[vb];
          a[vb].x += o[4 * rb] * f; a[vb].y += o[4 * rb + 1] * f; a[vb].z += o[4 * rb + 2] * f; a[vb].w += o[4 * rb + 3] * f;
        }
#pragma unroll
        for (int vb = 0; vb < VB; ++vb) *reinterpret_cast<float4*>(dst + 32 * vb + d) = a[vb];
      }
      if (p.lse && half == 0) {
        // p_j = 2^(s_j scale log2e + k0), so the denominator of the logits is
        // lsum_q * 2^-k0
        p.lse[row] = (__log2f(lsum_q) - B.k0) * kLn2;
      }
    }
  }

  // ---------------- exact top-k, one query block at a time
  __syncthreads();  // every wave is done with the ring; its bytes now hold candidate lists
  constexpr int kSlots = Shape::kSlots;
  const int qbase = (wv * kBlockQ + (lane & 31)) * kSlots;
  const int k_eff = min(p.topk, nbs);
  const uint16_t* kb0 = KB + static_cast<int64_t>(kt0) * kKeyTile * kD;
  auto finish = [&](QBlock<KMAX, D>& B, int x) {
    // clear the query's slots (each lane half clears one half of them)
    {
      const u32x4 z = {0u, 0u, 0u, 0u};
      uint64_t* const row = cand_key + qbase + half * (kSlots / 2);
#pragma unroll
      for (int e = 0; e < kSlots / 2; e += 2) *reinterpret_cast<u32x4*>(row + e) = z;
    }
    wave_lds_sync();
    // the query's candidate list: lane half 0 writes slots 1, 2, ... upward,
    // half 1 writes kCap, kCap - 1, ... downward; a write past the capacity
    // lands in the sink slot (0 or kCap + 1) and the query goes to the fallback
    int cpos = qbase + (half ? kCap : 1);
    const int climit = qbase + (half ? 0 : kCap + 1);
    const int cstep = half ? -1 : 1;
    int over = (B.ecnt >= kEnt || B.to_fix) ? 1 : 0;
    if (!over) {
      for (int e = 0; e < B.ecnt; ++e) {
        const uint32_t word = ent[(2 * e + x) * 256 + tid];
        const int base = static_cast<int>(word >> 16) * kKeyTile + 4 * half;
        uint32_t m = word & 0xFFFFu;
        while (m != 0u) {
          const int bpos = 31 - __clz(m);
          m ^= 1u << bpos;
          const int r = 15 - bpos;
          reinterpret_cast<uint32_t*>(cand_key + cpos)[0] = ~static_cast<uint32_t>(base + 8 * (r >> 2) + (r & 3));
          cpos = (cpos == climit) ? cpos : cpos + cstep;
        }
      }
    }
    // appended so far (a pointer parked on the sink slot counts as overflow)
    const int cnt = half ? qbase + kCap - cpos : cpos - (qbase + 1);
    over |= __shfl_xor(over, 32);
    const int cnt_other = __shfl_xor(cnt, 32);
    // kCap - 1: a lane parked on its sink also counts; relative block ids
    // must fit 16 bits
    const bool overflow = over || cnt + cnt_other > kCap - 1 || n_kt * kKeyTile > 65536;

    // the query's candidates as one list of tot entries: half 0's at slots
    // 1 .. cnt0, then half 1's at kCap + 1 - cnt1 .. kCap; the two lanes of
    // the query take alternate entries for the exact logits and the ranks,
    // so both run the same number of steps whichever lane found them
    const int tot = cnt + cnt_other;
    const int cnt0 = half ? cnt_other : cnt;
    const int tail0 = qbase + kCap + 1 - tot;   // slot of entry i >= cnt0 is tail0 + i
    auto slot_of = [&](int i) { return i < cnt0 ? qbase + 1 + i : tail0 + i; };
    wave_lds_sync();   // each lane now reads block ids the other lane of its query wrote
    // exact float32 logits of the candidates into the high key words
    if (B.valid && !overflow && tot > 0) {
      // products of bf16 pairs are exact in float32 (v_dot2_f32_bf16); four
      // partial sums keep the dependent chains short
      u32x4 qw[kD / 8];
#pragma unroll
      for (int c = 0; c < kD / 8; ++c) qw[c] = *reinterpret_cast<const u32x4*>(B.q_row + 8 * c);
      for (int i = half; i < tot; i += 2) {
        uint32_t* const slot = reinterpret_cast<uint32_t*>(cand_key + slot_of(i));
        const uint16_t* kr = kb0 + static_cast<int64_t>(~slot[0]) * kD;
        float sp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < kD / 8; ++c) {
          const u32x4 u = *reinterpret_cast<const u32x4*>(kr + 8 * c);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // (words through scalars: this compiler's __builtin_bit_cast of
            // a vector element reads element 0)
            const uint32_t ke = u[e], qe = qw[c][e];
            sp[e] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, ke), __builtin_bit_cast(bf16x2, qe),
                                                    sp[e], false);
          }
        }
        slot[1] = ordered_bits((sp[0] + sp[1]) + (sp[2] + sp[3]));
      }
    }
    wave_lds_sync();
    int32_t* out_sel = p.topk_idx + (static_cast<int64_t>(B.t) * p.h_kv + h) * p.topk;
    if (B.valid && overflow) {
      if (half == 0) {
        const int slot = atomicAdd(&p.fix[0], 1);
        p.fix[1 + slot] = B.qi * p.h_kv + h;
      }
    } else if (B.valid) {
      // a candidate's rank is the number of the query's keys above its own
      uint64_t keys[kSlots];
#pragma unroll
      for (int e = 0; e < kSlots; e += 2) {
        const u32x4 u = *reinterpret_cast<const u32x4*>(cand_key + qbase + e);
        keys[e] = (static_cast<uint64_t>(u[1]) << 32) | u[0];
        keys[e + 1] = (static_cast<uint64_t>(u[3]) << 32) | u[2];
      }
      const int jbase = kt0 * kKeyTile;
      for (int i = half; i < tot; i += 2) {
        const uint64_t ck = cand_key[slot_of(i)];
        int rank = 0;
#pragma unroll
        for (int e = 0; e < kSlots; ++e) rank += keys[e] > ck ? 1 : 0;
        if (rank < k_eff) out_sel[rank] = jbase + static_cast<int>(~static_cast<uint32_t>(ck));
      }
      if (half == 0)
        for (int r = k_eff; r < p.topk; ++r) out_sel[r] = -1;
    }
  };
  finish(blk[0], 0);
  wave_lds_sync();  // block A's lists are consumed (each wave owns its slots)
  finish(blk[1], 1);
}

// Exact top-k for the (sorted position, group) pairs whose candidate list
// overflowed: one workgroup per pair.  Each thread scores every 256th block
// of the sequence in float32 and keeps a sorted list of its best KMAX (value
// descending, block ascending); each wave then pops its KMAX best with wave
// reductions, and wave 0 ranks the 4 x KMAX survivors.
template <int KMAX, int D>
__global__ void __launch_bounds__(256)
topk_fixup_kernel(FwdParams p) {
  constexpr int kD = D;
  __shared__ float wv_val[4 * KMAX];
  __shared__ int wv_idx[4 * KMAX];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int n_fix = p.fix[0];
  const uint16_t* Q = static_cast<const uint16_t*>(p.q);
  for (int item = blockIdx.x; item < n_fix; item += gridDim.x) {
    const int entry = p.fix[1 + item];
    const int i = entry / p.h_kv, g = entry % p.h_kv;
    const int t = p.perm[i];
    int lo = 0, hi = p.batch - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.win_off[p.seq_win_off[mid]] <= i) lo = mid; else hi = mid - 1;
    }
    const int j0 = p.seq_blk_off[lo], j1 = p.seq_blk_off[lo + 1];
    // the query row stays packed: v_dot2_f32_bf16 (exact products, float32
    // sums, four partial sums) scores a block as the epilogue does
    u32x4 qw[kD / 8];
#pragma unroll
    for (int c = 0; c < kD / 8; ++c)
      qw[c] = *reinterpret_cast<const u32x4*>(Q + (static_cast<int64_t>(t) * p.h_q + g) * kD + 8 * c);
    const uint16_t* KB = static_cast<const uint16_t*>(p.kbar) + static_cast<int64_t>(g) * p.nb_cap * kD;
    float lv[KMAX];
    int li[KMAX];
#pragma unroll
    for (int e = 0; e < KMAX; ++e) { lv[e] = -FLT_MAX; li[e] = 0x7FFFFFFF; }
    for (int j = j0 + tid; j < j1; j += 256) {
      float sp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < kD / 8; ++c) {
        const u32x4 u = *reinterpret_cast<const u32x4*>(KB + static_cast<int64_t>(j) * kD + 8 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // (words through scalars: this compiler's __builtin_bit_cast of a
          // vector element reads element 0)
          const uint32_t ke = u[e], qe = qw[c][e];
          sp[e] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, ke), __builtin_bit_cast(bf16x2, qe), sp[e],
                                                  false);
        }
      }
      const float s = (sp[0] + sp[1]) + (sp[2] + sp[3]);
      // blocks arrive in increasing id, so a tie keeps the earlier (lower) id ahead
      if (s > lv[KMAX - 1]) {
        bool placed = false;
#pragma unroll
        for (int e = KMAX - 1; e >= 1; --e) {
          if (!placed) {
            if (s > lv[e - 1]) { lv[e] = lv[e - 1]; li[e] = li[e - 1]; }
            else { lv[e] = s; li[e] = j; placed = true; }
          }
        }
        if (!placed) { lv[0] = s; li[0] = j; }
      }
    }
    // each wave pops its KMAX best (value descending, block ascending)
    for (int r = 0; r < KMAX; ++r) {
      // (value, then lower block first) as one 64-bit key
      const uint64_t key = wave_max_key((static_cast<uint64_t>(ordered_bits(lv[0])) << 32) |
                                        static_cast<uint32_t>(~li[0]));
      const float bv = ordered_value(static_cast<uint32_t>(key >> 32));
      const int bi = static_cast<int>(~static_cast<uint32_t>(key));
      if (li[0] == bi) {
#pragma unroll
        for (int e = 0; e < KMAX - 1; ++e) { lv[e] = lv[e + 1]; li[e] = li[e + 1]; }
        lv[KMAX - 1] = -FLT_MAX;
        li[KMAX - 1] = 0x7FFFFFFF;
      }
      if (lane == 0) { wv_val[wv * KMAX + r] = bv; wv_idx[wv * KMAX + r] = bi; }
    }
    __syncthreads();
    // wave 0 ranks the survivors (an unused slot holds -FLT_MAX and the
    // largest id, so it ranks after every real block)
    const int k_eff = min(p.topk, j1 - j0);
    int32_t* out_sel = p.topk_idx + (static_cast<int64_t>(t) * p.h_kv + g) * p.topk;
    if (wv == 0) {
      for (int e = lane; e < 4 * KMAX; e += 64) {
        const float cv = wv_val[e];
        const int ci = wv_idx[e];
        int rank = 0;
        for (int o = 0; o < 4 * KMAX; ++o) {
          const float ov = wv_val[o];
          const int oi = wv_idx[o];
          rank += (ov > cv) || (ov == cv && oi < ci);
        }
        if (rank < k_eff) out_sel[rank] = ci;
      }
      for (int r = k_eff + lane; r < p.topk; r += 64) out_sel[r] = -1;
    }
    __syncthreads();  // the survivor arrays are reused by the next pair
  }
}

}  // namespace

void tile_prefix_kernel_launch(const FwdParams& p, hipStream_t stream) {
  tile_prefix_kernel<<<1, 64, 0, stream>>>(p);
}

// the query-tile prefix, the probe slots and the probe sets (the compressed
// kernel reads all three)
void probe_select_launch(const FwdParams& p, hipStream_t stream) {
  if (p.probe_slot && p.max_probe_slots > 0)
    probe_select_kernel<<<dim3(p.max_probe_slots, p.h_kv), 256, 0, stream>>>(p);
}

hipError_t launch_cmp_probe(const FwdParams& p, ssa_dtype /*dtype*/, hipStream_t stream) {
  tile_prefix_kernel_launch(p, stream);
  probe_select_launch(p, stream);
  return hipGetLastError();
}

hipError_t launch_cmp_mfma(const FwdParams& p, ssa_dtype /*dtype*/, hipStream_t stream) {
  const dim3 grid(p.max_tiles, p.h_q);
  if (p.d == 32) {
    if (p.topk <= 16) cmp_mfma_kernel<16, 32><<<grid, 256, 0, stream>>>(p);
    else cmp_mfma_kernel<32, 32><<<grid, 256, 0, stream>>>(p);
  } else {
    if (p.topk <= 16) cmp_mfma_kernel<16, 64><<<grid, 256, 0, stream>>>(p);
    else cmp_mfma_kernel<32, 64><<<grid, 256, 0, stream>>>(p);
  }
  return hipGetLastError();
}

hipError_t launch_topk_fixup(const FwdParams& p, ssa_dtype /*dtype*/, hipStream_t stream) {
  if (p.d == 32) {
    if (p.topk <= 16) topk_fixup_kernel<16, 32><<<2048, 256, 0, stream>>>(p);
    else topk_fixup_kernel<32, 32><<<2048, 256, 0, stream>>>(p);
  } else {
    if (p.topk <= 16) topk_fixup_kernel<16, 64><<<2048, 256, 0, stream>>>(p);
    else topk_fixup_kernel<32, 64><<<2048, 256, 0, stream>>>(p);
  }
  return hipGetLastError();
}

}  // namespace ssa
