// Compressed-block attention and top-k block selection for grouped query
// heads on MFMA (bf16, D = 32 or 64, 16 query heads per key/value head).
//
// Direct3D-S2 page, "Method": every query attends to the mean-pooled blocks of
// its sequence, and the attention scores choose the top-k blocks; LSRM
// article, its sparse-attention section: the selection is shared by the query
// heads of a key/value group.  Here the score of block j for a query token t
// and group g is the sum over the group's heads of the softmax probability of
// j, so the heads' softmax normalisers are needed before any block can be
// ranked.  Three kernels:
//
//  gqa_cmp_kernel: o_cmp of every (token, query head) with a streaming
//    softmax (S^T = Kbar Q^T, one running shift per query head, rescaled only
//    when a tile maximum exceeds it by 8 in log2 units, so the probabilities
//    stay below 256), adds G0 * o_cmp to the float32 branch accumulator and
//    stores the head's log2 normaliser c = shift * scale * log2 e + log2(sum),
//    so that the probability of block j is 2^(s_j * scale * log2 e - c).
//    Work split as in the one-head-per-group kernel: 256 sorted queries of one
//    sequence and one query head per workgroup, 4 waves x two 32-query
//    blocks, pooled keys / values streamed through a two-slot LDS ring.
//
//  gqa_topk_kernel: S = Q Kbar^T with the rows of the MFMA tile being
//    (token, head) pairs, 2 tokens x 16 heads, and the columns 32 blocks.  A
//    lane then holds one block and 8 heads of each token, so the group sum is
//    8 in-lane adds and one add across the lane halves.  Each lane keeps,
//    per token, its kLane = 6 best (score, block) pairs in float32 (an insertion
//    network: one v_med3 for the scores and two selects for the ids per
//    slot), and the 32 lanes' lists are merged by repeated wave maxima (equal
//    scores: lower block first).  A workgroup owns 16 sorted tokens of one
//    sequence and one group (4 waves x 2 row blocks).  A (token, group) pair
//    for which one lane's 6 kept pairs all reach the top k, while that lane
//    saw more blocks than it kept, is queued for gqa_fixup_kernel, which
//    ranks all blocks of the sequence exactly.
#include <float.h>
#include <limits.h>

#include <type_traits>

#include "ssa_internal.h"

namespace ssa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kGroup = 16;            // query heads per key/value head on this path
constexpr int kTopkTile = 16;         // sorted tokens per workgroup of the top-k kernel
// (score, block) pairs kept per lane and token.  A lane sees every 32nd block,
// so it rarely holds more than 5 of a query's top 16: measured on the
// 262144-token grouped workload, 8 pairs cost 18.8 ms with no fallback, 6
// pairs 17.0 ms plus 0.16 ms of fallback, 4 pairs 15.7 ms plus 5.4 ms.
constexpr int kLane = 6;
constexpr float kRescale = 8.0f;      // log2 headroom before the running shift moves
// bf16 P by truncation (the fixed-shift loop): the mean relative loss of
// truncating a float32 with a log-uniform mantissa to 8 significant bits is
// 2^-8 * (1/ln 2) * (1/2); p is scaled up by the inverse factor and the row
// sum divided by it again, so P V and the row sum agree on average
constexpr float kTruncLog2 = 0.0040711f;   // log2(1 / (1 - 2^-8 * 0.5 / ln 2))
constexpr float kTruncInv = 0.99718215f;   // 1 - 2^-8 * 0.5 / ln 2
// largest |q| max_j |Kbar_j| * scale * log2 e for which the fixed shift keeps
// every exponent within [-120, 0]
constexpr float kFixedBound = 60.f;
template <bool B>
using kBool = std::integral_constant<bool, B>;

__device__ __forceinline__ bf16x8 lds_b128(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ void seq_token_range(const FwdParams& p, int b, int* s0, int* s1) {
  *s0 = p.win_off[p.seq_win_off[b]];
  *s1 = p.win_off[p.seq_win_off[b + 1]];
}

__device__ __forceinline__ int find_tile_seq(const int32_t* pre, int batch, int tile) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// tile_pre2[b] = number of 16-token tiles of sequences before b
__global__ void gqa_tile_prefix_kernel(FwdParams p) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int run = 0;
  for (int b = 0; b < p.batch; ++b) {
    p.tile_pre2[b] = run;
    int s0, s1;
    seq_token_range(p, b, &s0, &s1);
    run += (s1 - s0 + kTopkTile - 1) / kTopkTile;
  }
  p.tile_pre2[p.batch] = run;
}

// seq_kmax2[g][b] = largest squared norm of sequence b's pooled keys of
// group g; one workgroup per (sequence, group)
__global__ void __launch_bounds__(256)
gqa_seq_kmax_kernel(FwdParams p) {
  __shared__ float wmax[4];
  const int b = blockIdx.x, g = blockIdx.y;
  const int j0 = p.seq_blk_off[b], j1 = p.seq_blk_off[b + 1];
  const float* n2 = p.knorm2 + static_cast<int64_t>(g) * p.nb_cap;
  float m = 0.f;
  for (int j = j0 + static_cast<int>(threadIdx.x); j < j1; j += 256) m = fmaxf(m, n2[j]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    p.seq_kmax2[static_cast<int64_t>(g) * p.batch + b] = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
}

// ------------------------------------------------------------ o_cmp + normalisers

// D = 32 runs four workgroups per compute unit (128 registers, a 12-byte
// spill; 5 % faster than two); D = 64 keeps two, since four would spill 224 bytes.
//
// A logit of query q is at most |q| max_j |Kbar_j| (Cauchy-Schwarz).  When
// that bound B_q, times scale * log2 e, is at most kFixedBound for every query
// of the workgroup, the softmax is shifted by B_q once: every exponent then
// lies in [-2 B_q, 0] c2 >= -120, so 2^x neither overflows nor flushes the row
// to zero, and no running maximum or rescaling is needed (P is truncated to
// bf16 with the mean-loss correction).  Otherwise the streaming softmax with a
// running shift runs.
template <int D>
__global__ void __launch_bounds__(256, D == 32 ? 4 : 2)
gqa_cmp_kernel(FwdParams p) {
  constexpr int KS = D / 16;            // MFMA k steps over the dims
  constexpr int VB = D / 32;            // 32-dim row blocks of O^T
  constexpr int kKRow = D + 8;          // padded key-tile row (bf16)
  constexpr int kVRow = kKeyTile + 8;   // padded value-tile row (bf16)
  constexpr int kKTile = kKeyTile * kKRow;
  constexpr int kVTile = D * kVRow;
  constexpr int kChunks = kKeyTile * D / 8;   // 16-byte chunks per tile
  __shared__ __align__(16) uint16_t k_lds[2 * kKTile];
  __shared__ __align__(16) uint16_t v_lds[2 * kVTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int half = lane >> 5;
  const int h = blockIdx.y;
  const int g = h / (p.h_q / p.h_kv);
  const int tile = blockIdx.x;
  if (tile >= p.tile_pre[p.batch]) return;
  const int b = find_tile_seq(p.tile_pre, p.batch, tile);
  int s0, s1;
  seq_token_range(p, b, &s0, &s1);
  const int q_begin = s0 + (tile - p.tile_pre[b]) * kQueryTile;
  const int q_end = min(q_begin + kQueryTile, s1);
  const int j0 = p.seq_blk_off[b], j1 = p.seq_blk_off[b + 1];
  const int kt0 = j0 / kKeyTile, kt1 = (j1 + kKeyTile - 1) / kKeyTile;
  const int n_kt = kt1 - kt0;
  const float c2 = p.scale * kLog2e;

  const uint16_t* Q = static_cast<const uint16_t*>(p.q);
  bf16x8 qb[2][KS];
  int t[2];
  bool valid[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int qi = q_begin + wv * 64 + x * 32 + (lane & 31);
    valid[x] = qi < q_end;
    t[x] = valid[x] ? p.perm[qi] : 0;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 u = {0u, 0u, 0u, 0u};
      if (valid[x]) u = *reinterpret_cast<const u32x4*>(Q + (static_cast<int64_t>(t[x]) * p.h_q + h) * D + 16 * ks + 8 * half);
      qb[x][ks] = __builtin_bit_cast(bf16x8, u);
    }
  }

  const uint16_t* KB = static_cast<const uint16_t*>(p.kbar) + static_cast<int64_t>(g) * p.nb_cap * D;
  const uint16_t* VT = static_cast<const uint16_t*>(p.vbar_t) + static_cast<int64_t>(g) * p.nb_cap * D;
  const bool stager = tid < kChunks;
  const int k_row = tid / (D / 8), k_c = tid % (D / 8);
  const int v_row = tid >> 2, v_c = tid & 3;
  const uint16_t* kg = KB + (static_cast<int64_t>(kt0) * kKeyTile + k_row) * D + 8 * k_c;
  const uint16_t* vg = VT + (static_cast<int64_t>(kt0) * D + v_row) * kKeyTile + 8 * v_c;
  auto load_k = [&](int rel) {
    return stager ? *reinterpret_cast<const u32x4*>(kg + static_cast<int64_t>(rel) * kKeyTile * D) : u32x4{0u, 0u, 0u, 0u};
  };
  auto load_v = [&](int rel) {
    return stager ? *reinterpret_cast<const u32x4*>(vg + static_cast<int64_t>(rel) * kKeyTile * D) : u32x4{0u, 0u, 0u, 0u};
  };
  const int ks_dst = k_row * kKRow + 8 * k_c;
  const int vs_dst = v_row * kVRow + 8 * v_c;
  auto store_k = [&](int slot, const u32x4& u) {
    if (stager) *reinterpret_cast<u32x4*>(k_lds + slot * kKTile + ks_dst) = u;
  };
  auto store_v = [&](int slot, const u32x4& u) {
    if (stager) *reinterpret_cast<u32x4*>(v_lds + slot * kVTile + vs_dst) = u;
  };

  // fixed shift per query (see above): k0 = -B_q c2 (+ the truncation
  // offset); the workgroup takes it only if every query's bound fits
  const float kmax2 = p.seq_kmax2[static_cast<int64_t>(g) * p.batch + b];
  float k0[2];
  bool fits = true;
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    float qn2 = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 u = __builtin_bit_cast(u32x4, qb[x][ks]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = __uint_as_float(u[e] << 16), hi = __uint_as_float(u[e] & 0xFFFF0000u);
        qn2 = fmaf(lo, lo, fmaf(hi, hi, qn2));
      }
    }
    qn2 += __shfl_xor(qn2, 32);
    const float bound = sqrtf(qn2 * kmax2) * c2;
    fits = fits && bound <= kFixedBound;
    k0[x] = -bound + kTruncLog2;
  }
  const bool fixed = __syncthreads_and(fits ? 1 : 0) != 0;

  // softmax state per block: running shift m (logit units; streaming loop
  // only), row-sum partials, O^T row blocks
  float m[2], l[2][2];
  f32x16 o[2][VB];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    m[x] = -FLT_MAX;
    l[x][0] = l[x][1] = 0.f;
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) o[x][vb] = f32x16{};
  }

  auto qk = [&](int slot, const bf16x8 (&q)[KS]) {
    const uint16_t* kl = k_lds + slot * kKTile + (lane & 31) * kKRow + 8 * half;
    f32x16 s = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128(kl + 16 * ks), q[ks], s, 0, 0, 0);
    return s;
  };
  // probabilities of block x for tile rel (keys outside [j0, j1) masked),
  // P^T as two bf16 operands, then O^T += Vbar^T P^T
  auto attend = [&](int x, int rel, int slot, f32x16& s, auto fixed_shift) {
    const int kt = kt0 + rel;
    if (kt * kKeyTile < j0 || kt * kKeyTile + kKeyTile > j1) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = kt * kKeyTile + 8 * (r >> 2) + 4 * half + (r & 3);
        if (j < j0 || j >= j1) s[r] = -FLT_MAX;
      }
    }
    bf16x8 pb[2];
    if constexpr (decltype(fixed_shift)::value) {
      float pr[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) pr[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c2, k0[x]));
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        l[x][0] += pr[r];
        l[x][1] += pr[r + 1];
      }
      // truncation: v_perm_b32 takes the high halves of two float32 values
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4 u;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          u[e] = __builtin_amdgcn_perm(__float_as_uint(pr[8 * ks + 2 * e + 1]), __float_as_uint(pr[8 * ks + 2 * e]),
                                       0x07060302u);
        pb[ks] = __builtin_bit_cast(bf16x8, u);
      }
    } else {
      float tm = fmaxf(s[0], s[1]);
#pragma unroll
      for (int r = 2; r < 16; r += 2) tm = fmaxf(tm, fmaxf(s[r], s[r + 1]));
      tm = fmaxf(tm, __shfl_xor(tm, 32));
      if ((tm - m[x]) * c2 > kRescale) {
        const float corr = m[x] == -FLT_MAX ? 0.f : __builtin_amdgcn_exp2f((m[x] - tm) * c2);
        l[x][0] *= corr;
#pragma unroll
        for (int vb = 0; vb < VB; ++vb)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[x][vb][r] *= corr;
        m[x] = tm;
      }
      const float mc = m[x] * c2;
      float pr[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        pr[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c2, -mc));
        l[x][0] += pr[r];
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < 8; ++i) pb[ks][i] = static_cast<__bf16>(pr[8 * ks + i]);
    }
    const uint16_t* vl = v_lds + slot * kVTile + (lane & 31) * kVRow + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int vb = 0; vb < VB; ++vb)
        o[x][vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128(vl + vb * 32 * kVRow + 16 * ks), pb[ks], o[x][vb], 0, 0, 0);
  };

  // ring: slot (rel & 1) holds key and value tile rel; register sets hold
  // tile rel + 1 until it is stored at the start of step rel + 1
  auto run = [&](auto fixed_shift) {
    u32x4 kr = load_k(0), vr = load_v(0);
    store_k(0, kr);
    store_v(0, vr);
    if (n_kt > 1) {
      kr = load_k(1);
      vr = load_v(1);
    }
    for (int rel = 0; rel < n_kt; ++rel) {
      __syncthreads();  // tiles rel stored; everyone is done with tiles rel - 1
      if (rel + 1 < n_kt) {
        store_k((rel + 1) & 1, kr);
        store_v((rel + 1) & 1, vr);
      }
      if (rel + 2 < n_kt) {
        kr = load_k(rel + 2);
        vr = load_v(rel + 2);
      }
      f32x16 s_a = qk(rel & 1, qb[0]);
      f32x16 s_b = qk(rel & 1, qb[1]);
      attend(0, rel, rel & 1, s_a, fixed_shift);
      attend(1, rel, rel & 1, s_b, fixed_shift);
    }
  };
  if (fixed) run(kBool<true>{});
  else run(kBool<false>{});

  // o_cmp times its gate into the accumulator; the head's log2 normaliser
  // c = log2 sum_j 2^(s_j c2), so that block j's probability is 2^(s_j c2 - c)
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const float lsum = l[x][0] + l[x][1];
    const float lq = lsum + __shfl_xor(lsum, 32);
    if (!valid[x]) continue;
    const int64_t row = static_cast<int64_t>(t[x]) * p.h_q + h;
    const float c = fixed ? __log2f(lq) - k0[x] : m[x] * c2 + __log2f(lq);
    if (half == 0) {
      p.norm[row] = c;
      if (p.lse) p.lse[row] = c * kLn2;
    }
    const uint16_t* gt = static_cast<const uint16_t*>(p.gates) + row * 3;
    const float f = bf16_bits_to_f32(gt[0]) / (fixed ? lq * kTruncInv : lq);
    float* dst = p.acc + row * D;
#pragma unroll
    for (int vb = 0; vb < VB; ++vb)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const int d = 32 * vb + 8 * rb + 4 * half;
        float4 a = *reinterpret_cast<float4*>(dst + d);
        a.x += o[x][vb][4 * rb] * f; a.y += o[x][vb][4 * rb + 1] * f;
        a.z += o[x][vb][4 * rb + 2] * f; a.w += o[x][vb][4 * rb + 3] * f;
        *reinterpret_cast<float4*>(dst + d) = a;
      }
  }
}

// ------------------------------------------------------------ group top-k

template <int D>
__global__ void __launch_bounds__(256)
gqa_topk_kernel(FwdParams p) {
  constexpr int KS = D / 16;
  constexpr int kKRow = D + 8;
  constexpr int kKTile = kKeyTile * kKRow;
  constexpr int kChunks = kKeyTile * D / 8;
  __shared__ __align__(16) uint16_t k_lds[2 * kKTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int half = lane >> 5;
  const int g = blockIdx.y;
  const int tile = blockIdx.x;
  if (tile >= p.tile_pre2[p.batch]) return;
  const int b = find_tile_seq(p.tile_pre2, p.batch, tile);
  int s0, s1;
  seq_token_range(p, b, &s0, &s1);
  const int t_begin = s0 + (tile - p.tile_pre2[b]) * kTopkTile;
  const int t_end = min(t_begin + kTopkTile, s1);
  const int j0 = p.seq_blk_off[b], j1 = p.seq_blk_off[b + 1];
  const int kt0 = j0 / kKeyTile, kt1 = (j1 + kKeyTile - 1) / kKeyTile;
  const int n_kt = kt1 - kt0;
  const float c2 = p.scale * kLog2e;
  const uint16_t* Q = static_cast<const uint16_t*>(p.q);

  // row blocks x = 0, 1 of this wave: tokens 4 wv + 2 x + {0, 1};
  // A operand row (lane % 32) = (token (lane % 32) / 16, head lane % 16)
  bf16x8 qa[2][KS];
  float cn[2][16];       // log2 normalisers of this lane's 16 accumulator rows
  int tk[2][2];          // sorted positions of the row block's two tokens
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    tk[x][0] = t_begin + 4 * wv + 2 * x;
    tk[x][1] = tk[x][0] + 1;
    const int mine = tk[x][(lane & 31) >> 4];
    const bool ok = mine < t_end;
    const int tt = ok ? p.perm[mine] : 0;
    const int hq = g * kGroup + (lane & 15);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 u = {0u, 0u, 0u, 0u};
      if (ok) u = *reinterpret_cast<const u32x4*>(Q + (static_cast<int64_t>(tt) * p.h_q + hq) * D + 16 * ks + 8 * half);
      qa[x][ks] = __builtin_bit_cast(bf16x8, u);
    }
    // accumulator row of entry r: 8 (r / 4) + 4 half + r % 4 = (token, head)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r >> 2) + 4 * half + (r & 3);
      const int pos = tk[x][row >> 4];
      cn[x][r] = FLT_MAX;  // no probability for a missing token
      if (pos < t_end)
        cn[x][r] = p.norm[static_cast<int64_t>(p.perm[pos]) * p.h_q + g * kGroup + (row & 15)];
    }
  }

  const uint16_t* KB = static_cast<const uint16_t*>(p.kbar) + static_cast<int64_t>(g) * p.nb_cap * D;
  const bool stager = tid < kChunks;
  const int k_row = tid / (D / 8), k_c = tid % (D / 8);
  const uint16_t* kg = KB + (static_cast<int64_t>(kt0) * kKeyTile + k_row) * D + 8 * k_c;
  auto load_k = [&](int rel) {
    return stager ? *reinterpret_cast<const u32x4*>(kg + static_cast<int64_t>(rel) * kKeyTile * D) : u32x4{0u, 0u, 0u, 0u};
  };
  const int ks_dst = k_row * kKRow + 8 * k_c;

  // per lane and row block: the lane's kLane best (score, block) pairs for
  // token `half` of the row block (both halves hold the same sums), score
  // descending, equal scores by block ascending; an empty slot holds -1
  // (every score is >= 0)
  float Lv[2][kLane];
  int Lj[2][kLane];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int i = 0; i < kLane; ++i) {
      Lv[x][i] = -1.f;
      Lj[x][i] = INT_MAX;
    }

  u32x4 kr = load_k(0);
  if (stager) *reinterpret_cast<u32x4*>(k_lds + ks_dst) = kr;
  if (n_kt > 1) kr = load_k(1);
  for (int rel = 0; rel < n_kt; ++rel) {
    __syncthreads();
    if (rel + 1 < n_kt && stager) *reinterpret_cast<u32x4*>(k_lds + ((rel + 1) & 1) * kKTile + ks_dst) = kr;
    if (rel + 2 < n_kt) kr = load_k(rel + 2);
    const uint16_t* kl = k_lds + (rel & 1) * kKTile + (lane & 31) * kKRow + 8 * half;
    bf16x8 kb[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kb[ks] = lds_b128(kl + 16 * ks);
    const int j = (kt0 + rel) * kKeyTile + (lane & 31);     // this lane's block
    const bool jok = j >= j0 && j < j1;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      f32x16 s = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[x][ks], kb[ks], s, 0, 0, 0);
      float sum0 = 0.f, sum1 = 0.f;
#pragma unroll
      for (int r = 0; r < 8; ++r) sum0 += __builtin_amdgcn_exp2f(fmaf(s[r], c2, -cn[x][r]));
#pragma unroll
      for (int r = 8; r < 16; ++r) sum1 += __builtin_amdgcn_exp2f(fmaf(s[r], c2, -cn[x][r]));
      sum0 += __shfl_xor(sum0, 32);
      sum1 += __shfl_xor(sum1, 32);
      // a block outside the sequence scores -2 and changes no slot
      const float sc = jok ? (half ? sum1 : sum0) : -2.f;
      // slot i takes slot i - 1 when sc beats it, else sc when sc beats slot i;
      // blocks of a lane arrive in increasing id, so an equal score stays behind
#pragma unroll
      for (int i = kLane - 1; i >= 1; --i) {
        const bool up = sc > Lv[x][i - 1];
        const bool here = sc > Lv[x][i];
        Lj[x][i] = up ? Lj[x][i - 1] : (here ? j : Lj[x][i]);
        Lv[x][i] = __builtin_amdgcn_fmed3f(Lv[x][i - 1], sc, Lv[x][i]);
      }
      const bool top = sc > Lv[x][0];
      Lj[x][0] = top ? j : Lj[x][0];
      Lv[x][0] = top ? sc : Lv[x][0];
    }
  }

  // merge the 32 lanes of each half by repeated maxima of the list heads
  // (equal scores: lower block first).  A lane holding more than kLane of the
  // sequence's blocks has dropped some; if all its kept pairs are taken, a
  // dropped one may belong to the top k, and the (token, group) pair is handed
  // to the exact fallback kernel.
  const int nbs = j1 - j0;
  const int k_eff = min(p.topk, nbs);
  const int l32 = lane & 31;
  const int n_mine = n_kt - (l32 < j0 - kt0 * kKeyTile ? 1 : 0) - (l32 >= j1 - (kt1 - 1) * kKeyTile ? 1 : 0);
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int pos = tk[x][half];
    const bool ok = pos < t_end;
    int32_t* out_sel = ok ? p.topk_idx + (static_cast<int64_t>(p.perm[pos]) * p.h_kv + g) * p.topk : nullptr;
    int used = 0;
    for (int r = 0; r < k_eff; ++r) {
      float bv = Lv[x][0];
      int bj = Lj[x][0];
#pragma unroll
      for (int off = 16; off > 0; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oj = __shfl_xor(bj, off);
        if (ov > bv || (ov == bv && oj < bj)) { bv = ov; bj = oj; }
      }
      if (bv >= 0.f && bj == Lj[x][0]) {
#pragma unroll
        for (int i = 0; i < kLane - 1; ++i) {
          Lv[x][i] = Lv[x][i + 1];
          Lj[x][i] = Lj[x][i + 1];
        }
        Lv[x][kLane - 1] = -1.f;
        Lj[x][kLane - 1] = INT_MAX;
        ++used;
      }
      if (ok && l32 == 0) out_sel[r] = bv >= 0.f ? bj : -1;
    }
    const uint64_t spill = __ballot(n_mine > kLane && used == kLane);
    const bool overflow = ((half ? spill >> 32 : spill) & 0xFFFFFFFFull) != 0;
    if (ok && l32 == 0) {
      for (int r = k_eff; r < p.topk; ++r) out_sel[r] = -1;
      if (overflow) {
        const int slot = atomicAdd(&p.fix[0], 1);
        p.fix[1 + slot] = pos * p.h_kv + g;
      }
    }
  }
}

// ------------------------------------------------------------ exact fallback

// One workgroup per (token, group) pair whose lane lists overflowed: every
// thread scores blocks j0 + tid, j0 + tid + 256, ... exactly as above (the
// group's 16 query rows and normalisers staged in LDS) and keeps its KMAX best
// pairs; each wave pops its KMAX best and wave 0 ranks the 4 x KMAX survivors.
template <int D, int KMAX>
__global__ void __launch_bounds__(256)
gqa_fixup_kernel(FwdParams p) {
  __shared__ float qs[kGroup * D];
  __shared__ float cs[kGroup];
  __shared__ float wv_val[4 * KMAX];
  __shared__ int wv_idx[4 * KMAX];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int n_fix = p.fix[0];
  const float c2 = p.scale * kLog2e;
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
    for (int e = tid; e < kGroup * D; e += 256)
      qs[e] = bf16_bits_to_f32(Q[(static_cast<int64_t>(t) * p.h_q + g * kGroup) * D + e]);
    if (tid < kGroup) cs[tid] = p.norm[static_cast<int64_t>(t) * p.h_q + g * kGroup + tid];
    __syncthreads();
    const uint16_t* KB = static_cast<const uint16_t*>(p.kbar) + static_cast<int64_t>(g) * p.nb_cap * D;
    float lv[KMAX];
    int li[KMAX];
#pragma unroll
    for (int e = 0; e < KMAX; ++e) { lv[e] = -1.f; li[e] = INT_MAX; }
    for (int j = j0 + tid; j < j1; j += 256) {
      float kf[D];
#pragma unroll
      for (int c = 0; c < D / 8; ++c) {
        const u32x4 u = *reinterpret_cast<const u32x4*>(KB + static_cast<int64_t>(j) * D + 8 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kf[8 * c + 2 * e] = __uint_as_float(u[e] << 16);
          kf[8 * c + 2 * e + 1] = __uint_as_float(u[e] & 0xFFFF0000u);
        }
      }
      float sc = 0.f;
      for (int hh = 0; hh < kGroup; ++hh) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < D; ++e) d = fmaf(qs[hh * D + e], kf[e], d);
        sc += __builtin_amdgcn_exp2f(fmaf(d, c2, -cs[hh]));
      }
      // blocks arrive in increasing id, so an equal score stays behind
      if (sc > lv[KMAX - 1]) {
        bool placed = false;
#pragma unroll
        for (int e = KMAX - 1; e >= 1; --e) {
          if (!placed) {
            if (sc > lv[e - 1]) { lv[e] = lv[e - 1]; li[e] = li[e - 1]; }
            else { lv[e] = sc; li[e] = j; placed = true; }
          }
        }
        if (!placed) { lv[0] = sc; li[0] = j; }
      }
    }
    for (int r = 0; r < KMAX; ++r) {
      float bv = lv[0];
      int bi = li[0];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
      }
      if (bv >= 0.f && li[0] == bi) {
#pragma unroll
        for (int e = 0; e < KMAX - 1; ++e) { lv[e] = lv[e + 1]; li[e] = li[e + 1]; }
        lv[KMAX - 1] = -1.f;
        li[KMAX - 1] = INT_MAX;
      }
      if (lane == 0) { wv_val[wv * KMAX + r] = bv; wv_idx[wv * KMAX + r] = bi; }
    }
    __syncthreads();
    // wave 0 ranks the survivors (an empty slot holds -1 and the largest id,
    // so it ranks after every real block)
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
    __syncthreads();  // LDS is reused by the next pair
  }
}

}  // namespace

hipError_t launch_gqa_cmp(const FwdParams& p, ssa_dtype /*dtype*/, hipStream_t stream) {
  tile_prefix_kernel_launch(p, stream);
  gqa_seq_kmax_kernel<<<dim3(p.batch, p.h_kv), 256, 0, stream>>>(p);
  const dim3 grid(p.max_tiles, p.h_q);
  if (p.d == 32) gqa_cmp_kernel<32><<<grid, 256, 0, stream>>>(p);
  else gqa_cmp_kernel<64><<<grid, 256, 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_gqa_topk(const FwdParams& p, ssa_dtype /*dtype*/, hipStream_t stream) {
  gqa_tile_prefix_kernel<<<1, 64, 0, stream>>>(p);
  const dim3 grid(p.max_tiles2, p.h_kv);
  if (p.d == 32) gqa_topk_kernel<32><<<grid, 256, 0, stream>>>(p);
  else gqa_topk_kernel<64><<<grid, 256, 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_gqa_fixup(const FwdParams& p, ssa_dtype /*dtype*/, hipStream_t stream) {
  // the number of pairs is read on the device, so the grid does not depend on it
  if (p.d == 32) {
    if (p.topk <= 16) gqa_fixup_kernel<32, 16><<<2048, 256, 0, stream>>>(p);
    else gqa_fixup_kernel<32, 32><<<2048, 256, 0, stream>>>(p);
  } else {
    if (p.topk <= 16) gqa_fixup_kernel<64, 16><<<2048, 256, 0, stream>>>(p);
    else gqa_fixup_kernel<64, 32><<<2048, 256, 0, stream>>>(p);
  }
  return hipGetLastError();
}

}  // namespace ssa
