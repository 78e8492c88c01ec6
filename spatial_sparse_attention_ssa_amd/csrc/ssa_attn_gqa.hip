// Compressed-block attention and top-k block selection for grouped query
// heads on MFMA (bf16, D = 32 or 64, 2 to 16 query heads per key/value head).
//
// Direct3D-S2 page, "Method": every query attends to the mean-pooled blocks of
// its sequence, and the attention scores choose the top-k blocks; LSRM
// article, its sparse-attention section: the selection is shared by the query
// heads of a key/value group.  Here the score of block j for a query token t
// and group g is the sum over the group's heads of the softmax probability of
// j, so the heads' softmax normalisers are needed before any block can be
// ranked.  Two kernels:
//
//  gqa_cmp_kernel: o_cmp of every (token, query head) (S^T = Kbar Q^T; the
//    softmax shift is the bound |q| max|Kbar| when it is small enough, else a
//    running shift per query head, rescaled only when a tile maximum exceeds
//    it by 8 in log2 units), adds G0 * o_cmp to the float32 branch
//    accumulator and stores the head's log2 normaliser c, so that the
//    probability of block j is 2^(s_j * scale * log2 e - c).  Work split as
//    in the one-head-per-group kernel: 256 sorted queries of one sequence and
//    one query head per workgroup, 4 waves x two 32-query blocks, pooled keys
//    / values streamed through a two-slot LDS ring.
//
//  gqa_topk_kernel: S = Q Kbar^T with the rows of the MFMA tile being
//    (token, head) pairs, 2 tokens x 16 heads, and the columns 32 blocks.  A
//    lane then holds one block and 8 heads of each token.  A workgroup owns
//    16 sorted tokens of one sequence and one group (4 waves x 2 row blocks).
//    A warm-up over the sequence's probe set gives each token a lower bound
//    on its k-th score; in the main pass a (token, block) pair is scored
//    exactly only when the bound 16 * max_h p_h reaches the admission score,
//    which most pairs do not, so most pairs cost an FMA and a max per head
//    instead of an exponential.  Exact: the top k of the blocks seen so far
//    are always among the admitted candidates (see the kernel).  A group of
//    G < 16 heads fills heads 0 .. G - 1 of the 16 and leaves the rest empty
//    (zero query, probability 0), so the group score and its order are those
//    of the G heads; the bound uses 2^ceil(log2 G) instead of 16.
#include <float.h>
#include <math.h>
#include <limits.h>

#include <type_traits>

#include "ssa_internal.h"

namespace ssa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kGroup = 16;            // heads per group in the top-k kernel's tiles (G <= 16 of them real)
constexpr int kTopkTile = 16;         // sorted tokens per workgroup of the top-k kernel
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

// maximum of 8 values (never NaN here) as a three-operand tree, which
// becomes v_maximum3_f32
__device__ __forceinline__ float max8(const float* v) {
  const float a = __builtin_elementwise_maximum(__builtin_elementwise_maximum(v[0], v[1]), v[2]);
  const float b = __builtin_elementwise_maximum(__builtin_elementwise_maximum(v[3], v[4]), v[5]);
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), __builtin_elementwise_maximum(v[6], v[7]));
}

__device__ __forceinline__ bf16x8 lds_b128(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// the larger of v in lane l and lane l ^ 32 (v_permlane32_swap, no LDS)
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// lane l and lane l ^ 32 exchange v (v_permlane32_swap, no LDS); the two
// results are v of both lanes, so their sum is the same on both lanes of a
// pair
__device__ __forceinline__ float pair_add(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
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

// Per wave: a ring of (token, block) pairs that passed the bound, scored in
// batches of up to 64, and per token a list of admitted candidates.
constexpr int kQCap = 128;     // queue entries per wave (at most 63 + 64 are pending)
constexpr int kLCap = 96;      // candidate keys per token
constexpr int kCompact = 32;   // a list longer than this is cut to its top k (k <= 32)

// D = 32: three workgroups per compute unit (LDS: 46 KB each; at most 168
// registers); D = 64 keeps two, since three would spill
template <int D>
__global__ void __launch_bounds__(256, D == 32 ? 3 : 2)
gqa_topk_kernel(FwdParams p) {
  constexpr int KS = D / 16;
  __shared__ __align__(16) float qy[4][kQCap][16];   // a pair's 16 values z_h (lane half h wrote 8 h ... 8 h + 7)
  __shared__ int qm[4][kQCap];                       // block << 2 | token of the wave
  __shared__ uint64_t lst[4][4][kLCap];              // candidate keys per wave and token

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
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
  const int nbs = j1 - j0;
  const int k_eff = min(p.topk, nbs);
  const float c2 = p.scale * kLog2e;
  const uint16_t* Q = static_cast<const uint16_t*>(p.q);
  const int G = p.h_q / p.h_kv;   // real heads of the 16 (2 .. 16)
  // log2 of the bound's factor (a power of two >= G) plus a rounding margin
  const float lg_bound = G > 8 ? 4.001f : G > 4 ? 3.001f : G > 2 ? 2.001f : 1.001f;

  // row blocks x = 0, 1 of this wave: tokens 4 wv + 2 x + {0, 1} (the wave's
  // tokens 2 x + 0 and 2 x + 1); A operand row (lane % 32) = (token
  // (lane % 32) / 16, head lane % 16)
  bf16x8 qa[2][KS];
  // -c_h / c2 for this lane's 16 accumulator rows (c_h: the head's log2
  // normaliser): the MFMA accumulators start there, so they hold
  // z = s - c_h / c2 and the head's probability of the block is 2^(z c2)
  float cz[2][16];
  int tk[2][2];          // sorted positions of the row block's two tokens
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    tk[x][0] = t_begin + 4 * wv + 2 * x;
    tk[x][1] = tk[x][0] + 1;
    const int mine = tk[x][l32 >> 4];
    const bool ok = mine < t_end && (lane & 15) < G;
    const int tt = ok ? p.perm[mine] : 0;
    const int hq = g * G + (lane & 15);
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
      cz[x][r] = -INFINITY;  // no probability for a missing token or an empty head
      if (pos < t_end && (row & 15) < G)
        cz[x][r] = -p.norm[static_cast<int64_t>(p.perm[pos]) * p.h_q + g * G + (row & 15)] / c2;
    }
  }

  const uint16_t* KB = static_cast<const uint16_t*>(p.kbar) + static_cast<int64_t>(g) * p.nb_cap * D;
  // Each lane loads its own MFMA operand of every key tile (16 bytes per k
  // step of row row_of(rel, lane % 32)), two tiles ahead; the four waves read
  // the same tiles at about the same time, mostly from L1, and need no
  // barrier, so a wave that stops to score a batch does not hold up the
  // others.
  auto stream_tiles = [&](int n_t, auto row_of, auto body) {
    auto load = [&](int rel, bf16x8 (&kb)[KS]) {
      const uint16_t* src = KB + static_cast<int64_t>(row_of(rel, l32)) * D + 8 * half;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kb[ks] = lds_b128(src + 16 * ks);
    };
    // three register sets used in turn (the loop is unrolled by three, so no
    // register is copied while its load is in flight): each set is reloaded
    // right after its step and has the next two steps to arrive
    bf16x8 ba[KS], bb[KS], bc[KS];
    load(0, ba);
    load(min(1, n_t - 1), bb);
    load(min(2, n_t - 1), bc);
    int rel = 0;
    for (; rel + 2 < n_t; rel += 3) {
      body(rel, ba);
      load(min(rel + 3, n_t - 1), ba);
      body(rel + 1, bb);
      load(min(rel + 4, n_t - 1), bb);
      body(rel + 2, bc);
      load(min(rel + 5, n_t - 1), bc);
    }
    if (rel < n_t) body(rel, ba);
    if (rel + 1 < n_t) body(rel + 1, bb);
  };
  // z of row block x against a key tile
  auto shifted = [&](int x, const bf16x8 (&kb)[KS]) {
    f32x16 z;
#pragma unroll
    for (int r = 0; r < 16; ++r) z[r] = cz[x][r];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) z = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[x][ks], kb[ks], z, 0, 0, 0);
    return z;
  };
  // a token's group score: each lane half sums the probabilities 2^(z c2)
  // of its 8 heads in order, then the two halves are added
  auto half_sum = [c2](const float* zv) {
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) sum += __builtin_amdgcn_exp2f(zv[r] * c2);
    return sum;
  };

  // ---------------- warm-up: a lower bound tau0 on each token's k-th score
  // The probe set (the sequence's kProbeBlocks pooled keys of largest norm,
  // which hold most of the top k) or, for a sequence of at most that many
  // blocks, the sequence itself, is scored exactly; each lane keeps the two
  // best scores it saw per token, and the k-th largest of the 64 values of a
  // token bounds its k-th score from below (they are scores of 64 distinct
  // blocks).
  const int pslot = p.probe_slot[b];
  const int32_t* pids =
      pslot >= 0 ? p.probe_ids + (static_cast<int64_t>(g) * p.max_probe_slots + pslot) * kProbeBlocks : nullptr;
  float w1[2] = {-2.f, -2.f}, w2[2] = {-2.f, -2.f};
  auto warm_body = [&](int rel, const bf16x8 (&kb)[KS]) {
    bool jok;
    if (pids) {
      jok = true;
    } else {
      const int j = (kt0 + rel) * kKeyTile + l32;
      jok = j >= j0 && j < j1;
    }
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const f32x16 z = shifted(x, kb);
      float y[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) y[r] = z[r];
      const float sum0 = pair_add(half_sum(y)), sum1 = pair_add(half_sum(y + 8));
      const float sc = jok ? (half ? sum1 : sum0) : -2.f;
      w2[x] = __builtin_amdgcn_fmed3f(w1[x], sc, w2[x]);
      w1[x] = fmaxf(w1[x], sc);
    }
  };
  if (pids) {
    stream_tiles(kProbeBlocks / kKeyTile, [&](int rel, int r) { return pids[rel * kKeyTile + r]; }, warm_body);
  } else {
    stream_tiles(n_kt, [&](int rel, int r) { return (kt0 + rel) * kKeyTile + r; }, warm_body);
  }

  // per wave token t = 2 x + h: admission key, bound threshold, list length
  uint64_t min_key[4];
  float theta[4];
  int cnt[4] = {0, 0, 0, 0};
  {
    float* wv_scr = &qy[wv][0][0];   // 256 floats: [x][h][l32][2]
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      wv_scr[((2 * x + half) * 32 + l32) * 2] = w1[x];
      wv_scr[((2 * x + half) * 32 + l32) * 2 + 1] = w2[x];
    }
    wave_lds_sync();
    float tau[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      // the k-th largest of the token's 64 values (or -1: fewer than k valid)
      const float* v = wv_scr + (2 * x + half) * 64;
      const float a = w1[x], c = w2[x];
      int gt_a = 0, ge_a = 0, gt_c = 0, ge_c = 0;
      for (int i = 0; i < 64; ++i) {
        const float vi = v[i];
        gt_a += vi > a ? 1 : 0;
        ge_a += vi >= a ? 1 : 0;
        gt_c += vi > c ? 1 : 0;
        ge_c += vi >= c ? 1 : 0;
      }
      float t = -FLT_MAX;
      if (gt_a < k_eff && ge_a >= k_eff) t = a;
      if (gt_c < k_eff && ge_c >= k_eff) t = c;
      // every lane of the half that holds the k-th value holds the same one
      t = fmaxf(t, __shfl_xor(t, 1));
      t = fmaxf(t, __shfl_xor(t, 2));
      t = fmaxf(t, __shfl_xor(t, 4));
      t = fmaxf(t, __shfl_xor(t, 8));
      t = fmaxf(t, __shfl_xor(t, 16));
      tau[x] = t;
    }
    wave_lds_sync();
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int x = t >> 1, h = t & 1;
      const float tau0 = __shfl(tau[x], 32 * h);
      if (tk[x][h] >= t_end) {
        min_key[t] = ~0ull;      // no token: admit nothing
        theta[t] = INFINITY;
      } else if (tau0 >= 0.f) {
        // scores are >= 0, so their float bits order like their values
        min_key[t] = static_cast<uint64_t>(__float_as_uint(tau0)) << 32;
        theta[t] = tau0 > 0.f ? (__log2f(tau0) - lg_bound) / c2 : -INFINITY;
      } else {
        min_key[t] = 0ull;       // fewer than k scored blocks: admit all
        theta[t] = -INFINITY;
      }
    }
  }

  // ---------------- main pass over the sequence's tiles
  // A pair (token, block) whose largest z over the heads, m, satisfies
  // 2^lg * 2^(m c2) < (the admission score) cannot be admitted, since its
  // score is a sum of G <= 2^lg terms 2^(z_h c2); theta holds log2 of that
  // score minus lg (and a margin for rounding), divided by c2.  Pairs that pass are queued
  // with their 16 values z; a batch computes their scores exactly (in the
  // warm-up's arithmetic), and a pair whose key
  // (score, then lower block first) reaches min_key joins its token's list.
  // A list longer than kCompact is cut to its top k by rank counting, and
  // min_key becomes one above the k-th key: the top k of the blocks seen so
  // far are always in the list, and no list exceeds kCompact + 64 entries.
  int qh = 0, qn = 0;   // queue head and pending entries (wave-uniform, qn < 64 between row blocks)
  const uint64_t lt_mask = (uint64_t(1) << lane) - 1;
  auto list_rank = [&](int t, int n, uint64_t& k1, uint64_t& k2, int& r1, int& r2) {
    const uint64_t* L = lst[wv][t];
    k1 = lane < n ? L[lane] : 0ull;
    k2 = lane + 64 < n ? L[lane + 64] : 0ull;
    r1 = 0;
    r2 = 0;
    for (int i = 0; i < n; ++i) {
      const uint64_t ki = L[i];
      r1 += ki > k1 ? 1 : 0;
      r2 += ki > k2 ? 1 : 0;
    }
  };
  auto compact = [&](int t) {
    const int n = cnt[t];
    uint64_t k1, k2;
    int r1, r2;
    list_rank(t, n, k1, k2, r1, r2);
    wave_lds_sync();
    uint64_t* L = lst[wv][t];
    if (lane < n && r1 < k_eff) L[r1] = k1;
    if (lane + 64 < n && r2 < k_eff) L[r2] = k2;
    wave_lds_sync();
    cnt[t] = k_eff;   // n > kCompact >= k_eff
    min_key[t] = L[k_eff - 1] + 1;
    const float smin = __uint_as_float(static_cast<uint32_t>(min_key[t] >> 32));
    theta[t] = smin > 0.f ? (__log2f(smin) - lg_bound) / c2 : -INFINITY;
  };
  auto process = [&]() {
    const int nbat = min(qn, 64);
    const bool act = lane < nbat;
    const int e = (qh + lane) & (kQCap - 1);
    uint64_t key = 0ull;
    int tok = -1;
    if (act) {
      float yv[16];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float4 u = *reinterpret_cast<const float4*>(&qy[wv][e][4 * c]);
        yv[4 * c] = u.x;
        yv[4 * c + 1] = u.y;
        yv[4 * c + 2] = u.z;
        yv[4 * c + 3] = u.w;
      }
      // the same two half sums, added as the warm-up adds them
      const float sc = half_sum(yv) + half_sum(yv + 8);
      const int m = qm[wv][e];
      tok = m & 3;
      key = (static_cast<uint64_t>(__float_as_uint(sc)) << 32) | static_cast<uint32_t>(~(m >> 2));
    }
    wave_lds_sync();
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bool adm = tok == t && key >= min_key[t];
      const uint64_t bt = __ballot(adm);
      if (adm) lst[wv][t][cnt[t] + __popcll(bt & lt_mask)] = key;
      cnt[t] += __popcll(bt);
    }
    qh = (qh + nbat) & (kQCap - 1);
    qn -= nbat;
    wave_lds_sync();
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (cnt[t] > kCompact) compact(t);
  };
  auto main_body = [&](int rel, const bf16x8 (&kb)[KS]) {
    const int j = (kt0 + rel) * kKeyTile + l32;
    const bool jok = j >= j0 && j < j1;
    const uint32_t below = (1u << l32) - 1u;
    // both row blocks' MFMAs first: block 1's run beside block 0's filter
    f32x16 yx[2];
    yx[0] = shifted(0, kb);
    yx[1] = shifted(1, kb);
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      float y[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) y[r] = yx[x][r];
      // the pair in lanes l and l + 32 passes when either half's maximum
      // does: both lanes take the larger of the two (v_permlane32_swap), so
      // they decide alike and the low half of the ballot has one bit per pair
      const float m0 = pair_max(max8(y)), m1 = pair_max(max8(y + 8));
      const bool p0 = (m0 >= theta[2 * x]) & jok, p1 = (m1 >= theta[2 * x + 1]) & jok;
      const uint32_t b0 = static_cast<uint32_t>(__ballot(p0));
      const uint32_t b1 = static_cast<uint32_t>(__ballot(p1));
      const int n0 = __popc(b0), n1 = __popc(b1);
      if (p0) {
        const int e = (qh + qn + __popc(b0 & below)) & (kQCap - 1);
        float4* dst = reinterpret_cast<float4*>(&qy[wv][e][8 * half]);
        dst[0] = make_float4(y[0], y[1], y[2], y[3]);
        dst[1] = make_float4(y[4], y[5], y[6], y[7]);
        if (half == 0) qm[wv][e] = (j << 2) | (2 * x);
      }
      if (p1) {
        const int e = (qh + qn + n0 + __popc(b1 & below)) & (kQCap - 1);
        float4* dst = reinterpret_cast<float4*>(&qy[wv][e][8 * half]);
        dst[0] = make_float4(y[8], y[9], y[10], y[11]);
        dst[1] = make_float4(y[12], y[13], y[14], y[15]);
        if (half == 0) qm[wv][e] = (j << 2) | (2 * x + 1);
      }
      qn += n0 + n1;
      if (qn >= 64) {
        wave_lds_sync();
        process();
      }
    }
  };
  stream_tiles(n_kt, [&](int rel, int r) { return (kt0 + rel) * kKeyTile + r; }, main_body);
  wave_lds_sync();
  while (qn > 0) process();

  // ---------------- each token's top k: rank its list (score descending,
  // equal scores by block ascending)
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int x = t >> 1, h = t & 1;
    const int pos = tk[x][h];
    if (pos >= t_end) continue;   // uniform
    int32_t* out_sel = p.topk_idx + (static_cast<int64_t>(p.perm[pos]) * p.h_kv + g) * p.topk;
    const int n = cnt[t];
    uint64_t k1, k2;
    int r1, r2;
    list_rank(t, n, k1, k2, r1, r2);
    if (lane < n && r1 < k_eff) out_sel[r1] = static_cast<int32_t>(~static_cast<uint32_t>(k1));
    if (lane + 64 < n && r2 < k_eff) out_sel[r2] = static_cast<int32_t>(~static_cast<uint32_t>(k2));
    for (int r = min(n, k_eff) + lane; r < p.topk; r += 64) out_sel[r] = -1;
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
  probe_select_launch(p, stream);
  const dim3 grid(p.max_tiles2, p.h_kv);
  if (p.d == 32) gqa_topk_kernel<32><<<grid, 256, 0, stream>>>(p);
  else gqa_topk_kernel<64><<<grid, 256, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace ssa
