// Compressed-block attention with top-k block selection, on MFMA (bf16, D = 64,
// one query head per key/value head).
//
// Direct3D-S2 page, "Method": every query attends to the mean-pooled blocks of
// its sequence, and the same query-to-block scores choose the top-k blocks
// for the selection branch.  With one query head per key/value group the
// score order is the logit order (softmax is monotone), so the ranking uses
// the float32 logits; ties go to the lower block id.
//
// Work split: a workgroup owns 128 consecutive sorted queries of one sequence
// and one head (4 waves x 32 queries) and streams the sequence's pooled keys
// and values through a two-slot LDS ring in tiles of 32 blocks: one barrier
// per tile, global loads issued two tiles ahead, loop unrolled by two so that
// ring slots and register sets are compile-time constants, and a two-stage
// software pipeline inside each wave (MFMAs of tile n next to the VALU work
// of tile n - 1).  Each tile is a
// v_mfma_f32_32x32x16_bf16 product S^T = Kbar Q^T; lane l then holds 16 block
// logits of query l % 32 (lanes l and l ^ 32 split the row between them).
//
// Two passes over the keys:
//  1. scan: per lane, the maximum of each tile's 16 logits (a "group max") is
//     merged into a sorted list of the KMAX largest group maxima with v_med3
//     (for a descending list L, inserting x gives L'[i] = med3(L[i-1], x, L[i])).
//     The row maximum is max(L0 of both lanes).  For every split a + b = KMAX
//     the two lanes hold a + b distinct elements no smaller than
//     min(L_A[a-1], L_B[b-1]); the largest such value, tau, bounds the KMAX-th
//     (so also the k-th, k <= KMAX) largest logit from below.
//  2. attend: recompute S, p = exp2((s - m) * scale * log2 e) with the exact
//     row maximum m (no rescaling), O^T += Vbar^T P^T on MFMA, and append the
//     logits >= tau with their block ids to the query's LDS candidate list
//     (its two lanes fill it from opposite ends).  Afterwards
//     each candidate's rank among the query's candidates (value descending,
//     block ascending) places it in the output.  A query whose list overflows
//     goes to the exact fallback kernel below.
#include <float.h>

#include <type_traits>

#include "ssa_internal.h"

namespace ssa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kD = 64;
constexpr int kKRow = kD + 8;          // LDS row of a key tile (bf16), padded against bank conflicts
constexpr int kVRow = kKeyTile + 8;    // LDS row of a transposed value tile (bf16)

__device__ __forceinline__ bf16x8 lds_b128(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// sorted position of sequence b's first token and one past its last
__device__ __forceinline__ void seq_token_range(const FwdParams& p, int b, int* s0, int* s1) {
  *s0 = p.win_off[p.seq_win_off[b]];
  *s1 = p.win_off[p.seq_win_off[b + 1]];
}

// tile_pre[b] = number of 128-query tiles of sequences before b
__global__ void tile_prefix_kernel(FwdParams p) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int run = 0;
  for (int b = 0; b < p.batch; ++b) {
    p.tile_pre[b] = run;
    int s0, s1;
    seq_token_range(p, b, &s0, &s1);
    run += (s1 - s0 + kQueryTile - 1) / kQueryTile;
  }
  p.tile_pre[p.batch] = run;
  p.fix[0] = 0;
}

template <int KMAX>
__global__ void __launch_bounds__(256, 3)
cmp_mfma_kernel(FwdParams p) {
  // candidate slots per query, shared by its two lanes (with the bound below
  // a query rarely has more than KMAX + 6; overflow goes to the fallback)
  constexpr int kCap = KMAX + KMAX / 2;
  __shared__ __align__(16) uint16_t k_lds[2][kKeyTile * kKRow];
  __shared__ __align__(16) uint16_t v_lds[2][kD * kVRow];
  // per query kCap data slots 1..kCap plus a sink slot at each end that
  // absorbs writes past the capacity: the logit, and the block id relative to
  // the sequence's first key tile (sequences with 65536 or more blocks take
  // the fallback for every query)
  __shared__ float cand_v[4 * 32 * (kCap + 2)];
  __shared__ uint16_t cand_j[4 * 32 * (kCap + 2)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
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

  // this lane's query (column l % 32 of the wave's 32 queries)
  const int qi = q_begin + wv * 32 + (lane & 31);
  const bool q_valid = qi < q_end;
  const int t = q_valid ? p.perm[qi] : 0;
  const int half = lane >> 5;          // which 8-wide k slice / which half of the keys

  // Q^T as the B operand: lane holds query (l % 32), d = 16 ks + 8 half + 0..7
  const uint16_t* Q = static_cast<const uint16_t*>(p.q);
  bf16x8 qb[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    u32x4 u = {0u, 0u, 0u, 0u};
    if (q_valid)
      u = *reinterpret_cast<const u32x4*>(Q + (static_cast<int64_t>(t) * p.h_q + h) * kD + 16 * ks + 8 * half);
    qb[ks] = __builtin_bit_cast(bf16x8, u);
  }

  const uint16_t* KB = static_cast<const uint16_t*>(p.kbar) + static_cast<int64_t>(h) * p.nb_cap * kD;
  const uint16_t* VT = static_cast<const uint16_t*>(p.vbar_t) + static_cast<int64_t>(h) * p.nb_cap * kD;
  const int kt0 = j0 / kKeyTile, kt1 = (j1 + kKeyTile - 1) / kKeyTile;
  const int n_kt = kt1 - kt0;

  // cooperative tile staging: thread -> 16 bytes of the key tile / value tile
  const int k_row = tid >> 3, k_chunk = tid & 7;      // key tile: 32 rows x 8 chunks
  const int v_row = tid >> 2, v_chunk = tid & 3;      // value tile: 64 rows x 4 chunks
  const uint16_t* kg = KB + (static_cast<int64_t>(kt0) * kKeyTile + k_row) * kD + 8 * k_chunk;
  const uint16_t* vg = VT + (static_cast<int64_t>(kt0) * kD + v_row) * kKeyTile + 8 * v_chunk;
  auto load_k = [&](int rel) { return *reinterpret_cast<const u32x4*>(kg + static_cast<int64_t>(rel) * kKeyTile * kD); };
  auto load_v = [&](int rel) { return *reinterpret_cast<const u32x4*>(vg + static_cast<int64_t>(rel) * kKeyTile * kD); };
  uint16_t* const ks_dst = &k_lds[0][k_row * kKRow + 8 * k_chunk];
  uint16_t* const vs_dst = &v_lds[0][v_row * kVRow + 8 * v_chunk];
  const uint16_t* const ka = &k_lds[0][(lane & 31) * kKRow + 8 * half];
  const uint16_t* const va = &v_lds[0][(lane & 31) * kVRow + 8 * half];

  // S^T of the key tile in ring slot `slot`
  auto qk = [&](int slot) {
    const uint16_t* kl = ka + slot * (kKeyTile * kKRow);
    f32x16 s = {};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128(kl + 16 * ks), qb[ks], s, 0, 0, 0);
    return s;
  };
  // keys of a partial tile outside [j0, j1) get -FLT_MAX
  auto mask = [&](int rel, f32x16& s) {
    const int kt = kt0 + rel;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = kt * kKeyTile + 8 * (r >> 2) + 4 * half + (r & 3);
      if (j < j0 || j >= j1) s[r] = -FLT_MAX;
    }
  };

  // Both passes run a two-stage software pipeline over the key tiles: step
  // `rel` issues the MFMAs of tile rel while the VALU works on the logits of
  // tile rel - 1, which are already in registers.  MFMA and VALU overlap only
  // within one wave's instruction stream on this hardware, so each wave needs
  // independent MFMA and VALU work side by side.  The first and last tile (the
  // only ones that can be partial) take the masking path.

  // ---------------- pass 1: sorted list of this lane's KMAX largest group maxima
  float L[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) L[i] = -FLT_MAX;
  auto list_insert = [&](const f32x16& s) {
    float m = fmaxf(s[0], fmaxf(s[1], s[2]));
#pragma unroll
    for (int r = 3; r < 15; r += 2) m = fmaxf(m, fmaxf(s[r], s[r + 1]));
    m = fmaxf(m, s[15]);
#pragma unroll
    for (int i = KMAX - 1; i >= 1; --i) L[i] = __builtin_amdgcn_fmed3f(L[i - 1], m, L[i]);
    L[0] = fmaxf(L[0], m);
  };
  {
    // ring: LDS slot (rel & 1) holds key tile rel; register set (rel & 1)
    // holds the tile two ahead of the one being stored
    u32x4 kr[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
    *reinterpret_cast<u32x4*>(ks_dst) = load_k(0);
    if (n_kt > 1) kr[1] = load_k(1);
    if (n_kt > 2) kr[0] = load_k(2);
    f32x16 s_prev;
    auto step = [&](int rel, auto slot_c, auto valu_c) {
      constexpr int slot = decltype(slot_c)::value;
      constexpr int valu = decltype(valu_c)::value;  // 0: none, 1: masked, 2: interior
      __syncthreads();  // key tile rel stored; the slot of tile rel - 1 is free
      if (rel + 1 < n_kt) *reinterpret_cast<u32x4*>(ks_dst + (slot ^ 1) * (kKeyTile * kKRow)) = kr[slot ^ 1];
      if (rel + 3 < n_kt) kr[slot ^ 1] = load_k(rel + 3);
      const f32x16 s_new = qk(slot);
      if (valu == 1) mask(rel - 1, s_prev);
      if (valu != 0) list_insert(s_prev);
      s_prev = s_new;
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using V0 = std::integral_constant<int, 0>;
    using V1 = std::integral_constant<int, 1>;
    using V2 = std::integral_constant<int, 2>;
    step(0, S0{}, V0{});
    if (n_kt > 1) step(1, S1{}, V1{});
    int rel = 2;
    for (; rel + 1 < n_kt; rel += 2) {
      step(rel, S0{}, V2{});
      step(rel + 1, S1{}, V2{});
    }
    if (rel < n_kt) step(rel, S0{}, V2{});
    mask(n_kt - 1, s_prev);
    list_insert(s_prev);
  }
  // row maximum, and the best lower bound on the KMAX-th largest logit (hence
  // on the k-th, k <= KMAX): for any split a + b = KMAX the two lanes hold a
  // and b distinct elements >= min(L_this[a-1], L_other[b-1])
  float Lo[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) Lo[i] = __shfl_xor(L[i], 32);
  const float row_max = fmaxf(L[0], Lo[0]);
  float tau = fmaxf(L[KMAX - 1], Lo[KMAX - 1]);
#pragma unroll
  for (int a = 1; a < KMAX; ++a) tau = fmaxf(tau, fminf(L[a - 1], Lo[KMAX - 1 - a]));

  // ---------------- pass 2: probabilities, P V, candidates
  const float c2 = p.scale * kLog2e;
  const float mc = row_max * c2;
  f32x16 o0 = {}, o1 = {};
  float lsum0 = 0.f, lsum1 = 0.f;
  // the query's candidate list: lane half 0 writes slots 1, 2, ... upward,
  // half 1 writes kCap, kCap - 1, ... downward; a write past the capacity
  // lands in the sink slot (0 or kCap + 1) and the query goes to the fallback
  const int qbase = (wv * 32 + (lane & 31)) * (kCap + 2);
  int cpos = qbase + (half ? kCap : 1);
  const int climit = qbase + (half ? 0 : kCap + 1);
  const int cstep = half ? -1 : 1;
  const float tau_eff = q_valid ? tau : __builtin_inff();  // columns without a query never hit
  const int key_lane = 4 * half;
  // probabilities, row sums and candidates of tile rel's logits; returns P^T
  // as two bf16 B operands
  auto softmax_tile = [&](int rel, const f32x16& s, bf16x8 (&pb)[2]) {
    float pr[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      pr[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c2, -mc));
      if (r & 1) lsum1 += pr[r]; else lsum0 += pr[r];
    }
    const int key0 = rel * kKeyTile + key_lane;   // relative to the first key tile
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (s[r] >= tau_eff) {
        cand_v[cpos] = s[r];
        cand_j[cpos] = static_cast<uint16_t>(key0 + 8 * (r >> 2) + (r & 3));
        cpos = (cpos == climit) ? cpos : cpos + cstep;
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[ks][i] = static_cast<__bf16>(pr[8 * ks + i]);
  };
  auto pv = [&](int slot, const bf16x8 (&pb)[2]) {
    const uint16_t* vl = va + slot * (kD * kVRow);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128(vl + 16 * ks), pb[ks], o0, 0, 0, 0);
      o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128(vl + 32 * kVRow + 16 * ks), pb[ks], o1, 0, 0, 0);
    }
  };
  {
    // key slot (rel & 1) holds key tile rel (read by the MFMAs of step rel);
    // value slot (rel & 1) holds value tile rel (read by step rel + 1)
    u32x4 kr[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
    u32x4 vr[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
    __syncthreads();  // every wave is done with pass 1's ring
    *reinterpret_cast<u32x4*>(ks_dst) = load_k(0);
    if (n_kt > 1) kr[1] = load_k(1);
    if (n_kt > 2) kr[0] = load_k(2);
    vr[0] = load_v(0);
    if (n_kt > 1) vr[1] = load_v(1);
    f32x16 s_prev;
    auto step = [&](int rel, auto slot_c, auto valu_c) {
      constexpr int slot = decltype(slot_c)::value;
      constexpr int valu = decltype(valu_c)::value;  // 0: none, 1: masked, 2: interior
      __syncthreads();  // key tile rel and value tile rel - 1 stored; older slots free
      if (rel + 1 < n_kt) *reinterpret_cast<u32x4*>(ks_dst + (slot ^ 1) * (kKeyTile * kKRow)) = kr[slot ^ 1];
      *reinterpret_cast<u32x4*>(vs_dst + slot * (kD * kVRow)) = vr[slot];
      if (rel + 3 < n_kt) kr[slot ^ 1] = load_k(rel + 3);
      if (rel + 2 < n_kt) vr[slot] = load_v(rel + 2);
      const f32x16 s_new = qk(slot);
      if (valu != 0) {
        if (valu == 1) mask(rel - 1, s_prev);
        bf16x8 pb[2];
        softmax_tile(rel - 1, s_prev, pb);
        pv(slot ^ 1, pb);
      }
      s_prev = s_new;
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using V0 = std::integral_constant<int, 0>;
    using V1 = std::integral_constant<int, 1>;
    using V2 = std::integral_constant<int, 2>;
    step(0, S0{}, V0{});
    if (n_kt > 1) step(1, S1{}, V1{});
    int rel = 2;
    for (; rel + 1 < n_kt; rel += 2) {
      step(rel, S0{}, V2{});
      step(rel + 1, S1{}, V2{});
    }
    if (rel < n_kt) step(rel, S0{}, V2{});
    // last tile: its values were stored by the final step
    __syncthreads();
    mask(n_kt - 1, s_prev);
    bf16x8 pb[2];
    softmax_tile(n_kt - 1, s_prev, pb);
    pv((n_kt - 1) & 1, pb);
  }
  // appended so far (a pointer parked on the sink slot counts as overflow)
  const int cnt = half ? qbase + kCap - cpos : cpos - (qbase + 1);

  // ---------------- o_cmp (times its gate) into the branch accumulator
  const float lsum = lsum0 + lsum1;
  const float l_q = lsum + __shfl_xor(lsum, 32);
  if (q_valid) {
    const uint16_t* gt = static_cast<const uint16_t*>(p.gates) + (static_cast<int64_t>(t) * p.h_q + h) * 3;
    const float f = bf16_bits_to_f32(gt[0]) / l_q;
    float* dst = p.acc + (static_cast<int64_t>(t) * p.h_q + h) * kD;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int d = 8 * rb + 4 * half;
      *reinterpret_cast<float4*>(dst + d) =
          make_float4(o0[4 * rb] * f, o0[4 * rb + 1] * f, o0[4 * rb + 2] * f, o0[4 * rb + 3] * f);
      *reinterpret_cast<float4*>(dst + 32 + d) =
          make_float4(o1[4 * rb] * f, o1[4 * rb + 1] * f, o1[4 * rb + 2] * f, o1[4 * rb + 3] * f);
    }
  }

  // ---------------- exact top-k among the candidates
  wave_lds_sync();
  const int cnt_other = __shfl_xor(cnt, 32);
  // kCap - 1: a lane parked on its sink also counts; relative block ids
  // must fit 16 bits
  const bool overflow = cnt + cnt_other > kCap - 1 || n_kt * kKeyTile > 65536;
  const int k_eff = min(p.topk, nbs);
  int32_t* out_sel = p.topk_idx + (static_cast<int64_t>(t) * p.h_kv + h) * p.topk;
  if (q_valid && overflow) {
    if (half == 0) {
      const int slot = atomicAdd(&p.fix[0], 1);
      p.fix[1 + slot] = qi * p.h_kv + h;
    }
  } else if (q_valid) {
    // the query's candidates: slots [1, 1 + c0) from lane half 0 and
    // [kCap + 1 - c1, kCap + 1) from lane half 1
    const int c0 = half ? cnt_other : cnt, c1 = half ? cnt : cnt_other;
    const int mine0 = qbase + (half ? kCap + 1 - cnt : 1);
    const int jbase = kt0 * kKeyTile;
    for (int i = 0; i < cnt; ++i) {
      const float cv = cand_v[mine0 + i];
      const int cj = cand_j[mine0 + i];
      int rank = 0;
      for (int e = qbase + 1; e < qbase + 1 + c0; ++e) {
        const float ov = cand_v[e];
        rank += (ov > cv) || (ov == cv && cand_j[e] < cj);
      }
      for (int e = qbase + kCap + 1 - c1; e < qbase + kCap + 1; ++e) {
        const float ov = cand_v[e];
        rank += (ov > cv) || (ov == cv && cand_j[e] < cj);
      }
      if (rank < k_eff) out_sel[rank] = jbase + cj;
    }
    if (half == 0)
      for (int r = k_eff; r < p.topk; ++r) out_sel[r] = -1;
  }
}

// Exact top-k for the (sorted position, group) pairs whose candidate list
// overflowed: one wave per pair, each lane keeps a sorted list of its strided blocks'
// logits, then the wave pops the best heads (value desc, block asc).
template <int KMAX>
__global__ void __launch_bounds__(256)
topk_fixup_kernel(FwdParams p) {
  const int lane = threadIdx.x & 63;
  const int n_fix = p.fix[0];
  const uint16_t* Q = static_cast<const uint16_t*>(p.q);
  for (int item = blockIdx.x * 4 + (threadIdx.x >> 6); item < n_fix; item += gridDim.x * 4) {
    const int entry = p.fix[1 + item];
    const int i = entry / p.h_kv, g = entry % p.h_kv;
    const int t = p.perm[i];
    const int tg = t * p.h_kv + g;
    int lo = 0, hi = p.batch - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.win_off[p.seq_win_off[mid]] <= i) lo = mid; else hi = mid - 1;
    }
    const int j0 = p.seq_blk_off[lo], j1 = p.seq_blk_off[lo + 1];
    float q[kD];
#pragma unroll
    for (int d = 0; d < kD; ++d) q[d] = bf16_bits_to_f32(Q[(static_cast<int64_t>(t) * p.h_q + g) * kD + d]);
    const uint16_t* KB = static_cast<const uint16_t*>(p.kbar) + static_cast<int64_t>(g) * p.nb_cap * kD;
    float lv[KMAX];
    int li[KMAX];
#pragma unroll
    for (int e = 0; e < KMAX; ++e) { lv[e] = -FLT_MAX; li[e] = 0x7FFFFFFF; }
    for (int j = j0 + lane; j < j1; j += 64) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < kD / 8; ++c) {
        const u32x4 u = *reinterpret_cast<const u32x4*>(KB + static_cast<int64_t>(j) * kD + 8 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s = fmaf(q[8 * c + 2 * e], __uint_as_float(u[e] << 16), s);
          s = fmaf(q[8 * c + 2 * e + 1], __uint_as_float(u[e] & 0xFFFF0000u), s);
        }
      }
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
    const int k_eff = min(p.topk, j1 - j0);
    int32_t* out_sel = p.topk_idx + static_cast<int64_t>(tg) * p.topk;
    for (int r = 0; r < k_eff; ++r) {
      float bv = lv[0];
      int bi = li[0];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
      }
      if (li[0] == bi) {
#pragma unroll
        for (int e = 0; e < KMAX - 1; ++e) { lv[e] = lv[e + 1]; li[e] = li[e + 1]; }
        lv[KMAX - 1] = -FLT_MAX;
        li[KMAX - 1] = 0x7FFFFFFF;
      }
      if (lane == 0) out_sel[r] = bi;
    }
    if (lane == 0)
      for (int r = k_eff; r < p.topk; ++r) out_sel[r] = -1;
  }
}

}  // namespace

hipError_t launch_cmp_mfma(const FwdParams& p, ssa_dtype /*dtype*/, hipStream_t stream) {
  tile_prefix_kernel<<<1, 64, 0, stream>>>(p);
  const dim3 grid(p.max_tiles, p.h_q);
  if (p.topk <= 16) cmp_mfma_kernel<16><<<grid, 256, 0, stream>>>(p);
  else cmp_mfma_kernel<32><<<grid, 256, 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_topk_fixup(const FwdParams& p, ssa_dtype /*dtype*/, hipStream_t stream) {
  if (p.topk <= 16) topk_fixup_kernel<16><<<1024, 256, 0, stream>>>(p);
  else topk_fixup_kernel<32><<<1024, 256, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace ssa
