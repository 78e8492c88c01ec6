// Selected-block attention and the gated sum (bf16, D = 32 or 64; query head
// h reads key/value head g = h / (h_q / h_kv) and the selection of group g).
// Groups of 16 query heads take the MFMA kernel at the end of this file.
//
// Direct3D-S2 page, "Method": all tokens of the top-k selected blocks take
// part in a second attention; the three branch outputs are summed with the
// predicted gates.  The window and compressed branches have already written
// G2 * o_win + G0 * o_cmp to the float32 accumulator; this kernel adds
// G1 * o_sel, rounds once to bfloat16 and writes the output row.
//
// D / 16 lanes serve one (token, head) pair, each owning 16 dims (two runs
// of 8, one in each half of the row); a wave
// covers 64 / (D / 16) pairs of one head (pairs are ordered head-major, so the rows
// gathered at any time belong to one or two heads and stay in the Infinity
// Cache).  Keys and values come from the head-major sorted copies, where a
// block is a contiguous run of rows.  First the pair's lanes turn its block
// list into a list of row positions in LDS (each lane expands every fourth
// block; one prefix over the four lanes places them), then the lanes stream
// the listed rows with an online softmax: every row's position is known up
// front, so a row's loads wait on no block offset.  (Streaming several rows
// per step measured slower: the extra registers cost occupancy.)  Rows past
// the LDS list's capacity, which only very large selections reach, are walked
// block by block afterwards.
#include <float.h>
#include <math.h>

#include "ssa_internal.h"

namespace ssa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kDL = 16;      // dims per lane
constexpr int kList = 64;    // row positions listed per pair
constexpr int kStep = 1;     // rows per step

__device__ __forceinline__ void load16(const uint16_t* p, float (&x)[kDL]) {
  const u32x4 a = *reinterpret_cast<const u32x4*>(p);
  const u32x4 b = *reinterpret_cast<const u32x4*>(p + 8);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = __uint_as_float(a[e] << 16);
    x[2 * e + 1] = __uint_as_float(a[e] & 0xFFFF0000u);
    x[8 + 2 * e] = __uint_as_float(b[e] << 16);
    x[8 + 2 * e + 1] = __uint_as_float(b[e] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// two packed bf16 values times two others, plus c (v_dot2_f32_bf16: the
// products are exact, the sum is float32); the words go through scalars
// because this compiler's __builtin_bit_cast of a vector element reads
// element 0
__device__ __forceinline__ float dot2(uint32_t x, uint32_t y, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), __builtin_bit_cast(bf16x2, y), c, false);
}

// 16 bf16 values of a row, packed: 8 at p and 8 at p + hoff (the lane's
// dims in the first and in the second half of the row)
struct Row16 {
  u32x4 a, b;
  __device__ __forceinline__ void load(const uint16_t* p, int hoff) {
    a = *reinterpret_cast<const u32x4*>(p);
    b = *reinterpret_cast<const u32x4*>(p + hoff);
  }
  // the row times 16 packed bf16 query values
  __device__ __forceinline__ float dot(const Row16& q) const {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t ae = a[e], be = b[e], qa = q.a[e], qb = q.b[e];
      s0 = dot2(ae, qa, s0);
      s1 = dot2(be, qb, s1);
    }
    return s0 + s1;
  }
  __device__ __forceinline__ void axpy(float w, float (&o)[kDL]) const {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[2 * e] = fmaf(w, bf_lo(a[e]), o[2 * e]);
      o[2 * e + 1] = fmaf(w, bf_hi(a[e]), o[2 * e + 1]);
      o[8 + 2 * e] = fmaf(w, bf_lo(b[e]), o[8 + 2 * e]);
      o[8 + 2 * e + 1] = fmaf(w, bf_hi(b[e]), o[8 + 2 * e + 1]);
    }
  }
};

// Online-softmax state of one lane (16 dims of one pair).
struct SelState {
  float m, l, o[kDL];
  __device__ __forceinline__ void init() {
    m = -FLT_MAX;
    l = 0.f;
#pragma unroll
    for (int e = 0; e < kDL; ++e) o[e] = 0.f;
  }
  // logits s2[u] (already times scale * log2 e; -FLT_MAX = absent) and their
  // value rows
  template <int U>
  __device__ __forceinline__ void add(const float (&s2)[U], const Row16 (&v)[U]) {
    float mx = m;
#pragma unroll
    for (int u = 0; u < U; ++u) mx = __builtin_elementwise_maximum(mx, s2[u]);
    if (mx > m) {
      const float corr = __builtin_amdgcn_exp2f(m - mx);
      l *= corr;
#pragma unroll
      for (int e = 0; e < kDL; ++e) o[e] *= corr;
      m = mx;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float pr = __builtin_amdgcn_exp2f(s2[u] - m);
      l += pr;
      v[u].axpy(pr, o);
    }
  }
};

// sum over the LP (2 or 4) lanes of a pair: DPP quad permutations (lane
// xor 1, then xor 2), no LDS round trip
template <int LP>
__device__ __forceinline__ float pair_sum(float s) {
  static_assert(LP == 2 || LP == 4, "pairs of 2 or 4 lanes");
  s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0xB1, 0xF, 0xF, false));  // [1,0,3,2]
  if (LP == 4) s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x4E, 0xF, 0xF, false));  // [2,3,0,1]
  return s;
}

template <int KMAX, int D>
__global__ void __launch_bounds__(256)
sel_combine_kernel(FwdParams p) {
  constexpr int kD = D;
  constexpr int LP = D / kDL;             // lanes per pair
  constexpr int NP = 256 / LP;            // pairs per workgroup
  // lane sub of a pair owns dims [8 sub, 8 sub + 8) and [D/2 + 8 sub, D/2 +
  // 8 sub + 8): each 16-byte load instruction of a pair then covers one
  // contiguous half row, so a row gather touches half as many 64-byte
  // sectors per instruction as with 16 consecutive dims per lane
  constexpr int kHalf = D / 2;
  constexpr int kLaneOff = kDL / 2;
  __shared__ int32_t rows[NP * kList];    // per pair: row positions
  __shared__ int2 ranges[NP * KMAX];      // per pair: the selected blocks' row ranges

  const int lane = threadIdx.x & 63;
  const int sub = lane & (LP - 1);                // which 16 dims / which rows to list
  const int pl = threadIdx.x / LP;                // pair within the workgroup
  const int64_t pair = static_cast<int64_t>(blockIdx.x) * NP + pl;
  const int64_t n_pairs = static_cast<int64_t>(p.n) * p.h_q;
  const bool active = pair < n_pairs;
  const int h = active ? static_cast<int>(pair / p.n) : 0;
  const int t = active ? static_cast<int>(pair % p.n) : 0;      // input token order
  const int g = h / (p.h_q / p.h_kv);
  const int nb = p.counts[SSA_COUNT_NB];
  const float c2 = p.scale * kLog2e;

  const uint16_t* KS = static_cast<const uint16_t*>(p.k_s) + static_cast<int64_t>(g) * p.n * kD + kLaneOff * sub;
  const uint16_t* VS = static_cast<const uint16_t*>(p.v_s) + static_cast<int64_t>(g) * p.n * kD + kLaneOff * sub;
  Row16 q;
  q.load(static_cast<const uint16_t*>(p.q) + (static_cast<int64_t>(t) * p.h_q + h) * kD + kLaneOff * sub, kHalf);
  const int32_t* sel = p.topk_idx + (static_cast<int64_t>(t) * p.h_kv + g) * p.topk;

  // ---------------- the selected blocks' row ranges, all loads in flight at once
  // Lane sub loads blocks sub, sub + LP, ... into LDS.  The list ends at the
  // first block id outside [0, nb) (the padding -1; the check also keeps a
  // corrupt list memory-safe): such a slot gets the range (-1, -1).
  int2* const rng = ranges + pl * KMAX;
#pragma unroll
  for (int i = 0; i < KMAX / LP; ++i) {
    const int r = sub + LP * i;
    const int id = (active && r < p.topk) ? sel[r] : -1;
    const bool ok = id >= 0 && id < nb;
    rng[r] = ok ? make_int2(p.blk_off[id], p.blk_off[id + 1]) : make_int2(-1, -1);
  }
  wave_lds_sync();
  // list: rows of block r start at the rows of blocks 0 .. r - 1; lane sub
  // writes every fourth row of each block
  int total = 0, k_eff = 0;
  for (; k_eff < KMAX; ++k_eff) {
    const int2 ab = rng[k_eff];
    if (ab.x < 0) break;
    for (int i = ab.x + sub; i < ab.y; i += LP) {
      const int idx = total + (i - ab.x);
      if (idx < kList) rows[pl * kList + idx] = i;
    }
    total += ab.y - ab.x;
  }
  wave_lds_sync();

  // ---------------- stream the listed rows
  SelState st;
  st.init();
  const int listed = min(total, kList);
  for (int i0 = 0; i0 < listed; i0 += kStep) {
    Row16 kr[kStep], vr[kStep];
#pragma unroll
    for (int u = 0; u < kStep; ++u) {
      const int64_t row = rows[pl * kList + min(i0 + u, listed - 1)];
      kr[u].load(KS + row * kD, kHalf);
      vr[u].load(VS + row * kD, kHalf);
    }
    float s2[kStep];
#pragma unroll
    for (int u = 0; u < kStep; ++u) {
      const float s = pair_sum<LP>(kr[u].dot(q));
      s2[u] = i0 + u < listed ? s * c2 : -FLT_MAX;
    }
    st.add<kStep>(s2, vr);
  }
  // ---------------- rows past the list (only selections of more than kList rows)
  if (total > kList) {
    int seen = 0;
    for (int r = 0; r < k_eff; ++r) {
      const int2 ab = rng[r];
      for (int i = ab.x; i < ab.y; ++i, ++seen) {
        if (seen < kList) continue;
        Row16 kr, vr[1];
        kr.load(KS + static_cast<int64_t>(i) * kD, kHalf);
        vr[0].load(VS + static_cast<int64_t>(i) * kD, kHalf);
        float s2[1] = {pair_sum<LP>(kr.dot(q)) * c2};
        st.add<1>(s2, vr);
      }
    }
  }

  if (!active) return;
  const int64_t orow = (static_cast<int64_t>(t) * p.h_q + h) * kD + kLaneOff * sub;
  if (p.lse && sub == 0)
    p.lse[static_cast<int64_t>(p.n) * p.h_q + static_cast<int64_t>(t) * p.h_q + h] = (st.m + __log2f(st.l)) * kLn2;
  const uint16_t* gt = static_cast<const uint16_t*>(p.gates) + (static_cast<int64_t>(t) * p.h_q + h) * 3;
  const float f = st.l > 0.f ? bf16_bits_to_f32(gt[1]) / st.l : 0.f;
  const float* acc = p.acc + orow;
  uint16_t res[kDL];
#pragma unroll
  for (int c = 0; c < kDL / 4; ++c) {
    const float4 a = *reinterpret_cast<const float4*>(acc + (c < 2 ? 4 * c : kHalf + 4 * (c - 2)));
    res[4 * c] = f32_to_bf16_bits(fmaf(st.o[4 * c], f, a.x));
    res[4 * c + 1] = f32_to_bf16_bits(fmaf(st.o[4 * c + 1], f, a.y));
    res[4 * c + 2] = f32_to_bf16_bits(fmaf(st.o[4 * c + 2], f, a.z));
    res[4 * c + 3] = f32_to_bf16_bits(fmaf(st.o[4 * c + 3], f, a.w));
  }
  u32x4 w0, w1;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    w0[e] = static_cast<uint32_t>(res[2 * e]) | (static_cast<uint32_t>(res[2 * e + 1]) << 16);
    w1[e] = static_cast<uint32_t>(res[8 + 2 * e]) | (static_cast<uint32_t>(res[8 + 2 * e + 1]) << 16);
  }
  uint16_t* out = static_cast<uint16_t*>(p.out) + orow;
  *reinterpret_cast<u32x4*>(out) = w0;
  *reinterpret_cast<u32x4*>(out + kHalf) = w1;
}

// ---------------------------------------------------------------------------
// Grouped heads (16 query heads per key/value head): the heads of a group
// share one selection, so one wave serves one (token, group) item and runs
// the branch on MFMA, 16 selected rows at a time:
//   S^T = K Q^T        (v_mfma_f32_16x16x32_bf16: rows x heads, k = dims)
//   O^T += V^T P^T     (v_mfma_f32_16x16x16_bf16: dims x heads, k = rows)
// A 16x16 accumulator puts rows 4 (l / 16) + v of column l % 16 in lane l,
// which is also how the second product takes its k = rows operand, so P^T
// feeds it from the lane's own registers, and every lane's softmax state and
// output belong to one head (l % 16).  The rows' values are staged
// transposed in LDS for the V^T operand; each key and value row is loaded
// once per group instead of once per head.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGroupHeads = 16;
constexpr int kVtRow = 16 + 4;   // LDS row of the transposed value chunk (bf16), padded against bank conflicts

template <int KMAX, int D>
__global__ void __launch_bounds__(256)
sel_group_kernel(FwdParams p) {
  constexpr int KQ = D / 32;   // 16x16x32 steps over the dims
  constexpr int NB = D / 16;   // 16-dim blocks of O^T
  __shared__ int off_s[4][KMAX + 1];
  __shared__ int start_s[4][KMAX];
  __shared__ __align__(16) uint16_t vt_s[4][D * kVtRow];

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int64_t n_items = static_cast<int64_t>(p.n) * p.h_kv;
  // items group-major in sorted token order: neighbouring waves select
  // neighbouring blocks of the same group
  const int64_t item = static_cast<int64_t>(blockIdx.x) * 4 + wv;
  if (item >= n_items) return;   // uniform over the wave; no barrier follows
  const int g = static_cast<int>(item / p.n);
  const int t = p.perm[static_cast<int>(item % p.n)];
  const int hq = g * kGroupHeads + col;
  const int nb = p.counts[SSA_COUNT_NB];
  const float c2 = p.scale * kLog2e;

  // selected blocks: lane i < KMAX takes entry i; the list ends at the first
  // id outside [0, nb)
  const int32_t* sel = p.topk_idx + (static_cast<int64_t>(t) * p.h_kv + g) * p.topk;
  int id = lane < KMAX && lane < p.topk ? sel[lane] : -1;
  const uint64_t bad = __ballot(!(id >= 0 && id < nb));   // lanes >= KMAX always count as ends
  const int k_eff = static_cast<int>(__builtin_ctzll(bad));
  int a = 0, size = 0;
  if (lane < k_eff) {
    a = p.blk_off[id];
    size = p.blk_off[id + 1] - a;
  }
  int incl = size;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  const int total = __shfl(incl, 63);
  if (lane < k_eff) {
    off_s[wv][lane + 1] = incl;
    start_s[wv][lane] = a;
  }
  if (lane == 0) off_s[wv][0] = 0;
  wave_lds_sync();

  // Q^T operands: head col, dims 8 grp .. 8 grp + 7 of each 32-dim step
  const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + (static_cast<int64_t>(t) * p.h_q + hq) * D;
  bf16x8 qb[KQ];
#pragma unroll
  for (int kq = 0; kq < KQ; ++kq) qb[kq] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + 32 * kq + 8 * grp));

  const uint16_t* KS = static_cast<const uint16_t*>(p.k_s) + static_cast<int64_t>(g) * p.n * D;
  const uint16_t* VS = static_cast<const uint16_t*>(p.v_s) + static_cast<int64_t>(g) * p.n * D;
  uint16_t* vt = vt_s[wv];
  float m = -FLT_MAX, l = 0.f;
  f32x4 o[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) o[b] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int c0 = 0; c0 < total; c0 += 16) {
    // row of list position c0 + col (this lane's K row and V row)
    const int pos = c0 + col;
    const bool ok = pos < total;
    u32x4 kr[KQ], vr[KQ];
    if (ok) {
      int lo = 0, hi = k_eff - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off_s[wv][mid] <= pos) lo = mid; else hi = mid - 1;
      }
      const int64_t row = start_s[wv][lo] + (pos - off_s[wv][lo]);
#pragma unroll
      for (int kq = 0; kq < KQ; ++kq) {
        kr[kq] = *reinterpret_cast<const u32x4*>(KS + row * D + 32 * kq + 8 * grp);
        vr[kq] = *reinterpret_cast<const u32x4*>(VS + row * D + 32 * kq + 8 * grp);
      }
    } else {
#pragma unroll
      for (int kq = 0; kq < KQ; ++kq) kr[kq] = vr[kq] = u32x4{0u, 0u, 0u, 0u};
    }
    // V^T chunk: element (dim, row col)
    wave_lds_sync();   // the previous chunk's V^T reads are done
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = 32 * kq + 8 * grp + 2 * e;
        vt[d * kVtRow + col] = static_cast<uint16_t>(vr[kq][e] & 0xFFFFu);
        vt[(d + 1) * kVtRow + col] = static_cast<uint16_t>(vr[kq][e] >> 16);
      }
    // S^T: rows 4 grp + v, head col
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[kq]), qb[kq], s, 0, 0, 0);
    float x[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) x[v] = c0 + 4 * grp + v < total ? s[v] * c2 : -INFINITY;
    // the head's chunk maximum over the four lane groups
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float corr = __builtin_amdgcn_exp2f(m - m_new);
    m = m_new;
    // P rounded to bf16; the row sum adds the rounded values, so the weights
    // of O and of the sum are the same numbers
    bf16x4 pb;
    float ps = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const __bf16 pv = static_cast<__bf16>(__builtin_amdgcn_exp2f(x[v] - m));
      pb[v] = pv;
      ps += static_cast<float>(pv);
    }
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    l = l * corr + ps;
    wave_lds_sync();   // V^T stored
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const bf16x4 va = __builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2*>(vt + (16 * b + col) * kVtRow + 4 * grp));
      o[b] *= corr;
      o[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, o[b], 0, 0, 0);
    }
  }

  // out = acc + G1 * o_sel / l for dims 16 b + 4 grp + v of head col
  const int64_t orow = (static_cast<int64_t>(t) * p.h_q + hq) * D;
  if (p.lse && grp == 0)
    p.lse[static_cast<int64_t>(p.n) * p.h_q + static_cast<int64_t>(t) * p.h_q + hq] =
        l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
  const uint16_t* gt = static_cast<const uint16_t*>(p.gates) + (static_cast<int64_t>(t) * p.h_q + hq) * 3;
  const float f = l > 0.f ? bf16_bits_to_f32(gt[1]) / l : 0.f;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int d = 16 * b + 4 * grp;
    const float4 av = *reinterpret_cast<const float4*>(p.acc + orow + d);
    uint2 w;
    w.x = static_cast<uint32_t>(f32_to_bf16_bits(fmaf(o[b][0], f, av.x))) |
          (static_cast<uint32_t>(f32_to_bf16_bits(fmaf(o[b][1], f, av.y))) << 16);
    w.y = static_cast<uint32_t>(f32_to_bf16_bits(fmaf(o[b][2], f, av.z))) |
          (static_cast<uint32_t>(f32_to_bf16_bits(fmaf(o[b][3], f, av.w))) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + orow + d) = w;
  }
}

}  // namespace

hipError_t launch_sel_combine(const FwdParams& p, ssa_dtype /*dtype*/, hipStream_t stream) {
  if (p.h_q == kGroupHeads * p.h_kv) {
    const int grid = static_cast<int>((static_cast<int64_t>(p.n) * p.h_kv + 3) / 4);
    if (p.d == 32) {
      if (p.topk <= 16) sel_group_kernel<16, 32><<<grid, 256, 0, stream>>>(p);
      else sel_group_kernel<32, 32><<<grid, 256, 0, stream>>>(p);
    } else {
      if (p.topk <= 16) sel_group_kernel<16, 64><<<grid, 256, 0, stream>>>(p);
      else sel_group_kernel<32, 64><<<grid, 256, 0, stream>>>(p);
    }
    return hipGetLastError();
  }
  const int64_t pairs = static_cast<int64_t>(p.n) * p.h_q;
  const int np = 256 / (p.d / kDL);
  const int grid = static_cast<int>((pairs + np - 1) / np);
  if (p.d == 32) {
    if (p.topk <= 16) sel_combine_kernel<16, 32><<<grid, 256, 0, stream>>>(p);
    else sel_combine_kernel<32, 32><<<grid, 256, 0, stream>>>(p);
  } else {
    if (p.topk <= 16) sel_combine_kernel<16, 64><<<grid, 256, 0, stream>>>(p);
    else sel_combine_kernel<32, 64><<<grid, 256, 0, stream>>>(p);
  }
  return hipGetLastError();
}

}  // namespace ssa
