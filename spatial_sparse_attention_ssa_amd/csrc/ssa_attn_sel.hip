// Selected-block attention and the gated sum (bf16, D = 32 or 64; query head
// h reads key/value head g = h / (h_q / h_kv) and the selection of group g).
//
// Direct3D-S2 page, "Method": all tokens of the top-k selected blocks take
// part in a second attention; the three branch outputs are summed with the
// predicted gates.  The window and compressed branches have already written
// G2 * o_win + G0 * o_cmp to the float32 accumulator; this kernel adds
// G1 * o_sel, rounds once to bfloat16 and writes the output row.
//
// D / 16 lanes serve one (token, head) pair, each owning 16 dims; a wave
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

#include "ssa_internal.h"

namespace ssa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

// 16 bf16 values of a row, packed
struct Row16 {
  u32x4 a, b;
  __device__ __forceinline__ void load(const uint16_t* p) {
    a = *reinterpret_cast<const u32x4*>(p);
    b = *reinterpret_cast<const u32x4*>(p + 8);
  }
  __device__ __forceinline__ float dot(const float (&q)[kDL]) const {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s0 = fmaf(q[2 * e], bf_lo(a[e]), s0);
      s1 = fmaf(q[2 * e + 1], bf_hi(a[e]), s1);
      s0 = fmaf(q[8 + 2 * e], bf_lo(b[e]), s0);
      s1 = fmaf(q[8 + 2 * e + 1], bf_hi(b[e]), s1);
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
    for (int u = 0; u < U; ++u) mx = fmaxf(mx, s2[u]);
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

// sum over the LP lanes of a pair
template <int LP>
__device__ __forceinline__ float pair_sum(float s) {
#pragma unroll
  for (int o = 1; o < LP; o <<= 1) s += __shfl_xor(s, o);
  return s;
}

template <int KMAX, int D>
__global__ void __launch_bounds__(256)
sel_combine_kernel(FwdParams p) {
  constexpr int kD = D;
  constexpr int LP = D / kDL;             // lanes per pair
  constexpr int NP = 256 / LP;            // pairs per workgroup
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

  const uint16_t* KS = static_cast<const uint16_t*>(p.k_s) + static_cast<int64_t>(g) * p.n * kD + kDL * sub;
  const uint16_t* VS = static_cast<const uint16_t*>(p.v_s) + static_cast<int64_t>(g) * p.n * kD + kDL * sub;
  float q[kDL];
  load16(static_cast<const uint16_t*>(p.q) + (static_cast<int64_t>(t) * p.h_q + h) * kD + kDL * sub, q);
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
      kr[u].load(KS + row * kD);
      vr[u].load(VS + row * kD);
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
        kr.load(KS + static_cast<int64_t>(i) * kD);
        vr[0].load(VS + static_cast<int64_t>(i) * kD);
        float s2[1] = {pair_sum<LP>(kr.dot(q)) * c2};
        st.add<1>(s2, vr);
      }
    }
  }

  if (!active) return;
  const int64_t orow = (static_cast<int64_t>(t) * p.h_q + h) * kD + kDL * sub;
  if (p.lse && sub == 0)
    p.lse[static_cast<int64_t>(p.n) * p.h_q + static_cast<int64_t>(t) * p.h_q + h] = (st.m + __log2f(st.l)) * kLn2;
  const uint16_t* gt = static_cast<const uint16_t*>(p.gates) + (static_cast<int64_t>(t) * p.h_q + h) * 3;
  const float f = st.l > 0.f ? bf16_bits_to_f32(gt[1]) / st.l : 0.f;
  const float* acc = p.acc + orow;
  uint16_t res[kDL];
#pragma unroll
  for (int c = 0; c < kDL / 4; ++c) {
    const float4 a = *reinterpret_cast<const float4*>(acc + 4 * c);
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
  *reinterpret_cast<u32x4*>(out + 8) = w1;
}

}  // namespace

hipError_t launch_sel_combine(const FwdParams& p, ssa_dtype /*dtype*/, hipStream_t stream) {
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
