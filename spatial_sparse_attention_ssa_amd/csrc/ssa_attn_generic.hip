// General SSA forward: one wave per (sorted token, key/value group).
//
// This kernel covers every supported layout (float32 or bfloat16 storage,
// D in {32, 64}, any group size, top-k <= 32) with plain VALU arithmetic.
// It computes, for each query head h of the group (Direct3D-S2 page,
// "Method", second paragraph):
//   o_cmp: softmax attention over the mean-pooled blocks of the sequence;
//   o_sel: softmax attention over every token of the top-k blocks, ranked by
//          the compressed-branch probability summed over the group's heads
//          (LSRM article, "Stage 1": grouped query heads share key/value
//          heads); ties go to the lower block id;
//   o_win: softmax attention over every token of the token's m_win^3 window;
//   out = G0 o_cmp + G1 o_sel + G2 o_win, rounded once to the storage type.
//
// Lanes stride over keys; each lane keeps its own running maximum, sum and
// D-vector, and the wave merges them with a butterfly reduce-scatter that
// leaves component d in lane d (mod D).  For the selection each lane keeps
// its own sorted top-KMAX list; the wave then pops the k best heads in turn.
#include <float.h>

#include "ssa_internal.h"

namespace ssa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <int D>
__device__ __forceinline__ void load_row(const float* __restrict__ p, float (&x)[D]) {
#pragma unroll
  for (int c = 0; c < D / 4; ++c) {
    const float4 u = reinterpret_cast<const float4*>(p)[c];
    x[4 * c] = u.x; x[4 * c + 1] = u.y; x[4 * c + 2] = u.z; x[4 * c + 3] = u.w;
  }
}

template <int D>
__device__ __forceinline__ void load_row(const uint16_t* __restrict__ p, float (&x)[D]) {
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    const uint4 u = reinterpret_cast<const uint4*>(p)[c];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[8 * c + 2 * e] = __uint_as_float(w[e] << 16);
      x[8 * c + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  }
}

template <int D>
__device__ __forceinline__ float dot(const float (&a)[D], const float (&b)[D]) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < D; ++e) s = fmaf(a[e], b[e], s);
  return s;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// Sum v[] over the 64 lanes; afterwards lane l holds the total of component
// l mod D (recursive halving; D in {32, 64}).
template <int D>
__device__ __forceinline__ float wave_reduce_scatter(float (&v)[D]) {
  const int lane = threadIdx.x & 63;
  if (D == 32) {
#pragma unroll
    for (int e = 0; e < D; ++e) v[e] += __shfl_xor(v[e], 32);
  }
#pragma unroll
  for (int h = D / 2; h >= 1; h >>= 1) {
    const bool upper = lane & h;
#pragma unroll
    for (int e = 0; e < h; ++e) {
      const float send = upper ? v[e] : v[e + h];
      const float keep = upper ? v[e + h] : v[e];
      v[e] = keep + __shfl_xor(send, h);
    }
  }
  return v[0];
}

// Per-lane online softmax state over a strided key set.
template <int D>
struct Acc {
  float m, l, o[D];
  __device__ __forceinline__ void init() {
    m = -FLT_MAX;
    l = 0.f;
#pragma unroll
    for (int e = 0; e < D; ++e) o[e] = 0.f;
  }
  // s2: logit in log2 units
  __device__ __forceinline__ void add(float s2, const float (&vrow)[D]) {
    if (s2 > m) {
      const float c = exp2f(m - s2);
      l *= c;
#pragma unroll
      for (int e = 0; e < D; ++e) o[e] *= c;
      m = s2;
    }
    const float p = exp2f(s2 - m);
    l += p;
#pragma unroll
    for (int e = 0; e < D; ++e) o[e] = fmaf(p, vrow[e], o[e]);
  }
  // merged result for component (lane mod D); *lse2 receives the log2 of
  // the softmax denominator of the log2-unit logits
  __device__ __forceinline__ float finish(float* lse2) {
    const float mm = wave_max(m);
    const float f = (l > 0.f) ? exp2f(m - mm) : 0.f;
    l *= f;
#pragma unroll
    for (int e = 0; e < D; ++e) o[e] *= f;
    const float ll = wave_sum(l);
    *lse2 = mm + log2f(ll);
    return wave_reduce_scatter<D>(o) / ll;
  }
};

template <typename T, int D, int KMAX>
__global__ void __launch_bounds__(256)
generic_fwd(FwdParams p) {
  extern __shared__ float smem[];
  const int lane = threadIdx.x & 63;
  const int ws = threadIdx.x >> 6;
  const int G = p.h_q / p.h_kv;
  // per-wave LDS: q of every head of the group [G][D], m/l per head, selection
  float* q_lds = smem + ws * (G * D + 2 * G + 2 * KMAX + 2);
  float* m_lds = q_lds + G * D;
  float* l_lds = m_lds + G;
  int* sel_lds = reinterpret_cast<int*>(l_lds + G);
  int* pre_lds = sel_lds + KMAX;  // KMAX + 2 entries

  const int64_t wid = static_cast<int64_t>(blockIdx.x) * 4 + ws;
  if (wid >= static_cast<int64_t>(p.n) * p.h_kv) return;
  const int i = static_cast<int>(wid / p.h_kv);
  const int g = static_cast<int>(wid % p.h_kv);
  const int t = p.perm[i];
  const int nw = p.counts[SSA_COUNT_NW];

  // window w containing sorted position i, and its sequence b
  int lo = 0, hi = nw - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.win_off[mid] <= i) lo = mid; else hi = mid - 1;
  }
  const int w = lo;
  lo = 0; hi = p.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.seq_win_off[mid] <= w) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const int j0 = p.seq_blk_off[b], j1 = p.seq_blk_off[b + 1];
  const int nbs = j1 - j0;

  const T* Q = static_cast<const T*>(p.q);
  const T* K = static_cast<const T*>(p.k);
  const T* V = static_cast<const T*>(p.v);
  const T* KB = static_cast<const T*>(p.kbar) + static_cast<int64_t>(g) * p.nb_cap * D;
  const T* VB = static_cast<const T*>(p.vbar) + static_cast<int64_t>(g) * p.nb_cap * D;
  const float c2 = p.scale * kLog2e;  // logits in log2 units

  // stage the group's queries in LDS
  for (int e = lane; e < G * D; e += 64) {
    const int hh = e / D, dd = e % D;
    q_lds[e] = Elt<T>::load(Q + (static_cast<int64_t>(t) * p.h_q + g * G + hh) * D + dd);
  }
  wave_lds_sync();

  float q[D], row[D], row2[D];

  // ---- per-head softmax statistics of the compressed branch (needed to sum
  //      probabilities over the group's heads)
  if (G > 1) {
    for (int hh = 0; hh < G; ++hh) {
#pragma unroll
      for (int e = 0; e < D; ++e) q[e] = q_lds[hh * D + e];
      float m = -FLT_MAX, l = 0.f;
      for (int j = j0 + lane; j < j1; j += 64) {
        load_row<D>(KB + static_cast<int64_t>(j) * D, row);
        const float s2 = c2 * dot<D>(q, row);
        if (s2 > m) { l *= exp2f(m - s2); m = s2; }
        l += exp2f(s2 - m);
      }
      const float mm = wave_max(m);
      l = (l > 0.f) ? l * exp2f(m - mm) : 0.f;
      const float ll = wave_sum(l);
      if (lane == 0) { m_lds[hh] = mm; l_lds[hh] = ll; }
    }
    wave_lds_sync();
  }

  // ---- selection score per block and a per-lane sorted top-KMAX list
  float lv[KMAX];
  int li[KMAX];
#pragma unroll
  for (int e = 0; e < KMAX; ++e) { lv[e] = -FLT_MAX; li[e] = 0x7FFFFFFF; }
  if (G == 1) {
#pragma unroll
    for (int e = 0; e < D; ++e) q[e] = q_lds[e];
  }
  for (int j = j0 + lane; j < j1; j += 64) {
    load_row<D>(KB + static_cast<int64_t>(j) * D, row);
    float score;
    if (G == 1) {
      score = dot<D>(q, row);  // one head: probability order == logit order
    } else {
      score = 0.f;
      for (int hh = 0; hh < G; ++hh) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < D; ++e) acc = fmaf(q_lds[hh * D + e], row[e], acc);
        score += exp2f(c2 * acc - m_lds[hh]) / l_lds[hh];
      }
    }
    if (score > lv[KMAX - 1]) {
      bool placed = false;
#pragma unroll
      for (int e = KMAX - 1; e >= 1; --e) {
        if (!placed) {
          if (score > lv[e - 1]) {
            lv[e] = lv[e - 1];
            li[e] = li[e - 1];
          } else {
            lv[e] = score;
            li[e] = j;
            placed = true;
          }
        }
      }
      if (!placed) { lv[0] = score; li[0] = j; }
    }
  }
  const int k_eff = nbs < p.topk ? nbs : p.topk;
  for (int r = 0; r < k_eff; ++r) {
    float bv = lv[0];
    int bi = li[0];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    if (li[0] == bi) {  // the winning lane pops its head
#pragma unroll
      for (int e = 0; e < KMAX - 1; ++e) { lv[e] = lv[e + 1]; li[e] = li[e + 1]; }
      lv[KMAX - 1] = -FLT_MAX;
      li[KMAX - 1] = 0x7FFFFFFF;
    }
    if (lane == 0) sel_lds[r] = bi;
  }
  wave_lds_sync();
  if (lane < p.topk) {
    p.topk_idx[(static_cast<int64_t>(t) * p.h_kv + g) * p.topk + lane] = lane < k_eff ? sel_lds[lane] : -1;
  }
  if (lane == 0) {
    int run = 0;
    for (int r = 0; r < k_eff; ++r) {
      pre_lds[r] = run;
      run += p.blk_off[sel_lds[r] + 1] - p.blk_off[sel_lds[r]];
    }
    pre_lds[k_eff] = run;
  }
  wave_lds_sync();
  const int n_sel = pre_lds[k_eff];
  const int wa = p.win_off[w], wb = p.win_off[w + 1];

  // ---- the three branches and the gated sum, head by head
  for (int hh = 0; hh < G; ++hh) {
    const int h = g * G + hh;
#pragma unroll
    for (int e = 0; e < D; ++e) q[e] = q_lds[hh * D + e];
    Acc<D> acc;

    acc.init();
    for (int j = j0 + lane; j < j1; j += 64) {
      load_row<D>(KB + static_cast<int64_t>(j) * D, row);
      load_row<D>(VB + static_cast<int64_t>(j) * D, row2);
      acc.add(c2 * dot<D>(q, row), row2);
    }
    float lse_c, lse_s, lse_w;
    const float o_cmp = acc.finish(&lse_c);

    acc.init();
    for (int f = lane; f < n_sel; f += 64) {
      int r = 0;
      while (r + 1 < k_eff && pre_lds[r + 1] <= f) ++r;
      const int pos = p.blk_off[sel_lds[r]] + (f - pre_lds[r]);
      const int64_t tok = p.perm[pos];
      load_row<D>(K + (tok * p.h_kv + g) * D, row);
      load_row<D>(V + (tok * p.h_kv + g) * D, row2);
      acc.add(c2 * dot<D>(q, row), row2);
    }
    const float o_sel = acc.finish(&lse_s);

    acc.init();
    for (int pos = wa + lane; pos < wb; pos += 64) {
      const int64_t tok = p.perm[pos];
      load_row<D>(K + (tok * p.h_kv + g) * D, row);
      load_row<D>(V + (tok * p.h_kv + g) * D, row2);
      acc.add(c2 * dot<D>(q, row), row2);
    }
    const float o_win = acc.finish(&lse_w);

    if (lane < D) {
      const T* gt = static_cast<const T*>(p.gates) + (static_cast<int64_t>(t) * p.h_q + h) * 3;
      const float o = Elt<T>::load(gt) * o_cmp + Elt<T>::load(gt + 1) * o_sel +
                      Elt<T>::load(gt + 2) * o_win;
      Elt<T>::store(static_cast<T*>(p.out) + (static_cast<int64_t>(t) * p.h_q + h) * D + lane, o);
      if (p.lse && lane == 0) {
        const int64_t nrow = static_cast<int64_t>(p.n) * p.h_q;
        const int64_t row = static_cast<int64_t>(t) * p.h_q + h;
        p.lse[row] = lse_c * kLn2;
        p.lse[nrow + row] = lse_s * kLn2;
        p.lse[2 * nrow + row] = lse_w * kLn2;
      }
    }
  }
}

template <typename T, int D, int KMAX>
hipError_t launch_generic_t(const FwdParams& p, hipStream_t stream) {
  const int G = p.h_q / p.h_kv;
  const size_t smem = 4 * sizeof(float) * (G * D + 2 * G + 2 * KMAX + 2);
  const int64_t waves = static_cast<int64_t>(p.n) * p.h_kv;
  const int grid = static_cast<int>((waves + 3) / 4);
  generic_fwd<T, D, KMAX><<<grid, 256, smem, stream>>>(p);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_generic_d(const FwdParams& p, hipStream_t stream) {
  if (p.d == 32) {
    return p.topk <= 16 ? launch_generic_t<T, 32, 16>(p, stream) : launch_generic_t<T, 32, 32>(p, stream);
  }
  return p.topk <= 16 ? launch_generic_t<T, 64, 16>(p, stream) : launch_generic_t<T, 64, 32>(p, stream);
}

}  // namespace

hipError_t launch_generic(const FwdParams& p, ssa_dtype dtype, hipStream_t stream) {
  if (p.n == 0) return hipSuccess;
  return dtype == SSA_BF16 ? launch_generic_d<uint16_t>(p, stream) : launch_generic_d<float>(p, stream);
}

}  // namespace ssa
