// SSA backward pass: gradients of L = sum(dout * out) with respect to q, k,
// v and the gates.
//
// Direct3D-S2 page, "Method": out = G0 o_cmp + G1 o_sel + G2 o_win, each o_x
// a softmax attention of the query over one key set (the sequence's pooled
// blocks, the tokens of the top-k blocks, the tokens of the query's window).
// For one branch with keys k_j, values v_j and probabilities P_j (recomputed
// from the log-sum-exp the forward saved):
//   dP_j = dout . v_j,   Delta = sum_j P_j dP_j  (= dout . o_x),
//   dS_j = P_j (dP_j - Delta)            (the logit gradient, per unit gate),
//   dq  += G_x scale sum_j dS_j k_j,  dk_j += G_x scale dS_j q,
//   dv_j += G_x P_j dout,             dG_x = Delta.
// The query-major kernels take Delta from the same float32 P they use, so
// that sum_j dS_j vanishes to float32 rounding: they accumulate
// A = sum_j P_j dP_j k_j and B = sum_j P_j k_j beside Delta and form
// A - Delta B at the end; the key-major kernels then read Delta.
// The top-k choice is held fixed (it is piecewise constant in q and k).  The
// compressed branch's key / value gradients land on the pooled rows; the
// pooling is a mean, so each token of block j receives 1 / n_j of its row's
// gradient (the one rounding of the pooled rows counts as the identity).
//
// These kernels work for both storage types and any group size with plain
// VALU arithmetic: D / 16 lanes share one row (16 dims each) and combine
// their partial dot products with lane shuffles.  Stages, in launch order:
//   sel_keys + sort      for every (group, block), the tokens whose selection
//                        holds it (an inverted top-k list): a stable radix sort
//                        of the top-k entries by (group, block), so each list
//                        lists its tokens in increasing order
//   cmp_dq_kernel        compressed branch: Delta, dgates, dq (first writer of dq_acc)
//   cmp_dkv_kernel       pooled-row gradients, block-major
//   win_dq_kernel        window branch: Delta, dgates, dq (adds)
//   win_dkv_kernel       dk / dv of each window's tokens (first writer of dk_acc / dv_acc)
//   sel_dq_kernel        selected branch: Delta, dgates, and dq in the input dtype
//   sel_dkv_kernel       dk / dv of each block's tokens over the queries that
//                        chose the block (adds)
//   bwd_finalize_kernel  dk, dv in the input dtype and input token order
#include <float.h>

#include <algorithm>

#include "ssa_internal.h"

namespace ssa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kDL = 16;  // dims per lane

// 16 consecutive elements of a row, widened to float
__device__ __forceinline__ void load16(const float* p, float (&x)[kDL]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float4 u = reinterpret_cast<const float4*>(p)[c];
    x[4 * c] = u.x; x[4 * c + 1] = u.y; x[4 * c + 2] = u.z; x[4 * c + 3] = u.w;
  }
}
__device__ __forceinline__ void load16(const uint16_t* p, float (&x)[kDL]) {
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const uint4 u = reinterpret_cast<const uint4*>(p)[c];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[8 * c + 2 * e] = __uint_as_float(w[e] << 16);
      x[8 * c + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  }
}
__device__ __forceinline__ void store16(float* p, const float (&x)[kDL]) {
#pragma unroll
  for (int c = 0; c < 4; ++c)
    reinterpret_cast<float4*>(p)[c] = make_float4(x[4 * c], x[4 * c + 1], x[4 * c + 2], x[4 * c + 3]);
}
__device__ __forceinline__ void store16(uint16_t* p, const float (&x)[kDL]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) store_bf16x4(p + 4 * c, x[4 * c], x[4 * c + 1], x[4 * c + 2], x[4 * c + 3]);
}

__device__ __forceinline__ float dot16(const float (&a)[kDL], const float (&b)[kDL]) {
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int e = 0; e < kDL; e += 2) {
    s0 = fmaf(a[e], b[e], s0);
    s1 = fmaf(a[e + 1], b[e + 1], s1);
  }
  return s0 + s1;
}

// sum over the LP lanes of a row (the row's lanes share their control
// flow): DPP quad permutations for LP 2 and 4, no LDS round trip
template <int LP>
__device__ __forceinline__ float row_sum(float s) {
  if (LP == 2 || LP == 4) {
    s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0xB1, 0xF, 0xF, false));  // [1,0,3,2]
    if (LP == 4) s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x4E, 0xF, 0xF, false));
    return s;
  }
#pragma unroll
  for (int o = 1; o < LP; o <<= 1) s += __shfl_xor(s, o);
  return s;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// 16 packed bf16 values (two 16-byte words) times 16 others: v_dot2_f32_bf16
// (exact products, float32 sums) on the raw words
__device__ __forceinline__ float dot16_bf16(const uint4 (&a)[2], const uint4 (&b)[2]) {
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const uint32_t x[4] = {a[c].x, a[c].y, a[c].z, a[c].w};
    const uint32_t y[4] = {b[c].x, b[c].y, b[c].z, b[c].w};
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x[e]), __builtin_bit_cast(bf16x2, y[e]), s0, false);
      s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x[e + 1]), __builtin_bit_cast(bf16x2, y[e + 1]), s1,
                                           false);
    }
  }
  return s0 + s1;
}
__device__ __forceinline__ void load_raw16(const uint16_t* p, uint4 (&w)[2]) {
  w[0] = reinterpret_cast<const uint4*>(p)[0];
  w[1] = reinterpret_cast<const uint4*>(p)[1];
}
__device__ __forceinline__ void widen16(const uint4 (&w)[2], float (&x)[kDL]) {
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const uint32_t u[4] = {w[c].x, w[c].y, w[c].z, w[c].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[8 * c + 2 * e] = __uint_as_float(u[e] << 16);
      x[8 * c + 2 * e + 1] = __uint_as_float(u[e] & 0xFFFF0000u);
    }
  }
}

__device__ __forceinline__ int seq_of_window(const int32_t* seq_win_off, int batch, int w) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (seq_win_off[mid] <= w) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ int window_of_pos(const int32_t* win_off, int nw, int i) {
  int lo = 0, hi = nw - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (win_off[mid] <= i) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Delta of branch x for one (token, head) row; also the gate's gradient.
template <typename T>
__device__ __forceinline__ void put_delta(const BwdParams& p, int x, int64_t qrow, float dl) {
  p.delta[x * static_cast<int64_t>(p.f.n) * p.f.h_q + qrow] = dl;
  if (p.dgates) Elt<T>::store(static_cast<T*>(p.dgates) + qrow * 3 + x, dl);
}

// ------------------------------------------------------------ inverted top-k lists

// key of entry e = (token * h_kv + group) * topk + rank: group * nb_cap +
// block, or h_kv * nb_cap (past every list) for a padding slot
__global__ void __launch_bounds__(256)
sel_keys_kernel(BwdParams p) {
  const int64_t m = static_cast<int64_t>(p.f.n) * p.f.h_kv * p.f.topk;
  const int nb = p.f.counts[SSA_COUNT_NB];
  const uint32_t none = static_cast<uint32_t>(p.f.h_kv) * static_cast<uint32_t>(p.f.nb_cap);
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < m;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int j = p.f.topk_idx[e];
    const int64_t tg = e / p.f.topk;
    const uint32_t g = static_cast<uint32_t>(tg % p.f.h_kv);
    p.sel_keys[e] = (j >= 0 && j < nb) ? g * static_cast<uint32_t>(p.f.nb_cap) + static_cast<uint32_t>(j) : none;
    p.sel_vals[e] = static_cast<int32_t>(tg / p.f.h_kv);
  }
}

// start of every list: the first sorted key >= the list's key
__global__ void __launch_bounds__(256)
sel_offsets_kernel(BwdParams p) {
  const int64_t m = static_cast<int64_t>(p.f.n) * p.f.h_kv * p.f.topk;
  const int64_t nl = static_cast<int64_t>(p.f.h_kv) * p.f.nb_cap;
  for (int64_t key = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; key <= nl;
       key += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    int64_t lo = 0, hi = m;
    while (lo < hi) {
      const int64_t mid = (lo + hi) >> 1;
      if (static_cast<int64_t>(p.sel_sorted_keys[mid]) < key) lo = mid + 1; else hi = mid;
    }
    p.sel_off[key] = static_cast<int32_t>(lo);
  }
}

// ------------------------------------------------------------ compressed branch

// dq of the compressed branch.  LP = D / 16 lanes per (sorted position,
// query head) row, rows head-major so that a workgroup reads one head's
// pooled rows.
template <typename T, int D>
__global__ void __launch_bounds__(256)
cmp_dq_kernel(BwdParams p) {
  constexpr int LP = D / kDL;
  constexpr int NR = 256 / LP;
  const FwdParams& f = p.f;
  const int sub = threadIdx.x % LP;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * NR + threadIdx.x / LP;
  const int64_t nrow = static_cast<int64_t>(f.n) * f.h_q;
  if (row >= nrow) return;
  const int h = static_cast<int>(row / f.n);
  const int i = static_cast<int>(row % f.n);
  const int g = h / (f.h_q / f.h_kv);
  const int t = f.perm[i];
  const int w = window_of_pos(f.win_off, f.counts[SSA_COUNT_NW], i);
  const int b = seq_of_window(f.seq_win_off, f.batch, w);
  const int j0 = f.seq_blk_off[b], j1 = f.seq_blk_off[b + 1];
  const int64_t qrow = static_cast<int64_t>(t) * f.h_q + h;
  const float c2 = f.scale * kLog2e;
  const float lse2 = p.lse[qrow] * kLog2e;

  float q[kDL], dO[kDL], aa[kDL], ab[kDL];
  load16(static_cast<const T*>(f.q) + qrow * D + kDL * sub, q);
  load16(static_cast<const T*>(p.dout) + qrow * D + kDL * sub, dO);
#pragma unroll
  for (int e = 0; e < kDL; ++e) aa[e] = ab[e] = 0.f;
  float dl = 0.f;
  const T* KB = static_cast<const T*>(f.kbar) + static_cast<int64_t>(g) * f.nb_cap * D + kDL * sub;
  const T* VB = static_cast<const T*>(f.vbar) + static_cast<int64_t>(g) * f.nb_cap * D + kDL * sub;
  for (int j = j0; j < j1; ++j) {
    float kr[kDL], vr[kDL];
    load16(KB + static_cast<int64_t>(j) * D, kr);
    load16(VB + static_cast<int64_t>(j) * D, vr);
    const float s = row_sum<LP>(dot16(q, kr));
    const float dp = row_sum<LP>(dot16(dO, vr));
    const float pr = exp2f(fmaf(s, c2, -lse2));
    const float pd = pr * dp;
    dl += pd;
#pragma unroll
    for (int e = 0; e < kDL; ++e) {
      aa[e] = fmaf(pd, kr[e], aa[e]);
      ab[e] = fmaf(pr, kr[e], ab[e]);
    }
  }
  const float gs = Elt<T>::load(static_cast<const T*>(f.gates) + qrow * 3) * f.scale;
#pragma unroll
  for (int e = 0; e < kDL; ++e) aa[e] = gs * fmaf(-dl, ab[e], aa[e]);
  store16(p.dq_acc + qrow * D + kDL * sub, aa);
  if (sub == 0) put_delta<T>(p, 0, qrow, dl);
}

// Gradients of the pooled rows: LP lanes per (group, block) row; each row
// walks every (query, head of the group) of its sequence.
template <typename T, int D>
__global__ void __launch_bounds__(256)
cmp_dkv_kernel(BwdParams p) {
  constexpr int LP = D / kDL;
  constexpr int NR = 256 / LP;
  const FwdParams& f = p.f;
  const int sub = threadIdx.x % LP;
  const int nb = f.counts[SSA_COUNT_NB];
  const int64_t row = static_cast<int64_t>(blockIdx.x) * NR + threadIdx.x / LP;
  if (row >= static_cast<int64_t>(f.h_kv) * nb) return;
  const int g = static_cast<int>(row / nb);
  const int j = static_cast<int>(row % nb);
  const int G = f.h_q / f.h_kv;
  // the block's sequence: the first window of the block's tokens
  const int w = window_of_pos(f.win_off, f.counts[SSA_COUNT_NW], f.blk_off[j]);
  const int b = seq_of_window(f.seq_win_off, f.batch, w);
  const int s0 = f.win_off[f.seq_win_off[b]], s1 = f.win_off[f.seq_win_off[b + 1]];
  const float c2 = f.scale * kLog2e;

  float kr[kDL], vr[kDL], ak[kDL], av[kDL];
  load16(static_cast<const T*>(f.kbar) + (static_cast<int64_t>(g) * f.nb_cap + j) * D + kDL * sub, kr);
  load16(static_cast<const T*>(f.vbar) + (static_cast<int64_t>(g) * f.nb_cap + j) * D + kDL * sub, vr);
#pragma unroll
  for (int e = 0; e < kDL; ++e) ak[e] = av[e] = 0.f;
  for (int i = s0; i < s1; ++i) {
    const int t = f.perm[i];
    for (int hh = 0; hh < G; ++hh) {
      const int64_t qrow = static_cast<int64_t>(t) * f.h_q + g * G + hh;
      float q[kDL], dO[kDL];
      load16(static_cast<const T*>(f.q) + qrow * D + kDL * sub, q);
      load16(static_cast<const T*>(p.dout) + qrow * D + kDL * sub, dO);
      const float s = row_sum<LP>(dot16(q, kr));
      const float dp = row_sum<LP>(dot16(dO, vr));
      const float g0 = Elt<T>::load(static_cast<const T*>(f.gates) + qrow * 3);
      const float pr = g0 * exp2f(fmaf(s, c2, -p.lse[qrow] * kLog2e));
      const float ds = pr * (dp - p.delta[qrow]);
#pragma unroll
      for (int e = 0; e < kDL; ++e) {
        ak[e] = fmaf(ds, q[e], ak[e]);
        av[e] = fmaf(pr, dO[e], av[e]);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < kDL; ++e) ak[e] *= f.scale;
  const int64_t o = (static_cast<int64_t>(g) * f.nb_cap + j) * D + kDL * sub;
  store16(p.dkbar + o, ak);
  store16(p.dvbar + o, av);
}

// ------------------------------------------------------------ window branch

// dq of the window branch: LP lanes per (sorted position, query head) row,
// rows head-major; keys are the window's run of the sorted copies.
template <typename T, int D>
__global__ void __launch_bounds__(256)
win_dq_kernel(BwdParams p) {
  constexpr int LP = D / kDL;
  constexpr int NR = 256 / LP;
  const FwdParams& f = p.f;
  const int sub = threadIdx.x % LP;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * NR + threadIdx.x / LP;
  const int64_t nrow = static_cast<int64_t>(f.n) * f.h_q;
  if (row >= nrow) return;
  const int h = static_cast<int>(row / f.n);
  const int i = static_cast<int>(row % f.n);
  const int g = h / (f.h_q / f.h_kv);
  const int t = f.perm[i];
  const int w = window_of_pos(f.win_off, f.counts[SSA_COUNT_NW], i);
  const int wa = f.win_off[w], wb = f.win_off[w + 1];
  const int64_t qrow = static_cast<int64_t>(t) * f.h_q + h;
  const float c2 = f.scale * kLog2e;
  const float lse2 = p.lse[2 * nrow + qrow] * kLog2e;
  float q[kDL], dO[kDL], aa[kDL], ab[kDL];
  load16(static_cast<const T*>(f.q) + qrow * D + kDL * sub, q);
  load16(static_cast<const T*>(p.dout) + qrow * D + kDL * sub, dO);
#pragma unroll
  for (int e = 0; e < kDL; ++e) aa[e] = ab[e] = 0.f;
  float dl = 0.f;
  const T* KS = static_cast<const T*>(f.k_s) + static_cast<int64_t>(g) * f.n * D + kDL * sub;
  const T* VS = static_cast<const T*>(f.v_s) + static_cast<int64_t>(g) * f.n * D + kDL * sub;
  for (int k = wa; k < wb; ++k) {
    float kr[kDL], vr[kDL];
    load16(KS + static_cast<int64_t>(k) * D, kr);
    load16(VS + static_cast<int64_t>(k) * D, vr);
    const float s = row_sum<LP>(dot16(q, kr));
    const float dp = row_sum<LP>(dot16(dO, vr));
    const float pr = exp2f(fmaf(s, c2, -lse2));
    const float pd = pr * dp;
    dl += pd;
#pragma unroll
    for (int e = 0; e < kDL; ++e) {
      aa[e] = fmaf(pd, kr[e], aa[e]);
      ab[e] = fmaf(pr, kr[e], ab[e]);
    }
  }
  const float gs = Elt<T>::load(static_cast<const T*>(f.gates) + qrow * 3 + 2) * f.scale;
  float* dst = p.dq_acc + qrow * D + kDL * sub;
  float cur[kDL];
  load16(dst, cur);
#pragma unroll
  for (int e = 0; e < kDL; ++e) cur[e] = fmaf(gs, fmaf(-dl, ab[e], aa[e]), cur[e]);
  store16(dst, cur);
  if (sub == 0) put_delta<T>(p, 2, qrow, dl);
}

// dk / dv of the window's tokens: one workgroup per (window, group), LP
// lanes per key token, each walking every (query, head of the group) of the
// window (first writer of dk_acc / dv_acc).
template <typename T, int D>
__global__ void __launch_bounds__(256)
win_dkv_kernel(BwdParams p) {
  constexpr int LP = D / kDL;
  constexpr int NR = 256 / LP;
  const FwdParams& f = p.f;
  const int sub = threadIdx.x % LP;
  const int rl = threadIdx.x / LP;
  const int nw = f.counts[SSA_COUNT_NW];
  const int G = f.h_q / f.h_kv;
  const float c2 = f.scale * kLog2e;
  const int64_t nrow = static_cast<int64_t>(f.n) * f.h_q;
  const float* lse = p.lse + 2 * nrow;
  const float* dlt = p.delta + 2 * nrow;
  const T* Q = static_cast<const T*>(f.q);
  const T* dO = static_cast<const T*>(p.dout);
  const T* gates = static_cast<const T*>(f.gates);
  for (int64_t item = blockIdx.x; item < static_cast<int64_t>(nw) * f.h_kv; item += gridDim.x) {
    const int g = static_cast<int>(item / nw);
    const int w = static_cast<int>(item % nw);
    const int wa = f.win_off[w], wb = f.win_off[w + 1];
    const int n_w = wb - wa;
    for (int r0 = 0; r0 < n_w; r0 += NR) {
      const int r = r0 + rl;
      if (r >= n_w) continue;
      const int64_t krow = (static_cast<int64_t>(g) * f.n + wa + r) * D + kDL * sub;
      float kr[kDL], vr[kDL], ak[kDL], av[kDL];
      load16(static_cast<const T*>(f.k_s) + krow, kr);
      load16(static_cast<const T*>(f.v_s) + krow, vr);
#pragma unroll
      for (int e = 0; e < kDL; ++e) ak[e] = av[e] = 0.f;
      for (int i = 0; i < n_w; ++i) {
        const int t = f.perm[wa + i];
        for (int hh = 0; hh < G; ++hh) {
          const int64_t qrow = static_cast<int64_t>(t) * f.h_q + g * G + hh;
          float q[kDL], d[kDL];
          load16(Q + qrow * D + kDL * sub, q);
          load16(dO + qrow * D + kDL * sub, d);
          const float s = row_sum<LP>(dot16(q, kr));
          const float dp = row_sum<LP>(dot16(d, vr));
          const float g2 = Elt<T>::load(gates + qrow * 3 + 2);
          const float pr = g2 * exp2f(fmaf(s, c2, -lse[qrow] * kLog2e));
          const float ds = pr * (dp - dlt[qrow]);
#pragma unroll
          for (int e = 0; e < kDL; ++e) {
            ak[e] = fmaf(ds, q[e], ak[e]);
            av[e] = fmaf(pr, d[e], av[e]);
          }
        }
      }
#pragma unroll
      for (int e = 0; e < kDL; ++e) ak[e] *= f.scale;
      store16(p.dk_acc + krow, ak);
      store16(p.dv_acc + krow, av);
    }
  }
}

// ------------------------------------------------------------ selected branch

// dk / dv of the tokens of block j for group g, over every query that chose
// the block (one workgroup per (group, block); adds to dk_acc / dv_acc).
template <typename T, int D>
__global__ void __launch_bounds__(256)
sel_dkv_kernel(BwdParams p) {
  constexpr int LP = D / kDL;
  constexpr int NR = 256 / LP;
  const FwdParams& f = p.f;
  const int sub = threadIdx.x % LP;
  const int rl = threadIdx.x / LP;
  const int nb = f.counts[SSA_COUNT_NB];
  const int G = f.h_q / f.h_kv;
  const float c2 = f.scale * kLog2e;
  const int64_t nrow = static_cast<int64_t>(f.n) * f.h_q;
  const float* lse = p.lse + nrow;
  const float* dlt = p.delta + nrow;
  const T* Q = static_cast<const T*>(f.q);
  const T* dO = static_cast<const T*>(p.dout);
  const T* gates = static_cast<const T*>(f.gates);
  for (int64_t item = blockIdx.x; item < static_cast<int64_t>(nb) * f.h_kv; item += gridDim.x) {
    const int g = static_cast<int>(item / nb);
    const int j = static_cast<int>(item % nb);
    const int64_t slot = static_cast<int64_t>(g) * f.nb_cap + j;
    const int e0 = p.sel_off[slot], e1 = p.sel_off[slot + 1];
    if (e0 == e1) continue;
    const int a = f.blk_off[j], bnd = f.blk_off[j + 1];
    for (int r0 = a; r0 < bnd; r0 += NR) {
      const int i = r0 + rl;
      if (i >= bnd) continue;
      const int64_t krow = (static_cast<int64_t>(g) * f.n + i) * D + kDL * sub;
      float kr[kDL], vr[kDL], ak[kDL], av[kDL];
      load16(static_cast<const T*>(f.k_s) + krow, kr);
      load16(static_cast<const T*>(f.v_s) + krow, vr);
#pragma unroll
      for (int e = 0; e < kDL; ++e) ak[e] = av[e] = 0.f;
      for (int e = e0; e < e1; ++e) {
        const int t = p.sel_list[e];
        for (int hh = 0; hh < G; ++hh) {
          const int64_t qrow = static_cast<int64_t>(t) * f.h_q + g * G + hh;
          float q[kDL], d[kDL];
          load16(Q + qrow * D + kDL * sub, q);
          load16(dO + qrow * D + kDL * sub, d);
          const float s = row_sum<LP>(dot16(q, kr));
          const float dp = row_sum<LP>(dot16(d, vr));
          const float g1 = Elt<T>::load(gates + qrow * 3 + 1);
          const float pr = g1 * exp2f(fmaf(s, c2, -lse[qrow] * kLog2e));
          const float ds = pr * (dp - dlt[qrow]);
#pragma unroll
          for (int x = 0; x < kDL; ++x) {
            ak[x] = fmaf(ds, q[x], ak[x]);
            av[x] = fmaf(pr, d[x], av[x]);
          }
        }
      }
      float ck[kDL], cv[kDL];
      load16(p.dk_acc + krow, ck);
      load16(p.dv_acc + krow, cv);
#pragma unroll
      for (int x = 0; x < kDL; ++x) {
        ck[x] = fmaf(f.scale, ak[x], ck[x]);
        cv[x] += av[x];
      }
      store16(p.dk_acc + krow, ck);
      store16(p.dv_acc + krow, cv);
    }
  }
}

// dq of the selected branch, added to the other branches' share, written in
// the input dtype.  LP lanes per (token, head) row, rows head-major.  As in the
// forward's selection kernel, the row's lanes first load its selected blocks'
// row ranges (all loads in flight at once) and list the first kList row
// positions in LDS, so the loads of a row wait on no block offset; rows past
// the list are walked block by block afterwards.  The rows are visited in
// rank order, block by block, exactly as a plain loop over the list would.
template <typename T, int D, int KMAX>
__global__ void __launch_bounds__(256, 4)
sel_dq_kernel(BwdParams p) {
  constexpr int LP = D / kDL;
  constexpr int NR = 256 / LP;
  constexpr int kList = 64;
  __shared__ int2 ranges[NR * KMAX];
  __shared__ int32_t rows_l[NR * kList];
  const FwdParams& f = p.f;
  const int sub = threadIdx.x % LP;
  const int pl = threadIdx.x / LP;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * NR + pl;
  const int64_t nrow = static_cast<int64_t>(f.n) * f.h_q;
  const bool active = row < nrow;
  const int h = active ? static_cast<int>(row / f.n) : 0;
  const int t = active ? static_cast<int>(row % f.n) : 0;
  const int g = h / (f.h_q / f.h_kv);
  const int nb = f.counts[SSA_COUNT_NB];
  const int64_t qrow = static_cast<int64_t>(t) * f.h_q + h;
  const float c2 = f.scale * kLog2e;
  const float l2 = active ? p.lse[nrow + qrow] * kLog2e : 0.f;
  // bf16 rows stay packed for the dot products (v_dot2); float rows widen
  constexpr bool kBf16 = sizeof(T) == 2;
  float q[kDL], d[kDL], aa[kDL], ab[kDL];
  uint4 qw[2], dw[2];
  if constexpr (kBf16) {
    load_raw16(reinterpret_cast<const uint16_t*>(f.q) + qrow * D + kDL * sub, qw);
    load_raw16(reinterpret_cast<const uint16_t*>(p.dout) + qrow * D + kDL * sub, dw);
  } else {
    load16(static_cast<const T*>(f.q) + qrow * D + kDL * sub, q);
    load16(static_cast<const T*>(p.dout) + qrow * D + kDL * sub, d);
  }
#pragma unroll
  for (int e = 0; e < kDL; ++e) aa[e] = ab[e] = 0.f;
  float dl = 0.f;
  const T* KS = static_cast<const T*>(f.k_s) + static_cast<int64_t>(g) * f.n * D + kDL * sub;
  const T* VS = static_cast<const T*>(f.v_s) + static_cast<int64_t>(g) * f.n * D + kDL * sub;
  const int32_t* sel = f.topk_idx + (static_cast<int64_t>(t) * f.h_kv + g) * f.topk;

  // the selected blocks' row ranges: lane sub loads ranks sub, sub + LP, ...;
  // the list ends at the first block id outside [0, nb)
  int2* const rng = ranges + pl * KMAX;
#pragma unroll
  for (int i = 0; i < KMAX / LP; ++i) {
    const int r = sub + LP * i;
    const int id = (active && r < f.topk) ? sel[r] : -1;
    const bool ok = id >= 0 && id < nb;
    rng[r] = ok ? make_int2(f.blk_off[id], f.blk_off[id + 1]) : make_int2(-1, -1);
  }
  wave_lds_sync();
  int total = 0, k_eff = 0;
  for (; k_eff < KMAX; ++k_eff) {
    const int2 r = rng[k_eff];
    if (r.x < 0) break;
    for (int i = r.x + sub; i < r.y; i += LP) {
      const int idx = total + (i - r.x);
      if (idx < kList) rows_l[pl * kList + idx] = i;
    }
    total += r.y - r.x;
  }
  wave_lds_sync();

  auto visit = [&](int64_t i) {
    float kr[kDL];
    float s, dp;
    if constexpr (kBf16) {
      uint4 kw[2], vw[2];
      load_raw16(reinterpret_cast<const uint16_t*>(KS) + i * D, kw);
      load_raw16(reinterpret_cast<const uint16_t*>(VS) + i * D, vw);
      s = row_sum<LP>(dot16_bf16(qw, kw));
      dp = row_sum<LP>(dot16_bf16(dw, vw));
      widen16(kw, kr);
    } else {
      float vr[kDL];
      load16(KS + i * D, kr);
      load16(VS + i * D, vr);
      s = row_sum<LP>(dot16(q, kr));
      dp = row_sum<LP>(dot16(d, vr));
    }
    const float pr = exp2f(fmaf(s, c2, -l2));
    const float pd = pr * dp;
    dl += pd;
#pragma unroll
    for (int e = 0; e < kDL; ++e) {
      aa[e] = fmaf(pd, kr[e], aa[e]);
      ab[e] = fmaf(pr, kr[e], ab[e]);
    }
  };
  const int listed = min(total, kList);
  for (int i = 0; i < listed; ++i) visit(rows_l[pl * kList + i]);
  if (total > kList) {
    int seen = 0;
    for (int r = 0; r < k_eff; ++r) {
      const int2 rr = rng[r];
      for (int i = rr.x; i < rr.y; ++i, ++seen)
        if (seen >= kList) visit(i);
    }
  }

  if (!active) return;
  const float gs = Elt<T>::load(static_cast<const T*>(f.gates) + qrow * 3 + 1) * f.scale;
  float cur[kDL];
  load16(p.dq_acc + qrow * D + kDL * sub, cur);
#pragma unroll
  for (int e = 0; e < kDL; ++e) cur[e] = fmaf(gs, fmaf(-dl, ab[e], aa[e]), cur[e]);
  store16(static_cast<T*>(p.dq) + qrow * D + kDL * sub, cur);
  if (sub == 0) put_delta<T>(p, 1, qrow, dl);
}

// ------------------------------------------------------------ dk, dv

// One workgroup per block (grid-stride): every token of the block gets its
// window and selection sums plus 1 / n_j of the pooled rows' gradients,
// written in the input dtype and input token order.
template <typename T, int D>
__global__ void __launch_bounds__(256)
bwd_finalize_kernel(BwdParams p) {
  constexpr int LP = D / kDL;
  const FwdParams& f = p.f;
  const int nb = f.counts[SSA_COUNT_NB];
  const int per_tok = f.h_kv * LP;  // threads per token
  for (int j = blockIdx.x; j < nb; j += gridDim.x) {
    const int a = f.blk_off[j], b = f.blk_off[j + 1];
    const float inv = 1.f / static_cast<float>(b - a);
    for (int e = threadIdx.x; e < (b - a) * per_tok; e += 256) {
      const int i = a + e / per_tok;
      const int g = (e % per_tok) / LP;
      const int sub = e % LP;
      const int t = f.perm[i];
      const int64_t src = (static_cast<int64_t>(g) * f.n + i) * D + kDL * sub;
      const int64_t pb = (static_cast<int64_t>(g) * f.nb_cap + j) * D + kDL * sub;
      const int64_t dst = (static_cast<int64_t>(t) * f.h_kv + g) * D + kDL * sub;
      float x[kDL], y[kDL];
      load16(p.dk_acc + src, x);
      load16(p.dkbar + pb, y);
#pragma unroll
      for (int c = 0; c < kDL; ++c) x[c] = fmaf(y[c], inv, x[c]);
      store16(static_cast<T*>(p.dk) + dst, x);
      load16(p.dv_acc + src, x);
      load16(p.dvbar + pb, y);
#pragma unroll
      for (int c = 0; c < kDL; ++c) x[c] = fmaf(y[c], inv, x[c]);
      store16(static_cast<T*>(p.dv) + dst, x);
    }
  }
}

// ------------------------------------------------------------ launchers

int rows_grid(int64_t rows, int per_block) {
  return static_cast<int>((rows + per_block - 1) / per_block);
}

}  // namespace

hipError_t launch_bwd_pool(const BwdParams& p, ssa_dtype dtype, hipStream_t stream) {
  return launch_pool(p.f, dtype, stream);
}

hipError_t launch_bwd_sel_index(const BwdParams& p, ssa_dtype /*dtype*/, hipStream_t stream) {
  const int64_t m = static_cast<int64_t>(p.f.n) * p.f.h_kv * p.f.topk;
  const int grid = static_cast<int>(std::min<int64_t>((m + 255) / 256, 8192));
  sel_keys_kernel<<<grid, 256, 0, stream>>>(p);
  hipError_t e = launch_sort_pairs(p.sel_keys, p.sel_vals, p.sel_keys_tmp, p.sel_vals_tmp,
                                   static_cast<int32_t>(m), p.sel_key_bits, p.sel_hist, stream);
  if (e != hipSuccess) return e;
  const int64_t nl = static_cast<int64_t>(p.f.h_kv) * p.f.nb_cap + 1;
  sel_offsets_kernel<<<static_cast<int>(std::min<int64_t>((nl + 255) / 256, 8192)), 256, 0, stream>>>(p);
  return hipGetLastError();
}

#define SSA_BWD_LAUNCH(KERNEL, GRID)                                          \
  do {                                                                        \
    if (dtype == SSA_BF16) {                                                  \
      if (p.f.d == 32) KERNEL<uint16_t, 32><<<(GRID), 256, 0, stream>>>(p);  \
      else KERNEL<uint16_t, 64><<<(GRID), 256, 0, stream>>>(p);              \
    } else {                                                                  \
      if (p.f.d == 32) KERNEL<float, 32><<<(GRID), 256, 0, stream>>>(p);     \
      else KERNEL<float, 64><<<(GRID), 256, 0, stream>>>(p);                 \
    }                                                                         \
  } while (0)

hipError_t launch_bwd_cmp_dq(const BwdParams& p, ssa_dtype dtype, hipStream_t stream) {
  const int nr = 256 / (p.f.d / kDL);
  const int grid = rows_grid(static_cast<int64_t>(p.f.n) * p.f.h_q, nr);
  SSA_BWD_LAUNCH(cmp_dq_kernel, grid);
  return hipGetLastError();
}

hipError_t launch_bwd_cmp_dkv(const BwdParams& p, ssa_dtype dtype, hipStream_t stream) {
  // rows = (group, block) with the block count read on the device: size the
  // grid for the capacity; rows past the count exit at once
  const int nr = 256 / (p.f.d / kDL);
  const int grid = rows_grid(static_cast<int64_t>(p.f.h_kv) * p.f.nb_cap, nr);
  SSA_BWD_LAUNCH(cmp_dkv_kernel, grid);
  return hipGetLastError();
}

hipError_t launch_bwd_win_dq(const BwdParams& p, ssa_dtype dtype, hipStream_t stream) {
  const int nr = 256 / (p.f.d / kDL);
  const int grid = rows_grid(static_cast<int64_t>(p.f.n) * p.f.h_q, nr);
  SSA_BWD_LAUNCH(win_dq_kernel, grid);
  return hipGetLastError();
}

hipError_t launch_bwd_win_dkv(const BwdParams& p, ssa_dtype dtype, hipStream_t stream) {
  SSA_BWD_LAUNCH(win_dkv_kernel, 4096);
  return hipGetLastError();
}

hipError_t launch_bwd_sel_dkv(const BwdParams& p, ssa_dtype dtype, hipStream_t stream) {
  SSA_BWD_LAUNCH(sel_dkv_kernel, 8192);
  return hipGetLastError();
}

template <int KMAX>
void launch_sel_dq_k(const BwdParams& p, ssa_dtype dtype, int grid, hipStream_t stream) {
  if (dtype == SSA_BF16) {
    if (p.f.d == 32) sel_dq_kernel<uint16_t, 32, KMAX><<<grid, 256, 0, stream>>>(p);
    else sel_dq_kernel<uint16_t, 64, KMAX><<<grid, 256, 0, stream>>>(p);
  } else {
    if (p.f.d == 32) sel_dq_kernel<float, 32, KMAX><<<grid, 256, 0, stream>>>(p);
    else sel_dq_kernel<float, 64, KMAX><<<grid, 256, 0, stream>>>(p);
  }
}

hipError_t launch_bwd_sel_dq(const BwdParams& p, ssa_dtype dtype, hipStream_t stream) {
  const int nr = 256 / (p.f.d / kDL);
  const int grid = rows_grid(static_cast<int64_t>(p.f.n) * p.f.h_q, nr);
  if (p.f.topk <= 16) launch_sel_dq_k<16>(p, dtype, grid, stream);
  else launch_sel_dq_k<32>(p, dtype, grid, stream);
  return hipGetLastError();
}

hipError_t launch_bwd_finalize(const BwdParams& p, ssa_dtype dtype, hipStream_t stream) {
  SSA_BWD_LAUNCH(bwd_finalize_kernel, 8192);
  return hipGetLastError();
}

}  // namespace ssa
