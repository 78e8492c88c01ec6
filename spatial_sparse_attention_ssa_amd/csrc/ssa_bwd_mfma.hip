// Compressed-branch backward on MFMA (bf16, D = 32 or 64, any group size).
//
// Direct3D-S2 page, "Method": the compressed branch is a softmax attention
// of every query over the mean-pooled blocks of its sequence.  With P the
// probabilities (from the log-sum-exp the forward saved), dP = dO Vbar^T and
// Delta = rowsum(P * dP):
//   dq    = G0 scale (P * (dP - Delta)) Kbar
//   dKbar = scale sum over the sequence's (query, head) rows of G0 P (dP - Delta) q
//   dVbar = sum over the same rows of G0 P dO
// Both kernels use v_mfma_f32_32x32x16_bf16 on 32 x 32 tiles.
//
// cmp_dq_mfma_kernel (query-major): a workgroup owns 128 sorted queries of
//   one sequence and one query head, a wave 32 of them.  Pooled key / value
//   rows stream through a two-slot LDS ring, 32 blocks per tile (the key
//   rows are read as they are and, for Kbar^T, with gfx950's transposing LDS
//   load).  Per tile: S^T = Kbar Q^T and dP^T = Vbar dO^T, then
//   P and P * dP in registers, and dq^T accumulates as A - Delta B with
//   A = Kbar^T (P * dP)^T and B = Kbar^T P^T, so Delta (summed on the fly)
//   comes from the same float32 P as the rest.  Writes dq_acc (first writer),
//   Delta and the gate gradient.
//
// cmp_dkv_mfma_kernel (block-major): a workgroup owns 128 blocks of one
//   sequence and one key/value group, a wave one 32-block tile whose pooled
//   rows stay in registers as MFMA operands.  The sequence's (query, head)
//   rows stream through LDS 32 at a time, row-major, read as they are for
//   S = Q Kbar^T and dP = dO Vbar^T and with the transposing LDS load for
//   dVbar^T += dO^T (G0 P)^T and dKbar^T += Q^T (G0 P (dP - Delta))^T.
//   Its 1D grid starts the chunks of the longest sequences first.  When
//   there are few block tiles (grouped heads: few key/value groups, many
//   rows), the rows are split over several workgroups whose partial tiles are
//   summed afterwards in split order.
//
// kv_grad_mfma_kernel: the same block-major product for the token keys of
//   the selected branch (the window branch's token keys come from
//   win_dkv_mfma_kernel): one workgroup per (group, block), the rows being
//   every (query, head) whose top-k list holds the block (the inverted
//   lists).  The key tile is up to 32 tokens of the block (sorted copies, in
//   registers); each wave streams its own share of the rows, gathered as
//   whole 16-byte chunks (8 lanes per 64-dim row) into a wave-private LDS
//   area, row-major, from which the A operands are read as they are and the
//   transposed operands through gfx950's transposing LDS load; the four
//   partial tiles are summed in LDS ([dim][token]), in wave order, at the
//   end.
#include <float.h>

#include <algorithm>

#include <type_traits>

#include "ssa_internal.h"

namespace ssa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kQT = 128;  // sorted queries per workgroup of the dq kernel (4 waves x 32)
constexpr int kBT = 4;    // 32-block tiles per workgroup of the dkv kernel (one per wave)

__device__ __forceinline__ bf16x8 lds_b128(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ bf16x8 pack8(const float* x) {
  bf16x8 b;
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = static_cast<__bf16>(x[i]);
  return b;
}

__device__ __forceinline__ void seq_bounds(const FwdParams& f, int b, int* s0, int* s1, int* j0, int* j1) {
  *s0 = f.win_off[f.seq_win_off[b]];
  *s1 = f.win_off[f.seq_win_off[b + 1]];
  *j0 = f.seq_blk_off[b];
  *j1 = f.seq_blk_off[b + 1];
}

// the sequence b with pre[b] <= tile < pre[b + 1]
__device__ __forceinline__ int find_seq(const int32_t* pre, int batch, int tile) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Up to this many sequences are put in cost order (more, and the tail of
// the grid is short anyway).
constexpr int kOrderMax = 1024;

// Tile prefixes of the two compressed-branch gradient kernels.  The
// query-tile prefix follows the sequence order; the block-chunk prefix
// follows seq_order, the sequences by decreasing token count, since a
// pooled-row workgroup costs in proportion to its sequence's rows: with the
// chunk index slowest in that kernel's grid, the costliest workgroups start
// first and the short ones fill the end (longest-first list scheduling).
__global__ void __launch_bounds__(256) bwd_tile_prefix_kernel(BwdParams p) {
  __shared__ int len[kOrderMax];
  __shared__ int ord[kOrderMax];
  const int batch = p.f.batch;
  const bool order = batch <= kOrderMax;
  if (order) {
    for (int b = threadIdx.x; b < batch; b += blockDim.x) {
      int s0, s1, j0, j1;
      seq_bounds(p.f, b, &s0, &s1, &j0, &j1);
      len[b] = s1 - s0;
    }
    __syncthreads();
    for (int b = threadIdx.x; b < batch; b += blockDim.x) {
      int rank = 0;
      for (int c = 0; c < batch; ++c) rank += (len[c] > len[b] || (len[c] == len[b] && c < b)) ? 1 : 0;
      ord[rank] = b;
    }
    __syncthreads();
  }
  for (int r = threadIdx.x; r < batch; r += blockDim.x) p.seq_order[r] = order ? ord[r] : r;
  if (threadIdx.x != 0) return;
  int rq = 0, rb = 0;
  for (int r = 0; r < batch; ++r) {
    p.qtile_pre[r] = rq;
    p.btile_pre[r] = rb;
    int s0, s1, j0, j1;
    seq_bounds(p.f, r, &s0, &s1, &j0, &j1);
    rq += (s1 - s0 + kQT - 1) / kQT;
    seq_bounds(p.f, order ? ord[r] : r, &s0, &s1, &j0, &j1);
    if (j1 > j0) {
      const int tiles = (j1 + kKeyTile - 1) / kKeyTile - j0 / kKeyTile;
      rb += (tiles + kBT - 1) / kBT;
    }
  }
  p.qtile_pre[batch] = rq;
  p.btile_pre[batch] = rb;
}

// ------------------------------------------------------------ dq (query-major)

// Three workgroups per compute unit: D = 64 then fits 168 registers without
// spilling, and the extra waves hide the tile loads (measured 8 % faster than
// two).
template <int D>
__global__ void __launch_bounds__(256, 3)
cmp_dq_mfma_kernel(BwdParams p) {
  constexpr int KS = D / 16;          // MFMA k steps over the dims
  constexpr int VB = D / 32;          // 32-dim row blocks of dq^T
  constexpr int kKRow = D + 8;        // padded key / value row (bf16)
  constexpr int kRowCh = kKeyTile * D / 8;   // 16-byte chunks of a 32-row tile
  constexpr int kKT = kKeyTile * kKRow;
  __shared__ __align__(16) uint16_t k_lds[2 * kKT];
  __shared__ __align__(16) uint16_t v_lds[2 * kKT];

  const FwdParams& f = p.f;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int half = lane >> 5;
  const int h = blockIdx.y;
  const int g = h / (f.h_q / f.h_kv);
  const int tile = blockIdx.x;
  if (tile >= p.qtile_pre[f.batch]) return;
  const int b = find_seq(p.qtile_pre, f.batch, tile);
  int s0, s1, j0, j1;
  seq_bounds(f, b, &s0, &s1, &j0, &j1);
  const int qi = s0 + (tile - p.qtile_pre[b]) * kQT + wv * 32 + (lane & 31);
  const bool valid = qi < s1;
  const int t = valid ? f.perm[qi] : 0;
  const int64_t qrow = static_cast<int64_t>(t) * f.h_q + h;
  const uint16_t* Q = static_cast<const uint16_t*>(f.q);
  const uint16_t* dO = static_cast<const uint16_t*>(p.dout);
  // B operands: the lane's query and output-gradient rows
  bf16x8 qb[KS], db[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 a = {0u, 0u, 0u, 0u}, c = {0u, 0u, 0u, 0u};
    if (valid) {
      a = *reinterpret_cast<const u32x4*>(Q + qrow * D + 16 * ks + 8 * half);
      c = *reinterpret_cast<const u32x4*>(dO + qrow * D + 16 * ks + 8 * half);
    }
    qb[ks] = __builtin_bit_cast(bf16x8, a);
    db[ks] = __builtin_bit_cast(bf16x8, c);
  }
  const float c2 = f.scale * kLog2e;
  const float l2 = valid ? p.lse[qrow] * kLog2e : 0.f;
  const int kt0 = j0 / kKeyTile;
  const int n_kt = (j1 + kKeyTile - 1) / kKeyTile - kt0;

  // staging: thread tid moves chunk tid of the key rows and of the value rows
  // (D = 32: threads below 128 only); the key rows serve both as they are
  // (S = K Q^T) and through the transposing LDS load (dq^T += K^T dS^T)
  const uint16_t* KB = static_cast<const uint16_t*>(f.kbar) + static_cast<int64_t>(g) * f.nb_cap * D;
  const uint16_t* VBR = static_cast<const uint16_t*>(f.vbar) + static_cast<int64_t>(g) * f.nb_cap * D;
  const bool stager = tid < kRowCh;
  const int r_row = tid / (D / 8), r_c = tid % (D / 8);   // key / value rows: row, 8-dim chunk
  const int64_t src_r = static_cast<int64_t>(r_row) * D + 8 * r_c;
  const int dst_r = r_row * kKRow + 8 * r_c;
  u32x4 rk = {0u, 0u, 0u, 0u}, rv = {0u, 0u, 0u, 0u};
  auto load = [&](int kt) {
    if (stager) {
      const int64_t base = static_cast<int64_t>(kt) * kKeyTile * D;
      rk = *reinterpret_cast<const u32x4*>(KB + base + src_r);
      rv = *reinterpret_cast<const u32x4*>(VBR + base + src_r);
    }
  };
  auto store = [&](int slot) {
    if (stager) {
      *reinterpret_cast<u32x4*>(k_lds + slot * kKT + dst_r) = rk;
      *reinterpret_cast<u32x4*>(v_lds + slot * kKT + dst_r) = rv;
    }
  };

  f32x16 aa[VB], ab[VB];
#pragma unroll
  for (int vb = 0; vb < VB; ++vb) {
    aa[vb] = f32x16{};
    ab[vb] = f32x16{};
  }
  float dl = 0.f;
  load(kt0);
  store(0);
  if (n_kt > 1) load(kt0 + 1);
  // the first and the last tile are the only ones that can hold blocks
  // outside [j0, j1): they run with the range check, the tiles between
  // without it
  auto step = [&](int rel, auto masked) {
    __syncthreads();  // tile rel stored; every wave is done with tile rel - 1
    if (rel + 1 < n_kt) store((rel + 1) & 1);
    if (rel + 2 < n_kt) load(kt0 + rel + 2);
    const int slot = rel & 1;
    const uint16_t* kl = k_lds + slot * kKT + (lane & 31) * kKRow + 8 * half;
    const uint16_t* vl = v_lds + slot * kKT + (lane & 31) * kKRow + 8 * half;
    f32x16 s = {}, dp = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128(kl + 16 * ks), qb[ks], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128(vl + 16 * ks), db[ks], dp, 0, 0, 0);
    }
    // entry r is block jb + 8 (r / 4) + 4 half + r % 4 of this query
    const int jb = (kt0 + rel) * kKeyTile + 4 * half;
    float pr[16], pd[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = __builtin_amdgcn_exp2f(fmaf(s[r], c2, -l2));
      if constexpr (decltype(masked)::value) {
        const int j = jb + 8 * (r >> 2) + (r & 3);
        if (j < j0 || j >= j1) x = 0.f;
      }
      pr[r] = x;
      pd[r] = x * dp[r];
      dl += pd[r];
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 pdb = pack8(pd + 8 * ks);
      const bf16x8 pb = pack8(pr + 8 * ks);
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) {
        const bf16x8 a = lds_tr_operand<kKRow>(k_lds + slot * kKT, lane, vb, ks);
        aa[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pdb, aa[vb], 0, 0, 0);
        ab[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, ab[vb], 0, 0, 0);
      }
    }
  };
  step(0, std::true_type{});
  for (int rel = 1; rel < n_kt - 1; ++rel) step(rel, std::false_type{});
  if (n_kt > 1) step(n_kt - 1, std::true_type{});
  dl += __shfl_xor(dl, 32);
  if (!valid) return;
  const float gs = bf16_bits_to_f32(static_cast<const uint16_t*>(f.gates)[qrow * 3]) * f.scale;
  float* dst = p.dq_acc + qrow * D;
#pragma unroll
  for (int vb = 0; vb < VB; ++vb)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int d = 32 * vb + 8 * rb + 4 * half;
      float4 o;
      o.x = gs * fmaf(-dl, ab[vb][4 * rb], aa[vb][4 * rb]);
      o.y = gs * fmaf(-dl, ab[vb][4 * rb + 1], aa[vb][4 * rb + 1]);
      o.z = gs * fmaf(-dl, ab[vb][4 * rb + 2], aa[vb][4 * rb + 2]);
      o.w = gs * fmaf(-dl, ab[vb][4 * rb + 3], aa[vb][4 * rb + 3]);
      *reinterpret_cast<float4*>(dst + d) = o;
    }
  if (half == 0) {
    p.delta[qrow] = dl;
    if (p.dgates) static_cast<uint16_t*>(p.dgates)[qrow * 3] = f32_to_bf16_bits(dl);
  }
}

// ------------------------------------------------------------ sorted (query, head) rows

// Row R = i * G + hh of group g is query head g * G + hh of the token at
// sorted position i.  rows_prep_kernel writes, per group, the rows of Q and
// dO in that order (row-major) and per row (log2 lse, Delta, gate) of the
// compressed and the window branch.  The block- and window-major gradient
// kernels then stage whole 16-byte chunks.
template <int D>
__global__ void __launch_bounds__(256)
rows_prep_kernel(BwdParams p) {
  constexpr int CPR = D / 8;   // 16-byte chunks of one (token, head) row
  constexpr int U = 8;         // chunks per thread in flight
  const FwdParams& f = p.f;
  const int tid = threadIdx.x;
  const int G = f.h_q / f.h_kv;
  const int64_t nrow = static_cast<int64_t>(f.n) * f.h_q;
  const int cpt = f.h_q * CPR;                          // chunks of a token's whole row (every head)
  const int n_pos = (p.rows_cap + G - 1) / G;           // sorted positions, the padding rows included
  const int ntile = (n_pos + kKeyTile - 1) / kKeyTile;
  const uint16_t* Q = static_cast<const uint16_t*>(f.q);
  const uint16_t* dO = static_cast<const uint16_t*>(p.dout);
  const uint16_t* gates = static_cast<const uint16_t*>(f.gates);
  // a workgroup takes 32 sorted positions: it reads their tokens' whole rows
  // (every head, contiguous in HBM) and writes each head's row to its
  // group's sorted row space, row i G + head % G
  for (int T = blockIdx.x; T < ntile; T += gridDim.x) {
    const int i0 = T * kKeyTile;
    const int n_ch = kKeyTile * cpt;
    for (int e0 = tid; e0 < n_ch; e0 += 256 * U) {
      u32x4 uq[U], ud[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = e0 + u * 256;
        uq[u] = ud[u] = u32x4{0u, 0u, 0u, 0u};
        const int i = i0 + e / cpt;
        if (e < n_ch && i < f.n) {
          const int64_t off = static_cast<int64_t>(f.perm[i]) * f.h_q * D + 8 * (e % cpt);
          uq[u] = *reinterpret_cast<const u32x4*>(Q + off);
          ud[u] = *reinterpret_cast<const u32x4*>(dO + off);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = e0 + u * 256;
        if (e >= n_ch) continue;
        const int i = i0 + e / cpt;
        const int cc = e % cpt, hh = cc / CPR, c = cc % CPR;
        const int64_t R = static_cast<int64_t>(i) * G + hh % G;
        if (R >= p.rows_cap) continue;
        const int64_t dst = (static_cast<int64_t>(hh / G) * p.rows_cap + R) * D + 8 * c;
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.q_rows) + dst) = uq[u];
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.do_rows) + dst) = ud[u];
      }
    }
    // per row (log2 lse, Delta, gate) of the compressed and the window branch
    for (int e = tid; e < kKeyTile * f.h_q; e += 256) {
      const int i = i0 + e / f.h_q, hh = e % f.h_q;
      const int64_t R = static_cast<int64_t>(i) * G + hh % G;
      if (R >= p.rows_cap) continue;
      float4 s0 = make_float4(FLT_MAX, 0.f, 0.f, 0.f), s2 = s0;   // a padding row has P = 0
      if (i < f.n) {
        const int64_t qrow = static_cast<int64_t>(f.perm[i]) * f.h_q + hh;
        s0 = make_float4(p.lse[qrow] * kLog2e, p.delta[qrow], bf16_bits_to_f32(gates[qrow * 3]), 0.f);
        s2 = make_float4(p.lse[2 * nrow + qrow] * kLog2e, p.delta[2 * nrow + qrow],
                         bf16_bits_to_f32(gates[qrow * 3 + 2]), 0.f);
      }
      const int64_t r = static_cast<int64_t>(hh / G) * p.rows_cap + R;
      p.st_rows[r] = s0;
      p.st_rows[static_cast<int64_t>(f.h_kv) * p.rows_cap + r] = s2;
    }
  }
}

// ------------------------------------------------------------ key gradients over sorted rows

// One workgroup, four waves, each wave one 32-key tile (its key and value
// rows in registers as MFMA B operands).  The rows [r_lo, r_hi) of group g
// (sorted row space, tiles aligned to 32; rows outside the range get P = 0)
// stream through a two-slot LDS ring, row-major: read as they are for the A
// operands of S = Q K^T and dP = dO V^T, and with the transposing LDS load
// for those of dV^T += dO^T (gate P)^T and dK^T += Q^T (gate P (dP - Delta))^T.
// Tiles [t_beg, t_end) of the range
// are this workgroup's share.  Writes scale * dK and dV rows of the valid
// keys to dk_row / dv_row (null: nothing to write).
template <int D>
__device__ __forceinline__ void rows_dkv_body(const BwdParams& p, int g, bool wave_on, const uint16_t* k_row,
                                              const uint16_t* v_row, int64_t r_lo, int64_t r_hi, int t_beg,
                                              int t_end, const float4* st, float* dk_row, float* dv_row,
                                              uint16_t* q_lds, uint16_t* d_lds, float4* st_lds) {
  constexpr int KS = D / 16;
  constexpr int VB = D / 32;
  constexpr int kRRow = D + 8;
  constexpr int kRT = kKeyTile * kRRow;
  constexpr int CPR = D / 8;
  const FwdParams& f = p.f;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const float c2 = f.scale * kLog2e;
  bf16x8 kb[KS], vb[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 a = {0u, 0u, 0u, 0u}, c = {0u, 0u, 0u, 0u};
    if (k_row) {
      a = *reinterpret_cast<const u32x4*>(k_row + 16 * ks + 8 * half);
      c = *reinterpret_cast<const u32x4*>(v_row + 16 * ks + 8 * half);
    }
    kb[ks] = __builtin_bit_cast(bf16x8, a);
    vb[ks] = __builtin_bit_cast(bf16x8, c);
  }
  const uint16_t* QR = static_cast<const uint16_t*>(p.q_rows) + static_cast<int64_t>(g) * p.rows_cap * D;
  const uint16_t* DR = static_cast<const uint16_t*>(p.do_rows) + static_cast<int64_t>(g) * p.rows_cap * D;
  // staging: thread tid moves chunk tid of each of the two tiles
  const bool stager = tid < kKeyTile * CPR;
  const int r_row = tid / CPR, r_c = tid % CPR;    // row, 8-dim chunk
  u32x4 rq = {0u, 0u, 0u, 0u}, rd = rq;
  float4 rs = make_float4(FLT_MAX, 0.f, 0.f, 0.f);
  auto load = [&](int T) {
    if (stager) {
      const int64_t ro = (static_cast<int64_t>(T) * kKeyTile + r_row) * D + 8 * r_c;
      rq = *reinterpret_cast<const u32x4*>(QR + ro);
      rd = *reinterpret_cast<const u32x4*>(DR + ro);
    }
    if (tid < kKeyTile) {
      const int64_t R = static_cast<int64_t>(T) * kKeyTile + tid;
      rs = (R >= r_lo && R < r_hi) ? st[R] : make_float4(FLT_MAX, 0.f, 0.f, 0.f);
    }
  };
  // per slot, three arrays over the tile's rows: -lse2 / c2 and -Delta (the
  // starting values of the S and dP accumulators, so that they hold
  // s - lse2 / c2 and dP - Delta) and the gate
  float* const st_f = reinterpret_cast<float*>(st_lds);
  auto store = [&](int slot) {
    if (stager) {
      *reinterpret_cast<u32x4*>(q_lds + slot * kRT + r_row * kRRow + 8 * r_c) = rq;
      *reinterpret_cast<u32x4*>(d_lds + slot * kRT + r_row * kRRow + 8 * r_c) = rd;
    }
    if (tid < kKeyTile) {
      float* const sf = st_f + slot * 4 * kKeyTile;
      sf[tid] = -rs.x / c2;
      sf[kKeyTile + tid] = -rs.y;
      sf[2 * kKeyTile + tid] = rs.z;
    }
  };

  f32x16 dk[VB], dv[VB];
#pragma unroll
  for (int x = 0; x < VB; ++x) {
    dk[x] = f32x16{};
    dv[x] = f32x16{};
  }
  const int n_rt = t_end - t_beg;
  if (n_rt > 0) {
    load(t_beg);
    store(0);
  }
  if (n_rt > 1) load(t_beg + 1);
  for (int rt = 0; rt < n_rt; ++rt) {
    __syncthreads();  // tile rt stored; every wave is done with tile rt - 1
    if (rt + 1 < n_rt) store((rt + 1) & 1);
    if (rt + 2 < n_rt) load(t_beg + rt + 2);
    if (!wave_on) continue;
    const int slot = rt & 1;
    const uint16_t* ql = q_lds + slot * kRT + (lane & 31) * kRRow + 8 * half;
    const uint16_t* dl = d_lds + slot * kRT + (lane & 31) * kRRow + 8 * half;
    // entry r is row 8 (r / 4) + 4 half + r % 4 of the tile, for this key:
    // rows 8 q + 4 half .. + 3 of each quarter q are one 16-byte read
    const float* sf = st_f + slot * 4 * kKeyTile + 4 * half;
    f32x16 s, dp;
    float gt[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 a = *reinterpret_cast<const float4*>(sf + 8 * q);
      const float4 b = *reinterpret_cast<const float4*>(sf + kKeyTile + 8 * q);
      const float4 c = *reinterpret_cast<const float4*>(sf + 2 * kKeyTile + 8 * q);
      s[4 * q] = a.x; s[4 * q + 1] = a.y; s[4 * q + 2] = a.z; s[4 * q + 3] = a.w;
      dp[4 * q] = b.x; dp[4 * q + 1] = b.y; dp[4 * q + 2] = b.z; dp[4 * q + 3] = b.w;
      gt[4 * q] = c.x; gt[4 * q + 1] = c.y; gt[4 * q + 2] = c.z; gt[4 * q + 3] = c.w;
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128(ql + 16 * ks), kb[ks], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128(dl + 16 * ks), vb[ks], dp, 0, 0, 0);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float pg[8], ds[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 8 * ks + i;
        const float x = gt[r] * __builtin_amdgcn_exp2f(s[r] * c2);
        pg[i] = x;
        ds[i] = x * dp[r];
      }
      const bf16x8 pb = pack8(pg);
      const bf16x8 sb = pack8(ds);
#pragma unroll
      for (int x = 0; x < VB; ++x) {
        dv[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_tr_operand<kRRow>(d_lds + slot * kRT, lane, x, ks), pb,
                                                        dv[x], 0, 0, 0);
        dk[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_tr_operand<kRRow>(q_lds + slot * kRT, lane, x, ks), sb,
                                                        dk[x], 0, 0, 0);
      }
    }
  }
  if (!dk_row) return;
#pragma unroll
  for (int x = 0; x < VB; ++x)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int d = 32 * x + 8 * rb + 4 * half;
      *reinterpret_cast<float4*>(dk_row + d) =
          make_float4(f.scale * dk[x][4 * rb], f.scale * dk[x][4 * rb + 1], f.scale * dk[x][4 * rb + 2],
                      f.scale * dk[x][4 * rb + 3]);
      *reinterpret_cast<float4*>(dv_row + d) =
          make_float4(dv[x][4 * rb], dv[x][4 * rb + 1], dv[x][4 * rb + 2], dv[x][4 * rb + 3]);
    }
}

#define SSA_ROWS_LDS(D)                                                   \
  __shared__ __align__(16) uint16_t q_lds[2 * kKeyTile * ((D) + 8)];    \
  __shared__ __align__(16) uint16_t d_lds[2 * kKeyTile * ((D) + 8)];    \
  __shared__ float4 st_lds[2 * kKeyTile]

// Pooled-row gradients: a workgroup owns 128 blocks (a 32-block tile per
// wave) of one sequence and group, over split z of the sequence's rows.  The
// 1D grid runs (chunk, split, group) with the group fastest and the chunk,
// in cost order, slowest.
template <int D>
__global__ void __launch_bounds__(256, 2)
cmp_dkv_mfma_kernel(BwdParams p) {
  SSA_ROWS_LDS(D);
  const FwdParams& f = p.f;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int g = static_cast<int>(blockIdx.x % f.h_kv);
  const int z = static_cast<int>((blockIdx.x / f.h_kv) % p.row_splits);
  const int G = f.h_q / f.h_kv;
  const int tile = static_cast<int>(blockIdx.x / (f.h_kv * p.row_splits));
  if (tile >= p.btile_pre[f.batch]) return;
  const int r = find_seq(p.btile_pre, f.batch, tile);
  int s0, s1, j0, j1;
  seq_bounds(f, p.seq_order[r], &s0, &s1, &j0, &j1);
  const int kt = j0 / kKeyTile + (tile - p.btile_pre[r]) * kBT + wv;
  const bool wave_on = kt < (j1 + kKeyTile - 1) / kKeyTile;
  const int j = kt * kKeyTile + (lane & 31);
  const bool jok = wave_on && j >= j0 && j < j1;
  const int64_t krow = (static_cast<int64_t>(g) * f.nb_cap + j) * D;
  const int64_t r_lo = static_cast<int64_t>(s0) * G, r_hi = static_cast<int64_t>(s1) * G;
  const int T0 = static_cast<int>(r_lo / kKeyTile);
  const int n_all = static_cast<int>((r_hi + kKeyTile - 1) / kKeyTile) - T0;
  const int per = (n_all + p.row_splits - 1) / p.row_splits;
  const int t_beg = T0 + min(n_all, z * per);
  const int t_end = T0 + min(n_all, (z + 1) * per);
  const int64_t part = p.row_splits > 1 ? static_cast<int64_t>(z) * f.h_kv * f.nb_cap * D : 0;
  float* ok = (p.row_splits > 1 ? p.dkbar_part : p.dkbar) + part;
  float* ov = (p.row_splits > 1 ? p.dvbar_part : p.dvbar) + part;
  rows_dkv_body<D>(p, g, wave_on, wave_on ? static_cast<const uint16_t*>(f.kbar) + krow : nullptr,
                   static_cast<const uint16_t*>(f.vbar) + krow, r_lo, r_hi, t_beg, t_end,
                   p.st_rows + static_cast<int64_t>(g) * p.rows_cap, jok ? ok + krow : nullptr,
                   ov + krow, q_lds, d_lds, st_lds);
}

// Window tokens' key / value gradients (first writer of dk_acc / dv_acc): a
// workgroup owns 128 tokens (a 32-token tile per wave) of one window and
// group, over all the window's rows; persistent grid over (group, window,
// 128-token chunk).
template <int D>
__global__ void __launch_bounds__(256, 2)
win_dkv_mfma_kernel(BwdParams p) {
  SSA_ROWS_LDS(D);
  const FwdParams& f = p.f;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int G = f.h_q / f.h_kv;
  const int nw = f.counts[SSA_COUNT_NW];
  const int cmax = (f.counts[SSA_COUNT_MAX_WIN] + 4 * kKeyTile - 1) / (4 * kKeyTile);
  const int64_t per_g = static_cast<int64_t>(nw) * cmax;
  for (int64_t item = blockIdx.x; item < per_g * f.h_kv; item += gridDim.x) {
    const int g = static_cast<int>(item / per_g);
    const int w = static_cast<int>((item % per_g) / cmax);
    const int c = static_cast<int>(item % cmax);
    const int wa = f.win_off[w], wb = f.win_off[w + 1];
    if (wa + 4 * kKeyTile * c >= wb) continue;
    const int i0 = wa + 4 * kKeyTile * c + kKeyTile * wv;
    const bool wave_on = i0 < wb;
    const int i = i0 + (lane & 31);
    const bool iok = wave_on && i < wb;
    const int64_t krow = (static_cast<int64_t>(g) * f.n + i) * D;
    const int64_t r_lo = static_cast<int64_t>(wa) * G, r_hi = static_cast<int64_t>(wb) * G;
    const int T0 = static_cast<int>(r_lo / kKeyTile);
    const int T1 = static_cast<int>((r_hi + kKeyTile - 1) / kKeyTile);
    rows_dkv_body<D>(p, g, wave_on, iok ? static_cast<const uint16_t*>(f.k_s) + krow : nullptr,
                     static_cast<const uint16_t*>(f.v_s) + krow, r_lo, r_hi, T0, T1,
                     p.st_rows + (static_cast<int64_t>(f.h_kv) + g) * p.rows_cap,
                     iok ? p.dk_acc + krow : nullptr, p.dv_acc + krow, q_lds, d_lds, st_lds);
    __syncthreads();  // the ring is reused by the next item
  }
}

// the pooled-row gradients: the row splits' partial sums, in split order
__global__ void __launch_bounds__(256)
dkv_split_sum_kernel(BwdParams p) {
  const int64_t per = static_cast<int64_t>(p.f.h_kv) * p.f.nb_cap * p.f.d;
  for (int64_t e = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4; e < per;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x * 4) {
    float4 k = *reinterpret_cast<const float4*>(p.dkbar_part + e);
    float4 v = *reinterpret_cast<const float4*>(p.dvbar_part + e);
    for (int z = 1; z < p.row_splits; ++z) {
      const float4 a = *reinterpret_cast<const float4*>(p.dkbar_part + z * per + e);
      const float4 c = *reinterpret_cast<const float4*>(p.dvbar_part + z * per + e);
      k.x += a.x; k.y += a.y; k.z += a.z; k.w += a.w;
      v.x += c.x; v.y += c.y; v.z += c.z; v.w += c.w;
    }
    *reinterpret_cast<float4*>(p.dkbar + e) = k;
    *reinterpret_cast<float4*>(p.dvbar + e) = v;
  }
}

// ------------------------------------------------------------ window branch dq

// dq of the window branch on MFMA: one workgroup per (window, query head)
// item (persistent grid, items head-major).  The window's key and value rows
// are staged row-major in LDS kWinChunk tokens at a time (the K^T operands
// come back through the transposing LDS load); each wave owns 32 of the
// window's queries and
// accumulates A = K^T (P * dP)^T and B = K^T P^T as in the compressed
// branch's dq kernel.  Adds to dq_acc; writes Delta and the gate gradient.
constexpr int kWinChunk = 128;

template <int D>
__global__ void __launch_bounds__(256, 2)
win_dq_mfma_kernel(BwdParams p) {
  constexpr int KS = D / 16;
  constexpr int VB = D / 32;
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int kKRow = D + 8;               // padded key / value row (bf16)
  __shared__ __align__(16) uint16_t k_lds[kWinChunk * kKRow];
  __shared__ __align__(16) uint16_t v_lds[kWinChunk * kKRow];

  const FwdParams& f = p.f;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int half = lane >> 5;
  const float c2 = f.scale * kLog2e;
  const int nw = f.counts[SSA_COUNT_NW];
  const int64_t nrow = static_cast<int64_t>(f.n) * f.h_q;
  const int64_t n_items = static_cast<int64_t>(nw) * f.h_q;
  const uint16_t* Q = static_cast<const uint16_t*>(f.q);
  const uint16_t* dO = static_cast<const uint16_t*>(p.dout);
  for (int64_t item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int h = static_cast<int>(item / nw);
    const int w = static_cast<int>(item % nw);
    const int wa = f.win_off[w], wb = f.win_off[w + 1];
    const int n_w = wb - wa;
    const int g = h / (f.h_q / f.h_kv);
    const uint16_t* KS_ = static_cast<const uint16_t*>(f.k_s) + (static_cast<int64_t>(g) * f.n + wa) * D;
    const uint16_t* VS_ = static_cast<const uint16_t*>(f.v_s) + (static_cast<int64_t>(g) * f.n + wa) * D;
    for (int qg0 = 0; qg0 < n_w; qg0 += 128) {
      const int qi = wa + qg0 + wv * 32 + (lane & 31);
      const bool valid = qi < wb;
      const int t = valid ? f.perm[qi] : 0;
      const int64_t qrow = static_cast<int64_t>(t) * f.h_q + h;
      bf16x8 qb[KS], db[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 a = {0u, 0u, 0u, 0u}, c = {0u, 0u, 0u, 0u};
        if (valid) {
          a = *reinterpret_cast<const u32x4*>(Q + qrow * D + 16 * ks + 8 * half);
          c = *reinterpret_cast<const u32x4*>(dO + qrow * D + 16 * ks + 8 * half);
        }
        qb[ks] = __builtin_bit_cast(bf16x8, a);
        db[ks] = __builtin_bit_cast(bf16x8, c);
      }
      const float l2 = valid ? p.lse[2 * nrow + qrow] * kLog2e : 0.f;
      f32x16 aa[VB], ab[VB];
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) {
        aa[vb] = f32x16{};
        ab[vb] = f32x16{};
      }
      float dl = 0.f;
      for (int kc = 0; kc < n_w; kc += kWinChunk) {
        const int nk = min(kWinChunk, n_w - kc);
        const int nk32 = (nk + 31) & ~31;
        __syncthreads();  // the previous chunk is consumed
        for (int e = tid; e < nk32 * CPR; e += 256) {
          const int row = e / CPR, c = e % CPR;
          u32x4 kr = {0u, 0u, 0u, 0u}, vr = {0u, 0u, 0u, 0u};
          if (row < nk) {
            const int64_t off = static_cast<int64_t>(kc + row) * D + 8 * c;
            kr = *reinterpret_cast<const u32x4*>(KS_ + off);
            vr = *reinterpret_cast<const u32x4*>(VS_ + off);
          }
          *reinterpret_cast<u32x4*>(k_lds + row * kKRow + 8 * c) = kr;
          *reinterpret_cast<u32x4*>(v_lds + row * kKRow + 8 * c) = vr;
        }
        __syncthreads();
        for (int kt = 0; kt < nk32; kt += kKeyTile) {
          const uint16_t* kl = k_lds + (kt + (lane & 31)) * kKRow + 8 * half;
          const uint16_t* vl = v_lds + (kt + (lane & 31)) * kKRow + 8 * half;
          f32x16 s = {}, dp = {};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128(kl + 16 * ks), qb[ks], s, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128(vl + 16 * ks), db[ks], dp, 0, 0, 0);
          }
          float pr[16], pd[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) pr[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c2, -l2));
          if (kt + kKeyTile > nk) {   // a partial last tile (uniform branch)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (kt + 8 * (r >> 2) + 4 * half + (r & 3) >= nk) pr[r] = 0.f;
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            pd[r] = pr[r] * dp[r];
            dl += pd[r];
          }
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const bf16x8 pdb = pack8(pd + 8 * ks);
            const bf16x8 pb = pack8(pr + 8 * ks);
#pragma unroll
            for (int vb = 0; vb < VB; ++vb) {
              const bf16x8 a = lds_tr_operand<kKRow>(k_lds + kt * kKRow, lane, vb, ks);
              aa[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pdb, aa[vb], 0, 0, 0);
              ab[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, ab[vb], 0, 0, 0);
            }
          }
        }
      }
      dl += __shfl_xor(dl, 32);
      if (valid) {
        const float gs = bf16_bits_to_f32(static_cast<const uint16_t*>(f.gates)[qrow * 3 + 2]) * f.scale;
        float* dst = p.dq_acc + qrow * D;
#pragma unroll
        for (int vb = 0; vb < VB; ++vb)
#pragma unroll
          for (int rb = 0; rb < 4; ++rb) {
            const int d = 32 * vb + 8 * rb + 4 * half;
            float4 o = *reinterpret_cast<const float4*>(dst + d);
            o.x = fmaf(gs, fmaf(-dl, ab[vb][4 * rb], aa[vb][4 * rb]), o.x);
            o.y = fmaf(gs, fmaf(-dl, ab[vb][4 * rb + 1], aa[vb][4 * rb + 1]), o.y);
            o.z = fmaf(gs, fmaf(-dl, ab[vb][4 * rb + 2], aa[vb][4 * rb + 2]), o.z);
            o.w = fmaf(gs, fmaf(-dl, ab[vb][4 * rb + 3], aa[vb][4 * rb + 3]), o.w);
            *reinterpret_cast<float4*>(dst + d) = o;
          }
        if (half == 0) {
          p.delta[2 * nrow + qrow] = dl;
          if (p.dgates) static_cast<uint16_t*>(p.dgates)[qrow * 3 + 2] = f32_to_bf16_bits(dl);
        }
      }
    }
  }
}

// ------------------------------------------------------------ token keys of the selected branch

constexpr int kSelBranch = 1;   // the selected branch's slot in lse / delta / gates

template <int D>
__global__ void __launch_bounds__(256, 2)
kv_grad_mfma_kernel(BwdParams p) {
  constexpr int KS = D / 16;
  constexpr int VB = D / 32;
  constexpr int kRowP = D + 8;                 // padded row of a gathered row tile (bf16)
  constexpr int kRT = kKeyTile * kRowP;
  constexpr int kTS = kKeyTile + 8;             // padded token row of a partial tile (floats)
  constexpr int kRed = D * kTS;                 // one partial tile, [dim][token] (floats)
  __shared__ __align__(16) uint16_t qr_lds[4 * kRT];   // per wave: its 32 gathered Q rows, row-major
  __shared__ __align__(16) uint16_t dr_lds[4 * kRT];   // per wave: dO rows
  __shared__ __align__(16) float st_lds[4 * 3 * kKeyTile];   // per wave: -lse2 / c2, -Delta, gate per row
  __shared__ float red_k[kRed];
  __shared__ float red_v[kRed];

  const FwdParams& f = p.f;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int half = lane >> 5;
  const int G = f.h_q / f.h_kv;
  const float c2 = f.scale * kLog2e;
  const int64_t nrow = static_cast<int64_t>(f.n) * f.h_q;
  const float* lse = p.lse + kSelBranch * nrow;
  const float* dlt = p.delta + kSelBranch * nrow;
  const uint16_t* Q = static_cast<const uint16_t*>(f.q);
  const uint16_t* dO = static_cast<const uint16_t*>(p.dout);
  const uint16_t* gates = static_cast<const uint16_t*>(f.gates);
  uint16_t* qr = qr_lds + wv * kRT;
  uint16_t* dr = dr_lds + wv * kRT;
  float* st = st_lds + wv * 3 * kKeyTile;
  const int n_units = f.counts[SSA_COUNT_NB];
  const int64_t n_items = static_cast<int64_t>(n_units) * f.h_kv;

  for (int64_t item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int g = static_cast<int>(item / n_units);
    const int u = static_cast<int>(item % n_units);
    const int64_t slot = static_cast<int64_t>(g) * f.nb_cap + u;
    const int e0 = p.sel_off[slot];
    const int R = (p.sel_off[slot + 1] - e0) * G;
    const int a = f.blk_off[u];
    const int bnd = f.blk_off[u + 1];
    if (R == 0) continue;
    const int n_rt = (R + kKeyTile - 1) / kKeyTile;
    for (int k0 = a; k0 < bnd; k0 += kKeyTile) {
      // B operands: the lane's key / value token of this tile
      const int i = k0 + (lane & 31);
      const bool iok = i < bnd;
      bf16x8 kb[KS], vb[KS];
      {
        const int64_t krow = (static_cast<int64_t>(g) * f.n + i) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
          if (iok) {
            x = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(f.k_s) + krow + 16 * ks + 8 * half);
            y = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(f.v_s) + krow + 16 * ks + 8 * half);
          }
          kb[ks] = __builtin_bit_cast(bf16x8, x);
          vb[ks] = __builtin_bit_cast(bf16x8, y);
        }
      }
      f32x16 dk[VB], dv[VB];
#pragma unroll
      for (int x = 0; x < VB; ++x) {
        dk[x] = f32x16{};
        dv[x] = f32x16{};
      }
      // rows of tile rt, prefetched one tile ahead: a row is CPR 16-byte
      // chunks, and load j of a lane moves chunk lane % CPR of row
      // j RPI + lane / CPR (so one load instruction covers RPI whole rows);
      // the row state is loaded by lanes 0..31, one row each
      constexpr int CPR = D / 8;
      constexpr int RPI = 64 / CPR;
      u32x4 nq[KS], nd[KS];
      // the row state: -lse2 / c2 and -Delta (the starting values of the S
      // and dP accumulators, so that they hold s - lse2 / c2 and dP - Delta)
      // and the gate
      float3 ns = make_float3(-FLT_MAX, 0.f, 0.f);
      auto load = [&](int rt) {
        const int r0 = rt * kKeyTile;
        const int rr = r0 + (lane & 31);
        int t = 0;
        ns = make_float3(-FLT_MAX, 0.f, 0.f);   // a missing row has P = 0
        if (half == 0 && rr < R) {
          t = p.sel_list[e0 + rr / G];
          const int64_t qrow = static_cast<int64_t>(t) * f.h_q + g * G + rr % G;
          ns = make_float3(-(lse[qrow] * kLog2e) / c2, -dlt[qrow], bf16_bits_to_f32(gates[qrow * 3 + kSelBranch]));
        }
#pragma unroll
        for (int j = 0; j < KS; ++j) {
          const int row = j * RPI + lane / CPR;
          const int tj = __shfl(t, row);
          nq[j] = nd[j] = u32x4{0u, 0u, 0u, 0u};
          if (r0 + row < R) {
            const int64_t qrow = static_cast<int64_t>(tj) * f.h_q + g * G + (r0 + row) % G;
            nq[j] = *reinterpret_cast<const u32x4*>(Q + qrow * D + 8 * (lane % CPR));
            nd[j] = *reinterpret_cast<const u32x4*>(dO + qrow * D + 8 * (lane % CPR));
          }
        }
      };
      if (wv < n_rt) load(wv);
      for (int rt = wv; rt < n_rt; rt += 4) {
        // the rows (row-major, 16-byte stores) and the row statistics,
        // wave-private; the operands, plain and transposed, are read back
#pragma unroll
        for (int j = 0; j < KS; ++j) {
          const int row = j * RPI + lane / CPR;
          *reinterpret_cast<u32x4*>(qr + row * kRowP + 8 * (lane % CPR)) = nq[j];
          *reinterpret_cast<u32x4*>(dr + row * kRowP + 8 * (lane % CPR)) = nd[j];
        }
        if (half == 0) {
          st[lane] = ns.x;
          st[kKeyTile + lane] = ns.y;
          st[2 * kKeyTile + lane] = ns.z;
        }
        wave_lds_sync();
        // entry r is row 8 (r / 4) + 4 half + r % 4 of the tile: rows
        // 8 q + 4 half .. + 3 of each quarter q are one 16-byte read
        f32x16 s, dp;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 a = *reinterpret_cast<const float4*>(st + 8 * q + 4 * half);
          const float4 b = *reinterpret_cast<const float4*>(st + kKeyTile + 8 * q + 4 * half);
          s[4 * q] = a.x; s[4 * q + 1] = a.y; s[4 * q + 2] = a.z; s[4 * q + 3] = a.w;
          dp[4 * q] = b.x; dp[4 * q + 1] = b.y; dp[4 * q + 2] = b.z; dp[4 * q + 3] = b.w;
        }
        const uint16_t* ql = qr + (lane & 31) * kRowP + 8 * half;
        const uint16_t* dl = dr + (lane & 31) * kRowP + 8 * half;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128(ql + 16 * ks), kb[ks], s, 0, 0, 0);
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128(dl + 16 * ks), vb[ks], dp, 0, 0, 0);
        }
        if (rt + 4 < n_rt) load(rt + 4);   // in flight during the rest of this tile
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          float pg[8], ds[8], gt[8];
          *reinterpret_cast<float4*>(gt) = *reinterpret_cast<const float4*>(st + 2 * kKeyTile + 16 * ks + 4 * half);
          *reinterpret_cast<float4*>(gt + 4) = *reinterpret_cast<const float4*>(st + 2 * kKeyTile + 16 * ks + 8 + 4 * half);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int r = 8 * ks + i;
            const float x = gt[i] * __builtin_amdgcn_exp2f(s[r] * c2);
            pg[i] = x;
            ds[i] = x * dp[r];
          }
          const bf16x8 pb = pack8(pg);
          const bf16x8 sb = pack8(ds);
#pragma unroll
          for (int x = 0; x < VB; ++x) {
            dv[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_tr_operand<kRowP>(dr, lane, x, ks), pb, dv[x], 0, 0, 0);
            dk[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_tr_operand<kRowP>(qr, lane, x, ks), sb, dk[x], 0, 0, 0);
          }
        }
        wave_lds_sync();  // the wave-private area is rewritten by the next row tile
      }
      // sum the four waves' partial tiles, [dim][token], in wave order (a
      // fixed order keeps the result identical from run to run); a lane
      // half's 32 tokens are 32 consecutive banks and the two halves' rows
      // (4 dims apart, 4 kTS = 32 mod 64 floats) the other 32
      for (int w = 0; w < 4; ++w) {
        __syncthreads();
        if (wv == w) {
#pragma unroll
          for (int x = 0; x < VB; ++x)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int e = (32 * x + 8 * (r >> 2) + 4 * half + (r & 3)) * kTS + (lane & 31);
              red_k[e] = w == 0 ? dk[x][r] : red_k[e] + dk[x][r];
              red_v[e] = w == 0 ? dv[x][r] : red_v[e] + dv[x][r];
            }
        }
      }
      __syncthreads();
      // add to the token rows (the window branch wrote them first)
      const int n_tok = min(kKeyTile, bnd - k0);
      for (int e = tid; e < n_tok * (D / 4); e += 256) {
        const int tok = e / (D / 4), d = 4 * (e % (D / 4));
        const int64_t o = (static_cast<int64_t>(g) * f.n + k0 + tok) * D + d;
        const float* pk = red_k + d * kTS + tok;
        const float* pv = red_v + d * kTS + tok;
        float4 rk = make_float4(f.scale * pk[0], f.scale * pk[kTS], f.scale * pk[2 * kTS], f.scale * pk[3 * kTS]);
        float4 rv = make_float4(pv[0], pv[kTS], pv[2 * kTS], pv[3 * kTS]);
        const float4 ck = *reinterpret_cast<const float4*>(p.dk_acc + o);
        const float4 cv = *reinterpret_cast<const float4*>(p.dv_acc + o);
        rk.x += ck.x; rk.y += ck.y; rk.z += ck.z; rk.w += ck.w;
        rv.x += cv.x; rv.y += cv.y; rv.z += cv.z; rv.w += cv.w;
        *reinterpret_cast<float4*>(p.dk_acc + o) = rk;
        *reinterpret_cast<float4*>(p.dv_acc + o) = rv;
      }
      __syncthreads();  // the reduction buffers are reused by the next tile
    }
  }
}

}  // namespace

hipError_t launch_bwd_kv_sel_mfma(const BwdParams& p, ssa_dtype /*dtype*/, hipStream_t stream) {
  if (p.f.d == 32) kv_grad_mfma_kernel<32><<<8192, 256, 0, stream>>>(p);
  else kv_grad_mfma_kernel<64><<<8192, 256, 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_bwd_kv_win_mfma(const BwdParams& p, ssa_dtype /*dtype*/, hipStream_t stream) {
  if (p.f.d == 32) win_dkv_mfma_kernel<32><<<4096, 256, 0, stream>>>(p);
  else win_dkv_mfma_kernel<64><<<4096, 256, 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_bwd_rows_prep(const BwdParams& p, ssa_dtype /*dtype*/, hipStream_t stream) {
  const int64_t G = p.f.h_q / p.f.h_kv;
  const int64_t tiles = ((p.rows_cap + G - 1) / G + kKeyTile - 1) / kKeyTile;
  const int grid = static_cast<int>(std::min<int64_t>(tiles, 8192));
  if (p.f.d == 32) rows_prep_kernel<32><<<grid, 256, 0, stream>>>(p);
  else rows_prep_kernel<64><<<grid, 256, 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_bwd_win_dq_mfma(const BwdParams& p, ssa_dtype /*dtype*/, hipStream_t stream) {
  if (p.f.d == 32) win_dq_mfma_kernel<32><<<4096, 256, 0, stream>>>(p);
  else win_dq_mfma_kernel<64><<<4096, 256, 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_bwd_cmp_dq_mfma(const BwdParams& p, ssa_dtype /*dtype*/, hipStream_t stream) {
  bwd_tile_prefix_kernel<<<1, 256, 0, stream>>>(p);
  const dim3 grid(p.max_qtiles, p.f.h_q);
  if (p.f.d == 32) cmp_dq_mfma_kernel<32><<<grid, 256, 0, stream>>>(p);
  else cmp_dq_mfma_kernel<64><<<grid, 256, 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_bwd_cmp_dkv_mfma(const BwdParams& p, ssa_dtype /*dtype*/, hipStream_t stream) {
  const int grid = p.max_btiles * p.f.h_kv * p.row_splits;
  if (p.f.d == 32) cmp_dkv_mfma_kernel<32><<<grid, 256, 0, stream>>>(p);
  else cmp_dkv_mfma_kernel<64><<<grid, 256, 0, stream>>>(p);
  if (p.row_splits > 1) {
    const int64_t n4 = static_cast<int64_t>(p.f.h_kv) * p.f.nb_cap * p.f.d / 4;
    dkv_split_sum_kernel<<<static_cast<int>(std::min<int64_t>((n4 + 255) / 256, 8192)), 256, 0, stream>>>(p);
  }
  return hipGetLastError();
}

}  // namespace ssa
