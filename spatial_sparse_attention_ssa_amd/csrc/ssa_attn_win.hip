// Window attention on MFMA (bf16, D = 64): every query attends to all tokens
// of its own m_win^3 window (Direct3D-S2 page, "Method": the sparse 3D window
// module splits tokens into non-overlapping windows and runs self-attention
// inside each).  Adds G2 * o_win to the branch accumulator.
//
// Work split: the same 128-query tiles of sorted tokens as the compressed
// kernel; each wave owns 32 consecutive sorted queries.  Windows are
// contiguous runs of sorted positions, so the keys of every window touching
// the wave's queries form one contiguous range; the wave streams it in tiles
// of 32 tokens (gathered through perm into its own LDS), computes
// S^T = K Q^T with v_mfma_f32_32x32x16_bf16, masks keys outside each query's
// window, and keeps an online softmax (running max, rescaled sum and O^T).
#include <float.h>

#include "ssa_internal.h"

namespace ssa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kD = 64;
constexpr int kKRow = kD + 8;
constexpr int kVRow = kKeyTile + 8;

__device__ __forceinline__ bf16x8 lds_b128(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ int mfma_key_pos(int jj) {
  const int lo = jj & 15;
  return (jj & 16) | (lo & 3) | ((lo & 4) << 1) | ((lo & 8) >> 1);
}

// last window id w in [lo, hi] with win_off[w] <= pos
__device__ __forceinline__ int window_of(const int32_t* win_off, int pos, int lo, int hi) {
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (win_off[mid] <= pos) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ void __launch_bounds__(256, 2)
win_mfma_kernel(FwdParams p) {
  __shared__ __align__(16) uint16_t k_lds[4][kKeyTile * kKRow];
  __shared__ __align__(16) uint16_t v_lds[4][kD * kVRow];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int h = blockIdx.y;
  const int tile = blockIdx.x;
  if (tile >= p.tile_pre[p.batch]) return;

  int lo = 0, hi = p.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.tile_pre[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const int w_seq0 = p.seq_win_off[b], w_seq1 = p.seq_win_off[b + 1];
  const int s0 = p.win_off[w_seq0], s1 = p.win_off[w_seq1];
  const int q_begin = s0 + (tile - p.tile_pre[b]) * kQueryTile + wv * 32;
  const int q_end = min(q_begin + 32, s1);
  if (q_begin >= q_end) return;  // this wave has no queries (waves never sync with each other)

  const int half = lane >> 5;
  const int qi = q_begin + (lane & 31);
  const bool q_valid = qi < q_end;
  const int t = q_valid ? p.perm[qi] : 0;
  // this query's window, and the key range of all windows the wave touches
  const int wq = window_of(p.win_off, q_valid ? qi : q_begin, w_seq0, w_seq1 - 1);
  const int wa = p.win_off[wq], wb = p.win_off[wq + 1];
  const int w_first = window_of(p.win_off, q_begin, w_seq0, w_seq1 - 1);
  const int w_last = window_of(p.win_off, q_end - 1, w_seq0, w_seq1 - 1);
  const int ka = p.win_off[w_first], kb = p.win_off[w_last + 1];

  const uint16_t* Q = static_cast<const uint16_t*>(p.q);
  const uint16_t* K = static_cast<const uint16_t*>(p.k);
  const uint16_t* V = static_cast<const uint16_t*>(p.v);
  bf16x8 qb[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    u32x4 u = {0u, 0u, 0u, 0u};
    if (q_valid)
      u = *reinterpret_cast<const u32x4*>(Q + (static_cast<int64_t>(t) * p.h_q + h) * kD + 16 * ks + 8 * half);
    qb[ks] = __builtin_bit_cast(bf16x8, u);
  }

  uint16_t* kl = k_lds[wv];
  uint16_t* vl = v_lds[wv];
  const float c2 = p.scale * kLog2e;
  float m = -FLT_MAX, l = 0.f;
  f32x16 o0 = {}, o1 = {};
  // staging: lane -> key row (lane / 2) of the tile, 4 chunks of 8 dims
  const int srow = lane >> 1, schunk0 = (lane & 1) * 4;
  for (int base = ka; base < kb; base += kKeyTile) {
    const int pos = base + srow;
    u32x4 kr[4], vr[4];
    if (pos < kb) {
      const int64_t tok = p.perm[pos];
      const uint16_t* krow = K + (tok * p.h_kv + h) * kD;
      const uint16_t* vrow = V + (tok * p.h_kv + h) * kD;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        kr[c] = *reinterpret_cast<const u32x4*>(krow + 8 * (schunk0 + c));
        vr[c] = *reinterpret_cast<const u32x4*>(vrow + 8 * (schunk0 + c));
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) kr[c] = vr[c] = u32x4{0u, 0u, 0u, 0u};
    }
    wave_lds_sync();  // previous tile fully consumed by this wave
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      *reinterpret_cast<u32x4*>(kl + srow * kKRow + 8 * (schunk0 + c)) = kr[c];
      const int kp = mfma_key_pos(srow);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = 8 * (schunk0 + c) + 2 * e;
        vl[d * kVRow + kp] = static_cast<uint16_t>(vr[c][e] & 0xFFFFu);
        vl[(d + 1) * kVRow + kp] = static_cast<uint16_t>(vr[c][e] >> 16);
      }
    }
    wave_lds_sync();
    f32x16 s = {};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 a = lds_b128(kl + (lane & 31) * kKRow + 16 * ks + 8 * half);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[ks], s, 0, 0, 0);
    }
    float tmax = -FLT_MAX;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kp = base + 8 * (r >> 2) + 4 * half + (r & 3);
      if (kp < wa || kp >= wb) s[r] = -FLT_MAX;
      tmax = fmaxf(tmax, s[r]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m, tmax);
    const float corr = __builtin_amdgcn_exp2f((m - m_new) * c2);
    const float mc = m_new * c2;
    m = m_new;
    float pr[16];
    float ls = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      pr[r] = (s[r] == -FLT_MAX) ? 0.f : __builtin_amdgcn_exp2f(fmaf(s[r], c2, -mc));
      ls += pr[r];
    }
    l = l * corr + ls;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      o0[r] *= corr;
      o1[r] *= corr;
    }
    bf16x8 pb[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[ks][i] = static_cast<__bf16>(pr[8 * ks + i]);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 a0 = lds_b128(vl + (lane & 31) * kVRow + 16 * ks + 8 * half);
      const bf16x8 a1 = lds_b128(vl + (32 + (lane & 31)) * kVRow + 16 * ks + 8 * half);
      o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, pb[ks], o0, 0, 0, 0);
      o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, pb[ks], o1, 0, 0, 0);
    }
  }
  const float l_q = l + __shfl_xor(l, 32);
  if (q_valid) {
    const uint16_t* gt = static_cast<const uint16_t*>(p.gates) + (static_cast<int64_t>(t) * p.h_q + h) * 3;
    const float f = bf16_bits_to_f32(gt[2]) / l_q;
    float* dst = p.acc + (static_cast<int64_t>(t) * p.h_q + h) * kD;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int d = 8 * rb + 4 * half;
      float4 a = *reinterpret_cast<float4*>(dst + d);
      a.x += o0[4 * rb] * f; a.y += o0[4 * rb + 1] * f; a.z += o0[4 * rb + 2] * f; a.w += o0[4 * rb + 3] * f;
      *reinterpret_cast<float4*>(dst + d) = a;
      float4 c = *reinterpret_cast<float4*>(dst + 32 + d);
      c.x += o1[4 * rb] * f; c.y += o1[4 * rb + 1] * f; c.z += o1[4 * rb + 2] * f; c.w += o1[4 * rb + 3] * f;
      *reinterpret_cast<float4*>(dst + 32 + d) = c;
    }
  }
}

}  // namespace

hipError_t launch_win_mfma(const FwdParams& p, ssa_dtype /*dtype*/, hipStream_t stream) {
  win_mfma_kernel<<<dim3(p.max_tiles, p.h_q), 256, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace ssa
