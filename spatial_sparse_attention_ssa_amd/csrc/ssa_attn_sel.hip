// Selected-block attention and the gated sum (bf16, D = 64, one query head
// per key/value head).
//
// Direct3D-S2 page, "Method": all tokens of the top-k selected blocks take
// part in a second attention; the three branch outputs are summed with the
// predicted gates.  The compressed and window branches have already added
// G0 * o_cmp + G2 * o_win to the float32 accumulator; this kernel adds
// G1 * o_sel, rounds once to bfloat16 and writes the output row.
//
// Four lanes serve one (token, head) pair, each owning 16 of the 64 dims; a
// wave covers 16 tokens of one head.  Pairs are ordered head-major, so the
// workgroups running at any time gather from one or two heads' key/value
// rows (32 MB per head at 131072 tokens), which stay in the MI355X's
// 256 MB Infinity Cache instead of streaming all heads from HBM.  The lanes
// walk the selected blocks' token runs (contiguous in sorted order) gathering
// key and value rows through perm, with an online softmax per pair.
#include <float.h>

#include "ssa_internal.h"

namespace ssa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kD = 64;
constexpr int kDL = 16;  // dims per lane

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

__global__ void __launch_bounds__(256)
sel_combine_kernel(FwdParams p) {
  const int lane = threadIdx.x & 63;
  const int sub = lane & 3;                       // which 16 dims
  const int64_t pair = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) >> 2;
  const int64_t n_pairs = static_cast<int64_t>(p.n) * p.h_q;
  const bool active0 = pair < n_pairs;
  const int h = active0 ? static_cast<int>(pair / p.n) : 0;
  const int t = active0 ? static_cast<int>(pair % p.n) : 0;      // input token order
  const int g = h;  // one query head per group on this path

  const uint16_t* Q = static_cast<const uint16_t*>(p.q);
  const uint16_t* K = static_cast<const uint16_t*>(p.k);
  const uint16_t* V = static_cast<const uint16_t*>(p.v);
  const float c2 = p.scale * kLog2e;

  float q[kDL];
  load16(Q + (static_cast<int64_t>(t) * p.h_q + h) * kD + kDL * sub, q);
  const int32_t* sel = p.topk_idx + (static_cast<int64_t>(t) * p.h_kv + g) * p.topk;

  // walk state: selection slot r, current sorted position and block end.
  // Block ids outside [0, nb) end the walk (they never occur in valid output
  // of the selection kernels; the check keeps a corrupt list memory-safe).
  const int nb = p.counts[SSA_COUNT_NB];
  int r = 0, pos = 0, end = 0;
  bool active = active0;
  if (active) {
    const int j = sel[0];
    if (j < 0 || j >= nb) active = false;
    else { pos = p.blk_off[j]; end = p.blk_off[j + 1]; active = pos < end; }
  }
  float m = -FLT_MAX, l = 0.f, o[kDL];
#pragma unroll
  for (int e = 0; e < kDL; ++e) o[e] = 0.f;
  while (__ballot(active)) {
    float kx[kDL], vx[kDL];
    float s = 0.f;
    if (active) {
      const int64_t tok = p.perm[pos];
      load16(K + (tok * p.h_kv + g) * kD + kDL * sub, kx);
      load16(V + (tok * p.h_kv + g) * kD + kDL * sub, vx);
#pragma unroll
      for (int e = 0; e < kDL; ++e) s = fmaf(q[e], kx[e], s);
    }
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    if (active) {
      const float s2 = s * c2;
      if (s2 > m) {
        const float corr = __builtin_amdgcn_exp2f(m - s2);
        l *= corr;
#pragma unroll
        for (int e = 0; e < kDL; ++e) o[e] *= corr;
        m = s2;
      }
      const float pr = __builtin_amdgcn_exp2f(s2 - m);
      l += pr;
#pragma unroll
      for (int e = 0; e < kDL; ++e) o[e] = fmaf(pr, vx[e], o[e]);
      if (++pos >= end) {
        ++r;
        const int j = r < p.topk ? sel[r] : -1;
        if (j < 0 || j >= nb) active = false;
        else { pos = p.blk_off[j]; end = p.blk_off[j + 1]; active = pos < end; }
      }
    }
  }
  if (!active0) return;
  const int64_t row = (static_cast<int64_t>(t) * p.h_q + h) * kD + kDL * sub;
  const uint16_t* gt = static_cast<const uint16_t*>(p.gates) + (static_cast<int64_t>(t) * p.h_q + h) * 3;
  const float f = bf16_bits_to_f32(gt[1]) / l;
  const float* acc = p.acc + row;
  uint16_t res[kDL];
#pragma unroll
  for (int c = 0; c < kDL / 4; ++c) {
    const float4 a = *reinterpret_cast<const float4*>(acc + 4 * c);
    res[4 * c] = f32_to_bf16_bits(fmaf(o[4 * c], f, a.x));
    res[4 * c + 1] = f32_to_bf16_bits(fmaf(o[4 * c + 1], f, a.y));
    res[4 * c + 2] = f32_to_bf16_bits(fmaf(o[4 * c + 2], f, a.z));
    res[4 * c + 3] = f32_to_bf16_bits(fmaf(o[4 * c + 3], f, a.w));
  }
  u32x4 w0, w1;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    w0[e] = static_cast<uint32_t>(res[2 * e]) | (static_cast<uint32_t>(res[2 * e + 1]) << 16);
    w1[e] = static_cast<uint32_t>(res[8 + 2 * e]) | (static_cast<uint32_t>(res[8 + 2 * e + 1]) << 16);
  }
  uint16_t* out = static_cast<uint16_t*>(p.out) + row;
  *reinterpret_cast<u32x4*>(out) = w0;
  *reinterpret_cast<u32x4*>(out + 8) = w1;
}

}  // namespace

hipError_t launch_sel_combine(const FwdParams& p, ssa_dtype /*dtype*/, hipStream_t stream) {
  const int64_t threads = static_cast<int64_t>(p.n) * p.h_q * 4;
  sel_combine_kernel<<<static_cast<int>((threads + 255) / 256), 256, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace ssa
