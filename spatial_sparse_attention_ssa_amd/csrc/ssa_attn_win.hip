// Window attention (bf16, D = 32 or 64; query head h reads key/value head
// h / (h_q / h_kv)).
//
// Direct3D-S2 page, "Method": every query attends to all tokens of its own
// m_win^3 window (the windows do not overlap).  Writes G2 * o_win to the
// float32 branch accumulator: every token lies in exactly one window, so this
// kernel runs first and the other branches add to what it wrote.
//
// Work split: one workgroup per (window, head) item (persistent grid, items
// head-major).  Keys and values come from the head-major sorted copies made by
// the pooling kernel, so a window is one contiguous run of rows.  The
// workgroup stages the window's key and value rows (row-major, 16-byte
// stores) in LDS, in chunks of up to 128 tokens; each of its 4 waves
// computes 32 queries with v_mfma_f32_32x32x16_bf16 (S^T = K Q^T over 32-key
// tiles), an online softmax (running max, rescaled sum and O^T), and
// O^T += V^T P^T with the V^T operands read through the transposing LDS load.
#include <float.h>

#include "ssa_internal.h"

namespace ssa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
// window tokens staged in LDS at a time: 128 (about the mean window size)
// keeps the LDS of four workgroups per compute unit within its 160 KB, twice
// the occupancy of 256-token chunks; larger windows take several chunks
constexpr int kChunk = 128;

__device__ __forceinline__ bf16x8 lds_b128(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

template <int D>
__global__ void __launch_bounds__(256, 4)
win_mfma_kernel(FwdParams p) {
  constexpr int kD = D;
  constexpr int KSTEPS = D / 16;         // MFMA k steps over the dims
  constexpr int VB = D / 32;             // 32-dim row blocks of O^T
  constexpr int CPR = D / 8;             // 16-byte chunks per row
  constexpr int kKRow = kD + 8;          // padded key row (bf16)
  __shared__ __align__(16) uint16_t k_lds[kChunk * kKRow];
  __shared__ __align__(16) uint16_t v_lds[kChunk * kKRow];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int half = lane >> 5;
  const uint16_t* Q = static_cast<const uint16_t*>(p.q);
  const float c2 = p.scale * kLog2e;
  const int nw = p.counts[SSA_COUNT_NW];
  const int64_t n_items = static_cast<int64_t>(nw) * p.h_q;
  for (int64_t item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int h = static_cast<int>(item / nw);
    const int w = static_cast<int>(item % nw);
    const int wa = p.win_off[w], wb = p.win_off[w + 1];
    const int n_w = wb - wa;
    const int kvh = h / (p.h_q / p.h_kv);
    const uint16_t* KS = static_cast<const uint16_t*>(p.k_s) + static_cast<int64_t>(kvh) * p.n * kD;
    const uint16_t* VS = static_cast<const uint16_t*>(p.v_s) + static_cast<int64_t>(kvh) * p.n * kD;

    // 128 queries per group round (32 per wave); every key chunk is staged
    // once per group round, so windows of up to 128 tokens are staged exactly
    // once
    for (int qg0 = 0; qg0 < n_w; qg0 += 128) {
      const int qi = wa + qg0 + wv * 32 + (lane & 31);
      const bool q_valid = qi < wb;
      // a wave whose 32 queries all lie past the window's end only helps to
      // stage the chunks (uniform over the wave)
      const bool wave_live = wa + qg0 + wv * 32 < wb;
      const int t = q_valid ? p.perm[qi] : 0;
      const uint16_t* q_row = Q + (static_cast<int64_t>(t) * p.h_q + h) * kD;
      bf16x8 qb[KSTEPS];
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        u32x4 u = {0u, 0u, 0u, 0u};
        if (q_valid) u = *reinterpret_cast<const u32x4*>(q_row + 16 * ks + 8 * half);
        qb[ks] = __builtin_bit_cast(bf16x8, u);
      }

      // ---------------- window attention
      float m = -FLT_MAX, l = 0.f;
      f32x16 o[VB];
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) o[vb] = f32x16{};
      for (int kc = 0; kc < n_w; kc += kChunk) {
        const int nk = min(kChunk, n_w - kc);
        const int nk32 = (nk + 31) & ~31;
        __syncthreads();  // previous chunk fully consumed
        // stage the keys and values of this chunk (row-major)
        for (int e = tid; e < nk32 * CPR; e += 256) {
          const int row = e / CPR, c = e % CPR;
          u32x4 kr = {0u, 0u, 0u, 0u}, vr = {0u, 0u, 0u, 0u};
          if (row < nk) {
            const int64_t off = static_cast<int64_t>(wa + kc + row) * kD + 8 * c;
            kr = *reinterpret_cast<const u32x4*>(KS + off);
            vr = *reinterpret_cast<const u32x4*>(VS + off);
          }
          *reinterpret_cast<u32x4*>(k_lds + row * kKRow + 8 * c) = kr;
          *reinterpret_cast<u32x4*>(v_lds + row * kKRow + 8 * c) = vr;
        }
        __syncthreads();
        for (int kt = 0; wave_live && kt < nk32; kt += kKeyTile) {
          f32x16 s = {};
#pragma unroll
          for (int ks = 0; ks < KSTEPS; ++ks) {
            const bf16x8 a = lds_b128(k_lds + (kt + (lane & 31)) * kKRow + 16 * ks + 8 * half);
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[ks], s, 0, 0, 0);
          }
          if (kt + kKeyTile > nk) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (kt + 8 * (r >> 2) + 4 * half + (r & 3) >= nk) s[r] = -FLT_MAX;
          }
          float tmax = -FLT_MAX;
#pragma unroll
          for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[r]);
          tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
          const float m_new = fmaxf(m, tmax);
          const float corr = __builtin_amdgcn_exp2f((m - m_new) * c2);
          const float mc = m_new * c2;
          m = m_new;
          float pr[16];
          float ls = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            pr[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c2, -mc));
            ls += pr[r];
          }
          l = l * corr + ls;
#pragma unroll
          for (int vb = 0; vb < VB; ++vb)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[vb][r] *= corr;
          bf16x8 pb[2];
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int i = 0; i < 8; ++i) pb[ks][i] = static_cast<__bf16>(pr[8 * ks + i]);
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int vb = 0; vb < VB; ++vb)
              o[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_tr_operand<kKRow>(v_lds + kt * kKRow, lane, vb, ks),
                                                              pb[ks], o[vb], 0, 0, 0);
          }
        }
      }
      const float l_win = l + __shfl_xor(l, 32);
      if (q_valid) {
        const int64_t row = static_cast<int64_t>(t) * p.h_q + h;
        const uint16_t* gt = static_cast<const uint16_t*>(p.gates) + row * 3;
        const float f = bf16_bits_to_f32(gt[2]) / l_win;
        float* dst = p.acc + row * kD;
#pragma unroll
        for (int vb = 0; vb < VB; ++vb)
#pragma unroll
          for (int rb = 0; rb < 4; ++rb) {
            const int d = 32 * vb + 8 * rb + 4 * half;
            *reinterpret_cast<float4*>(dst + d) = make_float4(o[vb][4 * rb] * f, o[vb][4 * rb + 1] * f,
                                                              o[vb][4 * rb + 2] * f, o[vb][4 * rb + 3] * f);
          }
        if (p.lse && half == 0)
          p.lse[2 * static_cast<int64_t>(p.n) * p.h_q + row] = (m * c2 + __log2f(l_win)) * kLn2;
      }
    }
  }
}

}  // namespace

hipError_t launch_win_mfma(const FwdParams& p, ssa_dtype /*dtype*/, hipStream_t stream) {
  // persistent grid over (window, head) items; the window count is read on
  // the device, so the grid does not depend on it
  if (p.d == 32) win_mfma_kernel<32><<<4096, 256, 0, stream>>>(p);
  else win_mfma_kernel<64><<<4096, 256, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace ssa
