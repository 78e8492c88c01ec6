// Compression: mean pooling of keys and values over each block's tokens.
//
// Direct3D-S2 page, "Method": keys and values of every m_cmp^3 block are
// compressed into one block-level token by mean pooling (the learned sparse
// convolution before the pooling is not part of this path); LSRM article,
// "Stage 2": average pooling inside each spatial block.  The mean runs over
// the block's occupied tokens, accumulates in float32 in sorted-token order and
// is rounded once to the input dtype.
//
// One workgroup per block (grid-stride over the device-side block count).
// Threads split a token row (h_kv * D elements, contiguous in HBM) into
// 4-element chunks; when a row has fewer than 256 chunks, several token
// slots run in parallel and are summed in slot order through LDS, so the
// result is deterministic.
#include "ssa_internal.h"

namespace ssa {
namespace {

__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4(const uint16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
}
__device__ __forceinline__ void store4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
__device__ __forceinline__ void store4(uint16_t* p, float4 v) {
  uint2 u;
  u.x = static_cast<uint32_t>(f32_to_bf16_bits(v.x)) | (static_cast<uint32_t>(f32_to_bf16_bits(v.y)) << 16);
  u.y = static_cast<uint32_t>(f32_to_bf16_bits(v.z)) | (static_cast<uint32_t>(f32_to_bf16_bits(v.w)) << 16);
  *reinterpret_cast<uint2*>(p) = u;
}

template <typename T>
__global__ void __launch_bounds__(256)
pool_kernel(const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ perm,
            const int32_t* __restrict__ blk_off, const int32_t* __restrict__ counts, int hkv, int d,
            int nb_cap, T* __restrict__ kbar, T* __restrict__ vbar, T* __restrict__ k_cmp,
            T* __restrict__ v_cmp) {
  __shared__ float4 red[256];
  const int e_per_tok = hkv * d;
  const int c_per_tok = e_per_tok / 4;                 // 4-element chunks per row
  const int tpt = c_per_tok < 256 ? c_per_tok : 256;  // threads per token row
  const int slots = 256 / tpt;
  const int slot = threadIdx.x / tpt;
  const int lc = threadIdx.x % tpt;
  const int nb = counts[SSA_COUNT_NB];
  for (int j = blockIdx.x; j < nb; j += gridDim.x) {
    const int a = blk_off[j], b = blk_off[j + 1];
    const float cnt = static_cast<float>(b - a);
    for (int c0 = 0; c0 < c_per_tok; c0 += tpt) {
      const int c = c0 + lc;
      for (int which = 0; which < 2; ++which) {
        const T* src = which ? v : k;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        if (slot < slots && c < c_per_tok) {
          for (int p = a + slot; p < b; p += slots) {
            const float4 x = load4(src + static_cast<int64_t>(perm[p]) * e_per_tok + 4 * c);
            acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
          }
        }
        red[threadIdx.x] = acc;
        __syncthreads();
        if (slot == 0 && c < c_per_tok) {
          float4 s = red[lc];
          for (int q = 1; q < slots; ++q) {
            const float4 y = red[q * tpt + lc];
            s.x += y.x; s.y += y.y; s.z += y.z; s.w += y.w;
          }
          s.x = s.x / cnt; s.y = s.y / cnt; s.z = s.z / cnt; s.w = s.w / cnt;
          const int e = 4 * c;
          const int g = e / d, dd = e % d;
          T* dst = which ? vbar : kbar;
          store4(dst + (static_cast<int64_t>(g) * nb_cap + j) * d + dd, s);
          T* pub = which ? v_cmp : k_cmp;
          if (pub) store4(pub + static_cast<int64_t>(j) * e_per_tok + e, s);
        }
        __syncthreads();
      }
    }
  }
}

}  // namespace

hipError_t launch_pool(const FwdParams& p, ssa_dtype dtype, hipStream_t stream) {
  const int grid = p.nb_cap < 16384 ? (p.nb_cap > 0 ? p.nb_cap : 1) : 16384;
  if (dtype == SSA_BF16) {
    pool_kernel<uint16_t><<<grid, 256, 0, stream>>>(
        static_cast<const uint16_t*>(p.k), static_cast<const uint16_t*>(p.v), p.perm, p.blk_off,
        p.counts, p.h_kv, p.d, p.nb_cap, static_cast<uint16_t*>(p.kbar),
        static_cast<uint16_t*>(p.vbar), static_cast<uint16_t*>(p.k_cmp),
        static_cast<uint16_t*>(p.v_cmp));
  } else {
    pool_kernel<float><<<grid, 256, 0, stream>>>(
        static_cast<const float*>(p.k), static_cast<const float*>(p.v), p.perm, p.blk_off,
        p.counts, p.h_kv, p.d, p.nb_cap, static_cast<float*>(p.kbar), static_cast<float*>(p.vbar),
        static_cast<float*>(p.k_cmp), static_cast<float*>(p.v_cmp));
  }
  return hipGetLastError();
}

}  // namespace ssa
