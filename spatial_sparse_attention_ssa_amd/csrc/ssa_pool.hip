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

// Position of key jj (0..31) of a 32-key tile in the MFMA operand order: the
// 32x32 accumulator gives lane group 0 the keys {0-3, 8-11} and lane group 1
// the keys {4-7, 12-15} of each 16-key half; the permutation is its own
// inverse.
__device__ __forceinline__ int mfma_key_pos(int jj) {
  const int lo = jj & 15;
  const int perm = (lo & 3) | ((lo & 4) << 1) | ((lo & 8) >> 1);
  return (jj & 16) | perm;
}

template <typename T>
__device__ __forceinline__ void store_vt(T* vt, int d, int nb_cap, int g, int j, int dd, float4 s) {
  if (!vt) return;
  const int64_t tile = static_cast<int64_t>(g) * (nb_cap / kKeyTile) + j / kKeyTile;
  T* base = vt + tile * d * kKeyTile + mfma_key_pos(j % kKeyTile);
  const float x[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) Elt<T>::store(base + (dd + e) * kKeyTile, x[e]);
}

template <typename T>
__global__ void __launch_bounds__(256)
pool_kernel(const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ perm,
            const int32_t* __restrict__ blk_off, const int32_t* __restrict__ counts, int hkv, int d,
            int nb_cap, T* __restrict__ kbar, T* __restrict__ vbar, T* __restrict__ vbar_t,
            T* __restrict__ k_cmp, T* __restrict__ v_cmp) {
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
          if (which) store_vt(vbar_t, d, nb_cap, g, j, dd, s);
          T* pub = which ? v_cmp : k_cmp;
          if (pub) store4(pub + static_cast<int64_t>(j) * e_per_tok + e, s);
        }
        __syncthreads();
      }
    }
  }
  // zero the rows between nb and nb_cap so padded key tiles hold finite values
  const int pad_rows = nb_cap - nb;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
       i < static_cast<int64_t>(hkv) * pad_rows * d; i += static_cast<int64_t>(gridDim.x) * 256) {
    const int g = static_cast<int>(i / (static_cast<int64_t>(pad_rows) * d));
    const int rem = static_cast<int>(i % (static_cast<int64_t>(pad_rows) * d));
    const int j = nb + rem / d, dd = rem % d;
    const int64_t row = (static_cast<int64_t>(g) * nb_cap + j) * d + dd;
    kbar[row] = T(0);
    vbar[row] = T(0);
    if (vbar_t) {
      const int64_t tile = static_cast<int64_t>(g) * (nb_cap / kKeyTile) + j / kKeyTile;
      vbar_t[(tile * d + dd) * kKeyTile + mfma_key_pos(j % kKeyTile)] = T(0);
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
        static_cast<uint16_t*>(p.vbar), static_cast<uint16_t*>(p.vbar_t),
        static_cast<uint16_t*>(p.k_cmp), static_cast<uint16_t*>(p.v_cmp));
  } else {
    pool_kernel<float><<<grid, 256, 0, stream>>>(
        static_cast<const float*>(p.k), static_cast<const float*>(p.v), p.perm, p.blk_off,
        p.counts, p.h_kv, p.d, p.nb_cap, static_cast<float*>(p.kbar), static_cast<float*>(p.vbar),
        static_cast<float*>(p.vbar_t), static_cast<float*>(p.k_cmp), static_cast<float*>(p.v_cmp));
  }
  return hipGetLastError();
}

}  // namespace ssa
