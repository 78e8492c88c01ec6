// Compression: mean pooling of keys and values over each block's tokens.
//
// Direct3D-S2 page, "Method": keys and values of every m_cmp^3 block are
// compressed into one block-level token by mean pooling (the learned sparse
// convolution before the pooling is not part of this path); LSRM article,
// "Stage 2": average pooling inside each spatial block.  The mean runs over
// the block's occupied tokens, accumulates in float32 in sorted-token order and
// is rounded once to the input dtype.
//
// pool_kernel: one workgroup per block (grid-stride over the device-side
// block count).  On the MFMA path it also writes the key and value rows in
// sorted order, head-major, for the window and selection kernels, and the
// squared norm of every pooled key row (of its bfloat16 values), from which
// the compressed kernel's probe set is chosen.  A token row (h_kv * D elements, contiguous in HBM) is split
// into 16-byte chunks, one per thread; rows with fewer than 256 chunks run
// several token slots side by side, summed afterwards in slot order through
// LDS (deterministic).  Each thread keeps four row loads in flight.
//
// vt_transpose_kernel: rewrites the pooled values of every 32-block tile as
// [D][32 blocks], blocks in the order the MFMA kernels' P^T operand uses.
#include <type_traits>

#include "ssa_internal.h"

namespace ssa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct Chunk;
template <> struct Chunk<uint16_t> {
  static constexpr int kN = 8;
  static __device__ __forceinline__ void add(float (&a)[8], u32x4 u) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[2 * e] += __uint_as_float(u[e] << 16);
      a[2 * e + 1] += __uint_as_float(u[e] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ u32x4 pack(const float (&a)[8]) {
    u32x4 u;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      u[e] = static_cast<uint32_t>(f32_to_bf16_bits(a[2 * e])) |
             (static_cast<uint32_t>(f32_to_bf16_bits(a[2 * e + 1])) << 16);
    return u;
  }
};
template <> struct Chunk<float> {
  static constexpr int kN = 4;
  static __device__ __forceinline__ void add(float (&a)[4], u32x4 u) {
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] += __uint_as_float(u[e]);
  }
  static __device__ __forceinline__ u32x4 pack(const float (&a)[4]) {
    u32x4 u;
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = __float_as_uint(a[e]);
    return u;
  }
};

template <typename T>
__global__ void __launch_bounds__(256)
pool_kernel(const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ perm,
            const int32_t* __restrict__ blk_off, const int32_t* __restrict__ counts, int n, int hkv, int d,
            int nb_cap, T* __restrict__ kbar, T* __restrict__ vbar, T* __restrict__ k_cmp,
            T* __restrict__ v_cmp, T* __restrict__ k_s, T* __restrict__ v_s, float* __restrict__ knorm2) {
  constexpr int EC = Chunk<T>::kN;                      // elements per 16-byte chunk
  __shared__ float red[256 * EC];
  const int e_per_tok = hkv * d;
  const int c_per_tok = e_per_tok / EC;                 // chunks per row
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
      const bool on = slot < slots && c < c_per_tok;
      float ak[EC], av[EC];
#pragma unroll
      for (int e = 0; e < EC; ++e) ak[e] = av[e] = 0.f;
      if (on) {
        for (int p0 = a + slot; p0 < b; p0 += 4 * slots) {
          u32x4 kx[4], vx[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int pp = p0 + u * slots;
            if (pp < b) {
              const int64_t off = static_cast<int64_t>(perm[pp]) * e_per_tok + EC * c;
              kx[u] = *reinterpret_cast<const u32x4*>(k + off);
              vx[u] = *reinterpret_cast<const u32x4*>(v + off);
            }
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            if (p0 + u * slots < b) {
              Chunk<T>::add(ak, kx[u]);
              Chunk<T>::add(av, vx[u]);
            }
          }
          if (k_s) {
            // the rows in sorted order, head-major
            const int e0 = EC * c;
            const int64_t dst0 = (static_cast<int64_t>(e0 / d) * n) * d + e0 % d;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int pp = p0 + u * slots;
              if (pp < b) {
                *reinterpret_cast<u32x4*>(k_s + dst0 + static_cast<int64_t>(pp) * d) = kx[u];
                *reinterpret_cast<u32x4*>(v_s + dst0 + static_cast<int64_t>(pp) * d) = vx[u];
              }
            }
          }
        }
      }
      for (int which = 0; which < 2; ++which) {
        const float* acc = which ? av : ak;
        if (slots > 1) {
#pragma unroll
          for (int e = 0; e < EC; ++e) red[threadIdx.x * EC + e] = acc[e];
          __syncthreads();
        }
        if (slot == 0 && c < c_per_tok) {
          float s[EC];
#pragma unroll
          for (int e = 0; e < EC; ++e) s[e] = acc[e];
          for (int q = 1; q < slots; ++q)
#pragma unroll
            for (int e = 0; e < EC; ++e) s[e] += red[(q * tpt + lc) * EC + e];
#pragma unroll
          for (int e = 0; e < EC; ++e) s[e] = s[e] / cnt;
          const u32x4 packed = Chunk<T>::pack(s);
          const int e0 = EC * c;
          const int g = e0 / d, dd = e0 % d;
          T* dst = which ? vbar : kbar;
          *reinterpret_cast<u32x4*>(dst + (static_cast<int64_t>(g) * nb_cap + j) * d + dd) = packed;
          T* pub = which ? v_cmp : k_cmp;
          if (pub) *reinterpret_cast<u32x4*>(pub + static_cast<int64_t>(j) * e_per_tok + e0) = packed;
          if constexpr (std::is_same<T, uint16_t>::value) {
            if (knorm2 && which == 0) {
              // squared norm of the rounded key row: the d / 8 threads of one
              // head are consecutive lanes (d / 8 divides tpt)
              float n2 = 0.f;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float lo = __uint_as_float(packed[e] << 16), hi = __uint_as_float(packed[e] & 0xFFFF0000u);
                n2 = fmaf(lo, lo, fmaf(hi, hi, n2));
              }
              n2 += __shfl_xor(n2, 1);
              n2 += __shfl_xor(n2, 2);
              if (d == 64) n2 += __shfl_xor(n2, 4);
              if (dd == 0) knorm2[static_cast<int64_t>(g) * nb_cap + j] = n2;
            }
          }
        }
        if (slots > 1) __syncthreads();
      }
    }
  }
  // zero the rows of the last, partial 32-block tile so every key tile the
  // MFMA kernels read holds finite values
  const int nb_pad = (nb + kKeyTile - 1) / kKeyTile * kKeyTile;
  const int pad_rows = nb_pad - nb;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
       i < static_cast<int64_t>(hkv) * pad_rows * d; i += static_cast<int64_t>(gridDim.x) * 256) {
    const int g = static_cast<int>(i / (static_cast<int64_t>(pad_rows) * d));
    const int rem = static_cast<int>(i % (static_cast<int64_t>(pad_rows) * d));
    const int64_t row = (static_cast<int64_t>(g) * nb_cap + nb + rem / d) * d + rem % d;
    kbar[row] = T(0);
    vbar[row] = T(0);
  }
}

// Position of block jj (0..31) of a 32-block tile in the MFMA operand order:
// the 32x32 accumulator gives lane group 0 the keys {0-3, 8-11} and lane
// group 1 the keys {4-7, 12-15} of each 16-key half; the permutation is its
// own inverse.
__device__ __forceinline__ int mfma_key_pos(int jj) {
  const int lo = jj & 15;
  return (jj & 16) | (lo & 3) | ((lo & 4) << 1) | ((lo & 8) >> 1);
}

// vbar [h_kv][nb_cap][D] -> vbar_t [h_kv][nb_cap / 32][D][32] (bf16)
template <int D>
__global__ void __launch_bounds__(256)
vt_transpose_kernel(const uint16_t* __restrict__ vbar, uint16_t* __restrict__ vbar_t,
                    const int32_t* __restrict__ counts, int hkv, int nb_cap) {
  constexpr int CPR = D / 8;   // 16-byte chunks per row
  __shared__ uint16_t tile_lds[kKeyTile][D + 2];
  const int n_tiles = (counts[SSA_COUNT_NB] + kKeyTile - 1) / kKeyTile;
  const int per_head = nb_cap / kKeyTile;
  for (int w = blockIdx.x; w < hkv * n_tiles; w += gridDim.x) {
    const int g = w / n_tiles, kt = w % n_tiles;
    const uint16_t* src = vbar + (static_cast<int64_t>(g) * nb_cap + static_cast<int64_t>(kt) * kKeyTile) * D;
    // 32 rows x D dims: thread -> 8 consecutive dims of one row
    if (threadIdx.x < kKeyTile * CPR) {
      const int row = threadIdx.x / CPR, c = threadIdx.x % CPR;
      const u32x4 u = *reinterpret_cast<const u32x4*>(src + row * D + 8 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        tile_lds[row][8 * c + 2 * e] = static_cast<uint16_t>(u[e] & 0xFFFFu);
        tile_lds[row][8 * c + 2 * e + 1] = static_cast<uint16_t>(u[e] >> 16);
      }
    }
    __syncthreads();
    // D dim rows x 32 positions: thread -> 8 consecutive positions of one dim
    if (threadIdx.x < D * 4) {
      const int dd = threadIdx.x >> 2, c = threadIdx.x & 3;
      u32x4 u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int p0 = 8 * c + 2 * e;
        u[e] = static_cast<uint32_t>(tile_lds[mfma_key_pos(p0)][dd]) |
               (static_cast<uint32_t>(tile_lds[mfma_key_pos(p0 + 1)][dd]) << 16);
      }
      uint16_t* dst = vbar_t + ((static_cast<int64_t>(g) * per_head + kt) * D + dd) * kKeyTile + 8 * c;
      *reinterpret_cast<u32x4*>(dst) = u;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_pool(const FwdParams& p, ssa_dtype dtype, hipStream_t stream) {
  const int grid = p.nb_cap < 8192 ? p.nb_cap : 8192;
  if (dtype == SSA_BF16) {
    pool_kernel<uint16_t><<<grid, 256, 0, stream>>>(
        static_cast<const uint16_t*>(p.k), static_cast<const uint16_t*>(p.v), p.perm, p.blk_off,
        p.counts, p.n, p.h_kv, p.d, p.nb_cap, static_cast<uint16_t*>(p.kbar),
        static_cast<uint16_t*>(p.vbar), static_cast<uint16_t*>(p.k_cmp),
        static_cast<uint16_t*>(p.v_cmp), static_cast<uint16_t*>(p.k_s), static_cast<uint16_t*>(p.v_s),
        p.knorm2);
  } else {
    pool_kernel<float><<<grid, 256, 0, stream>>>(
        static_cast<const float*>(p.k), static_cast<const float*>(p.v), p.perm, p.blk_off,
        p.counts, p.n, p.h_kv, p.d, p.nb_cap, static_cast<float*>(p.kbar), static_cast<float*>(p.vbar),
        static_cast<float*>(p.k_cmp), static_cast<float*>(p.v_cmp), static_cast<float*>(p.k_s),
        static_cast<float*>(p.v_s), nullptr);
  }
  return hipGetLastError();
}

// the pooled values of every 32-block tile as [D][32 blocks] for the
// compressed kernels (bf16 MFMA path only; the pooling kernel writes vbar first)
hipError_t launch_vt_transpose(const FwdParams& p, ssa_dtype /*dtype*/, hipStream_t stream) {
  if (!p.vbar_t) return hipSuccess;
  const int tiles = p.h_kv * (p.nb_cap / kKeyTile);
  const int grid_t = tiles < 4096 ? tiles : 4096;
  if (p.d == 32)
    vt_transpose_kernel<32><<<grid_t, 256, 0, stream>>>(
        static_cast<const uint16_t*>(p.vbar), static_cast<uint16_t*>(p.vbar_t), p.counts, p.h_kv, p.nb_cap);
  else
    vt_transpose_kernel<64><<<grid_t, 256, 0, stream>>>(
        static_cast<const uint16_t*>(p.vbar), static_cast<uint16_t*>(p.vbar_t), p.counts, p.h_kv, p.nb_cap);
  return hipGetLastError();
}

}  // namespace ssa
