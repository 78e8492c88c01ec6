// Geometric block routing: the top-k blocks nearest to each query voxel.
//
// LSRM article, "3D-aware block routing": a voxel token stands at its voxel's
// centre, and a query selects the blocks with the shortest Euclidean
// distance between it and the block's point set.  Here the distance of block
// j from the token at coordinate c is d_j = min over the block's tokens u of
// |c - c_u|^2, an exact integer; the k smallest (d_j, j) of the query's
// sequence are selected, the same list for every key/value group.
//
// block_cells_kernel: the m_cmp^3 cell of every block (from its first token).
//
// geo_topk_kernel: one wave per sorted query.  A block's cell bounds d_j from
// below: b_j = sum over the axes of the squared distance from c to the
// cell's voxel range.  The wave (1) takes the k blocks with the smallest
// (b_j, j), (2) computes their exact distances, whose maximum U bounds the
// k-th smallest exact distance from above, and (3) computes d_j exactly for
// every block with b_j <= U (no other block can be among the k nearest) and
// ranks those.  Per-lane sorted lists are merged by repeated wave minima.
#include <limits.h>

#include "ssa_internal.h"

namespace ssa {
namespace {

__global__ void __launch_bounds__(256)
block_cells_kernel(FwdParams p) {
  const int nb = p.counts[SSA_COUNT_NB];
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < nb; j += gridDim.x * blockDim.x) {
    const int t = p.perm[p.blk_off[j]];
    p.blk_cell[j] = make_int4(p.coords[3 * t] >> p.l_cmp, p.coords[3 * t + 1] >> p.l_cmp,
                              p.coords[3 * t + 2] >> p.l_cmp, 0);
  }
}

__device__ __forceinline__ int axis_gap(int c, int lo, int hi) {
  return c < lo ? lo - c : (c > hi ? c - hi : 0);
}

// a sorted list of the KMAX smallest (distance, block) pairs of one lane
template <int KMAX>
struct NearList {
  int d[KMAX];
  int j[KMAX];
  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int e = 0; e < KMAX; ++e) {
      d[e] = INT_MAX;
      j[e] = INT_MAX;
    }
  }
  // blocks arrive in increasing id, so an equal distance stays behind
  __device__ __forceinline__ void insert(int dist, int blk) {
    if (dist >= d[KMAX - 1]) return;
    bool placed = false;
#pragma unroll
    for (int e = KMAX - 1; e >= 1; --e) {
      if (!placed) {
        if (dist < d[e - 1]) {
          d[e] = d[e - 1];
          j[e] = j[e - 1];
        } else {
          d[e] = dist;
          j[e] = blk;
          placed = true;
        }
      }
    }
    if (!placed) {
      d[0] = dist;
      j[0] = blk;
    }
  }
  // the wave's next smallest pair (distance, then block); the owning lane pops it
  __device__ __forceinline__ void pop_min(int* bd, int* bj) {
    int vd = d[0], vj = j[0];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const int od = __shfl_xor(vd, off);
      const int oj = __shfl_xor(vj, off);
      if (od < vd || (od == vd && oj < vj)) {
        vd = od;
        vj = oj;
      }
    }
    if (j[0] == vj && vj != INT_MAX) {
#pragma unroll
      for (int e = 0; e < KMAX - 1; ++e) {
        d[e] = d[e + 1];
        j[e] = j[e + 1];
      }
      d[KMAX - 1] = INT_MAX;
      j[KMAX - 1] = INT_MAX;
    }
    *bd = vd;
    *bj = vj;
  }
};

template <int KMAX>
__global__ void __launch_bounds__(256)
geo_topk_kernel(FwdParams p) {
  __shared__ int sel_lds[4][KMAX];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int i = blockIdx.x * 4 + wv;   // sorted query position
  if (i >= p.n) return;
  // window, then sequence, of position i
  int lo = 0, hi = p.counts[SSA_COUNT_NW] - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.win_off[mid] <= i) lo = mid; else hi = mid - 1;
  }
  const int w = lo;
  lo = 0;
  hi = p.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.seq_win_off[mid] <= w) lo = mid; else hi = mid - 1;
  }
  const int j0 = p.seq_blk_off[lo], j1 = p.seq_blk_off[lo + 1];
  const int t = p.perm[i];
  const int cx = p.coords[3 * t], cy = p.coords[3 * t + 1], cz = p.coords[3 * t + 2];
  const int m = 1 << p.l_cmp;
  auto box = [&](int j) {
    const int4 cell = p.blk_cell[j];
    const int gx = axis_gap(cx, cell.x * m, cell.x * m + m - 1);
    const int gy = axis_gap(cy, cell.y * m, cell.y * m + m - 1);
    const int gz = axis_gap(cz, cell.z * m, cell.z * m + m - 1);
    return gx * gx + gy * gy + gz * gz;
  };
  auto exact = [&](int j) {
    int best = INT_MAX;
    for (int u = p.blk_off[j]; u < p.blk_off[j + 1]; ++u) {
      const int tu = p.perm[u];
      const int dx = p.coords[3 * tu] - cx, dy = p.coords[3 * tu + 1] - cy, dz = p.coords[3 * tu + 2] - cz;
      best = min(best, dx * dx + dy * dy + dz * dz);
    }
    return best;
  };
  const int k_eff = min(p.topk, j1 - j0);

  // (1) the k blocks nearest by cell
  NearList<KMAX> L;
  L.clear();
  for (int j = j0 + lane; j < j1; j += 64) L.insert(box(j), j);
  for (int r = 0; r < k_eff; ++r) {
    int bd, bj;
    L.pop_min(&bd, &bj);
    if (lane == 0) sel_lds[wv][r] = bj;
  }
  wave_lds_sync();
  // (2) their exact distances bound the k-th smallest from above
  int U = 0;
  for (int r = 0; r < k_eff; ++r) {
    const int j = sel_lds[wv][r];
    int best = INT_MAX;
    for (int u = p.blk_off[j] + lane; u < p.blk_off[j + 1]; u += 64) {
      const int tu = p.perm[u];
      const int dx = p.coords[3 * tu] - cx, dy = p.coords[3 * tu + 1] - cy, dz = p.coords[3 * tu + 2] - cz;
      best = min(best, dx * dx + dy * dy + dz * dz);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) best = min(best, __shfl_xor(best, off));
    U = max(U, best);
  }
  wave_lds_sync();
  // (3) exact distances of every block whose cell is within U
  L.clear();
  for (int j = j0 + lane; j < j1; j += 64)
    if (box(j) <= U) L.insert(exact(j), j);
  for (int r = 0; r < k_eff; ++r) {
    int bd, bj;
    L.pop_min(&bd, &bj);
    if (lane == 0) sel_lds[wv][r] = bj;
  }
  wave_lds_sync();
  for (int e = lane; e < p.h_kv * p.topk; e += 64) {
    const int r = e % p.topk;
    p.topk_idx[static_cast<int64_t>(t) * p.h_kv * p.topk + e] = r < k_eff ? sel_lds[wv][r] : -1;
  }
}

}  // namespace

hipError_t launch_geo_topk(const FwdParams& p, ssa_dtype /*dtype*/, hipStream_t stream) {
  const int grid_c = (p.nb_cap + 255) / 256 < 8192 ? (p.nb_cap + 255) / 256 : 8192;
  block_cells_kernel<<<grid_c, 256, 0, stream>>>(p);
  const int grid = (p.n + 3) / 4;
  if (p.topk <= 16) geo_topk_kernel<16><<<grid, 256, 0, stream>>>(p);
  else geo_topk_kernel<32><<<grid, 256, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace ssa
