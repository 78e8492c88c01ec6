// Block build: block keys, stable LSD radix sort, CSR segments.
//
// Tokens are grouped by 3D coordinate into m_cmp^3 blocks and m_win^3
// windows (Direct3D-S2 page, "Method": blocking follows the 3D coordinate,
// windows do not overlap).  One 32-bit hierarchical key per token orders
// tokens by (sequence, window cell, block cell); a stable sort on it yields
// both partitions at once, with ties kept in input order.
//
// Sort design (gfx950, wave64): least-significant-digit radix sort, 8-bit
// digits, three kernels per pass in the reduce-then-scan scheme of Merrill &
// Grimshaw ("High Performance and Scalable Radix Sorting", 2011): per-tile
// digit counts, one exclusive scan over (digit, tile), and a scatter in which
// each wave ranks 64 keys at a time with eight ballots (lanes whose digit
// bits all agree are peers; a key's rank is the number of peers in lower
// lanes plus the wave's running count for that digit).
#include "ssa_internal.h"

namespace ssa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kItems = kSortTile / 256;  // keys per thread per tile (16)

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & (kWave - 1);
  return (lane == 0) ? 0ull : (~0ull >> (64 - lane));
}

// counts, the one-sweep sort's digit totals and tile counters, and the
// segment pass's tile counter and look-back words
__global__ void init_counts_kernel(int32_t* counts, int32_t key_bits, uint32_t* glob_hist, int32_t* tile_ctr,
                                   int32_t* seg_ctr, uint64_t* seg_state, int32_t seg_tiles) {
  const int i = threadIdx.x;
  if (i < SSA_COUNTS) counts[i] = (i == SSA_COUNT_KEY_BITS) ? key_bits : 0;
  if (glob_hist)
    for (int j = i; j < kMaxPasses * 256; j += blockDim.x) glob_hist[j] = 0u;
  if (tile_ctr && i < kMaxPasses) tile_ctr[i] = 0;
  if (seg_ctr && i == 0) *seg_ctr = 0;
  if (seg_state)
    for (int j = i; j < seg_tiles; j += blockDim.x) seg_state[j] = 0ull;
}

// Offsets for an empty token set: every offset array holds zeros.
__global__ void empty_offsets_kernel(int32_t batch, int32_t* blk_off, int32_t* win_off,
                                     int32_t* win_blk_off, int32_t* seq_blk_off,
                                     int32_t* seq_win_off) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0) {
    blk_off[0] = 0;
    win_off[0] = 0;
    win_blk_off[0] = 0;
  }
  if (i <= batch) {
    seq_blk_off[i] = 0;
    seq_win_off[i] = 0;
  }
}

// Block key of token t (input order) from its coordinates c; an out-of-grid
// coordinate is clamped (keeping later stages in bounds) and counted as
// invalid.
__device__ __forceinline__ uint32_t block_key(int c0, int c1, int c2, const int32_t* __restrict__ cu, int32_t t,
                                              int32_t batch, const KeyLayout& kl, int32_t* __restrict__ counts) {
  // sequence b: the largest b < batch with cu[b] <= t (empty sequences skipped)
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  int c[3] = {c0, c1, c2};
  bool bad = false;
  for (int a = 0; a < 3; ++a) {
    if (c[a] < 0 || c[a] >= kl.grid_res) {
      bad = true;
      c[a] = c[a] < 0 ? 0 : kl.grid_res - 1;
    }
  }
  if (bad) atomicAdd(&counts[SSA_COUNT_INVALID], 1);
  const uint32_t rmask = (1u << kl.l_r) - 1u;
  uint64_t key = static_cast<uint64_t>(lo);
  for (int a = 0; a < 3; ++a) c[a] += kl.shift;   // shifted windows: cells of c + shift
  for (int a = 0; a < 3; ++a) key = (key << kl.l_rw) | static_cast<uint32_t>(c[a] >> kl.l_win);
  for (int a = 0; a < 3; ++a) key = (key << kl.l_r) | (static_cast<uint32_t>(c[a] >> kl.l_cmp) & rmask);
  return static_cast<uint32_t>(key);
}

// First radix pass, upsweep: every key of a 4096-token tile computed from its
// coordinates, written out, and counted into the tile's digit histogram.  A
// full tile gives each thread four runs of four consecutive tokens: their 12
// coordinates are three 16-byte loads, their keys one 16-byte store, and all
// loads are in flight before any key is formed.  The permutation starts as
// the identity, which the first scatter generates itself.
__global__ void __launch_bounds__(256)
radix_upsweep_keys(const int32_t* __restrict__ coords, const int32_t* __restrict__ cu, int32_t n, int32_t batch,
                   KeyLayout kl, uint32_t* __restrict__ keys, int32_t* __restrict__ counts,
                   uint32_t* __restrict__ tile_hist) {
  __shared__ uint32_t hist[4][256];
  for (int i = threadIdx.x; i < 4 * 256; i += 256) (&hist[0][0])[i] = 0;
  __syncthreads();
  uint32_t* const h = hist[threadIdx.x >> 6];
  const int base = blockIdx.x * kSortTile;
  if (base + kSortTile <= n) {
    u32x4 cv[4][3];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int t0 = base + 4 * (g * 256 + threadIdx.x);
      const u32x4* src = reinterpret_cast<const u32x4*>(coords + 3 * static_cast<int64_t>(t0));
#pragma unroll
      for (int w = 0; w < 3; ++w) cv[g][w] = src[w];
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int t0 = base + 4 * (g * 256 + threadIdx.x);
      int c[12];
#pragma unroll
      for (int w = 0; w < 3; ++w)
#pragma unroll
        for (int e = 0; e < 4; ++e) c[4 * w + e] = static_cast<int>(cv[g][w][e]);
      u32x4 kv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kv[e] = block_key(c[3 * e], c[3 * e + 1], c[3 * e + 2], cu, t0 + e, batch, kl, counts);
        atomicAdd(&h[kv[e] & 255u], 1u);
      }
      *reinterpret_cast<u32x4*>(keys + t0) = kv;
    }
  } else {
    for (int i = threadIdx.x; i < kSortTile; i += 256) {
      const int t = base + i;
      if (t < n) {
        const uint32_t key = block_key(coords[3 * t], coords[3 * t + 1], coords[3 * t + 2], cu, t, batch, kl, counts);
        keys[t] = key;
        atomicAdd(&h[key & 255u], 1u);
      }
    }
  }
  __syncthreads();
  const int d = threadIdx.x;
  tile_hist[static_cast<size_t>(blockIdx.x) * 256 + d] = hist[0][d] + hist[1][d] + hist[2][d] + hist[3][d];
}

// Keys and digit counts for the one-sweep sort: every key of a tile of
// 256 x ITEMS tokens computed from its coordinates and written out, its
// digits of every pass counted (one LDS histogram per wave and pass) and
// added to the passes' totals over all keys, and the tile's look-back words
// of every pass cleared.  A full tile gives each thread ITEMS / 4 runs of four
// consecutive tokens: their 12 coordinates are three 16-byte loads, their
// keys one 16-byte store, and all loads are in flight before any key is
// formed.  The
// permutation starts as the identity, which the first scatter generates.
template <int ITEMS>
__global__ void __launch_bounds__(256)
build_hist_kernel(const int32_t* __restrict__ coords, const int32_t* __restrict__ cu, int32_t n, int32_t batch,
                  KeyLayout kl, int passes, uint32_t* __restrict__ keys, int32_t* __restrict__ counts,
                  uint32_t* __restrict__ glob_hist, uint64_t* __restrict__ tile_state, int ntiles) {
  __shared__ uint32_t hist[kMaxPasses][4][256];
  for (int i = threadIdx.x; i < kMaxPasses * 4 * 256; i += 256) (&hist[0][0][0])[i] = 0;
  __syncthreads();
  const int wv = threadIdx.x >> 6;
  auto count = [&](uint32_t key) {
    for (int ps = 0; ps < passes; ++ps) atomicAdd(&hist[ps][wv][(key >> (kRadixBits * ps)) & 255u], 1u);
  };
  constexpr int TILE = 256 * ITEMS, G = ITEMS / 4;
  const int base = blockIdx.x * TILE;
  if (base + TILE <= n) {
    u32x4 cv[G][3];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int t0 = base + 4 * (g * 256 + threadIdx.x);
      const u32x4* src = reinterpret_cast<const u32x4*>(coords + 3 * static_cast<int64_t>(t0));
#pragma unroll
      for (int w = 0; w < 3; ++w) cv[g][w] = src[w];
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int t0 = base + 4 * (g * 256 + threadIdx.x);
      int c[12];
#pragma unroll
      for (int w = 0; w < 3; ++w)
#pragma unroll
        for (int e = 0; e < 4; ++e) c[4 * w + e] = static_cast<int>(cv[g][w][e]);
      u32x4 kv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kv[e] = block_key(c[3 * e], c[3 * e + 1], c[3 * e + 2], cu, t0 + e, batch, kl, counts);
        count(kv[e]);
      }
      *reinterpret_cast<u32x4*>(keys + t0) = kv;
    }
  } else {
    for (int i = threadIdx.x; i < TILE; i += 256) {
      const int t = base + i;
      if (t < n) {
        const uint32_t key = block_key(coords[3 * t], coords[3 * t + 1], coords[3 * t + 2], cu, t, batch, kl, counts);
        keys[t] = key;
        count(key);
      }
    }
  }
  __syncthreads();
  const int d = threadIdx.x;
  for (int ps = 0; ps < passes; ++ps) {
    const uint32_t c = hist[ps][0][d] + hist[ps][1][d] + hist[ps][2][d] + hist[ps][3][d];
    if (c) atomicAdd(&glob_hist[ps * 256 + d], c);
    tile_state[(static_cast<size_t>(ps) * ntiles + blockIdx.x) * 256 + d] = 0ull;
  }
}

// Digit counts of one 4096-key tile, written tile-major (one contiguous
// 1 KB row per tile: tile_hist[tile * 256 + digit]).  Full tiles are read as
// 16-byte vectors, four per thread, all in flight at once; each wave counts
// into its own LDS histogram.
__global__ void __launch_bounds__(256)
radix_upsweep(const uint32_t* __restrict__ keys, int32_t n, int shift,
              uint32_t* __restrict__ tile_hist) {
  __shared__ uint32_t hist[4][256];
  for (int i = threadIdx.x; i < 4 * 256; i += 256) (&hist[0][0])[i] = 0;
  __syncthreads();
  uint32_t* const h = hist[threadIdx.x >> 6];
  const int base = blockIdx.x * kSortTile;
  if (base + kSortTile <= n) {
    const u32x4* k4 = reinterpret_cast<const u32x4*>(keys + base);
    u32x4 v[kItems / 4];
#pragma unroll
    for (int j = 0; j < kItems / 4; ++j) v[j] = k4[threadIdx.x + 256 * j];
#pragma unroll
    for (int j = 0; j < kItems / 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) atomicAdd(&h[(v[j][e] >> shift) & 255u], 1u);
  } else {
    for (int i = threadIdx.x; i < kSortTile; i += 256) {
      const int p = base + i;
      if (p < n) atomicAdd(&h[(keys[p] >> shift) & 255u], 1u);
    }
  }
  __syncthreads();
  const int d = threadIdx.x;
  tile_hist[static_cast<size_t>(blockIdx.x) * 256 + d] = hist[0][d] + hist[1][d] + hist[2][d] + hist[3][d];
}

// Scan of the tile-major digit counts in (digit, tile) order, the order of
// the stable scatter's output: offset(t, d) = (all tiles' keys of digits
// below d) + (digit d's keys in tiles before t).  Thread d owns column d;
// every step reads or writes one contiguous 1 KB row.  Up to kColSmall
// tiles one workgroup does it all; above, tiles are taken `per` at a time
// (at least 8, and at most 256 chunks).
constexpr int kColSmall = 32;
constexpr int kColChunksMax = 256;

__host__ __device__ constexpr int hist_chunk_tiles(int64_t ntiles) {
  return static_cast<int>(ntiles > 8 * kColChunksMax ? (ntiles + kColChunksMax - 1) / kColChunksMax : 8);
}

// column totals of each chunk of `per` tiles
__global__ void __launch_bounds__(256) hist_col_sums(const uint32_t* __restrict__ hist, int ntiles, int per,
                                                     uint32_t* __restrict__ csum) {
  const int d = threadIdx.x;
  const int t0 = blockIdx.x * per, t1 = min(t0 + per, ntiles);
  uint32_t s = 0;
#pragma unroll 8
  for (int t = t0; t < t1; ++t) s += hist[static_cast<size_t>(t) * 256 + d];
  csum[static_cast<size_t>(blockIdx.x) * 256 + d] = s;
}

// One workgroup of 1024 threads, in place over `rows` rows of 256 counts
// (tiles, or chunk totals): each row becomes its exclusive (digit, row)-order
// offsets.  Thread (q, d) walks column d over the q-th quarter of the rows.
__global__ void __launch_bounds__(1024) hist_col_scan(uint32_t* __restrict__ rowsv, int rows) {
  __shared__ uint32_t part[4][256];
  __shared__ uint32_t scan[256];
  const int d = threadIdx.x & 255, q = threadIdx.x >> 8;
  const int quarter = (rows + 3) / 4;
  const int r0 = min(q * quarter, rows), r1 = min(r0 + quarter, rows);
  uint32_t s = 0;
#pragma unroll 8
  for (int r = r0; r < r1; ++r) s += rowsv[static_cast<size_t>(r) * 256 + d];
  part[q][d] = s;
  __syncthreads();
  const uint32_t tot = part[0][d] + part[1][d] + part[2][d] + part[3][d];
  if (q == 0) scan[d] = tot;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const uint32_t x = (q == 0 && d >= off) ? scan[d - off] : 0u;
    __syncthreads();
    if (q == 0) scan[d] += x;
    __syncthreads();
  }
  uint32_t run = scan[d] - tot;   // keys of the digits below d
  for (int k = 0; k < q; ++k) run += part[k][d];
#pragma unroll 8
  for (int r = r0; r < r1; ++r) {
    const size_t i = static_cast<size_t>(r) * 256 + d;
    const uint32_t v = rowsv[i];
    rowsv[i] = run;
    run += v;
  }
}

// each chunk's tiles rewritten with their offsets, from the chunk's scanned total
__global__ void __launch_bounds__(256) hist_col_apply(uint32_t* __restrict__ hist, int ntiles, int per,
                                                      const uint32_t* __restrict__ csum) {
  const int d = threadIdx.x;
  const int t0 = blockIdx.x * per, t1 = min(t0 + per, ntiles);
  uint32_t run = csum[static_cast<size_t>(blockIdx.x) * 256 + d];
#pragma unroll 8
  for (int t = t0; t < t1; ++t) {
    const size_t i = static_cast<size_t>(t) * 256 + d;
    const uint32_t v = hist[i];
    hist[i] = run;
    run += v;
  }
}

// Stable scatter of one 4096-key tile: every key's rank among the tile's keys
// of its digit (wave ballots, waves in order), the keys placed in LDS in
// (digit, rank) order, then written out in that order so that consecutive
// threads write consecutive addresses of a digit's output run.
__global__ void __launch_bounds__(256)
radix_downsweep(const uint32_t* __restrict__ keys_in, const int32_t* __restrict__ vals_in,
                uint32_t* __restrict__ keys_out, int32_t* __restrict__ vals_out, int32_t n,
                int shift, const uint32_t* __restrict__ tile_off) {
  __shared__ uint32_t whist[4][256];   // per wave: keys of each digit
  __shared__ uint32_t wbase[4][256];   // per wave: tile-local start of its keys of each digit
  __shared__ uint32_t lstart[256];     // tile-local start of each digit
  __shared__ uint32_t gbase[256];      // output position of the tile's first key of each digit
  __shared__ uint32_t scan[256];
  __shared__ uint32_t skeys[kSortTile];
  __shared__ int32_t svals[kSortTile];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 4 * 256; i += 256) (&whist[0][0])[i] = 0;
  __syncthreads();
  const int tile0 = blockIdx.x * kSortTile;
  const int base = tile0 + wave * (kSortTile / 4);
  const uint64_t lt = lanemask_lt();
  uint32_t kk[kItems], rk[kItems], dg[kItems];
  int32_t vv[kItems];
  // every load of the thread in flight before the ranking (which waits on
  // LDS and ballots between keys)
#pragma unroll
  for (int r = 0; r < kItems; ++r) {
    const int p = base + r * kWave + lane;
    kk[r] = p < n ? keys_in[p] : 0u;
    // the first pass starts from the identity permutation
    vv[r] = vals_in ? (p < n ? vals_in[p] : 0) : p;
  }
#pragma unroll
  for (int r = 0; r < kItems; ++r) {
    const int p = base + r * kWave + lane;
    const bool valid = p < n;
    const uint32_t key = kk[r];
    const uint32_t d = (key >> shift) & 255u;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < kRadixBits; ++b) {
      const bool bit = (d >> b) & 1u;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const uint32_t before = whist[wave][d];
    const uint32_t cnt = static_cast<uint32_t>(__popcll(peers));
    const bool leader = valid && ((peers & lt) == 0);
    // every lane of the wave has read its count before any leader writes
    __builtin_amdgcn_wave_barrier();
    if (leader) whist[wave][d] = before + cnt;
    __builtin_amdgcn_wave_barrier();
    rk[r] = valid ? before + static_cast<uint32_t>(__popcll(peers & lt)) : 0xFFFFFFFFu;
    dg[r] = d;
  }
  __syncthreads();
  {
    // exclusive scan over the digits of the tile's digit totals
    const int d = threadIdx.x;
    const uint32_t tot = whist[0][d] + whist[1][d] + whist[2][d] + whist[3][d];
    scan[d] = tot;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const uint32_t v = d >= off ? scan[d - off] : 0u;
      __syncthreads();
      scan[d] += v;
      __syncthreads();
    }
    uint32_t run = scan[d] - tot;
    lstart[d] = run;
    gbase[d] = tile_off[static_cast<size_t>(blockIdx.x) * 256 + d];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      wbase[w][d] = run;
      run += whist[w][d];
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kItems; ++r) {
    if (rk[r] != 0xFFFFFFFFu) {
      const uint32_t pos = wbase[wave][dg[r]] + rk[r];
      skeys[pos] = kk[r];
      svals[pos] = vv[r];
    }
  }
  __syncthreads();
  const int cnt = min(kSortTile, n - tile0);
  for (int i = threadIdx.x; i < cnt; i += 256) {
    const uint32_t key = skeys[i];
    const uint32_t d = (key >> shift) & 255u;
    const uint32_t dst = gbase[d] + (static_cast<uint32_t>(i) - lstart[d]);
    keys_out[dst] = key;
    vals_out[dst] = svals[i];
  }
}

// One pass of the one-sweep sort (decoupled look-back, as in Merrill & Garland,
// "Single-pass Parallel Prefix Scan with Decoupled Look-back", 2016, applied
// to the radix scatter): a workgroup takes the next tile index from a
// counter, ranks its 4096 keys as the scatter above does, publishes its
// per-digit key counts (flag 1), then walks back over the tiles before it,
// adding their counts until it meets an inclusive prefix (flag 2), and
// publishes its own inclusive prefix.  A tile waits only on tiles that
// started before it, so the walk always ends; the spin is bounded anyway
// (kSpinMax polls), so a fault in the protocol cannot keep the kernel from
// exiting.  Look-back word: (flag << 32) | count.
constexpr int kSpinMax = 1 << 20;
constexpr int kLook = 16;   // look-back words read per round
template <int ITEMS>
__global__ void __launch_bounds__(256)
onesweep_kernel(const uint32_t* __restrict__ keys_in, const int32_t* __restrict__ vals_in,
                uint32_t* __restrict__ keys_out, int32_t* __restrict__ vals_out, int32_t n, int shift,
                const uint32_t* __restrict__ glob_hist, int32_t* __restrict__ tile_ctr,
                uint64_t* __restrict__ tile_state) {
  __shared__ uint32_t whist[4][256];   // per wave: keys of each digit
  __shared__ uint32_t wbase[4][256];   // per wave: tile-local start of its keys of each digit
  __shared__ uint32_t lstart[256];     // tile-local start of each digit
  __shared__ uint32_t gbase[256];      // output position of the tile's first key of each digit
  __shared__ uint32_t scan[256];
  constexpr int TILE = 256 * ITEMS;
  __shared__ uint32_t ehist[4][256];   // per wave: keys of each digit, counted before the ranking
  __shared__ uint32_t skeys[TILE];
  __shared__ int32_t svals[TILE];
  __shared__ int s_tile;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int d0 = threadIdx.x;
  for (int i = threadIdx.x; i < 4 * 256; i += 256) {
    (&whist[0][0])[i] = 0;
    (&ehist[0][0])[i] = 0;
  }
  if (threadIdx.x == 0) s_tile = atomicAdd(tile_ctr, 1);
  __syncthreads();
  const int tile = s_tile;
  const int tile0 = tile * TILE;
  const int base = tile0 + wave * (TILE / 4);
  const uint64_t lt = lanemask_lt();
  uint32_t kk[ITEMS], rk[ITEMS], dg[ITEMS];
  int32_t vv[ITEMS];
#pragma unroll
  for (int r = 0; r < ITEMS; ++r) {
    const int p = base + r * kWave + lane;
    kk[r] = p < n ? keys_in[p] : 0u;
    vv[r] = vals_in ? (p < n ? vals_in[p] : 0) : p;
  }
  const uint32_t gcount = glob_hist[d0];
  // the tile's digit counts first, published before the (much longer)
  // ranking, so that later tiles' look-backs find them early
#pragma unroll
  for (int r = 0; r < ITEMS; ++r)
    if (base + r * kWave + lane < n) atomicAdd(&ehist[wave][(kk[r] >> shift) & 255u], 1u);
  __syncthreads();
  const uint32_t tot = ehist[0][d0] + ehist[1][d0] + ehist[2][d0] + ehist[3][d0];
  uint64_t* const st = tile_state + static_cast<size_t>(tile) * 256 + d0;
  __hip_atomic_store(st, (uint64_t(1) << 32) | tot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
  for (int r = 0; r < ITEMS; ++r) {
    const int p = base + r * kWave + lane;
    const bool valid = p < n;
    const uint32_t key = kk[r];
    const uint32_t d = (key >> shift) & 255u;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < kRadixBits; ++b) {
      const bool bit = (d >> b) & 1u;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const uint32_t before = whist[wave][d];
    const uint32_t cnt = static_cast<uint32_t>(__popcll(peers));
    const bool leader = valid && ((peers & lt) == 0);
    __builtin_amdgcn_wave_barrier();
    if (leader) whist[wave][d] = before + cnt;
    __builtin_amdgcn_wave_barrier();
    rk[r] = valid ? before + static_cast<uint32_t>(__popcll(peers & lt)) : 0xFFFFFFFFu;
    dg[r] = d;
  }
  __syncthreads();
  {
    const int d = d0;
    // exclusive prefix of digit d over the tiles before this one: kLook
    // earlier tiles' words per round, loaded together, consumed in order up
    // to the first inclusive prefix (done) or the first tile not yet
    // published (the next round starts there)
    uint32_t prefix = 0;
    int j = tile - 1, stall = 0;
    while (j >= 0) {
      uint64_t w[kLook];
#pragma unroll
      for (int k = 0; k < kLook; ++k)
        w[k] = j - k >= 0 ? __hip_atomic_load(tile_state + static_cast<size_t>(j - k) * 256 + d, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT)
                          : (uint64_t(2) << 32);   // before tile 0: an inclusive prefix of 0
      int used = 0;
      bool done = false;
#pragma unroll
      for (int k = 0; k < kLook; ++k) {
        const uint32_t f = static_cast<uint32_t>(w[k] >> 32);
        if (!done && used == k && f != 0) {
          prefix += static_cast<uint32_t>(w[k]);
          used = k + 1;
          done = f == 2;
        }
      }
      if (done) break;
      j -= used;
      if (used == 0) {
        if (++stall > kSpinMax) break;   // gave up: the output is wrong but stays in bounds
        __builtin_amdgcn_s_sleep(1);
      }
    }
    __hip_atomic_store(st, (uint64_t(2) << 32) | (prefix + tot), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // exclusive scans over the digits: of the tile's totals, and of all keys' totals
    scan[d] = tot;
    lstart[d] = gcount;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const uint32_t v = d >= off ? scan[d - off] : 0u;
      const uint32_t g = d >= off ? lstart[d - off] : 0u;
      __syncthreads();
      scan[d] += v;
      lstart[d] += g;
      __syncthreads();
    }
    const uint32_t gstart = lstart[d] - gcount;   // keys of all digits below d
    __syncthreads();
    uint32_t run = scan[d] - tot;
    lstart[d] = run;
    gbase[d] = gstart + prefix;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      wbase[w][d] = run;
      run += whist[w][d];
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < ITEMS; ++r) {
    if (rk[r] != 0xFFFFFFFFu) {
      const uint32_t pos = wbase[wave][dg[r]] + rk[r];
      skeys[pos] = kk[r];
      svals[pos] = vv[r];
    }
  }
  __syncthreads();
  const int cnt = min(TILE, n - tile0);
  for (int i = threadIdx.x; i < cnt; i += 256) {
    const uint32_t key = skeys[i];
    const uint32_t d = (key >> shift) & 255u;
    const uint32_t dst = gbase[d] + (static_cast<uint32_t>(i) - lstart[d]);
    keys_out[dst] = key;
    vals_out[dst] = svals[i];
  }
}

template <int ITEMS>
__global__ void __launch_bounds__(256)
seg_count(const uint32_t* __restrict__ keys, int32_t n, int win_shift, int32_t* __restrict__ tile_cnt) {
  __shared__ int32_t red[2][256];
  const int base = blockIdx.x * 256 * ITEMS;
  int cb = 0, cw = 0;
  uint32_t kc[ITEMS], kprev[ITEMS];
#pragma unroll
  for (int r = 0; r < ITEMS; ++r) {   // all loads in flight first
    const int p = base + r * 256 + threadIdx.x;
    kc[r] = p < n ? keys[p] : 0u;
    kprev[r] = (p < n && p > 0) ? keys[p - 1] : 0u;
  }
#pragma unroll
  for (int r = 0; r < ITEMS; ++r) {
    const int p = base + r * 256 + threadIdx.x;
    if (p < n) {
      if (p == 0) {
        cb += 1;
        cw += 1;
      } else {
        cb += (kc[r] != kprev[r]);
        cw += ((kc[r] >> win_shift) != (kprev[r] >> win_shift));
      }
    }
  }
  red[0][threadIdx.x] = cb;
  red[1][threadIdx.x] = cw;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off) {
      red[0][threadIdx.x] += red[0][threadIdx.x + off];
      red[1][threadIdx.x] += red[1][threadIdx.x + off];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    tile_cnt[2 * blockIdx.x] = red[0][0];
    tile_cnt[2 * blockIdx.x + 1] = red[1][0];
  }
}

// Exclusive scan of the per-tile (block, window) start counts; totals go to
// counts[NB] / counts[NW].
__global__ void __launch_bounds__(1024)
seg_scan(const int32_t* __restrict__ tile_cnt, int ntiles, int32_t* __restrict__ tile_base,
         int32_t* __restrict__ counts) {
  __shared__ int32_t part[2][1024];
  const int tid = threadIdx.x;
  const int per = (ntiles + 1023) / 1024;
  const int beg = min(tid * per, ntiles), end = min(beg + per, ntiles);
  int sb = 0, sw = 0;
  for (int i = beg; i < end; ++i) {
    sb += tile_cnt[2 * i];
    sw += tile_cnt[2 * i + 1];
  }
  part[0][tid] = sb;
  part[1][tid] = sw;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int vb = tid >= off ? part[0][tid - off] : 0;
    const int vw = tid >= off ? part[1][tid - off] : 0;
    __syncthreads();
    part[0][tid] += vb;
    part[1][tid] += vw;
    __syncthreads();
  }
  int rb = tid ? part[0][tid - 1] : 0, rw = tid ? part[1][tid - 1] : 0;
  for (int i = beg; i < end; ++i) {
    const int vb = tile_cnt[2 * i], vw = tile_cnt[2 * i + 1];
    tile_base[2 * i] = rb;
    tile_base[2 * i + 1] = rw;
    rb += vb;
    rw += vw;
  }
  if (tid == 1023) {
    counts[SSA_COUNT_NB] = part[0][1023];
    counts[SSA_COUNT_NW] = part[1][1023];
  }
}

__device__ __forceinline__ int seq_of(uint32_t key, int seq_shift) {
  return seq_shift < 0 ? 0 : static_cast<int>(key >> seq_shift);
}

// Segment look-back word of a tile: flag (1 = the tile's own counts, 2 = the
// counts of every tile up to and including it) in bits 62-63, block starts in
// bits 31-61, window starts in bits 0-30.
__device__ __forceinline__ uint64_t seg_word(uint64_t flag, uint32_t nb, uint32_t nw) {
  return (flag << 62) | (static_cast<uint64_t>(nb) << 31) | nw;
}

// CSR offsets from the sorted keys in one pass.  Tiles are taken in order
// from a counter; each counts its block and window starts (a key differs from
// the one before it; a window start also in the window bits), publishes the
// counts, finds the counts of all earlier tiles by a look-back over their
// words (wave 0, 64 words per round, bounded spin), publishes its inclusive
// counts and writes its starts: blk_off, win_off, win_blk_off and the
// sequences' first block and window.  The tile holding the last token writes
// the totals and the closing entries.
template <int ITEMS>
__global__ void __launch_bounds__(256)
seg_onesweep(const uint32_t* __restrict__ keys, int32_t n, int32_t batch, int win_shift, int seq_shift,
             int32_t* __restrict__ seg_ctr, uint64_t* __restrict__ seg_state, int32_t* __restrict__ counts,
             int32_t* __restrict__ blk_off, int32_t* __restrict__ win_off, int32_t* __restrict__ win_blk_off,
             int32_t* __restrict__ seq_blk_off, int32_t* __restrict__ seq_win_off) {
  __shared__ int32_t wcnt[2][4];
  __shared__ int32_t s_pre[2];
  __shared__ int s_tile;
  if (threadIdx.x == 0) s_tile = atomicAdd(seg_ctr, 1);
  __syncthreads();
  const int tile = s_tile;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int base = tile * 256 * ITEMS + wave * (64 * ITEMS);
  const uint64_t lt = lanemask_lt();
  int rb = 0, rw = 0;
  int rank_b[ITEMS], rank_w[ITEMS];
  static_assert(2 * ITEMS <= 32, "two boundary flags per row are packed into 32 bits");
  uint32_t flags = 0;
  uint32_t kc[ITEMS], kprev[ITEMS];
#pragma unroll
  for (int r = 0; r < ITEMS; ++r) {   // all loads in flight before the ballots
    const int p = base + r * kWave + lane;
    kc[r] = p < n ? keys[p] : 0u;
    kprev[r] = (p < n && p > 0) ? keys[p - 1] : 0u;
  }
#pragma unroll
  for (int r = 0; r < ITEMS; ++r) {
    const int p = base + r * kWave + lane;
    const bool valid = p < n;
    bool isb = false, isw = false;
    if (valid) {
      if (p == 0) {
        isb = isw = true;
      } else {
        isb = kc[r] != kprev[r];
        isw = (kc[r] >> win_shift) != (kprev[r] >> win_shift);
      }
    }
    const uint64_t mb = __ballot(isb), mw = __ballot(isw);
    rank_b[r] = rb + static_cast<int>(__popcll(mb & lt));
    rank_w[r] = rw + static_cast<int>(__popcll(mw & lt));
    rb += static_cast<int>(__popcll(mb));
    rw += static_cast<int>(__popcll(mw));
    flags |= (isb ? 1u : 0u) << (2 * r);
    flags |= (isw ? 1u : 0u) << (2 * r + 1);
  }
  if (lane == 0) {
    wcnt[0][wave] = rb;
    wcnt[1][wave] = rw;
  }
  __syncthreads();
  if (wave == 0) {
    // wave 0 looks back 64 tiles per round: lane k reads the word of tile
    // j - k; the run of published words from lane 0 up to the first
    // inclusive one (done) or up to the first unpublished one (the next
    // round starts there) is summed
    const uint32_t tb = wcnt[0][0] + wcnt[0][1] + wcnt[0][2] + wcnt[0][3];
    const uint32_t tw = wcnt[1][0] + wcnt[1][1] + wcnt[1][2] + wcnt[1][3];
    if (lane == 0)
      __hip_atomic_store(seg_state + tile, seg_word(1, tb, tw), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t pb = 0, pw = 0;
    int j = tile - 1, stall = 0;
    while (j >= 0) {
      const int idx = j - lane;
      const uint64_t w = idx >= 0 ? __hip_atomic_load(seg_state + idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                  : seg_word(2, 0, 0);   // before tile 0: inclusive counts of zero
      const uint32_t f = static_cast<uint32_t>(w >> 62);
      const uint64_t unpub = __ballot(f == 0), incl = __ballot(f == 2);
      const int z = unpub ? __builtin_ctzll(unpub) : 64;
      const int c = incl ? __builtin_ctzll(incl) : 64;
      const bool done = c < z;
      const int take = done ? c + 1 : z;   // lanes 0 .. take - 1
      uint32_t ab = lane < take ? (static_cast<uint32_t>(w >> 31) & 0x7FFFFFFFu) : 0u;
      uint32_t aw = lane < take ? (static_cast<uint32_t>(w) & 0x7FFFFFFFu) : 0u;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        ab += __shfl_xor(ab, o);
        aw += __shfl_xor(aw, o);
      }
      pb += ab;
      pw += aw;
      if (done) break;
      j -= take;
      if (take == 0) {
        if (++stall > kSpinMax) break;   // gave up: the offsets are wrong but stay in bounds
        __builtin_amdgcn_s_sleep(1);
      }
    }
    if (lane == 0) {
      __hip_atomic_store(seg_state + tile, seg_word(2, pb + tb, pw + tw), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      s_pre[0] = static_cast<int32_t>(pb);
      s_pre[1] = static_cast<int32_t>(pw);
    }
  }
  __syncthreads();
  int pb = s_pre[0], pw = s_pre[1];
  const int nb_tot = pb + wcnt[0][0] + wcnt[0][1] + wcnt[0][2] + wcnt[0][3];   // used by the last tile only
  const int nw_tot = pw + wcnt[1][0] + wcnt[1][1] + wcnt[1][2] + wcnt[1][3];
  for (int w = 0; w < wave; ++w) {
    pb += wcnt[0][w];
    pw += wcnt[1][w];
  }
#pragma unroll
  for (int r = 0; r < ITEMS; ++r) {
    const int p = base + r * kWave + lane;
    if (p >= n) continue;
    const bool isb = (flags >> (2 * r)) & 1u, isw = (flags >> (2 * r + 1)) & 1u;
    const int bid = pb + rank_b[r];
    if (isb) blk_off[bid] = p;
    if (isw) {
      const int wid = pw + rank_w[r];
      win_off[wid] = p;
      win_blk_off[wid] = bid;
      const int s = seq_of(kc[r], seq_shift);
      const int sp = p ? seq_of(kprev[r], seq_shift) : -1;
      for (int b = sp + 1; b <= s; ++b) {
        seq_blk_off[b] = bid;
        seq_win_off[b] = wid;
      }
    }
    if (p == n - 1) {
      const int s = seq_of(kc[r], seq_shift);
      for (int b = s + 1; b <= batch; ++b) {
        seq_blk_off[b] = nb_tot;
        seq_win_off[b] = nw_tot;
      }
      blk_off[nb_tot] = n;
      win_off[nw_tot] = n;
      win_blk_off[nw_tot] = nb_tot;
      counts[SSA_COUNT_NB] = nb_tot;
      counts[SSA_COUNT_NW] = nw_tot;
    }
  }
}

template <int ITEMS>
__global__ void __launch_bounds__(256)
seg_write(const uint32_t* __restrict__ keys, int32_t n, int32_t batch, int win_shift,
          int seq_shift, const int32_t* __restrict__ tile_base, const int32_t* __restrict__ counts,
          int32_t* __restrict__ blk_off, int32_t* __restrict__ win_off,
          int32_t* __restrict__ win_blk_off, int32_t* __restrict__ seq_blk_off,
          int32_t* __restrict__ seq_win_off) {
  __shared__ int32_t wcnt[2][4];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int base = blockIdx.x * 256 * ITEMS + wave * (64 * ITEMS);
  const uint64_t lt = lanemask_lt();
  int rb = 0, rw = 0;
  int rank_b[ITEMS], rank_w[ITEMS];
  static_assert(2 * ITEMS <= 32, "two boundary flags per row are packed into 32 bits");
  uint32_t flags = 0;
  uint32_t kc[ITEMS], kprev[ITEMS];
#pragma unroll
  for (int r = 0; r < ITEMS; ++r) {   // all loads in flight before the ballots
    const int p = base + r * kWave + lane;
    kc[r] = p < n ? keys[p] : 0u;
    kprev[r] = (p < n && p > 0) ? keys[p - 1] : 0u;
  }
#pragma unroll
  for (int r = 0; r < ITEMS; ++r) {
    const int p = base + r * kWave + lane;
    const bool valid = p < n;
    bool isb = false, isw = false;
    if (valid) {
      if (p == 0) {
        isb = isw = true;
      } else {
        isb = kc[r] != kprev[r];
        isw = (kc[r] >> win_shift) != (kprev[r] >> win_shift);
      }
    }
    const uint64_t mb = __ballot(isb), mw = __ballot(isw);
    rank_b[r] = rb + static_cast<int>(__popcll(mb & lt));
    rank_w[r] = rw + static_cast<int>(__popcll(mw & lt));
    rb += static_cast<int>(__popcll(mb));
    rw += static_cast<int>(__popcll(mw));
    flags |= (isb ? 1u : 0u) << (2 * r);
    flags |= (isw ? 1u : 0u) << (2 * r + 1);
  }
  if (lane == 0) {
    wcnt[0][wave] = rb;
    wcnt[1][wave] = rw;
  }
  __syncthreads();
  int pb = tile_base[2 * blockIdx.x], pw = tile_base[2 * blockIdx.x + 1];
  for (int w = 0; w < wave; ++w) {
    pb += wcnt[0][w];
    pw += wcnt[1][w];
  }
  const int nb_tot = counts[SSA_COUNT_NB];
  const int nw_tot = counts[SSA_COUNT_NW];
#pragma unroll
  for (int r = 0; r < ITEMS; ++r) {
    const int p = base + r * kWave + lane;
    if (p >= n) continue;
    const bool isb = (flags >> (2 * r)) & 1u, isw = (flags >> (2 * r + 1)) & 1u;
    const int bid = pb + rank_b[r];
    if (isb) blk_off[bid] = p;
    if (isw) {
      const int wid = pw + rank_w[r];
      win_off[wid] = p;
      win_blk_off[wid] = bid;
      const int s = seq_of(kc[r], seq_shift);
      const int sp = p ? seq_of(kprev[r], seq_shift) : -1;
      for (int b = sp + 1; b <= s; ++b) {
        seq_blk_off[b] = bid;
        seq_win_off[b] = wid;
      }
    }
    if (p == n - 1) {
      const int s = seq_of(kc[r], seq_shift);
      for (int b = s + 1; b <= batch; ++b) {
        seq_blk_off[b] = nb_tot;
        seq_win_off[b] = nw_tot;
      }
      blk_off[nb_tot] = n;
      win_off[nw_tot] = n;
      win_blk_off[nw_tot] = nb_tot;
    }
  }
}

__global__ void __launch_bounds__(256)
seg_stats(const int32_t* __restrict__ blk_off, const int32_t* __restrict__ win_off,
          int32_t* __restrict__ counts) {
  __shared__ int red[2][4];
  const int nb = counts[SSA_COUNT_NB], nw = counts[SSA_COUNT_NW];
  const int m = nb > nw ? nb : nw;
  int mb = 0, mw = 0;
  const int stride = gridDim.x * blockDim.x;
  // four segments per thread and step, their loads in flight together
  for (int i0 = blockIdx.x * blockDim.x + threadIdx.x; i0 < m; i0 += 4 * stride) {
    int b0[4], b1[4], w0[4], w1[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * stride;
      b0[u] = i < nb ? blk_off[i] : 0;
      b1[u] = i < nb ? blk_off[i + 1] : 0;
      w0[u] = i < nw ? win_off[i] : 0;
      w1[u] = i < nw ? win_off[i + 1] : 0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      mb = max(mb, b1[u] - b0[u]);
      mw = max(mw, w1[u] - w0[u]);
    }
  }
  for (int off = 32; off > 0; off >>= 1) {
    mb = max(mb, __shfl_xor(mb, off));
    mw = max(mw, __shfl_xor(mw, off));
  }
  if ((threadIdx.x & (kWave - 1)) == 0) {
    red[0][threadIdx.x >> 6] = mb;
    red[1][threadIdx.x >> 6] = mw;
  }
  __syncthreads();
  if (threadIdx.x == 0) {  // one atomic pair per workgroup
    atomicMax(&counts[SSA_COUNT_MAX_BLK], max(max(red[0][0], red[0][1]), max(red[0][2], red[0][3])));
    atomicMax(&counts[SSA_COUNT_MAX_WIN], max(max(red[1][0], red[1][1]), max(red[1][2], red[1][3])));
  }
}

inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

}  // namespace

// Up to 2^18 tokens the build sorts with the one-sweep kernels on 1024-key
// tiles (nine short launches; four times the workgroups of 4096-key tiles,
// whose per-workgroup latency otherwise sets a small build's time).  Above,
// the three-kernel reduce-then-scan passes on 4096-key tiles are faster:
// measured on MI355X, one-sweep 61 / 76 / 106 / 578 us against 74 / 88 / 96 /
// 466 us at 2^17 / 2^18 / 2^19 / 2^24 random voxel tokens.
bool build_onesweep(int64_t n) { return n <= (int64_t(1) << 18); }
// The segment pass is one look-back kernel up to 2^21 tokens; above, the
// count / scan / write kernels, whose tiles wait on no other tile, are faster
// (measured on MI355X: 57 / 98 / 188 / 497 us against 60 / 101 / 178 / 470 us
// for the whole build at 2^17 / 2^20 / 2^22 / 2^24 random voxel tokens).
bool seg_onesweep_path(int64_t n) { return n <= (int64_t(1) << 21); }
int build_items(int64_t n) { return build_onesweep(n) ? 4 : kItems; }
int64_t build_tiles(int64_t n) {
  const int64_t tile = 256 * build_items(n);
  return (n + tile - 1) / tile;
}

size_t build_workspace_bytes(int64_t n, int32_t /*batch*/) {
  const int64_t ntiles = build_tiles(n);
  size_t b = 0;
  b += 2 * align256(sizeof(uint32_t) * n);     // keys_a, keys_b
  b += align256(sizeof(int32_t) * n);          // vals_b
  if (build_onesweep(n)) {
    b += align256(sizeof(uint32_t) * kMaxPasses * 256);                    // digit totals
    b += align256(sizeof(int32_t) * kMaxPasses);                           // tile counters
    b += align256(sizeof(uint64_t) * kMaxPasses * 256 * (ntiles > 0 ? ntiles : 1));   // look-back words
  } else {
    b += align256(sort_pairs_hist_bytes(n));   // tile histograms and their scan's chunk sums
  }
  if (seg_onesweep_path(n)) {
    b += align256(sizeof(uint64_t) * (ntiles > 0 ? ntiles : 1));   // segment look-back words
    b += align256(sizeof(int32_t));                                  // segment tile counter
  } else {
    b += 2 * align256(sizeof(int32_t) * 2 * ntiles);                 // tile counts and bases
  }
  return b + 256;
}

void carve_build_workspace(void* ws, int64_t n, BuildWorkspace* out) {
  const int64_t ntiles = build_tiles(n);
  char* p = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255));
  out->keys_a = reinterpret_cast<uint32_t*>(p); p += align256(sizeof(uint32_t) * n);
  out->keys_b = reinterpret_cast<uint32_t*>(p); p += align256(sizeof(uint32_t) * n);
  out->vals_b = reinterpret_cast<int32_t*>(p); p += align256(sizeof(int32_t) * n);
  out->glob_hist = nullptr;
  out->tile_ctr = nullptr;
  out->tile_state = nullptr;
  out->tile_hist = nullptr;
  if (build_onesweep(n)) {
    out->glob_hist = reinterpret_cast<uint32_t*>(p); p += align256(sizeof(uint32_t) * kMaxPasses * 256);
    out->tile_ctr = reinterpret_cast<int32_t*>(p); p += align256(sizeof(int32_t) * kMaxPasses);
    out->tile_state = reinterpret_cast<uint64_t*>(p);
    p += align256(sizeof(uint64_t) * kMaxPasses * 256 * (ntiles > 0 ? ntiles : 1));
  } else {
    out->tile_hist = reinterpret_cast<uint32_t*>(p); p += align256(sort_pairs_hist_bytes(n));
  }
  out->seg_state = nullptr;
  out->seg_ctr = nullptr;
  out->tile_cnt = nullptr;
  out->tile_base = nullptr;
  if (seg_onesweep_path(n)) {
    out->seg_state = reinterpret_cast<uint64_t*>(p); p += align256(sizeof(uint64_t) * (ntiles > 0 ? ntiles : 1));
    out->seg_ctr = reinterpret_cast<int32_t*>(p);
  } else {
    out->tile_cnt = reinterpret_cast<int32_t*>(p); p += align256(sizeof(int32_t) * 2 * ntiles);
    out->tile_base = reinterpret_cast<int32_t*>(p);
  }
}

bool sort_pairs_lands_in_tmp(int key_bits) {
  return ((key_bits + kRadixBits - 1) / kRadixBits) % 2 == 1;
}

size_t sort_pairs_hist_bytes(int64_t n) {
  const int64_t ntiles = (n + kSortTile - 1) / kSortTile;
  const int64_t rows = ntiles > 0 ? ntiles : 1;
  // tile histograms, then the column totals of their chunks
  const int64_t per = hist_chunk_tiles(rows);
  return align256(sizeof(uint32_t) * 256 * rows) + sizeof(uint32_t) * 256 * ((rows + per - 1) / per);
}

namespace {

// the tile histograms' (digit, tile)-order offsets, in place: one workgroup
// up to kColSmall tiles, else column totals per chunk of tiles, their scan,
// and each chunk rewritten from its total (the totals live right after the
// histograms)
void scan_tile_hist(uint32_t* tile_hist, int ntiles, hipStream_t stream) {
  if (ntiles <= kColSmall) {
    hist_col_scan<<<1, 1024, 0, stream>>>(tile_hist, ntiles);
    return;
  }
  uint32_t* csum = tile_hist + align256(sizeof(uint32_t) * 256 * static_cast<size_t>(ntiles)) / sizeof(uint32_t);
  const int per = hist_chunk_tiles(ntiles);
  const int chunks = (ntiles + per - 1) / per;
  hist_col_sums<<<chunks, 256, 0, stream>>>(tile_hist, ntiles, per, csum);
  hist_col_scan<<<1, 1024, 0, stream>>>(csum, chunks);
  hist_col_apply<<<chunks, 256, 0, stream>>>(tile_hist, ntiles, per, csum);
}

}  // namespace

hipError_t launch_sort_pairs(uint32_t* keys, int32_t* vals, uint32_t* keys_tmp, int32_t* vals_tmp, int32_t n,
                             int key_bits, uint32_t* tile_hist, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int ntiles = (n + kSortTile - 1) / kSortTile;
  const int passes = (key_bits + kRadixBits - 1) / kRadixBits;
  uint32_t* kin = keys;
  int32_t* vin = vals;
  uint32_t* kout = keys_tmp;
  int32_t* vout = vals_tmp;
  for (int pass = 0; pass < passes; ++pass) {
    const int shift = pass * kRadixBits;
    radix_upsweep<<<ntiles, 256, 0, stream>>>(kin, n, shift, tile_hist);
    scan_tile_hist(tile_hist, ntiles, stream);
    radix_downsweep<<<ntiles, 256, 0, stream>>>(kin, vin, kout, vout, n, shift, tile_hist);
    uint32_t* tk = kin; kin = kout; kout = tk;
    int32_t* tv = vin; vin = vout; vout = tv;
  }
  return hipGetLastError();
}

namespace {

// the sorted keys land in ws.keys_a and the permutation in out.perm
void build_sort_onesweep(const int32_t* coords, const int32_t* cu_seqlens, int32_t n, int32_t batch,
                         const KeyLayout& kl, const ssa_blocks& out, const BuildWorkspace& ws, hipStream_t stream) {
  constexpr int ITEMS = 4;
  const int ntiles = static_cast<int>(build_tiles(n));
  const int passes = (kl.key_bits + kRadixBits - 1) / kRadixBits;
  // ping-pong so that the last pass lands in (keys_a, perm)
  uint32_t* kin = (passes % 2 == 0) ? ws.keys_a : ws.keys_b;
  int32_t* vin = (passes % 2 == 0) ? out.perm : ws.vals_b;
  uint32_t* kout = (passes % 2 == 0) ? ws.keys_b : ws.keys_a;
  int32_t* vout = (passes % 2 == 0) ? ws.vals_b : out.perm;
  build_hist_kernel<ITEMS><<<ntiles, 256, 0, stream>>>(coords, cu_seqlens, n, batch, kl, passes, kin, out.counts,
                                                       ws.glob_hist, ws.tile_state, ntiles);
  for (int pass = 0; pass < passes; ++pass) {
    const int shift = pass * kRadixBits;
    onesweep_kernel<ITEMS><<<ntiles, 256, 0, stream>>>(kin, pass == 0 ? nullptr : vin, kout, vout, n, shift,
                                                       ws.glob_hist + 256 * pass, ws.tile_ctr + pass,
                                                       ws.tile_state + static_cast<size_t>(pass) * ntiles * 256);
    uint32_t* tk = kin; kin = kout; kout = tk;
    int32_t* tv = vin; vin = vout; vout = tv;
  }
}

void build_sort_passes(const int32_t* coords, const int32_t* cu_seqlens, int32_t n, int32_t batch,
                       const KeyLayout& kl, const ssa_blocks& out, const BuildWorkspace& ws, hipStream_t stream) {
  const int ntiles = static_cast<int>(build_tiles(n));
  const int passes = (kl.key_bits + kRadixBits - 1) / kRadixBits;
  uint32_t* kin = (passes % 2 == 0) ? ws.keys_a : ws.keys_b;
  int32_t* vin = (passes % 2 == 0) ? out.perm : ws.vals_b;
  uint32_t* kout = (passes % 2 == 0) ? ws.keys_b : ws.keys_a;
  int32_t* vout = (passes % 2 == 0) ? ws.vals_b : out.perm;
  for (int pass = 0; pass < passes; ++pass) {
    const int shift = pass * kRadixBits;
    if (pass == 0)
      radix_upsweep_keys<<<ntiles, 256, 0, stream>>>(coords, cu_seqlens, n, batch, kl, kin, out.counts,
                                                     ws.tile_hist);
    else
      radix_upsweep<<<ntiles, 256, 0, stream>>>(kin, n, shift, ws.tile_hist);
    scan_tile_hist(ws.tile_hist, ntiles, stream);
    radix_downsweep<<<ntiles, 256, 0, stream>>>(kin, pass == 0 ? nullptr : vin, kout, vout, n, shift,
                                                ws.tile_hist);
    uint32_t* tk = kin; kin = kout; kout = tk;
    int32_t* tv = vin; vin = vout; vout = tv;
  }
}

// CSR offsets, counts and maxima from the sorted keys
template <int ITEMS>
void build_segments(int32_t n, int32_t batch, const KeyLayout& kl, const ssa_blocks& out, const BuildWorkspace& ws,
                    hipStream_t stream) {
  const int ntiles = static_cast<int>(build_tiles(n));
  const int win_shift = 3 * kl.l_r;
  const int seq_shift = kl.seq_bits ? 3 * (kl.l_rw + kl.l_r) : -1;
  if (seg_onesweep_path(n)) {
    seg_onesweep<ITEMS><<<ntiles, 256, 0, stream>>>(ws.keys_a, n, batch, win_shift, seq_shift, ws.seg_ctr,
                                                     ws.seg_state, out.counts, out.blk_off, out.win_off,
                                                     out.win_blk_off, out.seq_blk_off, out.seq_win_off);
  } else {
    seg_count<ITEMS><<<ntiles, 256, 0, stream>>>(ws.keys_a, n, win_shift, ws.tile_cnt);
    seg_scan<<<1, 1024, 0, stream>>>(ws.tile_cnt, ntiles, ws.tile_base, out.counts);
    seg_write<ITEMS><<<ntiles, 256, 0, stream>>>(ws.keys_a, n, batch, win_shift, seq_shift, ws.tile_base,
                                                 out.counts, out.blk_off, out.win_off, out.win_blk_off,
                                                 out.seq_blk_off, out.seq_win_off);
  }
  // one workgroup per 4096 tokens, at least 64 and at most 1024 (two atomics each)
  const int sgrid = max(64, min((n + 4095) / 4096, 1024));
  seg_stats<<<sgrid, 256, 0, stream>>>(out.blk_off, out.win_off, out.counts);
}

}  // namespace

hipError_t launch_build(const int32_t* coords, const int32_t* cu_seqlens, int32_t n, int32_t batch,
                        const KeyLayout& kl, const ssa_blocks& out, const BuildWorkspace& ws,
                        hipStream_t stream) {
  init_counts_kernel<<<1, 256, 0, stream>>>(out.counts, kl.key_bits, n > 0 ? ws.glob_hist : nullptr,
                                            n > 0 ? ws.tile_ctr : nullptr, n > 0 ? ws.seg_ctr : nullptr,
                                            n > 0 ? ws.seg_state : nullptr,
                                            ws.seg_state ? static_cast<int32_t>(build_tiles(n)) : 0);
  if (n == 0) {
    empty_offsets_kernel<<<(batch + 1 + 255) / 256, 256, 0, stream>>>(
        batch, out.blk_off, out.win_off, out.win_blk_off, out.seq_blk_off, out.seq_win_off);
    return hipGetLastError();
  }
  if (build_onesweep(n)) {
    build_sort_onesweep(coords, cu_seqlens, n, batch, kl, out, ws, stream);
    build_segments<4>(n, batch, kl, out, ws, stream);
  } else {
    build_sort_passes(coords, cu_seqlens, n, batch, kl, out, ws, stream);
    build_segments<kItems>(n, batch, kl, out, ws, stream);
  }
  return hipGetLastError();
}

}  // namespace ssa
