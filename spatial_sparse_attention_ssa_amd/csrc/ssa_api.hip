// Host side of libssa: argument validation, workspace layout and launches.
// Every check runs before anything is enqueued; the library allocates no
// memory and keeps no state beyond the thread-local error message.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "ssa_internal.h"

namespace {

thread_local std::string g_last_error;

ssa_status fail(ssa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

ssa_status ok() {
  g_last_error.clear();
  return SSA_OK;
}

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

int ilog2(int64_t v) {
  int l = 0;
  while ((int64_t(1) << (l + 1)) <= v) ++l;
  return l;
}

int ceil_log2(int64_t v) {
  int l = 0;
  while ((int64_t(1) << l) < v) ++l;
  return l;
}

inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

ssa_status check_geometry(const ssa_geometry* geo) {
  if (!geo) return fail(SSA_ERR_INVALID_ARGUMENT, "geometry is null");
  if (!is_pow2(geo->grid_res) || !is_pow2(geo->m_cmp) || !is_pow2(geo->m_win))
    return fail(SSA_ERR_INVALID_ARGUMENT, "grid_res (%d), m_cmp (%d) and m_win (%d) must be powers of two",
                geo->grid_res, geo->m_cmp, geo->m_win);
  if (geo->grid_res > 1024)
    return fail(SSA_ERR_INVALID_ARGUMENT, "grid_res %d exceeds 1024", geo->grid_res);
  if (geo->m_cmp > geo->m_win || geo->m_win > geo->grid_res)
    return fail(SSA_ERR_INVALID_ARGUMENT, "need m_cmp <= m_win <= grid_res (got %d, %d, %d)",
                geo->m_cmp, geo->m_win, geo->grid_res);
  if (geo->win_shift < 0 || geo->win_shift >= geo->m_win || geo->win_shift % geo->m_cmp)
    return fail(SSA_ERR_INVALID_ARGUMENT, "win_shift %d must be a multiple of m_cmp (%d) in [0, m_win = %d)",
                geo->win_shift, geo->m_cmp, geo->m_win);
  return SSA_OK;
}

ssa::KeyLayout key_layout(const ssa_geometry* geo, int32_t batch) {
  ssa::KeyLayout kl;
  kl.l_win = ilog2(geo->m_win);
  kl.l_cmp = ilog2(geo->m_cmp);
  // a shifted window grid has one more window per axis
  kl.l_rw = ilog2(geo->grid_res) - kl.l_win + (geo->win_shift ? 1 : 0);
  kl.l_r = kl.l_win - kl.l_cmp;
  kl.shift = geo->win_shift;
  kl.seq_bits = ceil_log2(batch);
  kl.key_bits = kl.seq_bits + 3 * (kl.l_rw + kl.l_r);
  kl.grid_res = geo->grid_res;
  return kl;
}

// The dtype field as the integer a C caller stored: any value may arrive
// through the C ABI, and loading one outside the enumerators through the C++
// enum type would be undefined.
int raw_dtype(const ssa_attn* a) {
  static_assert(sizeof(ssa_dtype) == sizeof(int), "ssa_dtype is stored as an int");
  int v;
  memcpy(&v, &a->dtype, sizeof(v));
  return v;
}

ssa_status check_attn(const ssa_attn* a) {
  if (!a) return fail(SSA_ERR_INVALID_ARGUMENT, "attn is null");
  if (a->h_q < 1 || a->h_kv < 1 || a->h_q % a->h_kv)
    return fail(SSA_ERR_INVALID_ARGUMENT, "need h_q, h_kv >= 1 and h_q %% h_kv == 0 (got %d, %d)",
                a->h_q, a->h_kv);
  if (raw_dtype(a) != SSA_F32 && raw_dtype(a) != SSA_BF16)
    return fail(SSA_ERR_INVALID_ARGUMENT, "unknown dtype %d", raw_dtype(a));
  if (a->head_dim < 1) return fail(SSA_ERR_INVALID_ARGUMENT, "head_dim %d < 1", a->head_dim);
  if (a->topk < 1) return fail(SSA_ERR_INVALID_ARGUMENT, "topk %d < 1", a->topk);
  if (a->head_dim != 32 && a->head_dim != 64)
    return fail(SSA_ERR_UNSUPPORTED, "head_dim %d not supported (32 or 64)", a->head_dim);
  if (a->topk > 32) return fail(SSA_ERR_UNSUPPORTED, "topk %d > 32 not supported", a->topk);
  if (a->h_q / a->h_kv > 32)
    return fail(SSA_ERR_UNSUPPORTED, "group size %d > 32 not supported", a->h_q / a->h_kv);
  if (!isfinite(a->scale)) return fail(SSA_ERR_INVALID_ARGUMENT, "scale is not finite");
  if (a->routing != SSA_ROUTE_SCORE && a->routing != SSA_ROUTE_GEOMETRIC)
    return fail(SSA_ERR_INVALID_ARGUMENT, "unknown routing %d", a->routing);
  return SSA_OK;
}

int elt_bytes(ssa_dtype d) { return d == SSA_BF16 ? 2 : 4; }

// pooled-row capacity: the block count when known, else the token count;
// rounded up to whole 32-block key tiles
int64_t nb_capacity(const ssa_blocks* b) {
  int64_t c = b->nb >= 0 ? b->nb : b->n_tokens;
  if (c < 1) c = 1;
  return (c + ssa::kKeyTile - 1) / ssa::kKeyTile * ssa::kKeyTile;
}

// the MFMA kernels cover bfloat16 with head_dim 32 or 64 and 1 to 16 query
// heads per key/value head (groups of 2 to 16 take the grouped kernels)
bool use_gqa_path(const ssa_attn* a) {
  const int group = a->h_q / a->h_kv;
  return a->dtype == SSA_BF16 && (a->head_dim == 32 || a->head_dim == 64) && group >= 2 && group <= 16;
}
bool use_mfma_path(const ssa_attn* a) {
  return (a->dtype == SSA_BF16 && (a->head_dim == 32 || a->head_dim == 64) && a->h_q == a->h_kv) ||
         use_gqa_path(a);
}

struct FwdLayout {
  size_t kbar, vbar, vbar_t, k_s, v_s, topk, tile_pre, fix, acc, norm, tile_pre2, blk_cell, knorm2, probe_slot,
      probe_seq, probe_maxn2, probe, probe_ids, seq_kmax2, total;
};

// probe sets of the one-head-per-group compressed kernel: one per sequence
// with more than kProbeBlocks blocks, so at most nb_cap / (kProbeBlocks + 1)
int32_t max_probe_slots(const ssa_blocks* b) {
  const int64_t by_blocks = nb_capacity(b) / (ssa::kProbeBlocks + 1);
  return static_cast<int32_t>(by_blocks < b->batch ? by_blocks : b->batch);
}

FwdLayout forward_layout(const ssa_blocks* b, const ssa_attn* a) {
  const size_t cap = static_cast<size_t>(nb_capacity(b));
  const size_t n = static_cast<size_t>(b->n_tokens);
  const size_t pooled = align256(static_cast<size_t>(elt_bytes(a->dtype)) * a->h_kv * cap * a->head_dim);
  FwdLayout L{};
  size_t off = 0;
  L.kbar = off; off += pooled;
  L.vbar = off; off += pooled;
  L.topk = off; off += align256(sizeof(int32_t) * n * a->h_kv * a->topk);
  if (use_mfma_path(a)) {
    L.vbar_t = off; off += pooled;
    const size_t sorted = align256(static_cast<size_t>(elt_bytes(a->dtype)) * a->h_kv * n * a->head_dim);
    L.k_s = off; off += sorted;
    L.v_s = off; off += sorted;
    L.tile_pre = off; off += align256(sizeof(int32_t) * (static_cast<size_t>(b->batch) + 1));
    L.fix = off; off += align256(sizeof(int32_t) * (1 + n * a->h_kv));
    L.acc = off; off += align256(sizeof(float) * n * a->h_q * a->head_dim);
    if (use_gqa_path(a)) {
      L.norm = off; off += align256(sizeof(float) * n * a->h_q);
      L.tile_pre2 = off; off += align256(sizeof(int32_t) * (static_cast<size_t>(b->batch) + 1));
      L.knorm2 = off; off += align256(sizeof(float) * a->h_kv * cap);
      L.seq_kmax2 = off; off += align256(sizeof(float) * a->h_kv * static_cast<size_t>(b->batch));
      const size_t slots = static_cast<size_t>(max_probe_slots(b));
      L.probe_slot = off; off += align256(sizeof(int32_t) * (static_cast<size_t>(b->batch) + 1));
      L.probe_seq = off; off += align256(sizeof(int32_t) * (slots + 1));
      L.probe_maxn2 = off; off += align256(sizeof(float) * a->h_kv * (slots + 1));
      L.probe_ids = off; off += align256(sizeof(int32_t) * a->h_kv * slots * ssa::kProbeBlocks);
    } else {
      const size_t slots = static_cast<size_t>(max_probe_slots(b));
      L.knorm2 = off; off += align256(sizeof(float) * a->h_kv * cap);
      L.probe_slot = off; off += align256(sizeof(int32_t) * (static_cast<size_t>(b->batch) + 1));
      L.probe_seq = off; off += align256(sizeof(int32_t) * (slots + 1));
      L.probe_maxn2 = off; off += align256(sizeof(float) * a->h_kv * (slots + 1));
      L.probe = off; off += align256(static_cast<size_t>(elt_bytes(a->dtype)) * a->h_kv * slots * ssa::kProbeBlocks *
                                     a->head_dim);
    }
    if (a->routing == SSA_ROUTE_GEOMETRIC) {
      L.blk_cell = off; off += align256(4 * sizeof(int32_t) * cap);
    }
  }
  L.total = off + 256;
  return L;
}

size_t forward_ws_bytes(const ssa_blocks* b, const ssa_attn* a) { return forward_layout(b, a).total; }

// A second stream and two events per host thread and device, on which the
// probe-set selection runs beside the window kernel (it reads only what
// the pooling kernel wrote, and only the compressed kernel reads what it
// writes).  Created on first use (default priority, non-blocking) and kept
// until the process ends; if creation fails the kernels run in order on the
// caller's stream.
struct SideStream {
  bool tried = false, ok = false;
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxSideDevices = 64;

SideStream* side_stream() {
  thread_local SideStream side[kMaxSideDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxSideDevices) return nullptr;
  SideStream& s = side[dev];
  if (!s.tried) {
    s.tried = true;
    s.ok = hipStreamCreateWithFlags(&s.stream, hipStreamNonBlocking) == hipSuccess &&
           hipEventCreateWithFlags(&s.fork, hipEventDisableTiming) == hipSuccess &&
           hipEventCreateWithFlags(&s.join, hipEventDisableTiming) == hipSuccess;
  }
  return s.ok ? &s : nullptr;
}

}  // namespace

extern "C" {

const char* ssa_status_string(ssa_status s) {
  switch (s) {
    case SSA_OK: return "ok";
    case SSA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SSA_ERR_UNSUPPORTED: return "unsupported";
    case SSA_ERR_WORKSPACE: return "workspace too small";
    case SSA_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

const char* ssa_last_error(void) { return g_last_error.c_str(); }

int32_t ssa_version(void) { return 100; }

size_t ssa_build_blocks_workspace(int64_t n_tokens, int32_t batch, const ssa_geometry* /*geo*/) {
  if (n_tokens < 0) return 0;
  return ssa::build_workspace_bytes(n_tokens, batch);
}

ssa_status ssa_build_blocks(const int32_t* coords, const int32_t* cu_seqlens, int64_t n_tokens,
                            int32_t batch, const ssa_geometry* geo, ssa_blocks* out,
                            int sync_counts, void* workspace, size_t ws_bytes, void* hip_stream) {
  if (n_tokens < 0 || n_tokens > 0x7FFFFFFE)
    return fail(SSA_ERR_INVALID_ARGUMENT, "n_tokens %lld out of range", static_cast<long long>(n_tokens));
  if (batch < 1) return fail(SSA_ERR_INVALID_ARGUMENT, "batch %d < 1", batch);
  ssa_status st = check_geometry(geo);
  if (st != SSA_OK) return st;
  if (!out) return fail(SSA_ERR_INVALID_ARGUMENT, "out is null");
  if (!cu_seqlens) return fail(SSA_ERR_INVALID_ARGUMENT, "cu_seqlens is null");
  if (n_tokens > 0 && !coords) return fail(SSA_ERR_INVALID_ARGUMENT, "coords is null");
  if (!out->perm || !out->blk_off || !out->win_off || !out->win_blk_off || !out->seq_blk_off ||
      !out->seq_win_off || !out->counts)
    return fail(SSA_ERR_INVALID_ARGUMENT, "an output buffer of ssa_blocks is null");
  const ssa::KeyLayout kl = key_layout(geo, batch);
  if (kl.key_bits > 32)
    return fail(SSA_ERR_UNSUPPORTED, "block key needs %d bits (> 32): batch %d, grid %d, m_cmp %d",
                kl.key_bits, batch, geo->grid_res, geo->m_cmp);
  const size_t need = ssa::build_workspace_bytes(n_tokens, batch);
  if (!workspace || ws_bytes < need)
    return fail(SSA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace ? ws_bytes : 0, need);

  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  ssa::BuildWorkspace ws;
  ssa::carve_build_workspace(workspace, n_tokens, &ws);
  hipError_t e = ssa::launch_build(coords, cu_seqlens, static_cast<int32_t>(n_tokens), batch, kl, *out, ws, stream);
  if (e != hipSuccess) return fail(SSA_ERR_DEVICE, "block build launch failed: %s", hipGetErrorString(e));
  out->n_tokens = n_tokens;
  out->batch = batch;
  out->geo = *geo;
  out->coords = coords;
  out->nb = out->nw = out->max_blk_tokens = out->max_win_tokens = -1;
  if (sync_counts) {
    int32_t h[SSA_COUNTS];
    e = hipMemcpyAsync(h, out->counts, sizeof(h), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return fail(SSA_ERR_DEVICE, "reading block counts failed: %s", hipGetErrorString(e));
    out->nb = h[SSA_COUNT_NB];
    out->nw = h[SSA_COUNT_NW];
    out->max_blk_tokens = h[SSA_COUNT_MAX_BLK];
    out->max_win_tokens = h[SSA_COUNT_MAX_WIN];
    if (h[SSA_COUNT_INVALID] > 0)
      return fail(SSA_ERR_INVALID_ARGUMENT, "%d token(s) have a coordinate outside [0, %d)",
                  h[SSA_COUNT_INVALID], geo->grid_res);
  }
  return ok();
}

size_t ssa_forward_workspace(const ssa_blocks* blocks, const ssa_attn* attn) {
  if (!blocks || !attn || blocks->n_tokens < 0 || attn->h_kv < 1 || attn->head_dim < 1 || attn->topk < 1)
    return 0;
  return forward_ws_bytes(blocks, attn);
}

}  // extern "C"

namespace {

// The kernels ssa_forward launches for a layout, in order.
struct Stage {
  const char* name;
  hipError_t (*launch)(const ssa::FwdParams&, ssa_dtype, hipStream_t);
};

int forward_plan(const ssa_attn* attn, Stage* stages) {
  stages[0] = Stage{"pool_kernel", ssa::launch_pool};
  if (!use_mfma_path(attn)) {
    stages[1] = Stage{"generic_fwd", ssa::launch_generic};
    return 2;
  }
  // the pooled values transposed for the compressed kernels; the window
  // kernel is the first writer of the float32 branch accumulator (every
  // token lies in exactly one window); the compressed kernels add to it
  stages[1] = Stage{"vt_transpose_kernel", ssa::launch_vt_transpose};
  stages[2] = Stage{"win_mfma_kernel", ssa::launch_win_mfma};
  int n = 3;
  if (use_gqa_path(attn)) {
    stages[n++] = Stage{"gqa_cmp_kernel", ssa::launch_gqa_cmp};
    stages[n++] = Stage{"gqa_topk_kernel", ssa::launch_gqa_topk};
  } else {
    stages[n++] = Stage{"probe_kernel", ssa::launch_cmp_probe};
    stages[n++] = Stage{"cmp_mfma_kernel", ssa::launch_cmp_mfma};
    stages[n++] = Stage{"topk_fixup_kernel", ssa::launch_topk_fixup};
  }
  // geometric routing replaces the score-ranked lists
  if (attn->routing == SSA_ROUTE_GEOMETRIC) stages[n++] = Stage{"geo_topk_kernel", ssa::launch_geo_topk};
  stages[n++] = Stage{"sel_combine_kernel", ssa::launch_sel_combine};
  return n;
}

// every argument check of the forward except the workspace's
ssa_status check_forward_args(const ssa_blocks* blocks, const ssa_attn* attn, const void* q, const void* k,
                              const void* v, const void* gates, const void* out) {
  if (!blocks) return fail(SSA_ERR_INVALID_ARGUMENT, "blocks is null");
  ssa_status st = check_attn(attn);
  if (st != SSA_OK) return st;
  if (blocks->n_tokens < 0 || blocks->n_tokens > 0x7FFFFFFE || blocks->batch < 1)
    return fail(SSA_ERR_INVALID_ARGUMENT, "blocks were not built (n_tokens %lld, batch %d)",
                static_cast<long long>(blocks->n_tokens), blocks->batch);
  if (!blocks->perm || !blocks->blk_off || !blocks->win_off || !blocks->seq_blk_off ||
      !blocks->seq_win_off || !blocks->counts)
    return fail(SSA_ERR_INVALID_ARGUMENT, "a device buffer of blocks is null");
  if (blocks->n_tokens > 0 && (!q || !k || !v || !gates || !out))
    return fail(SSA_ERR_INVALID_ARGUMENT, "q, k, v, gates and out must be non-null");
  if (attn->routing == SSA_ROUTE_GEOMETRIC) {
    if (!use_mfma_path(attn))
      return fail(SSA_ERR_UNSUPPORTED, "geometric routing needs a bfloat16 layout of the MFMA path");
    if (blocks->n_tokens > 0 && !blocks->coords)
      return fail(SSA_ERR_INVALID_ARGUMENT, "geometric routing needs the blocks' coordinates");
  }
  return SSA_OK;
}

// side_by_side: run the probe-set selection on a second stream beside the
// window kernel (the timed and allocation-free forwards run every kernel in
// order on the caller's stream)
ssa_status forward_impl(const ssa_blocks* blocks, const ssa_attn* attn, const void* q, const void* k,
                        const void* v, const void* gates, void* out, void* k_cmp, void* v_cmp,
                        int32_t* topk_idx, void* workspace, size_t ws_bytes, void* hip_stream,
                        float* stage_ms, int32_t* n_stages, float* lse = nullptr, bool side_by_side = false) {
  ssa_status st = check_forward_args(blocks, attn, q, k, v, gates, out);
  if (st != SSA_OK) return st;
  const size_t need = forward_ws_bytes(blocks, attn);
  if (!workspace || ws_bytes < need)
    return fail(SSA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace ? ws_bytes : 0, need);
  if (stage_ms)
    for (int i = 0; i < SSA_STAGES; ++i) stage_ms[i] = 0.f;
  if (n_stages) *n_stages = 0;
  if (blocks->n_tokens == 0) return ok();

  const int64_t cap = nb_capacity(blocks);
  const FwdLayout lay = forward_layout(blocks, attn);
  char* w = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(workspace) + 255) & ~uintptr_t(255));
  ssa::FwdParams p{};
  p.perm = blocks->perm;
  p.blk_off = blocks->blk_off;
  p.win_off = blocks->win_off;
  p.seq_blk_off = blocks->seq_blk_off;
  p.seq_win_off = blocks->seq_win_off;
  p.counts = blocks->counts;
  p.n = static_cast<int32_t>(blocks->n_tokens);
  p.batch = blocks->batch;
  p.nb_cap = static_cast<int32_t>(cap);
  p.h_q = attn->h_q;
  p.h_kv = attn->h_kv;
  p.d = attn->head_dim;
  p.topk = attn->topk;
  p.scale = attn->scale > 0.f ? attn->scale : 1.0f / sqrtf(static_cast<float>(attn->head_dim));
  p.q = q;
  p.k = k;
  p.v = v;
  p.gates = gates;
  p.out = out;
  p.kbar = w + lay.kbar;
  p.vbar = w + lay.vbar;
  p.k_cmp = k_cmp;
  p.v_cmp = v_cmp;
  p.topk_idx = topk_idx ? topk_idx : reinterpret_cast<int32_t*>(w + lay.topk);
  p.lse = lse;
  if (use_mfma_path(attn)) {
    p.vbar_t = w + lay.vbar_t;
    p.k_s = w + lay.k_s;
    p.v_s = w + lay.v_s;
    p.tile_pre = reinterpret_cast<int32_t*>(w + lay.tile_pre);
    p.fix = reinterpret_cast<int32_t*>(w + lay.fix);
    p.acc = reinterpret_cast<float*>(w + lay.acc);
    p.max_tiles = static_cast<int32_t>(blocks->n_tokens / ssa::kQueryTile + blocks->batch + 1);
    if (use_gqa_path(attn)) {
      p.norm = reinterpret_cast<float*>(w + lay.norm);
      p.tile_pre2 = reinterpret_cast<int32_t*>(w + lay.tile_pre2);
      p.max_tiles2 = static_cast<int32_t>(blocks->n_tokens / 16 + blocks->batch + 1);
      p.knorm2 = reinterpret_cast<float*>(w + lay.knorm2);
      p.seq_kmax2 = reinterpret_cast<float*>(w + lay.seq_kmax2);
      p.probe_slot = reinterpret_cast<int32_t*>(w + lay.probe_slot);
      p.probe_seq = reinterpret_cast<int32_t*>(w + lay.probe_seq);
      p.probe_maxn2 = reinterpret_cast<float*>(w + lay.probe_maxn2);
      p.probe_ids = reinterpret_cast<int32_t*>(w + lay.probe_ids);
      p.max_probe_slots = max_probe_slots(blocks);
    } else {
      p.knorm2 = reinterpret_cast<float*>(w + lay.knorm2);
      p.probe_slot = reinterpret_cast<int32_t*>(w + lay.probe_slot);
      p.probe_seq = reinterpret_cast<int32_t*>(w + lay.probe_seq);
      p.probe_maxn2 = reinterpret_cast<float*>(w + lay.probe_maxn2);
      p.probe = w + lay.probe;
      p.max_probe_slots = max_probe_slots(blocks);
    }
    if (attn->routing == SSA_ROUTE_GEOMETRIC) {
      p.coords = blocks->coords;
      p.blk_cell = reinterpret_cast<int4*>(w + lay.blk_cell);
      p.l_cmp = ilog2(blocks->geo.m_cmp);
    }
  }

  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  Stage stages[SSA_STAGES];
  const int ns = forward_plan(attn, stages);
  hipEvent_t ev[SSA_STAGES + 1] = {};
  hipError_t e = hipSuccess;
  if (stage_ms) {
    for (int i = 0; i <= ns && e == hipSuccess; ++i) e = hipEventCreate(&ev[i]);
    if (e == hipSuccess) e = hipEventRecord(ev[0], stream);
  }
  // the MFMA plans start with pooling, the transpose of the pooled values,
  // the window kernel and (one head per group) the probe stage: the transpose
  // and the probe stage run beside the window kernel, joined before the
  // compressed kernels
  SideStream* side = nullptr;
  if (side_by_side && !stage_ms && ns > 3 && stages[1].launch == ssa::launch_vt_transpose &&
      stages[2].launch == ssa::launch_win_mfma)
    side = side_stream();
  if (side) {
    const bool probe = stages[3].launch == ssa::launch_cmp_probe;
    e = stages[0].launch(p, attn->dtype, stream);
    if (e == hipSuccess) e = hipEventRecord(side->fork, stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(side->stream, side->fork, 0);
    if (e == hipSuccess) e = stages[1].launch(p, attn->dtype, side->stream);
    if (e == hipSuccess && probe) e = stages[3].launch(p, attn->dtype, side->stream);
    if (e == hipSuccess) e = hipEventRecord(side->join, side->stream);
    if (e == hipSuccess) e = stages[2].launch(p, attn->dtype, stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(stream, side->join, 0);
    for (int i = probe ? 4 : 3; i < ns && e == hipSuccess; ++i) e = stages[i].launch(p, attn->dtype, stream);
  } else {
    for (int i = 0; i < ns && e == hipSuccess; ++i) {
      e = stages[i].launch(p, attn->dtype, stream);
      if (e == hipSuccess && stage_ms) e = hipEventRecord(ev[i + 1], stream);
    }
  }
  if (stage_ms) {
    if (e == hipSuccess) e = hipEventSynchronize(ev[ns]);
    for (int i = 0; i < ns && e == hipSuccess; ++i) e = hipEventElapsedTime(&stage_ms[i], ev[i], ev[i + 1]);
    for (int i = 0; i <= ns; ++i)
      if (ev[i]) hipEventDestroy(ev[i]);
  }
  if (e != hipSuccess) return fail(SSA_ERR_DEVICE, "forward launch failed: %s", hipGetErrorString(e));
  if (n_stages) *n_stages = ns;
  return ok();
}

}  // namespace

extern "C" {

ssa_status ssa_forward(const ssa_blocks* blocks, const ssa_attn* attn, const void* q, const void* k,
                       const void* v, const void* gates, void* out, void* k_cmp, void* v_cmp,
                       int32_t* topk_idx, void* workspace, size_t ws_bytes, void* hip_stream) {
  return forward_impl(blocks, attn, q, k, v, gates, out, k_cmp, v_cmp, topk_idx, workspace, ws_bytes,
                      hip_stream, nullptr, nullptr, nullptr, true);
}

ssa_status ssa_forward_timed(const ssa_blocks* blocks, const ssa_attn* attn, const void* q,
                             const void* k, const void* v, const void* gates, void* out,
                             void* k_cmp, void* v_cmp, int32_t* topk_idx, void* workspace,
                             size_t ws_bytes, void* hip_stream, float* stage_ms, int32_t* n_stages) {
  if (!stage_ms) return fail(SSA_ERR_INVALID_ARGUMENT, "stage_ms is null");
  return forward_impl(blocks, attn, q, k, v, gates, out, k_cmp, v_cmp, topk_idx, workspace, ws_bytes,
                      hip_stream, stage_ms, n_stages);
}

ssa_status ssa_forward_train(const ssa_blocks* blocks, const ssa_attn* attn, const void* q,
                             const void* k, const void* v, const void* gates, void* out,
                             int32_t* topk_idx, float* lse, void* workspace, size_t ws_bytes,
                             void* hip_stream) {
  if (!topk_idx || !lse) return fail(SSA_ERR_INVALID_ARGUMENT, "topk_idx and lse must be non-null");
  return forward_impl(blocks, attn, q, k, v, gates, out, nullptr, nullptr, topk_idx, workspace, ws_bytes,
                      hip_stream, nullptr, nullptr, lse, true);
}

}  // extern "C"

// ---------------------------------------------------------------- allocation-free forward

namespace {

// The workspace of ssa_forward_noalloc.  In host code this name is only a
// stand-in for the symbol: the device address comes from hipGetSymbolAddress,
// once per device, and only that address is ever handed to a kernel.
__device__ __align__(256) unsigned char scratch[SSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// device address of this device's copy of `scratch` (null on failure, with
// the error recorded)
void* scratch_address() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    fail(SSA_ERR_DEVICE, "hipGetDevice failed: %s", hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    fail(SSA_ERR_DEVICE, "device %d is beyond the %d devices the scratch table holds", dev, kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      fail(SSA_ERR_DEVICE, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

ssa_status ssa_forward_noalloc(const ssa_blocks* blocks, const ssa_attn* attn, const void* q, const void* k,
                               const void* v, const void* gates, void* out, void* k_cmp, void* v_cmp,
                               int32_t* topk_idx, void* hip_stream) {
  ssa_status st = check_forward_args(blocks, attn, q, k, v, gates, out);
  if (st != SSA_OK) return st;
  // forward_layout aligns the workspace start to 256 bytes itself; the array
  // is 256-aligned, so the whole array is usable
  const size_t need = forward_ws_bytes(blocks, attn);
  if (need > SSA_NOALLOC_SCRATCH_BYTES)
    return fail(SSA_ERR_WORKSPACE, "forward needs %zu bytes of scratch, above the %zu of the allocation-free entry",
                need, static_cast<size_t>(SSA_NOALLOC_SCRATCH_BYTES));
  void* ws = scratch_address();
  if (!ws) return SSA_ERR_DEVICE;
  return forward_impl(blocks, attn, q, k, v, gates, out, k_cmp, v_cmp, topk_idx, ws, SSA_NOALLOC_SCRATCH_BYTES,
                      hip_stream, nullptr, nullptr);
}

const char* ssa_stage_name(const ssa_attn* attn, int32_t stage) {
  if (!attn || stage < 0 || stage >= SSA_STAGES) return "";
  Stage stages[SSA_STAGES];
  const int ns = forward_plan(attn, stages);
  return stage < ns ? stages[stage].name : "";
}

}  // extern "C"

// ---------------------------------------------------------------- backward

namespace {

struct BwdLayout {
  size_t kbar, vbar, k_s, v_s, delta, dq_acc, dk_acc, dv_acc, dkbar, dvbar, sel_keys, sel_vals, sel_keys_tmp,
      sel_vals_tmp, sel_hist, sel_off, qtile_pre, btile_pre, seq_order, dkbar_part, dvbar_part, q_rows, do_rows,
      st_rows, total;
};

// the sorted (query, head) rows of one group, rounded up to whole 32-row tiles
int64_t rows_capacity(const ssa_blocks* b, const ssa_attn* a) {
  return (b->n_tokens * (a->h_q / a->h_kv) + 31) / 32 * 32;
}

// 128-block chunks (an upper bound) and the row splits that give the
// pooled-row gradient kernel about 8192 workgroups
int32_t max_block_chunks(const ssa_blocks* b) { return static_cast<int32_t>(nb_capacity(b) / 128 + 2 * b->batch + 2); }
int32_t dkv_row_splits(const ssa_blocks* b, const ssa_attn* a) {
  const int64_t wg = static_cast<int64_t>(max_block_chunks(b)) * a->h_kv;
  const int64_t s = (8192 + wg - 1) / wg;
  return static_cast<int32_t>(s < 1 ? 1 : (s > 32 ? 32 : s));
}

// bits of the inverted-list sort keys: group * nb_cap + block, plus the
// padding key h_kv * nb_cap
int sel_key_bits(const ssa_blocks* b, const ssa_attn* a) {
  return ceil_log2(static_cast<int64_t>(a->h_kv) * nb_capacity(b) + 1);
}

// the compressed branch's backward runs on MFMA for bfloat16 (D = 32 or 64)
bool use_mfma_backward(const ssa_attn* a) { return a->dtype == SSA_BF16; }

BwdLayout backward_layout(const ssa_blocks* b, const ssa_attn* a) {
  const size_t cap = static_cast<size_t>(nb_capacity(b));
  const size_t n = static_cast<size_t>(b->n_tokens);
  const size_t eb = static_cast<size_t>(elt_bytes(a->dtype));
  const size_t D = static_cast<size_t>(a->head_dim);
  const size_t pooled = align256(eb * a->h_kv * cap * D);
  const size_t sorted = align256(eb * a->h_kv * n * D);
  BwdLayout L{};
  size_t off = 0;
  L.kbar = off; off += pooled;
  L.vbar = off; off += pooled;
  L.k_s = off; off += sorted;
  L.v_s = off; off += sorted;
  L.delta = off; off += align256(sizeof(float) * 3 * n * a->h_q);
  L.dq_acc = off; off += align256(sizeof(float) * n * a->h_q * D);
  L.dk_acc = off; off += align256(sizeof(float) * a->h_kv * n * D);
  L.dv_acc = off; off += align256(sizeof(float) * a->h_kv * n * D);
  L.dkbar = off; off += align256(sizeof(float) * a->h_kv * cap * D);
  L.dvbar = off; off += align256(sizeof(float) * a->h_kv * cap * D);
  const size_t m = n * a->h_kv * a->topk;
  L.sel_keys = off; off += align256(sizeof(uint32_t) * m);
  L.sel_vals = off; off += align256(sizeof(int32_t) * m);
  L.sel_keys_tmp = off; off += align256(sizeof(uint32_t) * m);
  L.sel_vals_tmp = off; off += align256(sizeof(int32_t) * m);
  L.sel_hist = off; off += align256(ssa::sort_pairs_hist_bytes(static_cast<int64_t>(m)));
  L.sel_off = off; off += align256(sizeof(int32_t) * (a->h_kv * cap + 1));
  if (use_mfma_backward(a)) {
    L.qtile_pre = off; off += align256(sizeof(int32_t) * (static_cast<size_t>(b->batch) + 1));
    L.btile_pre = off; off += align256(sizeof(int32_t) * (static_cast<size_t>(b->batch) + 1));
    L.seq_order = off; off += align256(sizeof(int32_t) * (static_cast<size_t>(b->batch) + 1));
    const size_t rows = static_cast<size_t>(a->h_kv) * static_cast<size_t>(rows_capacity(b, a));
    L.q_rows = off; off += align256(eb * rows * D);
    L.do_rows = off; off += align256(eb * rows * D);
    L.st_rows = off; off += align256(4 * sizeof(float) * 2 * rows);
    const size_t splits = static_cast<size_t>(dkv_row_splits(b, a));
    if (splits > 1) {
      L.dkbar_part = off; off += align256(sizeof(float) * splits * a->h_kv * cap * D);
      L.dvbar_part = off; off += align256(sizeof(float) * splits * a->h_kv * cap * D);
    }
  }
  L.total = off + 256;
  return L;
}

struct BStage {
  const char* name;
  hipError_t (*launch)(const ssa::BwdParams&, ssa_dtype, hipStream_t);
};

int backward_plan(const ssa_attn* attn, BStage* stages) {
  int n = 0;
  stages[n++] = BStage{"pool_kernel", ssa::launch_bwd_pool};
  stages[n++] = BStage{"sel_index", ssa::launch_bwd_sel_index};
  if (use_mfma_backward(attn)) {
    // the three dq kernels (which also give Delta), then the key / value
    // gradients over the sorted rows
    stages[n++] = BStage{"cmp_dq_mfma_kernel", ssa::launch_bwd_cmp_dq_mfma};
    stages[n++] = BStage{"win_dq_mfma_kernel", ssa::launch_bwd_win_dq_mfma};
    stages[n++] = BStage{"sel_dq_kernel", ssa::launch_bwd_sel_dq};
    stages[n++] = BStage{"rows_prep_kernel", ssa::launch_bwd_rows_prep};
    stages[n++] = BStage{"cmp_dkv_mfma_kernel", ssa::launch_bwd_cmp_dkv_mfma};
    stages[n++] = BStage{"win_dkv_mfma_kernel", ssa::launch_bwd_kv_win_mfma};
    stages[n++] = BStage{"kv_grad_mfma_kernel", ssa::launch_bwd_kv_sel_mfma};
  } else {
    stages[n++] = BStage{"cmp_dq_kernel", ssa::launch_bwd_cmp_dq};
    stages[n++] = BStage{"cmp_dkv_kernel", ssa::launch_bwd_cmp_dkv};
    stages[n++] = BStage{"win_dq_kernel", ssa::launch_bwd_win_dq};
    stages[n++] = BStage{"win_dkv_kernel", ssa::launch_bwd_win_dkv};
    stages[n++] = BStage{"sel_dq_kernel", ssa::launch_bwd_sel_dq};
    stages[n++] = BStage{"sel_dkv_kernel", ssa::launch_bwd_sel_dkv};
  }
  stages[n++] = BStage{"bwd_finalize_kernel", ssa::launch_bwd_finalize};
  return n;
}

ssa_status backward_impl(const ssa_blocks* blocks, const ssa_attn* attn, const void* q, const void* k,
                         const void* v, const void* gates, const void* dout, const int32_t* topk_idx,
                         const float* lse, void* dq, void* dk, void* dv, void* dgates, void* workspace,
                         size_t ws_bytes, void* hip_stream, float* stage_ms, int32_t* n_stages) {
  if (!blocks) return fail(SSA_ERR_INVALID_ARGUMENT, "blocks is null");
  ssa_status st = check_attn(attn);
  if (st != SSA_OK) return st;
  if (blocks->n_tokens < 0 || blocks->n_tokens > 0x7FFFFFFE || blocks->batch < 1)
    return fail(SSA_ERR_INVALID_ARGUMENT, "blocks were not built (n_tokens %lld, batch %d)",
                static_cast<long long>(blocks->n_tokens), blocks->batch);
  if (!blocks->perm || !blocks->blk_off || !blocks->win_off || !blocks->seq_blk_off ||
      !blocks->seq_win_off || !blocks->counts)
    return fail(SSA_ERR_INVALID_ARGUMENT, "a device buffer of blocks is null");
  if (blocks->n_tokens > 0 &&
      (!q || !k || !v || !gates || !dout || !topk_idx || !lse || !dq || !dk || !dv))
    return fail(SSA_ERR_INVALID_ARGUMENT, "q, k, v, gates, dout, topk_idx, lse, dq, dk and dv must be non-null");
  if (blocks->n_tokens * attn->h_kv * attn->topk > 0x7FFFFFFF)
    return fail(SSA_ERR_UNSUPPORTED, "n_tokens * h_kv * topk exceeds 2^31 - 1 top-k entries");
  if (sel_key_bits(blocks, attn) > 32)
    return fail(SSA_ERR_UNSUPPORTED, "h_kv * blocks exceeds 2^32");
  const BwdLayout lay = backward_layout(blocks, attn);
  if (!workspace || ws_bytes < lay.total)
    return fail(SSA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace ? ws_bytes : 0, lay.total);
  if (stage_ms)
    for (int i = 0; i < SSA_STAGES; ++i) stage_ms[i] = 0.f;
  if (n_stages) *n_stages = 0;
  if (blocks->n_tokens == 0) return ok();

  char* w = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(workspace) + 255) & ~uintptr_t(255));
  ssa::BwdParams bp{};
  ssa::FwdParams& p = bp.f;
  p.perm = blocks->perm;
  p.blk_off = blocks->blk_off;
  p.win_off = blocks->win_off;
  p.seq_blk_off = blocks->seq_blk_off;
  p.seq_win_off = blocks->seq_win_off;
  p.counts = blocks->counts;
  p.n = static_cast<int32_t>(blocks->n_tokens);
  p.batch = blocks->batch;
  p.nb_cap = static_cast<int32_t>(nb_capacity(blocks));
  p.h_q = attn->h_q;
  p.h_kv = attn->h_kv;
  p.d = attn->head_dim;
  p.topk = attn->topk;
  p.scale = attn->scale > 0.f ? attn->scale : 1.0f / sqrtf(static_cast<float>(attn->head_dim));
  p.q = q;
  p.k = k;
  p.v = v;
  p.gates = gates;
  p.kbar = w + lay.kbar;
  p.vbar = w + lay.vbar;
  p.k_s = w + lay.k_s;
  p.v_s = w + lay.v_s;
  p.topk_idx = const_cast<int32_t*>(topk_idx);
  bp.dout = dout;
  bp.lse = lse;
  bp.dq = dq;
  bp.dk = dk;
  bp.dv = dv;
  bp.dgates = dgates;
  bp.delta = reinterpret_cast<float*>(w + lay.delta);
  bp.dq_acc = reinterpret_cast<float*>(w + lay.dq_acc);
  bp.dk_acc = reinterpret_cast<float*>(w + lay.dk_acc);
  bp.dv_acc = reinterpret_cast<float*>(w + lay.dv_acc);
  bp.dkbar = reinterpret_cast<float*>(w + lay.dkbar);
  bp.dvbar = reinterpret_cast<float*>(w + lay.dvbar);
  bp.sel_keys = reinterpret_cast<uint32_t*>(w + lay.sel_keys);
  bp.sel_vals = reinterpret_cast<int32_t*>(w + lay.sel_vals);
  bp.sel_keys_tmp = reinterpret_cast<uint32_t*>(w + lay.sel_keys_tmp);
  bp.sel_vals_tmp = reinterpret_cast<int32_t*>(w + lay.sel_vals_tmp);
  bp.sel_hist = reinterpret_cast<uint32_t*>(w + lay.sel_hist);
  bp.sel_key_bits = sel_key_bits(blocks, attn);
  const bool in_tmp = ssa::sort_pairs_lands_in_tmp(bp.sel_key_bits);
  bp.sel_list = in_tmp ? bp.sel_vals_tmp : bp.sel_vals;
  bp.sel_sorted_keys = in_tmp ? bp.sel_keys_tmp : bp.sel_keys;
  bp.sel_off = reinterpret_cast<int32_t*>(w + lay.sel_off);
  if (use_mfma_backward(attn)) {
    bp.qtile_pre = reinterpret_cast<int32_t*>(w + lay.qtile_pre);
    bp.btile_pre = reinterpret_cast<int32_t*>(w + lay.btile_pre);
    bp.seq_order = reinterpret_cast<int32_t*>(w + lay.seq_order);
    bp.max_qtiles = static_cast<int32_t>(blocks->n_tokens / 128 + blocks->batch + 1);
    bp.max_btiles = max_block_chunks(blocks);
    bp.row_splits = dkv_row_splits(blocks, attn);
    bp.rows_cap = static_cast<int32_t>(rows_capacity(blocks, attn));
    bp.q_rows = w + lay.q_rows;
    bp.do_rows = w + lay.do_rows;
    bp.st_rows = reinterpret_cast<float4*>(w + lay.st_rows);
    if (bp.row_splits > 1) {
      bp.dkbar_part = reinterpret_cast<float*>(w + lay.dkbar_part);
      bp.dvbar_part = reinterpret_cast<float*>(w + lay.dvbar_part);
    }
  }

  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  BStage stages[SSA_STAGES];
  const int ns = backward_plan(attn, stages);
  hipEvent_t ev[SSA_STAGES + 1] = {};
  hipError_t e = hipSuccess;
  if (stage_ms) {
    for (int i = 0; i <= ns && e == hipSuccess; ++i) e = hipEventCreate(&ev[i]);
    if (e == hipSuccess) e = hipEventRecord(ev[0], stream);
  }
  for (int i = 0; i < ns && e == hipSuccess; ++i) {
    e = stages[i].launch(bp, attn->dtype, stream);
    if (e == hipSuccess && stage_ms) e = hipEventRecord(ev[i + 1], stream);
  }
  if (stage_ms) {
    if (e == hipSuccess) e = hipEventSynchronize(ev[ns]);
    for (int i = 0; i < ns && e == hipSuccess; ++i) e = hipEventElapsedTime(&stage_ms[i], ev[i], ev[i + 1]);
    for (int i = 0; i <= ns; ++i)
      if (ev[i]) hipEventDestroy(ev[i]);
  }
  if (e != hipSuccess) return fail(SSA_ERR_DEVICE, "backward launch failed: %s", hipGetErrorString(e));
  if (n_stages) *n_stages = ns;
  return ok();
}

}  // namespace

extern "C" {

size_t ssa_backward_workspace(const ssa_blocks* blocks, const ssa_attn* attn) {
  if (!blocks || !attn || blocks->n_tokens < 0 || attn->h_kv < 1 || attn->h_q < 1 || attn->head_dim < 1 ||
      attn->topk < 1)
    return 0;
  return backward_layout(blocks, attn).total;
}

ssa_status ssa_backward(const ssa_blocks* blocks, const ssa_attn* attn, const void* q, const void* k,
                        const void* v, const void* gates, const void* dout, const int32_t* topk_idx,
                        const float* lse, void* dq, void* dk, void* dv, void* dgates, void* workspace,
                        size_t ws_bytes, void* hip_stream) {
  return backward_impl(blocks, attn, q, k, v, gates, dout, topk_idx, lse, dq, dk, dv, dgates, workspace,
                       ws_bytes, hip_stream, nullptr, nullptr);
}

ssa_status ssa_backward_timed(const ssa_blocks* blocks, const ssa_attn* attn, const void* q, const void* k,
                              const void* v, const void* gates, const void* dout, const int32_t* topk_idx,
                              const float* lse, void* dq, void* dk, void* dv, void* dgates,
                              void* workspace, size_t ws_bytes, void* hip_stream, float* stage_ms,
                              int32_t* n_stages) {
  if (!stage_ms) return fail(SSA_ERR_INVALID_ARGUMENT, "stage_ms is null");
  return backward_impl(blocks, attn, q, k, v, gates, dout, topk_idx, lse, dq, dk, dv, dgates, workspace,
                       ws_bytes, hip_stream, stage_ms, n_stages);
}

const char* ssa_backward_stage_name(const ssa_attn* attn, int32_t stage) {
  if (!attn || stage < 0 || stage >= SSA_STAGES) return "";
  BStage stages[SSA_STAGES];
  const int ns = backward_plan(attn, stages);
  return stage < ns ? stages[stage].name : "";
}

}  // extern "C"
