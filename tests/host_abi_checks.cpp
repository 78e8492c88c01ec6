// Drives every host-side validation path of libssa's C ABI (no GPU work is
// launched: each call fails its argument checks before enqueueing anything, or
// only sizes a workspace).  Built with AddressSanitizer and UBSan on the host
// code by tests/test_host_sanitizers.py; any sanitizer report fails the test.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ssa.h"

static int g_fail = 0, g_checks = 0;
#define CHECK(cond)                                              \
  do {                                                           \
    ++g_checks;                                                  \
    if (!(cond)) {                                               \
      ++g_fail;                                                  \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
    }                                                            \
  } while (0)

static void* const kFake = reinterpret_cast<void*>(0x100000);   // never dereferenced

static ssa_blocks fake_blocks(int64_t n, int32_t batch, int32_t nb) {
  ssa_blocks b;
  memset(&b, 0, sizeof(b));
  int32_t* f = static_cast<int32_t*>(kFake);
  b.perm = b.blk_off = b.win_off = b.win_blk_off = b.seq_blk_off = b.seq_win_off = b.counts = f;
  b.n_tokens = n;
  b.batch = batch;
  b.nb = nb;
  b.nw = -1;
  return b;
}

// dtype as the integer a C caller stores (7 is no enumerator)
static ssa_attn attn(int hq, int hkv, int d, int k, int dtype = SSA_BF16, float scale = 0.f, int routing = 0) {
  ssa_attn a;
  memset(&a, 0, sizeof(a));
  a.h_q = hq;
  a.h_kv = hkv;
  a.head_dim = d;
  a.topk = k;
  a.scale = scale;
  memcpy(&a.dtype, &dtype, sizeof(dtype));
  a.routing = routing;
  return a;
}

static int build(int64_t n, int32_t batch, ssa_geometry g, bool out = true, const void* coords = kFake,
                 const void* cu = kFake, void* ws = nullptr, size_t ws_bytes = 0) {
  ssa_blocks b = fake_blocks(0, 0, -1);
  return ssa_build_blocks(static_cast<const int32_t*>(coords), static_cast<const int32_t*>(cu), n, batch, &g,
                          out ? &b : nullptr, 1, ws, ws_bytes, nullptr);
}

int main() {
  CHECK(ssa_version() == 100);
  for (int s = 0; s < 6; ++s) CHECK(ssa_status_string(static_cast<ssa_status>(s)) != nullptr);
  CHECK(strcmp(ssa_status_string(SSA_OK), "ok") == 0);

  // block build: geometry, sizes, pointers, key width, workspace
  const ssa_geometry bad_geo[] = {{63, 4, 8, 0}, {64, 3, 8, 0}, {64, 8, 4, 0}, {2048, 4, 8, 0}, {64, 4, 128, 0},
                                  {64, 4, 8, 2}, {64, 4, 8, 8}, {64, 4, 8, -4}, {64, 8, 8, 4}};
  for (const ssa_geometry& g : bad_geo) {
    CHECK(build(100, 1, g) == SSA_ERR_INVALID_ARGUMENT);
    CHECK(strlen(ssa_last_error()) > 0);
  }
  const ssa_geometry g64 = {64, 4, 8, 0};
  CHECK(build(-1, 1, g64) == SSA_ERR_INVALID_ARGUMENT);
  CHECK(build(0x7FFFFFFFLL + 5, 1, g64) == SSA_ERR_INVALID_ARGUMENT);
  CHECK(build(100, 0, g64) == SSA_ERR_INVALID_ARGUMENT);
  CHECK(build(100, 1, g64, false) == SSA_ERR_INVALID_ARGUMENT);
  CHECK(build(100, 1, g64, true, nullptr) == SSA_ERR_INVALID_ARGUMENT);
  CHECK(build(100, 1, g64, true, kFake, nullptr) == SSA_ERR_INVALID_ARGUMENT);
  CHECK(build(100, 8, ssa_geometry{1024, 1, 8, 0}) == SSA_ERR_UNSUPPORTED);
  CHECK(build(100, 1 << 30, ssa_geometry{1024, 4, 8, 0}) == SSA_ERR_UNSUPPORTED);
  const size_t need_b = ssa_build_blocks_workspace(100000, 1, &g64);
  CHECK(need_b >= size_t(3) * 4 * 100000);
  CHECK(build(100000, 1, g64) == SSA_ERR_WORKSPACE);
  CHECK(build(100000, 1, g64, true, kFake, kFake, kFake, need_b - 1) == SSA_ERR_WORKSPACE);
  CHECK(ssa_build_blocks_workspace(-5, 1, &g64) == 0);
  CHECK(ssa_build_blocks_workspace(0x7FFFFFFELL, 1 << 20, &g64) > size_t(0x7FFFFFFE) * 8);

  // forward: layouts, pointers, workspace
  struct Bad { ssa_attn a; int st; } bad[] = {
      {attn(16, 16, 48, 16), SSA_ERR_UNSUPPORTED},         {attn(16, 16, 128, 16), SSA_ERR_UNSUPPORTED},
      {attn(16, 16, 64, 0), SSA_ERR_INVALID_ARGUMENT},      {attn(16, 16, 64, 33), SSA_ERR_UNSUPPORTED},
      {attn(16, 3, 64, 16), SSA_ERR_INVALID_ARGUMENT},      {attn(0, 16, 64, 16), SSA_ERR_INVALID_ARGUMENT},
      {attn(64, 1, 64, 16), SSA_ERR_UNSUPPORTED},           {attn(16, 16, 64, 16, 7), SSA_ERR_INVALID_ARGUMENT},
      {attn(16, 16, 64, 16, SSA_BF16, 1.f / 0.f), SSA_ERR_INVALID_ARGUMENT},
      {attn(16, 16, 64, 16, SSA_BF16, 0.f, 5), SSA_ERR_INVALID_ARGUMENT},
      {attn(16, 16, 64, 16, SSA_F32, 0.f, 1), SSA_ERR_UNSUPPORTED},
      {attn(32, 1, 64, 16, SSA_BF16, 0.f, 1), SSA_ERR_UNSUPPORTED},   // geometric routing off the MFMA layouts
      {attn(16, 16, 64, 16, SSA_BF16, 0.f, 1), SSA_ERR_INVALID_ARGUMENT},   // no coordinates in the blocks
  };
  ssa_blocks fb = fake_blocks(1000, 1, -1);
  for (const Bad& x : bad) {
    CHECK(ssa_forward(&fb, &x.a, kFake, kFake, kFake, kFake, kFake, nullptr, nullptr, nullptr, nullptr, 0,
                      nullptr) == x.st);
    CHECK(strlen(ssa_last_error()) > 0);
    CHECK(ssa_forward_noalloc(&fb, &x.a, kFake, kFake, kFake, kFake, kFake, nullptr, nullptr, nullptr,
                              nullptr) == x.st);
  }
  const ssa_attn a = attn(16, 16, 64, 16);
  CHECK(ssa_forward(nullptr, &a, kFake, kFake, kFake, kFake, kFake, nullptr, nullptr, nullptr, nullptr, 0,
                    nullptr) == SSA_ERR_INVALID_ARGUMENT);
  CHECK(ssa_forward(&fb, nullptr, kFake, kFake, kFake, kFake, kFake, nullptr, nullptr, nullptr, nullptr, 0,
                    nullptr) == SSA_ERR_INVALID_ARGUMENT);
  CHECK(ssa_forward(&fb, &a, nullptr, kFake, kFake, kFake, kFake, nullptr, nullptr, nullptr, nullptr, 0,
                    nullptr) == SSA_ERR_INVALID_ARGUMENT);
  CHECK(ssa_forward(&fb, &a, kFake, kFake, kFake, kFake, kFake, nullptr, nullptr, nullptr, nullptr, 0,
                    nullptr) == SSA_ERR_WORKSPACE);
  float ms[SSA_STAGES];
  int32_t ns = 0;
  CHECK(ssa_forward_timed(&fb, &a, kFake, kFake, kFake, kFake, kFake, nullptr, nullptr, nullptr, nullptr, 0,
                          nullptr, nullptr, &ns) == SSA_ERR_INVALID_ARGUMENT);
  CHECK(ssa_forward_timed(&fb, &a, kFake, kFake, kFake, kFake, kFake, nullptr, nullptr, nullptr, nullptr, 0,
                          nullptr, ms, &ns) == SSA_ERR_WORKSPACE);
  CHECK(ssa_forward_train(&fb, &a, kFake, kFake, kFake, kFake, kFake, nullptr, static_cast<float*>(kFake), kFake,
                          size_t(1) << 40, nullptr) == SSA_ERR_INVALID_ARGUMENT);
  CHECK(ssa_forward_train(&fb, &a, kFake, kFake, kFake, kFake, kFake, static_cast<int32_t*>(kFake), nullptr, kFake,
                          size_t(1) << 40, nullptr) == SSA_ERR_INVALID_ARGUMENT);
  ssa_blocks fb50 = fake_blocks(1000, 1, 50);
  const size_t need_f = ssa_forward_workspace(&fb50, &a);
  CHECK(need_f >= size_t(2) * 50 * 16 * 64 * 2 + size_t(1000) * 16 * 16 * 4);
  CHECK(ssa_forward_workspace(&fb, &a) > need_f);
  CHECK(ssa_forward_workspace(nullptr, &a) == 0);
  // workspace sizes at the largest token count and batch (size_t arithmetic)
  ssa_blocks huge = fake_blocks(0x7FFFFFFE, 1 << 20, -1);
  const ssa_attn ag = attn(32, 2, 32, 32);
  CHECK(ssa_forward_workspace(&huge, &a) > size_t(0x7FFFFFFE) * 16 * 64 * 4);
  CHECK(ssa_forward_workspace(&huge, &ag) > size_t(0x7FFFFFFE) * 32 * 32 * 4);
  CHECK(ssa_backward_workspace(&huge, &a) > ssa_forward_workspace(&huge, &a));
  // the allocation-free forward: inputs beyond its scratch are refused
  ssa_blocks big = fake_blocks(60000, 1, -1);
  CHECK(ssa_forward_workspace(&big, &a) > SSA_NOALLOC_SCRATCH_BYTES);
  CHECK(ssa_forward_noalloc(&big, &a, kFake, kFake, kFake, kFake, kFake, nullptr, nullptr, nullptr, nullptr) ==
        SSA_ERR_WORKSPACE);
  CHECK(ssa_forward_noalloc(nullptr, &a, kFake, kFake, kFake, kFake, kFake, nullptr, nullptr, nullptr, nullptr) ==
        SSA_ERR_INVALID_ARGUMENT);
  for (int s = -1; s < SSA_STAGES + 2; ++s) CHECK(ssa_stage_name(&a, s) != nullptr);
  CHECK(strcmp(ssa_stage_name(&a, 0), "pool_kernel") == 0);
  CHECK(strcmp(ssa_stage_name(nullptr, 0), "") == 0);

  // backward
  struct BadB { ssa_attn a; int st; } badb[] = {
      {attn(16, 16, 48, 16), SSA_ERR_UNSUPPORTED}, {attn(16, 16, 64, 0), SSA_ERR_INVALID_ARGUMENT},
      {attn(16, 3, 64, 16), SSA_ERR_INVALID_ARGUMENT}, {attn(16, 16, 64, 16, 7), SSA_ERR_INVALID_ARGUMENT},
  };
  const int32_t* fi = static_cast<const int32_t*>(kFake);
  const float* ff = static_cast<const float*>(kFake);
  for (const BadB& x : badb) {
    CHECK(ssa_backward(&fb, &x.a, kFake, kFake, kFake, kFake, kFake, fi, ff, kFake, kFake, kFake, nullptr, nullptr,
                       0, nullptr) == x.st);
  }
  CHECK(ssa_backward(nullptr, &a, kFake, kFake, kFake, kFake, kFake, fi, ff, kFake, kFake, kFake, nullptr, nullptr,
                     0, nullptr) == SSA_ERR_INVALID_ARGUMENT);
  CHECK(ssa_backward(&fb, &a, kFake, kFake, kFake, kFake, kFake, fi, nullptr, kFake, kFake, kFake, nullptr, nullptr,
                     0, nullptr) == SSA_ERR_INVALID_ARGUMENT);
  CHECK(ssa_backward(&fb, &a, kFake, kFake, kFake, kFake, kFake, fi, ff, kFake, kFake, kFake, nullptr, nullptr, 0,
                     nullptr) == SSA_ERR_WORKSPACE);
  CHECK(ssa_backward_timed(&fb, &a, kFake, kFake, kFake, kFake, kFake, fi, ff, kFake, kFake, kFake, nullptr, nullptr,
                           0, nullptr, nullptr, nullptr) == SSA_ERR_INVALID_ARGUMENT);
  CHECK(ssa_backward_workspace(&fb50, &a) >= size_t(4) * 1000 * 16 * 64 * 3);
  CHECK(strcmp(ssa_backward_stage_name(&a, 0), "pool_kernel") == 0);
  CHECK(strcmp(ssa_backward_stage_name(&a, 99), "") == 0);

  printf("%d checks, %d failed\n", g_checks, g_fail);
  return g_fail ? 1 : 0;
}
