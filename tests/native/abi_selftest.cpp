// Host-side self-test of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (tests/test_host_sanitized.py).
// It sweeps the planners and workspace queries over ordinary and extreme
// shapes (including sizes whose products overflow 32 bits) and drives every
// entry point into each argument check, so that an out-of-bounds access, a
// signed overflow or a bad shift in that host code stops the program.  No
// kernel is launched: every call here is planned or rejected on the host.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <string>
#include <thread>
#include <vector>

#include "osx.h"

static int g_failures = 0;
#define EXPECT(cond, ...)                                     \
  do {                                                        \
    if (!(cond)) {                                            \
      ++g_failures;                                           \
      std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      std::fprintf(stderr, __VA_ARGS__);                      \
      std::fprintf(stderr, "\n");                             \
    }                                                         \
  } while (0)

// Aligned addresses that are never dereferenced: every call that receives them
// is rejected before a launch.
static void* fake(uintptr_t a) { return reinterpret_cast<void*>(a); }

static void status_strings() {
  const int codes[] = {OSX_OK, OSX_EINVAL, OSX_EUNSUPPORTED, OSX_EHIP, OSX_EWORKSPACE};
  for (int c : codes) EXPECT(std::strncmp(osx_status_string(c), "OSX_", 4) == 0, "status %d", c);
  EXPECT(std::strcmp(osx_status_string(12345), "unknown status") == 0, "unknown status");
  EXPECT(std::strcmp(osx_status_string(INT_MIN), "unknown status") == 0, "INT_MIN status");
  EXPECT(osx_version() >= 100, "version");
}

static int attn_checks = 0;
static void attn_plans() {
  const int dtypes[] = {OSX_F32, OSX_BF16, 2, -1};
  const int batches[] = {0, 1, 2, 7, 64, INT_MAX, -1};
  const int heads[][2] = {{1, 1}, {4, 1}, {32, 8}, {6, 4}, {4, 0}, {0, 4}, {INT_MAX, 1}, {1 << 20, 1 << 20}};
  const int seqs[] = {0, 1, 7, 64, 100, 4096, 1 << 20, INT_MAX, -3};
  const int dims[] = {0, 4, 16, 48, 64, 80, 128, 132, 256, -16};
  for (int dt : dtypes)
    for (int b : batches)
      for (auto& h : heads)
        for (int sq : seqs)
          for (int sk : seqs)
            for (int d : dims)
              for (int causal = 0; causal < 2; ++causal) {
                osx_plan p;
                std::memset(&p, 0xab, sizeof p);
                const int st = osx_attn_plan(dt, b, h[0], h[1], sq, sk, d, causal, &p);
                size_t ws = 12345;
                const int st2 = osx_attn_fwd_workspace(dt, b, h[0], h[1], sq, sk, d, causal, &ws);
                const size_t wb = osx_attn_fwd_workspace_bytes(dt, b, h[0], h[1], sq, sk, d, causal);
                EXPECT(st == st2, "plan %d vs workspace %d", st, st2);
                ++attn_checks;
                if (st == OSX_OK) {
                  EXPECT(ws == p.workspace_bytes && wb == ws, "workspace %zu / %zu / %zu", ws, wb, p.workspace_bytes);
                  EXPECT(p.grid >= 0, "grid %lld", (long long)p.grid);
                  EXPECT(p.kernel == OSX_KERNEL_NONE || (p.grid > 0 && p.threads > 0 && p.splits >= 1),
                         "plan kernel %d grid %lld threads %d splits %d", p.kernel, (long long)p.grid, p.threads,
                         p.splits);
                } else {
                  EXPECT(wb == 0 && ws == 0, "rejected shape reports workspace %zu / %zu", wb, ws);
                  EXPECT(osx_last_error()[0] != '\0', "no error detail");
                }
              }
  // a null plan pointer only skips the copy
  EXPECT(osx_attn_plan(OSX_F32, 1, 1, 1, 8, 8, 64, 0, nullptr) == OSX_OK, "null plan pointer");
}

static void attn_rejects() {
  void* q = fake(0x100000);
  void* k = fake(0x200000);
  void* v = fake(0x300000);
  void* o = fake(0x400000);
  // null pointers with work to do
  EXPECT(osx_attn_fwd(nullptr, k, v, o, OSX_BF16, 1, 4, 1, 64, 64, 128, 0, 0.f, nullptr, 0, nullptr) == OSX_EINVAL,
         "null q");
  EXPECT(osx_attn_fwd(q, k, v, nullptr, OSX_F32, 1, 1, 1, 64, 64, 64, 0, 0.f, nullptr, 0, nullptr) == OSX_EINVAL,
         "null o");
  // misaligned
  EXPECT(osx_attn_fwd(fake(0x100004), k, v, o, OSX_BF16, 1, 4, 1, 64, 64, 128, 0, 0.f, nullptr, 0, nullptr) ==
             OSX_EINVAL,
         "misaligned q");
  // output overlapping an input
  EXPECT(osx_attn_fwd(q, k, v, fake(0x100010), OSX_BF16, 1, 4, 1, 64, 64, 128, 0, 0.f, nullptr, 0, nullptr) ==
             OSX_EINVAL,
         "o overlaps q");
  // workspace missing or short where the plan needs one (one fp32 head: key split)
  const size_t need = osx_attn_fwd_workspace_bytes(OSX_F32, 1, 1, 1, 4096, 4096, 128, 0);
  EXPECT(need > 0, "fp32 single head needs a workspace");
  EXPECT(osx_attn_fwd(q, k, v, o, OSX_F32, 1, 1, 1, 4096, 4096, 128, 0, 0.f, nullptr, need, nullptr) ==
             OSX_EWORKSPACE,
         "null workspace");
  EXPECT(osx_attn_fwd(q, k, v, o, OSX_F32, 1, 1, 1, 4096, 4096, 128, 0, 0.f, fake(0x800000), need - 16, nullptr) ==
             OSX_EWORKSPACE,
         "short workspace");
  EXPECT(osx_attn_fwd(q, k, v, o, OSX_F32, 1, 1, 1, 4096, 4096, 128, 0, 0.f, fake(0x800008), need, nullptr) ==
             OSX_EINVAL,
         "misaligned workspace");
  // lse
  EXPECT(osx_attn_fwd_lse(q, k, v, o, nullptr, OSX_BF16, 1, 4, 1, 64, 64, 128, 0, 0.f, nullptr, 0, nullptr) ==
             OSX_EINVAL,
         "null lse");
  EXPECT(osx_attn_fwd_lse(q, k, v, o, (float*)fake(0x400002), OSX_BF16, 1, 4, 1, 64, 64, 128, 0, 0.f, nullptr, 0,
                          nullptr) == OSX_EINVAL,
         "misaligned lse");
  // a NaN, +inf or overflowing scale (scale * log2(e) past fp32) is rejected; <= 0 selects 1/sqrt(d)
  for (float bad : {std::numeric_limits<float>::quiet_NaN(), std::numeric_limits<float>::infinity(), 3.0e38f}) {
    EXPECT(osx_attn_fwd(q, k, v, o, OSX_BF16, 1, 4, 1, 64, 64, 128, 0, bad, nullptr, 0, nullptr) == OSX_EINVAL,
           "scale %g", (double)bad);
    EXPECT(osx_attn_fwd_normalised(q, k, v, o, nullptr, OSX_F32, 1, 1, 1, 64, 64, 64, 0, bad, nullptr, 0, nullptr) ==
               OSX_EINVAL,
           "normalised scale %g", (double)bad);
  }
  // the normalised-output recurrence is fp32 only
  EXPECT(osx_attn_fwd_normalised(q, k, v, o, nullptr, OSX_BF16, 1, 4, 1, 64, 64, 128, 0, 0.f, nullptr, 0, nullptr) ==
             OSX_EUNSUPPORTED,
         "normalised bf16");
  // no work: OK without any pointer
  EXPECT(osx_attn_fwd(nullptr, nullptr, nullptr, nullptr, OSX_BF16, 0, 4, 1, 64, 64, 128, 0, 0.f, nullptr, 0,
                      nullptr) == OSX_OK,
         "no work");
  // the allocation-free variant: a plan beyond its static scratch is refused
  // (one fp32 head of 65408 rows: two key slices, 68 MB of partial states)
  EXPECT(osx_attn_fwd_workspace_bytes(OSX_F32, 1, 1, 1, 65408, 65408, 128, 0) > OSX_NOALLOC_SCRATCH_BYTES,
         "scratch-limit case");
  EXPECT(osx_attn_fwd_noalloc(q, k, v, o, nullptr, OSX_F32, 1, 1, 1, 65408, 65408, 128, 0, 0.f, nullptr) ==
             OSX_EWORKSPACE,
         "noalloc scratch limit");
  // unfused comparator
  size_t uw = 0;
  EXPECT(osx_attn_fwd_unfused_workspace(OSX_BF16, 2, 32, 8, 4096, 4096, 128, 1, &uw) == OSX_OK && uw > 0,
         "unfused workspace");
  EXPECT(osx_attn_fwd_unfused_workspace(OSX_BF16, INT_MAX, INT_MAX, 1, INT_MAX, INT_MAX, 128, 0, &uw) != OSX_OK,
         "unfused workspace beyond any size");
}

static int softmax_checks = 0;
static void softmax_plans() {
  const int64_t rows[] = {0, 1, 4, 1000, 1 << 20, (int64_t)1 << 31, INT64_MAX, -1};
  const int64_t cols[] = {0, 1, 200, 2048, 2049, 8192, 8193, 1 << 24, (int64_t)1 << 31, INT64_MAX, -5};
  for (int64_t r : rows)
    for (int64_t c : cols) {
      osx_plan p;
      const int st = osx_softmax_rows_plan(r, c, &p);
      size_t ws = 999;
      const int st2 = osx_softmax_rows_workspace(r, c, &ws);
      const size_t wb = osx_softmax_rows_workspace_bytes(r, c);
      ++softmax_checks;
      EXPECT(st == st2, "softmax plan %d vs workspace %d (rows %lld cols %lld)", st, st2, (long long)r, (long long)c);
      if (st == OSX_OK)
        EXPECT(ws == p.workspace_bytes && wb == ws, "softmax workspace %zu / %zu / %zu", ws, wb, p.workspace_bytes);
      else
        EXPECT(wb == 0 && ws == 0, "rejected softmax shape reports workspace");
      for (int m = 0; m < 4; ++m) {
        size_t b3 = 0;
        (void)osx_softmax_rows_3pass_workspace(r, c, m, &b3);
      }
    }
  float* x = (float*)fake(0x100000000);
  float* y = (float*)fake(0x200000000);
  EXPECT(osx_softmax_rows(nullptr, y, 4, 200, nullptr, 0, nullptr) == OSX_EINVAL, "null x");
  EXPECT(osx_softmax_rows(x, (float*)fake(0x100000004), 4, 200, nullptr, 0, nullptr) == OSX_EINVAL, "partial overlap");
  EXPECT(osx_softmax_rows(x, (float*)fake(0x200000002), 4, 200, nullptr, 0, nullptr) == OSX_EINVAL, "misaligned y");
  EXPECT(osx_softmax_rows(x, y, 1, 1 << 24, nullptr, 0, nullptr) == OSX_EWORKSPACE, "split softmax workspace");
  EXPECT(osx_softmax_rows(nullptr, nullptr, 0, 200, nullptr, 0, nullptr) == OSX_OK, "no rows");
  EXPECT(osx_softmax_rows_ex(x, y, 7, 4, 200, 0, 1.0f, nullptr, 0, nullptr) == OSX_EINVAL, "bad dtype");
  EXPECT(osx_softmax_rows_ex(x, y, OSX_F32, 4, 200, 0, 0.0f / 0.0f, nullptr, 0, nullptr) == OSX_EINVAL, "NaN scale");
  EXPECT(osx_softmax_rows_ex(x, y, OSX_F32, 4, 200, -1, 1.0f, nullptr, 0, nullptr) == OSX_EINVAL, "negative period");
  EXPECT(osx_softmax_rows_3pass(x, y, 4, 200, 9, nullptr, 0, nullptr) != OSX_OK, "bad 3-pass method");
  EXPECT(osx_read_probe(fake(0x100000008), 64, nullptr, 0, nullptr) == OSX_EINVAL, "misaligned probe");
}

// The error detail is per thread: an error raised on another thread leaves
// this thread's message alone.
static void thread_local_errors() {
  osx_plan p;
  EXPECT(osx_attn_plan(OSX_BF16, 1, 6, 4, 8, 8, 128, 0, &p) == OSX_EINVAL, "heads ratio");
  const std::string mine = osx_last_error();
  std::vector<std::thread> ts;
  for (int i = 0; i < 4; ++i)
    ts.emplace_back([i] {
      osx_plan q;
      for (int j = 0; j < 200; ++j) (void)osx_attn_plan(OSX_F32, 1, 1, 1, 8, 8, 50 + i, 0, &q);
    });
  for (auto& t : ts) t.join();
  EXPECT(mine == osx_last_error(), "error detail changed by other threads: '%s' -> '%s'", mine.c_str(),
         osx_last_error());
}

int main() {
  status_strings();
  attn_plans();
  attn_rejects();
  softmax_plans();
  thread_local_errors();
  std::printf("abi_selftest: %d attention shapes, %d softmax shapes, %d failures\n", attn_checks, softmax_checks,
              g_failures);
  return g_failures == 0 ? 0 : 1;
}
