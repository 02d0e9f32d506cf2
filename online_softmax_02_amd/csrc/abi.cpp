// C ABI: argument checks, kernel planning and dispatch.  No device memory is
// allocated here and nothing synchronises the device.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "launch.hpp"
#include "osx.h"

namespace {

thread_local char g_err[512] = "";

// OSX_LOG=1 in the environment: one line on stderr per launching call, naming
// the kernel the plan chose (read once per process).
bool log_enabled() {
  static const bool on = [] {
    const char* v = std::getenv("OSX_LOG");
    return v && v[0] && std::strcmp(v, "0") != 0;
  }();
  return on;
}

const char* kernel_name(int k) {
  switch (k) {
    case OSX_KERNEL_NONE: return "none";
    case OSX_KERNEL_PREFILL_F32: return "prefill_f32";
    case OSX_KERNEL_PREFILL_BF16: return "prefill_bf16";
    case OSX_KERNEL_DECODE_BF16: return "decode_bf16";
    case OSX_KERNEL_SOFTMAX_ROW: return "softmax_row";
    case OSX_KERNEL_SOFTMAX_SPLIT: return "softmax_split";
    case OSX_KERNEL_SOFTMAX_WAVE: return "softmax_wave";
    default: return "?";
  }
}

void log_plan(const char* call, const osx_plan& p, const char* shape) {
  if (!log_enabled()) return;
  std::fprintf(stderr, "osx: %s %s -> %s grid=%lld threads=%d block_m=%d splits=%d heads_per_wg=%d workspace=%zu\n",
               call, shape, kernel_name(p.kernel), (long long)p.grid, p.threads, p.block_m, p.splits, p.heads_per_wg,
               p.workspace_bytes);
}

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return OSX_OK;
}

// ceil(a / b) for a >= 0, b > 0, without forming a + b - 1 (which overflows
// for a near INT64_MAX).
int64_t cdiv(int64_t a, int64_t b) { return a / b + (a % b != 0); }

// No tensor on one device comes near this (2^47 bytes = 128 TiB against
// 288 GB of HBM); below it every product the planners form fits in int64.
constexpr double kMaxTensorBytes = 140737488355328.0;

// Largest of 4, 2, 1 that divides the group size: that many query heads of one
// KV head share a workgroup; the remaining wavefronts take further row tiles.
int heads_per_wg(int groups) { return groups % 4 == 0 ? 4 : (groups % 2 == 0 ? 2 : 1); }

int plan_attn(int dtype, int batch, int heads_q, int heads_kv, int seq_q, int seq_k, int head_dim, int causal,
              osx_plan* p) {
  std::memset(p, 0, sizeof *p);
  if (dtype != OSX_F32 && dtype != OSX_BF16) return fail(OSX_EINVAL, "dtype %d is neither OSX_F32 nor OSX_BF16", dtype);
  if (batch < 0 || heads_q < 0 || heads_kv < 0 || seq_q < 0 || seq_k < 0 || head_dim < 0)
    return fail(OSX_EINVAL, "negative size (batch=%d heads_q=%d heads_kv=%d seq_q=%d seq_k=%d head_dim=%d)", batch,
                heads_q, heads_kv, seq_q, seq_k, head_dim);
  if (batch == 0 || heads_q == 0 || seq_q == 0) return ok();  // nothing to compute
  if (heads_kv == 0 || heads_q % heads_kv != 0)
    return fail(OSX_EINVAL, "heads_q (%d) must be a positive multiple of heads_kv (%d)", heads_q, heads_kv);
  if (seq_k == 0) return fail(OSX_EINVAL, "seq_k == 0 with seq_q > 0: softmax over no keys");
  if (head_dim == 0) return fail(OSX_EINVAL, "head_dim == 0");
  if (dtype == OSX_F32 && (head_dim % 4 != 0 || head_dim > 128))
    return fail(OSX_EUNSUPPORTED, "fp32 head_dim %d: must be a multiple of 4 and at most 128", head_dim);
  if (dtype == OSX_BF16 && (head_dim % 16 != 0 || head_dim > 128))
    return fail(OSX_EUNSUPPORTED, "bf16 head_dim %d: must be a multiple of 16 and at most 128", head_dim);
  // The kernels address one head's Q, K, V or O through 32-bit buffer ranges and
  // 32-bit element offsets: each must stay below 2^31 bytes.
  {
    const int64_t es = dtype == OSX_BF16 ? 2 : 4;
    const double q_bytes = (double)batch * heads_q * seq_q * head_dim * es;
    const double kv_bytes = (double)batch * heads_kv * seq_k * head_dim * es;
    if (q_bytes > kMaxTensorBytes || kv_bytes > kMaxTensorBytes)
      return fail(OSX_EUNSUPPORTED, "q/o of %.3g bytes or k/v of %.3g bytes: beyond any device", q_bytes, kv_bytes);
    const int64_t longest = (int64_t)(seq_q > seq_k ? seq_q : seq_k) * head_dim * es;
    if (longest >= (1LL << 31))
      return fail(OSX_EUNSUPPORTED, "one head of %lld positions x %d dims is %lld bytes: at most 2^31 - 1",
                  (long long)(seq_q > seq_k ? seq_q : seq_k), head_dim, (long long)longest);
  }
  if (causal && seq_q > 1 && seq_q != seq_k)
    return fail(OSX_EUNSUPPORTED, "causal with seq_q (%d) != seq_k (%d): mask alignment is not defined", seq_q,
                seq_k);
  const int groups = heads_q / heads_kv;
  if (dtype == OSX_BF16 && seq_q == 1 && groups <= osx::kDecodeMaxGroup) {
    const int64_t units = (int64_t)batch * heads_kv;
    int64_t splits = cdiv(osx::kDecodeTargetWgs, units);
    const int64_t max_splits = cdiv(seq_k, osx::kDecodeBlockN * osx::kAttnWaves);
    if (splits > max_splits) splits = max_splits;
    if (splits < 1) splits = 1;
    p->kernel = OSX_KERNEL_DECODE_BF16;
    p->threads = osx::kAttnThreads;
    p->block_m = groups;
    p->block_n = osx::kDecodeBlockN;
    p->splits = (int)splits;
    p->heads_per_wg = groups;
    p->grid = units * splits;
    // One split writes O directly; more write partial states for the combine kernel.
    p->workspace_bytes = splits == 1 ? 0 : (size_t)(units * splits * groups) * (size_t)(2 + head_dim) * sizeof(float);
    return ok();
  }
  const int hp = heads_per_wg(groups);
  // bf16: two groups of 4 wavefronts, the second on the rows after the first's.
  const int rows_per_wg = dtype == OSX_BF16 ? osx::kRowsPerWave * (osx::kPrefillWaves / hp)
                                            : osx::kRowsPerWave * (osx::kAttnWaves / hp);
  p->kernel = dtype == OSX_BF16 ? OSX_KERNEL_PREFILL_BF16 : OSX_KERNEL_PREFILL_F32;
  p->threads = dtype == OSX_BF16 ? osx::kPrefillThreads : osx::kAttnThreads;
  p->block_m = rows_per_wg;
  p->block_n = dtype == OSX_BF16 ? osx::kBf16BlockN : osx::kF32BlockN;
  p->splits = 1;
  p->heads_per_wg = hp;
  p->grid = (int64_t)batch * heads_kv * (groups / hp) * cdiv(seq_q, rows_per_wg);
  p->workspace_bytes = 0;
  if (dtype == OSX_F32 && p->grid < osx::kSplitTargetWgs) {
    // Too few row tiles to fill the GPU: split the keys (each slice at least
    // kSplitMinBlocks blocks) and merge the slices' partial states afterwards.
    int64_t splits = cdiv(osx::kSplitTargetWgs, p->grid);
    int64_t max_splits = seq_k / (osx::kF32BlockN * osx::kSplitMinBlocks);
    if (max_splits > osx::kWaveSize) max_splits = osx::kWaveSize;  // the combine gives each slice one lane
    if (splits > max_splits) splits = max_splits;
    if (splits > 1) {
      p->splits = (int)splits;
      p->grid *= splits;
      // (m, l) pairs, then the accumulators from the next 16-byte boundary.
      const int64_t parts = (int64_t)batch * heads_q * seq_q * splits;
      p->workspace_bytes = (size_t)((parts * 2 + 3) / 4 * 4 + parts * head_dim) * sizeof(float);
    }
  }
  if (p->grid > 0x7fffffff) return fail(OSX_EUNSUPPORTED, "problem needs %lld workgroups", (long long)p->grid);
  return ok();
}

int plan_softmax(int64_t rows, int64_t cols, osx_plan* p) {
  std::memset(p, 0, sizeof *p);
  if (rows < 0 || cols < 0) return fail(OSX_EINVAL, "negative size (rows=%lld cols=%lld)", (long long)rows,
                                        (long long)cols);
  if (rows == 0) return ok();
  if (cols == 0) return fail(OSX_EINVAL, "cols == 0 with rows > 0: softmax over nothing");
  if ((double)rows * (double)cols * 4.0 > kMaxTensorBytes)
    return fail(OSX_EUNSUPPORTED, "%lld x %lld elements: beyond any device", (long long)rows, (long long)cols);
  p->threads = osx::kSoftmaxThreads;
  if (cols <= osx::kSoftmaxWaveMax) {
    p->kernel = OSX_KERNEL_SOFTMAX_WAVE;
    p->block_m = (int)cols;
    p->splits = 1;
    p->grid = cdiv(rows, osx::kSoftmaxThreads / osx::kWaveSize);
    p->workspace_bytes = 0;
  } else if (cols <= osx::kSoftmaxRowMax) {
    p->kernel = OSX_KERNEL_SOFTMAX_ROW;
    p->block_m = (int)cols;
    p->splits = 1;
    p->grid = rows;
    p->workspace_bytes = 0;
  } else {
    const int64_t splits = cdiv(cols, osx::kSoftmaxChunk);
    p->kernel = OSX_KERNEL_SOFTMAX_SPLIT;
    p->block_m = (int)osx::kSoftmaxChunk;
    p->splits = (int)splits;
    p->grid = rows * splits;
    p->workspace_bytes = (size_t)(rows * splits) * 2 * sizeof(float);
  }
  if (p->grid > 0x7fffffff) return fail(OSX_EUNSUPPORTED, "problem needs %lld workgroups", (long long)p->grid);
  return ok();
}

// True when p is not a multiple of `align` bytes.
bool misaligned(const void* p, uintptr_t align) { return (reinterpret_cast<uintptr_t>(p) & (align - 1)) != 0; }

// The attention scale: scale <= 0 selects 1/sqrt(head_dim); NaN, +inf, or a
// scale so large that scale * log2(e) (the factor the kernels apply) is not a
// finite fp32 value, is rejected.
int attn_scale(float scale, int head_dim, float* out) {
  if (std::isnan(scale) || (scale > 0.0f && !std::isfinite((float)((double)scale * 1.4426950408889634))))
    return fail(OSX_EINVAL, "scale %g: must be finite with scale * log2(e) finite in fp32 (<= 0 selects 1/sqrt(d))",
                (double)scale);
  *out = scale > 0.0f ? scale : 1.0f / std::sqrt((float)head_dim);
  return OSX_OK;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const char* pa = (const char*)a;
  const char* pb = (const char*)b;
  return pa < pb + nb && pb < pa + na;
}

}  // namespace

namespace osx {

hipError_t device_cu_count(int* n_cu) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];  // 0 = not looked up yet
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDevices) {
    const int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) {
      *n_cu = n;
      return hipSuccess;
    }
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (n <= 0) return hipErrorInvalidDevice;
  if (dev >= 0 && dev < kMaxDevices) cache[dev].store(n, std::memory_order_relaxed);
  *n_cu = n;
  return hipSuccess;
}

}  // namespace osx

extern "C" {

int osx_attn_plan(int dtype, int batch, int heads_q, int heads_kv, int seq_q, int seq_k, int head_dim, int causal,
                  osx_plan* out) {
  osx_plan p;
  int st = plan_attn(dtype, batch, heads_q, heads_kv, seq_q, seq_k, head_dim, causal, &p);
  if (out) *out = p;
  return st;
}

int osx_attn_fwd_workspace(int dtype, int batch, int heads_q, int heads_kv, int seq_q, int seq_k, int head_dim,
                           int causal, size_t* bytes) {
  osx_plan p;
  int st = plan_attn(dtype, batch, heads_q, heads_kv, seq_q, seq_k, head_dim, causal, &p);
  if (bytes) *bytes = st == OSX_OK ? p.workspace_bytes : 0;
  return st;
}

size_t osx_attn_fwd_workspace_bytes(int dtype, int batch, int heads_q, int heads_kv, int seq_q, int seq_k,
                                    int head_dim, int causal) {
  osx_plan p;
  return plan_attn(dtype, batch, heads_q, heads_kv, seq_q, seq_k, head_dim, causal, &p) == OSX_OK ? p.workspace_bytes
                                                                                                : 0;
}

}  // extern "C"

namespace {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, bool want_lse, int dtype, int batch,
             int heads_q, int heads_kv, int seq_q, int seq_k, int head_dim, int causal, float scale, void* workspace,
             size_t workspace_bytes, void* stream, bool normalised = false) {
  osx_plan p;
  int st = plan_attn(dtype, batch, heads_q, heads_kv, seq_q, seq_k, head_dim, causal, &p);
  if (st != OSX_OK) return st;
  if (normalised && dtype != OSX_F32)
    return fail(OSX_EUNSUPPORTED, "the normalised-output recurrence is built for fp32 q, k, v and o only");
  if (p.kernel == OSX_KERNEL_NONE) return ok();
  if (!q || !k || !v || !o) return fail(OSX_EINVAL, "null q, k, v or o pointer");
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16))
    return fail(OSX_EINVAL, "q, k, v and o must be 16-byte aligned (the kernels read and write 16-byte vectors)");
  if (want_lse && !lse) return fail(OSX_EINVAL, "null lse pointer");
  if (lse && misaligned(lse, 4)) return fail(OSX_EINVAL, "lse must be 4-byte aligned");
  if (p.workspace_bytes > 0 && (!workspace || workspace_bytes < p.workspace_bytes))
    return fail(OSX_EWORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : (size_t)0,
                p.workspace_bytes);
  if (p.workspace_bytes > 0 && misaligned(workspace, 16)) return fail(OSX_EINVAL, "workspace must be 16-byte aligned");
  if ((st = attn_scale(scale, head_dim, &scale)) != OSX_OK) return st;
  if (log_enabled()) {
    char shape[160];
    std::snprintf(shape, sizeof shape, "%s B=%d Hq=%d Hkv=%d Sq=%d Sk=%d d=%d causal=%d%s%s",
                  dtype == OSX_BF16 ? "bf16" : "f32", batch, heads_q, heads_kv, seq_q, seq_k, head_dim, causal ? 1 : 0,
                  want_lse || lse ? " lse" : "", normalised ? " normalised" : "");
    log_plan("attn_fwd", p, shape);
  }
  const size_t es = dtype == OSX_BF16 ? 2 : 4;
  const size_t nq = (size_t)batch * heads_q * seq_q * head_dim * es;
  const size_t nkv = (size_t)batch * heads_kv * seq_k * head_dim * es;
  if (overlap(o, nq, q, nq) || overlap(o, nq, k, nkv) || overlap(o, nq, v, nkv) ||
      (p.workspace_bytes && overlap(o, nq, workspace, p.workspace_bytes)))
    return fail(OSX_EINVAL, "output overlaps an input or the workspace");
  if (p.workspace_bytes && (overlap(workspace, p.workspace_bytes, q, nq) || overlap(workspace, p.workspace_bytes, k, nkv) ||
                            overlap(workspace, p.workspace_bytes, v, nkv)))
    return fail(OSX_EINVAL, "workspace overlaps q, k or v");
  if (lse) {
    const size_t nl = (size_t)batch * heads_q * seq_q * sizeof(float);
    if (overlap(lse, nl, q, nq) || overlap(lse, nl, k, nkv) || overlap(lse, nl, v, nkv) || overlap(lse, nl, o, nq) ||
        (p.workspace_bytes && overlap(lse, nl, workspace, p.workspace_bytes)))
      return fail(OSX_EINVAL, "lse overlaps an input, the output or the workspace");
  }
  osx::AttnArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.batch = batch;
  a.heads_q = heads_q;
  a.heads_kv = heads_kv;
  a.seq_q = seq_q;
  a.seq_k = seq_k;
  a.head_dim = head_dim;
  a.causal = causal ? 1 : 0;
  a.c = (float)((double)scale * 1.4426950408889634);
  a.workspace = workspace;
  a.lse = lse;
  a.stream = (hipStream_t)stream;
  a.plan = p;
  a.normalised = normalised ? 1 : 0;
  hipError_t e;
  switch (p.kernel) {
    case OSX_KERNEL_PREFILL_BF16: e = osx::launch_prefill_bf16(a); break;
    case OSX_KERNEL_PREFILL_F32: e = osx::launch_prefill_f32(a); break;
    case OSX_KERNEL_DECODE_BF16: e = osx::launch_decode_bf16(a); break;
    default: return fail(OSX_EUNSUPPORTED, "no kernel for plan %d", p.kernel);
  }
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return fail(OSX_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

namespace osx {

int attn_fwd_call(const void* q, const void* k, const void* v, void* o, float* lse, bool want_lse, int dtype,
                  int batch, int heads_q, int heads_kv, int seq_q, int seq_k, int head_dim, int causal, float scale,
                  void* workspace, size_t workspace_bytes, void* stream, bool normalised) {
  return attn_fwd(q, k, v, o, lse, want_lse, dtype, batch, heads_q, heads_kv, seq_q, seq_k, head_dim, causal, scale,
                  workspace, workspace_bytes, stream, normalised);
}

int set_error(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

}  // namespace osx

extern "C" {

int osx_attn_fwd(const void* q, const void* k, const void* v, void* o, int dtype, int batch, int heads_q,
                 int heads_kv, int seq_q, int seq_k, int head_dim, int causal, float scale, void* workspace,
                 size_t workspace_bytes, void* stream) {
  return attn_fwd(q, k, v, o, nullptr, false, dtype, batch, heads_q, heads_kv, seq_q, seq_k, head_dim, causal, scale,
                  workspace, workspace_bytes, stream);
}

int osx_attn_fwd_lse(const void* q, const void* k, const void* v, void* o, float* lse, int dtype, int batch,
                     int heads_q, int heads_kv, int seq_q, int seq_k, int head_dim, int causal, float scale,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return attn_fwd(q, k, v, o, lse, true, dtype, batch, heads_q, heads_kv, seq_q, seq_k, head_dim, causal, scale,
                  workspace, workspace_bytes, stream);
}

int osx_attn_fwd_normalised(const void* q, const void* k, const void* v, void* o, float* lse, int dtype, int batch,
                            int heads_q, int heads_kv, int seq_q, int seq_k, int head_dim, int causal, float scale,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return attn_fwd(q, k, v, o, lse, false, dtype, batch, heads_q, heads_kv, seq_q, seq_k, head_dim, causal, scale,
                  workspace, workspace_bytes, stream, true);
}

int osx_softmax_rows_plan(int64_t rows, int64_t cols, osx_plan* out) {
  osx_plan p;
  int st = plan_softmax(rows, cols, &p);
  if (out) *out = p;
  return st;
}

int osx_softmax_rows_workspace(int64_t rows, int64_t cols, size_t* bytes) {
  osx_plan p;
  int st = plan_softmax(rows, cols, &p);
  if (bytes) *bytes = st == OSX_OK ? p.workspace_bytes : 0;
  return st;
}

size_t osx_softmax_rows_workspace_bytes(int64_t rows, int64_t cols) {
  osx_plan p;
  return plan_softmax(rows, cols, &p) == OSX_OK ? p.workspace_bytes : 0;
}

}  // extern "C"

namespace {

int softmax_rows(const void* x, void* y, int dtype, int64_t rows, int64_t cols, int64_t causal_period, float scale,
                 void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != OSX_F32 && dtype != OSX_BF16) return fail(OSX_EINVAL, "dtype %d: OSX_F32 or OSX_BF16", dtype);
  if (causal_period < 0) return fail(OSX_EINVAL, "negative causal_period %lld", (long long)causal_period);
  if (!(scale > 0.0f) || !std::isfinite(scale)) return fail(OSX_EINVAL, "scale must be positive and finite");
  osx_plan p;
  int st = plan_softmax(rows, cols, &p);
  if (st != OSX_OK) return st;
  if (p.kernel == OSX_KERNEL_NONE) return ok();
  if (!x || !y) return fail(OSX_EINVAL, "null x or y pointer");
  const uintptr_t es = dtype == OSX_BF16 ? 2 : 4;
  if (misaligned(x, es) || misaligned(y, es)) return fail(OSX_EINVAL, "x and y must be aligned to their element size");
  const size_t n = (size_t)rows * (size_t)cols * es;
  if (x != y && overlap(x, n, y, n)) return fail(OSX_EINVAL, "x and y overlap without being the same buffer");
  if (p.workspace_bytes > 0 && (!workspace || workspace_bytes < p.workspace_bytes))
    return fail(OSX_EWORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : (size_t)0,
                p.workspace_bytes);
  if (p.workspace_bytes > 0 && (overlap(workspace, p.workspace_bytes, x, n) || overlap(workspace, p.workspace_bytes, y, n)))
    return fail(OSX_EINVAL, "workspace overlaps x or y");
  if (p.workspace_bytes > 0 && misaligned(workspace, 4)) return fail(OSX_EINVAL, "workspace must be 4-byte aligned");
  if (log_enabled()) {
    char shape[128];
    std::snprintf(shape, sizeof shape, "%s rows=%lld cols=%lld causal_period=%lld%s",
                  dtype == OSX_BF16 ? "bf16" : "f32", (long long)rows, (long long)cols, (long long)causal_period,
                  x == y ? " in-place" : "");
    log_plan("softmax_rows", p, shape);
  }
  osx::SoftmaxArgs a;
  a.x = x;
  a.y = y;
  a.dtype = dtype;
  a.rows = rows;
  a.cols = cols;
  a.k = (float)((double)scale * 1.4426950408889634);
  a.period = causal_period;
  a.workspace = workspace;
  a.stream = (hipStream_t)stream;
  a.plan = p;
  hipError_t e = osx::launch_softmax_rows(a);
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return fail(OSX_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

// Chunks and workspace of the three-pass comparators.
int plan_3pass(int64_t rows, int64_t cols, int method, int* splits, int64_t* grid, size_t* ws) {
  if (method != OSX_3PASS_ATOMIC && method != OSX_3PASS_STASH)
    return fail(OSX_EINVAL, "method %d: OSX_3PASS_ATOMIC or OSX_3PASS_STASH", method);
  if (rows < 0 || cols < 0) return fail(OSX_EINVAL, "negative size (rows=%lld cols=%lld)", (long long)rows,
                                        (long long)cols);
  *splits = 0;
  *grid = 0;
  *ws = 0;
  if (rows == 0) return ok();
  if (cols == 0) return fail(OSX_EINVAL, "cols == 0 with rows > 0: softmax over nothing");
  if ((double)rows * (double)cols * 4.0 > kMaxTensorBytes)
    return fail(OSX_EUNSUPPORTED, "%lld x %lld elements: beyond any device", (long long)rows, (long long)cols);
  const int64_t sp = cdiv(cols, osx::softmax_3pass_chunk(method));
  if (rows * sp > 0x7fffffff) return fail(OSX_EUNSUPPORTED, "problem needs %lld workgroups", (long long)(rows * sp));
  *splits = (int)sp;
  *grid = rows * sp;
  *ws = (size_t)(method == OSX_3PASS_ATOMIC ? rows : rows * sp) * 2 * sizeof(float);
  return ok();
}

// Unfused attention: the [B*Hq, Sq, Sk] fp32 score matrix, then the row
// softmax's own workspace (rows longer than one workgroup holds).
int plan_unfused(int dtype, int batch, int heads_q, int heads_kv, int seq_q, int seq_k, int head_dim, int causal,
                 size_t* s_bytes, size_t* total) {
  *s_bytes = 0;
  *total = 0;
  osx_plan p;
  int st = plan_attn(dtype, batch, heads_q, heads_kv, seq_q, seq_k, head_dim, causal, &p);
  if (st != OSX_OK) return st;
  if (p.kernel == OSX_KERNEL_NONE) return ok();
  if (dtype != OSX_BF16) return fail(OSX_EUNSUPPORTED, "unfused attention takes bf16 q, k, v, o");
  if (head_dim != 64 && head_dim != 128)
    return fail(OSX_EUNSUPPORTED, "unfused attention: head_dim %d, must be 64 or 128", head_dim);
  if ((int64_t)batch * heads_q > 65535)
    return fail(OSX_EUNSUPPORTED, "unfused attention: batch * heads_q = %lld exceeds 65535",
                (long long)batch * heads_q);
  if ((int64_t)seq_q * seq_k > (1LL << 29))
    return fail(OSX_EUNSUPPORTED, "unfused attention: seq_q * seq_k = %lld exceeds 2^29 scores per head",
                (long long)seq_q * seq_k);
  const int64_t rows = (int64_t)batch * heads_q * seq_q;
  osx_plan sp;
  st = plan_softmax(rows, seq_k, &sp);
  if (st != OSX_OK) return st;
  *s_bytes = (size_t)rows * (size_t)seq_k * sizeof(float);
  *total = *s_bytes + sp.workspace_bytes;
  return ok();
}

}  // namespace

extern "C" {

int osx_softmax_rows(const float* x, float* y, int64_t rows, int64_t cols, void* workspace, size_t workspace_bytes,
                     void* stream) {
  return softmax_rows(x, y, OSX_F32, rows, cols, 0, 1.0f, workspace, workspace_bytes, stream);
}

int osx_softmax_rows_ex(const void* x, void* y, int dtype, int64_t rows, int64_t cols, int64_t causal_period,
                        float scale, void* workspace, size_t workspace_bytes, void* stream) {
  return softmax_rows(x, y, dtype, rows, cols, causal_period, scale, workspace, workspace_bytes, stream);
}

int osx_attn_fwd_unfused_workspace(int dtype, int batch, int heads_q, int heads_kv, int seq_q, int seq_k,
                                   int head_dim, int causal, size_t* bytes) {
  size_t s_bytes, total;
  const int st = plan_unfused(dtype, batch, heads_q, heads_kv, seq_q, seq_k, head_dim, causal, &s_bytes, &total);
  if (bytes) *bytes = st == OSX_OK ? total : 0;
  return st;
}

int osx_attn_fwd_unfused(const void* q, const void* k, const void* v, void* o, int dtype, int batch, int heads_q,
                         int heads_kv, int seq_q, int seq_k, int head_dim, int causal, float scale, void* workspace,
                         size_t workspace_bytes, void* stream) {
  size_t s_bytes, need;
  int st = plan_unfused(dtype, batch, heads_q, heads_kv, seq_q, seq_k, head_dim, causal, &s_bytes, &need);
  if (st != OSX_OK) return st;
  if (need == 0) return ok();
  if (!q || !k || !v || !o) return fail(OSX_EINVAL, "null q, k, v or o pointer");
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16))
    return fail(OSX_EINVAL, "q, k, v and o must be 16-byte aligned (the kernels read and write 16-byte vectors)");
  if (workspace && misaligned(workspace, 16)) return fail(OSX_EINVAL, "workspace must be 16-byte aligned");
  if (!workspace || workspace_bytes < need)
    return fail(OSX_EWORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : (size_t)0,
                need);
  if ((st = attn_scale(scale, head_dim, &scale)) != OSX_OK) return st;
  const size_t nq = (size_t)batch * heads_q * seq_q * head_dim * 2;
  const size_t nkv = (size_t)batch * heads_kv * seq_k * head_dim * 2;
  if (overlap(o, nq, q, nq) || overlap(o, nq, k, nkv) || overlap(o, nq, v, nkv) || overlap(o, nq, workspace, need))
    return fail(OSX_EINVAL, "output overlaps an input or the workspace");
  if (overlap(workspace, need, q, nq) || overlap(workspace, need, k, nkv) || overlap(workspace, need, v, nkv))
    return fail(OSX_EINVAL, "workspace overlaps an input");
  osx::AttnArgs a = {};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.batch = batch;
  a.heads_q = heads_q;
  a.heads_kv = heads_kv;
  a.seq_q = seq_q;
  a.seq_k = seq_k;
  a.head_dim = head_dim;
  a.causal = causal ? 1 : 0;
  a.stream = (hipStream_t)stream;
  float* S = static_cast<float*>(workspace);
  hipError_t e = osx::launch_unfused_scores(a, S, scale);
  if (e != hipSuccess) return fail(OSX_EHIP, "score kernel launch failed: %s", hipGetErrorString(e));
  // Row r of S is query r mod seq_q of its head; causal keeps keys <= that query.
  st = softmax_rows(S, S, OSX_F32, (int64_t)batch * heads_q * seq_q, seq_k, causal && seq_q > 1 ? seq_q : 0, 1.0f,
                    static_cast<char*>(workspace) + s_bytes, need - s_bytes, stream);
  if (st != OSX_OK) return st;
  e = osx::launch_unfused_pv(a, S);
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return fail(OSX_EHIP, "P V kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

int osx_softmax_rows_3pass_workspace(int64_t rows, int64_t cols, int method, size_t* bytes) {
  int splits;
  int64_t grid;
  size_t ws = 0;
  const int st = plan_3pass(rows, cols, method, &splits, &grid, &ws);
  if (bytes) *bytes = st == OSX_OK ? ws : 0;
  return st;
}

int osx_softmax_rows_3pass(const float* x, float* y, int64_t rows, int64_t cols, int method, void* workspace,
                           size_t workspace_bytes, void* stream) {
  int splits;
  int64_t grid;
  size_t need;
  int st = plan_3pass(rows, cols, method, &splits, &grid, &need);
  if (st != OSX_OK) return st;
  if (grid == 0) return ok();
  if (!x || !y) return fail(OSX_EINVAL, "null x or y pointer");
  if (misaligned(x, 4) || misaligned(y, 4)) return fail(OSX_EINVAL, "x and y must be 4-byte aligned");
  const size_t n = (size_t)rows * (size_t)cols * sizeof(float);
  if (x != y && overlap(x, n, y, n)) return fail(OSX_EINVAL, "x and y overlap without being the same buffer");
  if (workspace && misaligned(workspace, 4)) return fail(OSX_EINVAL, "workspace must be 4-byte aligned");
  if (!workspace || workspace_bytes < need)
    return fail(OSX_EWORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : (size_t)0,
                need);
  if (overlap(workspace, need, x, n) || overlap(workspace, need, y, n))
    return fail(OSX_EINVAL, "workspace overlaps x or y");
  osx::Softmax3PassArgs a;
  a.x = x;
  a.y = y;
  a.rows = rows;
  a.cols = cols;
  a.method = method;
  a.splits = splits;
  a.chunk = osx::softmax_3pass_chunk(method);
  a.grid = grid;
  a.workspace = workspace;
  a.stream = (hipStream_t)stream;
  hipError_t e = osx::launch_softmax_3pass(a);
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return fail(OSX_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t osx_read_probe_sink_bytes(void) { return osx::kProbeSinkBytes; }

int osx_read_probe(const void* x, size_t bytes, void* sink, size_t sink_bytes, void* stream) {
  if (bytes == 0) return ok();
  if (!x || !sink) return fail(OSX_EINVAL, "null x or sink pointer");
  if ((reinterpret_cast<uintptr_t>(x) & 15) || (bytes & 15))
    return fail(OSX_EINVAL, "x must be 16-byte aligned and bytes a multiple of 16 (got %zu)", bytes);
  if (sink_bytes < osx::kProbeSinkBytes)
    return fail(OSX_EWORKSPACE, "sink of %zu bytes given, %zu needed", sink_bytes, osx::kProbeSinkBytes);
  if (overlap(x, bytes, sink, osx::kProbeSinkBytes)) return fail(OSX_EINVAL, "sink overlaps x");
  hipError_t e = osx::launch_read_probe(x, bytes, sink, (hipStream_t)stream);
  if (e != hipSuccess) return fail(OSX_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

const char* osx_status_string(int status) {
  switch (status) {
    case OSX_OK: return "OSX_OK";
    case OSX_EINVAL: return "OSX_EINVAL: invalid argument";
    case OSX_EUNSUPPORTED: return "OSX_EUNSUPPORTED: valid but not implemented";
    case OSX_EHIP: return "OSX_EHIP: HIP runtime error";
    case OSX_EWORKSPACE: return "OSX_EWORKSPACE: workspace missing or too small";
    default: return "unknown status";
  }
}

const char* osx_last_error(void) { return g_err; }

int osx_version(void) { return 100; }

}  // extern "C"
