// osx_attn_fwd_noalloc: the attention call for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  Where osx_attn_fwd takes a caller-allocated
// workspace for the partial (m, l, acc) states of split keys, this entry point
// uses a fixed array in the library's own device memory, `scratch`, of
// OSX_NOALLOC_SCRATCH_BYTES.  Each GPU the library runs on holds its own copy
// until the process ends.
//
// The array's name is only a host-side stand-in in host code: its device
// address is looked up once per device with hipGetSymbolAddress (on the
// first call on that device, with that device current) and that address is
// what the kernels receive, exactly as they receive a caller's workspace.
// No kernel needs the scratch cleared: every partial state is written before
// it is read.  All calls on one GPU share its array, so calls that overlap in
// time on one GPU (two streams, two host threads) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"
#include "osx.h"

namespace {

static __device__ __align__(256) unsigned char scratch[OSX_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device (null: not looked up yet)

// Device address of the current device's `scratch`.
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return osx::set_error(OSX_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return osx::set_error(OSX_EUNSUPPORTED, "device %d: the static scratch is tracked for devices 0..%d", dev,
                          kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return osx::set_error(OSX_EHIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                            hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return OSX_OK;
}

}  // namespace

extern "C" int osx_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int dtype,
                                    int batch, int heads_q, int heads_kv, int seq_q, int seq_k, int head_dim,
                                    int causal, float scale, void* stream) {
  osx_plan p;
  int st = osx_attn_plan(dtype, batch, heads_q, heads_kv, seq_q, seq_k, head_dim, causal, &p);
  if (st != OSX_OK) return st;
  if (p.workspace_bytes > OSX_NOALLOC_SCRATCH_BYTES)
    return osx::set_error(OSX_EWORKSPACE,
                          "this problem needs %zu bytes of scratch; the static scratch of osx_attn_fwd_noalloc holds "
                          "%zu (use osx_attn_fwd with a workspace)",
                          p.workspace_bytes, (size_t)OSX_NOALLOC_SCRATCH_BYTES);
  if (p.kernel == OSX_KERNEL_NONE) return osx_attn_fwd(q, k, v, o, dtype, batch, heads_q, heads_kv, seq_q, seq_k,
                                                       head_dim, causal, scale, nullptr, 0, stream);
  // Looked up on every device's first call, whether or not this problem
  // needs scratch, so that later calls (under capture, say) find it set.
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != OSX_OK) return st;
  return osx::attn_fwd_call(q, k, v, o, lse, lse != nullptr, dtype, batch, heads_q, heads_kv, seq_q, seq_k, head_dim,
                            causal, scale, ws, OSX_NOALLOC_SCRATCH_BYTES, stream, false);
}
