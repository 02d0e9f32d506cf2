// A plain streaming read of device memory: the reference the benchmark times
// beside the HBM-bound kernels on the same GPU (what 16-byte loads alone
// reach), not a step of the method.
//
// Workgroup w reads whole chunks of 256 x 8 consecutive 16-byte vectors
// (chunks w, w + grid, ...), each thread eight vectors 4 KiB apart, all
// issued before use, with non-temporal loads; every word read is folded into
// one XOR per wavefront, which lane 0 stores to the sink.  The XOR of all sink
// words is the XOR of all words of the buffer, so a test can check that every
// word was read exactly once.
#include "common.hpp"
#include "launch.hpp"

namespace osx {
namespace {

constexpr int kUnroll = 8;

__device__ __forceinline__ uint32_t fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4* __restrict__ x, size_t n_vec,
                                                                   uint32_t* __restrict__ sink) {
  const size_t chunk = (size_t)kProbeThreads * kUnroll;
  const size_t step = (size_t)gridDim.x * chunk;
  size_t base = (size_t)blockIdx.x * chunk + threadIdx.x;
  uint32_t acc = 0;
  // Whole chunks: this thread's eight vectors all lie below n_vec.
  for (; base + (kUnroll - 1) * kProbeThreads < n_vec; base += step) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(x + base + u * kProbeThreads);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= fold(v[u]);
  }
  // The one chunk that straddles n_vec (every later chunk lies past it).
#pragma unroll
  for (int u = 0; u < kUnroll; ++u)
    if (base + u * kProbeThreads < n_vec) acc ^= fold(__builtin_nontemporal_load(x + base + u * kProbeThreads));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
  if ((threadIdx.x & 63) == 0) sink[(size_t)blockIdx.x * (kProbeThreads / 64) + threadIdx.x / 64] = acc;
}

}  // namespace

hipError_t launch_read_probe(const void* x, size_t bytes, void* sink, hipStream_t stream) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(kProbeWgs), dim3(kProbeThreads), 0, stream,
                     static_cast<const u32x4*>(x), bytes / 16, static_cast<uint32_t*>(sink));
  return hipGetLastError();
}

}  // namespace osx
