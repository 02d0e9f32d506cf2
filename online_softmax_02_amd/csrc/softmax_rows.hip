// Two-pass row softmax for gfx950.
//
// Pass 1 keeps an online state per thread -- the running max m and the sum l
// of exp(x - m) -- rescaling l by exp(m_old - m_new) whenever the max grows,
// then merges the per-thread states across the wavefront and the workgroup
// (page "Softmax 算子的实现与优化", section Online Softmax: the boxed update
// and the invariant l = sum_j e^{x_j - m}).  Pass 2 reads x again and writes
// y = exp(x - m) / l.  Out-of-range positions contribute nothing (-inf to the
// max, 0 to the sum).
//
// Two shapes of launch:
//  * rows up to kSoftmaxRowMax elements: one workgroup per row does both
//    passes (the pages keep (m, l) inside one program for consistency);
//  * longer rows: the row is cut into kSoftmaxChunk-element chunks, one
//    workgroup each.  Pass 1 writes one (m, l) partial per chunk; pass 2 merges
//    a row's partials with the same rescaling rule, then normalises its chunk.
//    This replaces the single-program scan, which cannot use more than one CU.
//
// Exponentials are 2^((x - m) * log2 e) on the transcendental unit.
#include "common.hpp"
#include "launch.hpp"

namespace osx {
namespace {

constexpr int kThreads = kSoftmaxThreads;
constexpr int kWaves = kThreads / kWaveSize;

// Natural-units online state: l = sum exp(x - m) over the elements seen.
struct State {
  float m, l;
};

__device__ __forceinline__ void merge_state(State& s, float mb, float lb) {
  const float mn = fmaxf(s.m, mb);
  if (mn == kNegInf) return;  // both empty
  s.l = s.l * exp2_fast((s.m - mn) * kLog2e) + lb * exp2_fast((mb - mn) * kLog2e);
  s.m = mn;
}

// Fold a group of values into the state: one max over the group, one rescale.
template <int N>
__device__ __forceinline__ void update(State& s, const float (&v)[N]) {
  float mb = v[0];
#pragma unroll
  for (int i = 1; i < N; ++i) mb = fmaxf(mb, v[i]);
  const float mn = fmaxf(s.m, mb);
  if (mn == kNegInf) return;
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) sum += exp2_fast((v[i] - mn) * kLog2e);
  s.l = s.l * exp2_fast((s.m - mn) * kLog2e) + sum;
  s.m = mn;
}

// Merge the states of all threads of the workgroup; every thread gets the result.
__device__ __forceinline__ State block_merge(State s, float* sm /* 2*kWaves floats */) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float mb = __shfl_xor(s.m, o, 64);
    const float lb = __shfl_xor(s.l, o, 64);
    merge_state(s, mb, lb);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    sm[2 * wave] = s.m;
    sm[2 * wave + 1] = s.l;
  }
  __syncthreads();
  State r = {sm[0], sm[1]};
#pragma unroll
  for (int w = 1; w < kWaves; ++w) merge_state(r, sm[2 * w], sm[2 * w + 1]);
  return r;
}

__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void st4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }

// Online pass over x[begin, end) of one row; VEC = 4 uses 16-byte loads
// (begin, end multiples of 4, x 16-byte aligned).
template <int VEC>
__device__ __forceinline__ State scan(const float* __restrict__ x, int64_t begin, int64_t end) {
  State s = {kNegInf, 0.f};
  const int tid = threadIdx.x;
  if (VEC == 4) {
    const int64_t n4 = (end - begin) >> 2;
    const float* xb = x + begin;
    int64_t i = tid;
    for (; i + 3 * kThreads < n4; i += 4 * kThreads) {
      f32x4 a = ld4(xb + 4 * i), b = ld4(xb + 4 * (i + kThreads)), c = ld4(xb + 4 * (i + 2 * kThreads)),
            d = ld4(xb + 4 * (i + 3 * kThreads));
      const float v[16] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w, c.x, c.y, c.z, c.w, d.x, d.y, d.z, d.w};
      update(s, v);
    }
    for (; i < n4; i += kThreads) {
      f32x4 a = ld4(xb + 4 * i);
      const float v[4] = {a.x, a.y, a.z, a.w};
      update(s, v);
    }
  } else {
    for (int64_t i = begin + tid; i < end; i += kThreads) {
      const float v[1] = {x[i]};
      update(s, v);
    }
  }
  return s;
}

// Normalise pass over [begin, end): y = 2^((x - m) log2 e) / l.
template <int VEC>
__device__ __forceinline__ void normalise(const float* __restrict__ x, float* __restrict__ y, int64_t begin,
                                          int64_t end, float m, float inv_l) {
  const int tid = threadIdx.x;
  if (VEC == 4) {
    const int64_t n4 = (end - begin) >> 2;
    const float* xb = x + begin;
    float* yb = y + begin;
    for (int64_t i = tid; i < n4; i += kThreads) {
      f32x4 a = ld4(xb + 4 * i);
      f32x4 r;
      r.x = exp2_fast((a.x - m) * kLog2e) * inv_l;
      r.y = exp2_fast((a.y - m) * kLog2e) * inv_l;
      r.z = exp2_fast((a.z - m) * kLog2e) * inv_l;
      r.w = exp2_fast((a.w - m) * kLog2e) * inv_l;
      st4(yb + 4 * i, r);
    }
  } else {
    for (int64_t i = begin + tid; i < end; i += kThreads) y[i] = exp2_fast((x[i] - m) * kLog2e) * inv_l;
  }
}

// A full chunk of kSoftmaxChunk elements, 16-byte loads: every thread issues
// all of its kChunkVec loads before using any, so a workgroup keeps its whole
// chunk in flight.  Thread state: its exact max, then the sum of
// 2^((x - m) log2 e) over its values (the block-level merge is the rescaling
// rule).  Pass 1 loads normally so x stays cached for pass 2; pass 2 is the
// last use of x and streams y out with non-temporal accesses.
constexpr int kChunkVec = (int)(kSoftmaxChunk / 4 / kThreads);  // float4 per thread per chunk

__device__ __forceinline__ State scan_chunk(const float* __restrict__ xb) {
  f32x4 v[kChunkVec];
#pragma unroll
  for (int i = 0; i < kChunkVec; ++i) v[i] = reinterpret_cast<const f32x4*>(xb)[threadIdx.x + i * kThreads];
  float m = v[0].x;
#pragma unroll
  for (int i = 0; i < kChunkVec; ++i) m = fmaxf(fmaxf(m, fmaxf(v[i].x, v[i].y)), fmaxf(v[i].z, v[i].w));
  float l = 0.f;
#pragma unroll
  for (int i = 0; i < kChunkVec; ++i)
    l += (exp2_fast((v[i].x - m) * kLog2e) + exp2_fast((v[i].y - m) * kLog2e)) +
         (exp2_fast((v[i].z - m) * kLog2e) + exp2_fast((v[i].w - m) * kLog2e));
  return State{m, l};
}

__device__ __forceinline__ void normalise_chunk(const float* xb, float* yb, float m, float inv_l) {
  f32x4 v[kChunkVec];
#pragma unroll
  for (int i = 0; i < kChunkVec; ++i) v[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(xb) + threadIdx.x + i * kThreads);
#pragma unroll
  for (int i = 0; i < kChunkVec; ++i) {
    f32x4 r;
    r.x = exp2_fast((v[i].x - m) * kLog2e) * inv_l;
    r.y = exp2_fast((v[i].y - m) * kLog2e) * inv_l;
    r.z = exp2_fast((v[i].z - m) * kLog2e) * inv_l;
    r.w = exp2_fast((v[i].w - m) * kLog2e) * inv_l;
    __builtin_nontemporal_store(r, reinterpret_cast<f32x4*>(yb) + threadIdx.x + i * kThreads);
  }
}

// One workgroup per row: both passes.  x and y may be the same buffer.
template <int VEC>
__global__ __launch_bounds__(kThreads) void softmax_row_kernel(const float* x, float* y, int64_t cols) {
  __shared__ float sm[2 * kWaves];
  const int64_t row = blockIdx.x;
  const float* xr = x + row * cols;
  float* yr = y + row * cols;
  State s = scan<VEC>(xr, 0, cols);
  s = block_merge(s, sm);
  normalise<VEC>(xr, yr, 0, cols, s.m, 1.0f / s.l);
}

// Split rows, pass 1: the (m, l) partial of one chunk.
template <int VEC>
__global__ __launch_bounds__(kThreads) void softmax_split_pass1(const float* __restrict__ x, float* __restrict__ part,
                                                                int64_t cols, int splits, int64_t chunk) {
  __shared__ float sm[2 * kWaves];
  const int64_t id = blockIdx.x;
  const int64_t row = id / splits;
  const int64_t ck = id - row * splits;
  const int64_t begin = ck * chunk;
  const int64_t end = begin + chunk < cols ? begin + chunk : cols;
  State s = (VEC == 4 && end - begin == kSoftmaxChunk) ? scan_chunk(x + row * cols + begin)
                                                        : scan<VEC>(x + row * cols, begin, end);
  s = block_merge(s, sm);
  if (threadIdx.x == 0) {
    part[2 * id] = s.m;
    part[2 * id + 1] = s.l;
  }
}

// Split rows, pass 2: merge the row's partials, then normalise one chunk.
template <int VEC>
__global__ __launch_bounds__(kThreads) void softmax_split_pass2(const float* x, float* y,
                                                                const float* __restrict__ part, int64_t cols,
                                                                int splits, int64_t chunk) {
  __shared__ float sm[2 * kWaves];
  const int64_t id = blockIdx.x;
  const int64_t row = id / splits;
  const int64_t ck = id - row * splits;
  State s = {kNegInf, 0.f};
  const float* pr = part + 2 * row * splits;
  for (int i = threadIdx.x; i < splits; i += kThreads) merge_state(s, pr[2 * i], pr[2 * i + 1]);
  s = block_merge(s, sm);
  const int64_t begin = ck * chunk;
  const int64_t end = begin + chunk < cols ? begin + chunk : cols;
  if (VEC == 4 && end - begin == kSoftmaxChunk)
    normalise_chunk(x + row * cols + begin, y + row * cols + begin, s.m, 1.0f / s.l);
  else
    normalise<VEC>(x + row * cols, y + row * cols, begin, end, s.m, 1.0f / s.l);
}

}  // namespace

hipError_t launch_softmax_rows(const SoftmaxArgs& a) {
  const bool vec = (a.cols % 4 == 0) && ((reinterpret_cast<uintptr_t>(a.x) & 15) == 0) &&
                   ((reinterpret_cast<uintptr_t>(a.y) & 15) == 0);
  const dim3 block(kThreads);
  if (a.plan.kernel == OSX_KERNEL_SOFTMAX_ROW) {
    const dim3 grid((unsigned)a.rows);
    if (vec)
      hipLaunchKernelGGL(softmax_row_kernel<4>, grid, block, 0, a.stream, a.x, a.y, a.cols);
    else
      hipLaunchKernelGGL(softmax_row_kernel<1>, grid, block, 0, a.stream, a.x, a.y, a.cols);
    return hipGetLastError();
  }
  float* part = static_cast<float*>(a.workspace);
  const dim3 grid((unsigned)a.plan.grid);
  const int64_t chunk = a.plan.block_m;
  if (vec) {
    hipLaunchKernelGGL(softmax_split_pass1<4>, grid, block, 0, a.stream, a.x, part, a.cols, a.plan.splits, chunk);
    hipLaunchKernelGGL(softmax_split_pass2<4>, grid, block, 0, a.stream, a.x, a.y, part, a.cols, a.plan.splits,
                       chunk);
  } else {
    hipLaunchKernelGGL(softmax_split_pass1<1>, grid, block, 0, a.stream, a.x, part, a.cols, a.plan.splits, chunk);
    hipLaunchKernelGGL(softmax_split_pass2<1>, grid, block, 0, a.stream, a.x, a.y, part, a.cols, a.plan.splits,
                       chunk);
  }
  return hipGetLastError();
}

}  // namespace osx
