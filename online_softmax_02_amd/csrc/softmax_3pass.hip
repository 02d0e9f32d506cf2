// Three-pass row softmax designs, kept as comparators for the two-pass online
// softmax: each reads x three times (or reads and writes y twice) where the
// online pass needs two reads (or one, for rows held in registers).
//
// OSX_3PASS_ATOMIC -- page "Softmax 算子的实现与优化", section Baseline: a max
//   launch, a sum-of-exponentials launch and a normalising launch.  The
//   programs of one row combine their partial max and partial sum through
//   atomic updates of one (m, l) pair per row, which a fourth small launch sets
//   to (-inf, 0) first.
// OSX_3PASS_STASH -- same page, section CUDA 版本: pass 1 finds the max, pass 2
//   writes e^{x - m} into y while summing it, pass 3 multiplies y by 1/l.  The
//   page runs one 256-thread block over the whole vector (one CU); here every
//   pass is spread over chunk workgroups, whose per-chunk partials (a max, then
//   a sum) the next pass combines.
//
// fp32 in and out.  Rows are cut into chunks (softmax_3pass_chunk), one
// workgroup each, as in the split two-pass kernels; 16-byte loads when the
// row length is a multiple of 4 and x / y are 16-byte aligned.
#include "common.hpp"
#include "launch.hpp"

namespace osx {
namespace {

constexpr int kThreads = kSoftmaxThreads;
constexpr int kWaves = kThreads / kWaveSize;

// Four consecutive values of a row starting at idx (a multiple of 4); past
// `end` they read as -inf, which adds nothing to a max or a sum of exp.
template <bool VEC>
__device__ __forceinline__ void load4(const float* __restrict__ p, int64_t idx, int64_t end, float (&v)[4]) {
  if (VEC) {
    const f32x4 w = *reinterpret_cast<const f32x4*>(p + idx);
    v[0] = w.x;
    v[1] = w.y;
    v[2] = w.z;
    v[3] = w.w;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = idx + e < end ? p[idx + e] : kNegInf;
  }
}

template <bool VEC>
__device__ __forceinline__ void store4(float* __restrict__ p, int64_t idx, int64_t end, const float (&v)[4]) {
  if (VEC) {
    *reinterpret_cast<f32x4*>(p + idx) = f32x4{v[0], v[1], v[2], v[3]};
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (idx + e < end) p[idx + e] = v[e];
  }
}

__device__ __forceinline__ float block_max(float v, float* sm) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = sm[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = fmaxf(r, sm[w]);
  return r;
}

__device__ __forceinline__ float block_sum(float v, float* sm) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = sm[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r += sm[w];
  return r;
}

// Atomic max of a float through its bit pattern: non-negative floats order as
// signed integers, negative ones in reverse as unsigned integers, and every
// non-negative float is above every negative one, so one integer atomic on the
// right branch leaves the larger float in *p.  Exact; NaN inputs are not
// expected (softmax of NaN is NaN anyway).
__device__ __forceinline__ void atomic_max_f32(float* p, float v) {
  if (v >= 0.f)
    atomicMax(reinterpret_cast<int*>(p), __float_as_int(v));
  else
    atomicMin(reinterpret_cast<unsigned int*>(p), __float_as_uint(v));
}

struct Chunk {
  int64_t row, id, begin, end;
};

__device__ __forceinline__ Chunk chunk_of(int64_t cols, int splits, int64_t chunk) {
  Chunk c;
  c.id = blockIdx.x;
  c.row = c.id / splits;
  c.begin = (c.id - c.row * splits) * chunk;
  c.end = c.begin + chunk < cols ? c.begin + chunk : cols;
  return c;
}

// ---- OSX_3PASS_ATOMIC -------------------------------------------------------

__global__ __launch_bounds__(kThreads) void row_state_init(float* __restrict__ ml, int64_t rows) {
  const int64_t r = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (r < rows) {
    ml[2 * r] = kNegInf;
    ml[2 * r + 1] = 0.f;
  }
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void atomic_max_pass(const float* __restrict__ x, float* __restrict__ ml,
                                                            int64_t cols, int splits, int64_t chunk) {
  __shared__ float sm[kWaves];
  const Chunk c = chunk_of(cols, splits, chunk);
  const float* xr = x + c.row * cols;
  float m = kNegInf;
  for (int64_t i = c.begin + 4 * (int64_t)threadIdx.x; i < c.end; i += 4 * kThreads) {
    float v[4];
    load4<VEC>(xr, i, c.end, v);
    m = fmaxf(m, fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
  }
  m = block_max(m, sm);
  if (threadIdx.x == 0) atomic_max_f32(&ml[2 * c.row], m);
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void atomic_sum_pass(const float* __restrict__ x, float* __restrict__ ml,
                                                            int64_t cols, int splits, int64_t chunk) {
  __shared__ float sm[kWaves];
  const Chunk c = chunk_of(cols, splits, chunk);
  const float* xr = x + c.row * cols;
  const float m = ml[2 * c.row];
  float l = 0.f;
  for (int64_t i = c.begin + 4 * (int64_t)threadIdx.x; i < c.end; i += 4 * kThreads) {
    float v[4];
    load4<VEC>(xr, i, c.end, v);
#pragma unroll
    for (int e = 0; e < 4; ++e) l += exp2_fast((v[e] - m) * kLog2e);
  }
  l = block_sum(l, sm);
  if (threadIdx.x == 0) atomicAdd(&ml[2 * c.row + 1], l);
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void atomic_normalise_pass(const float* x, float* y,
                                                                  const float* __restrict__ ml, int64_t cols,
                                                                  int splits, int64_t chunk) {
  const Chunk c = chunk_of(cols, splits, chunk);
  const float* xr = x + c.row * cols;
  float* yr = y + c.row * cols;
  const float m = ml[2 * c.row], inv_l = 1.0f / ml[2 * c.row + 1];
  for (int64_t i = c.begin + 4 * (int64_t)threadIdx.x; i < c.end; i += 4 * kThreads) {
    float v[4];
    load4<VEC>(xr, i, c.end, v);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = exp2_fast((v[e] - m) * kLog2e) * inv_l;
    store4<VEC>(yr, i, c.end, v);
  }
}

// ---- OSX_3PASS_STASH --------------------------------------------------------

template <bool VEC>
__global__ __launch_bounds__(kThreads) void stash_max_pass(const float* __restrict__ x, float* __restrict__ part,
                                                           int64_t cols, int splits, int64_t chunk) {
  __shared__ float sm[kWaves];
  const Chunk c = chunk_of(cols, splits, chunk);
  const float* xr = x + c.row * cols;
  float m = kNegInf;
  for (int64_t i = c.begin + 4 * (int64_t)threadIdx.x; i < c.end; i += 4 * kThreads) {
    float v[4];
    load4<VEC>(xr, i, c.end, v);
    m = fmaxf(m, fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
  }
  m = block_max(m, sm);
  if (threadIdx.x == 0) part[2 * c.id] = m;
}

// The row max from its chunk partials, then y = e^{x - m} and the chunk's sum of it.
template <bool VEC>
__global__ __launch_bounds__(kThreads) void stash_exp_pass(const float* x, float* y, float* __restrict__ part,
                                                           int64_t cols, int splits, int64_t chunk) {
  __shared__ float sm[kWaves];
  const Chunk c = chunk_of(cols, splits, chunk);
  const float* pr = part + 2 * c.row * splits;
  float m = kNegInf;
  for (int i = threadIdx.x; i < splits; i += kThreads) m = fmaxf(m, pr[2 * i]);
  m = block_max(m, sm);
  __syncthreads();  // sm is reused by the sum below
  const float* xr = x + c.row * cols;
  float* yr = y + c.row * cols;
  float l = 0.f;
  for (int64_t i = c.begin + 4 * (int64_t)threadIdx.x; i < c.end; i += 4 * kThreads) {
    float v[4];
    load4<VEC>(xr, i, c.end, v);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = exp2_fast((v[e] - m) * kLog2e);
      l += v[e];
    }
    store4<VEC>(yr, i, c.end, v);
  }
  l = block_sum(l, sm);
  if (threadIdx.x == 0) part[2 * c.id + 1] = l;
}

// The row sum from its chunk partials, then y *= 1/l.
template <bool VEC>
__global__ __launch_bounds__(kThreads) void stash_scale_pass(float* y, const float* __restrict__ part, int64_t cols,
                                                             int splits, int64_t chunk) {
  __shared__ float sm[kWaves];
  const Chunk c = chunk_of(cols, splits, chunk);
  const float* pr = part + 2 * c.row * splits;
  float l = 0.f;
  for (int i = threadIdx.x; i < splits; i += kThreads) l += pr[2 * i + 1];
  const float inv_l = 1.0f / block_sum(l, sm);
  float* yr = y + c.row * cols;
  for (int64_t i = c.begin + 4 * (int64_t)threadIdx.x; i < c.end; i += 4 * kThreads) {
    float v[4];
    load4<VEC>(yr, i, c.end, v);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] *= inv_l;
    store4<VEC>(yr, i, c.end, v);
  }
}

template <bool VEC>
hipError_t launch_v(const Softmax3PassArgs& a) {
  const float* x = static_cast<const float*>(a.x);
  float* y = static_cast<float*>(a.y);
  float* ws = static_cast<float*>(a.workspace);
  const dim3 grid((unsigned)a.grid), block(kThreads);
  hipError_t e;
  if (a.method == OSX_3PASS_ATOMIC) {
    hipLaunchKernelGGL(row_state_init, dim3((unsigned)((a.rows + kThreads - 1) / kThreads)), block, 0, a.stream, ws,
                       a.rows);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((atomic_max_pass<VEC>), grid, block, 0, a.stream, x, ws, a.cols, a.splits, a.chunk);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((atomic_sum_pass<VEC>), grid, block, 0, a.stream, x, ws, a.cols, a.splits, a.chunk);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((atomic_normalise_pass<VEC>), grid, block, 0, a.stream, x, y, ws, a.cols, a.splits, a.chunk);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((stash_max_pass<VEC>), grid, block, 0, a.stream, x, ws, a.cols, a.splits, a.chunk);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((stash_exp_pass<VEC>), grid, block, 0, a.stream, x, y, ws, a.cols, a.splits, a.chunk);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((stash_scale_pass<VEC>), grid, block, 0, a.stream, y, ws, a.cols, a.splits, a.chunk);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_softmax_3pass(const Softmax3PassArgs& a) {
  const bool vec = (a.cols % 4 == 0) && ((reinterpret_cast<uintptr_t>(a.x) & 15) == 0) &&
                   ((reinterpret_cast<uintptr_t>(a.y) & 15) == 0);
  return vec ? launch_v<true>(a) : launch_v<false>(a);
}

}  // namespace osx
