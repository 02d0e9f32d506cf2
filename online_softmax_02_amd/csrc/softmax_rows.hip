// Two-pass row softmax for gfx950: y = softmax(scale * x) along each row,
// optionally with a causal mask, fp32 or bf16 in and out (fp32 arithmetic).
//
// Pass 1 keeps an online state per thread -- the running max m and the sum l
// of exp(scale (x - m)) -- rescaling l by exp(scale (m_old - m_new)) whenever
// the max grows, then merges the per-thread states across the wavefront and
// the workgroup (page "Softmax 算子的实现与优化", section Online Softmax: the
// boxed update and the invariant l = sum_j e^{x_j - m}).  Pass 2 reads x again
// and writes y = exp(scale (x - m)) / l.  Out-of-range positions contribute
// nothing (-inf to the max, 0 to the sum).
//
// Causal mask (page "从零开始写Qwen3（五-其一）使用Triton实现自注意力", section
// softmax的triton实现: keep column <= row, the rest counts as -inf): for a
// causal period P > 0, row r keeps columns c <= r mod P, i.e. the rows are
// stacked [P, cols] score matrices of several heads.  Masked columns are never
// read; they are written as 0.
//
// Three shapes of launch, by row length:
//  * rows up to kSoftmaxWaveMax elements: one wavefront per row, the row held
//    in its registers, so x is read from memory once; the per-lane states merge
//    by lane shuffles, with no barrier;
//  * rows up to kSoftmaxRowMax elements: the same with one workgroup per row,
//    merged through LDS (the pages keep (m, l) inside one program);
//  * longer rows: the row is cut into kSoftmaxChunk-element chunks, one
//    workgroup each.  Pass 1 writes one (m, l) partial per chunk; pass 2
//    issues the loads of its chunk (x read again), merges the row's partials
//    with the same rescaling rule while they are in flight, then normalises
//    the chunk.  This replaces the single-program scan, which cannot use more
//    than one CU.
//
// Exponentials are 2^((x - m) * k) with k = scale * log2 e, on the
// transcendental unit.  The split-row kernels form the exponent as one FMA,
// x k - m k, with m k rounded once per thread: its rounding is a factor common
// to a chunk's sum and to the outputs normalised with the same m, and it saves
// one vector instruction per element in each pass.
#include "common.hpp"
#include "launch.hpp"

namespace osx {
namespace {

constexpr int kThreads = kSoftmaxThreads;
constexpr int kWaves = kThreads / kWaveSize;

// Element types: fp32, or bf16 held as its 16-bit pattern.  A 16-byte vector
// holds E elements.
template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int E = 4;
  static __device__ __forceinline__ float get(const float* p) { return *p; }
  static __device__ __forceinline__ void put(float* p, float v) { *p = v; }
  // The whole vector is bit-cast: ROCm 7.2 clang lowers a bit-cast of one
  // ext-vector component (w.y) as a load from the vector's first element.
  static __device__ __forceinline__ void unpack(u32x4 w, float (&v)[E]) {
    const f32x4 f = __builtin_bit_cast(f32x4, w);
    v[0] = f.x;
    v[1] = f.y;
    v[2] = f.z;
    v[3] = f.w;
  }
  static __device__ __forceinline__ u32x4 pack(const float (&v)[E]) {
    return __builtin_bit_cast(u32x4, f32x4{v[0], v[1], v[2], v[3]});
  }
};
template <>
struct Elem<uint16_t> {
  static constexpr int E = 8;
  static __device__ __forceinline__ float get(const uint16_t* p) { return bf16_lo((uint32_t)*p); }
  static __device__ __forceinline__ void put(uint16_t* p, float v) { *p = (uint16_t)(pack_bf16x2(v, 0.f) & 0xffffu); }
  static __device__ __forceinline__ void unpack(u32x4 w, float (&v)[E]) {
    v[0] = bf16_lo(w.x);
    v[1] = bf16_hi(w.x);
    v[2] = bf16_lo(w.y);
    v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z);
    v[5] = bf16_hi(w.z);
    v[6] = bf16_lo(w.w);
    v[7] = bf16_hi(w.w);
  }
  static __device__ __forceinline__ u32x4 pack(const float (&v)[E]) {
    return u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
  }
};

template <typename T>
__device__ __forceinline__ u32x4 ld16(const T* p) { return *reinterpret_cast<const u32x4*>(p); }
template <typename T>
__device__ __forceinline__ void st16(T* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Online state: m is a max of x, l = sum 2^((x - m) k) over the elements seen.
struct State {
  float m, l;
};

__device__ __forceinline__ void merge_state(State& s, float mb, float lb, float k) {
  const float mn = fmaxf(s.m, mb);
  if (mn == kNegInf) return;  // both empty
  s.l = s.l * exp2_fast((s.m - mn) * k) + lb * exp2_fast((mb - mn) * k);
  s.m = mn;
}

// Fold a group of values into the state: one max over the group, one rescale.
template <int N>
__device__ __forceinline__ void update(State& s, const float (&v)[N], float k) {
  float mb = v[0];
#pragma unroll
  for (int i = 1; i < N; ++i) mb = fmaxf(mb, v[i]);
  const float mn = fmaxf(s.m, mb);
  if (mn == kNegInf) return;
  float sum = 0.f;
  const float mk = mn * k;
#pragma unroll
  for (int i = 0; i < N; ++i) sum += exp2_fast(fmaf(v[i], k, -mk));
  s.l = s.l * exp2_fast((s.m - mn) * k) + sum;
  s.m = mn;
}

// Merge the states of the 64 lanes of a wavefront; every lane gets the result.
__device__ __forceinline__ State wave_merge(State s, float k) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float mb = __shfl_xor(s.m, o, 64);
    const float lb = __shfl_xor(s.l, o, 64);
    merge_state(s, mb, lb, k);
  }
  return s;
}

// Merge the states of all threads of the workgroup; every thread gets the result.
__device__ __forceinline__ State block_merge(State s, float* sm /* 2*kWaves floats */, float k) {
  s = wave_merge(s, k);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    sm[2 * wave] = s.m;
    sm[2 * wave + 1] = s.l;
  }
  __syncthreads();
  OSX_DEBUG_SYNC_WG();
  State r = {sm[0], sm[1]};
#pragma unroll
  for (int w = 1; w < kWaves; ++w) merge_state(r, sm[2 * w], sm[2 * w + 1], k);
  OSX_DEBUG_SYNC_WG();
  return r;
}

// Online pass over x[begin, end) of one row.  VEC: 16-byte loads of E
// elements (begin a multiple of E, x 16-byte aligned) plus a scalar tail.
template <typename T, bool VEC>
__device__ __forceinline__ State scan(const T* __restrict__ x, int64_t begin, int64_t end, float k) {
  using L = Elem<T>;
  constexpr int E = L::E;
  State s = {kNegInf, 0.f};
  const int tid = threadIdx.x;
  int64_t tail = begin;
  if (VEC && end > begin) {
    const int64_t nv = (end - begin) / E;
    const T* xb = x + begin;
    int64_t i = tid;
    for (; i + kThreads < nv; i += 2 * kThreads) {
      const u32x4 a = ld16(xb + E * i), b = ld16(xb + E * (i + kThreads));
      float va[E], vb[E], v[2 * E];
      L::unpack(a, va);
      L::unpack(b, vb);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        v[e] = va[e];
        v[E + e] = vb[e];
      }
      update(s, v, k);
    }
    for (; i < nv; i += kThreads) {
      float v[E];
      L::unpack(ld16(xb + E * i), v);
      update(s, v, k);
    }
    tail = begin + nv * E;
  }
  for (int64_t i = tail + tid; i < end; i += kThreads) {
    const float v[1] = {L::get(x + i)};
    update(s, v, k);
  }
  return s;
}

// Normalise pass over [begin, end): y = 2^((x - m) k) * inv_l.
template <typename T, bool VEC>
__device__ __forceinline__ void normalise(const T* __restrict__ x, T* __restrict__ y, int64_t begin, int64_t end,
                                          float m, float inv_l, float k) {
  using L = Elem<T>;
  constexpr int E = L::E;
  const int tid = threadIdx.x;
  const float mk = m * k;
  int64_t tail = begin;
  if (VEC && end > begin) {
    const int64_t nv = (end - begin) / E;
    for (int64_t i = tid; i < nv; i += kThreads) {
      float v[E];
      L::unpack(ld16(x + begin + E * i), v);
#pragma unroll
      for (int e = 0; e < E; ++e) v[e] = exp2_fast(fmaf(v[e], k, -mk)) * inv_l;
      st16(y + begin + E * i, L::pack(v));
    }
    tail = begin + nv * E;
  }
  for (int64_t i = tail + tid; i < end; i += kThreads) L::put(y + i, exp2_fast(fmaf(L::get(x + i), k, -mk)) * inv_l);
}

// Masked columns [begin, end) of a row: y = 0.
template <typename T, bool VEC>
__device__ __forceinline__ void zero_fill(T* __restrict__ y, int64_t begin, int64_t end) {
  using L = Elem<T>;
  constexpr int E = L::E;
  const int tid = threadIdx.x;
  if (end <= begin) return;
  int64_t head = end;  // scalar stores cover [begin, head)
  if (VEC) {
    head = (begin + E - 1) / E * E;  // the row starts 16-byte aligned, so this is too
    if (head > end) head = end;
    const int64_t nv = (end - head) / E;
    for (int64_t i = tid; i < nv; i += kThreads) st16(y + head + E * i, u32x4{0u, 0u, 0u, 0u});
    for (int64_t i = head + nv * E + tid; i < end; i += kThreads) L::put(y + i, 0.f);
  }
  for (int64_t i = begin + tid; i < head; i += kThreads) L::put(y + i, 0.f);
}

// Visible columns of a row: all, or c <= row mod period.
__device__ __forceinline__ int64_t row_limit(int64_t row, int64_t cols, int64_t period) {
  if (period <= 0) return cols;
  const int64_t lim = row % period + 1;
  return lim < cols ? lim : cols;
}

// A full unmasked chunk of kSoftmaxChunk elements, 16-byte loads: every thread
// issues all of its loads before using any, so a workgroup keeps its whole
// chunk in flight.  Thread state: its exact max, then the sum of
// 2^((x - m) k) over its values (the block-level merge is the rescaling rule).
// Pass 1 loads normally so x stays cached for pass 2; pass 2 is the last use
// of x and streams y out with non-temporal accesses.
template <typename T>
__device__ __forceinline__ State scan_chunk(const T* __restrict__ xb, float k) {
  using L = Elem<T>;
  constexpr int E = L::E, NV = (int)(kSoftmaxChunk / E / kThreads);
  u32x4 w[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) w[i] = ld16(xb + E * (threadIdx.x + i * kThreads));
  // Folded in groups of GV vectors, in load order, so the arithmetic on the
  // first groups runs while the later ones are still arriving.
  constexpr int GV = NV < 8 ? NV : 8;
  float m = kNegInf, l = 0.f;
#pragma unroll
  for (int g0 = 0; g0 < NV; g0 += GV) {
    float gm = kNegInf;
#pragma unroll
    for (int i = g0; i < g0 + GV; ++i) {
      float v[E];
      L::unpack(w[i], v);
#pragma unroll
      for (int e = 0; e < E; e += 2) gm = fmaxf(gm, fmaxf(v[e], v[e + 1]));
    }
    const float mn = fmaxf(m, gm);
    l *= exp2_fast((m - mn) * k);  // 0 for the first group (m = -inf)
    m = mn;
    const float mk = m * k;
#pragma unroll
    for (int i = g0; i < g0 + GV; ++i) {
      float v[E];
      L::unpack(w[i], v);
#pragma unroll
      for (int e = 0; e < E; e += 2) l += exp2_fast(fmaf(v[e], k, -mk)) + exp2_fast(fmaf(v[e + 1], k, -mk));
    }
  }
  return State{m, l};
}

// A whole chunk's 16-byte vectors per thread, loaded by chunk_load and
// normalised from the registers by normalise_chunk.
template <typename T>
constexpr int kChunkVecs = (int)(kSoftmaxChunk / Elem<T>::E / kThreads);

template <typename T>
__device__ __forceinline__ void chunk_load(const T* xb, u32x4 (&w)[kChunkVecs<T>]) {
#pragma unroll
  for (int i = 0; i < kChunkVecs<T>; ++i)
    w[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xb) + threadIdx.x + i * kThreads);
}

template <typename T>
__device__ __forceinline__ void normalise_chunk(const u32x4 (&w)[kChunkVecs<T>], T* yb, float m, float inv_l,
                                                float k) {
  using L = Elem<T>;
  constexpr int E = L::E, NV = kChunkVecs<T>;
  const float mk = m * k;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    float v[E];
    L::unpack(w[i], v);
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = exp2_fast(fmaf(v[e], k, -mk)) * inv_l;
    __builtin_nontemporal_store(L::pack(v), reinterpret_cast<u32x4*>(yb) + threadIdx.x + i * kThreads);
  }
}

// A row held in registers: R threads (one wavefront, or the whole workgroup)
// cover one row, thread t holding the 16-byte vectors t, t + R, ... (VEC) or
// the elements t, t + R, ... (scalar), NV vectors' worth either way.  Each
// thread folds its visible values into (m, l); the states merge across the R
// threads; the outputs come from the registers, so x is read once.  x and y
// may be the same buffer: a row's reads all feed the merge, which comes before
// its first store, and its zero stores (the masked vectors) never overlap the
// vectors it reads.

constexpr int kNonTemporal = 2;               // buffer-op cache policy: x and y are streamed once
constexpr uint32_t kOffNowhere = 0x80000000u;  // a buffer offset past any row: the store is dropped

// 16-byte path, first half of a row: load the nvis vectors that hold a visible
// column; the buffer returns 0 past them.  The loads are unconditional buffer
// operations, so they issue back to back and the compiler's wait counts are
// exact.
template <typename T, int NV, int R>
__device__ __forceinline__ void vec_issue(const T* xr, uint32_t nvis, int t, u32x4 (&w)[NV]) {
  const __amdgpu_buffer_rsrc_t xs = make_rsrc(xr, nvis * 16u);
#pragma unroll
  for (int i = 0; i < NV; ++i)
    w[i] = __builtin_amdgcn_raw_buffer_load_b128(xs, 16u * (uint32_t)(t + R * i), 0, kNonTemporal);
}

// Second half: (m, l) of the visible values (column < lim), merged over the
// R threads; then y = 2^((x - m) k) / l for the nvis loaded vectors (0 for
// their masked columns).  Each thread keeps p = 2^((x - m_t) k) against its
// own max m_t from the sum and scales it by 2^((m_t - m) k) / l for the
// output, so every element takes one exponential.  Vector slot i holds
// vectors t + R i of the R threads: when R i >= nvis no thread's slot-i vector
// holds a visible column, and the slot's exponentials and stores are skipped
// (a branch that is uniform over the group).  Last, 0 goes to the masked
// vectors (nvis <= vi < nv), again through unconditional buffer stores: the
// range check drops the visible ones.  (Issued after the row's own stores
// rather than while its loads are in flight, they measured 3% faster on
// causal bf16 rows of 2048 columns.)
template <typename T, int NV, int R>
__device__ __forceinline__ void vec_finish(T* yr, int lim, uint32_t nvis, uint32_t nv, int t, const u32x4 (&w)[NV],
                                           float k, float* sm) {
  using L = Elem<T>;
  constexpr int E = L::E, N = NV * E;
  float v[N];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    float f[E];
    L::unpack(w[i], f);
    const int c0 = E * (t + R * i);  // resident rows have at most kSoftmaxRowMax columns
#pragma unroll
    for (int e = 0; e < E; ++e) v[i * E + e] = c0 + e < lim ? f[e] : kNegInf;
  }
  float m = v[0];
#pragma unroll
  for (int j = 1; j < N; ++j) m = fmaxf(m, v[j]);
  const float m_use = m == kNegInf ? 0.f : m;  // a thread with nothing visible: every p is 2^-inf = 0
  float l = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    if ((uint32_t)(R * i) >= nvis) break;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      v[i * E + e] = exp2_fast((v[i * E + e] - m_use) * k);
      l += v[i * E + e];
    }
  }
  State s = {m, l};
  s = R == kWaveSize ? wave_merge(s, k) : block_merge(s, sm, k);
  const float scale = m == kNegInf ? 0.f : exp2_fast((m - s.m) * k) / s.l;
  const __amdgpu_buffer_rsrc_t ys = make_rsrc(yr, nvis * 16u);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    if ((uint32_t)(R * i) >= nvis) break;
    float f[E];
#pragma unroll
    for (int e = 0; e < E; ++e) f[e] = v[i * E + e] * scale;
    __builtin_amdgcn_raw_buffer_store_b128(L::pack(f), ys, 16u * (uint32_t)(t + R * i), 0, kNonTemporal);
  }
  const __amdgpu_buffer_rsrc_t zs = make_rsrc(yr, nv * 16u);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const uint32_t vi = (uint32_t)(t + R * i);
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, zs, vi >= nvis ? 16u * vi : kOffNowhere, 0,
                                           kNonTemporal);
  }
}

// Scalar path (cols not a multiple of the vector width, or x / y not 16-byte
// aligned): one row, elements t, t + R, ...
template <typename T, int NV, int R>
__device__ __forceinline__ void scalar_row(const T* xr, T* yr, int64_t lim, int64_t cols, int t, float k, float* sm) {
  using L = Elem<T>;
  constexpr int N = NV * L::E;
  float v[N];
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const int64_t c = t + (int64_t)R * j;
    v[j] = c < lim ? L::get(xr + c) : kNegInf;
  }
  float m = v[0];
#pragma unroll
  for (int j = 1; j < N; ++j) m = fmaxf(m, v[j]);
  float l = 0.f;
  if (m != kNegInf) {
#pragma unroll
    for (int j = 0; j < N; ++j) l += exp2_fast((v[j] - m) * k);
  }
  State s = {m, l};
  s = R == kWaveSize ? wave_merge(s, k) : block_merge(s, sm, k);
  const float inv_l = 1.0f / s.l;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const int64_t c = t + (int64_t)R * j;
    if (c >= cols) break;
    L::put(yr + c, exp2_fast((v[j] - s.m) * k) * inv_l);  // 0 where masked (x = -inf)
  }
}

// One wavefront per row, four rows per workgroup.
template <typename T, bool VEC, int NV>
__global__ __launch_bounds__(kThreads) void softmax_wave_kernel(const T* x, T* y, int64_t rows, int64_t cols, float k,
                                                                int64_t period) {
  constexpr int E = Elem<T>::E;
  const int t = (int)threadIdx.x & (kWaveSize - 1);
  const int64_t row = (int64_t)blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWaveSize);
  if (row >= rows) return;  // a whole wavefront; no barrier follows
  const int lim = (int)row_limit(row, cols, period);  // resident rows have at most kSoftmaxRowMax columns
  if (VEC) {
    const uint32_t nvis = __builtin_amdgcn_readfirstlane((uint32_t)((lim + E - 1) / E));
    u32x4 w[NV];
    vec_issue<T, NV, kWaveSize>(x + row * cols, nvis, t, w);
    vec_finish<T, NV, kWaveSize>(y + row * cols, lim, nvis, (uint32_t)(cols / E), t, w, k, nullptr);
  } else {
    scalar_row<T, NV, kWaveSize>(x + row * cols, y + row * cols, lim, cols, t, k, nullptr);
  }
}

// One workgroup per row.
template <typename T, bool VEC, int NV>
__global__ __launch_bounds__(kThreads) void softmax_row_kernel(const T* x, T* y, int64_t cols, float k,
                                                               int64_t period) {
  constexpr int E = Elem<T>::E;
  __shared__ float sm[2 * kWaves];
  const int64_t row = blockIdx.x;
  const int64_t lim = row_limit(row, cols, period);
  const int t = (int)threadIdx.x;
  if (VEC) {
    const uint32_t nvis = __builtin_amdgcn_readfirstlane((uint32_t)((lim + E - 1) / E));
    u32x4 w[NV];
    vec_issue<T, NV, kThreads>(x + row * cols, nvis, t, w);
    vec_finish<T, NV, kThreads>(y + row * cols, (int)lim, nvis, (uint32_t)(cols / E), t, w, k, sm);
  } else {
    scalar_row<T, NV, kThreads>(x + row * cols, y + row * cols, lim, cols, t, k, sm);
  }
}

// Split rows, pass 1: the (m, l) partial of one chunk (empty when the chunk is
// wholly masked).
template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void softmax_split_pass1(const T* __restrict__ x, float* __restrict__ part,
                                                                int64_t cols, int splits, int64_t chunk, float k,
                                                                int64_t period) {
  __shared__ float sm[2 * kWaves];
  const int64_t id = blockIdx.x;
  const int64_t row = id / splits;
  const int64_t ck = id - row * splits;
  const int64_t lim = row_limit(row, cols, period);
  const int64_t begin = ck * chunk;
  int64_t end = begin + chunk < cols ? begin + chunk : cols;
  if (end > lim) end = lim;
  State s = (VEC && end - begin == kSoftmaxChunk) ? scan_chunk(x + row * cols + begin, k)
                                                  : scan<T, VEC>(x + row * cols, begin, end, k);
  s = block_merge(s, sm, k);
  if (threadIdx.x == 0) {
    part[2 * id] = s.m;
    part[2 * id + 1] = s.l;
  }
}

// Split rows, pass 2: merge the row's partials, then normalise one chunk.  A
// whole chunk's loads are issued first, so they are in flight while the
// partials are read and merged.  Workgroups are dealt to the 8 XCDs round-robin, so chunk id runs on XCD
// id mod 8 in both passes; pass 2 walks each XCD's chunks in reverse, so it
// starts with the chunks pass 1 read last, which are still in that XCD's L2
// (2% faster on a 2^24-element row than the same order).
template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void softmax_split_pass2(const T* x, T* y, const float* __restrict__ part,
                                                                int64_t cols, int splits, int64_t chunk, float k,
                                                                int64_t period) {
  __shared__ float sm[2 * kWaves];
  const int64_t nwg = gridDim.x;
  const int64_t id =
      nwg % 8 == 0 ? (nwg / 8 - 1 - (int64_t)blockIdx.x / 8) * 8 + blockIdx.x % 8 : (int64_t)blockIdx.x;
  const int64_t row = id / splits;
  const int64_t ck = id - row * splits;
  const int64_t lim = row_limit(row, cols, period);
  const int64_t begin = ck * chunk;
  const int64_t end = begin + chunk < cols ? begin + chunk : cols;
  const int64_t vis = end < lim ? end : lim;
  const bool whole = VEC && vis - begin == kSoftmaxChunk;  // uniform across the workgroup
  u32x4 w[kChunkVecs<T>];
  if (whole) chunk_load(x + row * cols + begin, w);
  State s = {kNegInf, 0.f};
  const float* pr = part + 2 * row * splits;
  for (int i = threadIdx.x; i < splits; i += kThreads) merge_state(s, pr[2 * i], pr[2 * i + 1], k);
  s = block_merge(s, sm, k);
  if (whole)
    normalise_chunk(w, y + row * cols + begin, s.m, 1.0f / s.l, k);
  else
    normalise<T, VEC>(x + row * cols, y + row * cols, begin, vis, s.m, 1.0f / s.l, k);
  zero_fill<T, VEC>(y + row * cols, vis > begin ? vis : begin, end);
}

// Vectors per thread for a row held by R threads: cols / (R E), rounded up to
// a power of two (at most 8: the planner keeps rows within 32 elements per thread).
template <typename T>
int vectors_per_thread(int64_t cols, int R) {
  const int64_t per = (cols + (int64_t)R * Elem<T>::E - 1) / ((int64_t)R * Elem<T>::E);
  return per <= 1 ? 1 : per <= 2 ? 2 : per <= 4 ? 4 : per <= 8 ? 8 : 0;
}

template <typename T, bool VEC, int NV>
hipError_t launch_wave_nv(const SoftmaxArgs& a, const T* x, T* y) {
  if constexpr (NV * Elem<T>::E > 32) return hipErrorInvalidValue;  // never planned: at most 32 elements per lane
  hipLaunchKernelGGL((softmax_wave_kernel<T, VEC, NV>), dim3((unsigned)a.plan.grid), dim3(kThreads), 0, a.stream, x, y,
                     a.rows, a.cols, a.k, a.period);
  return hipGetLastError();
}

template <typename T, bool VEC, int NV>
hipError_t launch_row_nv(const SoftmaxArgs& a, const T* x, T* y) {
  if constexpr (NV * Elem<T>::E > 32) return hipErrorInvalidValue;  // never planned: at most 32 elements per thread
  hipLaunchKernelGGL((softmax_row_kernel<T, VEC, NV>), dim3((unsigned)a.plan.grid), dim3(kThreads), 0, a.stream, x, y,
                     a.cols, a.k, a.period);
  return hipGetLastError();
}

template <typename T, bool VEC>
hipError_t launch_resident(const SoftmaxArgs& a) {
  const T* x = static_cast<const T*>(a.x);
  T* y = static_cast<T*>(a.y);
  if (a.plan.kernel == OSX_KERNEL_SOFTMAX_WAVE) {
    switch (vectors_per_thread<T>(a.cols, kWaveSize)) {
      case 1: return launch_wave_nv<T, VEC, 1>(a, x, y);
      case 2: return launch_wave_nv<T, VEC, 2>(a, x, y);
      case 4: return launch_wave_nv<T, VEC, 4>(a, x, y);
      case 8: return launch_wave_nv<T, VEC, 8>(a, x, y);
      default: return hipErrorInvalidValue;
    }
  }
  switch (vectors_per_thread<T>(a.cols, kThreads)) {
    case 1: return launch_row_nv<T, VEC, 1>(a, x, y);
    case 2: return launch_row_nv<T, VEC, 2>(a, x, y);
    case 4: return launch_row_nv<T, VEC, 4>(a, x, y);
    case 8: return launch_row_nv<T, VEC, 8>(a, x, y);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, bool VEC>
hipError_t launch_t(const SoftmaxArgs& a) {
  const T* x = static_cast<const T*>(a.x);
  T* y = static_cast<T*>(a.y);
  const dim3 block(kThreads);
  if (a.plan.kernel == OSX_KERNEL_SOFTMAX_WAVE || a.plan.kernel == OSX_KERNEL_SOFTMAX_ROW)
    return launch_resident<T, VEC>(a);
  float* part = static_cast<float*>(a.workspace);
  const dim3 grid((unsigned)a.plan.grid);
  const int64_t chunk = a.plan.block_m;
  hipLaunchKernelGGL((softmax_split_pass1<T, VEC>), grid, block, 0, a.stream, x, part, a.cols, a.plan.splits, chunk,
                     a.k, a.period);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((softmax_split_pass2<T, VEC>), grid, block, 0, a.stream, x, y, part, a.cols, a.plan.splits,
                     chunk, a.k, a.period);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_softmax_rows(const SoftmaxArgs& a) {
  const int E = a.dtype == OSX_BF16 ? Elem<uint16_t>::E : Elem<float>::E;
  const bool vec = (a.cols % E == 0) && ((reinterpret_cast<uintptr_t>(a.x) & 15) == 0) &&
                   ((reinterpret_cast<uintptr_t>(a.y) & 15) == 0);
  if (a.dtype == OSX_BF16) return vec ? launch_t<uint16_t, true>(a) : launch_t<uint16_t, false>(a);
  return vec ? launch_t<float, true>(a) : launch_t<float, false>(a);
}

}  // namespace osx
