// Attention forward for one query token per sequence (decode), bf16, gfx950.
//
// The method is the same online recurrence (page "softmax_attention", section
// 实现思路); the shape makes it a stream over K/V: every (batch, KV head) has
// only G query vectors, so the work is bound by reading K and V once from HBM.
//
//  * One workgroup per (batch, KV head, split of the keys).  All G query heads
//    of that KV head are packed into the 16 columns of a 16x16x32 MFMA tile, so
//    every K/V byte is read once and serves all G heads.
//  * Each of the 4 wavefronts walks its own 32-key blocks of the split with
//    16-byte loads, the next block loading while the current one is computed;
//    two workgroups per CU.  K feeds S^T = K Q^T directly from registers; V is written
//    to the wavefront's LDS slice transposed (keys permuted so each lane's 8
//    keys are one 16-byte read) and feeds O^T += V^T P^T.
//  * A head dimension d that is a multiple of 16 and not 64 or 128 runs in
//    the 64- or 128-wide kernel: padded columns of Q, K and V read as zeros
//    (their loads go to an offset past the buffer range), add nothing to the
//    scores and are never stored (page "softmax_attention", section 实现思路,
//    pads d up to the block width and masks the extra lanes).
//  * The 4 wavefront states are merged in LDS.  With one split that state is
//    final and the workgroup writes O = acc / l itself; otherwise it writes
//    one partial (m, l, acc) per split and a second kernel merges the splits
//    of each query head with the rule of page "Softmax 算子的实现与优化",
//    section Online Softmax, applied to partial states: m = max m_s,
//    l = sum l_s 2^(m_s - m), acc = sum acc_s 2^(m_s - m), then O = acc / l.
#include "common.hpp"
#include "launch.hpp"

namespace osx {
namespace {

constexpr int BN = kDecodeBlockN;  // 32 keys per wavefront step
constexpr int NCOL = 16;           // MFMA columns available for query heads
constexpr uint32_t kOffNowhere = 0x80000000u;  // a buffer offset past any head (heads are < 2^31 bytes)

template <int D>
struct DecTile {
  static constexpr int CH = D / 8;        // 16-byte chunks per row
  static constexpr int KC = D / 32;       // k-steps of the QK MFMA
  static constexpr int DT = D / 16;       // 16-row d tiles of the PV MFMA
  static constexpr int VT_BYTES = D * BN * 2;  // one wavefront's V^T slice
  static constexpr int VU = 8 * CH / kWaveSize;  // (4 keys x 16 bytes) V units per lane
};

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }
// K and V are read exactly once: non-temporal buffer loads (cache policy 2).
__device__ __forceinline__ u32x4 ld16_nt(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 2);
}

// V^T row (64 bytes = 4 chunks of 8 keys) swizzle: 16 consecutive rows hit 16
// distinct bank groups.
__device__ __forceinline__ int vt_swz(int d) { return (d >> 2) & 3; }

template <int D>
struct Regs {
  u32x4 k[2][DecTile<D>::KC];  // [sub-tile][k-step]
  u32x4 v[DecTile<D>::VU][4];  // [unit][key in quad]
};

// Keys past the split's end (and so past Sk) read as zeros through the buffer
// range; the score mask removes them (their weights are exactly 0).  Global
// rows are d elements long; columns d .. D-1 (padding) read as zeros.
template <int D>
__device__ __forceinline__ void load_regs(Regs<D>& R, __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr, int j0,
                                          int lane, int d) {
  using T = DecTile<D>;
  const int l16 = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int j = j0 + 16 * t + l16;
#pragma unroll
    for (int kc = 0; kc < T::KC; ++kc) {
      const int col = 32 * kc + 8 * grp;
      R.k[t][kc] = ld16_nt(kr, col < d ? (uint32_t)(j * d + col) * 2 : kOffNowhere);
    }
  }
#pragma unroll
  for (int r = 0; r < T::VU; ++r) {
    const int u = lane + kWaveSize * r;
    const int kq = u / T::CH, ch = u % T::CH;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      R.v[r][jj] = ld16_nt(vr, 8 * ch < d ? (uint32_t)((j0 + 4 * kq + jj) * d + 8 * ch) * 2 : kOffNowhere);
  }
}

// D: the kernel's (padded) head dimension, 64 or 128.  PAD: the true head
// dimension d_arg (a multiple of 16, at most D) is smaller; global rows, the
// output and the partial states are d_arg elements long.
template <int D, bool PAD>
__global__ __launch_bounds__(kAttnThreads, 2) void decode_bf16_kernel(
    const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg, const uint16_t* __restrict__ Vg,
    float* __restrict__ ws, uint16_t* __restrict__ Og, float* __restrict__ Lse, int Hq, int Hkv, int Sk, int d_arg,
    float c, int splits, int keys_per_split) {
  using T = DecTile<D>;
  const int d = PAD ? d_arg : D;
  // V^T slices during the stream; reused for the wavefront merge afterwards.
  constexpr int MERGE_BYTES = kAttnWaves * NCOL * (D + 2) * 4;
  constexpr int LDS_BYTES = kAttnWaves * T::VT_BYTES > MERGE_BYTES ? kAttnWaves * T::VT_BYTES : MERGE_BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, grp = lane >> 4;

  // Workgroups are dealt to the 8 XCDs round-robin in launch order; numbering
  // them so that each XCD streams a contiguous run of (b, KV head, split)
  // units measured 1% faster than the launch order.
  const int nwg = gridDim.x;
  const int wg = nwg % 8 == 0 ? (int)((blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8) : (int)blockIdx.x;
  const int split = wg % splits;
  const int bkv = wg / splits;
  const int b = bkv / Hkv, kvh = bkv % Hkv;
  const int G = Hq / Hkv;

  const int k_begin = split * keys_per_split;
  int k_end = k_begin + keys_per_split;
  if (k_end > Sk) k_end = Sk;

  // The resources end at the split's last key: loads past it return zeros
  // without touching memory, so the stream below can prefetch one block past
  // its end unconditionally (those keys are masked).
  const int k_lim = k_end > k_begin ? k_end : k_begin;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(Kg + (size_t)bkv * Sk * d, (uint32_t)k_lim * d * 2);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(Vg + (size_t)bkv * Sk * d, (uint32_t)k_lim * d * 2);

  // Q^T as the B operand: column l16 is query head kvh*G + l16 (zero past G).
  bf16x8 qop[T::KC];
  {
    const int hq = kvh * G + (l16 < G ? l16 : 0);
    const uint16_t* qp = Qg + (size_t)(b * Hq + hq) * d;
#pragma unroll
    for (int kc = 0; kc < T::KC; ++kc) {
      const int col = 32 * kc + 8 * grp;
      u32x4 x = col < d ? ld16(qp + col) : u32x4{0u, 0u, 0u, 0u};
      if (l16 >= G) x = u32x4{0u, 0u, 0u, 0u};
      qop[kc] = __builtin_bit_cast(bf16x8, x);
    }
  }

  unsigned char* vt = lds + wave * T::VT_BYTES;
  f32x4 acc[T::DT];
#pragma unroll
  for (int i = 0; i < T::DT; ++i) acc[i] = f32x4{};
  float m_run = kNegInf, l_run = 0.f;

  auto compute = [&](const Regs<D>& R, int j0) {
    // ---- S^T = K Q^T: two 16-key sub-tiles; lane (col l16, grp) holds keys 16t + 4grp + j ----
    f32x4 s[2] = {f32x4{}, f32x4{}};
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int kc = 0; kc < T::KC; ++kc)
        s[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, R.k[t][kc]), qop[kc], s[t], 0, 0,
                                                       0);
    if (j0 + BN > k_end) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (j0 + 16 * t + 4 * grp + j >= k_end) s[t][j] = kNegInf;
    }
    float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx * c);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2_fast(m_run - m_use);
    // P is rounded to bf16 once; the PV MFMA and the denominator use the same values.
    float p[8];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) p[4 * t + j] = exp2_fast(fmaf(s[t][j], c, -m_use));
    l_run *= alpha;
    const bf16x8 pb = pack_bf16x8_sum(p, l_run);
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < T::DT; ++i) acc[i] *= alpha;

    // ---- stage V^T: VT[d][pos(key)], pos = 8*((key>>2)&3) + 4*(key>>4) + (key&3) ----
#pragma unroll
    for (int r = 0; r < T::VU; ++r) {
      const int u = lane + kWaveSize * r;
      const int kq = u / T::CH, ch = u % T::CH;
      const int cc = kq & 3, half = kq >> 2;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        uint32_t lo, hi;
        if (e & 1) {
          lo = (R.v[r][0][w] >> 16) | (R.v[r][1][w] & 0xffff0000u);
          hi = (R.v[r][2][w] >> 16) | (R.v[r][3][w] & 0xffff0000u);
        } else {
          lo = (R.v[r][0][w] & 0xffffu) | (R.v[r][1][w] << 16);
          hi = (R.v[r][2][w] & 0xffffu) | (R.v[r][3][w] << 16);
        }
        const int d = 8 * ch + e;
        const u32x2 val = {lo, hi};
        *reinterpret_cast<u32x2*>(vt + d * (BN * 2) + ((cc ^ vt_swz(d)) << 4) + 8 * half) = val;
      }
    }
    OSX_DEBUG_SYNC_WAVE();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- O^T += V^T P^T: P^T lane (col, grp) element i is key 16(i/4) + 4grp + i%4 ----
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) {
      const int d = 16 * dt + l16;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(vt + d * (BN * 2) + ((grp ^ vt_swz(d)) << 4));
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, acc[dt], 0, 0, 0);
    }
    OSX_DEBUG_SYNC_WAVE();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // ---- stream this wavefront's blocks: k_begin + BN*(wave + 4i) ----
  // Two register sets: block i + 1 is loading while block i is computed.  The
  // loop runs over pairs of blocks with no exit in between (the last prefetch
  // of an even count lies past the split and reads zeros without touching
  // memory); an odd last block follows it.  sched_barrier keeps each prefetch
  // ahead of the compute, which would otherwise be hoisted above it and then
  // wait for the prefetch too.
  //
  // With the keys split, every workgroup starts its walk at a different block
  // of its split (block i of the walk is block (i + wg) mod nblk): the splits
  // start at addresses a power of two apart, and walks in step with each
  // other kept landing on the same memory channels (a batch of 8 sequences of
  // 32768 keys streamed at 5.1 TB/s in step, 6.7 TB/s rotated).  The order of
  // the blocks does not change the result beyond rounding, and it is fixed for
  // each workgroup.  Past its last block the walk reads past the split's range.
  constexpr int kStep = BN * kAttnWaves;
  const int j_first = k_begin + BN * wave;
  const int nblk = j_first < k_end ? (k_end - j_first + kStep - 1) / kStep : 0;
  const int rot = splits > 1 && nblk > 0 ? wg % nblk : 0;
  auto jb = [&](int i) { return i < nblk ? j_first + kStep * ((i + rot) % nblk) : k_lim + kStep; };
  Regs<D> ra, rb;
  load_regs<D>(ra, kr, vr, jb(0), lane, d);
  for (int pair = 0; pair < nblk / 2; ++pair) {
    load_regs<D>(rb, kr, vr, jb(2 * pair + 1), lane, d);
    __builtin_amdgcn_sched_barrier(0);
    compute(ra, jb(2 * pair));
    load_regs<D>(ra, kr, vr, jb(2 * pair + 2), lane, d);
    __builtin_amdgcn_sched_barrier(0);
    compute(rb, jb(2 * pair + 1));
  }
  if (nblk & 1) compute(ra, jb(nblk - 1));

  // ---- merge the 4 wavefront states in LDS ----
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  __syncthreads();  // every wavefront is done with its V^T slice
  float* ml = reinterpret_cast<float*>(lds);               // [wave][col][2]
  float* accl = ml + kAttnWaves * NCOL * 2;                // [wave][col][D]
  if (grp == 0) {
    ml[(wave * NCOL + l16) * 2] = m_run;
    ml[(wave * NCOL + l16) * 2 + 1] = l_run;
  }
#pragma unroll
  for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) accl[(wave * NCOL + l16) * D + 16 * dt + 4 * grp + j] = acc[dt][j];
  __syncthreads();
  OSX_DEBUG_SYNC_WG();

  float* ws_ml = ws;
  const size_t n_part = (size_t)gridDim.x * G;
  float* ws_acc = ws + 2 * n_part;
  const size_t part0 = (size_t)wg * G;
  for (int idx = tid; idx < G * d; idx += kAttnThreads) {
    const int col = idx / d, dd = idx % d;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, ml[(w * NCOL + col) * 2]);
    float lsum = 0.f, asum = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) {
        const float f = exp2_fast(ml[(w * NCOL + col) * 2] - M);
        lsum += ml[(w * NCOL + col) * 2 + 1] * f;
        asum += accl[(w * NCOL + col) * D + dd] * f;
      }
    }
    if (splits == 1) {
      // The workgroup saw every key: its merged state is final, O = acc / l.
      // (Every key split holds at least one key, so l > 0.)
      const size_t bh = (size_t)b * Hq + kvh * G + col;
      Og[bh * d + dd] = (uint16_t)(pack_bf16x2(asum / lsum, 0.f) & 0xffffu);
      // log sum_j exp(scale * s_j) = ln 2 * (M + log2 l), M in the log2 domain
      if (Lse && dd == 0) Lse[bh] = (M + log2f(lsum)) * kLn2;
    } else {
      ws_acc[(part0 + col) * d + dd] = asum;
      if (dd == 0) {
        ws_ml[(part0 + col) * 2] = M;
        ws_ml[(part0 + col) * 2 + 1] = lsum;
      }
    }
  }
}

// Merge the splits of one (batch, query head): with M = max_s m_s,
// O = sum_s acc_s 2^(m_s - M) / sum_s l_s 2^(m_s - M).  One thread per output
// column (the launch has d threads).  Every load is unconditional (indices
// past the last split are clamped to it and weighted 0), so the (m, l) pairs
// of all splits, staged in LDS, and each column's first kBatch accumulator
// values are in flight together: up to kBatch splits cost one memory round
// trip, where loads guarded per split went out one after another.  The launch
// takes the smallest kBatch that covers the splits (64 beyond that), so few
// splits issue few redundant loads.
template <int kBatch>
__global__ __launch_bounds__(128) void decode_combine_kernel(const float* __restrict__ ws, uint16_t* __restrict__ Og,
                                                             float* __restrict__ Lse, int Hq, int Hkv, int splits,
                                                             int n_wg, int D) {
  __shared__ __align__(16) float sm_m[kDecodeMaxSplits];
  __shared__ float sm_l[kDecodeMaxSplits];
  const int bh = blockIdx.x;
  const int b = bh / Hq, hq = bh % Hq;
  const int G = Hq / Hkv;
  const int kvh = hq / G, g = hq % G;
  const int bkv = b * Hkv + kvh;
  const size_t n_part = (size_t)n_wg * G;
  const float* ws_ml = ws;
  const float* ws_acc = ws + 2 * n_part;
  const int dd = threadIdx.x;
  auto part = [&](int sp) { return (size_t)(bkv * splits + sp) * G + g; };
  float as[kBatch];
#pragma unroll
  for (int i = 0; i < kBatch; ++i) as[i] = ws_acc[part(min(i, splits - 1)) * D + dd];
  const int padded = (splits + 3) & ~3;
  for (int sp = dd; sp < padded; sp += blockDim.x) {
    float2 ml = {kNegInf, 0.f};  // the padding: an empty split
    if (sp < splits) ml = *reinterpret_cast<const float2*>(ws_ml + part(sp) * 2);
    sm_m[sp] = ml.x;
    sm_l[sp] = ml.y;
  }
  __syncthreads();
  float M = kNegInf;
  for (int sp = 0; sp < padded; sp += 4) {
    const float4 m4 = *reinterpret_cast<const float4*>(sm_m + sp);
    M = fmaxf(M, fmaxf(fmaxf(m4.x, m4.y), fmaxf(m4.z, m4.w)));
  }
  float l = 0.f, a = 0.f;
  for (int s0 = 0; s0 < splits; s0 += kBatch) {
    if (s0 > 0) {
#pragma unroll
      for (int i = 0; i < kBatch; ++i) as[i] = ws_acc[part(min(s0 + i, splits - 1)) * D + dd];
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int sp = min(s0 + i, splits - 1);
      const float f = s0 + i < splits ? exp2_fast(sm_m[sp] - M) : 0.f;  // 0 for an empty split (m = -inf)
      l += sm_l[sp] * f;
      a += as[i] * f;
    }
  }
  const float o = a / l;
  // log sum_j exp(scale * s_j) = ln 2 * (M + log2 l), M in the log2 domain
  if (Lse && dd == 0) Lse[bh] = (M + log2f(l)) * kLn2;
  const uint32_t w = pack_bf16x2(o, 0.f);
  Og[(size_t)bh * D + dd] = (uint16_t)(w & 0xffffu);
}

template <int D, bool PAD>
hipError_t launch(const AttnArgs& a) {
  const int splits = a.plan.splits;
  int kps = (a.seq_k + splits - 1) / splits;
  kps = (kps + BN - 1) / BN * BN;
  float* ws = static_cast<float*>(a.workspace);
  hipLaunchKernelGGL((decode_bf16_kernel<D, PAD>), dim3((unsigned)a.plan.grid), dim3(kAttnThreads), 0, a.stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), ws, static_cast<uint16_t*>(a.o), a.lse, a.heads_q, a.heads_kv,
                     a.seq_k, a.head_dim, a.c, splits, kps);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  if (splits > kDecodeMaxSplits) return hipErrorInvalidValue;  // beyond the combine's LDS staging
  auto combine = splits <= 4    ? decode_combine_kernel<4>
                 : splits <= 8  ? decode_combine_kernel<8>
                 : splits <= 16 ? decode_combine_kernel<16>
                 : splits <= 32 ? decode_combine_kernel<32>
                                : decode_combine_kernel<64>;
  hipLaunchKernelGGL(combine, dim3((unsigned)(a.batch * a.heads_q)), dim3((unsigned)a.head_dim), 0, a.stream, ws,
                     static_cast<uint16_t*>(a.o), a.lse, a.heads_q, a.heads_kv, splits, (int)a.plan.grid, a.head_dim);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const AttnArgs& a) {
  if (a.head_dim % 16 != 0 || a.head_dim <= 0 || a.head_dim > 128) return hipErrorInvalidValue;
  if (a.head_dim == 64) return launch<64, false>(a);
  if (a.head_dim == 128) return launch<128, false>(a);
  return a.head_dim < 64 ? launch<64, true>(a) : launch<128, true>(a);
}

}  // namespace osx
