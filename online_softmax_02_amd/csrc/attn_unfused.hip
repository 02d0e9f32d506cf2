// Unfused attention, kept as a comparator for the single-pass kernels: the
// three-kernel pipeline of page "从零开始写Qwen3（五-其一）使用Triton实现自注意力"
// (sections 免转置矩阵乘法, softmax的triton实现 and 串起来):
//   1. S = scale * Q K^T into an [Sq, Sk] fp32 matrix per query head, with K
//      read row-major along d (no transposed copy of K);
//   2. the row softmax of S in place, with the causal mask column <= row
//      (the library's row softmax, run by the caller of these kernels);
//   3. O = P V.
// S is materialised in HBM and read back twice, which is the traffic the
// single-pass kernels avoid.  bf16 q, k, v and o; S and P stay fp32 as on the
// page; P is rounded to bf16 for the P V products, as in the fused path.
//
// Both products run on v_mfma_f32_32x32x16_bf16.  The scores are computed
// transposed, S^T = K Q^T, so both operands are rows read along d straight
// from memory and a lane's 16 results are 4 runs of 4 consecutive keys of one
// query (16-byte stores).  The output is O^T = V^T P^T: P rows (8 consecutive
// keys per lane) from memory, V staged row-major in LDS and read transposed.
#include "common.hpp"
#include "launch.hpp"

#include <type_traits>

namespace osx {
namespace {

constexpr int kThreads = 256;  // 4 wavefronts, 32 query rows each
constexpr int kRowsPerWg = 128;
constexpr int kKeyBlock = 64;  // keys per LDS block of V

typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

struct Head {
  int64_t q, kv;  // flat query head (b * Hq + h) and its KV head (b * Hkv + h / G)
  int qb;         // 128-query block within the head
};

// Workgroup -> (query head, query block).  Workgroups are dealt to the 8 XCDs
// round-robin in launch order; numbering them so that each XCD receives a
// contiguous run of (head, block) pairs keeps the workgroups of one XCD on the
// same few K or V heads (one L2 per XCD) and writing neighbouring rows.
__device__ __forceinline__ Head head_of(int Hq, int Hkv) {
  const int64_t gx = gridDim.x, total = gx * gridDim.y, L = blockIdx.y * gx + blockIdx.x;
  const int64_t id = total % 8 == 0 ? (L % 8) * (total / 8) + L / 8 : L;
  Head h;
  h.q = id / gx;
  h.qb = (int)(id - h.q * gx);
  const int64_t b = h.q / Hq;
  const int hq = (int)(h.q - b * Hq);
  h.kv = b * Hkv + hq / (Hq / Hkv);
  return h;
}

// ---- 1. S = scale * Q K^T -----------------------------------------------------
// Workgroup: 128 queries of one head, all keys; wavefront w: queries
// 32w .. 32w + 31 of them.  Lane (i = lane % 32, hf = lane / 32) holds the B
// operand Q[q0 + i][16 kc + 8 hf .. + 7] for every k-step kc, and per 32-key
// block loads the A operand K[j0 + i][16 kc + 8 hf .. + 7]; the next block's
// K is loaded while the current one is multiplied.  kGroupBlocks blocks (a
// 32 x 128 group of scores) accumulate in registers and then pass through the
// wavefront's own LDS tile, so that each store instruction writes two whole
// 512-byte row segments: long runs in each DRAM page rather than 128-byte
// pieces of 32 rows.  Rows past Sq or Sk load as zero (buffer range check);
// a store to a row past Sq or a column past Sk goes to an offset outside the
// head's score matrix and is dropped.
constexpr int kGroupBlocks = 4;
constexpr int kNonTemporal = 2;               // buffer-op cache policy: S is streamed once
constexpr uint32_t kOffNowhere = 0x80000000u;  // an offset past any head's scores (at most 2^31 bytes)

template <int D>
__global__ __launch_bounds__(kThreads) void scores_bf16_kernel(const uint16_t* __restrict__ Q,
                                                               const uint16_t* __restrict__ K, float* __restrict__ S,
                                                               int Hq, int Hkv, int Sq, int Sk, float scale) {
  constexpr int KC = D / 16;
  constexpr int NB = kGroupBlocks;
  constexpr int GK = 32 * NB;           // keys per group
  constexpr int kTileStride = GK + 4;   // floats per LDS tile row: 16-byte aligned, consecutive rows 4 banks apart
  __shared__ __attribute__((aligned(16))) float tiles[kThreads / 64][32 * kTileStride];
  const Head hd = head_of(Hq, Hkv);
  const int lane = threadIdx.x & 63, i = lane & 31, hf = lane >> 5;
  const int q0 = hd.qb * kRowsPerWg + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * 32;
  const int q = q0 + i;
  float* tile = tiles[threadIdx.x >> 6];
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(Q + hd.q * Sq * D, (uint32_t)Sq * D * 2);
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(K + hd.kv * Sk * D, (uint32_t)Sk * D * 2);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(S + hd.q * (int64_t)Sq * Sk, (uint32_t)((int64_t)Sq * Sk * 4));
  bf16x8 qf[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
    qf[kc] = __builtin_bit_cast(bf16x8, buf_ld16(qr, (uint32_t)(q * D + 16 * kc + 8 * hf) * 2));
  const int ngrp = (Sk + GK - 1) / GK;
  const bool vec = (Sk & 3) == 0;
  bf16x8 ka[KC], kb[KC];
  // Loads past Sk (the last group's tail and the prefetch after it) return zeros.
  auto load_k = [&](int jb, bf16x8 (&dst)[KC]) {
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
      dst[kc] = __builtin_bit_cast(bf16x8, buf_ld16(kr, (uint32_t)((jb * 32 + i) * D + 16 * kc + 8 * hf) * 2));
  };
  auto mma = [&](const bf16x8 (&kf)[KC]) {
    f32x16 acc = f32x16{};
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kc], qf[kc], acc, 0, 0, 0);
    return acc;
  };
  // Group g's tile to S.  Store s: the lanes of half hf write keys
  // g GK + 4 i .. + 3 of tile row 2 s + hf, one 16-byte store each when rows are
  // 16-byte aligned (Sk % 4 == 0), else four 4-byte stores.
  auto store_group = [&](int g, const float* t, auto aligned) {
    const int j = g * GK + 4 * i;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const int r = 2 * s + hf;
      const f32x4 v = *reinterpret_cast<const f32x4*>(t + r * kTileStride + 4 * i);
      const bool row_ok = q0 + r < Sq;
      const uint32_t base = (uint32_t)(q0 + r) * (uint32_t)Sk + (uint32_t)j;  // < 2^29 where it is used
      if constexpr (decltype(aligned)::value) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), sr,
                                               row_ok && j < Sk ? 4u * base : kOffNowhere, 0, kNonTemporal);
      } else {
        const u32x4 w = __builtin_bit_cast(u32x4, v);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          __builtin_amdgcn_raw_buffer_store_b32(w[e], sr, row_ok && j + e < Sk ? 4u * (base + e) : kOffNowhere, 0,
                                                kNonTemporal);
      }
    }
  };
  load_k(0, ka);
  for (int g = 0; g < ngrp; ++g) {
    // Two register sets for K: block jb + 1 loads while block jb is multiplied.
    f32x16 acc[NB];
#pragma unroll
    for (int b = 0; b < NB; b += 2) {
      const int jb = g * NB + b;
      load_k(jb + 1, kb);
      acc[b] = mma(ka);
      load_k(jb + 2, ka);
      acc[b + 1] = mma(kb);
    }
    // acc[b][4a + e] is S[q0 + i][g GK + 32 b + 8 a + 4 hf + e]: into tile row i.
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *reinterpret_cast<f32x4*>(tile + i * kTileStride + 32 * b + 8 * a + 4 * hf) =
            f32x4{acc[b][4 * a] * scale, acc[b][4 * a + 1] * scale, acc[b][4 * a + 2] * scale,
                  acc[b][4 * a + 3] * scale};
    if (vec)
      store_group(g, tile, std::true_type{});
    else
      store_group(g, tile, std::false_type{});
  }
}

// ---- 3. O = P V -----------------------------------------------------------------
// Workgroup: 128 queries of one head; wavefront w: queries 32w .. 32w + 31,
// all D output columns (D / 32 accumulator tiles of O^T).  Per 64-key block
// the workgroup stages V[64, D] and P[128 queries, 64 keys] in LDS (two
// buffers each: the next block is loaded into registers while the current one
// is multiplied).  P is read from memory in whole 256-byte row segments (each
// load instruction covers 4 rows), rounded to bf16 on the way into LDS, and
// read back as the B operand P[q][k0 + 16 u + 8 hf .. + 7] (u = 0..3).  The A
// operand, V[k0 + 16 u + 8 hf .. + 7][d], comes from two transposed LDS reads.
// Keys past Sk: their V rows load as zero, so whatever finite P the load
// returns there adds nothing.
template <int D>
struct PvTile {
  static constexpr int CH = D / 8;                // 16-byte chunks per V row
  static constexpr int DT = D / 32;               // 32-column tiles of O^T
  static constexpr int ROW = D * 2;               // bytes per V row in LDS
  static constexpr int BLOCK_BYTES = kKeyBlock * ROW;
  static constexpr int CHUNKS = kKeyBlock * CH / kThreads;  // 16-byte chunks per thread per block
  static constexpr int P_ROW = kKeyBlock * 2;     // bytes per bf16 P row in LDS (8 chunks of 8 keys)
  static constexpr int P_BYTES = kRowsPerWg * P_ROW;
  static constexpr int P_CHUNKS = kRowsPerWg * kKeyBlock / 4 / kThreads;  // fp32 16-byte chunks per thread
};

// P row swizzle: a B-operand read takes one 16-byte chunk from each of 32
// consecutive 128-byte rows; XOR-ing the chunk index with (row / 2) % 8 spreads
// each 16-row group over all the banks.
__device__ __forceinline__ int p_swizzle(int row) { return (row >> 1) & 7; }

// V row swizzle for the transposed reads: one ds_read_b64_tr_b16 serves 16 lanes
// from 4 consecutive rows, 32 bytes of each; XOR-ing the chunk index with a
// multiple of 4 puts those rows' segments in distinct bank groups.
template <int CH>
__device__ __forceinline__ int v_swizzle(int row) {
  return CH % 16 == 0 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
}

template <int D>
__global__ __launch_bounds__(kThreads) void pv_bf16_kernel(const float* __restrict__ P,
                                                           const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                                                           int Hq, int Hkv, int Sq, int Sk) {
  using T = PvTile<D>;
  __shared__ __attribute__((aligned(16))) unsigned char lds_v[2][T::BLOCK_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char lds_p[2][T::P_BYTES];
  const Head hd = head_of(Hq, Hkv);
  const int lane = threadIdx.x & 63, i = lane & 31, hf = lane >> 5;
  const int wave = threadIdx.x >> 6;
  const int q0 = hd.qb * kRowsPerWg;
  const int q = q0 + wave * 32 + i;
  const __amdgpu_buffer_rsrc_t pr = make_rsrc(P + hd.q * (int64_t)Sq * Sk, (uint32_t)((int64_t)Sq * Sk * 4));
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(V + hd.kv * Sk * D, (uint32_t)Sk * D * 2);
  const int nblk = (Sk + kKeyBlock - 1) / kKeyBlock;

  // V staging: thread t moves chunks t, t + 256, ... of the block.
  u32x4 vst[T::CHUNKS];
  auto load_v = [&](int kb) {
#pragma unroll
    for (int n = 0; n < T::CHUNKS; ++n) {
      const int c = threadIdx.x + kThreads * n, row = c / T::CH, ch = c % T::CH;
      vst[n] = buf_ld16(vr, (uint32_t)((kb * kKeyBlock + row) * D + ch * 8) * 2);
    }
  };
  auto store_v = [&](unsigned char* dst) {
#pragma unroll
    for (int n = 0; n < T::CHUNKS; ++n) {
      const int c = threadIdx.x + kThreads * n, row = c / T::CH, ch = c % T::CH;
      *reinterpret_cast<u32x4*>(dst + row * T::ROW + ((ch ^ v_swizzle<T::CH>(row)) << 4)) = vst[n];
    }
  };
  // P staging: fp32 chunk c = t + 256 n of the block is keys 4 (c % 16) .. + 3 of
  // query row c / 16 (so each load instruction reads 4 whole 256-byte row
  // segments); rounded to bf16, it fills half of LDS chunk (c % 16) / 2.
  f32x4 pst[T::P_CHUNKS];
  auto load_p = [&](int kb) {
#pragma unroll
    for (int n = 0; n < T::P_CHUNKS; ++n) {
      const int c = threadIdx.x + kThreads * n, row = c >> 4, ch = c & 15;
      pst[n] = buf_ld16f(pr, (uint32_t)(((int64_t)(q0 + row) * Sk + kb * kKeyBlock + 4 * ch) * 4));
    }
  };
  auto store_p = [&](unsigned char* dst) {
#pragma unroll
    for (int n = 0; n < T::P_CHUNKS; ++n) {
      const int c = threadIdx.x + kThreads * n, row = c >> 4, ch = c & 15;
      const u32x2 w = {pack_bf16x2(pst[n].x, pst[n].y), pack_bf16x2(pst[n].z, pst[n].w)};
      *reinterpret_cast<u32x2*>(dst + row * T::P_ROW + ((((ch >> 1) ^ p_swizzle(row)) << 4) | ((ch & 1) << 3))) = w;
    }
  };
  // B operand of step u: P[q][16 u + 8 hf .. + 7] of this wavefront's row i.
  auto p_frag = [&](const unsigned char* buf, int u) -> bf16x8 {
    const int row = wave * 32 + i;
    return *reinterpret_cast<const bf16x8*>(buf + row * T::P_ROW + (((2 * u + hf) ^ p_swizzle(row)) << 4));
  };
  // Transposed V read: in each 16-lane group, lane s addresses row base + s / 4,
  // columns c0 + 4 (s % 4) .. + 3; lane s then receives column c0 + s of those
  // 4 rows.  Groups 0 / 1 cover columns 0-15 / 16-31 of a tile for hf = 0,
  // groups 2 / 3 the same for hf = 1.
  const int grp = lane >> 4, s16 = lane & 15;
  const int v_col = 16 * (grp & 1) + 4 * (s16 & 3);
  const int v_row = 8 * (grp >> 1) + (s16 >> 2);
  auto v_frag = [&](const unsigned char* buf, int u, int dt) -> bf16x8 {
    const int col = 32 * dt + v_col;
    const int r0 = 16 * u + v_row, r1 = r0 + 4;
    const unsigned char* a0 = buf + r0 * T::ROW + (((col >> 3) ^ v_swizzle<T::CH>(r0)) << 4) + (col & 7) * 2;
    const unsigned char* a1 = buf + r1 * T::ROW + (((col >> 3) ^ v_swizzle<T::CH>(r1)) << 4) + (col & 7) * 2;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)a0);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)a1);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x16 acc[T::DT];
#pragma unroll
  for (int dt = 0; dt < T::DT; ++dt) acc[dt] = f32x16{};
  load_v(0);
  load_p(0);
  store_v(lds_v[0]);
  store_p(lds_p[0]);
  __syncthreads();
  for (int kb = 0; kb < nblk; ++kb) {
    const unsigned char* cur_v = lds_v[kb & 1];
    const unsigned char* cur_p = lds_p[kb & 1];
    const bool more = kb + 1 < nblk;
    if (more) {
      load_v(kb + 1);
      load_p(kb + 1);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bf16x8 pb = p_frag(cur_p, u);
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt)
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_frag(cur_v, u, dt), pb, acc[dt], 0, 0, 0);
    }
    if (more) {
      store_v(lds_v[(kb + 1) & 1]);
      store_p(lds_p[(kb + 1) & 1]);
    }
    __syncthreads();
  }
  if (q >= Sq) return;
  // acc[dt][4a + e] is O[q][32 dt + 8 a + 4 hf + e].
  uint16_t* orow = O + (hd.q * Sq + q) * (int64_t)D;
#pragma unroll
  for (int dt = 0; dt < T::DT; ++dt) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const u32x2 w = {pack_bf16x2(acc[dt][4 * a], acc[dt][4 * a + 1]),
                       pack_bf16x2(acc[dt][4 * a + 2], acc[dt][4 * a + 3])};
      *reinterpret_cast<u32x2*>(orow + 32 * dt + 8 * a + 4 * hf) = w;
    }
  }
}

template <int D>
hipError_t launch_scores(const AttnArgs& a, float* s, float scale) {
  const dim3 grid((unsigned)((a.seq_q + kRowsPerWg - 1) / kRowsPerWg), (unsigned)(a.batch * a.heads_q));
  hipLaunchKernelGGL((scores_bf16_kernel<D>), grid, dim3(kThreads), 0, a.stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k), s, a.heads_q, a.heads_kv,
                     a.seq_q, a.seq_k, scale);
  return hipGetLastError();
}

template <int D>
hipError_t launch_pv(const AttnArgs& a, const float* p) {
  const dim3 grid((unsigned)((a.seq_q + kRowsPerWg - 1) / kRowsPerWg), (unsigned)(a.batch * a.heads_q));
  hipLaunchKernelGGL((pv_bf16_kernel<D>), grid, dim3(kThreads), 0, a.stream, p, static_cast<const uint16_t*>(a.v),
                     static_cast<uint16_t*>(a.o), a.heads_q, a.heads_kv, a.seq_q, a.seq_k);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_unfused_scores(const AttnArgs& a, float* s, float scale) {
  return a.head_dim == 64 ? launch_scores<64>(a, s, scale) : launch_scores<128>(a, s, scale);
}

hipError_t launch_unfused_pv(const AttnArgs& a, const float* p) {
  return a.head_dim == 64 ? launch_pv<64>(a, p) : launch_pv<128>(a, p);
}

}  // namespace osx
