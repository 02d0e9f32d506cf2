// Single-pass attention forward, bf16 inputs, fp32 accumulation, gfx950.
//
// What is computed (page "softmax_attention", section 实现思路; page
// "从零开始写Qwen3（五-其一）使用Triton实现自注意力", sections 自注意力原理 and GQA):
// for every query row, keys are visited block by block; each block's scores
// s = q.k are scaled, masked (keys past the end and, when causal, keys after the
// query get -inf -- never a zero score), and folded into a running max m, a
// running denominator l and an unnormalised accumulator acc, both rescaled by
// 2^(m_old - m_new) when the max grows.  At the end O = acc / l.
//
// How it maps onto CDNA4:
//  * A workgroup is 4 wavefronts.  Each wavefront owns 32 query rows of one
//    query head; the workgroup's wavefronts share one KV head (GQA: query head h
//    reads KV head h / G), either 4 heads x 32 rows, 2 x 64 or 1 x 128.
//  * K and V blocks of 64 keys are staged through LDS (double buffered, one
//    barrier per block) with 16-byte global loads.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    a lane then holds 16 keys of ONE query, so the row max and row sum are
//    mostly lane-local (one cross-half exchange for the max per block) and the
//    rescale factor is a per-lane scalar.
//  * The output is also accumulated transposed, O^T += V^T P^T, with the
//    probabilities P (rounded to bf16) taken straight from the score registers
//    as the B operand.  V is written to LDS transposed, with its keys permuted
//    so each lane's 8 keys are one 16-byte read.
//  * exp is 2^(s*c - m) with c = scale*log2(e) folded into one FMA; m lives in
//    that log2 domain.
//  * Causal: key blocks wholly after the workgroup's last query are never
//    visited, only blocks that straddle the diagonal are masked, and tiles are
//    dispatched heaviest first.
#include "common.hpp"
#include "launch.hpp"

namespace osx {
namespace {

constexpr int BN = kBf16BlockN;  // 64 keys per block

template <int D>
struct Bf16Tile {
  static constexpr int CH = D / 8;               // 16-byte chunks per K row
  static constexpr int KC = D / 16;              // k-steps of the QK MFMA
  static constexpr int DT = D / 32;              // 32-row d tiles of the PV MFMA
  static constexpr int K_BYTES = BN * D * 2;     // one K block in LDS
  static constexpr int V_BYTES = D * BN * 2;     // one V^T block in LDS
  static constexpr int BUF = K_BYTES + V_BYTES;  // one stage
  static constexpr int KU = BN * CH / kAttnThreads;  // K 16-byte loads per thread
  static constexpr int VQ = 16 * CH;                 // (4 keys x 16 bytes) V units per block
};

// Chunk swizzle of a K row so 16 consecutive rows hit 16 distinct bank groups.
template <int CH>
__device__ __forceinline__ int k_swz(int row) {
  return CH % 16 == 0 ? (row & 15) : ((row >> 1) & 7);
}
// Chunk swizzle of a V^T row (128 bytes = 8 chunks).
__device__ __forceinline__ int v_swz(int d) { return (d >> 1) & 7; }

// LDS position of key `kq*4` inside a 64-key V^T row: bits 2 and 3 of the key
// swapped, so that the 8 keys one lane feeds to a PV MFMA are contiguous.
__device__ __forceinline__ int v_pos4(int kq) {
  return ((kq & 0xC) | ((kq & 1) << 1) | ((kq >> 1) & 1)) * 4;
}

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

template <int D>
__global__ __launch_bounds__(kAttnThreads, 2) void prefill_bf16_kernel(
    const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg, const uint16_t* __restrict__ Vg,
    uint16_t* __restrict__ Og, int Hq, int Hkv, int Sq, int Sk, int causal, float c, int hp, int n_hgroups,
    int n_qtiles, int units_per_tile) {
  using T = Bf16Tile<D>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * T::BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;

  // ---- work decomposition (consecutive workgroups share the q tile and walk
  // (batch, KV head); the 8 XCDs then each keep a fixed set of KV heads) ----
  int qt = blockIdx.x / units_per_tile;
  const int rem = blockIdx.x - qt * units_per_tile;
  if (causal) qt = n_qtiles - 1 - qt;  // heaviest tiles first
  const int G = Hq / Hkv;
  const int b = rem / (Hkv * n_hgroups);
  const int kvh = (rem / n_hgroups) % Hkv;
  const int hg = rem % n_hgroups;
  const int rs = kAttnWaves / hp;
  const int head = kvh * G + hg * hp + (wave % hp);
  const int wg_row0 = qt * kRowsPerWave * rs;
  const int row0 = wg_row0 + (wave / hp) * kRowsPerWave;
  const int q = row0 + l32;
  const int qc = q < Sq ? q : Sq - 1;

  const size_t q_base = (size_t)(b * Hq + head) * Sq * D;
  const size_t kv_base = (size_t)(b * Hkv + kvh) * Sk * D;
  const uint16_t* Kb = Kg + kv_base;
  const uint16_t* Vb = Vg + kv_base;

  // ---- Q as the B operand: lane (query l32, half hf) holds d = 16kc + 8hf .. +8 ----
  bf16x8 qreg[T::KC];
#pragma unroll
  for (int kc = 0; kc < T::KC; ++kc)
    qreg[kc] = __builtin_bit_cast(bf16x8, ld16(Qg + q_base + (size_t)qc * D + kc * 16 + hf * 8));

  // ---- key range ----
  int wg_row_end = wg_row0 + kRowsPerWave * rs;
  if (wg_row_end > Sq) wg_row_end = Sq;
  const bool cmask = causal && Sq > 1;
  const int n_keys = cmask ? (wg_row_end < Sk ? wg_row_end : Sk) : Sk;
  const int nblk = (n_keys + BN - 1) / BN;
  const int wave_row_last = row0 + kRowsPerWave - 1;

  u32x4 kst[T::KU];
  u32x4 vst[4];
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  auto load_block = [&](int j0) {
#pragma unroll
    for (int r = 0; r < T::KU; ++r) {
      const int u = tid + kAttnThreads * r;
      const int key = u / T::CH, ch = u % T::CH;
      const int j = j0 + key;
      kst[r] = j < Sk ? ld16(Kb + (size_t)j * D + ch * 8) : zero4;
    }
    if (tid < T::VQ) {
      const int kq = tid / T::CH, ch = tid % T::CH;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = j0 + kq * 4 + jj;
        vst[jj] = j < Sk ? ld16(Vb + (size_t)j * D + ch * 8) : zero4;
      }
    }
  };

  auto store_block = [&](int buf) {
    unsigned char* kl = lds + buf * T::BUF;
    unsigned char* vl = kl + T::K_BYTES;
#pragma unroll
    for (int r = 0; r < T::KU; ++r) {
      const int u = tid + kAttnThreads * r;
      const int key = u / T::CH, ch = u % T::CH;
      *reinterpret_cast<u32x4*>(kl + key * (D * 2) + ((ch ^ k_swz<T::CH>(key)) << 4)) = kst[r];
    }
    if (tid < T::VQ) {
      const int kq = tid / T::CH, ch = tid % T::CH;
      const int pos = v_pos4(kq);
      const int cc = pos >> 3, half = (pos >> 2) & 1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        uint32_t lo, hi;
        if (e & 1) {
          lo = (vst[0][w] >> 16) | (vst[1][w] & 0xffff0000u);
          hi = (vst[2][w] >> 16) | (vst[3][w] & 0xffff0000u);
        } else {
          lo = (vst[0][w] & 0xffffu) | (vst[1][w] << 16);
          hi = (vst[2][w] & 0xffffu) | (vst[3][w] << 16);
        }
        const int d = ch * 8 + e;
        const u32x2 val = {lo, hi};
        *reinterpret_cast<u32x2*>(vl + d * (BN * 2) + ((cc ^ v_swz(d)) << 4) + half * 8) = val;
      }
    }
  };

  f32x16 acc[T::DT];
#pragma unroll
  for (int i = 0; i < T::DT; ++i) acc[i] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;

  if (nblk > 0) {
    load_block(0);
    store_block(0);
  }
  __syncthreads();

  for (int jb = 0; jb < nblk; ++jb) {
    const int j0 = jb * BN;
    const bool has_next = jb + 1 < nblk;
    if (has_next) load_block(j0 + BN);

    // A wavefront whose rows all precede this block sees none of it.
    const bool active = !(cmask && j0 > wave_row_last);
    if (active) {
      const unsigned char* kl = lds + (jb & 1) * T::BUF;
      const unsigned char* vl = kl + T::K_BYTES;

      // ---- S^T = K Q^T : two 32-key sub-tiles ----
      f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int kc = 0; kc < T::KC; ++kc) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int key = 32 * t + l32;
          const int ch = 2 * kc + hf;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(kl + key * (D * 2) + ((ch ^ k_swz<T::CH>(key)) << 4));
          s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[kc], s[t], 0, 0, 0);
        }
      }

      // ---- mask: keys past the end, keys after the query (causal) ----
      const bool need_mask = (j0 + BN > Sk) || (cmask && j0 + BN - 1 > row0);
      if (need_mask) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kidx = j0 + 32 * t + 8 * (r >> 2) + 4 * hf + (r & 3);
            const bool ok = kidx < Sk && (!cmask || kidx <= q);
            s[t][r] = ok ? s[t][r] : kNegInf;
          }
      }

      // ---- online softmax (log2 domain) ----
      float mx = s[0][0];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx * c);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = exp2_fast(m_run - m_use);
      // P is rounded to bf16 once; the same rounded values feed the PV MFMA and
      // the denominator, so the weights of a row sum to exactly one.
      bf16x8 pb[2][2];
      float rsum = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          float p[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) p[i] = exp2_fast(fmaf(s[t][8 * u + i], c, -m_use));
          pb[t][u] = pack_bf16x8_sum(p, rsum);
        }
      l_run = l_run * alpha + rsum;
      m_run = m_new;
      if (__ballot(alpha != 1.0f)) {
#pragma unroll
        for (int i = 0; i < T::DT; ++i) acc[i] *= alpha;
      }

      // ---- O^T += V^T P^T ----
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int cc = 4 * t + 2 * u + hf;
#pragma unroll
          for (int dt = 0; dt < T::DT; ++dt) {
            const int d = 32 * dt + l32;
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(vl + d * (BN * 2) + ((cc ^ v_swz(d)) << 4));
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[t][u], acc[dt], 0, 0, 0);
          }
        }
    }

    if (has_next) store_block((jb + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, bf16 round-to-nearest-even ----
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
  if (q < Sq) {
    uint16_t* op = Og + q_base + (size_t)q * D;
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * dt + 8 * g + 4 * hf;
        const u32x2 w = {pack_bf16x2(acc[dt][4 * g] * inv, acc[dt][4 * g + 1] * inv),
                         pack_bf16x2(acc[dt][4 * g + 2] * inv, acc[dt][4 * g + 3] * inv)};
        *reinterpret_cast<u32x2*>(op + d0) = w;
      }
  }
}

template <int D>
hipError_t launch(const AttnArgs& a) {
  const int G = a.heads_q / a.heads_kv;
  const int hp = a.plan.heads_per_wg;
  const int n_hgroups = G / hp;
  const int rows_per_wg = a.plan.block_m;
  const int n_qtiles = (a.seq_q + rows_per_wg - 1) / rows_per_wg;
  const int units_per_tile = a.batch * a.heads_kv * n_hgroups;
  hipLaunchKernelGGL(prefill_bf16_kernel<D>, dim3((unsigned)a.plan.grid), dim3(kAttnThreads), 0, a.stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.heads_q, a.heads_kv, a.seq_q,
                     a.seq_k, a.causal, a.c, hp, n_hgroups, n_qtiles, units_per_tile);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const AttnArgs& a) {
  switch (a.head_dim) {
    case 64: return launch<64>(a);
    case 128: return launch<128>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace osx
