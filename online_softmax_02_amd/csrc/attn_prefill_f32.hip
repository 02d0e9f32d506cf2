// Single-pass attention forward, fp32 inputs and outputs, gfx950.
//
// Same method and mapping as the bf16 kernel (page "softmax_attention",
// section 实现思路: blocks of keys, running max / denominator / accumulator,
// rescale by 2^(m_old - m_new), ragged tail masked to -inf), in true fp32:
// v_mfma_f32_32x32x2_f32 computes S^T = K Q^T and O^T += V^T P^T with IEEE
// fp32 products and fp32 accumulation (no reduced-precision inputs; page
// "从零开始写Qwen3（五-其一）使用Triton实现自注意力" notes that a TF32 shortcut
// loses precision).
//
// Each MFMA lane supplies a single k value, so P^T comes straight from the
// score registers and V is read from a row-major (chunk-swizzled) LDS block.  The head
// dimension d (a multiple of 4, at most 128) is padded with zeros up to DP,
// a multiple of 32; padded columns are never stored.  Blocks are 32 keys.
//
// With NORM the kernel runs the normalised-output form of the recurrence
// (page "Puzzle 9: Simple FlashAttention", the recurrence under its scalar
// FlashAttention spec), applied per block of keys: the denominator d' of the
// keys seen so far is complete after each block's exponentials, the
// accumulator is multiplied by (d'_old / d'_new) 2^(m_old - m_new) and the
// block's weights by 1 / d'_new before the P V product, so the accumulator is
// the normalised output at every step and needs no final division.  Over one
// block this is the per-key recurrence composed across the block's keys.
//
// Few heads with long sequences (one 4096-row head gives 32 workgroups) would
// leave most of the 256 CUs idle, so the keys can be split: workgroup
// (tile, split) runs the recurrence over its slice of the keys and writes the
// partial state (m, l, acc) of each row; a combine kernel merges the slices
// with the rescaling rule of page "Softmax 算子的实现与优化", section Online
// Softmax: m = max m_s, l = sum l_s 2^(m_s - m), O = sum acc_s 2^(m_s - m) / l.
#include "common.hpp"
#include "launch.hpp"

namespace osx {
namespace {

constexpr int BN = kF32BlockN;  // 32 keys per block
constexpr uint32_t kOffNowhere = 0x80000000u;  // a buffer offset past any head (heads are < 2^31 bytes)

template <int DP>
struct F32Tile {
  static constexpr int CH = DP / 4;                 // 16-byte chunks per K or V row
  static constexpr int HALF = DP / 2;               // d values per MFMA half-wave
  static constexpr int DT = DP / 32;                // 32-row d tiles of the PV MFMA
  static constexpr int ROW = DP * 4;                // bytes per K or V row in LDS
  static constexpr int BLOCK_BYTES = BN * ROW;      // one K or V block
  static constexpr int DMA_PER_WAVE = BLOCK_BYTES / 1024 / kAttnWaves;  // 1-KiB loads per wavefront per block
};
static_assert(F32Tile<32>::DMA_PER_WAVE * 1024 * kAttnWaves == F32Tile<32>::BLOCK_BYTES, "whole 1-KiB loads");
static_assert(F32Tile<96>::DMA_PER_WAVE * 1024 * kAttnWaves == F32Tile<96>::BLOCK_BYTES, "whole 1-KiB loads");

// Chunk swizzles (16-byte chunk index XOR a function of the row).  K: the QK
// read takes one chunk of each of 32 consecutive rows.  V: the PV read takes 8
// consecutive chunks of row key (lanes 0-31) and of row key + 4 (lanes 32-63);
// flipping bit 3 of the chunk index on rows with bit 2 set puts the two halves
// in opposite halves of the banks (when a row holds a multiple of 16 chunks;
// otherwise V is not swizzled and that read is 2-way conflicted).  Both XORs
// stay inside the row.
template <int CH>
__device__ __forceinline__ int k_swz(int row) {
  return CH % 16 == 0 ? (row & 15) : ((row >> 1) & 7);
}
template <int CH>
__device__ __forceinline__ int v_swz(int row) {
  return CH % 16 == 0 ? ((row >> 2) & 1) << 3 : 0;
}

// s_waitcnt with vmcnt = N (bits 3:0 and 15:14), expcnt and lgkmcnt not waited on.
template <int N>
__device__ __forceinline__ void wait_vmcnt_le() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
// Wavefront priority 0..3 (an immediate operand, hence the branches; p is uniform).
__device__ __forceinline__ void set_prio(int p) {
  if (p >= 3) __builtin_amdgcn_s_setprio(3);
  else if (p == 2) __builtin_amdgcn_s_setprio(2);
  else if (p == 1) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

template <int DP, bool NORM>
__global__ __launch_bounds__(kAttnThreads, 2) void prefill_f32_kernel(
    const float* __restrict__ Qg, const float* __restrict__ Kg, const float* __restrict__ Vg, float* __restrict__ Og,
    float* __restrict__ Lse, int Hq, int Hkv, int Sq, int Sk, int d, int causal, float c, int hp, int n_hgroups,
    int n_qtiles, int units_per_tile, int splits, int keys_per_split, float* __restrict__ ws_ml,
    float* __restrict__ ws_acc) {
  using T = F32Tile<DP>;
  // Two K blocks, then two V blocks.
  __shared__ __attribute__((aligned(16))) unsigned char lds[4 * T::BLOCK_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps per-wave values in SGPRs
  const int l32 = lane & 31, hf = lane >> 5;

  const int split = blockIdx.x % splits;
  const int tile_id = blockIdx.x / splits;
  int qt = tile_id / units_per_tile;
  const int rem = tile_id - qt * units_per_tile;
  if (causal) qt = n_qtiles - 1 - qt;
  const int G = Hq / Hkv;
  const int b = rem / (Hkv * n_hgroups);
  const int kvh = (rem / n_hgroups) % Hkv;
  const int hg = rem % n_hgroups;
  const int rs = kAttnWaves / hp;
  const int head = kvh * G + hg * hp + (wave % hp);
  const int wg_row0 = qt * kRowsPerWave * rs;
  const int row0 = wg_row0 + (wave / hp) * kRowsPerWave;
  const int q = row0 + l32;

  const size_t q_base = (size_t)(b * Hq + head) * Sq * d;
  const size_t kv_base = (size_t)(b * Hkv + kvh) * Sk * d;
  // Rows past Sq / Sk read as zeros; so do the padded columns (d <= col < DP),
  // whose loads are sent to an offset past the buffer.  (A select on the
  // loaded value instead would make each load wait for its data where it is
  // issued, exposing the next block's load latency in every block.)
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(Qg + q_base, (uint32_t)Sq * d * 4);
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(Kg + kv_base, (uint32_t)Sk * d * 4);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(Vg + kv_base, (uint32_t)Sk * d * 4);

  // Q as the B operand: lane (query l32, half hf) holds d = hf*DP/2 + j.
  // Issued after the first K block (see the prologue), in the order the
  // score products consume it.
  float qv[T::HALF];
  auto load_q = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < T::HALF; j += 4) {
      const int col = hf * T::HALF + j;
      const f32x4 x = buf_ld16f(qr, col < d ? (uint32_t)(q * d + col) * 4 : kOffNowhere);
      qv[j] = x.x;
      qv[j + 1] = x.y;
      qv[j + 2] = x.z;
      qv[j + 3] = x.w;
    }
  };

  int wg_row_end = wg_row0 + kRowsPerWave * rs;
  if (wg_row_end > Sq) wg_row_end = Sq;
  const bool cmask = causal && Sq > 1;
  int n_keys = cmask ? (wg_row_end < Sk ? wg_row_end : Sk) : Sk;
  // This workgroup's slice of the keys: blocks [jb0, nblk).
  const int k_begin = split * keys_per_split;
  if (n_keys > k_begin + keys_per_split) n_keys = k_begin + keys_per_split;
  const int jb0 = k_begin / BN;
  const int nblk = (n_keys + BN - 1) / BN;
  const size_t row_id = (size_t)(b * Hq + head) * Sq + q;  // partial-state row (split mode)

  // K and V pass through separate double-buffered LDS blocks, K one block
  // further ahead than V: while block j's weights are formed and multiplied
  // by V(j), the scores of block j + 1 are already computed (from K(j + 1)),
  // so the softmax arithmetic of one block runs under the matrix products of
  // the next.  Blocks are copied with direct-to-LDS buffer loads: a 16-byte
  // load of lane i lands at M0 + 16 i, so each lane fetches the global chunk
  // that belongs in its swizzled slot; padded columns (d <= col < DP) and rows
  // past Sk read as zeros.
  unsigned char* const lds_k = lds;
  unsigned char* const lds_v = lds + 2 * T::BLOCK_BYTES;
  // Lane offset of load n of this wavefront within a block (row-major rows of
  // d floats in global memory), or an offset past the buffer for a padded column.
  auto dma_voff = [&](int n, bool is_v) -> uint32_t {
    const int pos = (n * kAttnWaves + wave) * 1024 + 16 * lane;  // byte in the block
    const int row = pos / T::ROW, slot = (pos % T::ROW) >> 4;
    const int ch = slot ^ (is_v ? v_swz<T::CH>(row) : k_swz<T::CH>(row));
    return 4 * ch < d ? (uint32_t)(row * d + 4 * ch) * 4 : kOffNowhere;
  };
  // The block offset is added to the lane's VGPR offset, which the hardware
  // checks against the range (the scalar offset, which it does not check,
  // stays 0): rows of the last block past Sk read as zeros without touching
  // memory, and an offset past the range stays past it.
  auto dma = [&](__amdgpu_buffer_rsrc_t rsrc, bool is_v, unsigned char* dst, int j0) __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < T::DMA_PER_WAVE; ++n) {
      const int inst = n * kAttnWaves + wave;  // uniform
      const uint32_t voff = dma_voff(n, is_v) + (uint32_t)j0 * (uint32_t)(d * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(dst + inst * 1024),
                                               16, voff, 0, 0, 0);
    }
  };
  auto load_k = [&](int j0, int buf) { dma(kr, false, lds_k + buf * T::BLOCK_BYTES, j0); };
  auto load_v = [&](int j0, int buf) { dma(vr, true, lds_v + buf * T::BLOCK_BYTES, j0); };

  f32x16 acc[T::DT];
#pragma unroll
  for (int i = 0; i < T::DT; ++i) acc[i] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;

  if (jb0 >= nblk) {
    // Causal slice entirely after this tile's rows: an empty partial state.
    if (q < Sq) {
      if (hf == 0) {
        ws_ml[(row_id * splits + split) * 2] = kNegInf;
        ws_ml[(row_id * splits + split) * 2 + 1] = 0.f;
      }
      float* pa = ws_acc + (row_id * splits + split) * d;
      for (int c0 = 4 * hf; c0 < d; c0 += 8) *reinterpret_cast<f32x4*>(pa + c0) = f32x4{};
    }
    return;
  }

  // S^T = K Q^T over the padded head dimension, from K block buffer `buf`.
  auto qk = [&](int buf) {
    const unsigned char* kl = lds_k + buf * T::BLOCK_BYTES;
    f32x16 s = f32x16{};
#pragma unroll
    for (int j = 0; j < T::HALF; j += 4) {
      const int ch = (hf * T::HALF + j) >> 2;
      const f32x4 a = *reinterpret_cast<const f32x4*>(kl + l32 * (DP * 4) + ((ch ^ k_swz<T::CH>(l32)) << 4));
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, qv[j], s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, qv[j + 1], s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, qv[j + 2], s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, qv[j + 3], s, 0, 0, 0);
    }
    return s;
  };

  // The last key this lane's row may see: keys past Sk and (causal) after the
  // row are masked to -inf.  The mask is applied to every block without a
  // branch, so that a block's softmax and the next block's QK products form
  // one straight-line region the compiler can interleave.
  const int key_last = cmask ? (q < Sk - 1 ? q : Sk - 1) : Sk - 1;

  // Softmax of block j0's scores s (in place: s becomes the weights P) and the
  // update of m and l; returns the factor the accumulator must be multiplied
  // by (applied by rescale(), outside the straight-line region).
  auto softmax = [&](f32x16& s, int j0) -> float {
    const int rel = key_last - j0 - 4 * hf;  // key j0 + 8 (r / 4) + 4 hf + r % 4 is visible iff 8 (r / 4) + r % 4 <= rel
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 8 * (r >> 2) + (r & 3) <= rel ? s[r] : kNegInf;
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = pair_max(mx);
    const float m_new = fmaxf(m_run, mx * c);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2_fast(m_run - m_use);
    float rsum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = exp2_fast(fmaf(s[r], c, -m_use));
      s[r] = p;
      rsum += p;
    }
    if constexpr (NORM) {
      // d'_new = d'_old 2^(m_old - m_new) + the block's sum over both halves
      // of the row (l_run holds the whole row's d' in both halves).  A row
      // with nothing visible yet keeps d' = 0 and an all-zero accumulator.
      const float d_new = l_run * alpha + pair_sum(rsum);
      const float inv_d = d_new > 0.f ? 1.0f / d_new : 0.f;
      const float beta = l_run * alpha * inv_d;  // (d'_old / d'_new) 2^(m_old - m_new)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] *= inv_d;
      l_run = d_new;
      m_run = m_new;
      return beta;
    } else {
      l_run = l_run * alpha + rsum;
      m_run = m_new;
      return alpha;
    }
  };
  // acc *= f; without NORM only when some row's max moved (f != 1), which is
  // rare once the first blocks are seen.
  auto rescale = [&](float f) {
    if (NORM || __ballot(f != 1.0f)) {
#pragma unroll
      for (int i = 0; i < T::DT; ++i) acc[i] *= f;
    }
  };

  // O^T += V^T P^T from V block buffer `buf`: lane (d, hf) reads V[key(r, hf)][d],
  // stored in chunk (d / 4) ^ v_swz(key) of its row.
  auto pv = [&](const f32x16& s, int buf) {
    const float* vl = reinterpret_cast<const float*>(lds_v + buf * T::BLOCK_BYTES);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 8 * (r >> 2) + 4 * hf + (r & 3);
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt) {
        const int col = 32 * dt + l32;
        const float a = vl[key * DP + ((((col >> 2) ^ v_swz<T::CH>(key)) << 2) | (col & 3))];
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[r], acc[dt], 0, 0, 0);
      }
    }
  };

  // Prologue: K of the first block, this wavefront's Q rows, V of the first
  // block and K of the second.  Every slice that is not empty starts with a
  // visible key for every row.  All workgroups start at once and their first
  // loads queue behind each other, so the first score products do not wait
  // for all of them: each wavefront waits for its share of K(jb0) only (loads
  // complete in issue order), the barrier makes the whole block visible, and
  // the products then take the Q registers as they arrive (the compiler waits
  // for each on its first use).  The barrier carries no memory fence, which
  // would wait for every outstanding load.
  load_k(jb0 * BN, jb0 & 1);
  load_q();
  load_v(jb0 * BN, jb0 & 1);
  if (jb0 + 1 < nblk) load_k((jb0 + 1) * BN, (jb0 + 1) & 1);
  wait_vmcnt_le<T::HALF / 4 + T::DMA_PER_WAVE>();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  f32x16 s_cur = qk(jb0 & 1);
  // The first iteration reads V(jb0) and reloads this K buffer (with block
  // jb0 + 2): every load has landed and every wavefront has read K(jb0).
  wait_vmem();
  __syncthreads();
  OSX_DEBUG_SYNC_WG();

  for (int jb = jb0; jb < nblk; ++jb) {
    const int j0 = jb * BN;
    // Two workgroups share each CU and, left alone, the older one's
    // wavefronts win the issue arbitration: it finishes long before the
    // other, which then runs its remaining blocks with the matrix cores half
    // idle.  Priority falls with progress (3 for the first quarter of the
    // slice, down to 0 for the last), so the workgroup that is behind is served
    // first and the two finish together.
    set_prio(3 - (4 * (jb - jb0)) / (nblk - jb0));
    const bool has1 = jb + 1 < nblk, has2 = jb + 2 < nblk;
    // K(jb + 2) replaces K(jb) and V(jb + 1) replaces V(jb - 1): both were
    // last read before the previous barrier.
    if (has2) load_k(j0 + 2 * BN, jb & 1);
    if (has1) load_v(j0 + BN, (jb + 1) & 1);
    // Causal: a block whose first key comes after this wavefront's last row
    // is skipped (it would only add zero weights); the loads above still run,
    // the other wavefronts need them.
    const bool cur_live = !cmask || j0 <= row0 + kRowsPerWave - 1;
    const bool next_live = has1 && (!cmask || j0 + BN <= row0 + kRowsPerWave - 1);
    f32x16 s_next = f32x16{};
    if (cur_live) {
      float f;
      if (next_live) {
        s_next = qk((jb + 1) & 1);
        f = softmax(s_cur, j0);
      } else {
        f = softmax(s_cur, j0);
      }
      rescale(f);
      pv(s_cur, jb & 1);
    }
    wait_vmem();
    __syncthreads();
    OSX_DEBUG_SYNC_WG();  // nblk is the same for every wavefront of the workgroup
    s_cur = s_next;
  }

  const float l_tot = NORM ? l_run : l_run + __shfl_xor(l_run, 32, 64);
  if (q < Sq) {
    if (splits == 1) {
      // log sum_j exp(scale * s_j) = ln 2 * (m + log2 l), m in the log2 domain
      if (Lse && hf == 0) Lse[row_id] = (m_run + log2f(l_tot)) * kLn2;
      const float inv = NORM ? 1.0f : 1.0f / l_tot;
      float* op = Og + q_base + (size_t)q * d;
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * dt + 8 * g + 4 * hf;
          if (d0 < d) {
            const f32x4 w = {acc[dt][4 * g] * inv, acc[dt][4 * g + 1] * inv, acc[dt][4 * g + 2] * inv,
                             acc[dt][4 * g + 3] * inv};
            *reinterpret_cast<f32x4*>(op + d0) = w;
          }
        }
    } else {
      // partial state of this slice: m (log2 domain), l and acc (unnormalised,
      // or with NORM the slice's normalised output)
      if (hf == 0) {
        ws_ml[(row_id * splits + split) * 2] = m_run;
        ws_ml[(row_id * splits + split) * 2 + 1] = l_tot;
      }
      float* pa = ws_acc + (row_id * splits + split) * d;
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * dt + 8 * g + 4 * hf;
          if (d0 < d)
            *reinterpret_cast<f32x4*>(pa + d0) = f32x4{acc[dt][4 * g], acc[dt][4 * g + 1], acc[dt][4 * g + 2],
                                                       acc[dt][4 * g + 3]};
        }
    }
  }
}

// Merge the key slices of each query row: one wavefront per row.  Lane s
// (< splits <= 64) loads slice s's (m, l); the wavefront max and the weights
// 2^(m_s - m) are shared by shuffles; lane c owns output columns c and c + 64.
// With NORM the slices hold normalised outputs O'_s, weighted by
// l_s 2^(m_s - m): O = sum_s l_s 2^(m_s - m) O'_s / l.
template <bool NORM>
__global__ __launch_bounds__(256) void combine_f32_kernel(const float* __restrict__ ws_ml,
                                                          const float* __restrict__ ws_acc, float* __restrict__ Og,
                                                          float* __restrict__ Lse, int64_t rows, int splits, int d) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float* ml = ws_ml + row * splits * 2;
  const float m_s = lane < splits ? ml[2 * lane] : kNegInf;
  const float l_s = lane < splits ? ml[2 * lane + 1] : 0.f;
  const float M = wave_max(m_s);
  const float e_s = lane < splits ? exp2_fast(m_s - M) : 0.f;  // 0 for an empty slice
  const float L = wave_sum(l_s * e_s);
  const float w_s = NORM ? l_s * e_s : e_s;
  const float* pa = ws_acc + row * splits * d;
  float a0 = 0.f, a1 = 0.f;
  // Eight slices' partial outputs are loaded before any is used, so their load
  // latencies overlap instead of adding up.
  constexpr int kBatch = 8;
  for (int s0 = 0; s0 < splits; s0 += kBatch) {
    float x0[kBatch], x1[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int s = s0 + b;
      x0[b] = s < splits && lane < d ? pa[(int64_t)s * d + lane] : 0.f;
      x1[b] = s < splits && lane + 64 < d ? pa[(int64_t)s * d + lane + 64] : 0.f;
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const float w = __shfl(w_s, (s0 + b) & 63, 64);  // 0 past the last slice (w_s is 0 there)
      a0 += x0[b] * w;
      a1 += x1[b] * w;
    }
  }
  const float inv = 1.0f / L;
  if (Lse && lane == 0) Lse[row] = (M + log2f(L)) * kLn2;
  if (lane < d) Og[row * d + lane] = a0 * inv;
  if (lane + 64 < d) Og[row * d + lane + 64] = a1 * inv;
}

template <int DP>
hipError_t launch(const AttnArgs& a) {
  const int G = a.heads_q / a.heads_kv;
  const int hp = a.plan.heads_per_wg;
  const int n_hgroups = G / hp;
  const int rows_per_wg = a.plan.block_m;
  const int n_qtiles = (a.seq_q + rows_per_wg - 1) / rows_per_wg;
  const int units_per_tile = a.batch * a.heads_kv * n_hgroups;
  const int splits = a.plan.splits;
  const int kps = splits == 1 ? a.seq_k : ((a.seq_k + splits - 1) / splits + BN - 1) / BN * BN;
  const int64_t rows = (int64_t)a.batch * a.heads_q * a.seq_q;
  float* ws_ml = static_cast<float*>(a.workspace);
  // The slice accumulators start at the first 16-byte boundary after the (m, l) pairs.
  float* ws_acc = splits == 1 ? nullptr : ws_ml + (rows * splits * 2 + 3) / 4 * 4;
  auto kernel = a.normalised ? prefill_f32_kernel<DP, true> : prefill_f32_kernel<DP, false>;
  hipLaunchKernelGGL(kernel, dim3((unsigned)a.plan.grid), dim3(kAttnThreads), 0, a.stream,
                     static_cast<const float*>(a.q), static_cast<const float*>(a.k), static_cast<const float*>(a.v),
                     static_cast<float*>(a.o), a.lse, a.heads_q, a.heads_kv, a.seq_q, a.seq_k, a.head_dim, a.causal,
                     a.c, hp, n_hgroups, n_qtiles, units_per_tile, splits, kps, ws_ml, ws_acc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  auto combine = a.normalised ? combine_f32_kernel<true> : combine_f32_kernel<false>;
  hipLaunchKernelGGL(combine, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, a.stream, ws_ml, ws_acc,
                     static_cast<float*>(a.o), a.lse, rows, splits, a.head_dim);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_f32(const AttnArgs& a) {
  if (a.head_dim <= 32) return launch<32>(a);
  if (a.head_dim <= 64) return launch<64>(a);
  if (a.head_dim <= 96) return launch<96>(a);
  if (a.head_dim <= 128) return launch<128>(a);
  return hipErrorInvalidValue;
}

}  // namespace osx
