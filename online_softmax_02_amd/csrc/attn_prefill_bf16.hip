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
//  * K and V blocks of 64 keys are staged through LDS (two buffers each, one
//    barrier per block) with 16-byte direct-to-LDS buffer loads (no register
//    staging); rows past the end read as 0.
//    K runs one block ahead: the QK MFMAs of block j+1 are issued while the
//    exponentials of block j run on the VALU, then block j's PV MFMAs follow.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    a lane then holds 16 scores of ONE query, so the row max and row sum are
//    lane-local (plus one cross-half exchange for the max per block) and the
//    rescale factor is a per-lane scalar.
//  * The output is also accumulated transposed, O^T += V^T P^T, with P (rounded
//    to bf16 once) taken straight from the score registers as the B operand.
//    V stays row-major in LDS; ds_read_b64_tr_b16 delivers it transposed.
//  * exp is 2^(s*c - m) with c = scale*log2(e) folded into one FMA; m lives in
//    that log2 domain.  The reference m used in the exponent is moved (and acc,
//    l rescaled by 2^(m_old - m_new)) only when a row's running max exceeds it
//    by more than 2^8; the result is identical in exact arithmetic (the page's
//    shift invariance) and the exponentials stay <= 2^8.
//  * Causal: key blocks wholly after the workgroup's last query are never
//    visited; blocks that need no mask (the prefix before the diagonal) run a
//    mask-free copy of the loop body; tiles are dispatched heaviest first.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace osx {
namespace {

constexpr int BN = kBf16BlockN;  // 64 keys per block
constexpr float kRescaleSlack = 8.0f;  // log2 units a row max may exceed the reference before a rescale

typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <int D>
struct Bf16Tile {
  static constexpr int CH = D / 8;               // 16-byte chunks per K/V row
  static constexpr int KC = D / 16;              // k-steps of the QK MFMA
  static constexpr int DT = D / 32;              // 32-row d tiles of the PV MFMA
  static constexpr int ROW = D * 2;              // bytes per K/V row in LDS
  static constexpr int K_BYTES = BN * ROW;       // one K block in LDS
  static constexpr int V_BYTES = BN * ROW;       // one V block in LDS
  static constexpr int KU = BN * CH / kAttnThreads;  // 16-byte loads per thread, K (and V)
};

// K row chunk swizzle: the 16 rows one MFMA read touches land in 16 distinct
// 16-byte bank groups.
template <int CH>
__device__ __forceinline__ int k_swz(int row) {
  return CH % 16 == 0 ? (row & 15) : ((row >> 1) & 7);
}
// V row swizzle: a ds_read_b64_tr_b16 serves 32 lanes from 4 consecutive rows,
// 64 bytes (4 chunks) of each; XOR-ing the chunk index with a multiple of 4
// puts those 4 row segments in 4 distinct 64-byte bank groups (for 128-byte
// rows, rows r and r+1 already sit in different bank halves).
template <int CH>
__device__ __forceinline__ int v_swz(int row) {
  return CH % 16 == 0 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
}

template <int D>
__global__ __launch_bounds__(kAttnThreads, 2) void prefill_bf16_kernel(
    const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg, const uint16_t* __restrict__ Vg,
    uint16_t* __restrict__ Og, int Hq, int Hkv, int Sq, int Sk, int causal, float c, int hp, int n_hgroups,
    int n_qtiles, int units_per_tile) {
  using T = Bf16Tile<D>;
  // Four separate LDS objects (two K, two V buffers): the compiler can then
  // tell a read of one buffer from a DMA into another and does not wait for
  // the DMA before the read.
  __shared__ __attribute__((aligned(16))) unsigned char lds_k0[T::K_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char lds_k1[T::K_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char lds_v0[T::V_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char lds_v1[T::V_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps per-wave values in SGPRs
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

  const size_t q_base = (size_t)(b * Hq + head) * Sq * D;
  const size_t kv_base = (size_t)(b * Hkv + kvh) * Sk * D;
  // Rows past Sq (queries) or Sk (keys) read as zeros.
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(Qg + q_base, (uint32_t)Sq * D * 2);
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(Kg + kv_base, (uint32_t)Sk * D * 2);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(Vg + kv_base, (uint32_t)Sk * D * 2);

  // ---- Q as the B operand: lane (query l32, half hf) holds d = 16kc + 8hf .. +8 ----
  bf16x8 qreg[T::KC];
#pragma unroll
  for (int kc = 0; kc < T::KC; ++kc)
    qreg[kc] = __builtin_bit_cast(bf16x8, buf_ld16(qr, (uint32_t)(q * D + kc * 16 + hf * 8) * 2));

  // ---- key range ----
  int wg_row_end = wg_row0 + kRowsPerWave * rs;
  if (wg_row_end > Sq) wg_row_end = Sq;
  const bool cmask = causal && Sq > 1;
  const int n_keys = cmask ? (wg_row_end < Sk ? wg_row_end : Sk) : Sk;
  const int nblk = (n_keys + BN - 1) / BN;
  // Blocks [0, n_full) need no mask for any row of the workgroup.
  int n_full = Sk / BN;
  if (cmask) {
    const int diag = (wg_row0 + 1) / BN;  // blocks with j0 + BN - 1 <= wg_row0
    n_full = n_full < diag ? n_full : diag;
  }
  if (n_full > nblk) n_full = nblk;
  const int wave_row_last = row0 + kRowsPerWave - 1;

  // ---- global -> LDS staging with buffer_load_dwordx4 ... lds ----
  // LDS holds two K buffers and two V buffers.  K runs one block ahead of V:
  // while block jb's softmax and PV run, the QK of block jb+1 is issued.
  // A direct-to-LDS load writes lane i's 16 bytes at M0 + 16 i, so each lane
  // fetches the global chunk that belongs in its (swizzled) LDS slot.
  // One wavefront instruction fills LDS_ROWS rows; the block needs LDS_STEPS
  // such instructions, spread over the 4 wavefronts.
  constexpr int LDS_ROWS = 64 / T::CH;                 // rows per 1 KiB instruction
  constexpr int LDS_STEPS = BN / LDS_ROWS / kAttnWaves;  // instructions per wavefront per block
  const int dma_row = lane / T::CH, dma_chunk = lane % T::CH;
  // The swizzle of a row depends only on its position within 16 rows, which
  // the instruction index does not change: the lane's byte offset is fixed and
  // the block and instruction offsets go into the scalar soffset.
  const int dma_row0 = wave * LDS_ROWS + dma_row;
  const int k_voff = (dma_row0 * D + ((dma_chunk ^ k_swz<T::CH>(dma_row0)) << 3)) * 2;
  const int v_voff = (dma_row0 * D + ((dma_chunk ^ v_swz<T::CH>(dma_row0)) << 3)) * 2;
  static_assert((kAttnWaves * LDS_ROWS) % 16 == 0, "row swizzle must repeat every instruction step");
  auto dma_block = [&](__amdgpu_buffer_rsrc_t rsrc, int j0, unsigned char* dst, bool is_v) {
#pragma unroll
    for (int r = 0; r < LDS_STEPS; ++r) {
      const int inst = r * kAttnWaves + wave;  // uniform
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(dst + inst * 1024),
                                               16, is_v ? v_voff : k_voff,
                                               (j0 + r * kAttnWaves * LDS_ROWS) * D * 2, 0, 0);
    }
  };

  // ---- per-lane constants of the transposed V read (ds_read_b64_tr_b16) ----
  // In each 16-lane group, source lane s points at row base + s/4, columns
  // c0 + 4(s%4) .. +4; lane i then receives column c0 + i of those 4 rows.
  // Lane (d = l32, hf) needs keys 16u + 4hf + 0..3 and 16u + 8 + 4hf + 0..3 of
  // column d; with groups 0/1 = (hf 0, d 0-15 / 16-31) and 2/3 = (hf 1, ...):
  const int grp16 = lane >> 4, s16 = lane & 15;
  const int v_col = 16 * (grp16 & 1) + 4 * (s16 & 3);  // + 32 dt
  const int v_row = 4 * (grp16 >> 1) + (s16 >> 2);     // + 32 t + 16 u (+ 8 for the upper 4 keys)

  f32x16 acc[T::DT];
#pragma unroll
  for (int i = 0; i < T::DT; ++i) acc[i] = f32x16{};
  float m_ref = kNegInf, l_run = 0.f;

  // S^T = K Q^T for the block in K buffer `buf`: two 32-key sub-tiles.
  auto qk = [&](const unsigned char* kl, f32x16 (&s)[2]) {
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int kc = 0; kc < T::KC; ++kc) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int key = 32 * t + l32;
        const int ch = 2 * kc + hf;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kl + key * T::ROW + ((ch ^ k_swz<T::CH>(key)) << 4));
        s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[kc], s[t], 0, 0, 0);
      }
    }
  };

  f32x16 s_a[2], s_b[2];  // scores of the block being finished and of the next one; roles swap each block

  // Block jb: softmax of its scores s, QK of block jb+1 (K in k_next) into
  // s_next, then O^T += V^T P^T for block jb (V in vl).
  auto compute = [&](int jb, const unsigned char* k_next, const unsigned char* vl, f32x16(&s)[2],
                     f32x16(&s_next)[2], auto masked) {
    constexpr bool MASK = decltype(masked)::value;
    const int j0 = jb * BN;

    // ---- mask: keys past the end, keys after the query (causal) ----
    if (MASK) {
      // key j0 + 4hf + o is visible iff o < lim, o = 32t + 8(r/4) + r%4
      int lim = cmask ? (q + 1 < Sk ? q + 1 : Sk) : Sk;
      lim -= j0 + 4 * hf;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int o = 32 * t + 8 * (r >> 2) + (r & 3);
          s[t][r] = o < lim ? s[t][r] : kNegInf;
        }
    }

    // ---- online softmax (log2 domain) ----
    float mx = s[0][0];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
    mx = pair_max(mx) * c;
    // Move the reference only when the max outgrows it by more than 2^8.
    if (__ballot(mx > m_ref + kRescaleSlack)) {
      const float m_new = fmaxf(m_ref, mx);
      if (m_new != kNegInf) {  // a row with no visible key yet keeps the empty state
        const float alpha = exp2_fast(m_ref - m_new);  // 0 on the first visible block
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < T::DT; ++i) acc[i] *= alpha;
        m_ref = m_new;
      }
    }
    const float m_use = m_ref == kNegInf ? 0.f : m_ref;

    // ---- next block's scores (MFMA), overlapping the exponentials below (VALU).
    // The masked body scores the next block after its PV instead (fewer live
    // registers; it runs on a few blocks per tile only). ----
    if (!MASK) qk(k_next, s_next);

    // P is rounded to bf16 once; the same rounded values feed the PV MFMA and
    // the denominator, so the weights of a row sum to exactly one.
    bf16x8 pb[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = exp2_fast(fmaf(s[t][8 * u + i], c, -m_use));
        pb[t][u] = pack_bf16x8_sum(p, l_run);
      }

    // ---- O^T += V^T P^T: A operand = 8 keys of column d, two transposed reads ----
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int dt = 0; dt < T::DT; ++dt) {
          const int col = 32 * dt + v_col;
          const int r0 = 32 * t + 16 * u + v_row, r1 = r0 + 8;
          const unsigned char* p0 = vl + r0 * T::ROW + (((col >> 3) ^ v_swz<T::CH>(r0)) << 4) + (col & 7) * 2;
          const unsigned char* p1 = vl + r1 * T::ROW + (((col >> 3) ^ v_swz<T::CH>(r1)) << 4) + (col & 7) * 2;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
          const i16x8 v8 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v8), pb[t][u], acc[dt], 0,
                                                            0, 0);
        }
      }
  };

  // ---- prologue: K0, V0, K1 in LDS; scores of block 0 ----
  // nblk >= 1: every query row sees at least key 0.
  dma_block(kr, 0, lds_k0, false);
  dma_block(vr, 0, lds_v0, true);
  if (nblk > 1) dma_block(kr, BN, lds_k1, false);
  wait_vmem();
  __syncthreads();
  qk(lds_k0, s_a);

  // Iteration jb streams K[jb+2] into the K buffer block jb used and V[jb+1]
  // into the V buffer block jb-1 used (both free since the last barrier), then
  // runs block jb.  Block jb's K and V sit in buffers jb % 2.
  auto step = [&](int jb, unsigned char* k_cur, unsigned char* k_nxt, unsigned char* v_cur, unsigned char* v_nxt,
                  f32x16(&s)[2], f32x16(&s_next)[2], auto masked) {
    const bool next1 = jb + 1 < nblk, next2 = jb + 2 < nblk;
    if (next2) dma_block(kr, (jb + 2) * BN, k_cur, false);
    if (next1) dma_block(vr, (jb + 1) * BN, v_nxt, true);
    // A wavefront whose rows all precede this block sees none of it.
    if (!decltype(masked)::value || !(cmask && jb * BN > wave_row_last)) compute(jb, k_nxt, v_cur, s, s_next, masked);
    if (decltype(masked)::value && next1) qk(k_nxt, s_next);
    wait_vmem();
    __syncthreads();
  };
  // Blocks [0, n_free) run the mask-free body, two at a time so that every
  // buffer and score set is fixed at compile time (the compiler then sees that
  // the DMA of one buffer cannot alias reads of another).  The rest (diagonal
  // blocks, a ragged tail, and always the last block, which has no next block
  // to score) run the masked body with the buffers picked at run time.
  const int n_free = n_full < nblk - 1 ? n_full : nblk - 1;
  int jb = 0;
  for (; jb + 2 <= n_free; jb += 2) {
    step(jb, lds_k0, lds_k1, lds_v0, lds_v1, s_a, s_b, std::false_type{});
    step(jb + 1, lds_k1, lds_k0, lds_v1, lds_v0, s_b, s_a, std::false_type{});
  }
  if (jb < n_free) {
    step(jb, lds_k0, lds_k1, lds_v0, lds_v1, s_a, s_b, std::false_type{});
    ++jb;
#pragma unroll
    for (int t = 0; t < 2; ++t) s_a[t] = s_b[t];
  }
  for (; jb < nblk; ++jb) {
    const bool odd = jb & 1;
    step(jb, odd ? lds_k1 : lds_k0, odd ? lds_k0 : lds_k1, odd ? lds_v1 : lds_v0, odd ? lds_v0 : lds_v1, s_a, s_a,
         std::true_type{});
  }

  // ---- epilogue: O = acc / l, bf16 round-to-nearest-even ----
  const float l_tot = pair_sum(l_run);
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
