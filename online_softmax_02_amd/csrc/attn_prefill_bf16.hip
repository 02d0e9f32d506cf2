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
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * T::K_BYTES + 2 * T::V_BYTES];

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
  auto dma_block = [&](__amdgpu_buffer_rsrc_t rsrc, int j0, int lds_off, bool is_v) {
#pragma unroll
    for (int r = 0; r < LDS_STEPS; ++r) {
      const int inst = r * kAttnWaves + wave;  // uniform
      const int row = inst * LDS_ROWS + dma_row;
      const int src_chunk = dma_chunk ^ (is_v ? v_swz<T::CH>(row) : k_swz<T::CH>(row));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (__attribute__((address_space(3))) void*)(lds + lds_off + inst * 1024), 16,
          (int)((uint32_t)((j0 + row) * D + src_chunk * 8) * 2), 0, 0, 0);
    }
  };
  auto load_k = [&](int j0, int buf) { dma_block(kr, j0, buf * T::K_BYTES, false); };
  auto load_v = [&](int j0, int buf) { dma_block(vr, j0, 2 * T::K_BYTES + buf * T::V_BYTES, true); };

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
  auto qk = [&](int buf, f32x16 (&s)[2]) {
    const unsigned char* kl = lds + buf * T::K_BYTES;
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

  f32x16 s_cur[2], s_nxt[2];

  // Softmax of block jb (scores in s_cur), QK of block jb+1 into s_nxt, then
  // O^T += V^T P^T for block jb.
  auto compute = [&](int jb, auto masked) {
    constexpr bool MASK = decltype(masked)::value;
    const int j0 = jb * BN;
    f32x16(&s)[2] = s_cur;

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
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * c;
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
    // On the last block this reads the other K buffer's stale contents and the
    // result is discarded; computing it unconditionally keeps the loop body
    // branch-free. ----
    qk((jb + 1) & 1, s_nxt);

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
    const unsigned char* vl = lds + 2 * T::K_BYTES + (jb & 1) * T::V_BYTES;
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
  load_k(0, 0);
  load_v(0, 0);
  if (nblk > 1) load_k(BN, 1);
  wait_vmem();
  __syncthreads();
  qk(0, s_cur);

  // Iteration jb: streams K[jb+2] into the K buffer block jb used and V[jb+1]
  // into the V buffer block jb-1 used (both free since the last barrier),
  // then runs block jb.
  auto step = [&](int jb, auto masked) {
    const bool next1 = jb + 1 < nblk, next2 = jb + 2 < nblk;
    if (next2) load_k((jb + 2) * BN, jb & 1);
    if (next1) load_v((jb + 1) * BN, (jb + 1) & 1);
    // A wavefront whose rows all precede this block sees none of it (its
    // scores for the next block are still computed: they may be visible).
    if (!decltype(masked)::value || !(cmask && jb * BN > wave_row_last)) {
      compute(jb, masked);
    } else {
      qk((jb + 1) & 1, s_nxt);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) s_cur[t] = s_nxt[t];
    wait_vmem();
    __syncthreads();
  };
  int jb = 0;
  for (; jb < n_full; ++jb) step(jb, std::false_type{});
  for (; jb < nblk; ++jb) step(jb, std::true_type{});

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
