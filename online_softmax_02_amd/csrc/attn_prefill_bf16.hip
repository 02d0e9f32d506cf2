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
//  * A workgroup is 8 wavefronts in two groups of 4, one workgroup per CU, so
//    each SIMD runs one wavefront of each group.  Each wavefront owns 32 query
//    rows of one query head; all 8 share one KV head (GQA: query head h reads
//    KV head h / G).  The second group holds the 32-row tiles that follow the
//    first group's.
//  * The groups alternate between two phases, separated by workgroup barriers:
//    an MFMA phase (scores of key block j+1, then O += P V for block j) and a
//    softmax phase (max, exponentials, bf16 P and row sums for block j+1).
//    Group B runs one phase behind group A, so on every SIMD one wavefront
//    feeds the matrix cores while the other runs the exponentials.
//  * K and V blocks of 64 keys are staged through LDS in 4 stages with 16-byte
//    direct-to-LDS buffer loads; stage s holds K
//    of block j+1 and V of block j for j = s mod 4.  A stage is loaded three
//    blocks before its MFMA phase, by all 8 wavefronts, each of which waits
//    for all its loads at the end of its next softmax phase (loads past the
//    last block are issued anyway, so every wait has a fixed count).  The loop
//    is unrolled by 4 so every stage is a fixed LDS object: the compiler then
//    knows that a read of one stage does not wait for a load into another.
//  * Row sums l of the bf16 weights are taken on the matrix cores too, with a
//    16x16x32 MFMA per 16 keys that reads the PV step's P^T register as is.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    a lane then holds 16 scores of ONE query, so the row max and row sum are
//    lane-local (plus one permlane exchange between the two lane halves) and
//    the rescale factor is a per-lane scalar.
//  * The output is also accumulated transposed, O^T += V^T P^T, with P (rounded
//    to bf16 once) taken from the score registers as the B operand.  V stays
//    row-major in LDS; ds_read_b64_tr_b16 delivers it transposed.
//  * exp is 2^(s*c - m) with c = scale*log2(e) folded into one FMA; m lives in
//    that log2 domain.  The reference m used in the exponent is moved (and acc,
//    l rescaled by 2^(m_old - m_new)) only when a row's running max exceeds it
//    by more than 2^8; the result is identical in exact arithmetic (the page's
//    shift invariance) and the exponentials stay <= 2^8.
//  * Causal: key blocks wholly after the workgroup's last query are never
//    visited, a wavefront skips the work of blocks that lie wholly after its
//    own rows, and only blocks that cross the diagonal (or the end of the keys)
//    are masked; tiles are dispatched heaviest first.
//  * Every global offset (row, column, block) goes into the buffer
//    instruction's VGPR offset, which the hardware checks against the
//    resource's range; the scalar offset, which it does not check, is always
//    0.  Rows past the end of a head, blocks past the last one and padded
//    head-dimension columns therefore read as zeros without touching memory.
//  * A head dimension d that is a multiple of 16 below 64 or between 64 and
//    128 runs in the 64- or 128-wide kernel: the padded columns of Q, K and V
//    read as zeros (page "softmax_attention", section 实现思路, pads d up to
//    the block width and masks the extra lanes the same way), add nothing to
//    the scores, and are never stored.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace osx {
namespace {

constexpr int BN = kBf16BlockN;        // 64 keys per block
constexpr int kGroupWaves = kPrefillWaves / 2;
constexpr int kStages = 4;
constexpr float kRescaleSlack = 8.0f;  // log2 units a row max may exceed the reference before a rescale
constexpr uint32_t kOffNowhere = 0x80000000u;  // a buffer offset past any head (heads are < 2^31 bytes)

typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <int D>
struct Bf16Tile {
  static constexpr int CH = D / 8;                       // 16-byte chunks per K/V row
  static constexpr int KC = D / 16;                      // k-steps of the QK MFMA
  static constexpr int DT = D / 32;                      // 32-row d tiles of the PV MFMA
  static constexpr int ROW = D * 2;                      // bytes per K/V row in LDS
  static constexpr int BLOCK_BYTES = BN * ROW;           // one K or V block in LDS
  static constexpr int LDS_ROWS = 64 / CH;               // rows per 1 KiB direct-to-LDS instruction
  static constexpr int DMA_INSTS = BN / LDS_ROWS;        // instructions per K (or V) block
  static constexpr int DMA_PER_WAVE = DMA_INSTS / kPrefillWaves;
  static_assert(DMA_INSTS % kPrefillWaves == 0, "each wavefront loads an equal share of a block");
  static_assert((kPrefillWaves * LDS_ROWS) % 16 == 0, "a wavefront's rows keep their swizzle across instructions");
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

// s_waitcnt immediates (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}
// Phase boundary: no instruction is scheduled across it, every LDS read of
// the phase has returned, and all 8 wavefronts arrive before any goes on.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  OSX_DEBUG_SYNC_WG();  // every wavefront passes the same number of phase barriers
}

// D: the kernel's (padded) head dimension, 64 or 128.  PAD: the true head
// dimension d_arg (a multiple of 16, at most D) is smaller; global rows are
// d_arg elements long.
template <int D, bool PAD>
__global__ __launch_bounds__(kPrefillThreads, 1) void prefill_bf16_kernel(
    const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg, const uint16_t* __restrict__ Vg,
    uint16_t* __restrict__ Og, float* __restrict__ Lse, int Hq, int Hkv, int Sq, int Sk, int d_arg, int causal,
    float c, int hp, int n_hgroups, int n_qtiles, int units_per_tile) {
  using T = Bf16Tile<D>;
  const int d = PAD ? d_arg : D;  // elements per global row
  // One LDS object per stage and operand, so that every access names a fixed object.
  __shared__ __attribute__((aligned(16))) unsigned char lds_k0[T::BLOCK_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char lds_k1[T::BLOCK_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char lds_k2[T::BLOCK_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char lds_k3[T::BLOCK_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char lds_v0[T::BLOCK_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char lds_v1[T::BLOCK_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char lds_v2[T::BLOCK_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char lds_v3[T::BLOCK_BYTES];
  // Stages are indexed with constants only (every call below passes a literal
  // stage), so after inlining each access names one fixed LDS object.
  unsigned char* const k_stage[kStages] = {lds_k0, lds_k1, lds_k2, lds_k3};
  unsigned char* const v_stage[kStages] = {lds_v0, lds_v1, lds_v2, lds_v3};

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps per-wave values in SGPRs
  const int grp = wave / kGroupWaves, wq = wave % kGroupWaves;
  const int l32 = lane & 31, hf = lane >> 5;

  // ---- work decomposition ----
  // Tiles (a row tile of hp query heads of one KV head) are numbered tile =
  // qt * units_per_tile + (batch, KV head, head group), with qt reversed when
  // causal so the list runs heaviest first.  The launch has one workgroup per
  // CU (or fewer when there are fewer tiles); workgroup w takes tile
  // r * W + w in even rounds r and r * W + (W - 1 - w) in odd ones, so heavy
  // and light causal tiles pair up.  Consecutive workgroups of a round walk
  // (batch, KV head), so each XCD keeps a fixed set of KV heads.
  const int G = Hq / Hkv;
  const int W = gridDim.x;
  const int n_tiles = n_qtiles * units_per_tile;
  const int rs = kGroupWaves / hp;  // 32-row tiles per group and head
  const int wg_rows = 2 * kRowsPerWave * rs;
  const bool cmask = causal && Sq > 1;
  auto tile_index = [&](int r) {
    const int w = (r & 1) ? W - 1 - (int)blockIdx.x : (int)blockIdx.x;
    const int idx = r * W + w;
    return idx < n_tiles ? idx : -1;
  };
  auto tile_qt = [&](int idx) {
    const int qt = idx / units_per_tile;
    return causal ? n_qtiles - 1 - qt : qt;
  };
  auto tile_nblk = [&](int idx) {
    int end = tile_qt(idx) * wg_rows + wg_rows;
    if (end > Sq) end = Sq;
    const int n_keys = cmask ? (end < Sk ? end : Sk) : Sk;
    return (n_keys + BN - 1) / BN;  // >= 1: the tile's first row exists and sees key 0
  };
  auto tile_kv_base = [&](int idx) {
    const int rem = idx % units_per_tile;
    return (size_t)((rem / (Hkv * n_hgroups)) * Hkv + (rem / n_hgroups) % Hkv) * Sk * d;
  };

  // The tile whose rows this wavefront is computing: its query head and rows.
  int head = 0, row0 = 0, q = 0, nblk = 1, wave_row_last = 0;
  bool wave_live = false;
  size_t q_base = 0;
  auto enter_tile = [&](int idx) __attribute__((always_inline)) {
    const int qt = tile_qt(idx);
    const int rem = idx % units_per_tile;
    const int b = rem / (Hkv * n_hgroups);
    const int kvh = (rem / n_hgroups) % Hkv;
    const int hg = rem % n_hgroups;
    head = b * Hq + kvh * G + hg * hp + (wq % hp);  // (batch, query head) flattened
    row0 = qt * wg_rows + (grp * rs + wq / hp) * kRowsPerWave;
    q = row0 + l32;
    nblk = tile_nblk(idx);
    wave_live = row0 < Sq;
    wave_row_last = row0 + kRowsPerWave - 1;
    q_base = (size_t)head * Sq * d;
  };
  // Does this wavefront's work include block j of its tile?  (Blocks wholly
  // after its rows do not.)  The tests are combined without short-circuit
  // branches, and the softmax phase marks its rare paths (a tile boundary, the
  // next tile's Q, a masked block, a rescale) unlikely, so that the common
  // path falls through with few taken branches.
  auto visible = [&](int j) { return wave_live & (j < nblk) & (!cmask | (j * BN <= wave_row_last)); };
  // Does block j need the mask for some row of this wavefront?
  auto needs_mask = [&](int j) { return j * BN + BN > Sk || (cmask && j * BN + BN - 1 > row0); };

  // ---- Q as the B operand: lane (query l32, half hf) holds columns 16kc + 8hf .. +8 ----
  // Rows past Sq and padded columns read as zeros.
  bf16x8 qreg[T::KC];
  auto load_q = [&](int idx) __attribute__((always_inline)) {
    const int qt = tile_qt(idx);
    const int rem = idx % units_per_tile;
    const int hq = (rem / (Hkv * n_hgroups)) * Hq + ((rem / n_hgroups) % Hkv) * G + (rem % n_hgroups) * hp + (wq % hp);
    const int qq = qt * wg_rows + (grp * rs + wq / hp) * kRowsPerWave + l32;
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(Qg + (size_t)hq * Sq * d, (uint32_t)Sq * d * 2);
#pragma unroll
    for (int kc = 0; kc < T::KC; ++kc) {
      const int col = kc * 16 + hf * 8;
      qreg[kc] = __builtin_bit_cast(bf16x8, buf_ld16(qr, col < d ? (uint32_t)(qq * d + col) * 2 : kOffNowhere));
    }
  };

  // ---- global -> LDS staging with buffer_load_dwordx4 ... lds ----
  // A direct-to-LDS load writes lane i's 16 bytes at M0 + 16 i, so each lane
  // fetches the global chunk that belongs in its (swizzled) LDS slot.  One
  // instruction fills LDS_ROWS rows; instructions r * 8 + wave are this
  // wavefront's.  The swizzle of a row depends only on its position within 16
  // rows, which r does not change: the lane's byte offset within a block is
  // fixed (or past the range, for a padded column), and the block and
  // instruction offsets are added to it.  Everything sits in the range-checked
  // VGPR offset, so rows past Sk -- the ragged tail and the blocks the load
  // cursors run through after a workgroup's last block -- read as zeros
  // without touching memory (a row offset past the range stays past it: a
  // head is below 2^31 bytes and the cursors run at most a few blocks beyond
  // it, so no offset wraps).
  const int dma_row = lane / T::CH, dma_chunk = lane % T::CH;
  const int dma_row0 = wave * T::LDS_ROWS + dma_row;
  const uint32_t k_voff = (dma_chunk ^ k_swz<T::CH>(dma_row0)) * 8 < d
                              ? (uint32_t)(dma_row0 * d + ((dma_chunk ^ k_swz<T::CH>(dma_row0)) << 3)) * 2
                              : kOffNowhere;
  const uint32_t v_voff = (dma_chunk ^ v_swz<T::CH>(dma_row0)) * 8 < d
                              ? (uint32_t)(dma_row0 * d + ((dma_chunk ^ v_swz<T::CH>(dma_row0)) << 3)) * 2
                              : kOffNowhere;
  auto dma_one = [&](const uint16_t* base, uint32_t voff, int j0, unsigned char* dst, int r)
                     __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(base, (uint32_t)Sk * d * 2);
    const int inst = r * kPrefillWaves + wave;  // uniform
    // A padded column's offset stays past the range as it is (adding the
    // block offset to it could wrap a 32-bit offset back into the range).
    const uint32_t off = PAD && voff == kOffNowhere
                             ? kOffNowhere
                             : voff + (uint32_t)(j0 + r * kPrefillWaves * T::LDS_ROWS) * (uint32_t)(d * 2);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(dst + inst * 1024), 16,
                                             off, 0, 0, 0);
  };
  // The load stream walks the workgroup's blocks (all its tiles, in order)
  // ahead of the compute: cursor v at the block whose V is loaded next, cursor
  // k one block further (its K is loaded with that V).  Past the last block
  // the cursors keep stepping through the last tile (rows past the end read as
  // zeros or are never used), so every phase issues the same loads.
  struct Cursor {
    int r, j, nblk;
    size_t kv_base;
  };
  auto cursor_at = [&](int r) {
    const int idx = tile_index(r);
    return Cursor{r, 0, tile_nblk(idx), tile_kv_base(idx)};
  };
  auto advance = [&](Cursor& cu) __attribute__((always_inline)) {
    if (__builtin_expect(++cu.j == cu.nblk, 0) && tile_index(cu.r + 1) >= 0) cu = cursor_at(cu.r + 1);
  };
  Cursor cur_v = cursor_at(0), cur_k = cursor_at(0);
  // Stage s: V of the block at cursor v and K of the block at cursor k (the
  // block after it), then both cursors step on.  Every stage is issued whole,
  // so each phase issues a fixed number of loads and every wait below has a
  // fixed count; the compiler can then tell which loads have landed.
  auto load_k_only = [&](int stage) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < T::DMA_PER_WAVE; ++r) dma_one(Kg + cur_k.kv_base, k_voff, cur_k.j * BN, k_stage[stage], r);
    advance(cur_k);
  };
  auto load_stage = [&](int stage) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < T::DMA_PER_WAVE; ++r) {
      dma_one(Vg + cur_v.kv_base, v_voff, cur_v.j * BN, v_stage[stage % kStages], r);
      dma_one(Kg + cur_k.kv_base, k_voff, cur_k.j * BN, k_stage[stage % kStages], r);
    }
    advance(cur_v);
    advance(cur_k);
  };
  constexpr int kStageLoads = 2 * T::DMA_PER_WAVE;  // per wavefront
  static_assert(kStageLoads < 16, "vmcnt immediate");

  // ---- per-lane constants of the transposed V read (ds_read_b64_tr_b16) ----
  // In each 16-lane group, source lane s points at row base + s/4, columns
  // c0 + 4(s%4) .. +4; lane i then receives column c0 + i of those 4 rows.
  // Lane (d = l32, hf) needs keys 16u + 4hf + 0..3 and 16u + 8 + 4hf + 0..3 of
  // column d; with groups 0/1 = (hf 0, d 0-15 / 16-31) and 2/3 = (hf 1, ...):
  const int grp16 = lane >> 4, s16 = lane & 15;
  const int v_col = 16 * (grp16 & 1) + 4 * (s16 & 3);  // + 32 dt
  const int v_row = 4 * (grp16 >> 1) + (s16 >> 2);     // + 32 t + 16 u (+ 8 for the upper 4 keys)

  // Per-lane LDS byte offsets inside a stage buffer.  K fragment (kc, t) sits
  // at k_off[kc] + 32 t rows; V fragment (t, u, dt) at v_off[dt] + (32 t + 16 u)
  // rows (+ 8 rows for its upper half): the row terms keep the swizzle
  // unchanged, so they are instruction immediates.
  int k_off[T::KC], v_off[T::DT];
#pragma unroll
  for (int kc = 0; kc < T::KC; ++kc) k_off[kc] = l32 * T::ROW + (((2 * kc + hf) ^ k_swz<T::CH>(l32)) << 4);
#pragma unroll
  for (int dt = 0; dt < T::DT; ++dt) {
    const int col = 32 * dt + v_col;
    v_off[dt] = v_row * T::ROW + (((col >> 3) ^ v_swz<T::CH>(v_row)) << 4) + (col & 7) * 2;
  }
  auto k_addr = [&](const unsigned char* kl, int kc, int t) { return kl + k_off[kc] + 32 * t * T::ROW; };
  auto v_addr = [&](const unsigned char* vl, int t, int u, int dt, int hi) {
    return vl + v_off[dt] + (32 * t + 16 * u + 8 * hi) * T::ROW;
  };

  f32x16 acc[T::DT];
#pragma unroll
  for (int i = 0; i < T::DT; ++i) acc[i] = f32x16{};
  float m_ref = kNegInf;
  // Row sums of the bf16 weights, accumulated on the matrix cores (in fp32,
  // exactly as the PV sees P) with a 16x16x32 MFMA: its B operand is the P^T
  // register of the PV step as it is, which it reads as 16 columns n of four
  // 8-key groups (queries n and n + 16, both lane halves); an A operand that
  // selects groups 0 and 2 for output rows 0-7 and groups 1 and 3 for rows
  // 8-15 makes rows 0-7 the sums of query n and rows 8-15 those of query
  // n + 16.  Half the matrix cycles of a 32x32x16 MFMA with an all-ones A and
  // a quarter of its registers; lanes 16-31 then hold the sum of query
  // l32 - 16 and lanes 32-47 that of query l32 + 16 (rows 1 and 2 of the
  // wavefront swapped), which the rare rescale and the epilogue undo.
  f32x4 acc_l = f32x4{};
  const int l_src = (lane >> 4) == 1 ? lane + 16 : ((lane >> 4) == 2 ? lane - 16 : lane);
  f32x16 s[2];      // scores of the block the next softmax phase handles
  bf16x8 pb[2][2];  // its bf16 weights, the B operand of the next PV

  // S^T = K Q^T for one block: two 32-key sub-tiles.
  auto qk = [&](const unsigned char* kl) __attribute__((always_inline)) {
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int kc = 0; kc < T::KC; ++kc) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(k_addr(kl, kc, t));
        s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[kc], s[t], 0, 0, 0);
      }
    }
  };

  // MFMA phase: scores of the next block (K in kl), O^T += V^T P^T for this
  // block (V in vl; the A operand is 8 keys of column d, from two transposed
  // reads) and the next stage's loads (at the load cursors) into k_dst /
  // v_dst.  The order is fixed by
  // hand (sched_barrier fences): the LDS read of each MFMA's fragment is
  // issued kAhead MFMAs earlier, into a ring of registers, and the loads of
  // the later stage are spread over the score MFMAs.
  auto gemm_fast = [&](const unsigned char* kl, const unsigned char* vl, unsigned char* k_dst,
                       unsigned char* v_dst) __attribute__((always_inline)) {
    constexpr int NQ = 2 * T::KC, NP = 4 * T::DT, N = NQ + NP;
    constexpr int kAhead = 4, kRing = 6;
    auto frag = [&](int m) -> bf16x8 {
      if (m < NQ) return *reinterpret_cast<const bf16x8*>(k_addr(kl, m >> 1, m & 1));
      const int i = m - NQ;
      const int t = i / (2 * T::DT), u = (i / T::DT) % 2, dt = i % T::DT;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v_addr(vl, t, u, dt, 0)));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v_addr(vl, t, u, dt, 1)));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    constexpr int kDmaEvery = NQ / (2 * T::DMA_PER_WAVE);
    const uint32_t sel = ((lane >> 4) & 1) == ((lane & 15) >> 3) ? 0x3f803f80u : 0u;  // bf16 1.0 pairs or 0
    const bf16x8 kSel = __builtin_bit_cast(bf16x8, u32x4{sel, sel, sel, sel});
    bf16x8 ring[kRing];
#pragma unroll
    for (int m = 0; m < kAhead; ++m) ring[m % kRing] = frag(m);
    // Row sums of this block's P first: they need no LDS data, so they cover
    // the latency of the first reads.
#pragma unroll
    for (int tu = 0; tu < 4; ++tu) {
      __builtin_amdgcn_sched_barrier(0);
      acc_l = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kSel, pb[tu >> 1][tu & 1], acc_l, 0, 0, 0);
    }
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int m = 0; m < N; ++m) {
      __builtin_amdgcn_sched_barrier(0);
      if (m + kAhead < N) ring[(m + kAhead) % kRing] = frag(m + kAhead);
      if (m < NQ) {
        s[m & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[m % kRing], qreg[m >> 1], s[m & 1], 0, 0, 0);
        if (m % kDmaEvery == kDmaEvery - 1) {  // one direct-to-LDS load of stage jn
          const int d = m / kDmaEvery;           // 0 .. 2 * DMA_PER_WAVE - 1
          const int r = d % T::DMA_PER_WAVE;
          if (d < T::DMA_PER_WAVE) dma_one(Kg + cur_k.kv_base, k_voff, cur_k.j * BN, k_dst, r);
          else dma_one(Vg + cur_v.kv_base, v_voff, cur_v.j * BN, v_dst, r);
        }
      } else {
        const int i = m - NQ;
        acc[i % T::DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[m % kRing], pb[i / (2 * T::DT)][(i / T::DT) % 2],
                                                                 acc[i % T::DT], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // Softmax of block j (scores in s): mask, running max and lazy rescale,
  // exponentials and bf16 weights into pb (their row sums are taken with the
  // PV on the matrix cores).
  auto softmax = [&](int j) __attribute__((always_inline)) {
    const int j0 = j * BN;
    if (__builtin_expect(needs_mask(j), 0)) {
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
    float mx = s[0][0];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
    mx = pair_max(mx) * c;
    // Move the reference only when the max outgrows it by more than 2^8.
    if (__builtin_expect(__ballot(mx > m_ref + kRescaleSlack) != 0, 0)) {
      // Every lane takes part (the row sums are held in a layout swapped across
      // lanes, so the factor travels by a shuffle); a row with no visible key
      // yet keeps the empty state with a factor of one.
      const float m_new = fmaxf(m_ref, mx);
      const bool empty = m_new == kNegInf;
      const float alpha = empty ? 1.0f : exp2_fast(m_ref - m_new);  // 0 on the first visible block
      acc_l *= __shfl(alpha, l_src, 64);
#pragma unroll
      for (int i = 0; i < T::DT; ++i) acc[i] *= alpha;
      m_ref = empty ? m_ref : m_new;
    }
    const float m_use = m_ref == kNegInf ? 0.f : m_ref;
    // P is rounded to bf16 once; the same rounded values feed the PV MFMA and
    // the denominator, so the weights of a row sum to one (up to fp32 rounding
    // of the sum).
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = exp2_fast(fmaf(s[t][8 * u + i], c, -m_use));
        pb[t][u] = pack_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
      }
  };

  // ---- epilogue of a tile: O = acc / l (bf16, round to nearest even) and, if
  // asked, the log-sum-exp ln 2 * (m + log2 l): the sum of 2^(s c) is 2^m l for
  // whatever reference m the row ended with ----
  auto store_tile = [&]() __attribute__((always_inline)) {
    const float l_tot = __shfl(acc_l[0], l_src, 64);
    const float inv = 1.0f / l_tot;
    if (Lse && hf == 0 && q < Sq) Lse[(size_t)head * Sq + q] = (m_ref + log2f(l_tot)) * kLn2;
    // Lane (query q, half hf) holds, per 32-row tile dt and group g, columns
    // 32 dt + 8 g + 4 hf .. +3 of its row.  One v_permlane32_swap per word
    // (with every lane active) trades the two halves' pieces so that each lane
    // holds 8 consecutive columns -- hf = 0 those of groups 2k, hf = 1 those of
    // groups 2k + 1 -- and writes them as one 16-byte store: half the store
    // instructions and requests of 8-byte pieces.
    uint16_t* op = Og + q_base + (size_t)q * d;
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        u32x4 w;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t ev = pack_bf16x2(acc[dt][8 * k + 2 * h] * inv, acc[dt][8 * k + 2 * h + 1] * inv);
          const uint32_t od = pack_bf16x2(acc[dt][8 * k + 4 + 2 * h] * inv, acc[dt][8 * k + 5 + 2 * h] * inv);
          // the upper half's even-group word for the lower half's odd-group word
          const auto r = __builtin_amdgcn_permlane32_swap(ev, od, false, false);
          w[h] = r[0];      // hf = 0: its own columns 16k + 2h ..; hf = 1: the partner's 16k + 8 + 2h ..
          w[2 + h] = r[1];  // hf = 0: the partner's columns 16k + 4 + 2h ..; hf = 1: its own 16k + 12 + 2h ..
        }
        const int d0 = 32 * dt + 16 * k + 8 * hf;
        if (q < Sq && d0 < d) *reinterpret_cast<u32x4*>(op + d0) = w;  // padded columns are not stored
      }
  };

  // The block the next softmax phase handles: block jc of tile rc (ordinal
  // among this workgroup's tiles).
  int rc = 0, jc = 0;
  bool finished = false;
  // Softmax phase.  With `next`, it moves to the following block first; when
  // that starts a new tile, the finished tile is stored (its last PV was
  // issued in the MFMA phase just ended) and the running state restarts (the
  // first visible block rescales acc and l by 2^-inf = 0).  When the block is
  // the last of its tile, the next tile's Q is loaded here, for the scores the
  // next MFMA phase computes.  Ends by waiting for this wavefront's loads of
  // the stage two blocks ahead (and for Q, when it was loaded).
  auto softmax_phase = [&](bool next) __attribute__((always_inline)) {
    if (next) {
      if (__builtin_expect(jc + 1 < nblk, 1)) {
        ++jc;
      } else {
        store_tile();
        const int idx = tile_index(rc + 1);
        if (idx < 0) {
          finished = true;
        } else {
          ++rc;
          jc = 0;
          enter_tile(idx);
          m_ref = kNegInf;
        }
      }
    }
    auto weights = [&]() __attribute__((always_inline)) {
      if (__builtin_expect(!finished && visible(jc), 1)) {
        softmax(jc);
      } else {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int u = 0; u < 2; ++u) pb[t][u] = bf16x8{};
      }
    };
    // The next tile's Q is loaded before this block's weights are formed, so
    // its latency overlaps the exponentials.  Every softmax phase ends by
    // waiting for all of this wavefront's loads: the compiler then knows on
    // every path that Q has landed and adds no waits before the score MFMAs.
    // (The wait also covers the stage loads issued in the MFMA phase just
    // ended, three blocks ahead of their use.)
    const int next_q = !finished && jc + 1 == nblk ? tile_index(rc + 1) : -1;
    if (__builtin_expect(next_q >= 0, 0)) load_q(next_q);
    weights();
    wait_vmcnt<0>();
  };

  // Global block g at stage P = g mod 4 (g counts the blocks of all this
  // workgroup's tiles).  MFMA phase: scores of block g+1 (K in stage P), O += P V
  // for block g (V in stage P), loads of stage P+3 (V of block g+3, K of block
  // g+4).  Softmax phase: block g+1.
  auto block = [&](int P) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(3);  // the MFMA phase wins issue slots over the other group's softmax
    // Always the full MFMA phase: a block this wavefront cannot see has zero
    // weights (its PV adds nothing) and its scores go unused.
    gemm_fast(k_stage[P], v_stage[P], k_stage[(P + 3) % kStages], v_stage[(P + 3) % kStages]);
    phase_barrier();
    __builtin_amdgcn_s_setprio(0);
    // The load cursors step on here, in the softmax phase, which has slack:
    // their scalar arithmetic (the next tile's indices) would otherwise sit at
    // the end of the MFMA phase, ahead of its barrier.
    advance(cur_v);
    advance(cur_k);
    softmax_phase(true);
    phase_barrier();
  };

  // ---- prologue: Q of the first tile; K of block 0 into stage 3, stages 0..2;
  // scores and softmax of block 0 ----
  int n_blocks = 0;  // blocks of all this workgroup's tiles
  for (int r = 0; tile_index(r) >= 0; ++r) n_blocks += tile_nblk(tile_index(r));
  enter_tile(tile_index(0));
  load_q(tile_index(0));
  load_k_only(3);
  load_stage(0);
  load_stage(1);
  load_stage(2);
  // Stage 1 is read in the third phase, before group B's first wait; so only
  // stage 2 may still be in flight at the first barrier.
  wait_vmcnt<kStageLoads>();
  phase_barrier();
  qk(k_stage[3]);
  softmax_phase(false);
  phase_barrier();
  if (grp == 1) phase_barrier();  // group B runs one phase behind group A

  int g = 0;
  for (; g + kStages <= n_blocks; g += kStages) {
    block(0);
    block(1);
    block(2);
    block(3);
  }
  if (g < n_blocks) block(0);
  if (g + 1 < n_blocks) block(1);
  if (g + 2 < n_blocks) block(2);
  if (grp == 0) phase_barrier();  // group A ends one phase ahead: keep the barrier counts equal
  wait_vmcnt<0>();  // no load into LDS may land after the workgroup has ended
}

template <int D, bool PAD>
hipError_t launch(const AttnArgs& a) {
  const int G = a.heads_q / a.heads_kv;
  const int hp = a.plan.heads_per_wg;
  const int n_hgroups = G / hp;
  const int rows_per_wg = a.plan.block_m;
  const int n_qtiles = (a.seq_q + rows_per_wg - 1) / rows_per_wg;
  const int units_per_tile = a.batch * a.heads_kv * n_hgroups;
  // One persistent workgroup per CU (fewer when there are fewer tiles); they
  // walk the plan's tiles.
  int n_cu = 0;
  const hipError_t e = device_cu_count(&n_cu);
  if (e != hipSuccess) return e;
  const int64_t grid = a.plan.grid < n_cu ? a.plan.grid : n_cu;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, PAD>), dim3((unsigned)grid), dim3(kPrefillThreads), 0, a.stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse, a.heads_q, a.heads_kv,
                     a.seq_q, a.seq_k, a.head_dim, a.causal, a.c, hp, n_hgroups, n_qtiles, units_per_tile);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const AttnArgs& a) {
  if (a.head_dim % 16 != 0 || a.head_dim <= 0 || a.head_dim > 128) return hipErrorInvalidValue;
  if (a.head_dim == 64) return launch<64, false>(a);
  if (a.head_dim == 128) return launch<128, false>(a);
  return a.head_dim < 64 ? launch<64, true>(a) : launch<128, true>(a);
}

}  // namespace osx
