// Host-side interface between the C ABI (abi.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "osx.h"

namespace osx {

// Tile constants shared by the planner and the kernels.
constexpr int kWaveSize = 64;
constexpr int kAttnThreads = 256;     // 4 wavefronts per workgroup
constexpr int kAttnWaves = 4;
constexpr int kRowsPerWave = 32;      // query rows per wavefront (one 32-wide MFMA column tile)
constexpr int kPrefillThreads = 512;  // bf16 prefill: 8 wavefronts in two alternating groups of 4
constexpr int kPrefillWaves = 8;
constexpr int kBf16BlockN = 64;       // keys per LDS block, bf16 prefill
constexpr int kF32BlockN = 32;        // keys per LDS block, fp32 prefill
constexpr int kDecodeBlockN = 32;     // keys per wavefront step, decode
constexpr int kDecodeMaxGroup = 16;   // query heads per KV head the decode kernel can pack
constexpr int kDecodeTargetWgs = 512;
constexpr int kDecodeMaxSplits = kDecodeTargetWgs;  // splits = ceil(target / units) <= target
constexpr int kSplitTargetWgs = 512;   // fp32 prefill: split the keys below this many workgroups
constexpr int kSplitMinBlocks = 2;     // ... keeping at least this many key blocks per slice
constexpr int kSoftmaxThreads = 256;
constexpr int64_t kSoftmaxWaveMax = 2048;  // longest row held by one wavefront (32 elements per lane)
constexpr int64_t kSoftmaxRowMax = 8192;   // longest row held by one workgroup (32 elements per thread)
constexpr int64_t kSoftmaxChunk = 32768;   // elements per workgroup when a row is split
// Chunk lengths of the three-pass comparators, each the faster of 16384 and
// 32768 for its own design on a 2^24-element row.
constexpr int64_t kSoftmax3PassChunkAtomic = 32768;
constexpr int64_t kSoftmax3PassChunkStash = 16384;
constexpr int64_t softmax_3pass_chunk(int method) {
  return method == OSX_3PASS_ATOMIC ? kSoftmax3PassChunkAtomic : kSoftmax3PassChunkStash;
}

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int batch, heads_q, heads_kv, seq_q, seq_k, head_dim, causal;
  float c;  // scale * log2(e): scores are exponentiated as 2^(s*c - m)
  void* workspace;
  float* lse;  // optional: natural-log sum of exp(scaled, masked scores) per query row, or null
  hipStream_t stream;
  osx_plan plan;
  int normalised = 0;  // fp32 only: run the normalised-output form of the recurrence
};

struct SoftmaxArgs {
  const void* x;
  void* y;
  int dtype;       // OSX_F32 or OSX_BF16, for x and y
  int64_t rows, cols;
  float k;         // scale * log2(e): y = 2^((x - max) k) / sum
  int64_t period;  // causal period (row r keeps columns <= r mod period), 0 = no mask
  void* workspace;
  hipStream_t stream;
  osx_plan plan;
};

struct Softmax3PassArgs {
  const void* x;
  void* y;
  int64_t rows, cols;
  int method;      // OSX_3PASS_ATOMIC or OSX_3PASS_STASH
  int splits;      // chunks per row
  int64_t chunk;   // elements per chunk (one workgroup each)
  int64_t grid;    // rows * splits
  void* workspace; // ATOMIC: (m, l) per row; STASH: (max, sum) per chunk; fp32
  hipStream_t stream;
};

// Plain streaming read (a measurement reference): kProbeWgs workgroups of
// kProbeThreads threads; the sink takes one 32-bit word per wavefront.
constexpr int kProbeWgs = 2048;
constexpr int kProbeThreads = 256;
constexpr size_t kProbeSinkBytes = (size_t)kProbeWgs * (kProbeThreads / 64) * 4;
hipError_t launch_read_probe(const void* x, size_t bytes, void* sink, hipStream_t stream);

// Compute units of the current device, queried once per device and cached.
hipError_t device_cu_count(int* n_cu);

// The checked attention call behind osx_attn_fwd / _lse / _normalised
// (argument checks, plan, launch); returns an OSX_* status and sets the
// thread's error message.
int attn_fwd_call(const void* q, const void* k, const void* v, void* o, float* lse, bool want_lse, int dtype,
                  int batch, int heads_q, int heads_kv, int seq_q, int seq_k, int head_dim, int causal, float scale,
                  void* workspace, size_t workspace_bytes, void* stream, bool normalised);
// Sets the thread's error message (printf format) and returns `status`.
int set_error(int status, const char* fmt, ...);

hipError_t launch_prefill_bf16(const AttnArgs& a);
hipError_t launch_prefill_f32(const AttnArgs& a);
hipError_t launch_decode_bf16(const AttnArgs& a);
hipError_t launch_softmax_rows(const SoftmaxArgs& a);
hipError_t launch_unfused_scores(const AttnArgs& a, float* s, float scale);  // bf16, head_dim 64 or 128
hipError_t launch_unfused_pv(const AttnArgs& a, const float* p);
hipError_t launch_softmax_3pass(const Softmax3PassArgs& a);

}  // namespace osx
