/*
 * osx.h -- C ABI of the MI355X (gfx950) online-softmax attention library.
 *
 * Two operations, both computed by hand-written HIP kernels:
 *
 *   osx_attn_fwd      O = softmax(mask(Q K^T * scale)) V, one pass over K/V
 *                     with a running max, denominator and unnormalised
 *                     accumulator (page "softmax_attention", section 实现思路;
 *                     GQA and causal masking as in page
 *                     "从零开始写Qwen3（五-其一）使用Triton实现自注意力",
 *                     sections 自注意力原理 and GQA).
 *   osx_softmax_rows  y = softmax(x) along each row, two passes: an online
 *                     (max, sum) pass, then a normalise pass (page
 *                     "Softmax 算子的实现与优化", section Online Softmax;
 *                     page "Puzzle 8: Long Softmax").
 *
 * Conventions for every entry point:
 *   - Pointers q, k, v, o, x, y, workspace are DEVICE pointers owned by the
 *     caller; the library allocates no device memory and keeps no pointer
 *     after it returns.  Its only global state: a thread-local error message,
 *     a per-device cache of the compute-unit count, and the static scratch of
 *     osx_attn_fwd_noalloc with its per-device address.
 *   - Every call works on the calling thread's current HIP device: the
 *     buffers must be that device's memory and `stream` must belong to it
 *     (the bf16 prefill sizes its persistent grid by that device's
 *     compute-unit count).  The plan and workspace queries make no HIP call.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously on it; nothing synchronises the device.  Buffers must stay
 *     alive until that work has finished.
 *   - Alignment: the attention calls read and write 16-byte vectors, so q, k,
 *     v, o and their workspace must be 16-byte aligned (lse 4-byte); the row
 *     softmax calls need x and y aligned to their element size (2 or 4 bytes;
 *     16-byte alignment selects the vector path) and a 4-byte aligned
 *     workspace.  Anything else is OSX_EINVAL.
 *   - Arguments are checked on the host before anything is launched.  On error
 *     nothing is launched and a negative status is returned; osx_last_error()
 *     then describes the failure.  A call with no work (an empty batch, zero
 *     query rows, zero softmax rows) returns OSX_OK and launches nothing; a
 *     softmax over zero columns of a non-empty row is OSX_EINVAL.
 *   - With OSX_LOG=1 in the environment (read once per process) every call of
 *     osx_attn_fwd* and osx_softmax_rows* that launches work prints one line on
 *     stderr: the problem and the kernel, grid and workspace the plan chose.
 */
#ifndef OSX_H
#define OSX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define OSX_OK 0
#define OSX_EINVAL (-1)      /* bad argument: null pointer, negative size, Hq % Hkv != 0, overlap, a softmax over
                                nothing (seq_k == 0 with query rows, cols == 0 with rows) */
#define OSX_EUNSUPPORTED (-2) /* valid request outside what the kernels implement (head_dim, causal with Sq != Sk,
                                 one head's Q/K/V of 2^31 bytes or more) */
#define OSX_EHIP (-3)        /* the HIP runtime reported an error at launch */
#define OSX_EWORKSPACE (-4)  /* workspace missing or smaller than the size the query returns */

/* Element types of q, k, v, o.  Accumulation is fp32 in both. */
#define OSX_F32 0
#define OSX_BF16 1

/* Kernel families chosen by the planner. */
#define OSX_KERNEL_NONE 0          /* no work */
#define OSX_KERNEL_PREFILL_F32 1   /* fp32 MFMA tiles, any seq_q */
#define OSX_KERNEL_PREFILL_BF16 2  /* bf16 MFMA tiles, any seq_q */
#define OSX_KERNEL_DECODE_BF16 3   /* bf16, seq_q == 1: K/V split across workgroups (+ combine when split) */
#define OSX_KERNEL_SOFTMAX_ROW 4   /* one workgroup per row, the row held in registers */
#define OSX_KERNEL_SOFTMAX_SPLIT 5 /* rows split across workgroups, (m, l) partials merged */
#define OSX_KERNEL_SOFTMAX_WAVE 6  /* one wavefront per row, the row held in registers */

/* What the library will launch for a given problem (filled by the plan calls). */
typedef struct osx_plan {
  int kernel;             /* OSX_KERNEL_* */
  int threads;            /* threads per workgroup of the main kernel */
  int block_m;            /* query rows (attention) or elements (softmax) per workgroup */
  int block_n;            /* keys per LDS block (attention) */
  int splits;             /* K/V splits per (batch, KV head) (decode) or chunks per row (softmax) */
  int heads_per_wg;       /* query heads sharing one workgroup (attention) */
  int64_t grid;           /* workgroups of the main kernel */
  size_t workspace_bytes; /* bytes of workspace the call needs (0 = none) */
} osx_plan;

/*
 * osx_attn_plan -- choose the kernel for an attention problem; no HIP calls.
 *
 * Shapes (all tensors contiguous, last dimension stride 1, row-major):
 *   q, o : [batch, heads_q,  seq_q, head_dim]
 *   k, v : [batch, heads_kv, seq_k, head_dim]
 * Query head h reads KV head h / (heads_q / heads_kv) (page
 * "从零开始写Qwen3（五-其一）使用Triton实现自注意力", section GQA).
 * causal != 0 keeps key j for query i only when j <= i, and only when
 * seq_q > 1 (the eager reference of section 自注意力原理 skips the mask for a
 * single query row); with seq_q > 1 it requires seq_q == seq_k.
 * Supported head_dim: fp32 any multiple of 4 in [4, 128]; bf16 any multiple of
 * 16 in [16, 128].  Head dims that are not a multiple of the kernel's tile
 * width (32 for fp32; 64 or 128 for bf16) run with the missing columns read as
 * zeros and never stored (page "softmax_attention", section 实现思路, pads the
 * head dimension up to the block width and masks the padded lanes).
 * Returns OSX_OK, OSX_EINVAL or OSX_EUNSUPPORTED; `out` may be NULL.
 */
int osx_attn_plan(int dtype, int batch, int heads_q, int heads_kv, int seq_q, int seq_k, int head_dim, int causal,
                  osx_plan* out);

/*
 * Workspace bytes osx_attn_fwd needs for this problem, via *bytes: the partial
 * (m, l, acc) states when the keys are split across workgroups (fp32 with few
 * row tiles, decode with few (batch, KV head) units); 0 otherwise (bf16
 * prefill, and decode that runs as one split).
 */
int osx_attn_fwd_workspace(int dtype, int batch, int heads_q, int heads_kv, int seq_q, int seq_k, int head_dim,
                           int causal, size_t* bytes);

/*
 * The same size as a return value: the bytes of caller-allocated scratch
 * osx_attn_fwd needs for this problem (page "Softmax 算子的实现与优化", section
 * Baseline: the host allocates the scratch buffers the kernels combine
 * through).  0 when none is needed -- and also for a problem osx_attn_fwd
 * would reject (the reason is then in osx_last_error(); osx_attn_plan returns
 * the status).
 */
size_t osx_attn_fwd_workspace_bytes(int dtype, int batch, int heads_q, int heads_kv, int seq_q, int seq_k,
                                    int head_dim, int causal);

/*
 * osx_attn_fwd -- single-pass attention forward.
 *
 * q, k, v, o: device pointers in the layouts above, all of element type
 * `dtype` (OSX_F32 or OSX_BF16); o is written in full.  scale <= 0 selects
 * 1/sqrt(head_dim) (page "softmax_attention": scores are multiplied by
 * d^-0.5); a NaN or +inf scale, or one so large that scale * log2(e)
 * overflows fp32, is OSX_EINVAL.  workspace: device buffer of at least the bytes
 * osx_attn_fwd_workspace reports (may be NULL when that is 0); its contents
 * on entry do not matter.  o must not overlap q, k, v or the workspace, nor
 * the workspace q, k or v (OSX_EINVAL).
 */
int osx_attn_fwd(const void* q, const void* k, const void* v, void* o, int dtype, int batch, int heads_q,
                 int heads_kv, int seq_q, int seq_k, int head_dim, int causal, float scale, void* workspace,
                 size_t workspace_bytes, void* stream);

/*
 * osx_attn_fwd_lse -- osx_attn_fwd that also writes, for every query row, the
 * natural log of its softmax denominator:
 *     lse[(b * heads_q + h) * seq_q + i] = log sum_j exp(scale * q_i . k_j)
 * over the keys visible to row i.  This is the final state of the online
 * recurrence (page "Softmax 算子的实现与优化", section Online Softmax: the
 * running max m and l = sum_j e^{x_j - m} after the last block) folded into
 * one number, lse = m + log l; with it O (or the weights) of two key ranges
 * can be merged later.
 *
 * lse: device pointer to batch * heads_q * seq_q fp32 values, written in full
 * (NULL -> OSX_EINVAL); it must not overlap q, k, v, o or the workspace.
 * Everything else as osx_attn_fwd.
 */
int osx_attn_fwd_lse(const void* q, const void* k, const void* v, void* o, float* lse, int dtype, int batch,
                     int heads_q, int heads_kv, int seq_q, int seq_k, int head_dim, int causal, float scale,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * osx_attn_fwd_normalised -- the same O as osx_attn_fwd, computed with the
 * normalised-output form of the recurrence (page "Puzzle 9: Simple
 * FlashAttention", the recurrence under its scalar FlashAttention spec):
 *     m_i  = max(m_{i-1}, x_i)
 *     d'_i = d'_{i-1} e^{m_{i-1} - m_i} + e^{x_i - m_i}
 *     O'_i = O'_{i-1} (d'_{i-1} / d'_i) e^{m_{i-1} - m_i} + (e^{x_i - m_i} / d'_i) V_i
 * applied per block of 32 keys, so the accumulator holds the normalised output
 * after every block and the epilogue divides by nothing.  When the keys are
 * split across workgroups (the same plan as osx_attn_fwd), the slices'
 * normalised outputs are merged with weights d'_s e^{m_s - m} / sum.
 *
 * fp32 only: dtype OSX_BF16 returns OSX_EUNSUPPORTED (the bf16 kernels sum
 * the denominator on the matrix cores after the P V product, which this form
 * needs before it).  lse: NULL, or a device pointer to batch * heads_q * seq_q
 * fp32 values written as by osx_attn_fwd_lse.  The workspace is the size
 * osx_attn_fwd_workspace reports for the same fp32 problem.  Everything else,
 * errors included, as osx_attn_fwd.
 */
int osx_attn_fwd_normalised(const void* q, const void* k, const void* v, void* o, float* lse, int dtype, int batch,
                            int heads_q, int heads_kv, int seq_q, int seq_k, int head_dim, int causal, float scale,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * osx_attn_fwd_unfused -- the same O as osx_attn_fwd, computed the unfused way
 * as a comparator: the three kernels of page "从零开始写Qwen3（五-其一）使用Triton
 * 实现自注意力" (sections 免转置矩阵乘法, softmax的triton实现, 串起来):
 *   1. S = scale * Q K^T, written as an fp32 [batch * heads_q, seq_q, seq_k]
 *      matrix in the workspace (K read along head_dim, not transposed);
 *   2. the row softmax of S in place (osx_softmax_rows_ex, fp32; causal keeps
 *      key <= query);
 *   3. O = P V, with P rounded to bf16 for the products (fp32 accumulation).
 * All keys are multiplied, masked ones included, as on the page.
 *
 * dtype must be OSX_BF16 (else OSX_EUNSUPPORTED); head_dim 64 or 128 (others
 * OSX_EUNSUPPORTED);
 * seq_q * seq_k at most 2^29 (OSX_EUNSUPPORTED above).  Layouts, GQA, causal
 * and scale as osx_attn_fwd.  workspace: osx_attn_fwd_unfused_workspace bytes
 * (the score matrix, 4 bytes per score, plus the softmax's own workspace);
 * it must not overlap q, k, v or o.  Errors as osx_attn_fwd.
 */
int osx_attn_fwd_unfused_workspace(int dtype, int batch, int heads_q, int heads_kv, int seq_q, int seq_k,
                                   int head_dim, int causal, size_t* bytes);
int osx_attn_fwd_unfused(const void* q, const void* k, const void* v, void* o, int dtype, int batch, int heads_q,
                         int heads_kv, int seq_q, int seq_k, int head_dim, int causal, float scale, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * osx_attn_fwd_noalloc -- osx_attn_fwd for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  It takes no workspace and allocates nothing: the partial
 * (m, l, acc) states that osx_attn_fwd keeps in the caller's workspace go to
 * a fixed array in the library's own device memory, OSX_NOALLOC_SCRATCH_BYTES
 * per GPU, held until the process ends.  A problem whose plan needs more
 * (osx_attn_plan's workspace_bytes) returns OSX_EWORKSPACE before anything is
 * launched.  No kernel needs the array cleared between calls.
 *
 * The first call on each device (with that device current) looks up the
 * array's device address; make that first call outside any graph capture.
 * All calls on one GPU share the array: calls that overlap in time on one GPU
 * (two streams, two host threads) race on it, and the caller must order them.
 * `stream` must belong to the current device.  lse: NULL, or a device pointer
 * to batch * heads_q * seq_q fp32 values written as by osx_attn_fwd_lse.
 * Everything else, errors included, as osx_attn_fwd.
 */
#define OSX_NOALLOC_SCRATCH_BYTES (64u << 20)
int osx_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int dtype, int batch,
                         int heads_q, int heads_kv, int seq_q, int seq_k, int head_dim, int causal, float scale,
                         void* stream);

/* osx_softmax_rows_plan -- kernel choice for x[rows, cols]; no HIP calls. */
int osx_softmax_rows_plan(int64_t rows, int64_t cols, osx_plan* out);

/* Workspace bytes osx_softmax_rows needs for x[rows, cols] (0 unless rows are split), via *bytes. */
int osx_softmax_rows_workspace(int64_t rows, int64_t cols, size_t* bytes);

/*
 * The same size as a return value (page "Softmax 算子的实现与优化", section
 * Baseline: the caller allocates the scratch that per-chunk partials are
 * merged through).  0 when none is needed, and for a shape osx_softmax_rows
 * would reject (negative sizes, cols == 0 with rows > 0).
 */
size_t osx_softmax_rows_workspace_bytes(int64_t rows, int64_t cols);

/*
 * osx_softmax_rows -- y[r, :] = exp(x[r, :] - m_r) / l_r for every row r, with
 * m_r the row max and l_r = sum_j exp(x[r, j] - m_r), found in one online pass
 * over x, then a second pass over x writes y (page "Softmax 算子的实现与优化",
 * section Online Softmax).  Rows of up to 8192 columns are held on chip
 * between the passes, so x is read from memory once; longer rows are read
 * twice.
 *
 * x, y: device fp32 [rows, cols], contiguous.  y == x (in place) is allowed;
 * any other overlap is OSX_EINVAL.  cols == 0 with rows > 0 is OSX_EINVAL (a
 * softmax over nothing).  workspace as for osx_attn_fwd.
 */
int osx_softmax_rows(const float* x, float* y, int64_t rows, int64_t cols, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * osx_softmax_rows_ex -- osx_softmax_rows with options:
 *     y[r, c] = exp(scale x[r, c]) / sum_{c' visible} exp(scale x[r, c'])
 * for visible c, and y[r, c] = 0 for masked c.
 *
 * dtype: OSX_F32 or OSX_BF16, the element type of both x and y (bf16 values
 * are read exactly and y is rounded to nearest even; the arithmetic is fp32).
 * causal_period: 0 for no mask; P > 0 keeps, in row r, the columns
 * c <= r mod P (x is a stack of [P, cols] score matrices, one per head, and
 * the mask is page "从零开始写Qwen3（五-其一）使用Triton实现自注意力", section
 * softmax的triton实现: column <= row, the rest loaded as -inf).  Every row
 * keeps column 0.  Masked columns of x beyond the 16-byte vector holding a
 * row's last visible column are not read.
 * scale: positive and finite (1 for none); it multiplies x before the
 * softmax (the attention scale d^-1/2 of page "softmax_attention").
 * workspace: as for osx_softmax_rows (osx_softmax_rows_workspace gives the
 * size; it does not depend on dtype, mask or scale).  x == y is allowed.
 */
int osx_softmax_rows_ex(const void* x, void* y, int dtype, int64_t rows, int64_t cols, int64_t causal_period,
                        float scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Three-pass row softmax designs, kept as comparators for osx_softmax_rows:
 * the same y (fp32, x and y [rows, cols] contiguous, y == x allowed), computed
 * the way page "Softmax 算子的实现与优化" does before its Online Softmax
 * section.  method:
 *   OSX_3PASS_ATOMIC  section Baseline: three launches, each reading x -- the
 *                     max, the sum of e^{x - max}, the normalised output.  The
 *                     workgroups of a row combine their partials with atomic
 *                     max / atomic add on one (max, sum) pair per row in the
 *                     workspace, which a first small launch resets.  The sum's
 *                     rounding depends on the order the atomics land in.
 *   OSX_3PASS_STASH   section CUDA 版本: the max; then e^{x - max} written to y
 *                     and summed; then y multiplied by 1/sum.  Per-chunk
 *                     partials in the workspace instead of the page's single
 *                     256-thread block, so long rows use the whole GPU.
 * Each row is cut into chunks of 32768 (ATOMIC) or 16384 (STASH) elements, one
 * workgroup per chunk.
 * Errors as osx_softmax_rows; an unknown method is OSX_EINVAL.
 */
#define OSX_3PASS_ATOMIC 1
#define OSX_3PASS_STASH 2

/* Workspace bytes osx_softmax_rows_3pass needs (always > 0 for a non-empty problem), via *bytes. */
int osx_softmax_rows_3pass_workspace(int64_t rows, int64_t cols, int method, size_t* bytes);

int osx_softmax_rows_3pass(const float* x, float* y, int64_t rows, int64_t cols, int method, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * osx_read_probe -- a measurement aid, not a step of the method: a plain
 * streaming read of `bytes` of device memory at x (16-byte aligned, bytes a
 * multiple of 16) with 16-byte non-temporal loads, each word read once.  The
 * benchmark times it beside the HBM-bound kernels as the bandwidth that loads
 * alone reach on the same GPU.  Every word read is folded into an XOR, one
 * 32-bit word per wavefront written to `sink` (a device buffer of at least
 * osx_read_probe_sink_bytes() bytes, not overlapping x): the XOR of all sink
 * words equals the XOR of all words of x.  bytes == 0: OSX_OK, nothing
 * launched.  Errors: null pointers or misalignment -> OSX_EINVAL, short sink
 * -> OSX_EWORKSPACE.
 */
size_t osx_read_probe_sink_bytes(void);
int osx_read_probe(const void* x, size_t bytes, void* sink, size_t sink_bytes, void* stream);

/* Static text for a status code. */
const char* osx_status_string(int status);

/* Detail of the last failing call on this thread ("" if none). */
const char* osx_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int osx_version(void);

#ifdef __cplusplus
}
#endif

#endif /* OSX_H */
