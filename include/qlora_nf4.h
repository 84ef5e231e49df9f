/*
 * qlora_nf4.h -- C ABI of the MI355X (gfx950) library for the frozen-NF4
 * linear layer with a LoRA side path.
 *
 * The method (QLoRA): the pretrained weight W is quantised once to 4-bit
 * NormalFloat codes with blockwise absmax constants, the constants are
 * themselves quantised to 8 bits (double quantisation), and every training
 * step dequantises W on the fly in the bf16 compute dtype, adds the low-rank
 * adapter branch and backpropagates through the frozen W into the adapters.
 * Sources (page title, section):
 *   - "QLoRA: Fine-Tuning a 70B on One GPU": "NF4 Quantization" (lookup table
 *     of 16 normal-CDF levels, nearest-level mapping, done once before
 *     training), "Double Quantization" (the block constants quantised to INT8,
 *     on-the-fly dequantisation for the matmul), "Practical Implementation"
 *     (nf4 type, double-quant flag, bf16 compute dtype, LoRA r / lora_alpha).
 *   - inquiringlines.com note on QLoRA cutting 65B finetuning memory to <48 GB,
 *     mechanism paragraph (frozen 4-bit base, gradients through it into LoRA
 *     adapters; equal-share normal bins; quantising the constants themselves).
 *   - xingyuzhitong guide "Fine-Tuning Memory Requirements", section "LoRA:
 *     freeze the base, train small adapters" (the r x (d_in + d_out) adapter
 *     pair beside the frozen weight).
 * Readings of points the pages leave open (fixed by this library):
 *   block of 64 weights per absmax, 256 absmax per second-level scale, one
 *   float32 mean per tensor, signed int8 constants with scale max|d|/127,
 *   codes packed two per byte with the even element in the low nibble,
 *   nearest level with ties to the lower level, LoRA scale s = alpha / r.
 *
 * Conventions.
 *   - W is [rows = N, cols = K] row-major (out x in, PyTorch Linear layout);
 *     X [M, K], A [r, K], B [N, r], Y [M, N], dY [M, N], dX [M, K], all
 *     row-major and dense.  bf16 tensors are passed as raw uint16 bits.
 *   - Every pointer argument is device memory owned by the caller, except the
 *     descriptor structs and the codebook output, which are host memory.  The
 *     library never allocates or frees device memory; scratch comes from the
 *     caller's workspace, sized by the *_workspace_bytes queries.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Work is
 *     enqueued on it and the call returns before it completes; no call
 *     synchronises the host.  Inputs must stay alive until the stream has
 *     passed the call.  Calls that share a workspace must be ordered on one
 *     stream.
 *   - Errors: argument checks run on the host before anything is enqueued and
 *     return a status with nothing launched.  A failed launch returns
 *     QLORA_ERR_HIP.  Outputs are overwritten, never accumulated into.
 *   - Preconditions not checked on the hot path: W is finite; input and output
 *     buffers do not overlap.
 */
#ifndef QLORA_NF4_H
#define QLORA_NF4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QLORA_OK = 0,
  QLORA_ERR_INVALID_ARG = 1,   /* null pointer, bad size, bad block sizes */
  QLORA_ERR_UNSUPPORTED = 2,   /* shape outside what the kernels handle (e.g. K % 64) */
  QLORA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than the query says */
  QLORA_ERR_HIP = 4            /* a HIP launch failed */
} qlora_status;

typedef enum { QLORA_F32 = 0, QLORA_BF16 = 1 } qlora_dtype;

typedef uint16_t qlora_bf16;   /* raw bfloat16 bits */

#define QLORA_NF4_BLOCK 64     /* weights per first-level absmax */
#define QLORA_DQ_BLOCK 256     /* first-level constants per second-level scale */
#define QLORA_MAX_RANK 128

/* 4-bit types (qlora_nf4_tensor.quant_type). */
#define QLORA_QUANT_NF4 0      /* the normal-quantile table (default) */
#define QLORA_QUANT_INT4 1     /* the uniform table NF4 is set against */

/* Quantised-weight descriptor (host struct; buffers are device memory the
 * caller allocates).  With n = rows*cols, nb = ceil(n/64), nd = ceil(nb/256):
 *   codes        uint8[ceil(n/2)]  element 2i in the low nibble of byte i
 * and, with double quantisation (dq_block = 256):
 *   absmax_q     int8[nb]          8-bit first-level constants
 *   absmax_scale float32[nd]       second-level scale of each 256 constants
 *   absmax_mean  float32[1]        per-tensor mean of the first-level constants
 * The reconstructed constant of block b is fma(absmax_q[b], absmax_scale[b/256],
 * absmax_mean[0]).  Without it (dq_block = 0; the double-quant switch of
 * "QLoRA: Fine-Tuning a 70B on One GPU", section "Practical Implementation"):
 *   absmax       float32[nb]       the block absmax itself
 * and the three pointers above are unused.  Weight i dequantises to
 * level[code_i] * the constant of its block, level from the table of
 * quant_type.  Zero-initialise the struct: the fields after absmax_mean came
 * later, and zero means NF4 with double quantisation. */
typedef struct {
  int64_t rows, cols;
  int32_t block;      /* must be 64 */
  int32_t dq_block;   /* 256 (double quantisation) or 0 (float32 constants) */
  uint8_t* codes;
  int8_t* absmax_q;
  float* absmax_scale;
  float* absmax_mean;
  float* absmax;      /* float32[nb] when dq_block == 0 */
  int32_t quant_type; /* QLORA_QUANT_NF4 or QLORA_QUANT_INT4 */
  int32_t reserved;   /* must be 0 */
} qlora_nf4_tensor;

/* Host copy of the 16 NF4 levels, ascending: 7 negative levels, an exact +0.0
 * and 8 positive levels; level 0 is -1 and level 15 is +1.  Each half takes
 * normal quantiles at equal probability steps from 1/2 to 31/32, divided by
 * the 31/32 quantile ("NF4 Quantization" section: levels from the normal CDF;
 * inquiringlines note: equal share of a zero-centred normal per bin). */
void qlora_nf4_codebook(float out[16]);

/* Host copy of the 16 levels of a 4-bit type, ascending.  QLORA_QUANT_NF4 is
 * the table above.  QLORA_QUANT_INT4 is the uniform table the NF4 section
 * ("NF4 Quantization: Beyond Standard INT4") sets NF4 against: the sixteen
 * 4-bit integers k = -8..7 over the block absmax scaled to 7, level k/7 (in
 * double, rounded once to float32); -8/7 lies below -1 and is never the
 * nearest level.  Returns QLORA_ERR_INVALID_ARG for another type or a null
 * out. */
qlora_status qlora_codebook(int32_t quant_type, float out[16]);

const char* qlora_status_string(qlora_status s);

/* Bytes of workspace qlora_quantize_nf4 needs for a rows x cols tensor. */
size_t qlora_quantize_workspace_bytes(int64_t rows, int64_t cols);

/* Blockwise 4-bit quantisation with double quantisation ("NF4 Quantization" and
 * "Double Quantization" sections), to the table of q->quant_type, and without
 * the second level when q->dq_block is 0.
 *   W   float32[rows*cols], device, read-only.
 *   q   descriptor whose buffers receive the quantised state.
 *   ws  device workspace of at least qlora_quantize_workspace_bytes(); on
 *       return (once the stream passes) its first nb floats hold the exact
 *       first-level absmax of each 64-block (with double quantisation; without
 *       it they go to q->absmax and the workspace is not written).
 * Steps: absmax of each block; x = w / absmax (IEEE float division; an all-zero
 * block gives x = 0); code = nearest level, ties to the lower; then the mean
 * of all absmax (exact binary tree of pairwise float64 sums, divided by nb and
 * rounded to float32), deviations d = absmax - mean, per 256 constants
 * scale = max|d| / 127 and q = clamp(rint(d / scale), -127, 127) (0 when the
 * scale is 0).  Any 1 <= rows*cols <= 2^37 is accepted; a larger tensor
 * returns QLORA_ERR_UNSUPPORTED (as do the dequantise calls). */
qlora_status qlora_quantize_nf4(const float* W, const qlora_nf4_tensor* q, void* ws,
                                size_t ws_bytes, void* stream);

/* qlora_quantize_nf4 for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops, harnesses that forbid hipMalloc):
 * the same launches and results, with the scratch in a fixed array of
 * 32 MiB + 64 KiB that the library keeps on each GPU it runs on until the
 * process ends, so tensors of up to 2^29 weights (536,870,912) are
 * accepted; a larger one returns QLORA_ERR_UNSUPPORTED with nothing
 * launched.  Allocates nothing and needs no workspace.  All calls on one
 * GPU share its array, which keeps the last call's contents: calls that
 * overlap on one GPU (several streams or host threads) race and must be
 * ordered by the caller.  The exact block absmax is not returned. */
qlora_status qlora_quantize_nf4_noalloc(const float* W, const qlora_nf4_tensor* q,
                                        void* stream);

/* Bytes of workspace qlora_quantize_nf4_batch needs for count tensors of
 * rows[i] x cols[i] (host arrays): the sum of qlora_quantize_workspace_bytes
 * over them; 0 for count 0 or when a size is out of range. */
size_t qlora_quantize_batch_workspace_bytes(const int64_t* rows, const int64_t* cols,
                                            int32_t count);

/* qlora_quantize_nf4 over count tensors in one call (a model's weights, say):
 * q[i] receives exactly what qlora_quantize_nf4(W[i], &q[i], ...) would give,
 * but up to 32 tensors share each launch (their codes in one launch, the
 * levels of the mean tree and the second-level constants in a few more), so
 * small tensors cost no launches of their own.
 *   W   host array of count device pointers, float32[rows*cols] each,
 *       16-byte aligned, read-only.
 *   q   host array of count descriptors; no two may share an output buffer.
 *   ws  device workspace of at least qlora_quantize_batch_workspace_bytes();
 *       its contents on return are unspecified.
 * count 0 does nothing.  Errors as qlora_quantize_nf4, for the first tensor
 * that fails a check, before anything is launched. */
qlora_status qlora_quantize_nf4_batch(const float* const* W, const qlora_nf4_tensor* q,
                                      int32_t count, void* ws, size_t ws_bytes, void* stream);

/* Dequantise to float32 or bf16 (round to nearest even) into out[rows*cols]
 * ("Double Quantization" section: NF4 weights converted back to the compute
 * dtype).  The float32 result is the single product level[code] * constant. */
qlora_status qlora_dequantize_nf4(const qlora_nf4_tensor* q, qlora_dtype out_dtype, void* out,
                                  void* stream);

/* qlora_dequantize_nf4 over count tensors: q[i] (host array of descriptors)
 * into out[i] (host array of count device pointers, 16-byte aligned, not
 * overlapping), up to 32 tensors per launch; the results equal count separate
 * calls.  count 0 does nothing.  Errors as qlora_dequantize_nf4, before
 * anything is launched. */
qlora_status qlora_dequantize_nf4_batch(const qlora_nf4_tensor* q, int32_t count,
                                        qlora_dtype out_dtype, void* const* out, void* stream);

/* The constant each 64-block dequantises with, float32[nb]: reconstructed from
 * the 8-bit state, or a copy of q->absmax without double quantisation. */
qlora_status qlora_dequantize_absmax(const qlora_nf4_tensor* q, float* out, void* stream);

/* Bytes of workspace qlora_linear_fwd / qlora_linear_bwd need. */
size_t qlora_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t r);

/* Forward of the adapted frozen linear:
 *     Y = X . W'^T + s . (X . A^T) . B^T,   s = alpha / r,
 * W' the dequantised W (rows N, cols K), computed in bf16 on the matrix cores
 * with float32 accumulation and Y rounded to bf16.  W' is rebuilt from the
 * 4-bit codes inside the kernel and never written to memory.
 *   X [M, K], A [r, K], B [N, r], Y [M, N] (bf16).  XA_out (nullable) receives
 *   bf16(X . A^T) [M, r] for reuse by the backward.
 * Requires K % 64 == 0, M >= 1, 1 <= r <= 128; X, A, B, Y, dY, dX 16-byte
 * aligned.  The kernels address X, Y, dY and dX and the codes with 32-bit
 * offsets: M*K, M*N and N*K/2 must each be below 2^32, else
 * QLORA_ERR_UNSUPPORTED (and the workspace query returns 0).  M <= 16 takes
 * the bandwidth-bound decode path (same result definition). */
qlora_status qlora_linear_fwd(const qlora_nf4_tensor* W, const qlora_bf16* X, int64_t M,
                              const qlora_bf16* A, const qlora_bf16* B, int32_t r, float alpha,
                              qlora_bf16* Y, qlora_bf16* XA_out, void* ws, size_t ws_bytes,
                              void* stream);

/* Several independent adapted linears with one token count M and one rank
 * (a layer's query, key and value projections, or its gate and up
 * projections, each with its own 4-bit weight, input and adapter pair: LoRA
 * adapts all seven projections, "Fine-Tuning Memory Requirements: Full
 * Training vs LoRA vs QLoRA", section "LoRA: freeze the base, train small
 * adapters").
 * For M <= 16 (decode) up to 8 of them share one weight-streaming launch and
 * one finish launch, so the small ones cost no launches of their own; each
 * Y (and XA) equals what qlora_linear_fwd gives for that job alone.  For
 * M > 16 two consecutive jobs with one K and 4-bit type, large enough to need
 * no split of K, share one GEMM launch (their column tiles in one grid, so a
 * partial last round of one fills with the other's tiles); the results equal
 * the single calls' as well.
 *   jobs   host array of count jobs; per job W, X [M, K], A [r, K], B [N, r],
 *          Y [M, N] (16-byte aligned) and XA_out [M, r] or NULL, all device
 *          memory, as in qlora_linear_fwd; no two jobs may share an output.
 *   ws     device workspace of at least qlora_linear_batch_workspace_bytes()
 *          (the jobs' own workspaces side by side).
 * Without dropout.  count 0 does nothing.  Errors as qlora_linear_fwd, for
 * the first job that fails a check, before anything is launched. */
typedef struct qlora_linear_job {
  const qlora_nf4_tensor* W;
  const qlora_bf16* X;
  const qlora_bf16* A;
  const qlora_bf16* B;
  qlora_bf16* Y;
  qlora_bf16* XA_out;
} qlora_linear_job;
size_t qlora_linear_batch_workspace_bytes(const qlora_linear_job* jobs, int32_t count, int64_t M,
                                          int32_t r);
qlora_status qlora_linear_fwd_batch(const qlora_linear_job* jobs, int32_t count, int64_t M,
                                    int32_t r, float alpha, void* ws, size_t ws_bytes,
                                    void* stream);

/* Backward of the same layer with W frozen (no gradient for W; the gradient
 * flows through W' into the adapters):
 *     G  = dY . B
 *     dX = dY . W' + s . G . A          (bf16 [M, K]; nullable: skipped)
 *     dA = s . G^T . X                  (float32 [r, K], overwritten)
 *     dB = s . dY^T . (X . A^T)         (float32 [N, r], overwritten)
 * XA_in (nullable) is bf16(X . A^T) [M, r] from the forward; when NULL it is
 * recomputed.  The reductions over M use a fixed split and order, so results
 * are identical run to run.  Same shape requirements as the forward. */
qlora_status qlora_linear_bwd(const qlora_nf4_tensor* W, const qlora_bf16* X, int64_t M,
                              const qlora_bf16* A, const qlora_bf16* B, int32_t r, float alpha,
                              const qlora_bf16* dY, const qlora_bf16* XA_in, qlora_bf16* dX,
                              float* dA, float* dB, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * LoRA dropout ("QLoRA: Fine-Tuning a 70B on One GPU", section "Practical
 * Implementation": the lora_dropout knob of the LoRA configuration).  Only the
 * adapter path sees the dropped input:
 *     Y = X . W'^T + s . (D(X) . A^T) . B^T,
 *     D(X)[m][k] = keep(m, k) ? X[m][k] / (1 - p) : 0.
 * keep comes from the counter-based generator Philox4x32-10 (Salmon, Moraes,
 * Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011), so
 * the backward regenerates the forward's mask instead of storing it: element
 * e = m K + k of X takes output word e mod 4 of counter (e div 4 as a 64-bit
 * value in words 0 and 1, words 2 and 3 zero) under key (seed & 0xFFFFFFFF,
 * seed >> 32), and is kept when that word >= floor(p * 2^32).  The same
 * (p, seed) must be passed to the forward and the backward of one step; a
 * new seed per step and per layer draws a new mask. */
typedef struct {
  double p;        /* drop probability, 0 <= p < 1; 0 is no dropout */
  uint64_t seed;
} qlora_dropout;

/* qlora_linear_fwd with dropout on the adapter input: XA_out receives
 * bf16(D(X) . A^T).  keep_bits_out (nullable, device, M * K / 8 bytes)
 * receives the mask as bits: bit e % 8 of byte e / 8 is 1 if element
 * e = m K + k is kept.  drop NULL or drop->p == 0 is qlora_linear_fwd (the
 * bits are then not written).  Same shapes, workspace and errors, plus
 * QLORA_ERR_INVALID_ARG for p outside [0, 1) or not a number. */
qlora_status qlora_linear_fwd_dropout(const qlora_nf4_tensor* W, const qlora_bf16* X, int64_t M,
                                      const qlora_bf16* A, const qlora_bf16* B, int32_t r,
                                      float alpha, const qlora_dropout* drop,
                                      uint8_t* keep_bits_out, qlora_bf16* Y, qlora_bf16* XA_out,
                                      void* ws, size_t ws_bytes, void* stream);

/* qlora_linear_bwd of the dropped layer (same drop as the forward):
 *     dX = dY . W' + (s . G . A) * keep / (1 - p)   (element by element)
 *     dA = s . G^T . D(X),   dB = s . dY^T . (D(X) . A^T)
 * XA_in (nullable) must be the XA_out of qlora_linear_fwd_dropout with the
 * same drop; when NULL, D(X) . A^T is recomputed.  keep_bits_in (nullable)
 * must be the forward's keep_bits_out for the same drop: the backward then
 * reads the mask instead of regenerating it (same result, less work). */
qlora_status qlora_linear_bwd_dropout(const qlora_nf4_tensor* W, const qlora_bf16* X, int64_t M,
                                      const qlora_bf16* A, const qlora_bf16* B, int32_t r,
                                      float alpha, const qlora_dropout* drop,
                                      const uint8_t* keep_bits_in, const qlora_bf16* dY,
                                      const qlora_bf16* XA_in, qlora_bf16* dX, float* dA,
                                      float* dB, void* ws, size_t ws_bytes, void* stream);

/* The keep flags of an [M, K] input under drop: out[m * K + k] = 1 if the
 * element is kept, else 0 (uint8, device memory, M * K bytes).  The mask the
 * two calls above apply, for inspection and tests.  M, K >= 0;
 * QLORA_ERR_UNSUPPORTED from 2^34 - 1024 elements on. */
qlora_status qlora_dropout_mask(int64_t M, int64_t K, const qlora_dropout* drop, uint8_t* out,
                                void* stream);

/* ------------------------------------------------------------------------
 * Grouped linear: the projections of a layer that read the same input (the
 * query, key and value projections; the gate and up projections) run as one
 * fused weight, so one GEMM makes one pass over X for all of them.  LoRA puts
 * an adapter pair at each of these projections ("Fine-Tuning Memory
 * Requirements: Full Training vs LoRA vs QLoRA", section "LoRA: freeze the
 * base, train small adapters": rank r on all seven linear projections), so
 * group g (rows [e_(g-1), e_g) of W, e_g the running sum of group_rows) keeps
 * its own A_g [r, K] and B_g [N_g, r]:
 *     A [G r, K]   the A_g stacked;
 *     B [N, G r]   block-diagonal: rows of group g hold B_g in columns
 *                  [g r, (g+1) r) and zeros elsewhere (the caller keeps the
 *                  zeros; the backward never moves them);
 * and the call computes, for every group, Y_g = X . W_g'^T + (alpha/r)
 * (X . A_g^T) . B_g^T (Y [M, N] holds the Y_g side by side; XA [M, G r] the
 * X . A_g^T side by side).  The backward gives dX = sum_g of the groups'
 * input gradients, dA [G r, K] stacked, and dB [N, G r] with the diagonal
 * blocks' gradients and exact zeros elsewhere.  1 <= G <= 8, G r <= 128.
 * Without dropout (each projection's dropout draws its own mask).  W is one
 * 4-bit tensor of the concatenated rows (its double quantisation spans the
 * groups).  Other requirements and errors as qlora_linear_fwd / _bwd. */
size_t qlora_grouped_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t r, int32_t groups);
qlora_status qlora_grouped_fwd(const qlora_nf4_tensor* W, const qlora_bf16* X, int64_t M,
                               const qlora_bf16* A, const qlora_bf16* B, int32_t r,
                               int32_t groups, const int64_t* group_rows, float alpha,
                               qlora_bf16* Y, qlora_bf16* XA_out, void* ws, size_t ws_bytes,
                               void* stream);
qlora_status qlora_grouped_bwd(const qlora_nf4_tensor* W, const qlora_bf16* X, int64_t M,
                               const qlora_bf16* A, const qlora_bf16* B, int32_t r,
                               int32_t groups, const int64_t* group_rows, float alpha,
                               const qlora_bf16* dY, const qlora_bf16* XA_in, qlora_bf16* dX,
                               float* dA, float* dB, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Adapter merge for deployment.  The adapter pair is a low-rank update of the
 * frozen weight ("Fine-Tuning Memory Requirements: Full Training vs LoRA vs
 * QLoRA", section "LoRA: freeze the base, train small adapters"), so it folds
 * into it:
 *     merged = W' + s . B . A,   s = alpha / r,
 * elementwise merged[n][k] = fl32(W'[n][k] + fl32(s * p)), p the float32 sum
 * of B[n][j] * A[j][k] over j = 0 .. r-1 in order, one fused multiply-add per
 * term; W' is the dequantised weight (as qlora_dequantize_nf4 gives it).  The
 * merged float32 weight is then quantised into `out` exactly as
 * qlora_quantize_nf4 would quantise it (its table, its double-quantisation
 * switch).  `out` may be W itself: W is read completely before any of out is
 * written (stream order). */

/* Bytes of workspace for qlora_merge_requantize with merged == NULL (room for
 * the float32 merged weight plus the quantiser's scratch); with a caller
 * buffer for merged, qlora_quantize_workspace_bytes(rows, cols) suffices. */
size_t qlora_merge_workspace_bytes(int64_t rows, int64_t cols);

/* W, out: valid 4-bit tensors of the same rows x cols.  A [r, K], B [N, r]
 * bf16 (2-byte aligned), 1 <= r <= 128.  merged (nullable, 16-byte aligned):
 * receives the float32 merged weight [N, K]; when NULL it lives in the
 * workspace.  Errors as qlora_quantize_nf4, plus QLORA_ERR_UNSUPPORTED when
 * rows * cols reaches about 2^36 (the merge launch's grid). */
qlora_status qlora_merge_requantize(const qlora_nf4_tensor* W, const qlora_bf16* A,
                                    const qlora_bf16* B, int32_t r, float alpha,
                                    const qlora_nf4_tensor* out, float* merged, void* ws,
                                    size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Adapter optimiser.  AdamW keeps a running mean m and a running mean v of
 * the squared gradient for every trainable parameter ("QLoRA: Fine-Tuning a
 * 70B on One GPU", section "Paged Optimizers"); the adapters train as float32
 * master weights with float32 gradients and statistics ("Fine-Tuning Memory
 * Requirements: Full Training vs LoRA vs QLoRA", sections "Where training
 * memory goes" and "LoRA: freeze the base, train small adapters").  One call
 * applies step t (1-based) of Adam with decoupled weight decay to every
 * tensor, element by element in float32:
 *     p <- p * (1 - lr * weight_decay)
 *     m <- beta1 * m + (1 - beta1) * g
 *     v <- beta2 * v + (1 - beta2) * g^2
 *     p <- p - lr / (1 - beta1^t) * m / (sqrt(v) / sqrt(1 - beta2^t) + eps)
 * and writes bf16(p) to param_bf16 when it is set (the adapter operand of
 * qlora_linear_fwd / _bwd).  The kernel's float32 coefficients beta1,
 * 1 - beta1, beta2, 1 - beta2, eps, 1 - lr * weight_decay, lr / (1 - beta1^t)
 * and 1 / sqrt(1 - beta2^t) are each formed in double on the host from the
 * double hyperparameters and rounded to float once. */
typedef struct {
  float* param;            /* float32 master weights [numel], updated in place */
  const float* grad;       /* float32 gradient [numel] (dA or dB of the backward) */
  float* exp_avg;          /* m [numel], updated in place */
  float* exp_avg_sq;       /* v [numel], updated in place */
  qlora_bf16* param_bf16;  /* nullable: receives bf16(param) after the update */
  int64_t numel;           /* >= 0; 0 skips the tensor */
} qlora_adamw_tensor;

typedef struct {
  double lr;            /* >= 0 */
  double beta1, beta2;  /* in [0, 1) */
  double eps;           /* > 0 */
  double weight_decay;  /* >= 0 */
} qlora_adamw_hparams;

/* One AdamW step (number `step` >= 1) over `count` tensors, asynchronously on
 * `stream` (up to 64 tensors per launch).  All pointers of a tensor with
 * numel > 0 must be non-null and 4-byte aligned (param_bf16: 2-byte); 16-byte
 * alignment takes the vector path.  The tensors must not overlap.  exp_avg
 * and exp_avg_sq (and the others) may be device memory or host memory from
 * qlora_host_state_alloc.  Returns QLORA_ERR_INVALID_ARG for bad
 * hyperparameters, step, count or tensors (nothing launched). */
qlora_status qlora_adamw_step(const qlora_adamw_hparams* h, int64_t step,
                              const qlora_adamw_tensor* tensors, int32_t count, void* stream);

/* AdamW with 8-bit statistics (the 8-bit paged AdamW named in the training
 * arguments of the addaly.com lesson "Fitting a fine-tune in 16 GB"; the
 * pages fix no 8-bit format).  The statistics are kept blockwise in 8 bits,
 * as the method keeps its block constants ("QLoRA: Fine-Tuning a 70B on One
 * GPU", section "Double Quantization": 8-bit integers with a float32 scale):
 * element e of a tensor lies in block e / 256, and
 *     m      = exp_avg_q[e] * exp_avg_scale[e / 256]          (int8 codes)
 *     sqrt(v) = exp_avg_sq_q[e] * exp_avg_sq_scale[e / 256]   (uint8 codes)
 * One call applies step t of the float32 update of qlora_adamw_step to the
 * dequantised statistics (the new sqrt(v), one correctly rounded square
 * root, serves both the update and the new codes) and quantises them again
 * per block:
 *     exp_avg_scale    = max |m| / 127,   exp_avg_q    = clamp(rint(m / scale), -127, 127)
 *     exp_avg_sq_scale = max sqrt(v) / 255, exp_avg_sq_q = clamp(rint(sqrt(v) / scale), 0, 255)
 * with code 0 where a block's scale is 0 (rint: half to even; every
 * operation one IEEE float32 rounding, no contraction).  All-zero codes and
 * scales are the zero state of step 1.  2 + 8/256 bytes of state per
 * parameter instead of 8.  The state may be device memory or host memory
 * from qlora_host_state_alloc. */
#define QLORA_ADAMW8_BLOCK 256
typedef struct {
  float* param;              /* float32 master weights [numel], updated in place */
  const float* grad;         /* float32 gradient [numel] */
  int8_t* exp_avg_q;         /* [numel], updated in place */
  float* exp_avg_scale;      /* [ceil(numel / 256)], updated in place */
  uint8_t* exp_avg_sq_q;     /* [numel], codes of sqrt(v), updated in place */
  float* exp_avg_sq_scale;   /* [ceil(numel / 256)], updated in place */
  qlora_bf16* param_bf16;    /* nullable: receives bf16(param) after the update */
  int64_t numel;             /* >= 0; 0 skips the tensor */
} qlora_adamw8_tensor;

/* One AdamW step with 8-bit statistics over `count` tensors (up to 48 per
 * launch), asynchronously on `stream`.  param, grad and the scales must be
 * 4-byte aligned (param_bf16: 2-byte); 16-byte param and grad with 4-byte
 * codes take the vector path.  Tensors must not overlap.  Returns
 * QLORA_ERR_INVALID_ARG for bad hyperparameters, step, count or tensors
 * (nothing launched). */
qlora_status qlora_adamw8_step(const qlora_adamw_hparams* h, int64_t step,
                               const qlora_adamw8_tensor* tensors, int32_t count, void* stream);

/* Optimiser state kept in host memory ("QLoRA: Fine-Tuning a 70B on One
 * GPU", section "Paged Optimizers": host RAM serves as an extension of device
 * memory for the optimiser statistics).  Allocates `bytes` of pinned,
 * coherent host memory mapped into the device address space at the same
 * address, so qlora_adamw_step reads and writes it in place over the host
 * link while the device memory holds only the weights and gradients.  The
 * caller owns it and releases it with qlora_host_state_free; its contents
 * start undefined.  QLORA_ERR_UNSUPPORTED if the mapping would need a
 * different device address. */
qlora_status qlora_host_state_alloc(size_t bytes, void** ptr);
qlora_status qlora_host_state_free(void* ptr);

/* ------------------------------------------------------------------------
 * Kernel timing (benchmark instrumentation; not part of the method).
 * Between qlora_trace_begin and qlora_trace_end, every launch of a kernel whose
 * bit is set in `kernel_mask` (1 << qlora_kernel) records its own start and end
 * into a pair of HIP events (hipExtLaunchKernel: the dispatch itself takes the
 * timestamps, so no extra packets sit between kernels), for at most `capacity`
 * launches per kernel.  qlora_trace_pause(1) stops recording (the launches run
 * untimed, with no event work) until qlora_trace_pause(0); qlora_trace_begin
 * starts unpaused.  A timed dispatch leaves the GPU idle for a few
 * microseconds around it, so a benchmark times a sample of its launches.
 * qlora_trace_end waits for those events (host synchronisation on
 * them only), writes the number of timed launches and their summed duration in
 * milliseconds into launches[QLORA_KERNEL_COUNT] / total_ms[QLORA_KERNEL_COUNT],
 * and releases the events.  Process-global state: not for concurrent use from
 * several host threads.  Returns QLORA_ERR_INVALID_ARG for a bad mask or
 * capacity, QLORA_ERR_HIP if an event call fails. */
typedef enum {
  QLORA_KERNEL_FWD_GEMM = 0,   /* dequant-fused forward GEMM (M > 16) */
  QLORA_KERNEL_DX_GEMM = 1,    /* dequant-fused dX GEMM */
  QLORA_KERNEL_QUANTIZE = 2,   /* first-level absmax + NF4 codes */
  QLORA_KERNEL_DEQUANT = 3,    /* dequantise to float32 / bf16 */
  QLORA_KERNEL_GEMV = 4,       /* decode forward (M <= 16), main kernel */
  QLORA_KERNEL_SPLIT_REDUCE = 5, /* sum of split-K GEMM partials -> bf16 */
  QLORA_KERNEL_ADAMW = 6,      /* optimiser step */
  QLORA_KERNEL_ADAMW8 = 7,     /* optimiser step with 8-bit statistics */
  QLORA_KERNEL_COUNT = 8
} qlora_kernel;

qlora_status qlora_trace_begin(uint32_t kernel_mask, int32_t capacity);
qlora_status qlora_trace_pause(int32_t paused);
qlora_status qlora_trace_end(int32_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_NF4_H */
