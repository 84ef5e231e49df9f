// C ABI of the library (declared in include/qlora_nf4.h): argument checks,
// workspace carving and the launch sequence of each call.  No device memory
// is allocated here; everything is enqueued on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cmath>
#include <cstring>
#include <vector>

#include "../../include/qlora_nf4.h"
#include "launch.h"
#include "optim.h"

using namespace qnf4;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int64_t nblocks(int64_t n) { return ceil_div(n, kBlock); }

// Largest sizes the kernels address.  The GEMM tile loaders take 32-bit
// element offsets into X / dX [M, K], Y / dY [M, N], the codes (N K / 2
// bytes) and the constant table [K/64][N]; one-dimensional launches over the
// block constants or the dropout elements must stay under 2^32 threads.
constexpr int64_t kOff32 = (int64_t)1 << 32;
constexpr int64_t kMaxWeights = (int64_t)1 << 37;   // nb = n / 64 <= 2^31

// a * b < lim for a, b >= 1, without forming the product
bool below(int64_t a, int64_t b, int64_t lim) { return a <= (lim - 1) / b; }

bool linear_fits(int64_t M, int64_t N, int64_t K) {
  return below(M, K, kOff32) && below(M, N, kOff32) && below(N, K / 2 > 0 ? K / 2 : 1, kOff32);
}

bool valid_tensor(const qlora_nf4_tensor* q) {
  if (!q || q->rows < 1 || q->cols < 1) return false;
  if (q->block != QLORA_NF4_BLOCK) return false;
  if (q->quant_type != QLORA_QUANT_NF4 && q->quant_type != QLORA_QUANT_INT4) return false;
  if (q->reserved != 0 || !q->codes || !aligned(q->codes, 4)) return false;
  if (q->dq_block == QLORA_DQ_BLOCK) {
    if (!q->absmax_q || !q->absmax_scale || !q->absmax_mean) return false;
    if (!aligned(q->absmax_q, 4) || !aligned(q->absmax_scale, 4) || !aligned(q->absmax_mean, 4))
      return false;
  } else if (q->dq_block == 0) {
    if (!q->absmax || !aligned(q->absmax, 4)) return false;
  } else {
    return false;
  }
  if (q->rows > INT64_MAX / q->cols) return false;
  return true;
}

// the quantise / dequantise launches handle at most kMaxWeights weights
bool tensor_fits(const qlora_nf4_tensor* q) { return below(q->rows, q->cols, kMaxWeights + 1); }

// float32 block constants of a tensor quantised without double quantisation
const float* f32_consts(const qlora_nf4_tensor* q) { return q->dq_block == 0 ? q->absmax : nullptr; }

qlora_status hip_status(hipError_t e) { return e == hipSuccess ? QLORA_OK : QLORA_ERR_HIP; }

// ----------------------------------------------------- quantise workspace
struct QuantWs {
  size_t absmax, pa, pb, total;
};
QuantWs quant_layout(int64_t n) {
  const int64_t nb = nblocks(n);
  const int64_t c1 = ceil_div(nb, 2048), c2 = ceil_div(c1, 2048);
  QuantWs w;
  size_t off = 0;
  w.absmax = off; off = align_up(off + (size_t)nb * sizeof(float));
  w.pa = off;     off = align_up(off + (size_t)c1 * sizeof(double));
  w.pb = off;     off = align_up(off + (size_t)(c2 > 0 ? c2 : 1) * sizeof(double));
  w.total = off;
  return w;
}

// ------------------------------------------------------- linear workspace
struct LinearWs {
  int r32;
  int64_t mp, np;             // token count padded to 32, N padded to 128
  int gemv_splits, sa, sb;    // split counts
  int sf, sx;                 // split-K slices of the forward / dX GEMM
  size_t ahat_t, xas, gemv_part, bt, gs, gt, xat, part_a, part_b, gemm_part;
  size_t sk_k, sk_n;          // skinny-product slice partials (inner dim K / N)
  size_t dec_xa;              // decode: down-projection slice partials
  size_t total;
};

LinearWs linear_layout(int64_t M, int64_t N, int64_t K, int r) {
  LinearWs w;
  w.r32 = (int)ceil_div(r, 32) * 32;
  w.mp = ceil_div(M, 32) * 32;
  w.np = ceil_div(N, 128) * 128;
  w.gemv_splits = M <= 16 ? qnf4::gemv_splits(N, K) : 0;
  w.sa = lora_grad_splits(M, K);
  w.sb = lora_grad_splits(M, N);
  w.sf = M > 16 ? fwd_splits(M, N, K) : 1;
  w.sx = dx_splits(M, N, K);
  size_t off = 0;
  w.ahat_t = off;    off = align_up(off + (size_t)(K / kBlock) * N * sizeof(float));
  w.xas = off;       off = align_up(off + (size_t)M * w.r32 * 2);
  w.gemv_part = off; off = align_up(off + (size_t)w.gemv_splits * M * N * sizeof(float));
  w.bt = off;        off = align_up(off + (size_t)r * w.np * 2);
  w.gs = off;        off = align_up(off + (size_t)M * w.r32 * 2);
  w.gt = off;        off = align_up(off + (size_t)r * w.mp * 2);
  w.xat = off;       off = align_up(off + (size_t)r * w.mp * 2);
  w.part_a = off;    off = align_up(off + (size_t)w.sa * r * K * sizeof(float));
  w.part_b = off;    off = align_up(off + (size_t)w.sb * N * r * sizeof(float));
  const size_t gp = std::max((size_t)(w.sf > 1 ? w.sf : 0) * M * N,
                             (size_t)(w.sx > 1 ? w.sx : 0) * M * K);
  w.gemm_part = off; off = align_up(off + gp * sizeof(float));
  w.sk_k = off;      off = align_up(off + skinny_part_floats(M, K, r) * sizeof(float));
  w.sk_n = off;      off = align_up(off + skinny_part_floats(M, N, r) * sizeof(float));
  w.dec_xa = off;
  if (M <= 16)
    off = align_up(off + (size_t)decode_xa_slices(K) * M * skinny_rpad(r) * sizeof(float));
  w.total = off;
  return w;
}

template <typename T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

// ------------------------------------------------------ timing instrumentation
struct Trace {
  uint32_t mask = 0;
  bool paused = false;
  int32_t capacity = 0;
  hipEvent_t* ev[QLORA_KERNEL_COUNT] = {};   // 2 * capacity events per kernel
  int32_t used[QLORA_KERNEL_COUNT] = {};
};
Trace g_trace;

}  // namespace

namespace qnf4 {
PendingTiming& pending_timing() {
  static PendingTiming t;
  return t;
}
}  // namespace qnf4

namespace {

// Runs `launch` (one kernel); when kernel `k` is traced, that dispatch records
// its own start and end into the next event pair.
template <typename F>
hipError_t traced(int k, hipStream_t s, F&& launch) {
  (void)s;
  const bool on =
      !g_trace.paused && ((g_trace.mask >> k) & 1u) && g_trace.used[k] < g_trace.capacity;
  if (on) {
    pending_timing().start = g_trace.ev[k][2 * g_trace.used[k]];
    pending_timing().stop = g_trace.ev[k][2 * g_trace.used[k] + 1];
  }
  hipError_t e = launch();
  const bool consumed = on && pending_timing().start == nullptr;
  pending_timing() = PendingTiming{};
  if (consumed && e == hipSuccess) ++g_trace.used[k];
  return e;
}

void trace_release() {
  for (int k = 0; k < QLORA_KERNEL_COUNT; ++k) {
    if (g_trace.ev[k]) {
      for (int i = 0; i < 2 * g_trace.capacity; ++i) (void)hipEventDestroy(g_trace.ev[k][i]);
      delete[] g_trace.ev[k];
      g_trace.ev[k] = nullptr;
    }
    g_trace.used[k] = 0;
  }
  g_trace.mask = 0;
  g_trace.paused = false;
  g_trace.capacity = 0;
}

qlora_status check_linear(const qlora_nf4_tensor* W, const void* X, int64_t M, const void* A,
                          const void* B, int32_t r, float alpha) {
  if (!valid_tensor(W) || !X || !A || !B) return QLORA_ERR_INVALID_ARG;
  if (M < 1 || r < 1 || r > QLORA_MAX_RANK) return QLORA_ERR_INVALID_ARG;
  if (!(alpha == alpha)) return QLORA_ERR_INVALID_ARG;
  if (W->cols % QLORA_NF4_BLOCK != 0) return QLORA_ERR_UNSUPPORTED;
  if (!linear_fits(M, W->rows, W->cols)) return QLORA_ERR_UNSUPPORTED;
  if (!aligned(X, 16) || !aligned(A, 16) || !aligned(B, 16)) return QLORA_ERR_INVALID_ARG;
  return QLORA_OK;
}

// Kernel parameters of a dropout of an input with rows of K elements: keep
// when the element's generator word >= floor(p 2^32).  NULL, or a p whose
// threshold is 0, is no dropout.  False for p outside [0, 1) or NaN.
bool dropout_params(const qlora_dropout* d, int64_t K, DropoutParams* out) {
  *out = DropoutParams{};
  if (!d) return true;
  if (!(d->p >= 0.0 && d->p < 1.0)) return false;
  const double t = std::floor(d->p * 4294967296.0);
  const uint32_t thr = t >= 4294967295.0 ? 0xFFFFFFFFu : (uint32_t)t;
  if (thr == 0) return true;
  out->thr = thr;
  out->inv = (float)(1.0 / (1.0 - d->p));
  out->k0 = (uint32_t)(d->seed & 0xFFFFFFFFu);
  out->k1 = (uint32_t)(d->seed >> 32);
  out->cols = K;
  return true;
}

}  // namespace

extern "C" {

void qlora_nf4_codebook(float out[16]) {
  if (out) std::memcpy(out, host_tables().level, sizeof(float) * 16);
}

qlora_status qlora_codebook(int32_t quant_type, float out[16]) {
  if (!out || (quant_type != QLORA_QUANT_NF4 && quant_type != QLORA_QUANT_INT4))
    return QLORA_ERR_INVALID_ARG;
  std::memcpy(out, host_tables(quant_type).level, sizeof(float) * 16);
  return QLORA_OK;
}

const char* qlora_status_string(qlora_status s) {
  switch (s) {
    case QLORA_OK: return "ok";
    case QLORA_ERR_INVALID_ARG: return "invalid argument";
    case QLORA_ERR_UNSUPPORTED: return "unsupported shape";
    case QLORA_ERR_WORKSPACE: return "workspace missing or too small";
    case QLORA_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

size_t qlora_quantize_workspace_bytes(int64_t rows, int64_t cols) {
  if (rows < 1 || cols < 1 || !below(rows, cols, kMaxWeights + 1)) return 0;
  return quant_layout(rows * cols).total;
}

// The quantiser's view of a descriptor, with its scratch at ws (layout L).
static QuantTensor quant_tensor(const float* W, const qlora_nf4_tensor* q, void* ws,
                                const QuantWs& L) {
  QuantTensor t{};
  t.w = W;
  t.n = q->rows * q->cols;
  t.kind = q->quant_type;
  t.codes = q->codes;
  if (q->dq_block == 0) {
    t.absmax = q->absmax;          // without double quantisation the exact absmax is stored
  } else {
    t.absmax = at<float>(ws, L.absmax);
    t.q = q->absmax_q;
    t.scale = q->absmax_scale;
    t.mean = q->absmax_mean;
    t.pa = at<double>(ws, L.pa);
    t.pb = at<double>(ws, L.pb);
  }
  return t;
}

static DequantTensor dequant_tensor(const qlora_nf4_tensor* q, void* out) {
  return DequantTensor{q->codes, q->absmax_q, q->absmax_scale, q->absmax_mean, f32_consts(q),
                       q->rows * q->cols, q->quant_type, out};
}

// Launch sequence of the quantiser on tensors whose arguments and workspace
// the caller has checked: per group of kQuantBatch tensors, the codes in one
// launch, then the second-level constants.
static qlora_status quantize_on(const QuantTensor* t, int64_t count, hipStream_t s) {
  for (int64_t i = 0; i < count; i += kQuantBatch) {
    const int m = (int)std::min<int64_t>(kQuantBatch, count - i);
    hipError_t e = traced(QLORA_KERNEL_QUANTIZE, s, [&] { return launch_quant_codes(t + i, m, s); });
    if (e == hipSuccess) e = launch_quant_consts(t + i, m, s);
    if (e != hipSuccess) return hip_status(e);
  }
  return QLORA_OK;
}

// Dequantiser launches: tensors with float32 constants and with the 8-bit
// state in separate groups (the constant source is a kernel template switch).
static qlora_status dequantize_on(const qlora_nf4_tensor* q, int64_t count, bool bf16,
                                  void* const* out, hipStream_t s) {
  DequantTensor group[kQuantBatch];
  for (int f32 = 0; f32 < 2; ++f32) {
    int m = 0;
    for (int64_t i = 0; i <= count; ++i) {
      if (i < count && (f32_consts(&q[i]) != nullptr) == (f32 == 1))
        group[m++] = dequant_tensor(&q[i], out[i]);
      if (m > 0 && (m == kQuantBatch || i == count)) {
        const hipError_t e = traced(QLORA_KERNEL_DEQUANT, s,
                                    [&] { return launch_dequantize(group, m, bf16, s); });
        if (e != hipSuccess) return hip_status(e);
        m = 0;
      }
    }
  }
  return QLORA_OK;
}

qlora_status qlora_quantize_nf4(const float* W, const qlora_nf4_tensor* q, void* ws,
                                size_t ws_bytes, void* stream) {
  if (!W || !valid_tensor(q) || !aligned(W, 16)) return QLORA_ERR_INVALID_ARG;
  if (!tensor_fits(q)) return QLORA_ERR_UNSUPPORTED;
  const QuantWs L = quant_layout(q->rows * q->cols);
  if (!ws || ws_bytes < L.total || !aligned(ws, kAlign)) return QLORA_ERR_WORKSPACE;
  const QuantTensor t = quant_tensor(W, q, ws, L);
  return quantize_on(&t, 1, static_cast<hipStream_t>(stream));
}

qlora_status qlora_quantize_nf4_noalloc(const float* W, const qlora_nf4_tensor* q,
                                        void* stream) {
  if (!W || !valid_tensor(q) || !aligned(W, 16)) return QLORA_ERR_INVALID_ARG;
  // at most 2^29 weights (the stated limit); the layout of that size fits the
  // array, which the second check confirms
  if (!below(q->rows, q->cols, ((int64_t)1 << 29) + 1)) return QLORA_ERR_UNSUPPORTED;
  const QuantWs L = quant_layout(q->rows * q->cols);
  if (L.total > quant_scratch_bytes()) return QLORA_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if (quant_scratch(&ws) != hipSuccess) return QLORA_ERR_HIP;
  const QuantTensor t = quant_tensor(W, q, ws, L);
  return quantize_on(&t, 1, static_cast<hipStream_t>(stream));
}

size_t qlora_quantize_batch_workspace_bytes(const int64_t* rows, const int64_t* cols,
                                            int32_t count) {
  if (count < 0 || (count > 0 && (!rows || !cols))) return 0;
  size_t total = 0;
  for (int32_t i = 0; i < count; ++i) {
    if (rows[i] < 1 || cols[i] < 1 || !below(rows[i], cols[i], kMaxWeights + 1)) return 0;
    total += quant_layout(rows[i] * cols[i]).total;
  }
  return total;
}

qlora_status qlora_quantize_nf4_batch(const float* const* W, const qlora_nf4_tensor* q,
                                      int32_t count, void* ws, size_t ws_bytes, void* stream) {
  if (count < 0 || (count > 0 && (!W || !q))) return QLORA_ERR_INVALID_ARG;
  size_t need = 0;
  for (int32_t i = 0; i < count; ++i) {
    if (!W[i] || !valid_tensor(&q[i]) || !aligned(W[i], 16)) return QLORA_ERR_INVALID_ARG;
    if (!tensor_fits(&q[i])) return QLORA_ERR_UNSUPPORTED;
    need += quant_layout(q[i].rows * q[i].cols).total;
  }
  if (count == 0) return QLORA_OK;
  if (!ws || ws_bytes < need || !aligned(ws, kAlign)) return QLORA_ERR_WORKSPACE;
  std::vector<QuantTensor> t((size_t)count);
  size_t off = 0;
  for (int32_t i = 0; i < count; ++i) {
    const QuantWs L = quant_layout(q[i].rows * q[i].cols);
    t[i] = quant_tensor(W[i], &q[i], at<uint8_t>(ws, off), L);
    off += L.total;
  }
  return quantize_on(t.data(), count, static_cast<hipStream_t>(stream));
}

qlora_status qlora_dequantize_nf4(const qlora_nf4_tensor* q, qlora_dtype out_dtype, void* out,
                                  void* stream) {
  if (!valid_tensor(q) || !out || !aligned(out, 16)) return QLORA_ERR_INVALID_ARG;
  if (out_dtype != QLORA_F32 && out_dtype != QLORA_BF16) return QLORA_ERR_INVALID_ARG;
  if (!tensor_fits(q)) return QLORA_ERR_UNSUPPORTED;
  return dequantize_on(q, 1, out_dtype == QLORA_BF16, &out, static_cast<hipStream_t>(stream));
}

qlora_status qlora_dequantize_nf4_batch(const qlora_nf4_tensor* q, int32_t count,
                                        qlora_dtype out_dtype, void* const* out, void* stream) {
  if (count < 0 || (count > 0 && (!q || !out))) return QLORA_ERR_INVALID_ARG;
  if (out_dtype != QLORA_F32 && out_dtype != QLORA_BF16) return QLORA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < count; ++i) {
    if (!valid_tensor(&q[i]) || !out[i] || !aligned(out[i], 16)) return QLORA_ERR_INVALID_ARG;
    if (!tensor_fits(&q[i])) return QLORA_ERR_UNSUPPORTED;
  }
  return dequantize_on(q, count, out_dtype == QLORA_BF16, out, static_cast<hipStream_t>(stream));
}

qlora_status qlora_dequantize_absmax(const qlora_nf4_tensor* q, float* out, void* stream) {
  if (!valid_tensor(q) || !out) return QLORA_ERR_INVALID_ARG;
  if (!tensor_fits(q)) return QLORA_ERR_UNSUPPORTED;
  return hip_status(launch_absmax_recon(q->absmax_q, q->absmax_scale, q->absmax_mean,
                                        f32_consts(q), nblocks(q->rows * q->cols), out,
                                        static_cast<hipStream_t>(stream)));
}

size_t qlora_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t r) {
  if (M < 1 || N < 1 || K < 1 || r < 1 || r > QLORA_MAX_RANK) return 0;
  if (!linear_fits(M, N, K)) return 0;
  return linear_layout(M, N, K, r).total;
}

qlora_status qlora_linear_fwd(const qlora_nf4_tensor* W, const qlora_bf16* X, int64_t M,
                              const qlora_bf16* A, const qlora_bf16* B, int32_t r, float alpha,
                              qlora_bf16* Y, qlora_bf16* XA_out, void* ws, size_t ws_bytes,
                              void* stream) {
  return qlora_linear_fwd_dropout(W, X, M, A, B, r, alpha, nullptr, nullptr, Y, XA_out, ws,
                                  ws_bytes, stream);
}

// The forward's work before its GEMM (M > 16): X.A^T -> bf16(s.XA) [M, r32]
// (GEMM tail) and bf16(XA) [M, r] (caller), with the block constants
// reconstructed in the same launch; fills the GEMM job of the linear.
static hipError_t fwd_prep(const qlora_nf4_tensor* W, const qlora_bf16* X, int64_t M,
                           const qlora_bf16* A, const qlora_bf16* B, int32_t r, float scale,
                           const DropoutParams& dp, qlora_bf16* Y, qlora_bf16* XA_out, void* ws,
                           const LinearWs& L, hipStream_t s, FwdGemmJob* job) {
  const int64_t N = W->rows, K = W->cols;
  float* ahat_t = at<float>(ws, L.ahat_t);
  uint16_t* xas = at<uint16_t>(ws, L.xas);
  SkinnyJob xa{X, K, K, A, K, 0, 0, at<float>(ws, L.sk_k), scale, xas, XA_out, nullptr, 0};
  xa.drop = dp;
  skinny_plan(&xa, M, r);
  const ReconJob rc{W->absmax_q, W->absmax_scale, W->absmax_mean, N, K / kBlock, ahat_t,
                    f32_consts(W)};
  *job = FwdGemmJob{X, W->codes, N, ahat_t, xas, B, Y};
  return launch_skinny(&xa, 1, M, r, L.r32, &rc, s);
}

qlora_status qlora_linear_fwd_dropout(const qlora_nf4_tensor* W, const qlora_bf16* X, int64_t M,
                                      const qlora_bf16* A, const qlora_bf16* B, int32_t r,
                                      float alpha, const qlora_dropout* drop,
                                      uint8_t* keep_bits_out, qlora_bf16* Y, qlora_bf16* XA_out,
                                      void* ws, size_t ws_bytes, void* stream) {
  qlora_status st = check_linear(W, X, M, A, B, r, alpha);
  if (st != QLORA_OK) return st;
  DropoutParams dp;
  if (!dropout_params(drop, W->cols, &dp)) return QLORA_ERR_INVALID_ARG;
  if (dp.thr != 0) dp.bits_out = keep_bits_out;
  if (!Y || !aligned(Y, 16)) return QLORA_ERR_INVALID_ARG;
  const int64_t N = W->rows, K = W->cols;
  const LinearWs L = linear_layout(M, N, K, r);
  if (!ws || ws_bytes < L.total || !aligned(ws, kAlign)) return QLORA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float scale = alpha / (float)r;
  hipError_t e;
  if (M <= 16) {
    const NF4Ref w{W->codes, W->absmax_q, W->absmax_scale, W->absmax_mean, f32_consts(W),
                   W->quant_type};
    const DecodeJob d{X, K, w, N, A, B, at<float>(ws, L.gemv_part), at<float>(ws, L.dec_xa), Y,
                      XA_out, dp};
    e = traced(QLORA_KERNEL_GEMV, s, [&] { return launch_decode(&d, 1, M, r, scale, s); });
    return hip_status(e);
  }
  FwdGemmJob job;
  if (fwd_prep(W, X, M, A, B, r, scale, dp, Y, XA_out, ws, L, s, &job) != hipSuccess)
    return QLORA_ERR_HIP;
  float* part = at<float>(ws, L.gemm_part);
  e = traced(QLORA_KERNEL_FWD_GEMM, s, [&] {
    return launch_fwd_gemm(&job, 1, M, K, r, L.r32, L.sf, part, W->quant_type, s);
  });
  if (e == hipSuccess && L.sf > 1)
    e = traced(QLORA_KERNEL_SPLIT_REDUCE, s,
               [&] { return launch_split_reduce(part, L.sf, M * N, Y, s); });
  return hip_status(e);
}

// Decode workspace of one job of a batch: its split partials, then its
// down-projection slice partials.
static size_t decode_job_bytes(int64_t M, int64_t N, int64_t K, int32_t r) {
  return align_up((size_t)gemv_splits(N, K) * M * N * sizeof(float)) +
         align_up((size_t)decode_xa_slices(K) * M * skinny_rpad(r) * sizeof(float));
}

size_t qlora_linear_batch_workspace_bytes(const qlora_linear_job* jobs, int32_t count, int64_t M,
                                          int32_t r) {
  if (count < 0 || (count > 0 && !jobs) || M < 1 || r < 1 || r > QLORA_MAX_RANK) return 0;
  size_t total = 0;
  for (int32_t i = 0; i < count; ++i) {
    const qlora_nf4_tensor* W = jobs[i].W;
    if (!valid_tensor(W) || !linear_fits(M, W->rows, W->cols)) return 0;
    total += M <= 16 ? decode_job_bytes(M, W->rows, W->cols, r)
                     : linear_layout(M, W->rows, W->cols, r).total;
  }
  return total;
}

qlora_status qlora_linear_fwd_batch(const qlora_linear_job* jobs, int32_t count, int64_t M,
                                    int32_t r, float alpha, void* ws, size_t ws_bytes,
                                    void* stream) {
  if (count < 0 || (count > 0 && !jobs)) return QLORA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < count; ++i) {
    const qlora_linear_job& j = jobs[i];
    const qlora_status st = check_linear(j.W, j.X, M, j.A, j.B, r, alpha);
    if (st != QLORA_OK) return st;
    if (!j.Y || !aligned(j.Y, 16)) return QLORA_ERR_INVALID_ARG;
  }
  if (count == 0) return QLORA_OK;
  const size_t need = qlora_linear_batch_workspace_bytes(jobs, count, M, r);
  if (!ws || ws_bytes < need || !aligned(ws, kAlign)) return QLORA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float scale = alpha / (float)r;
  if (M > 16) {
    // the GEMM path, each job on its own workspace region; two consecutive
    // jobs with one K and table kind and no split share one GEMM launch
    size_t off = 0;
    for (int32_t i = 0; i < count;) {
      const qlora_linear_job& a = jobs[i];
      const LinearWs La = linear_layout(M, a.W->rows, a.W->cols, r);
      void* wa = at<uint8_t>(ws, off);
      bool pair = false;
      LinearWs Lb{};
      if (i + 1 < count) {
        const qlora_linear_job& b = jobs[i + 1];
        Lb = linear_layout(M, b.W->rows, b.W->cols, r);
        pair = b.W->cols == a.W->cols && b.W->quant_type == a.W->quant_type && La.sf == 1 &&
               Lb.sf == 1;
      }
      if (!pair) {
        const qlora_status st = qlora_linear_fwd_dropout(a.W, a.X, M, a.A, a.B, r, alpha,
                                                         nullptr, nullptr, a.Y, a.XA_out, wa,
                                                         La.total, stream);
        if (st != QLORA_OK) return st;
        off += La.total;
        i += 1;
        continue;
      }
      const qlora_linear_job& b = jobs[i + 1];
      void* wb = at<uint8_t>(ws, off + La.total);
      FwdGemmJob g[2];
      hipError_t e = fwd_prep(a.W, a.X, M, a.A, a.B, r, scale, DropoutParams{}, a.Y, a.XA_out,
                              wa, La, s, &g[0]);
      if (e == hipSuccess)
        e = fwd_prep(b.W, b.X, M, b.A, b.B, r, scale, DropoutParams{}, b.Y, b.XA_out, wb, Lb, s,
                     &g[1]);
      if (e == hipSuccess)
        e = traced(QLORA_KERNEL_FWD_GEMM, s, [&] {
          return launch_fwd_gemm(g, 2, M, a.W->cols, r, La.r32, 1, nullptr, a.W->quant_type, s);
        });
      if (e != hipSuccess) return hip_status(e);
      off += La.total + Lb.total;
      i += 2;
    }
    return QLORA_OK;
  }
  DecodeJob group[kDecodeBatch];
  size_t off = 0;
  int m = 0;
  for (int32_t i = 0; i < count; ++i) {
    const qlora_linear_job& j = jobs[i];
    const qlora_nf4_tensor* W = j.W;
    const int64_t N = W->rows, K = W->cols;
    const NF4Ref w{W->codes, W->absmax_q, W->absmax_scale, W->absmax_mean, f32_consts(W),
                   W->quant_type};
    float* part = at<float>(ws, off);
    float* xa_part = at<float>(ws, off + align_up((size_t)gemv_splits(N, K) * M * N * sizeof(float)));
    off += decode_job_bytes(M, N, K, r);
    group[m++] = DecodeJob{j.X, K, w, N, j.A, j.B, part, xa_part, j.Y, j.XA_out, DropoutParams{}};
    if (m == kDecodeBatch || i == count - 1) {
      const hipError_t e =
          traced(QLORA_KERNEL_GEMV, s, [&] { return launch_decode(group, m, M, r, scale, s); });
      if (e != hipSuccess) return hip_status(e);
      m = 0;
    }
  }
  return QLORA_OK;
}

qlora_status qlora_linear_bwd(const qlora_nf4_tensor* W, const qlora_bf16* X, int64_t M,
                              const qlora_bf16* A, const qlora_bf16* B, int32_t r, float alpha,
                              const qlora_bf16* dY, const qlora_bf16* XA_in, qlora_bf16* dX,
                              float* dA, float* dB, void* ws, size_t ws_bytes, void* stream) {
  return qlora_linear_bwd_dropout(W, X, M, A, B, r, alpha, nullptr, nullptr, dY, XA_in, dX, dA,
                                  dB, ws,
                                  ws_bytes, stream);
}

// The backward; `grp` (nullable) makes dB block-diagonal (grouped linear).
static qlora_status linear_bwd_impl(const qlora_nf4_tensor* W, const qlora_bf16* X, int64_t M,
                                    const qlora_bf16* A, const qlora_bf16* B, int32_t r,
                                    float alpha, const qlora_dropout* drop,
                                    const uint8_t* keep_bits_in, const qlora_bf16* dY,
                                    const qlora_bf16* XA_in, qlora_bf16* dX, float* dA,
                                    float* dB, void* ws, size_t ws_bytes, void* stream,
                                    const GradJob* grp) {
  qlora_status st = check_linear(W, X, M, A, B, r, alpha);
  if (st != QLORA_OK) return st;
  DropoutParams dp;
  if (!dropout_params(drop, W->cols, &dp)) return QLORA_ERR_INVALID_ARG;
  if (dp.thr != 0) dp.bits = keep_bits_in;
  if (!dY || !dA || !dB || !aligned(dY, 16)) return QLORA_ERR_INVALID_ARG;
  if (dX && !aligned(dX, 16)) return QLORA_ERR_INVALID_ARG;
  const int64_t N = W->rows, K = W->cols;
  const LinearWs L = linear_layout(M, N, K, r);
  if (!ws || ws_bytes < L.total || !aligned(ws, kAlign)) return QLORA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float scale = alpha / (float)r;
  float* ahat_t = at<float>(ws, L.ahat_t);
  uint16_t* bt = at<uint16_t>(ws, L.bt);
  uint16_t* gs = at<uint16_t>(ws, L.gs);
  uint16_t* gt = at<uint16_t>(ws, L.gt);
  uint16_t* xat = at<uint16_t>(ws, L.xat);
  hipError_t e;
#define QL_TRY(call) do { e = (call); if (e != hipSuccess) return QLORA_ERR_HIP; } while (0)
  // one launch: B^T [r, N128] for G = dY.B; XA^T [r, M32] for dB from the
  // forward's copy; the block constants for the dX GEMM
  TransposeJob tj[2];
  int nt = 0;
  tj[nt++] = TransposeJob{B, N, r, bt, L.np};
  if (XA_in) tj[nt++] = TransposeJob{XA_in, M, r, xat, L.mp};
  const ReconJob rc{W->absmax_q, W->absmax_scale, W->absmax_mean, N, K / kBlock, ahat_t,
                    f32_consts(W)};
  QL_TRY(launch_prep(tj, nt, dX ? &rc : nullptr, s));
  // G = dY.B as bf16(s.G) [M, r32] (dX tail) and bf16(G)^T [r, M32] (dA);
  // without the forward's XA, X.A^T is recomputed beside it
  SkinnyJob sj[2];
  int nj = 0;
  sj[nj++] = SkinnyJob{dY, N, N, bt, L.np, 0, 0, at<float>(ws, L.sk_n), scale, gs, nullptr, gt,
                       L.mp};
  if (!XA_in) {
    sj[nj++] = SkinnyJob{X, K, K, A, K, 0, 0, at<float>(ws, L.sk_k), 1.0f, nullptr, nullptr, xat,
                         L.mp};
    sj[nj - 1].drop = dp;
  }
  for (int i = 0; i < nj; ++i) skinny_plan(&sj[i], M, r);
  QL_TRY(launch_skinny(sj, nj, M, r, L.r32, nullptr, s));
  if (dX) {
    float* part = at<float>(ws, L.gemm_part);
    QL_TRY(traced(QLORA_KERNEL_DX_GEMM, s, [&] {
      return launch_dx_gemm(dY, M, N, W->codes, K, ahat_t, gs, A, r, L.r32, dX, L.sx, part,
                            W->quant_type, &dp, s);
    }));
    if (L.sx > 1)
      QL_TRY(traced(QLORA_KERNEL_SPLIT_REDUCE, s,
                    [&] { return launch_split_reduce(part, L.sx, M * K, dX, s); }));
  }
  // dA = s . G^T X  (reduce over tokens into [r, K]);  dB = s . dY^T XA  ([N, r])
  GradJob gj[2] = {
      GradJob{X, K, gt, L.mp, L.sa, at<float>(ws, L.part_a), scale, 1, dA},
      GradJob{dY, N, xat, L.mp, L.sb, at<float>(ws, L.part_b), scale, 0, dB}};
  gj[0].drop = dp;   // dA reads D(X)
  if (grp) {
    gj[1].groups = grp->groups;
    gj[1].gr = grp->gr;
    for (int g = 0; g < kMaxGroups; ++g) gj[1].end[g] = grp->end[g];
  }
  QL_TRY(launch_lora_grads(gj, 2, M, r, s));
#undef QL_TRY
  return QLORA_OK;
}

qlora_status qlora_linear_bwd_dropout(const qlora_nf4_tensor* W, const qlora_bf16* X, int64_t M,
                                      const qlora_bf16* A, const qlora_bf16* B, int32_t r,
                                      float alpha, const qlora_dropout* drop,
                                      const uint8_t* keep_bits_in, const qlora_bf16* dY,
                                      const qlora_bf16* XA_in, qlora_bf16* dX, float* dA,
                                      float* dB, void* ws, size_t ws_bytes, void* stream) {
  return linear_bwd_impl(W, X, M, A, B, r, alpha, drop, keep_bits_in, dY, XA_in, dX, dA, dB, ws,
                         ws_bytes,
                         stream, nullptr);
}

// Grouping of a fused weight: G segments of rows ending at the running sums
// of group_rows, r adapter rows each.  False for a bad grouping.
static bool grouping(const qlora_nf4_tensor* W, int32_t r, int32_t groups,
                     const int64_t* group_rows, GradJob* g) {
  if (!W || groups < 1 || groups > kMaxGroups || !group_rows || r < 1) return false;
  if ((int64_t)groups * r > QLORA_MAX_RANK) return false;
  g->groups = groups;
  g->gr = r;
  int64_t sum = 0;
  for (int i = 0; i < groups; ++i) {
    if (group_rows[i] < 1) return false;
    sum += group_rows[i];
    g->end[i] = sum;
  }
  return sum == W->rows;
}

size_t qlora_grouped_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t r, int32_t groups) {
  if (groups < 1 || groups > kMaxGroups || (int64_t)groups * r > QLORA_MAX_RANK) return 0;
  return qlora_linear_workspace_bytes(M, N, K, groups * r);
}

qlora_status qlora_grouped_fwd(const qlora_nf4_tensor* W, const qlora_bf16* X, int64_t M,
                               const qlora_bf16* A, const qlora_bf16* B, int32_t r,
                               int32_t groups, const int64_t* group_rows, float alpha,
                               qlora_bf16* Y, qlora_bf16* XA_out, void* ws, size_t ws_bytes,
                               void* stream) {
  GradJob g{};
  if (!valid_tensor(W) || !grouping(W, r, groups, group_rows, &g)) return QLORA_ERR_INVALID_ARG;
  // rank G r with alpha G keeps every group's scale at alpha / r
  return qlora_linear_fwd_dropout(W, X, M, A, B, groups * r, alpha * (float)groups, nullptr,
                                  nullptr, Y, XA_out, ws, ws_bytes, stream);
}

qlora_status qlora_grouped_bwd(const qlora_nf4_tensor* W, const qlora_bf16* X, int64_t M,
                               const qlora_bf16* A, const qlora_bf16* B, int32_t r,
                               int32_t groups, const int64_t* group_rows, float alpha,
                               const qlora_bf16* dY, const qlora_bf16* XA_in, qlora_bf16* dX,
                               float* dA, float* dB, void* ws, size_t ws_bytes, void* stream) {
  GradJob g{};
  if (!valid_tensor(W) || !grouping(W, r, groups, group_rows, &g)) return QLORA_ERR_INVALID_ARG;
  return linear_bwd_impl(W, X, M, A, B, groups * r, alpha * (float)groups, nullptr, nullptr, dY,
                         XA_in,
                         dX, dA, dB, ws, ws_bytes, stream, &g);
}

qlora_status qlora_dropout_mask(int64_t M, int64_t K, const qlora_dropout* drop, uint8_t* out,
                                void* stream) {
  if (!drop || M < 0 || K < 0) return QLORA_ERR_INVALID_ARG;
  if (K > 0 && M > INT64_MAX / K) return QLORA_ERR_INVALID_ARG;
  if (M * K > 0 && !out) return QLORA_ERR_INVALID_ARG;
  // one thread per 4 elements, in one grid dimension
  if (M * K >= 4 * (kOff32 - 256)) return QLORA_ERR_UNSUPPORTED;
  DropoutParams dp;
  if (!dropout_params(drop, K, &dp)) return QLORA_ERR_INVALID_ARG;
  return hip_status(launch_dropout_mask(M, K, dp, out, static_cast<hipStream_t>(stream)));
}

size_t qlora_merge_workspace_bytes(int64_t rows, int64_t cols) {
  if (rows < 1 || cols < 1 || !below(rows, cols, kMaxWeights + 1)) return 0;
  if (!merge_fits(rows, cols)) return 0;
  const int64_t n = rows * cols;
  return align_up((size_t)n * sizeof(float)) + quant_layout(n).total;
}

qlora_status qlora_merge_requantize(const qlora_nf4_tensor* W, const qlora_bf16* A,
                                    const qlora_bf16* B, int32_t r, float alpha,
                                    const qlora_nf4_tensor* out, float* merged, void* ws,
                                    size_t ws_bytes, void* stream) {
  if (!valid_tensor(W) || !valid_tensor(out) || !A || !B) return QLORA_ERR_INVALID_ARG;
  if (out->rows != W->rows || out->cols != W->cols) return QLORA_ERR_INVALID_ARG;
  if (!tensor_fits(W) || !merge_fits(W->rows, W->cols)) return QLORA_ERR_UNSUPPORTED;
  if (r < 1 || r > QLORA_MAX_RANK || !std::isfinite(alpha)) return QLORA_ERR_INVALID_ARG;
  if (!aligned(A, 2) || !aligned(B, 2) || (merged && !aligned(merged, 16)))
    return QLORA_ERR_INVALID_ARG;
  const int64_t N = W->rows, K = W->cols, n = N * K;
  const QuantWs Q = quant_layout(n);
  const size_t moff = merged ? 0 : align_up((size_t)n * sizeof(float));
  if (!ws || ws_bytes < moff + Q.total || !aligned(ws, kAlign)) return QLORA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* mbuf = merged ? merged : at<float>(ws, 0);
  void* qws = at<uint8_t>(ws, moff);
  const DequantTensor d = dequant_tensor(W, mbuf);
  hipError_t e = launch_dequantize(&d, 1, 0, s);
  if (e == hipSuccess) e = launch_merge_lora_add(mbuf, N, K, A, B, r, alpha / (float)r, s);
  if (e != hipSuccess) return QLORA_ERR_HIP;
  const QuantTensor t = quant_tensor(mbuf, out, qws, Q);
  e = launch_quant_codes(&t, 1, s);
  if (e == hipSuccess) e = launch_quant_consts(&t, 1, s);
  return hip_status(e);
}

// Checks the hyperparameters and folds them into the float32 coefficients of
// step `step`, each formed in double and rounded once.
static qlora_status adam_hyper(const qlora_adamw_hparams* h, int64_t step, int32_t count,
                               bool have_tensors, AdamHyper* out) {
  if (!h || step < 1 || count < 0 || (count > 0 && !have_tensors)) return QLORA_ERR_INVALID_ARG;
  if (!(h->lr >= 0.0) || !(h->beta1 >= 0.0 && h->beta1 < 1.0) ||
      !(h->beta2 >= 0.0 && h->beta2 < 1.0) || !(h->eps > 0.0) || !(h->weight_decay >= 0.0) ||
      !std::isfinite(h->lr) || !std::isfinite(h->eps) || !std::isfinite(h->weight_decay))
    return QLORA_ERR_INVALID_ARG;
  const double lr = h->lr, b1 = h->beta1, b2 = h->beta2;
  AdamHyper hp;
  hp.decay = (float)(1.0 - lr * h->weight_decay);
  hp.b1 = (float)b1;
  hp.one_minus_b1 = (float)(1.0 - b1);
  hp.b2 = (float)b2;
  hp.one_minus_b2 = (float)(1.0 - b2);
  hp.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(1.0 - std::pow(b2, (double)step)));
  hp.eps = (float)h->eps;
  hp.step_size = (float)(lr / (1.0 - std::pow(b1, (double)step)));
  if (!(hp.eps > 0.f)) return QLORA_ERR_INVALID_ARG;   // eps below float's range
  *out = hp;
  return QLORA_OK;
}

qlora_status qlora_adamw_step(const qlora_adamw_hparams* h, int64_t step,
                              const qlora_adamw_tensor* tensors, int32_t count, void* stream) {
  AdamHyper hp;
  const qlora_status st = adam_hyper(h, step, count, tensors != nullptr, &hp);
  if (st != QLORA_OK) return st;
  for (int32_t i = 0; i < count; ++i) {
    const qlora_adamw_tensor& t = tensors[i];
    if (t.numel < 0) return QLORA_ERR_INVALID_ARG;
    if (t.numel == 0) continue;
    if (!t.param || !t.grad || !t.exp_avg || !t.exp_avg_sq) return QLORA_ERR_INVALID_ARG;
    if (!aligned(t.param, 4) || !aligned(t.grad, 4) || !aligned(t.exp_avg, 4) ||
        !aligned(t.exp_avg_sq, 4) || (t.param_bf16 && !aligned(t.param_bf16, 2)))
      return QLORA_ERR_INVALID_ARG;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int32_t i0 = 0; i0 < count; i0 += kAdamBatch) {
    AdamBatch bt{};
    bt.count = std::min(count - i0, kAdamBatch);
    bt.chunk_start[0] = 0;
    for (int j = 0; j < bt.count; ++j) {
      const qlora_adamw_tensor& t = tensors[i0 + j];
      bt.t[j] = AdamTensor{t.param, t.grad, t.exp_avg, t.exp_avg_sq,
                           reinterpret_cast<uint16_t*>(t.param_bf16), t.numel};
      bt.chunk_start[j + 1] = bt.chunk_start[j] + adamw_chunks(t.numel);
    }
    const hipError_t e = traced(QLORA_KERNEL_ADAMW, s, [&] { return launch_adamw(bt, hp, s); });
    if (e != hipSuccess) return QLORA_ERR_HIP;
  }
  return QLORA_OK;
}

qlora_status qlora_adamw8_step(const qlora_adamw_hparams* h, int64_t step,
                               const qlora_adamw8_tensor* tensors, int32_t count, void* stream) {
  AdamHyper hp;
  const qlora_status st = adam_hyper(h, step, count, tensors != nullptr, &hp);
  if (st != QLORA_OK) return st;
  for (int32_t i = 0; i < count; ++i) {
    const qlora_adamw8_tensor& t = tensors[i];
    if (t.numel < 0) return QLORA_ERR_INVALID_ARG;
    if (t.numel == 0) continue;
    if (!t.param || !t.grad || !t.exp_avg_q || !t.exp_avg_scale || !t.exp_avg_sq_q ||
        !t.exp_avg_sq_scale)
      return QLORA_ERR_INVALID_ARG;
    if (!aligned(t.param, 4) || !aligned(t.grad, 4) || !aligned(t.exp_avg_scale, 4) ||
        !aligned(t.exp_avg_sq_scale, 4) || (t.param_bf16 && !aligned(t.param_bf16, 2)))
      return QLORA_ERR_INVALID_ARG;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int32_t i0 = 0; i0 < count; i0 += kAdam8Batch) {
    Adam8Batch bt{};
    bt.count = std::min(count - i0, kAdam8Batch);
    bt.wg_start[0] = 0;
    for (int j = 0; j < bt.count; ++j) {
      const qlora_adamw8_tensor& t = tensors[i0 + j];
      bt.t[j] = Adam8Tensor{t.param, t.grad, t.exp_avg_q, t.exp_avg_scale, t.exp_avg_sq_q,
                            t.exp_avg_sq_scale, reinterpret_cast<uint16_t*>(t.param_bf16),
                            t.numel};
      bt.wg_start[j + 1] = bt.wg_start[j] + adamw8_workgroups(t.numel);
    }
    const hipError_t e = traced(QLORA_KERNEL_ADAMW8, s, [&] { return launch_adamw8(bt, hp, s); });
    if (e != hipSuccess) return QLORA_ERR_HIP;
  }
  return QLORA_OK;
}

qlora_status qlora_host_state_alloc(size_t bytes, void** ptr) {
  if (!ptr || bytes == 0) return QLORA_ERR_INVALID_ARG;
  *ptr = nullptr;
  void* p = nullptr;
  if (hipHostMalloc(&p, bytes, hipHostMallocMapped | hipHostMallocCoherent) != hipSuccess)
    return QLORA_ERR_HIP;
  void* d = nullptr;
  if (hipHostGetDevicePointer(&d, p, 0) != hipSuccess || d != p) {
    (void)hipHostFree(p);
    return QLORA_ERR_UNSUPPORTED;
  }
  *ptr = p;
  return QLORA_OK;
}

qlora_status qlora_host_state_free(void* ptr) {
  if (!ptr) return QLORA_OK;
  return hipHostFree(ptr) == hipSuccess ? QLORA_OK : QLORA_ERR_HIP;
}

qlora_status qlora_trace_begin(uint32_t kernel_mask, int32_t capacity) {
  if (kernel_mask == 0 || kernel_mask >= (1u << QLORA_KERNEL_COUNT) || capacity < 1 ||
      capacity > (1 << 20))
    return QLORA_ERR_INVALID_ARG;
  trace_release();
  for (int k = 0; k < QLORA_KERNEL_COUNT; ++k) {
    if (!((kernel_mask >> k) & 1u)) continue;
    g_trace.ev[k] = new hipEvent_t[2 * capacity];
    for (int i = 0; i < 2 * capacity; ++i) {
      if (hipEventCreate(&g_trace.ev[k][i]) != hipSuccess) {
        for (int j = 0; j < i; ++j) (void)hipEventDestroy(g_trace.ev[k][j]);
        delete[] g_trace.ev[k];
        g_trace.ev[k] = nullptr;
        trace_release();
        return QLORA_ERR_HIP;
      }
    }
  }
  g_trace.mask = kernel_mask;
  g_trace.capacity = capacity;
  return QLORA_OK;
}

qlora_status qlora_trace_pause(int32_t paused) {
  g_trace.paused = paused != 0;
  return QLORA_OK;
}

qlora_status qlora_trace_end(int32_t* launches, double* total_ms) {
  if (!launches || !total_ms) return QLORA_ERR_INVALID_ARG;
  qlora_status st = QLORA_OK;
  for (int k = 0; k < QLORA_KERNEL_COUNT; ++k) {
    launches[k] = g_trace.used[k];
    total_ms[k] = 0.0;
    for (int i = 0; i < g_trace.used[k]; ++i) {
      float ms = 0.f;
      if (hipEventSynchronize(g_trace.ev[k][2 * i + 1]) != hipSuccess ||
          hipEventElapsedTime(&ms, g_trace.ev[k][2 * i], g_trace.ev[k][2 * i + 1]) != hipSuccess) {
        st = QLORA_ERR_HIP;
        break;
      }
      total_ms[k] += ms;
    }
  }
  trace_release();
  return st;
}

}  // extern "C"
