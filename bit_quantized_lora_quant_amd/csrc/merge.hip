// Adapter merge for deployment: the trained adapter pair folds into the
// frozen weight, W_merged = W' + s . B . A (s = alpha / r), which is then
// quantised again to the 4-bit format.  LoRA's adapters are a low-rank update
// of the weight beside it ("Fine-Tuning Memory Requirements: Full Training vs
// LoRA vs QLoRA", section "LoRA: freeze the base, train small adapters"), so
// the merged weight alone reproduces the adapted layer.
//
// W' comes from the dequantisation kernel (bit-exact); this kernel adds the
// low-rank product in place:
//     merged[n][k] = fl32(merged[n][k] + fl32(s * p)),
//     p = B[n][0] A[0][k] + ... + B[n][r-1] A[r-1][k]
// accumulated in float32 in j order with one fused multiply-add per term
// (the bf16 products are exact in float32).  The r-wide inner products are
// tiny next to the weight's traffic (2 N K r flop against 8 N K bytes), so
// they run on the vector ALUs from LDS.
#include "launch.h"

namespace qnf4 {
namespace {

constexpr int kMergeCols = 256;   // columns k per workgroup (one per thread)
constexpr int kMergeRows = 16;    // rows n per workgroup
constexpr int kMergeJ = 32;       // adapter rows of A staged per pass

// Workgroup (row tile, column tile): B[n0 .. n0+15, :] and, 32 adapter rows
// at a time, A[j0 .. j0+31, k0 .. k0+255] staged in LDS as float32 (40 KB);
// thread t owns column k0 + t of the 16 rows.
__global__ __launch_bounds__(kMergeCols) void k_merge_lora_add(
    float* __restrict__ merged, int64_t N, int64_t K, const uint16_t* __restrict__ A,
    const uint16_t* __restrict__ B, int r, float scale) {
  __shared__ float As[kMergeJ][kMergeCols];
  __shared__ float Bs[kMergeRows][kMaxRank];
  const int t = threadIdx.x;
  const int64_t ktiles = ceil_div(K, kMergeCols);
  const int64_t n0 = (blockIdx.x / ktiles) * kMergeRows;
  const int64_t k0 = (blockIdx.x % ktiles) * kMergeCols;
  const int64_t k = k0 + t;
  for (int i = t; i < kMergeRows * r; i += kMergeCols) {
    const int64_t n = n0 + i / r;
    Bs[i / r][i % r] = n < N ? bf16_to_f32(B[n * r + (i % r)]) : 0.f;
  }
  float p[kMergeRows];
#pragma unroll
  for (int i = 0; i < kMergeRows; ++i) p[i] = 0.f;
  for (int j0 = 0; j0 < r; j0 += kMergeJ) {
    const int jn = r - j0 < kMergeJ ? r - j0 : kMergeJ;
    __syncthreads();   // the previous pass's reads are done
    for (int j = 0; j < jn; ++j)
      As[j][t] = k < K ? bf16_to_f32(A[(int64_t)(j0 + j) * K + k]) : 0.f;
    __syncthreads();
    for (int j = 0; j < jn; ++j) {
      const float a = As[j][t];
#pragma unroll
      for (int i = 0; i < kMergeRows; ++i) p[i] = __builtin_fmaf(Bs[i][j0 + j], a, p[i]);
    }
  }
  if (k >= K) return;
#pragma unroll
  for (int i = 0; i < kMergeRows; ++i) {
    const int64_t n = n0 + i;
    if (n < N) merged[n * K + k] = merged[n * K + k] + scale * p[i];
  }
}

}  // namespace

bool merge_fits(int64_t N, int64_t K) {
  // one grid dimension: fewer than 2^32 threads
  const int64_t rows = ceil_div(N, kMergeRows), cols = ceil_div(K, kMergeCols);
  return rows <= (((int64_t)1 << 32) / kMergeCols - 1) / cols;
}

hipError_t launch_merge_lora_add(float* merged, int64_t N, int64_t K, const uint16_t* A,
                                 const uint16_t* B, int r, float scale, hipStream_t s) {
  const int64_t blocks = ceil_div(N, kMergeRows) * ceil_div(K, kMergeCols);
  if (!merge_fits(N, K)) return hipErrorInvalidValue;
  if (r < 1 || r > kMaxRank) return hipErrorInvalidValue;
  launch_kernel(k_merge_lora_add, dim3((unsigned)blocks), dim3(kMergeCols), s, merged, N, K, A,
                B, r, scale);
  return hipGetLastError();
}

}  // namespace qnf4
