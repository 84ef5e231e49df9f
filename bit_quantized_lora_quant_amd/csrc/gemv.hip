// Decode path (M <= 16 tokens): the forward streams the 4-bit weights once
// and is bound by HBM bandwidth, not by the matrix cores.  Tokens are padded
// to the 16 rows of one MFMA; each lane rebuilds bf16(level[code] * constant)
// for 32 contiguous weights of one row per step, so every weight byte is read
// once and dequantised once.  The inner dimension is split across
// workgroups to put enough loads in flight; the float32 partial sums are
// added in split order by a second small kernel, which also adds the LoRA
// branch and rounds to bf16.
#include "nf4_common.h"

namespace qnf4 {
namespace {

constexpr int kRowsPerWg = 64;   // 4 waves x 16 rows
constexpr int kKStep = 128;      // inner indices per lane-group step (4 x 32)

__device__ __forceinline__ uint4 dequant8(uint32_t c, float a, const float* lvl) {
  uint4 r;
  r.x = pack_bf16x2(lvl[c & 15u] * a, lvl[(c >> 4) & 15u] * a);
  r.y = pack_bf16x2(lvl[(c >> 8) & 15u] * a, lvl[(c >> 12) & 15u] * a);
  r.z = pack_bf16x2(lvl[(c >> 16) & 15u] * a, lvl[(c >> 20) & 15u] * a);
  r.w = pack_bf16x2(lvl[(c >> 24) & 15u] * a, lvl[(c >> 28) & 15u] * a);
  return r;
}

// partial[split][m][n] = sum over the split's inner range of X[m][k] W'[n][k]
__global__ __launch_bounds__(256) void k_qlora_gemv(const uint16_t* __restrict__ X, int64_t M,
                                                    int64_t K, const uint8_t* __restrict__ codes,
                                                    int64_t N, const float* __restrict__ ahat_t,
                                                    NF4Tables tab, int64_t kchunk,
                                                    float* __restrict__ partial) {
  __shared__ float lvl[16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int j16 = lane & 15, g = lane >> 4;
  if (tid < 16) lvl[tid] = tab.level[tid];
  __syncthreads();
  const int64_t n = (int64_t)blockIdx.x * kRowsPerWg + 16 * wv + j16;
  const int64_t nl = n < N ? n : N - 1;
  const int split = blockIdx.y;
  const int64_t kbeg = (int64_t)split * kchunk;
  int64_t kend = kbeg + kchunk;
  kend = kend < K ? kend : K;
  const bool tok = j16 < M;                      // A operand row = token j16
  const uint16_t* xrow = X + (int64_t)(tok ? j16 : 0) * K;
  const uint8_t* crow = codes + nl * (K / 2);

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int64_t k = kbeg; k < kend; k += kKStep) {
    // this lane's 32 inner indices; a final half step (K % 128 == 64) leaves
    // groups 2 and 3 idle, as zero operands (MFMA needs the whole wave)
    const int64_t kk = k + 32 * g;
    const bool in = kk < kend;
    const uint4 c = in ? *reinterpret_cast<const uint4*>(crow + kk / 2) : make_uint4(0u, 0u, 0u, 0u);
    const float a = in ? ahat_t[(kk / kBlock) * N + nl] : 0.f;
    uint4 xa[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
      xa[s] = (tok && in) ? *reinterpret_cast<const uint4*>(xrow + kk + 8 * s)
                          : make_uint4(0u, 0u, 0u, 0u);
    acc = mfma16x16x32(xa[0], dequant8(c.x, a, lvl), acc);
    acc = mfma16x16x32(xa[1], dequant8(c.y, a, lvl), acc);
    acc = mfma16x16x32(xa[2], dequant8(c.z, a, lvl), acc);
    acc = mfma16x16x32(xa[3], dequant8(c.w, a, lvl), acc);
  }
  // D[token 4g + v][row j16]
  float* base = partial + (int64_t)split * M * N;
  if (n < N) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t m = 4 * g + v;
      if (m < M) base[m * N + n] = acc[v];
    }
  }
}

// Y[m][n] = bf16( sum_split partial + sum_j xas[m][j] * B[n][j] )
__global__ __launch_bounds__(256) void k_gemv_finish(const float* __restrict__ partial,
                                                     int splits, int64_t M, int64_t N,
                                                     const uint16_t* __restrict__ xas, int r,
                                                     int r32, const uint16_t* __restrict__ B,
                                                     uint16_t* __restrict__ Y) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= M * N) return;
  const int64_t m = idx / N, n = idx % N;
  float s = 0.f;
  for (int k = 0; k < splits; ++k) s += partial[(int64_t)k * M * N + idx];
  float l = 0.f;
  for (int j = 0; j < r; ++j) l = __builtin_fmaf(bf16_to_f32(xas[m * r32 + j]), bf16_to_f32(B[n * r + j]), l);
  Y[idx] = (uint16_t)(pack_bf16x2(s + l, 0.f) & 0xFFFF);
}

}  // namespace

int gemv_splits(int64_t N, int64_t K) {
  const int64_t groups = ceil_div(N, kRowsPerWg);
  int64_t splits = ceil_div(1024, groups);
  const int64_t maxs = K / 256 > 0 ? K / 256 : 1;
  if (splits > maxs) splits = maxs;
  if (splits < 1) splits = 1;
  return (int)splits;
}

hipError_t launch_gemv(const uint16_t* X, int64_t M, int64_t K, const uint8_t* codes, int64_t N,
                       const float* ahat_t, int splits, float* partial, hipStream_t s) {
  // split boundaries on 128 so each lane-group step stays inside one split
  const int64_t kchunk = ceil_div(ceil_div(K, splits), kKStep) * kKStep;
  return launch_kernel(k_qlora_gemv, dim3((unsigned)ceil_div(N, kRowsPerWg), (unsigned)splits),
                       dim3(256), s, X, M, K, codes, N, ahat_t, host_tables(), kchunk, partial);
}

hipError_t launch_gemv_finish(const float* partial, int splits, int64_t M, int64_t N,
                              const uint16_t* xas, int r, int r32, const uint16_t* B, uint16_t* Y,
                              hipStream_t s) {
  hipLaunchKernelGGL(k_gemv_finish, dim3((unsigned)ceil_div(M * N, 256)), dim3(256), 0, s, partial,
                     splits, M, N, xas, r, r32, B, Y);
  return hipGetLastError();
}

}  // namespace qnf4
