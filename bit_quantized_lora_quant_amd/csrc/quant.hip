// Blockwise NF4 quantisation, double quantisation of the block constants,
// and dequantisation -- the HBM-bound kernels of the path.
//
// "QLoRA: Fine-Tuning a 70B on One GPU", sections "NF4 Quantization" (each
// weight goes to the closest of 16 normal-CDF levels, after blockwise scaling)
// and "Double Quantization" (the block constants are quantised again, to 8
// bits, and everything is dequantised on the fly for the matmul).
//
// Arithmetic that decides a code or a constant is IEEE float32 with round to
// nearest even (this file is built with -ffp-contract=off); the one fused
// operation is the explicit fmaf that rebuilds a constant.
#include "nf4_common.h"

namespace qnf4 {
namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------- quantise
// One thread per 8 consecutive weights, 8 threads per 64-block (an aligned
// group of 8 lanes), so the block absmax is three DPP max steps.  Loads are
// two 16-byte vectors per thread; the 8 codes leave as one 32-bit store.
__global__ __launch_bounds__(kThreads) void k_quant_absmax_nf4(const float* __restrict__ w,
                                                               int64_t n, NF4Tables tab,
                                                               uint8_t* __restrict__ codes,
                                                               float* __restrict__ absmax) {
  const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t e0 = g * 8;
  float v[8];
  if (e0 + 8 <= n) {
    const float4 a = *reinterpret_cast<const float4*>(w + e0);
    const float4 b = *reinterpret_cast<const float4*>(w + e0 + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (e0 + i < n) ? w[e0 + i] : 0.0f;
  }
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  const float a = group8_max(m);
  const int64_t blk = g >> 3;
  if ((threadIdx.x & 7) == 0 && blk * kBlock < n) absmax[blk] = a;
  if (e0 >= n) return;
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float x = (a == 0.0f) ? 0.0f : v[i] / a;
    packed |= nf4_code(x, tab) << (4 * i);
  }
  if (e0 + 8 <= n) {
    *reinterpret_cast<uint32_t*>(codes + (e0 >> 1)) = packed;
  } else {
    const int64_t cnt = n - e0;            // 1..7 elements
    for (int64_t i = 0; i < (cnt + 1) / 2; ++i) {
      uint8_t byte = (uint8_t)(packed >> (8 * i));
      if (2 * i + 1 >= cnt) byte &= 0x0F;   // missing odd element: high nibble 0
      codes[(e0 >> 1) + i] = byte;
    }
  }
}

// -------------------------------------------------------- mean of absmax
// Binary tree of adjacent-pair float64 sums over the constants padded with
// +0.0 to a power of two.  A workgroup reduces an aligned chunk of 2048
// values: 8 per thread as a local tree, then xor-butterflies of increasing
// lane distance (x + y == y + x in IEEE, so every lane holds the same tree
// node), then the four wave sums as (w0 + w1) + (w2 + w3).  Chunk sums are
// nodes of the global tree, so repeating the kernel over them until one value
// is left reproduces the whole tree.
constexpr int kTreeChunk = 2048;

__device__ __forceinline__ double shfl_xor_f64(double v, int mask) {
  return __shfl_xor(v, mask, 64);
}

template <typename InT>
__global__ __launch_bounds__(kThreads) void k_tree_sum(const InT* __restrict__ in, int64_t cnt,
                                                       double* __restrict__ out,
                                                       float* __restrict__ mean_out,
                                                       int64_t mean_count) {
  __shared__ double wave_sum[4];
  const int64_t base = (int64_t)blockIdx.x * kTreeChunk + threadIdx.x * 8;
  double v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (base + i < cnt) ? (double)in[base + i] : 0.0;
  double s01 = v[0] + v[1], s23 = v[2] + v[3], s45 = v[4] + v[5], s67 = v[6] + v[7];
  double s = (s01 + s23) + (s45 + s67);
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) s = s + shfl_xor_f64(s, d);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (lane == 0) wave_sum[wv] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    const double t = (wave_sum[0] + wave_sum[1]) + (wave_sum[2] + wave_sum[3]);
    out[blockIdx.x] = t;
    if (mean_out) *mean_out = (float)(t / (double)mean_count);
  }
}

// -------------------------------------------------- second-level constants
// One wave per 256 constants (4 per lane): deviation from the mean, wave max
// of |d|, scale = max / 127, q = clamp(rint(d / scale), +-127).
__global__ __launch_bounds__(kThreads) void k_dq_blocks(const float* __restrict__ absmax,
                                                        int64_t nb,
                                                        const float* __restrict__ mean,
                                                        int8_t* __restrict__ q,
                                                        float* __restrict__ scale) {
  const int64_t dqb = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t b0 = dqb * kDqBlock + lane * 4;
  const float mu = *mean;
  float d[4];
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    d[i] = (b0 + i < nb) ? absmax[b0 + i] - mu : 0.0f;
    m = fmaxf(m, fabsf(d[i]));
  }
#pragma unroll
  for (int dd = 1; dd < 64; dd <<= 1) m = fmaxf(m, __shfl_xor(m, dd, 64));
  if (dqb * kDqBlock >= nb) return;
  const float S = m / 127.0f;
  if (lane == 0) scale[dqb] = S;
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float r = (S == 0.0f) ? 0.0f : __builtin_rintf(d[i] / S);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    packed |= ((uint32_t)(uint8_t)(int8_t)(int)r) << (8 * i);
  }
  if (b0 + 4 <= nb) {
    *reinterpret_cast<uint32_t*>(q + b0) = packed;
  } else {
    for (int i = 0; i < 4; ++i)
      if (b0 + i < nb) q[b0 + i] = (int8_t)(packed >> (8 * i));
  }
}

// ------------------------------------------------------------- dequantise

// One thread per 8 weights (one 32-bit word of codes, all inside one block).
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_dequant_nf4(const uint8_t* __restrict__ codes,
                                                          const int8_t* __restrict__ q,
                                                          const float* __restrict__ scale,
                                                          const float* __restrict__ mean,
                                                          int64_t n, NF4Tables tab,
                                                          void* __restrict__ out) {
  __shared__ float lvl[16];
  if (threadIdx.x < 16) lvl[threadIdx.x] = tab.level[threadIdx.x];
  __syncthreads();
  const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t e0 = g * 8;
  if (e0 >= n) return;
  const float a = absmax_recon(q, scale, *mean, e0 / kBlock);
  const bool full = e0 + 8 <= n;
  uint32_t c;
  if (full) {
    c = *reinterpret_cast<const uint32_t*>(codes + (e0 >> 1));
  } else {
    c = 0;
    for (int64_t i = 0; i < (n - e0 + 1) / 2; ++i) c |= (uint32_t)codes[(e0 >> 1) + i] << (8 * i);
  }
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = lvl[(c >> (4 * i)) & 15u] * a;
  if (BF16) {
    uint16_t* o = reinterpret_cast<uint16_t*>(out) + e0;
    if (full) {
      uint4 p;
      p.x = pack_bf16x2(v[0], v[1]); p.y = pack_bf16x2(v[2], v[3]);
      p.z = pack_bf16x2(v[4], v[5]); p.w = pack_bf16x2(v[6], v[7]);
      *reinterpret_cast<uint4*>(o) = p;
    } else {
      for (int64_t i = 0; i < n - e0; ++i) o[i] = (uint16_t)(pack_bf16x2(v[i], 0.0f) & 0xFFFF);
    }
  } else {
    float* o = reinterpret_cast<float*>(out) + e0;
    if (full) {
      *reinterpret_cast<float4*>(o) = make_float4(v[0], v[1], v[2], v[3]);
      *reinterpret_cast<float4*>(o + 4) = make_float4(v[4], v[5], v[6], v[7]);
    } else {
      for (int64_t i = 0; i < n - e0; ++i) o[i] = v[i];
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_absmax_recon(const int8_t* __restrict__ q,
                                                           const float* __restrict__ scale,
                                                           const float* __restrict__ mean,
                                                           int64_t nb, float* __restrict__ out) {
  const int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (b < nb) out[b] = absmax_recon(q, scale, *mean, b);
}

// Constants rebuilt into [K/64][N]: out[kb * N + n] is the constant of row n,
// column block kb (block index n * K/64 + kb).  Threads run along n so the
// stores are contiguous.

}  // namespace

hipError_t launch_quant_absmax(const float* w, int64_t n, uint8_t* codes, float* absmax,
                               hipStream_t s) {
  const int64_t threads = ceil_div(n, 8);
  const int64_t grid = ceil_div(threads, kThreads);
  launch_kernel(k_quant_absmax_nf4, dim3((unsigned)grid), dim3(kThreads), s, w, n,
                     host_tables(), codes, absmax);
  return hipGetLastError();
}

hipError_t launch_dq(const float* absmax, int64_t nb, int8_t* q, float* scale, float* mean,
                     double* pa, double* pb, hipStream_t s) {
  // first pass over the float constants, then over float64 partials
  int64_t cnt = ceil_div(nb, kTreeChunk);
  hipLaunchKernelGGL(k_tree_sum<float>, dim3((unsigned)cnt), dim3(kThreads), 0, s, absmax, nb, pa,
                     cnt == 1 ? mean : nullptr, nb);
  double* src = pa;
  double* dst = pb;
  while (cnt > 1) {
    const int64_t next = ceil_div(cnt, kTreeChunk);
    hipLaunchKernelGGL(k_tree_sum<double>, dim3((unsigned)next), dim3(kThreads), 0, s, src, cnt,
                       dst, next == 1 ? mean : nullptr, nb);
    cnt = next;
    double* t = src; src = dst; dst = t;
  }
  const int64_t nd = ceil_div(nb, kDqBlock);
  hipLaunchKernelGGL(k_dq_blocks, dim3((unsigned)ceil_div(nd, kThreads / 64)), dim3(kThreads), 0,
                     s, absmax, nb, mean, q, scale);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* codes, const int8_t* q, const float* scale,
                          const float* mean, int64_t n, int out_bf16, void* out, hipStream_t s) {
  const int64_t grid = ceil_div(ceil_div(n, 8), kThreads);
  if (out_bf16)
    launch_kernel(k_dequant_nf4<true>, dim3((unsigned)grid), dim3(kThreads), s, codes, q,
                       scale, mean, n, host_tables(), out);
  else
    launch_kernel(k_dequant_nf4<false>, dim3((unsigned)grid), dim3(kThreads), s, codes, q,
                       scale, mean, n, host_tables(), out);
  return hipGetLastError();
}

hipError_t launch_absmax_recon(const int8_t* q, const float* scale, const float* mean, int64_t nb,
                               float* out, hipStream_t s) {
  hipLaunchKernelGGL(k_absmax_recon, dim3((unsigned)ceil_div(nb, kThreads)), dim3(kThreads), 0, s,
                     q, scale, mean, nb, out);
  return hipGetLastError();
}


}  // namespace qnf4
