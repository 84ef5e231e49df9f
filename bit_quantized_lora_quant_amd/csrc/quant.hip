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
// A wave takes 1024-weight chunks (grid-stride).  In load i (0..3) lane l
// reads the float4 at chunk + 256 i + 4 l, so each load instruction covers 1
// KB contiguously; the 16 lanes of a DPP row then hold exactly one 64-block,
// whose absmax is four DPP max steps.  The 4 codes of a lane leave as one
// 16-bit store (128 contiguous bytes per wave).
constexpr int kQChunk = 1024;

// Nearest-level code of x in [-1, 1] = number of thresholds below x, found
// through 256 equal buckets of [-1, 1]: bucket b holds the count of
// thresholds under its interval and the one threshold inside it (+inf if
// none), so the code is base + (x > thr).  Built per workgroup in LDS (one
// entry per thread) from the thresholds in the argument segment.
struct Bucket {
  uint32_t base;
  float thr;
};

__device__ __forceinline__ void build_buckets(Bucket* lds, const NF4Tables& tab) {
  const int b = threadIdx.x;                 // kThreads == 256 buckets
  const float lo = (float)b * (1.0f / 128.0f) - 1.0f;          // exact
  const float hi = (float)(b + 1) * (1.0f / 128.0f) - 1.0f;    // exact
  uint32_t base = 0;
  float thr = __builtin_inff();
#pragma unroll
  for (int j = 0; j < 15; ++j) {
    const float t = tab.thresh[j];
    base += t < lo ? 1u : 0u;
    if (t >= lo && t < hi) thr = t;
  }
  lds[b] = Bucket{base, thr};
}

__device__ __forceinline__ uint32_t nf4_code(float x, const Bucket* lds) {
  // 128 x is exact, so t is 128 x + 128 rounded once; x in [-1, 1] gives
  // t in [0, 256]
  const float t = __builtin_fmaf(x, 128.0f, 128.0f);
  int b = (int)t;
  b = b < 255 ? b : 255;
  const Bucket e = lds[b];
  return e.base + (x > e.thr ? 1u : 0u);
}

__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f32<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_f32<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppRowMirror>(v));
  return v;
}

__global__ __launch_bounds__(kThreads) void k_quant_absmax_nf4(const float* __restrict__ w,
                                                               int64_t n, NF4Tables tab,
                                                               uint8_t* __restrict__ codes,
                                                               float* __restrict__ absmax) {
  __shared__ Bucket buckets[256];
  build_buckets(buckets, tab);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * kThreads) >> 6;
  const int64_t nchunks = ceil_div(n, kQChunk);
  for (int64_t c = wave; c < nchunks; c += nwaves) {
    const int64_t base = c * kQChunk;
    const bool full = base + kQChunk <= n;
    float v[4][4];
    if (full) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 t = *reinterpret_cast<const float4*>(w + base + 256 * i + 4 * lane);
        v[i][0] = t.x; v[i][1] = t.y; v[i][2] = t.z; v[i][3] = t.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t idx = base + 256 * i + 4 * lane + e;
          v[i][e] = idx < n ? w[idx] : 0.0f;
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float m = fmaxf(fmaxf(fabsf(v[i][0]), fabsf(v[i][1])), fmaxf(fabsf(v[i][2]), fabsf(v[i][3])));
      const float a = row16_max(m);
      const int64_t e0 = base + 256 * i + 4 * lane;          // first element of this lane
      const int64_t blk = e0 / kBlock;
      if ((lane & 15) == 0 && e0 < n) absmax[blk] = a;
      uint32_t packed = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = (a == 0.0f) ? 0.0f : v[i][e] / a;
        packed |= nf4_code(x, buckets) << (4 * e);
      }
      if (full) {
        *reinterpret_cast<uint16_t*>(codes + (e0 >> 1)) = (uint16_t)packed;
      } else {
        // bytes holding elements (e0, e0+1) and (e0+2, e0+3); a missing odd
        // element leaves its high nibble 0
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int64_t el = e0 + 2 * k;
          if (el < n) {
            uint8_t byte = (uint8_t)(packed >> (8 * k));
            if (el + 1 >= n) byte &= 0x0F;
            codes[el >> 1] = byte;
          }
        }
      }
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

// A wave takes 2048-weight chunks (grid-stride): in sub-step i (0..3) lane l
// rebuilds the 8 weights at chunk + 512 i + 8 l from one 32-bit word of codes
// (256 contiguous bytes per load instruction, 1 KB of bf16 per store), with
// all four code loads of a chunk in flight together.
constexpr int kDqChunk = 2048;

// F32: float32 block constants (no double quantisation); a template switch,
// since a per-load choice between the two constant sources makes the
// compiler wait for each chunk's loads before the next chunk's.
template <bool BF16, bool F32>
__global__ __launch_bounds__(kThreads) void k_dequant_nf4(const uint8_t* __restrict__ codes,
                                                          const int8_t* __restrict__ q,
                                                          const float* __restrict__ scale,
                                                          const float* __restrict__ mean,
                                                          const float* __restrict__ f32,
                                                          int64_t n, NF4Tables tab,
                                                          void* __restrict__ out) {
  __shared__ float lvl[16];
  if (threadIdx.x < 16) lvl[threadIdx.x] = tab.level[threadIdx.x];
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * kThreads) >> 6;
  const int64_t nchunks = ceil_div(n, kDqChunk);
  const float mu = F32 ? 0.0f : *mean;
  for (int64_t c = wave; c < nchunks; c += nwaves) {
    const int64_t base = c * kDqChunk;
    const bool full = base + kDqChunk <= n;
    uint32_t cw[4];
    float a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t e0 = base + 512 * i + 8 * lane;
      if (full) {
        cw[i] = *reinterpret_cast<const uint32_t*>(codes + (e0 >> 1));
      } else {
        cw[i] = 0;
        for (int64_t k = 0; k < 4; ++k)
          if (e0 + 2 * k < n) cw[i] |= (uint32_t)codes[(e0 >> 1) + k] << (8 * k);
      }
      const int64_t b = (e0 < n ? e0 : n - 1) / kBlock;
      if constexpr (F32) a[i] = f32[b];
      else a[i] = absmax_recon(q, scale, mu, b);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t e0 = base + 512 * i + 8 * lane;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = lvl[(cw[i] >> (4 * e)) & 15u] * a[i];
      if (full || e0 + 8 <= n) {
        if (BF16) {
          uint4 p;
          p.x = pack_bf16x2(v[0], v[1]); p.y = pack_bf16x2(v[2], v[3]);
          p.z = pack_bf16x2(v[4], v[5]); p.w = pack_bf16x2(v[6], v[7]);
          *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + e0) = p;
        } else {
          float* o = reinterpret_cast<float*>(out) + e0;
          *reinterpret_cast<float4*>(o) = make_float4(v[0], v[1], v[2], v[3]);
          *reinterpret_cast<float4*>(o + 4) = make_float4(v[4], v[5], v[6], v[7]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (e0 + e < n) {
            if (BF16)
              reinterpret_cast<uint16_t*>(out)[e0 + e] = (uint16_t)(pack_bf16x2(v[e], 0.0f) & 0xFFFF);
            else
              reinterpret_cast<float*>(out)[e0 + e] = v[e];
          }
        }
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_absmax_recon(const int8_t* __restrict__ q,
                                                           const float* __restrict__ scale,
                                                           const float* __restrict__ mean,
                                                           const float* __restrict__ f32,
                                                           int64_t nb, float* __restrict__ out) {
  const int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (b < nb) out[b] = f32 ? f32[b] : absmax_recon(q, scale, *mean, b);
}

// Constants rebuilt into [K/64][N]: out[kb * N + n] is the constant of row n,
// column block kb (block index n * K/64 + kb).  Threads run along n so the
// stores are contiguous.

}  // namespace

// Grid-stride launches: about 32 waves per CU, fewer for small tensors.
static int64_t stream_grid(int64_t chunks) {
  const int64_t waves = chunks < 8192 ? chunks : 8192;
  return ceil_div(waves > 0 ? waves : 1, kThreads / 64);
}

hipError_t launch_quant_absmax(const float* w, int64_t n, uint8_t* codes, float* absmax,
                               int kind, hipStream_t s) {
  const NF4Tables& tab = host_tables(kind);
  if (!tab.bucket_ok) return hipErrorInvalidValue;
  return launch_kernel(k_quant_absmax_nf4, dim3((unsigned)stream_grid(ceil_div(n, kQChunk))),
                       dim3(kThreads), s, w, n, tab, codes, absmax);
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
                          const float* mean, const float* f32, int64_t n, int out_bf16,
                          void* out, int kind, hipStream_t s) {
  const dim3 grid((unsigned)stream_grid(ceil_div(n, kDqChunk)));
  const auto k = out_bf16 ? (f32 ? k_dequant_nf4<true, true> : k_dequant_nf4<true, false>)
                          : (f32 ? k_dequant_nf4<false, true> : k_dequant_nf4<false, false>);
  return launch_kernel(k, grid, dim3(kThreads), s, codes, q, scale, mean, f32, n,
                       host_tables(kind), out);
}

hipError_t launch_absmax_recon(const int8_t* q, const float* scale, const float* mean,
                               const float* f32, int64_t nb, float* out, hipStream_t s) {
  hipLaunchKernelGGL(k_absmax_recon, dim3((unsigned)ceil_div(nb, kThreads)), dim3(kThreads), 0, s,
                     q, scale, mean, f32, nb, out);
  return hipGetLastError();
}


}  // namespace qnf4
