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
#include <cstring>
#include <mutex>

#include "launch.h"

namespace qnf4 {
namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------- quantise
// A wave takes 2048-weight chunks (grid-stride).  In load i (0..7) lane l
// reads the float4 at chunk + 256 i + 4 l, so each load instruction covers 1
// KB contiguously and a lane has eight 16-byte loads in flight (2% faster
// than four); the 16 lanes of a DPP row then hold exactly one 64-block,
// whose absmax is four DPP max steps.  In a whole chunk the 4 codes of a
// lane and load go to a per-wave LDS stage, and the chunk's 1 KB of codes
// leaves as one non-temporal 16-byte store per lane (3% faster than sixteen-
// bit stores straight from the coding loop); its 32 block constants leave as
// one 4-byte store on 32 lanes.  A ragged chunk stores element by element.
constexpr int kQChunk = 2048;

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

// Job lookup in a batched launch: first[j] is the first work item of job j
// in the launch's item space (first[0] = 0, first[count] = all items).  The
// item is wave-uniform, so the search runs on scalar loads of the kernel
// arguments.
__device__ __forceinline__ int job_of(const int64_t* first, int count, int64_t item) {
  int lo = 0, hi = count - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (first[mid] <= item) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Up to kQuantBatch tensors share a launch: the 2048-weight chunks of all of
// them form one grid-stride space, so small tensors cost no launch of their
// own.
struct QuantJob {
  const float* w;
  uint8_t* codes;
  float* absmax;
  int64_t n;
  int kind;
};
struct QuantBatch {
  QuantJob job[kQuantBatch];
  int64_t first[kQuantBatch + 1];   // first chunk of each tensor
  int count;
  NF4Tables tab[2];                 // by kind
};

__global__ __launch_bounds__(kThreads) void k_quant_absmax_nf4(const QuantBatch b) {
  __shared__ Bucket buckets[2][256];
  // per wave: the chunk's codes and block constants, staged so that they
  // leave as one 16-byte store per lane and one 4-byte store per lane
  __shared__ __attribute__((aligned(16))) uint8_t cstage[kThreads / 64][kQChunk / 2];
  __shared__ float astage[kThreads / 64][kQChunk / kBlock];
  build_buckets(buckets[0], b.tab[0]);
  build_buckets(buckets[1], b.tab[1]);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wi = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint8_t* const cst = cstage[wi];
  float* const ast = astage[wi];
  const int64_t wave = (int64_t)blockIdx.x * (kThreads / 64) + wi;
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);
  const int64_t total = b.first[b.count];
  int j = 0;
  for (int64_t c = wave; c < total; c += nwaves) {
    while (c >= b.first[j + 1]) ++j;       // chunks ascend, so the job index only grows
    const float* __restrict__ w = b.job[j].w;
    uint8_t* __restrict__ codes = b.job[j].codes;
    float* __restrict__ absmax = b.job[j].absmax;
    const int64_t n = b.job[j].n;
    const Bucket* __restrict__ bk = buckets[b.job[j].kind];
    const int64_t base = (c - b.first[j]) * kQChunk;
    const bool full = base + kQChunk <= n;
    float v[8][4];
    if (full) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // read once: nontemporal, so the stream does not displace cached lines
        const f32x4_t t = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4_t*>(w + base + 256 * i + 4 * lane));
        v[i][0] = t.x; v[i][1] = t.y; v[i][2] = t.z; v[i][3] = t.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t idx = base + 256 * i + 4 * lane + e;
          v[i][e] = idx < n ? w[idx] : 0.0f;
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float m = fmaxf(fmaxf(fabsf(v[i][0]), fabsf(v[i][1])), fmaxf(fabsf(v[i][2]), fabsf(v[i][3])));
      const float a = row16_max(m);
      const int64_t e0 = base + 256 * i + 4 * lane;          // first element of this lane
      const int64_t blk = e0 / kBlock;
      if ((lane & 15) == 0) {
        if (full) ast[4 * i + (lane >> 4)] = a;
        else if (e0 < n) absmax[blk] = a;
      }
      uint32_t packed = 0;
      // x = w / a, correctly rounded.  When every block of the wave has its
      // absmax in [2^-60, 2^60] (or 0): one IEEE reciprocal r = 1/a per block
      // and, per weight, q0 = w r corrected by its residual, fma(w - q0 a, r,
      // q0) -- the correctly rounded quotient by Markstein's theorem (r within
      // half an ulp of 1/a, q0 within an ulp of w/a, the residual exact).  The
      // range keeps r and the residual normal for every quotient of magnitude
      // 2^-20 or more; smaller ones fall in the zero level's interval of both
      // tables, whatever their last bits.  Otherwise the IEEE division.
      const bool tame = a == 0.0f || (a >= 0x1p-60f && a <= 0x1p60f);
      if (__all(tame)) {
        const float r = a == 0.0f ? 0.0f : 1.0f / a;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float q0 = v[i][e] * r;
          const float x = __builtin_fmaf(__builtin_fmaf(-q0, a, v[i][e]), r, q0);
          packed |= nf4_code(x, bk) << (4 * e);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = (a == 0.0f) ? 0.0f : v[i][e] / a;
          packed |= nf4_code(x, bk) << (4 * e);
        }
      }
      if (full) {
        *reinterpret_cast<uint16_t*>(cst + 128 * i + 2 * lane) = (uint16_t)packed;
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
    if (full) {
      // lane l stores bytes 16 l .. 16 l + 15 of the chunk's codes, and lanes
      // 0..31 its 32 block constants (the stage is this wave's own)
      __builtin_amdgcn_wave_barrier();
      const uint4 o = *reinterpret_cast<const uint4*>(cst + 16 * lane);
      __builtin_nontemporal_store(u32x4_t{o.x, o.y, o.z, o.w},
                                  reinterpret_cast<u32x4_t*>(codes + (base >> 1) + 16 * lane));
      if (lane < kQChunk / kBlock) absmax[base / kBlock + lane] = ast[lane];
      __builtin_amdgcn_wave_barrier();
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

// One tree level of several tensors in one launch: a workgroup per chunk.
struct TreeJob {
  const void* in;     // float constants (first level) or float64 partials
  int64_t cnt;
  double* out;        // one sum per chunk
  float* mean;        // non-null on the level that leaves one value
  int64_t mean_count;
};
struct TreeBatch {
  TreeJob job[kQuantBatch];
  int64_t first[kQuantBatch + 1];   // first chunk of each tensor
  int count;
};

template <typename InT>
__global__ __launch_bounds__(kThreads) void k_tree_sum(const TreeBatch b) {
  __shared__ double wave_sum[4];
  const int j = job_of(b.first, b.count, blockIdx.x);
  const InT* __restrict__ in = static_cast<const InT*>(b.job[j].in);
  const int64_t cnt = b.job[j].cnt;
  const int64_t chunk = (int64_t)blockIdx.x - b.first[j];
  const int64_t base = chunk * kTreeChunk + threadIdx.x * 8;
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
    b.job[j].out[chunk] = t;
    if (b.job[j].mean) *b.job[j].mean = (float)(t / (double)b.job[j].mean_count);
  }
}

// -------------------------------------------------- second-level constants
// One wave per 256 constants (4 per lane): deviation from the mean, wave max
// of |d|, scale = max / 127, q = clamp(rint(d / scale), +-127).
struct DqJob {
  const float* absmax;
  int64_t nb;
  const float* mean;
  int8_t* q;
  float* scale;
};
struct DqBatch {
  DqJob job[kQuantBatch];
  int64_t first[kQuantBatch + 1];   // first 256-constant block of each tensor
  int count;
};

__global__ __launch_bounds__(kThreads) void k_dq_blocks(const DqBatch b) {
  const int64_t item =
      (int64_t)blockIdx.x * (kThreads / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (item >= b.first[b.count]) return;            // whole waves only
  const int j = job_of(b.first, b.count, item);
  const float* __restrict__ absmax = b.job[j].absmax;
  const int64_t nb = b.job[j].nb;
  int8_t* __restrict__ q = b.job[j].q;
  const int64_t dqb = item - b.first[j];
  const int lane = threadIdx.x & 63;
  const int64_t b0 = dqb * kDqBlock + lane * 4;
  const float mu = *b.job[j].mean;
  float d[4];
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    d[i] = (b0 + i < nb) ? absmax[b0 + i] - mu : 0.0f;
    m = fmaxf(m, fabsf(d[i]));
  }
#pragma unroll
  for (int dd = 1; dd < 64; dd <<= 1) m = fmaxf(m, __shfl_xor(m, dd, 64));
  const float S = m / 127.0f;
  if (lane == 0) b.job[j].scale[dqb] = S;
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

// A wave takes 4096-weight chunks (grid-stride): in sub-step i (0..7) lane l
// rebuilds the 8 weights at chunk + 512 i + 8 l from one 32-bit word of codes
// (256 contiguous bytes per load instruction, 1 KB of bf16 per store), with
// all eight code loads of a chunk in flight together (4% faster than four).
constexpr int kDqChunk = 4096;

// F32: float32 block constants (no double quantisation); a template switch,
// since a per-load choice between the two constant sources makes the
// compiler wait for each chunk's loads before the next chunk's.
struct DeqJob {
  const uint8_t* codes;
  const int8_t* q;
  const float* scale;
  const float* mean;
  const float* f32;
  void* out;
  int64_t n;
  int kind;
};
struct DeqBatch {
  DeqJob job[kQuantBatch];
  int64_t first[kQuantBatch + 1];   // first 4096-weight chunk of each tensor
  int count;
  float level[2][16];               // by kind
};

template <bool BF16, bool F32>
__global__ __launch_bounds__(kThreads) void k_dequant_nf4(const DeqBatch b) {
  __shared__ float lvl[2][16];
  if (threadIdx.x < 32) lvl[threadIdx.x >> 4][threadIdx.x & 15] = b.level[threadIdx.x >> 4][threadIdx.x & 15];
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t wave =
      (int64_t)blockIdx.x * (kThreads / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);
  const int64_t total = b.first[b.count];
  int j = 0;
  for (int64_t c = wave; c < total; c += nwaves) {
    while (c >= b.first[j + 1]) ++j;       // chunks ascend, so the job index only grows
    const uint8_t* __restrict__ codes = b.job[j].codes;
    const int8_t* __restrict__ q = b.job[j].q;
    const float* __restrict__ scale = b.job[j].scale;
    const float* __restrict__ f32 = b.job[j].f32;
    void* __restrict__ out = b.job[j].out;
    const int64_t n = b.job[j].n;
    const float* __restrict__ tl = lvl[b.job[j].kind];
    const float mu = F32 ? 0.0f : *b.job[j].mean;
    const int64_t base = (c - b.first[j]) * kDqChunk;
    const bool full = base + kDqChunk <= n;
    uint32_t cw[8];
    float a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t e0 = base + 512 * i + 8 * lane;
      if (full) {
        cw[i] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(codes + (e0 >> 1)));
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
    for (int i = 0; i < 8; ++i) {
      const int64_t e0 = base + 512 * i + 8 * lane;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = tl[(cw[i] >> (4 * e)) & 15u] * a[i];
      if (full || e0 + 8 <= n) {
        if (BF16) {
          uint4 p;
          p.x = pack_bf16x2(v[0], v[1]); p.y = pack_bf16x2(v[2], v[3]);
          p.z = pack_bf16x2(v[4], v[5]); p.w = pack_bf16x2(v[6], v[7]);
          // written once: nontemporal stores
          const u32x4_t pv = {p.x, p.y, p.z, p.w};
          __builtin_nontemporal_store(pv, reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(out) + e0));
        } else {
          float* o = reinterpret_cast<float*>(out) + e0;
          f32x4_t o0 = {v[0], v[1], v[2], v[3]}, o1 = {v[4], v[5], v[6], v[7]};
          __builtin_nontemporal_store(o0, reinterpret_cast<f32x4_t*>(o));
          __builtin_nontemporal_store(o1, reinterpret_cast<f32x4_t*>(o + 4));
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

// ------------------------------------------------- allocation-free scratch
// The quantiser's scratch (the exact block absmax and the mean tree's
// float64 partials) for callers that cannot allocate: one file-scope device
// array, which each GPU the library runs on holds until the process ends.
// Host code uses only the device address hipGetSymbolAddress gives for the
// current device (the array's name is a host-side stand-in).
namespace {
constexpr size_t kQuantScratchBytes = (32u << 20) + (64u << 10);
__device__ __align__(256) uint8_t scratch[kQuantScratchBytes];
}  // namespace

size_t quant_scratch_bytes() { return kQuantScratchBytes; }

hipError_t quant_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static void* addr[kMaxDevices] = {};
  static std::mutex lock;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(lock);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

// Grid-stride launches: up to 128 waves per CU (four times the resident
// waves, so the tail of the pass is spread thin), fewer for small tensors.
static int64_t stream_grid(int64_t chunks) {
  const int64_t waves = chunks < 32768 ? chunks : 32768;
  return ceil_div(waves > 0 ? waves : 1, kThreads / 64);
}

hipError_t launch_quant_codes(const QuantTensor* t, int count, hipStream_t s) {
  if (count < 1 || count > kQuantBatch) return hipErrorInvalidValue;
  QuantBatch b{};
  b.tab[kQuantNf4] = host_tables(kQuantNf4);
  b.tab[kQuantInt4] = host_tables(kQuantInt4);
  int64_t chunks = 0;
  for (int i = 0; i < count; ++i) {
    if (!host_tables(t[i].kind).bucket_ok) return hipErrorInvalidValue;
    b.job[i] = QuantJob{t[i].w, t[i].codes, t[i].absmax, t[i].n, t[i].kind};
    b.first[i] = chunks;
    chunks += ceil_div(t[i].n, kQChunk);
  }
  b.first[count] = chunks;
  b.count = count;
  return launch_kernel(k_quant_absmax_nf4, dim3((unsigned)stream_grid(chunks)), dim3(kThreads),
                       s, b);
}

hipError_t launch_quant_consts(const QuantTensor* t, int count, hipStream_t s) {
  if (count < 0 || count > kQuantBatch) return hipErrorInvalidValue;
  // the mean tree, one launch per level: the first over the float constants,
  // the next over the float64 partials of the tensors that still have more
  // than one (each level's input and output alternate between pa and pb)
  int64_t cur[kQuantBatch];
  for (int i = 0; i < count; ++i) cur[i] = t[i].q ? ceil_div(t[i].n, (int64_t)kBlock) : 0;
  for (int level = 0;; ++level) {
    TreeBatch b{};
    int m = 0;
    int64_t chunks = 0;
    for (int i = 0; i < count; ++i) {
      if (!t[i].q || (level > 0 && cur[i] <= 1)) continue;
      const int64_t next = ceil_div(cur[i], kTreeChunk);
      const void* in = level == 0 ? static_cast<const void*>(t[i].absmax)
                                  : (level & 1 ? t[i].pa : t[i].pb);
      double* out = level & 1 ? t[i].pb : t[i].pa;
      b.job[m] = TreeJob{in, cur[i], out, next == 1 ? t[i].mean : nullptr,
                         ceil_div(t[i].n, (int64_t)kBlock)};
      b.first[m++] = chunks;
      chunks += next;
      cur[i] = next;
    }
    if (m == 0) break;
    b.first[m] = chunks;
    b.count = m;
    hipError_t e = level == 0
        ? launch_kernel(k_tree_sum<float>, dim3((unsigned)chunks), dim3(kThreads), s, b)
        : launch_kernel(k_tree_sum<double>, dim3((unsigned)chunks), dim3(kThreads), s, b);
    if (e != hipSuccess) return e;
  }
  // second-level constants: a wave per 256 constants
  DqBatch b{};
  int m = 0;
  int64_t items = 0;
  for (int i = 0; i < count; ++i) {
    if (!t[i].q) continue;
    const int64_t nb = ceil_div(t[i].n, (int64_t)kBlock);
    b.job[m] = DqJob{t[i].absmax, nb, t[i].mean, t[i].q, t[i].scale};
    b.first[m++] = items;
    items += ceil_div(nb, kDqBlock);
  }
  if (m == 0) return hipSuccess;
  b.first[m] = items;
  b.count = m;
  return launch_kernel(k_dq_blocks, dim3((unsigned)ceil_div(items, kThreads / 64)),
                       dim3(kThreads), s, b);
}

hipError_t launch_dequantize(const DequantTensor* t, int count, int out_bf16, hipStream_t s) {
  if (count < 1 || count > kQuantBatch) return hipErrorInvalidValue;
  const bool f32 = t[0].f32 != nullptr;
  DeqBatch b{};
  std::memcpy(b.level[kQuantNf4], host_tables(kQuantNf4).level, sizeof(b.level[0]));
  std::memcpy(b.level[kQuantInt4], host_tables(kQuantInt4).level, sizeof(b.level[0]));
  int64_t chunks = 0;
  for (int i = 0; i < count; ++i) {
    if ((t[i].f32 != nullptr) != f32) return hipErrorInvalidValue;
    b.job[i] = DeqJob{t[i].codes, t[i].q, t[i].scale, t[i].mean, t[i].f32, t[i].out, t[i].n,
                      t[i].kind};
    b.first[i] = chunks;
    chunks += ceil_div(t[i].n, kDqChunk);
  }
  b.first[count] = chunks;
  b.count = count;
  const dim3 grid((unsigned)stream_grid(chunks));
  const auto k = out_bf16 ? (f32 ? k_dequant_nf4<true, true> : k_dequant_nf4<true, false>)
                          : (f32 ? k_dequant_nf4<false, true> : k_dequant_nf4<false, false>);
  return launch_kernel(k, grid, dim3(kThreads), s, b);
}

hipError_t launch_absmax_recon(const int8_t* q, const float* scale, const float* mean,
                               const float* f32, int64_t nb, float* out, hipStream_t s) {
  hipLaunchKernelGGL(k_absmax_recon, dim3((unsigned)ceil_div(nb, kThreads)), dim3(kThreads), 0, s,
                     q, scale, mean, f32, nb, out);
  return hipGetLastError();
}


}  // namespace qnf4
