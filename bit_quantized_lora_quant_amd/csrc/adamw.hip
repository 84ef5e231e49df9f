// Adapter optimiser: one AdamW step over many adapter tensors in one launch.
// AdamW keeps a running mean and a running mean of the square of each
// trainable parameter's gradient ("QLoRA: Fine-Tuning a 70B on One GPU",
// section "Paged Optimizers"); the adapter training state is a float32
// master weight, a float32 gradient and the two float32 statistics ("Fine-
// Tuning Memory Requirements: Full Training vs LoRA vs QLoRA", sections
// "Where training memory goes" and "LoRA: freeze the base, train small
// adapters").  The update is Adam with decoupled weight decay, per element,
// in float32:
//
//     p <- p * (1 - lr wd)
//     m <- b1 m + (1 - b1) g
//     v <- b2 v + (1 - b2) g^2
//     p <- p - (lr / (1 - b1^t)) * m / (sqrt(v) / sqrt(1 - b2^t) + eps)
//
// with the bf16 copy of the new p (the GEMMs' adapter operand) written in
// the same pass.  The step streams 16 bytes in and 12 (+2) out per
// parameter: HBM-bound, every access 16 bytes wide, all of a thread's loads
// issued before its first update.
//
// The statistics may live in pinned host memory mapped into the device
// address space (the paged placement): the same kernel then streams them
// over the host link.
#include "optim.h"

namespace qnf4 {
namespace {

constexpr int kAdamThreads = 256;
constexpr int kAdamPer = 4;                              // float4 per thread and pass
constexpr int kAdamChunk = kAdamThreads * kAdamPer * 4;  // elements per workgroup

__device__ __forceinline__ void adam_elem(float& p, float g, float& m, float& v,
                                          const AdamHyper& h) {
  p = p * h.decay;
  m = h.b1 * m + h.one_minus_b1 * g;
  v = h.b2 * v + h.one_minus_b2 * (g * g);
  const float denom = __builtin_sqrtf(v) * h.inv_sqrt_bc2 + h.eps;
  p = p - h.step_size * (m / denom);
}

// Workgroup b takes chunk b of the batch: the tensor whose chunk range holds
// b, elements [chunk * kAdamChunk, + kAdamChunk) of it.
__global__ __launch_bounds__(kAdamThreads) void k_adamw(AdamBatch bt, AdamHyper h) {
  const int64_t b = blockIdx.x;
  int i = 0;
  while (i + 1 < bt.count && bt.chunk_start[i + 1] <= b) ++i;   // uniform
  const AdamTensor T = bt.t[i];
  const int64_t base = (b - bt.chunk_start[i]) * kAdamChunk;
  const int64_t end = base + kAdamChunk < T.n ? base + kAdamChunk : T.n;
  const bool vec = ((reinterpret_cast<uintptr_t>(T.p) | reinterpret_cast<uintptr_t>(T.g) |
                     reinterpret_cast<uintptr_t>(T.m) | reinterpret_cast<uintptr_t>(T.v)) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(T.pb) & 7) == 0;
  if (vec && end - base == kAdamChunk) {
    // whole chunk: kAdamPer float4 per thread, all loads issued first
    float4 p[kAdamPer], g[kAdamPer], m[kAdamPer], v[kAdamPer];
#pragma unroll
    for (int q = 0; q < kAdamPer; ++q) {
      const int64_t e = base + ((int64_t)q * kAdamThreads + threadIdx.x) * 4;
      p[q] = *reinterpret_cast<const float4*>(T.p + e);
      g[q] = *reinterpret_cast<const float4*>(T.g + e);
      m[q] = *reinterpret_cast<const float4*>(T.m + e);
      v[q] = *reinterpret_cast<const float4*>(T.v + e);
    }
#pragma unroll
    for (int q = 0; q < kAdamPer; ++q) {
      const int64_t e = base + ((int64_t)q * kAdamThreads + threadIdx.x) * 4;
      adam_elem(p[q].x, g[q].x, m[q].x, v[q].x, h);
      adam_elem(p[q].y, g[q].y, m[q].y, v[q].y, h);
      adam_elem(p[q].z, g[q].z, m[q].z, v[q].z, h);
      adam_elem(p[q].w, g[q].w, m[q].w, v[q].w, h);
      *reinterpret_cast<float4*>(T.p + e) = p[q];
      *reinterpret_cast<float4*>(T.m + e) = m[q];
      *reinterpret_cast<float4*>(T.v + e) = v[q];
      if (T.pb) {
        uint2 o;
        o.x = pack_bf16x2(p[q].x, p[q].y);
        o.y = pack_bf16x2(p[q].z, p[q].w);
        *reinterpret_cast<uint2*>(T.pb + e) = o;
      }
    }
    return;
  }
  // a tensor's last, partial chunk, or unaligned pointers: one element per
  // thread and pass
  for (int64_t e = base + threadIdx.x; e < end; e += kAdamThreads) {
    float p = T.p[e], m = T.m[e], v = T.v[e];
    adam_elem(p, T.g[e], m, v, h);
    T.p[e] = p;
    T.m[e] = m;
    T.v[e] = v;
    if (T.pb) T.pb[e] = (uint16_t)(pack_bf16x2(p, 0.f) & 0xFFFF);
  }
}

// ------------------------------------------------------------ 8-bit state
// The two statistics kept in 8 bits (the 8-bit paged AdamW of the training
// arguments in "Fitting a fine-tune in 16 GB"), blockwise like the method's
// own quantised block constants ("Double Quantization": 8-bit integers with
// a float32 scale per block): per block of 256 statistics,
//     m:        int8  code, scale = max|m| / 127, m = code * scale
//     sqrt(v):  uint8 code, scale = max sqrt(v) / 255, v = (code * scale)^2
// One step dequantises, applies the float32 update above (with the new
// sqrt(v) serving both the update and the new codes) and quantises again,
// code = rint(x / scale) clamped (0 for a zero scale).  One wave owns one
// block: 4 statistics per lane, the block maxima by lane exchanges (max is
// exact in any order).  Per parameter 10 bytes come in and 8 go out (with
// the bf16 copy), against 16 and 14 with float32 statistics.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
  return v;
}

__device__ __forceinline__ void adam8_elem(float& p, float g, float& m, float& u,
                                           const AdamHyper& h) {
  float v = u * u;
  p = p * h.decay;
  m = h.b1 * m + h.one_minus_b1 * g;
  v = h.b2 * v + h.one_minus_b2 * (g * g);
  u = __builtin_sqrtf(v);
  p = p - h.step_size * (m / (u * h.inv_sqrt_bc2 + h.eps));
}

__device__ __forceinline__ int code_of(float x, float s, float top, float bottom) {
  if (s == 0.0f) return 0;
  const float q = __builtin_rintf(x / s);
  return (int)fminf(fmaxf(q, bottom), top);
}

__global__ __launch_bounds__(64 * kAdam8Waves) void k_adamw8(Adam8Batch bt, AdamHyper h) {
  const int64_t b = blockIdx.x;
  int i = 0;
  while (i + 1 < bt.count && bt.wg_start[i + 1] <= b) ++i;   // uniform
  const Adam8Tensor T = bt.t[i];
  const int lane = threadIdx.x & 63;
  const int64_t blk = (b - bt.wg_start[i]) * kAdam8Waves + (threadIdx.x >> 6);
  const int64_t e0 = blk * kStateBlock;
  if (e0 >= T.n) return;                         // the tensor's last workgroup
  const int64_t e = e0 + 4 * lane;
  const float sm = T.ms[blk], su = T.vs[blk];
  float p[4], g[4], m[4], u[4];
  const bool vec = e0 + kStateBlock <= T.n &&
                   ((reinterpret_cast<uintptr_t>(T.p) | reinterpret_cast<uintptr_t>(T.g)) & 15) == 0 &&
                   ((reinterpret_cast<uintptr_t>(T.mq) | reinterpret_cast<uintptr_t>(T.vq)) & 3) == 0 &&
                   (reinterpret_cast<uintptr_t>(T.pb) & 7) == 0;
  if (vec) {
    const float4 pv = *reinterpret_cast<const float4*>(T.p + e);
    const float4 gv = *reinterpret_cast<const float4*>(T.g + e);
    const uint32_t mw = *reinterpret_cast<const uint32_t*>(T.mq + e);
    const uint32_t vw = *reinterpret_cast<const uint32_t*>(T.vq + e);
    p[0] = pv.x; p[1] = pv.y; p[2] = pv.z; p[3] = pv.w;
    g[0] = gv.x; g[1] = gv.y; g[2] = gv.z; g[3] = gv.w;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      m[k] = (float)(int8_t)((mw >> (8 * k)) & 0xFFu) * sm;
      u[k] = (float)((vw >> (8 * k)) & 0xFFu) * su;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bool in = e + k < T.n;
      p[k] = in ? T.p[e + k] : 0.0f;
      g[k] = in ? T.g[e + k] : 0.0f;
      m[k] = in ? (float)T.mq[e + k] * sm : 0.0f;
      u[k] = in ? (float)T.vq[e + k] * su : 0.0f;
    }
  }
  float am = 0.0f, au = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    adam8_elem(p[k], g[k], m[k], u[k], h);
    if (vec || e + k < T.n) {
      am = fmaxf(am, fabsf(m[k]));
      au = fmaxf(au, u[k]);
    }
  }
  const float nsm = wave_max(am) / 127.0f, nsu = wave_max(au) / 255.0f;
  if (lane == 0) {
    T.ms[blk] = nsm;
    T.vs[blk] = nsu;
  }
  uint32_t mw = 0, vw = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    mw |= ((uint32_t)(uint8_t)(int8_t)code_of(m[k], nsm, 127.0f, -127.0f)) << (8 * k);
    vw |= ((uint32_t)code_of(u[k], nsu, 255.0f, 0.0f)) << (8 * k);
  }
  if (vec) {
    *reinterpret_cast<float4*>(T.p + e) = make_float4(p[0], p[1], p[2], p[3]);
    *reinterpret_cast<uint32_t*>(T.mq + e) = mw;
    *reinterpret_cast<uint32_t*>(T.vq + e) = vw;
    if (T.pb) {
      uint2 o;
      o.x = pack_bf16x2(p[0], p[1]);
      o.y = pack_bf16x2(p[2], p[3]);
      *reinterpret_cast<uint2*>(T.pb + e) = o;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (e + k >= T.n) continue;
      T.p[e + k] = p[k];
      T.mq[e + k] = (int8_t)(mw >> (8 * k));
      T.vq[e + k] = (uint8_t)(vw >> (8 * k));
      if (T.pb) T.pb[e + k] = (uint16_t)(pack_bf16x2(p[k], 0.f) & 0xFFFF);
    }
  }
}

}  // namespace

int64_t adamw_chunks(int64_t n) { return ceil_div(n, kAdamChunk); }

int64_t adamw8_workgroups(int64_t n) { return ceil_div(n, (int64_t)kStateBlock * kAdam8Waves); }

hipError_t launch_adamw8(const Adam8Batch& bt, const AdamHyper& h, hipStream_t s) {
  const int64_t blocks = bt.wg_start[bt.count];
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF / (64 * kAdam8Waves)) return hipErrorInvalidValue;
  launch_kernel(k_adamw8, dim3((unsigned)blocks), dim3(64 * kAdam8Waves), s, bt, h);
  return hipGetLastError();
}

hipError_t launch_adamw(const AdamBatch& bt, const AdamHyper& h, hipStream_t s) {
  const int64_t blocks = bt.chunk_start[bt.count];
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  launch_kernel(k_adamw, dim3((unsigned)blocks), dim3(kAdamThreads), s, bt, h);
  return hipGetLastError();
}

}  // namespace qnf4
