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

}  // namespace

int64_t adamw_chunks(int64_t n) { return ceil_div(n, kAdamChunk); }

hipError_t launch_adamw(const AdamBatch& bt, const AdamHyper& h, hipStream_t s) {
  const int64_t blocks = bt.chunk_start[bt.count];
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  launch_kernel(k_adamw, dim3((unsigned)blocks), dim3(kAdamThreads), s, bt, h);
  return hipGetLastError();
}

}  // namespace qnf4
