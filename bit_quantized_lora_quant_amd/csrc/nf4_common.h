// Shared device helpers and the internal launcher interface of the gfx950
// NF4 + LoRA library.  Everything here is CDNA4-specific: wave64, bf16 MFMA
// (v_mfma_f32_16x16x32_bf16), DPP lane exchanges, v_cvt_pk_bf16_f32.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "philox.h"

namespace qnf4 {

// Benchmark instrumentation: when an event pair is pending, the next launch
// through launch_kernel records its own start and end into it (from the
// dispatch itself, so no extra packets sit between kernels).  Set and cleared
// by the tracer around one launcher call; process-global, single host thread.
struct PendingTiming {
  hipEvent_t start = nullptr, stop = nullptr;
};
PendingTiming& pending_timing();

template <typename... Params, typename... Args>
inline hipError_t launch_kernel_lds(void (*k)(Params...), dim3 grid, dim3 block, size_t lds,
                                    hipStream_t s, Args... args) {
  PendingTiming& t = pending_timing();
  if (t.start) {
    const hipEvent_t a = t.start, b = t.stop;
    t.start = t.stop = nullptr;
    hipExtLaunchKernelGGL(k, grid, block, (uint32_t)lds, s, a, b, 0, static_cast<Params>(args)...);
  } else {
    hipLaunchKernelGGL(k, grid, block, lds, s, static_cast<Params>(args)...);
  }
  return hipGetLastError();
}

template <typename... Params, typename... Args>
inline hipError_t launch_kernel(void (*k)(Params...), dim3 grid, dim3 block, hipStream_t s,
                                Args... args) {
  return launch_kernel_lds(k, grid, block, 0, s, args...);
}

constexpr int kBlock = 64;     // weights per first-level absmax
constexpr int kMaxRank = 128;  // largest adapter rank
constexpr int kMaxGroups = 8;  // projections fused into one grouped linear
constexpr int kDqBlock = 256;  // first-level constants per second-level scale

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// The 16 levels and the 15 decision thresholds, passed by value in the kernel
// argument segment (they land in scalar registers).  thresh[j] is the largest
// float not above the exact midpoint of level[j] and level[j+1], so
// "x > thresh[j]" is exactly "x is nearer level[j+1], ties to level[j]".
struct NF4Tables {
  float level[16];
  float thresh[15];
  int bucket_ok;   // the thresholds suit the quantiser's 256-bucket search
};

// 4-bit types: the normal-quantile table and the uniform INT4 table.
constexpr int kQuantNf4 = 0;
constexpr int kQuantInt4 = 1;
// Host-side tables of a type, built once (NF4 from the normal quantile
// function, INT4 as k / 7).
const NF4Tables& host_tables(int kind = kQuantNf4);

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};   // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

__device__ __forceinline__ f32x4_t mfma16x16x32(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// DPP lane exchanges inside a row of 16 lanes (no LDS traffic).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                             0xF, 0xF, false));
}
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // reverse each group of 8 lanes
constexpr int kDppRowMirror = 0x140;  // reverse each row of 16 lanes

// max over each aligned group of 8 lanes, result in all 8
__device__ __forceinline__ float group8_max(float v) {
  v = fmaxf(v, dpp_f32<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_f32<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  return v;
}

__host__ __device__ __forceinline__ int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

typedef __attribute__((address_space(3))) void lds_void_t;

// One LDS-DMA load (global_load_lds_dwordx4): 16 bytes per lane from `g`
// land at LDS address lds + 16 * lane.  Issued from inline asm so that the
// wait-count pass does not track it: while a compiler-visible LDS DMA is in
// flight that pass can no longer count LDS reads precisely and waits for all
// of them (lgkmcnt(0)) at every use.  The callers wait for the DMA
// themselves (vmcnt and a barrier) before the tile is read; the memory
// clobber keeps LDS reads of a stage ahead of the DMA that refills it.  An
// M0 write needs one wait state before the DMA reads it.
__device__ __forceinline__ void dma16(const void* g, const void* lds) {
  const uint32_t a = (uint32_t)(uintptr_t)(lds_void_t*)lds;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(a) : "m0", "memory");
}

// Same, 4 bytes per lane (global_load_lds_dword).
__device__ __forceinline__ void dma4(const void* g, const void* lds) {
  const uint32_t a = (uint32_t)(uintptr_t)(lds_void_t*)lds;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(g), "s"(a) : "m0", "memory");
}


// Reconstructed block constant b: one fused multiply-add, q * S + mean.
__device__ __forceinline__ float absmax_recon(const int8_t* q, const float* scale, float mu,
                                              int64_t b) {
  return __builtin_fmaf((float)q[b], scale[b / kDqBlock], mu);
}

}  // namespace qnf4
