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

// ---------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.  All pointers are device.

// kind: kQuantNf4 or kQuantInt4.  f32 (nullable): float32 block constants in
// place of the double-quantised state (q, scale and mean then unused).
hipError_t launch_quant_absmax(const float* w, int64_t n, uint8_t* codes, float* absmax,
                               int kind, hipStream_t s);
hipError_t launch_dq(const float* absmax, int64_t nb, int8_t* q, float* scale, float* mean,
                     double* partial_a, double* partial_b, hipStream_t s);
hipError_t launch_dequant(const uint8_t* codes, const int8_t* q, const float* scale,
                          const float* mean, const float* f32, int64_t n, int out_bf16,
                          void* out, int kind, hipStream_t s);
hipError_t launch_absmax_recon(const int8_t* q, const float* scale, const float* mean,
                               const float* f32, int64_t nb, float* out, hipStream_t s);

// ------------------------------------------------ side-path job launches
// Several small independent steps share one launch (each is a few
// microseconds of work; separate launches would cost more than the work).

// Reconstructed constants laid out [K/64][N]: out[kb * N + n] = â of block
// (n, kb), from the double-quantised state or (f32 non-null) the float32
// constants.
struct ReconJob {
  const int8_t* q;
  const float* scale;
  const float* mean;
  int64_t N, KB;
  float* out;
  const float* f32;
};
// bf16 transpose [rows, cols] -> [cols, ldo], zero for i in [rows, ldo)
struct TransposeJob {
  const uint16_t* in;
  int64_t rows, cols;
  uint16_t* out;
  int64_t ldo;
};
// Skinny product P = T . U^T over the inner dim kin: T [M, kin] (row stride
// ldt), U [r, kin] (row stride ldu).  The inner dim is cut into `ks` slices
// whose float32 partials [ks][M][rpad] go to `part`; the finish step adds
// them in slice order and writes (each output nullable)
//   out_s  bf16(scale * P) [M, r32]   (zero columns r..r32)
//   out    bf16(P)         [M, r]
//   out_t  bf16(P)^T       [r, ldo_t] (zero for m in [M, ldo_t))
struct SkinnyJob {
  const uint16_t* T;
  int64_t kin, ldt;
  const uint16_t* U;
  int64_t ldu;
  int ks;
  int64_t kslice;
  float* part;
  float scale;
  uint16_t* out_s;
  uint16_t* out;
  uint16_t* out_t;
  int64_t ldo_t;
  int part_only;   // write the slice partials even as a single slice
  // dropout of T (T = X only): dropped elements read as zero, sums times
  // drop.inv
  DropoutParams drop{};
};
// Padded rank of the partial rows (16, 32, 64 or 128).
int skinny_rpad(int r);
int skinny_slices(int64_t M, int64_t kin);
// Floats of `part` a job with these sizes needs.
size_t skinny_part_floats(int64_t M, int64_t kin, int r);
// Fills ks / kslice of each job from its kin.
void skinny_plan(SkinnyJob* j, int64_t M);
// Slice launch (jobs + optional recon), then the finish launch.
hipError_t launch_skinny(const SkinnyJob* jobs, int njobs, int64_t M, int r, int r32,
                         const ReconJob* recon, hipStream_t s);
// Up to two transposes and a recon in one launch.
hipError_t launch_prep(const TransposeJob* t, int nt, const ReconJob* recon, hipStream_t s);

// Adapter gradient: out = scale * sum_m T[m][p] U[j][m], T [M, P] (row stride
// P), U [r, ldu] (zero for m in [M, ldu)).  Token range cut into `splits`
// slices with float32 partials [splits][P][r]; out is [r][P] when
// `transposed`, else [P][r].
struct GradJob {
  const uint16_t* T;
  int64_t P;
  const uint16_t* U;
  int64_t ldu;
  int splits;
  float* partial;
  float scale;
  int transposed;
  float* out;
  DropoutParams drop{};   // dropout of T (T = X only), as in SkinnyJob
  // Block-diagonal output ([P][r] layout only): rows p of group g are
  // [end[g-1], end[g]) and own columns [g gr, (g+1) gr); the reduction writes
  // 0 everywhere else.  groups == 0: the whole output.
  int groups = 0;
  int gr = 0;
  int64_t end[kMaxGroups] = {};
};
int lora_grad_splits(int64_t M, int64_t P);
// Both jobs' partial launch, then both reductions.
hipError_t launch_lora_grads(const GradJob* jobs, int njobs, int64_t M, int r, hipStream_t s);

// The GEMMs split their inner loop into `splits` slices (one workgroup per
// tile and slice) when the output tiles alone cannot fill the chip; with
// splits > 1 each slice writes float32 partials [splits][M][N or K] to `part`
// and launch_split_reduce adds them in slice order into the bf16 output.
// The *_splits functions return the slice count (every slice non-empty).
int fwd_splits(int64_t M, int64_t N, int64_t K);
int dx_splits(int64_t M, int64_t N, int64_t K);
hipError_t launch_fwd_gemm(const uint16_t* X, int64_t M, int64_t K, const uint8_t* codes,
                           int64_t N, const float* ahat_t, const uint16_t* xas, const uint16_t* B,
                           int r, int r32, uint16_t* Y, int splits, float* part, int kind,
                           hipStream_t s);
// drop (nullable): the LoRA term of dX passes through the dropout of X,
// dX = dY . W' + keep / (1 - p) * (s.G . A), element by element.
hipError_t launch_dx_gemm(const uint16_t* dY, int64_t M, int64_t N, const uint8_t* codes,
                          int64_t K, const float* ahat_t, const uint16_t* gs, const uint16_t* A,
                          int r, int r32, uint16_t* dX, int splits, float* part, int kind,
                          const DropoutParams* drop, hipStream_t s);
// keep flags (1 kept, 0 dropped) of the M x K elements of X
hipError_t launch_dropout_mask(int64_t M, int64_t K, const DropoutParams& d, uint8_t* out,
                               hipStream_t s);
hipError_t launch_split_reduce(const float* part, int splits, int64_t count, uint16_t* out,
                               hipStream_t s);

// decode path (M <= 16): weight streaming with the block constants rebuilt
// in registers, plus the LoRA down-projection slices, then one finish launch
// (split sum + LoRA up-projection + bf16).  partial: [splits][M][N] floats;
// xa_part: [decode_xa_slices(K)][M][skinny_rpad(r)] floats.
struct NF4Ref {
  const uint8_t* codes;
  const int8_t* q;
  const float* scale;
  const float* mean;
  const float* f32;   // float32 block constants in place of q/scale/mean
  int kind;           // kQuantNf4 or kQuantInt4
};
int gemv_splits(int64_t N, int64_t K);
int decode_xa_slices(int64_t K);
hipError_t launch_decode(const uint16_t* X, int64_t M, int64_t K, const NF4Ref& W, int64_t N,
                         const uint16_t* A, const uint16_t* B, int r, float scale, int splits,
                         float* partial, float* xa_part, uint16_t* Y, uint16_t* XA_out,
                         const DropoutParams& drop, hipStream_t s);

// ------------------------------------------------------------ optimiser
// One AdamW step over up to kAdamBatch tensors per launch (the batch travels
// by value in the kernel arguments).  Tensor i covers workgroups
// [chunk_start[i], chunk_start[i + 1]).  Hyperparameters are folded on the
// host in double: decay = 1 - lr wd, step_size = lr / (1 - b1^t),
// inv_sqrt_bc2 = 1 / sqrt(1 - b2^t).
struct AdamTensor {
  float* p;
  const float* g;
  float* m;
  float* v;
  uint16_t* pb;   // nullable bf16 copy of p
  int64_t n;
};
constexpr int kAdamBatch = 64;   // 3.6 KB of kernel arguments
struct AdamBatch {
  int count;
  int64_t chunk_start[kAdamBatch + 1];
  AdamTensor t[kAdamBatch];
};
struct AdamHyper {
  float decay, b1, one_minus_b1, b2, one_minus_b2, inv_sqrt_bc2, eps, step_size;
};
int64_t adamw_chunks(int64_t n);
// merged[n][k] += s * sum_j B[n][j] A[j][k] (float32, j in order, fused
// multiply-add per term), merged [N, K] float32, A [r, K], B [N, r] bf16
hipError_t launch_merge_lora_add(float* merged, int64_t N, int64_t K, const uint16_t* A,
                                 const uint16_t* B, int r, float scale, hipStream_t s);
// whether the merge launch's grid can cover an N x K weight
bool merge_fits(int64_t N, int64_t K);
hipError_t launch_adamw(const AdamBatch& batch, const AdamHyper& h, hipStream_t s);

}  // namespace qnf4
