// Internal launcher interface of the library: one declaration per launch
// sequence, with the job descriptors of the side-path launches.  Device
// helpers are in nf4_common.h; the optimiser's launcher is in optim.h.
#pragma once

#include "nf4_common.h"

namespace qnf4 {

// ---------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.  All pointers are device.

// The quantiser and dequantiser take up to kQuantBatch tensors per launch
// (kernel-argument arrays).
constexpr int kQuantBatch = 32;

// One tensor to quantise.  kind: kQuantNf4 or kQuantInt4.  absmax receives
// the exact block constants (the stored float32 constants when q is null,
// i.e. without double quantisation; else scratch of nb floats).  With double
// quantisation, pa and pb hold the mean tree's float64 partials: at least
// ceil(nb / 2048) and ceil(nb / 2048^2) values.
struct QuantTensor {
  const float* w;
  int64_t n;
  int kind;
  uint8_t* codes;
  float* absmax;
  int8_t* q;        // null: no second level (scale, mean, pa, pb unused)
  float* scale;
  float* mean;
  double* pa;
  double* pb;
};
// Codes and exact absmax of count tensors, one launch.
hipError_t launch_quant_codes(const QuantTensor* t, int count, hipStream_t s);
// Mean tree (one launch per level) and second-level constants (one launch)
// of the tensors with double quantisation, after launch_quant_codes.
hipError_t launch_quant_consts(const QuantTensor* t, int count, hipStream_t s);

// One tensor to dequantise; f32 (nullable): float32 block constants in place
// of the double-quantised state (q, scale and mean then unused).  All tensors
// of one launch have f32 set, or none has.
struct DequantTensor {
  const uint8_t* codes;
  const int8_t* q;
  const float* scale;
  const float* mean;
  const float* f32;
  int64_t n;
  int kind;
  void* out;
};
hipError_t launch_dequantize(const DequantTensor* t, int count, int out_bf16, hipStream_t s);
// The quantiser's allocation-free scratch on the current device: its size,
// and its device address (looked up once per device).
size_t quant_scratch_bytes();
hipError_t quant_scratch(void** ptr);
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
  int staged = 0;  // set by skinny_plan: LDS-staged kernel (ranks 17..64)
  // dropout of T (T = X only): dropped elements read as zero, sums times
  // drop.inv
  DropoutParams drop{};
};
// Padded rank of the partial rows (16, 32, 64 or 128).
int skinny_rpad(int r);
int skinny_slices(int64_t M, int64_t kin, int r);
// Floats of `part` a job with these sizes needs.
size_t skinny_part_floats(int64_t M, int64_t kin, int r);
// Fills ks / kslice of each job from its kin.
void skinny_plan(SkinnyJob* j, int64_t M, int r);
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
// One linear of a forward GEMM launch: X [M, K], the 4-bit codes and the
// reconstructed constants [K/64][N] of W, bf16(s XA) [M, r32], B [N, r],
// Y [M, N].  A launch takes one linear, or two with one M, K, rank and table
// kind (and no split), the second's column tiles after the first's.
struct FwdGemmJob {
  const uint16_t* X;
  const uint8_t* codes;
  int64_t N;
  const float* ahat_t;
  const uint16_t* xas;
  const uint16_t* B;
  uint16_t* Y;
};
hipError_t launch_fwd_gemm(const FwdGemmJob* jobs, int count, int64_t M, int64_t K, int r,
                           int r32, int splits, float* part, int kind, hipStream_t s);
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
// One linear of a decode launch: partial holds gemv_splits(N, K) x M x N
// floats, xa_part decode_xa_slices(K) x M x skinny_rpad(r).
struct DecodeJob {
  const uint16_t* X;
  int64_t K;
  NF4Ref W;
  int64_t N;
  const uint16_t* A;
  const uint16_t* B;
  float* partial;
  float* xa_part;
  uint16_t* Y;
  uint16_t* XA_out;
  DropoutParams drop;
};
// Independent linears with one M and rank per launch pair (streaming, then
// finish); count <= kDecodeBatch.
constexpr int kDecodeBatch = 8;
hipError_t launch_decode(const DecodeJob* jobs, int count, int64_t M, int r, float scale,
                         hipStream_t s);

// merged[n][k] += s * sum_j B[n][j] A[j][k] (float32, j in order, fused
// multiply-add per term), merged [N, K] float32, A [r, K], B [N, r] bf16
hipError_t launch_merge_lora_add(float* merged, int64_t N, int64_t K, const uint16_t* A,
                                 const uint16_t* B, int r, float scale, hipStream_t s);
// whether the merge launch's grid can cover an N x K weight
bool merge_fits(int64_t N, int64_t K);

}  // namespace qnf4
