// Launcher interface of the adapter optimiser step.
#pragma once

#include "nf4_common.h"

namespace qnf4 {

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
hipError_t launch_adamw(const AdamBatch& batch, const AdamHyper& h, hipStream_t s);

// 8-bit statistics: blocks of kStateBlock elements, m as int8 codes with a
// float32 scale max|m| / 127 per block, sqrt(v) as uint8 codes with a scale
// max sqrt(v) / 255 per block.  Tensor i covers workgroups [wg_start[i],
// wg_start[i + 1]), kAdam8Waves state blocks per workgroup.
constexpr int kStateBlock = 256;
constexpr int kAdam8Waves = 4;
struct Adam8Tensor {
  float* p;
  const float* g;
  int8_t* mq;
  float* ms;
  uint8_t* vq;
  float* vs;
  uint16_t* pb;   // nullable bf16 copy of p
  int64_t n;
};
constexpr int kAdam8Batch = 48;   // 3.5 KB of kernel arguments
struct Adam8Batch {
  int count;
  int64_t wg_start[kAdam8Batch + 1];
  Adam8Tensor t[kAdam8Batch];
};
int64_t adamw8_workgroups(int64_t n);
hipError_t launch_adamw8(const Adam8Batch& batch, const AdamHyper& h, hipStream_t s);

}  // namespace qnf4
