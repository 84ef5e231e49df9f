// The low-rank side path: skinny products against the adapters and the
// adapter gradients.  LoRA pairs a down-projection A [r, K] with an
// up-projection B [N, r] beside the frozen weight (xingyuzhitong guide,
// section "LoRA: freeze the base, train small adapters"; r and lora_alpha are
// the PEFT knobs of "QLoRA: Fine-Tuning a 70B on One GPU", section "Practical
// Implementation").  All contractions run on v_mfma_f32_16x16x32_bf16 with
// float32 accumulation; reductions over tokens use a fixed split and a fixed
// summation order, so results repeat bit for bit.
#include "nf4_common.h"

namespace qnf4 {
namespace {

__device__ __forceinline__ uint4 load8_bf16(const uint16_t* __restrict__ p, int64_t idx,
                                            int64_t limit, bool vec) {
  // 8 consecutive bf16 at p[idx..idx+7]; entries at or past `limit` read 0
  if (vec && idx + 8 <= limit) return *reinterpret_cast<const uint4*>(p + idx);
  uint16_t e[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) e[q] = (idx + q < limit) ? p[idx + q] : (uint16_t)0;
  uint4 v;
  v.x = e[0] | ((uint32_t)e[1] << 16);
  v.y = e[2] | ((uint32_t)e[3] << 16);
  v.z = e[4] | ((uint32_t)e[5] << 16);
  v.w = e[6] | ((uint32_t)e[7] << 16);
  return v;
}

// ------------------------------------------------------------ skinny NT
// P[m][j] = sum_k T[m][k] U[j][k] for 16 rows m per workgroup.  The 8 waves
// take interleaved 128-wide inner steps; lane (j16, g) reads the 32
// contiguous inner indices 32g..32g+31 of the step from both operands (four
// MFMA sub-steps).  The wave partials are summed in wave order through LDS.
template <int RT>
__global__ __launch_bounds__(512) void k_skinny_nt(const uint16_t* __restrict__ T, int64_t M,
                                                   int64_t kin, int64_t ldt,
                                                   const uint16_t* __restrict__ U, int r,
                                                   int64_t ldu, float scale,
                                                   uint16_t* __restrict__ out_s, int r32,
                                                   uint16_t* __restrict__ out,
                                                   uint16_t* __restrict__ out_t, int64_t ldo_t,
                                                   int vec) {
  __shared__ float red[8][RT][4][64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int j16 = lane & 15, g = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * 16;
  int64_t mrow = m0 + j16;
  mrow = mrow < M ? mrow : M - 1;
  const bool tv = vec && (ldt % 8) == 0;
  const bool uv = vec && (ldu % 8) == 0;

  f32x4_t acc[RT];
#pragma unroll
  for (int jt = 0; jt < RT; ++jt) acc[jt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int64_t k = (int64_t)wv * 128; k < kin; k += 8 * 128) {
    const int64_t kk = k + 32 * g;
    uint4 a[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) a[s] = load8_bf16(T + mrow * ldt, kk + 8 * s, kin, tv);
#pragma unroll
    for (int jt = 0; jt < RT; ++jt) {
      const int u = jt * 16 + j16;
      uint4 b[4];
      if (u < r) {
#pragma unroll
        for (int s = 0; s < 4; ++s) b[s] = load8_bf16(U + (int64_t)u * ldu, kk + 8 * s, kin, uv);
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) b[s] = make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) acc[jt] = mfma16x16x32(a[s], b[s], acc[jt]);
    }
  }
#pragma unroll
  for (int jt = 0; jt < RT; ++jt)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wv][jt][v][lane] = acc[jt][v];
  __syncthreads();
  if (wv != 0) return;
  // lane holds P[m0 + 4g + v][16 jt + j16]
#pragma unroll
  for (int jt = 0; jt < RT; ++jt) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < 8; ++w) sum += red[w][jt][v][lane];
      const int64_t m = m0 + 4 * g + v;
      const int j = jt * 16 + j16;
      if (m < M) {
        if (out_s && j < r32) out_s[m * r32 + j] = (uint16_t)(pack_bf16x2(j < r ? scale * sum : 0.f, 0.f) & 0xFFFF);
        if (out && j < r) out[m * r + j] = (uint16_t)(pack_bf16x2(sum, 0.f) & 0xFFFF);
      }
      if (out_t && j < r && m < ldo_t)
        out_t[(int64_t)j * ldo_t + m] = m < M ? (uint16_t)(pack_bf16x2(sum, 0.f) & 0xFFFF) : (uint16_t)0;
    }
  }
  // zero padding columns of out_s beyond the computed tiles
  if (out_s) {
    for (int j = RT * 16 + j16; j < r32; j += 16)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t m = m0 + 4 * g + v;
        if (m < M) out_s[m * r32 + j] = 0;
      }
  }
}

__global__ __launch_bounds__(256) void k_transpose_bf16(const uint16_t* __restrict__ in,
                                                        int64_t rows, int64_t cols,
                                                        uint16_t* __restrict__ out, int64_t ldo) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // output index along ldo
  const int64_t j = blockIdx.y;                                  // output row (= input column)
  if (i < ldo) out[j * ldo + i] = (i < rows) ? in[i * cols + j] : (uint16_t)0;
}

// ------------------------------------------------------- adapter gradients
// partial[split][p][j] = sum_{m in split} T[m][p] U[j][m]
// T [M, P] row-major, U [r, ldu] (U[j][m] = 0 for m >= M).  Wave = 128
// consecutive p.  Lane (i16, g) loads 8 rows m (8g..8g+7 of a 32-step) x 8
// consecutive p (8 i16 .. 8 i16 + 7) and regroups them into the A operands of
// 8 MFMAs: MFMA t handles p = p0 + 8 i + t, so the transpose of T costs one
// 16-bit regroup per pair of rows, no LDS.
template <int RT>
__global__ __launch_bounds__(256) void k_lora_grad(const uint16_t* __restrict__ T, int64_t M,
                                                   int64_t P, const uint16_t* __restrict__ U,
                                                   int r, int64_t ldu, int64_t mchunk,
                                                   float* __restrict__ partial, int vec) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  const int64_t p0 = ((int64_t)blockIdx.x * 4 + wv) * 128;
  if (p0 >= P) return;
  const int split = blockIdx.y;
  const int64_t mbeg = (int64_t)split * mchunk;
  int64_t mend = mbeg + mchunk;
  mend = mend < M ? mend : M;
  const int64_t pc = p0 + 8 * i16;
  const bool pv = vec && (P % 8) == 0;

  f32x4_t acc[8][RT];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int jt = 0; jt < RT; ++jt) acc[t][jt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int64_t mb = mbeg; mb < mend; mb += 32) {
    uint4 rows[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int64_t m = mb + 8 * g + e;
      m = m < M ? m : M - 1;                // U is zero there
      rows[e] = load8_bf16(T + m * P, pc, P, pv);
    }
    uint4 bu[RT];
#pragma unroll
    for (int jt = 0; jt < RT; ++jt) {
      const int u = jt * 16 + i16;
      bu[jt] = (u < r) ? *reinterpret_cast<const uint4*>(U + (int64_t)u * ldu + mb + 8 * g)
                       : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w = (t < 2) ? rows[e].x : (t < 4) ? rows[e].y : (t < 6) ? rows[e].z : rows[e].w;
        h[e] = (t & 1) ? (w >> 16) : (w & 0xFFFFu);
      }
      uint4 a;
      a.x = h[0] | (h[1] << 16);
      a.y = h[2] | (h[3] << 16);
      a.z = h[4] | (h[5] << 16);
      a.w = h[6] | (h[7] << 16);
#pragma unroll
      for (int jt = 0; jt < RT; ++jt) acc[t][jt] = mfma16x16x32(a, bu[jt], acc[t][jt]);
    }
  }
  // D[i = 4g + v][j16] of MFMA (t, jt): p = p0 + 8 (4g + v) + t, j = 16 jt + j16
  float* base = partial + (int64_t)split * P * r;
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int jt = 0; jt < RT; ++jt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t p = p0 + 8 * (4 * g + v) + t;
        const int j = jt * 16 + i16;
        if (p < P && j < r) base[p * r + j] = acc[t][jt][v];
      }
}

__global__ __launch_bounds__(256) void k_lora_grad_reduce(const float* __restrict__ partial,
                                                          int splits, int64_t P, int r,
                                                          float scale, int transposed,
                                                          float* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= P * r) return;
  int64_t p, j;
  if (transposed) { j = idx / P; p = idx % P; } else { p = idx / r; j = idx % r; }
  float s = 0.f;
  for (int k = 0; k < splits; ++k) s += partial[(int64_t)k * P * r + p * r + j];
  out[idx] = scale * s;
}

template <int RT>
hipError_t skinny_rt(const uint16_t* T, int64_t M, int64_t kin, int64_t ldt, const uint16_t* U,
                     int r, int64_t ldu, float scale, uint16_t* out_s, int r32, uint16_t* out,
                     uint16_t* out_t, int64_t ldo_t, hipStream_t s) {
  int64_t rows = M;
  if (out_t && ldo_t > rows) rows = ldo_t;
  hipLaunchKernelGGL(k_skinny_nt<RT>, dim3((unsigned)ceil_div(rows, 16)), dim3(512), 0, s, T, M,
                     kin, ldt, U, r, ldu, scale, out_s, r32, out, out_t, ldo_t, 1);
  return hipGetLastError();
}

template <int RT>
hipError_t grad_rt(const uint16_t* T, int64_t M, int64_t P, const uint16_t* U, int r, int64_t ldu,
                   int splits, float* partial, hipStream_t s) {
  const int64_t mchunk = ceil_div(ceil_div(M, splits), 32) * 32;
  hipLaunchKernelGGL(k_lora_grad<RT>, dim3((unsigned)ceil_div(P, 512), (unsigned)splits), dim3(256),
                     0, s, T, M, P, U, r, ldu, mchunk, partial, 1);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_skinny_nt(const uint16_t* T, int64_t M, int64_t kin, int64_t ldt,
                            const uint16_t* U, int r, int64_t ldu, float scale, uint16_t* out_s,
                            int r32, uint16_t* out, uint16_t* out_t, int64_t ldo_t,
                            hipStream_t s) {
  if (r <= 16) return skinny_rt<1>(T, M, kin, ldt, U, r, ldu, scale, out_s, r32, out, out_t, ldo_t, s);
  if (r <= 32) return skinny_rt<2>(T, M, kin, ldt, U, r, ldu, scale, out_s, r32, out, out_t, ldo_t, s);
  if (r <= 64) return skinny_rt<4>(T, M, kin, ldt, U, r, ldu, scale, out_s, r32, out, out_t, ldo_t, s);
  return skinny_rt<8>(T, M, kin, ldt, U, r, ldu, scale, out_s, r32, out, out_t, ldo_t, s);
}

hipError_t launch_transpose_bf16(const uint16_t* in, int64_t rows, int64_t cols, uint16_t* out,
                                 int64_t ldo, hipStream_t s) {
  hipLaunchKernelGGL(k_transpose_bf16, dim3((unsigned)ceil_div(ldo, 256), (unsigned)cols),
                     dim3(256), 0, s, in, rows, cols, out, ldo);
  return hipGetLastError();
}

int lora_grad_splits(int64_t M, int64_t P) {
  // enough workgroups to cover the chip, at least 256 tokens per split
  const int64_t groups = ceil_div(P, 512);
  int64_t splits = ceil_div(1024, groups);
  const int64_t maxs = ceil_div(M, 256);
  if (splits > maxs) splits = maxs;
  if (splits < 1) splits = 1;
  return (int)splits;
}

hipError_t launch_lora_grad(const uint16_t* T, int64_t M, int64_t P, const uint16_t* U, int r,
                            int64_t ldu, int splits, float* partial, hipStream_t s) {
  if (r <= 16) return grad_rt<1>(T, M, P, U, r, ldu, splits, partial, s);
  if (r <= 32) return grad_rt<2>(T, M, P, U, r, ldu, splits, partial, s);
  if (r <= 64) return grad_rt<4>(T, M, P, U, r, ldu, splits, partial, s);
  return grad_rt<8>(T, M, P, U, r, ldu, splits, partial, s);
}

hipError_t launch_lora_grad_reduce(const float* partial, int splits, int64_t P, int r, float scale,
                                   int transposed, float* out, hipStream_t s) {
  hipLaunchKernelGGL(k_lora_grad_reduce, dim3((unsigned)ceil_div(P * r, 256)), dim3(256), 0, s,
                     partial, splits, P, r, scale, transposed, out);
  return hipGetLastError();
}

}  // namespace qnf4
