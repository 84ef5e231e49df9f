// Skinny products P = T . U^T (rank-r side of the LoRA path) as one slice of
// a workgroup: shared by the side-path launches and the decode kernel.
#pragma once

#include "launch.h"

namespace qnf4 {

constexpr int kSkStep = 128;    // inner indices per wave step (4 lane groups x 32)

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

// Raw buffer view of `bytes` bytes at p (reads past the end return zero).
// Buffer loads take a wave-uniform byte offset in a scalar register on top
// of a fixed per-lane offset, so a streaming loop that moves its base per
// step does no vector address arithmetic (which, between a step's loads and
// the previous step's MFMAs, makes the compiler drain the loads in flight).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_view(const void* p, int64_t bytes) {
  const int n = bytes < 0x7FFFFFFF ? (int)bytes : 0x7FFFFFFF;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, n, 0x00020000);
}
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t v, uint32_t lane_off,
                                               uint32_t uniform_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                       v, (int)lane_off, (int)uniform_off, 0));
}
// byte offsets of a buffer view are 32-bit
constexpr int64_t kBufferMax = 0x7FFFFFFF;

// v if keep (an all-ones mask), else 0: a value select the compiler cannot
// turn into a branch around the load
__device__ __forceinline__ uint4 keep_if(uint4 v, uint32_t keep) {
  return make_uint4(v.x & keep, v.y & keep, v.z & keep, v.w & keep);
}

__device__ __forceinline__ uint16_t to_bf16(float v) {
  return (uint16_t)(pack_bf16x2(v, 0.f) & 0xFFFF);
}

// ------------------------------------------------------------ skinny NT
// Workgroup (row group, slice): 16 rows of T, inner indices [kbeg, kend).
// The W waves take interleaved 128-wide steps; lane (j16, g) reads the 32
// contiguous inner indices 32g..32g+31 of a step from both operands (four
// MFMA sub-steps).  Wave partials are added in wave order through LDS.  With
// DROP, a job whose J.drop is set reads T through the dropout mask (T = X,
// element e = m K + k) and scales its sums by J.drop.inv.
template <int RT, int W, bool DROP = false>
__device__ __forceinline__ void skinny_slice(const SkinnyJob& J, int64_t M, int r, int r32,
                                             int64_t b) {
  __shared__ float red[W][RT][4][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int j16 = lane & 15, g = lane >> 4;
  const int ks = (int)(b % J.ks);
  const int64_t m0 = (b / J.ks) * 16;
  int64_t mrow = m0 + j16;
  mrow = mrow < M ? mrow : M - 1;
  const int64_t kbeg = (int64_t)ks * J.kslice;
  int64_t kend = kbeg + J.kslice;
  kend = kend < J.kin ? kend : J.kin;
  const bool tv = (J.ldt % 8) == 0;
  const bool uv = (J.ldu % 8) == 0;
  const uint16_t* trow = J.T + mrow * J.ldt;

  f32x4_t acc[RT];
#pragma unroll
  for (int jt = 0; jt < RT; ++jt) acc[jt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // this lane's adapter rows, clamped: a row past r feeds only output column
  // u >= r, which is never stored
  const uint16_t* urow[RT];
#pragma unroll
  for (int jt = 0; jt < RT; ++jt) {
    const int u = jt * 16 + j16;
    urow[jt] = J.U + (int64_t)(u < r ? u : r - 1) * J.ldu;
  }
  // the fast path reads both operands through buffer views: fixed byte
  // offsets per lane, 2 k per step as the uniform offset
  const int64_t tbytes = (M > 0 ? (M - 1) * J.ldt + J.kin : 0) * 2;
  const int64_t ubytes = ((int64_t)(r - 1) * J.ldu + J.kin) * 2;
  const __amdgpu_buffer_rsrc_t tview = buffer_view(J.T, tbytes);
  const __amdgpu_buffer_rsrc_t uview = buffer_view(J.U, ubytes);
  const uint32_t toff = (uint32_t)(mrow * J.ldt + 8 * g) * 2;
  uint32_t uoff[RT];
#pragma unroll
  for (int jt = 0; jt < RT; ++jt) uoff[jt] = (uint32_t)((urow[jt] - J.U) + 8 * g) * 2;
  auto mfmas = [&](const uint4 (&a)[4], const uint4 (&bv)[RT][4]) {
#pragma unroll
    for (int jt = 0; jt < RT; ++jt)
#pragma unroll
      for (int s = 0; s < 4; ++s) acc[jt] = mfma16x16x32(a[s], bv[jt][s], acc[jt]);
  };
  // dropout of the T operand of the step at k (wave-uniform switch); a lane
  // of a real row also stores the keep bits when the forward keeps them
  const bool dj = DROP && J.drop.thr != 0;
  const uint64_t erow = (uint64_t)mrow * (uint64_t)J.drop.cols + 8 * g;
  const bool wbits = DROP && J.drop.bits_out && m0 + j16 < M;
  auto drop_t = [&](int64_t k, uint4 (&a)[4]) {
    if constexpr (DROP) {
      if (dj) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint64_t e = erow + k + 32 * s;
          const uint32_t kb = dropout_byte(e, J.drop);
          a[s] = and4(a[s], byte_mask8(kb));
          if (wbits && k + 32 * s + 8 * g < J.kin) J.drop.bits_out[e >> 3] = (uint8_t)kb;
        }
      }
    }
  };
  // Operands of one step: sub-step s takes inner indices k + 32 s + 8 g ..
  // + 7 from lane group g, so each load instruction reads 64 contiguous bytes
  // per row.  Whole steps of a slice whose rows are 16-byte aligned run on
  // plain vector loads with no branch and no per-lane select between them,
  // two steps in flight: the next step's loads are issued before this
  // step's MFMAs.
  const bool vec = tv && uv && tbytes <= kBufferMax && ubytes <= kBufferMax;
  const int64_t nfull = vec ? (kend - kbeg) / kSkStep : 0;        // whole steps
  const int64_t cnt = nfull > wv ? (nfull - wv + W - 1) / W : 0;   // this wave's
  auto kat = [&](int64_t i) { return kbeg + (wv + i * W) * (int64_t)kSkStep; };
  auto load_fast = [&](int64_t k, uint4 (&a)[4], uint4 (&bv)[RT][4]) {
    const uint32_t kb = (uint32_t)k * 2;
#pragma unroll
    for (int s = 0; s < 4; ++s) a[s] = buffer_load16(tview, toff + 64 * s, kb);
#pragma unroll
    for (int jt = 0; jt < RT; ++jt)
#pragma unroll
      for (int s = 0; s < 4; ++s) bv[jt][s] = buffer_load16(uview, uoff[jt] + 64 * s, kb);
  };
  if (cnt > 0) {
    if constexpr (RT <= 4) {
      uint4 a0[4], b0[RT][4], a1[4], b1[RT][4];
      load_fast(kat(0), a0, b0);
      // (scheduling barriers keep the compiler from sinking the loads next
      // to their MFMAs; the last one or two steps are peeled)
      int64_t i = 0;
      for (; i + 2 < cnt; i += 2) {
        load_fast(kat(i + 1), a1, b1);
        __builtin_amdgcn_sched_barrier(0);
        drop_t(kat(i), a0);
        mfmas(a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        load_fast(kat(i + 2), a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        drop_t(kat(i + 1), a1);
        mfmas(a1, b1);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (i + 1 < cnt) {
        load_fast(kat(i + 1), a1, b1);
        __builtin_amdgcn_sched_barrier(0);
        drop_t(kat(i), a0);
        mfmas(a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        drop_t(kat(i + 1), a1);
        mfmas(a1, b1);
      } else {
        drop_t(kat(i), a0);
        mfmas(a0, b0);
      }
    } else {
      for (int64_t i = 0; i < cnt; ++i) {   // r > 64: one step at a time
        uint4 a0[4], b0[RT][4];
        load_fast(kat(i), a0, b0);
        drop_t(kat(i), a0);
        mfmas(a0, b0);
      }
    }
  }
  // the remaining steps (a partial last step, or every step of unaligned
  // rows): element-wise loads with bounds
  for (int64_t k = kat(cnt); k < kend; k += (int64_t)W * kSkStep) {
    uint4 a0[4], b0[RT][4];
#pragma unroll
    for (int s = 0; s < 4; ++s) a0[s] = load8_bf16(trow, k + 32 * s + 8 * g, J.kin, tv);
#pragma unroll
    for (int jt = 0; jt < RT; ++jt)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        b0[jt][s] = load8_bf16(urow[jt], k + 32 * s + 8 * g, J.kin, uv);
    drop_t(k, a0);
    mfmas(a0, b0);
  }
#pragma unroll
  for (int jt = 0; jt < RT; ++jt)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wv][jt][v][lane] = acc[jt][v];
  __syncthreads();
  if (wv != 0) return;
  // lane holds P[m0 + 4g + v][16 jt + j16]; a single slice writes the final
  // outputs, several write float32 partials for the finish step
  float* part = J.part + (int64_t)ks * M * (RT * 16);
#pragma unroll
  for (int jt = 0; jt < RT; ++jt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float sum = red[0][jt][v][lane];
#pragma unroll
      for (int w = 1; w < W; ++w) sum += red[w][jt][v][lane];
      if constexpr (DROP) sum *= J.drop.inv;
      const int64_t m = m0 + 4 * g + v;
      const int j = jt * 16 + j16;
      if (J.ks > 1 || J.part_only) {
        if (m < M) part[m * (RT * 16) + j] = sum;
        continue;
      }
      if (m < M) {
        if (J.out_s && j < r32) J.out_s[m * r32 + j] = to_bf16(j < r ? J.scale * sum : 0.f);
        if (J.out && j < r) J.out[m * r + j] = to_bf16(sum);
      }
      if (J.out_t && j < r && m < J.ldo_t)
        J.out_t[(int64_t)j * J.ldo_t + m] = m < M ? to_bf16(sum) : 0;
    }
  if (J.ks == 1 && !J.part_only && J.out_s) {   // padding columns of out_s past the tiles
    for (int j = RT * 16 + j16; j < r32; j += 16)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t m = m0 + 4 * g + v;
        if (m < M) J.out_s[m * r32 + j] = 0;
      }
  }
}

}  // namespace qnf4
