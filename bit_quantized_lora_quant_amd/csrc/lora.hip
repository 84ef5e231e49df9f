// The low-rank side path: skinny products against the adapters and the
// adapter gradients.  LoRA pairs a down-projection A [r, K] with an
// up-projection B [N, r] beside the frozen weight (xingyuzhitong guide,
// section "LoRA: freeze the base, train small adapters"; r and lora_alpha are
// the PEFT knobs of "QLoRA: Fine-Tuning a 70B on One GPU", section "Practical
// Implementation").  All contractions run on v_mfma_f32_16x16x32_bf16 with
// float32 accumulation; reductions over the inner dimension or the tokens use
// fixed slices and a fixed summation order, so results repeat bit for bit.
//
// These steps stream one activation tensor each and are bound by HBM; they
// are cut into enough workgroups to cover the chip, and independent small
// steps share a launch.
#include "skinny.h"

namespace qnf4 {
namespace {

constexpr int kSkWaves = 8;     // waves per skinny workgroup at ranks above 16
// rank <= 16 keeps few registers per lane: 16 waves (1024 threads) put twice
// the loads in flight per CU
template <int RT>
constexpr int sk_waves() { return RT == 1 ? 16 : kSkWaves; }

// One thread per element of [KB][N]: out[kb * N + n] = â(n * KB + kb).
__device__ __forceinline__ void recon_elems(const ReconJob& J, int64_t b) {
  const int64_t e = b * blockDim.x + threadIdx.x;
  if (e >= J.N * J.KB) return;
  const int64_t kb = e / J.N, n = e - kb * J.N;
  J.out[e] = J.f32 ? J.f32[n * J.KB + kb] : absmax_recon(J.q, J.scale, *J.mean, n * J.KB + kb);
}


// Row groups of a job: past M only when out_t needs zero padding.
__device__ __host__ __forceinline__ int64_t skinny_rows(const SkinnyJob& J, int64_t M) {
  return (J.ks == 1 && J.out_t && J.ldo_t > M) ? J.ldo_t : M;
}

__device__ __forceinline__ int64_t skinny_blocks(const SkinnyJob& J, int64_t M) {
  return ceil_div(skinny_rows(J, M), 16) * J.ks;
}

// DROP: some job reads X through the dropout mask
template <int RT, bool DROP>
__global__ __launch_bounds__(sk_waves<RT>() * 64) void k_skinny_slices(SkinnyJob j0, SkinnyJob j1, int nj,
                                                       int64_t M, int r, int r32, ReconJob rc,
                                                       int has_rc) {
  int64_t b = blockIdx.x;
  const int64_t b0 = skinny_blocks(j0, M);
  if (b < b0) { skinny_slice<RT, sk_waves<RT>(), DROP>(j0, M, r, r32, b); return; }
  b -= b0;
  if (nj > 1) {
    const int64_t b1 = skinny_blocks(j1, M);
    if (b < b1) { skinny_slice<RT, sk_waves<RT>(), DROP>(j1, M, r, r32, b); return; }
    b -= b1;
  }
  if (has_rc) recon_elems(rc, b);
}

// Thread per (row m, column j < r32) of one job: adds the slices in order.
__device__ __forceinline__ void skinny_finish_elem(const SkinnyJob& J, int64_t M, int r, int r32,
                                                   int rpad, int64_t e) {
  const int64_t rows = (J.out_t && J.ldo_t > M) ? J.ldo_t : M;
  if (e >= rows * r32) return;
  const int64_t m = e / r32;
  const int j = (int)(e - m * r32);
  float sum = 0.f;
  if (m < M && j < r) {
    sum = J.part[m * rpad + j];
    for (int k = 1; k < J.ks; ++k) sum += J.part[((int64_t)k * M + m) * rpad + j];
  }
  if (m < M) {
    if (J.out_s) J.out_s[m * r32 + j] = to_bf16(j < r ? J.scale * sum : 0.f);
    if (J.out && j < r) J.out[m * r + j] = to_bf16(sum);
  }
  if (J.out_t && j < r && m < J.ldo_t) J.out_t[(int64_t)j * J.ldo_t + m] = m < M ? to_bf16(sum) : 0;
}

// (jobs run as a single slice wrote their outputs directly: no finish)
__device__ __host__ __forceinline__ int64_t finish_blocks(const SkinnyJob& J, int64_t M,
                                                          int r32) {
  if (J.ks == 1) return 0;
  const int64_t rows = (J.out_t && J.ldo_t > M) ? J.ldo_t : M;
  return ceil_div(rows * r32, 256);
}

__global__ __launch_bounds__(256) void k_skinny_finish(SkinnyJob j0, SkinnyJob j1, int nj,
                                                       int64_t M, int r, int r32, int rpad) {
  int64_t b = blockIdx.x;
  const int64_t b0 = finish_blocks(j0, M, r32);
  if (b < b0) { skinny_finish_elem(j0, M, r, r32, rpad, b * 256 + threadIdx.x); return; }
  b -= b0;
  if (nj > 1) skinny_finish_elem(j1, M, r, r32, rpad, b * 256 + threadIdx.x);
}

// ------------------------------------------------------------------ prep
__device__ __forceinline__ void transpose_elem(const TransposeJob& J, int64_t e) {
  if (e >= J.cols * J.ldo) return;
  const int64_t j = e / J.ldo, i = e - j * J.ldo;   // output row j (= input column), column i
  J.out[e] = (i < J.rows) ? J.in[i * J.cols + j] : (uint16_t)0;
}

__global__ __launch_bounds__(256) void k_prep(TransposeJob t0, TransposeJob t1, int nt,
                                              ReconJob rc, int has_rc) {
  int64_t b = blockIdx.x;
  if (nt > 0) {
    const int64_t n0 = ceil_div(t0.cols * t0.ldo, 256);
    if (b < n0) { transpose_elem(t0, b * 256 + threadIdx.x); return; }
    b -= n0;
  }
  if (nt > 1) {
    const int64_t n1 = ceil_div(t1.cols * t1.ldo, 256);
    if (b < n1) { transpose_elem(t1, b * 256 + threadIdx.x); return; }
    b -= n1;
  }
  if (has_rc) recon_elems(rc, b);
}

// ------------------------------------------------------- adapter gradients
// Workgroup (128 consecutive p, token slice): the 4 waves take interleaved
// 32-token steps.  Lane (i16, g) loads 8 rows m (8g..8g+7 of a step) x 8
// consecutive p (8 i16 .. 8 i16 + 7) of T and regroups them into the A
// operands of 8 MFMAs: MFMA t handles p = p0 + 8 i + t, so the transpose of T
// costs one 16-bit regroup per pair of rows, no LDS.  Wave partials are added
// in wave order through LDS, one MFMA column t at a time.  With DROP, a job
// whose J.drop is set reads T = X through the dropout mask and scales its
// partials by J.drop.inv.
template <int RT, bool DROP>
__device__ __forceinline__ void grad_slice(const GradJob& J, int64_t M, int r, int64_t b) {
  __shared__ float red[4][RT][4][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int i16 = lane & 15, g = lane >> 4;
  const int split = (int)(b % J.splits);
  const int64_t p0 = (b / J.splits) * 128;
  const int64_t mchunk = ceil_div(ceil_div(M, J.splits), 32) * 32;
  const int64_t mbeg = (int64_t)split * mchunk;
  int64_t mend = mbeg + mchunk;
  mend = mend < M ? mend : M;
  const int64_t pc = p0 + 8 * i16;
  const bool pv = (J.P % 8) == 0;

  f32x4_t acc[8][RT];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int jt = 0; jt < RT; ++jt) acc[t][jt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const bool fast = pv && p0 + 128 <= J.P;   // workgroup-uniform
  // this lane's rows of U, clamped: a row past r feeds only output column
  // j >= r, which is never stored (no branch or select around the loads, which
  // would cost the two-steps-in-flight schedule)
  const uint16_t* urow[RT];
#pragma unroll
  for (int jt = 0; jt < RT; ++jt) {
    const int u = jt * 16 + i16;
    urow[jt] = J.U + (int64_t)(u < r ? u : r - 1) * J.ldu;
  }
  // step mb: rows mb + 8g + e of T (clamped below M; U is zero there) and
  // columns mb + 8g .. + 7 of U (within ldu, a multiple of 32)
  auto load_u = [&](int64_t mb, uint4 (&bu)[RT]) {
#pragma unroll
    for (int jt = 0; jt < RT; ++jt)
      bu[jt] = *reinterpret_cast<const uint4*>(urow[jt] + mb + 8 * g);
  };
  auto load_step = [&](int64_t mb, uint4 (&rows)[8], uint4 (&bu)[RT]) {   // 128 columns in range
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int64_t m = mb + 8 * g + e;
      m = m < M ? m : M - 1;
      rows[e] = *reinterpret_cast<const uint4*>(J.T + m * J.P + pc);
    }
    load_u(mb, bu);
  };
  auto load_step_ragged = [&](int64_t mb, uint4 (&rows)[8], uint4 (&bu)[RT]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int64_t m = mb + 8 * g + e;
      m = m < M ? m : M - 1;
      rows[e] = load8_bf16(J.T + m * J.P, pc, J.P, pv);
    }
    load_u(mb, bu);
  };
  auto mfmas = [&](const uint4 (&rows)[8], const uint4 (&bu)[RT]) {
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
  };
  // dropout of T's rows of step mb (wave-uniform switch); rows past M are
  // clamped copies that meet zero columns of U
  const bool dj = DROP && J.drop.thr != 0;
  auto drop_t = [&](int64_t mb, uint4 (&rows)[8]) {
    if constexpr (DROP) {
      if (dj) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          int64_t m = mb + 8 * g + e;
          m = m < M ? m : M - 1;
          rows[e] = and4(rows[e], dropout_keep8((uint64_t)m * (uint64_t)J.drop.cols + pc, J.drop));
        }
      }
    }
  };
  // this wave's steps: mb = first + 128 i, i < cnt
  const int64_t first = mbeg + 32 * wv;
  const int64_t cnt = first < mend ? (mend - first + 127) / 128 : 0;
  // Steps of 32 whole rows with 128 columns in range, at rank <= 32, read
  // through buffer views (fixed byte offsets per lane, the step's base as the
  // uniform offset), two steps in flight: the next step's loads are issued
  // before this step's MFMAs.
  const int64_t tbytes = M * J.P * 2, ubytes = (int64_t)r * J.ldu * 2;
  const bool bufs = fast && RT <= 2 && tbytes <= kBufferMax && ubytes <= kBufferMax;
  const int64_t cnt_fast = bufs && first + 32 <= mend ? (mend - first - 32) / 128 + 1 : 0;
  if (cnt_fast > 0) {
    const __amdgpu_buffer_rsrc_t tview = buffer_view(J.T, tbytes);
    const __amdgpu_buffer_rsrc_t uview = buffer_view(J.U, ubytes);
    uint32_t roff[8], uoff[RT];
#pragma unroll
    for (int e = 0; e < 8; ++e) roff[e] = (uint32_t)((8 * g + e) * J.P + pc) * 2;
#pragma unroll
    for (int jt = 0; jt < RT; ++jt) uoff[jt] = (uint32_t)((urow[jt] - J.U) + 8 * g) * 2;
    auto load_fast = [&](int64_t i, uint4 (&rows)[8], uint4 (&bu)[RT]) {
      const int64_t mb = first + 128 * i;
      const uint32_t tb = (uint32_t)(mb * J.P) * 2, ub = (uint32_t)mb * 2;
#pragma unroll
      for (int e = 0; e < 8; ++e) rows[e] = buffer_load16(tview, roff[e], tb);
#pragma unroll
      for (int jt = 0; jt < RT; ++jt) bu[jt] = buffer_load16(uview, uoff[jt], ub);
    };
    uint4 r0[8], u0[RT], r1[8], u1[RT];
    load_fast(0, r0, u0);
    int64_t i = 0;
    for (; i + 2 < cnt_fast; i += 2) {
      load_fast(i + 1, r1, u1);
      __builtin_amdgcn_sched_barrier(0);
      drop_t(first + 128 * i, r0);
      mfmas(r0, u0);
      __builtin_amdgcn_sched_barrier(0);
      load_fast(i + 2, r0, u0);
      __builtin_amdgcn_sched_barrier(0);
      drop_t(first + 128 * (i + 1), r1);
      mfmas(r1, u1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (i + 1 < cnt_fast) {   // the last one or two steps, peeled
      load_fast(i + 1, r1, u1);
      __builtin_amdgcn_sched_barrier(0);
      drop_t(first + 128 * i, r0);
      mfmas(r0, u0);
      __builtin_amdgcn_sched_barrier(0);
      drop_t(first + 128 * (i + 1), r1);
      mfmas(r1, u1);
    } else {
      drop_t(first + 128 * i, r0);
      mfmas(r0, u0);
    }
  }
  // the rest (a last step of fewer rows, ragged columns, or wide ranks whose
  // accumulators fill the register file): one step at a time, rows clamped
  for (int64_t i = cnt_fast; i < cnt; ++i) {
    uint4 r0[8], u0[RT];
    if (fast) load_step(first + 128 * i, r0, u0);
    else load_step_ragged(first + 128 * i, r0, u0);
    drop_t(first + 128 * i, r0);
    mfmas(r0, u0);
  }
  // D[i = 4g + v][j16] of MFMA (t, jt): p = p0 + 8 (4g + v) + t, j = 16 jt + j16
  float* base = J.partial + (int64_t)split * J.P * r;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
#pragma unroll
    for (int jt = 0; jt < RT; ++jt)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[wv][jt][v][lane] = acc[t][jt][v];
    __syncthreads();
    if (wv == 0) {
#pragma unroll
      for (int jt = 0; jt < RT; ++jt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float s = red[0][jt][v][lane];
#pragma unroll
          for (int w = 1; w < 4; ++w) s += red[w][jt][v][lane];
          if constexpr (DROP) s *= J.drop.inv;
          const int64_t p = p0 + 8 * (4 * g + v) + t;
          const int j = jt * 16 + i16;
          if (p < J.P && j < r) base[p * r + j] = s;
        }
    }
    __syncthreads();
  }
}

__device__ __forceinline__ int64_t grad_blocks(const GradJob& J) {
  return ceil_div(J.P, 128) * J.splits;
}

template <int RT, bool DROP>
__global__ __launch_bounds__(256) void k_lora_grads(GradJob j0, GradJob j1, int nj, int64_t M,
                                                    int r) {
  int64_t b = blockIdx.x;
  const int64_t b0 = grad_blocks(j0);
  if (b < b0) { grad_slice<RT, DROP>(j0, M, r, b); return; }
  if (nj > 1) grad_slice<RT, DROP>(j1, M, r, b - b0);
}

__device__ __forceinline__ void grad_reduce_elem(const GradJob& J, int r, int64_t idx) {
  if (idx >= J.P * r) return;
  int64_t p, j;
  if (J.transposed) { j = idx / J.P; p = idx - j * J.P; } else { p = idx / r; j = idx - p * r; }
  if (J.groups > 0) {   // off the diagonal blocks of a grouped linear: zero
    int g = 0;
    while (g + 1 < J.groups && p >= J.end[g]) ++g;
    if (j / J.gr != g) { J.out[idx] = 0.f; return; }
  }
  float s = J.partial[p * r + j];
  for (int k = 1; k < J.splits; ++k) s += J.partial[(int64_t)k * J.P * r + p * r + j];
  J.out[idx] = J.scale * s;
}

__global__ __launch_bounds__(256) void k_lora_grad_reduce(GradJob j0, GradJob j1, int nj, int r) {
  const int64_t b0 = ceil_div(j0.P * r, 256);
  const int64_t b = blockIdx.x;
  if (b < b0) { grad_reduce_elem(j0, r, b * 256 + threadIdx.x); return; }
  if (nj > 1) grad_reduce_elem(j1, r, (b - b0) * 256 + threadIdx.x);
}

template <int RT>
hipError_t skinny_rt(const SkinnyJob* jobs, int nj, int64_t M, int r, int r32, const ReconJob* rc,
                     hipStream_t s) {
  int64_t blocks = 0;
  for (int i = 0; i < nj; ++i) blocks += ceil_div(skinny_rows(jobs[i], M), 16) * jobs[i].ks;
  blocks += rc ? ceil_div(rc->N * rc->KB, sk_waves<RT>() * 64) : 0;
  const ReconJob none{};
  bool drop = false;
  for (int i = 0; i < nj; ++i) drop |= jobs[i].drop.thr != 0;
  const auto kern = drop ? k_skinny_slices<RT, true> : k_skinny_slices<RT, false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(sk_waves<RT>() * 64), 0, s,
                     jobs[0], nj > 1 ? jobs[1] : jobs[0], nj, M, r, r32, rc ? *rc : none,
                     rc ? 1 : 0);
  return hipGetLastError();
}

template <int RT>
hipError_t grads_rt(const GradJob* jobs, int nj, int64_t M, int r, hipStream_t s) {
  int64_t blocks = 0;
  for (int i = 0; i < nj; ++i) blocks += ceil_div(jobs[i].P, 128) * jobs[i].splits;
  bool drop = false;
  for (int i = 0; i < nj; ++i) drop |= jobs[i].drop.thr != 0;
  const auto kern = drop ? k_lora_grads<RT, true> : k_lora_grads<RT, false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, s, jobs[0],
                     nj > 1 ? jobs[1] : jobs[0], nj, M, r);
  return hipGetLastError();
}

}  // namespace

int skinny_rpad(int r) { return r <= 16 ? 16 : r <= 32 ? 32 : r <= 64 ? 64 : 128; }

int skinny_slices(int64_t M, int64_t kin) {
  // one slice once there are enough row groups to spread over the chip (no
  // finish step then); else about 256 workgroups, at least one 128-wide
  // step per wave
  const int64_t groups = ceil_div(M, 16);
  // a long inner dimension over fewer row groups than CUs: two slices, so
  // the launch covers the chip (the finish step costs less than the idle half)
  if (groups >= 64) return groups < 256 && kin >= 8192 ? 2 : 1;
  int64_t ks = ceil_div(256, groups);
  const int64_t maxs = ceil_div(kin, (int64_t)kSkWaves * kSkStep);
  if (ks > maxs) ks = maxs;
  if (ks < 1) ks = 1;
  return (int)ks;
}

size_t skinny_part_floats(int64_t M, int64_t kin, int r) {
  return (size_t)skinny_slices(M, kin) * (size_t)M * (size_t)skinny_rpad(r);
}

void skinny_plan(SkinnyJob* j, int64_t M) {
  const int ks = skinny_slices(M, j->kin);
  // slice length a multiple of the wave step; every slice non-empty
  j->kslice = ceil_div(ceil_div(j->kin, ks), kSkStep) * kSkStep;
  j->ks = (int)ceil_div(j->kin, j->kslice);
}

hipError_t launch_skinny(const SkinnyJob* jobs, int nj, int64_t M, int r, int r32,
                         const ReconJob* recon, hipStream_t s) {
  const int rpad = skinny_rpad(r);
  hipError_t e;
  switch (rpad) {
    case 16: e = skinny_rt<1>(jobs, nj, M, r, r32, recon, s); break;
    case 32: e = skinny_rt<2>(jobs, nj, M, r, r32, recon, s); break;
    case 64: e = skinny_rt<4>(jobs, nj, M, r, r32, recon, s); break;
    default: e = skinny_rt<8>(jobs, nj, M, r, r32, recon, s); break;
  }
  if (e != hipSuccess) return e;
  bool finish = false;
  for (int i = 0; i < nj; ++i) finish |= jobs[i].ks > 1;
  if (!finish) return hipSuccess;
  int64_t blocks = 0;
  for (int i = 0; i < nj; ++i) blocks += finish_blocks(jobs[i], M, r32);
  hipLaunchKernelGGL(k_skinny_finish, dim3((unsigned)blocks), dim3(256), 0, s, jobs[0],
                     nj > 1 ? jobs[1] : jobs[0], nj, M, r, r32, rpad);
  return hipGetLastError();
}

hipError_t launch_prep(const TransposeJob* t, int nt, const ReconJob* recon, hipStream_t s) {
  int64_t blocks = 0;
  for (int i = 0; i < nt; ++i) blocks += ceil_div(t[i].cols * t[i].ldo, 256);
  blocks += recon ? ceil_div(recon->N * recon->KB, 256) : 0;
  if (blocks == 0) return hipSuccess;
  const TransposeJob tn{};
  const ReconJob rn{};
  hipLaunchKernelGGL(k_prep, dim3((unsigned)blocks), dim3(256), 0, s, nt > 0 ? t[0] : tn,
                     nt > 1 ? t[1] : tn, nt, recon ? *recon : rn, recon ? 1 : 0);
  return hipGetLastError();
}

int lora_grad_splits(int64_t M, int64_t P) {
  // about 512 workgroups over the chip, at least 256 tokens per split (two
  // steps per wave)
  const int64_t groups = ceil_div(P, 128);
  int64_t splits = ceil_div(512, groups);
  const int64_t maxs = ceil_div(M, 256);
  if (splits > maxs) splits = maxs;
  if (splits < 1) splits = 1;
  return (int)splits;
}

hipError_t launch_lora_grads(const GradJob* jobs, int nj, int64_t M, int r, hipStream_t s) {
  hipError_t e;
  const int rpad = skinny_rpad(r);
  switch (rpad) {
    case 16: e = grads_rt<1>(jobs, nj, M, r, s); break;
    case 32: e = grads_rt<2>(jobs, nj, M, r, s); break;
    case 64: e = grads_rt<4>(jobs, nj, M, r, s); break;
    default: e = grads_rt<8>(jobs, nj, M, r, s); break;
  }
  if (e != hipSuccess) return e;
  int64_t blocks = 0;
  for (int i = 0; i < nj; ++i) blocks += ceil_div(jobs[i].P * r, 256);
  hipLaunchKernelGGL(k_lora_grad_reduce, dim3((unsigned)blocks), dim3(256), 0, s, jobs[0],
                     nj > 1 ? jobs[1] : jobs[0], nj, r);
  return hipGetLastError();
}

}  // namespace qnf4
