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

// Block constants rebuilt into [KB][N]: out[kb * N + n] = â(n * KB + kb).
// Workgroup b takes a tile of 64 rows n x 64 column blocks kb through LDS, so
// both sides are coalesced: the int8 (or float32) constants are read along
// kb (64 consecutive per row), the float32 table is written along n.
constexpr int kReconTile = 64;

__device__ __forceinline__ int64_t recon_blocks(const ReconJob& J) {
  return ceil_div(J.N, kReconTile) * ceil_div(J.KB, kReconTile);
}

__device__ __forceinline__ void recon_tile(const ReconJob& J, int64_t b,
                                           float (*tile)[kReconTile + 1]) {
  const int64_t tiles_kb = ceil_div(J.KB, kReconTile);
  const int64_t n0 = (b / tiles_kb) * kReconTile, kb0 = (b % tiles_kb) * kReconTile;
  const float mu = J.f32 ? 0.f : *J.mean;
  for (int idx = threadIdx.x; idx < kReconTile * kReconTile; idx += blockDim.x) {
    const int nl = idx / kReconTile, kl = idx % kReconTile;
    const int64_t n = n0 + nl, kb = kb0 + kl;
    if (n < J.N && kb < J.KB) {
      const int64_t e = n * J.KB + kb;
      tile[kl][nl] = J.f32 ? J.f32[e] : absmax_recon(J.q, J.scale, mu, e);
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < kReconTile * kReconTile; idx += blockDim.x) {
    const int kl = idx / kReconTile, nl = idx % kReconTile;
    const int64_t n = n0 + nl, kb = kb0 + kl;
    if (n < J.N && kb < J.KB) J.out[kb * J.N + n] = tile[kl][nl];
  }
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
  if (has_rc) {
    __shared__ float tile[kReconTile][kReconTile + 1];
    recon_tile(rc, b, tile);
  }
}

// ------------------------------------------------ skinny NT, LDS-staged
// For ranks 17..64 (RT = 2, 4) over an inner dimension that is a multiple of
// 64: a workgroup of 8 waves takes 128 rows of T (16 per wave) and one inner
// slice.  Per 64-wide step both tiles stream into LDS by DMA, three stages
// deep: T [128 rows][64] (16 KB) and U [16 RT rows][64] (2 RT KB), 16-byte
// chunks XOR-swizzled by row.  Every wave then reads all of U from LDS, so U
// crosses the L2 once per 128 rows of T instead of once per 16 (the reason:
// per 16 rows U is RT times the bytes of T, and those re-reads, not HBM, set
// the time of the per-wave form).  A wave owns its rows outright: no
// cross-wave reduction.  Slices write float32 partials [ks][M][16 RT] that
// k_skinny_finish adds in order.
constexpr int kSk2Waves = 8;
constexpr int kSk2Rows = 16 * kSk2Waves;
constexpr int kSk2Step = 64;
constexpr int kSk2TBytes = kSk2Rows * kSk2Step * 2;          // 16 KB
template <int RT>
constexpr int sk2_stage_bytes() { return kSk2TBytes + RT * 16 * kSk2Step * 2; }

__device__ __forceinline__ uint4 lds_chunk64(const uint16_t* lds, int row, int chunk) {
  return *reinterpret_cast<const uint4*>(lds + row * kSk2Step + ((chunk ^ (row & 7)) * 8));
}

template <int N>
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14)); }

template <int RT, bool DROP>
__device__ __forceinline__ void skinny2_slice(const SkinnyJob& J, int64_t M, int r, int r32,
                                              int64_t b, uint8_t* arena) {
  constexpr int kU = RT * 16;                  // U rows per tile
  constexpr int kUw = kU / 8;                  // 1 KB DMA loads of U per step (2 or ...)
  constexpr int kUper = kUw >= kSk2Waves ? kUw / kSk2Waves : 1;   // per issuing wave
  constexpr int kUwaves = kUw >= kSk2Waves ? kSk2Waves : kUw;     // waves issuing U loads
  static_assert(kUper * kUwaves == kUw, "U tile split");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j16 = lane & 15, g = lane >> 4;
  const int ks = (int)(b % J.ks);
  const int64_t mbase = (b / J.ks) * kSk2Rows;
  const int64_t kbeg = (int64_t)ks * J.kslice;
  const int64_t kend = kbeg + J.kslice < J.kin ? kbeg + J.kslice : J.kin;
  const int nsteps = (int)((kend - kbeg) / kSk2Step);   // >= 1, every step whole
  // DMA sources: T load q = 2 wv + i covers tile rows 8q .. 8q + 7; lane t
  // fetches chunk (t % 8) ^ (t / 8) of row 8q + t / 8 (rows clamped below M)
  const int c = (lane & 7) ^ (lane >> 3);
  const uint16_t* tsrc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    int64_t m = mbase + 8 * (2 * wv + i) + (lane >> 3);
    m = m < M ? m : M - 1;
    tsrc[i] = J.T + m * J.ldt + kbeg + c * 8;
  }
  const uint16_t* usrc[kUper];
#pragma unroll
  for (int i = 0; i < kUper; ++i) {
    int u = 8 * (kUper * wv + i) + (lane >> 3);
    u = u < r ? u : r - 1;   // rows past r feed output columns that are never stored
    usrc[i] = J.U + (int64_t)u * J.ldu + kbeg + c * 8;
  }
  const bool uw = wv < kUwaves;
  auto issue = [&](int st, int i) {   // DMA of step i into stage st
    uint8_t* base = arena + st * sk2_stage_bytes<RT>();
#pragma unroll
    for (int q = 0; q < 2; ++q)
      dma16(tsrc[q] + i * kSk2Step, base + (2 * wv + q) * 1024);
    if (uw) {
#pragma unroll
      for (int q = 0; q < kUper; ++q)
        dma16(usrc[q] + i * kSk2Step, base + kSk2TBytes + (kUper * wv + q) * 1024);
    }
  };
  // the wait for step i's loads, with step i + 1's (if any) still in flight
  auto wait_step = [&](bool next) {
    if (!next) { wait_vm<0>(); return; }
    if (uw) wait_vm<2 + kUper>();
    else wait_vm<2>();
  };
  const int mw = 16 * wv + j16;                       // this lane's tile row
  const int64_t mrow = mbase + mw;
  const bool dj = DROP && J.drop.thr != 0;
  const uint64_t erow = (uint64_t)(mrow < M ? mrow : M - 1) * (uint64_t)J.drop.cols + 8 * g;
  const bool wbits = DROP && J.drop.bits_out && mrow < M;

  f32x4_t acc[RT];
#pragma unroll
  for (int jt = 0; jt < RT; ++jt) acc[jt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  issue(0, 0);
  if (nsteps > 1) issue(1, 1);
  for (int i = 0; i < nsteps; ++i) {
    wait_step(i + 1 < nsteps);
    __syncthreads();                                   // step i resident; step i - 1 read
    if (i + 2 < nsteps) issue((i + 2) % 3, i + 2);
    const uint8_t* base = arena + (i % 3) * sk2_stage_bytes<RT>();
    const uint16_t* ts = reinterpret_cast<const uint16_t*>(base);
    const uint16_t* us = reinterpret_cast<const uint16_t*>(base + kSk2TBytes);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      uint4 a = lds_chunk64(ts, mw, 4 * s + g);
      if constexpr (DROP) {
        if (dj) {   // dropout of T = X, element m K + k
          const uint64_t e = erow + kbeg + (int64_t)i * kSk2Step + 32 * s;
          const uint32_t kb = dropout_byte(e, J.drop);
          a = and4(a, byte_mask8(kb));
          if (wbits) J.drop.bits_out[e >> 3] = (uint8_t)kb;
        }
      }
#pragma unroll
      for (int jt = 0; jt < RT; ++jt)
        acc[jt] = mfma16x16x32(a, lds_chunk64(us, jt * 16 + j16, 4 * s + g), acc[jt]);
    }
  }
  // lane holds P[mbase + 16 wv + 4 g + v][16 jt + j16]
  float* part = J.part + (int64_t)ks * M * (RT * 16);
#pragma unroll
  for (int jt = 0; jt < RT; ++jt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float sum = acc[jt][v];
      if constexpr (DROP) sum *= J.drop.inv;
      const int64_t m = mbase + 16 * wv + 4 * g + v;
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
}

__device__ __forceinline__ int64_t skinny2_blocks(const SkinnyJob& J, int64_t M) {
  return ceil_div(skinny_rows(J, M), kSk2Rows) * J.ks;
}

// Staged jobs (and optionally the constant table) in one launch; one LDS
// arena serves whichever branch a workgroup takes.
template <int RT, bool DROP>
__global__ __launch_bounds__(kSk2Waves * 64) void k_skinny2(SkinnyJob j0, SkinnyJob j1, int nj,
                                                            int64_t M, int r, int r32,
                                                            ReconJob rc, int has_rc) {
  __shared__ __attribute__((aligned(1024))) uint8_t arena[3 * sk2_stage_bytes<RT>()];
  int64_t b = blockIdx.x;
  const int64_t b0 = skinny2_blocks(j0, M);
  if (b < b0) { skinny2_slice<RT, DROP>(j0, M, r, r32, b, arena); return; }
  b -= b0;
  if (nj > 1) {
    const int64_t b1 = skinny2_blocks(j1, M);
    if (b < b1) { skinny2_slice<RT, DROP>(j1, M, r, r32, b, arena); return; }
    b -= b1;
  }
  if (has_rc) recon_tile(rc, b, reinterpret_cast<float (*)[kReconTile + 1]>(arena));
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
// bf16 transpose [rows, cols] -> [cols, ldo] (zero for i in [rows, ldo)), a
// 64 x 64 tile per workgroup through LDS: rows of the input are read along
// cols, rows of the output written along i, both coalesced.
constexpr int kTrTile = 64;

__device__ __forceinline__ int64_t transpose_blocks(const TransposeJob& J) {
  return ceil_div(J.ldo, kTrTile) * ceil_div(J.cols, kTrTile);
}

__device__ __forceinline__ void transpose_tile(const TransposeJob& J, int64_t b,
                                               uint16_t (*tile)[kTrTile + 2]) {
  const int64_t tiles_j = ceil_div(J.cols, kTrTile);
  const int64_t i0 = (b / tiles_j) * kTrTile, j0 = (b % tiles_j) * kTrTile;
  for (int idx = threadIdx.x; idx < kTrTile * kTrTile; idx += blockDim.x) {
    const int il = idx / kTrTile, jl = idx % kTrTile;
    const int64_t i = i0 + il, j = j0 + jl;
    if (j < J.cols) tile[jl][il] = i < J.rows ? J.in[i * J.cols + j] : (uint16_t)0;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < kTrTile * kTrTile; idx += blockDim.x) {
    const int jl = idx / kTrTile, il = idx % kTrTile;
    const int64_t i = i0 + il, j = j0 + jl;
    if (j < J.cols && i < J.ldo) J.out[j * J.ldo + i] = tile[jl][il];
  }
}

__global__ __launch_bounds__(256) void k_prep(TransposeJob t0, TransposeJob t1, int nt,
                                              ReconJob rc, int has_rc) {
  __shared__ float lds[kReconTile * (kReconTile + 1)];
  int64_t b = blockIdx.x;
  auto tr = reinterpret_cast<uint16_t (*)[kTrTile + 2]>(lds);
  if (nt > 0) {
    const int64_t n0 = transpose_blocks(t0);
    if (b < n0) { transpose_tile(t0, b, tr); return; }
    b -= n0;
  }
  if (nt > 1) {
    const int64_t n1 = transpose_blocks(t1);
    if (b < n1) { transpose_tile(t1, b, tr); return; }
    b -= n1;
  }
  if (has_rc) recon_tile(rc, b, reinterpret_cast<float (*)[kReconTile + 1]>(lds));
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
  const bool bufs = fast && RT <= 4 && tbytes <= kBufferMax && ubytes <= kBufferMax;
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
          // partials in the output's own layout, so the reduce reads them
          // contiguously
          if (p < J.P && j < r) base[J.transposed ? (int64_t)j * J.P + p : p * r + j] = s;
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
  float s = J.partial[idx];
  for (int k = 1; k < J.splits; ++k) s += J.partial[(int64_t)k * J.P * r + idx];
  J.out[idx] = J.scale * s;
}

// Four consecutive elements of the [P][r] (untransposed, ungrouped) output
// per thread: float4 loads of the partials, in slice order.
__device__ __forceinline__ void grad_reduce_vec4(const GradJob& J, int r, int64_t idx4) {
  const int64_t idx = 4 * idx4;
  const int64_t stride = J.P * r;
  if (idx >= stride) return;
  if (idx + 4 > stride) {   // the last, partial group
    for (int64_t e = idx; e < stride; ++e) grad_reduce_elem(J, r, e);
    return;
  }
  float4 s = *reinterpret_cast<const float4*>(J.partial + idx);
  for (int k = 1; k < J.splits; ++k) {
    const float4 v = *reinterpret_cast<const float4*>(J.partial + (int64_t)k * stride + idx);
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  *reinterpret_cast<float4*>(J.out + idx) =
      make_float4(J.scale * s.x, J.scale * s.y, J.scale * s.z, J.scale * s.w);
}

__device__ __host__ __forceinline__ bool grad_vec4(const GradJob& J, int r) {
  // every slice's partials 16-byte aligned too
  return J.groups == 0 && (J.P * r) % 4 == 0 &&
         ((reinterpret_cast<uintptr_t>(J.out) | reinterpret_cast<uintptr_t>(J.partial)) & 15) == 0;
}

__device__ __host__ __forceinline__ int64_t grad_reduce_blocks(const GradJob& J, int r, bool vec) {
  return ceil_div(vec ? ceil_div(J.P * r, 4) : J.P * r, 256);
}

__global__ __launch_bounds__(256) void k_lora_grad_reduce(GradJob j0, GradJob j1, int nj, int r) {
  const bool v0 = grad_vec4(j0, r);
  const int64_t b0 = grad_reduce_blocks(j0, r, v0);
  const int64_t b = blockIdx.x;
  if (b < b0) {
    if (v0) grad_reduce_vec4(j0, r, b * 256 + threadIdx.x);
    else grad_reduce_elem(j0, r, b * 256 + threadIdx.x);
    return;
  }
  if (nj > 1) {
    const int64_t e = (b - b0) * 256 + threadIdx.x;
    if (grad_vec4(j1, r)) grad_reduce_vec4(j1, r, e);
    else grad_reduce_elem(j1, r, e);
  }
}

template <int RT>
hipError_t skinny_rt(const SkinnyJob* jobs, int nj, int64_t M, int r, int r32, const ReconJob* rc,
                     hipStream_t s) {
  int64_t blocks = 0;
  for (int i = 0; i < nj; ++i) blocks += ceil_div(skinny_rows(jobs[i], M), 16) * jobs[i].ks;
  blocks += rc ? ceil_div(rc->N, kReconTile) * ceil_div(rc->KB, kReconTile) : 0;
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
hipError_t skinny2_rt(const SkinnyJob* jobs, int nj, int64_t M, int r, int r32,
                      const ReconJob* rc, hipStream_t s) {
  int64_t blocks = 0;
  for (int i = 0; i < nj; ++i) blocks += ceil_div(skinny_rows(jobs[i], M), kSk2Rows) * jobs[i].ks;
  blocks += rc ? ceil_div(rc->N, kReconTile) * ceil_div(rc->KB, kReconTile) : 0;
  const ReconJob none{};
  bool drop = false;
  for (int i = 0; i < nj; ++i) drop |= jobs[i].drop.thr != 0;
  const auto kern = drop ? k_skinny2<RT, true> : k_skinny2<RT, false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kSk2Waves * 64), 0, s, jobs[0],
                     nj > 1 ? jobs[1] : jobs[0], nj, M, r, r32, rc ? *rc : none, rc ? 1 : 0);
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

// The LDS-staged form: ranks 17..64, whole 64-wide steps, 16-byte rows.
static bool skinny_staged(const SkinnyJob& j, int r) {
  const int rp = skinny_rpad(r);
  return (rp == 32 || rp == 64) && j.kin % kSk2Step == 0 && j.ldt % 8 == 0 &&
         j.ldu % 8 == 0 && (reinterpret_cast<uintptr_t>(j.T) & 15) == 0 &&
         (reinterpret_cast<uintptr_t>(j.U) & 15) == 0;
}

// Slices of the staged form: about 256 workgroups, at least 4 steps each.
static int skinny2_slices(int64_t M, int64_t kin) {
  const int64_t groups = ceil_div(M, kSk2Rows);
  const int64_t steps = kin / kSk2Step;
  int64_t ks = ceil_div(256, groups);
  const int64_t maxs = steps / 4 > 0 ? steps / 4 : 1;
  if (ks > maxs) ks = maxs;
  if (ks < 1) ks = 1;
  return (int)ks;
}

static int skinny1_slices(int64_t M, int64_t kin) {
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

int skinny_slices(int64_t M, int64_t kin, int r) {
  // the larger of the two forms' slice counts (workspace sizing)
  const int rp = skinny_rpad(r);
  const int s1 = skinny1_slices(M, kin);
  const int s2 = (rp == 32 || rp == 64) && kin % kSk2Step == 0 ? skinny2_slices(M, kin) : 1;
  return s1 > s2 ? s1 : s2;
}

size_t skinny_part_floats(int64_t M, int64_t kin, int r) {
  return (size_t)skinny_slices(M, kin, r) * (size_t)M * (size_t)skinny_rpad(r);
}

void skinny_plan(SkinnyJob* j, int64_t M, int r) {
  j->staged = skinny_staged(*j, r) ? 1 : 0;
  const int ks = j->staged ? skinny2_slices(M, j->kin) : skinny1_slices(M, j->kin);
  // slice length a multiple of the step; every slice non-empty
  const int64_t step = j->staged ? kSk2Step : kSkStep;
  j->kslice = ceil_div(ceil_div(j->kin, ks), step) * step;
  j->ks = (int)ceil_div(j->kin, j->kslice);
}

hipError_t launch_skinny(const SkinnyJob* jobs, int nj, int64_t M, int r, int r32,
                         const ReconJob* recon, hipStream_t s) {
  const int rpad = skinny_rpad(r);
  // staged jobs in one launch (with the constant table), the rest in another
  SkinnyJob st[2], pl[2];
  int ns = 0, np = 0;
  for (int i = 0; i < nj; ++i) (jobs[i].staged ? st[ns++] : pl[np++]) = jobs[i];
  hipError_t e = hipSuccess;
  if (ns > 0) {
    e = rpad == 32 ? skinny2_rt<2>(st, ns, M, r, r32, recon, s)
                   : skinny2_rt<4>(st, ns, M, r, r32, recon, s);
    if (e != hipSuccess) return e;
    recon = nullptr;
  }
  if (np > 0) {
    switch (rpad) {
      case 16: e = skinny_rt<1>(pl, np, M, r, r32, recon, s); break;
      case 32: e = skinny_rt<2>(pl, np, M, r, r32, recon, s); break;
      case 64: e = skinny_rt<4>(pl, np, M, r, r32, recon, s); break;
      default: e = skinny_rt<8>(pl, np, M, r, r32, recon, s); break;
    }
    if (e != hipSuccess) return e;
  }
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
  for (int i = 0; i < nt; ++i) blocks += ceil_div(t[i].ldo, kTrTile) * ceil_div(t[i].cols, kTrTile);
  blocks += recon ? ceil_div(recon->N, kReconTile) * ceil_div(recon->KB, kReconTile) : 0;
  if (blocks == 0) return hipSuccess;
  const TransposeJob tn{};
  const ReconJob rn{};
  hipLaunchKernelGGL(k_prep, dim3((unsigned)blocks), dim3(256), 0, s, nt > 0 ? t[0] : tn,
                     nt > 1 ? t[1] : tn, nt, recon ? *recon : rn, recon ? 1 : 0);
  return hipGetLastError();
}

int lora_grad_splits(int64_t M, int64_t P) {
  // about 256 workgroups over the chip per job, at least 512 tokens per split
  // (four steps per wave)
  const int64_t groups = ceil_div(P, 128);
  int64_t splits = ceil_div(256, groups);
  const int64_t maxs = ceil_div(M, 512);
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
  for (int i = 0; i < nj; ++i) blocks += grad_reduce_blocks(jobs[i], r, grad_vec4(jobs[i], r));
  hipLaunchKernelGGL(k_lora_grad_reduce, dim3((unsigned)blocks), dim3(256), 0, s, jobs[0],
                     nj > 1 ? jobs[1] : jobs[0], nj, r);
  return hipGetLastError();
}

}  // namespace qnf4
