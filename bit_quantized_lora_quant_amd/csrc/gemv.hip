// Decode path (M <= 16 tokens): the forward streams the 4-bit weights once
// and is bound by HBM bandwidth, not by the matrix cores.
//
// Two launches per call.  The first holds two kinds of workgroup:
//  * LoRA down-projection slices: X . A^T over inner-index slices (first in
//    the grid, so they start early and leave no tail);
//  * weight streamers: 64 rows of W (128 beyond 4 tokens) by at most 8
//    64-blocks (512 inner indices), 16 rows per wave.  A streamer stages its code tile and its slice of X in LDS
//    by DMA (4 rows x 256 contiguous bytes per load), then per 64-block turns each lane's
//    16 codes into bf16 levels through a 16-entry LDS table at address 0
//    (one conflict-free 16-bit lookup per code, no multiply: a 256-entry
//    table of level pairs halves the lookups but its random rows collide in
//    the LDS banks, which cost more); two MFMAs (tokens padded to 16) give
//    the block's dot products, and the block constant -- rebuilt in
//    registers from its int8 code, the scale and the mean -- scales them as
//    they are accumulated.  No dequantised weight and no constant table is
//    written.
// The second launch adds the float32 partials in split order, adds
// bf16(s XA) . B^T and rounds to bf16.
//
// The per-block factoring computes sum_b a_b (sum_k x_k bf16(level_k)), where
// the GEMMs compute sum_k x_k bf16(level_k a_b): both round each weight once
// to bf16, and both stay inside the forward's tolerance.
#include <cstring>

#include "skinny.h"

namespace qnf4 {
namespace {

// dma16 marked non-temporal: the code tiles are streamed once and no other
// workgroup reads them again (2% faster decode than the default policy).
__device__ __forceinline__ void dma16_nt(const void* g, const void* lds) {
  const uint32_t a = (uint32_t)(uintptr_t)(lds_void_t*)lds;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :: "v"(g), "s"(a) : "m0", "memory");
}

// Weight rows per streaming workgroup: 16 per wave, 4 waves up to 4 tokens
// and 8 beyond, where the X slice in LDS is as large as the code tile and
// twice the rows share it (3% faster at 16 tokens; 3-4% slower at one, where
// the smaller workgroups keep more tiles in flight).
constexpr int dec_waves(int64_t M) { return M <= 4 ? 4 : 8; }
// 8 blocks (a 16 KB code tile) rather than 16: twice the workgroups fit in
// LDS at once, so more tiles are in flight while others compute (14-18%
// faster at 16 tokens, 6-10% at one)
constexpr int kDecBlocks = 8;     // 64-blocks per streaming workgroup (at most)
constexpr int kDecXStride = kDecBlocks * 64 + 8;   // LDS row of X (bf16), padded
constexpr int kDecRowBytes = kDecBlocks * 32;      // codes of one W row in a tile
constexpr int kDecRowChunks = kDecRowBytes / 16;   // its 16-byte chunks
constexpr int kDecDmaRows = 1024 / kDecRowBytes;   // W rows per 1 KB DMA load
constexpr int kDecXPieces = kDecBlocks / 8;        // 1 KB DMA loads per X row
static_assert(kDecRowChunks >= 16 && kDecRowChunks <= 64, "swizzle by row & 15");
constexpr int kXaWaves = 4;

struct DecodeArgs {
  const uint16_t* X;
  int64_t M, K, N;
  const uint8_t* codes;
  const int8_t* q;
  const float* scale;
  const float* mean;
  const float* f32;             // float32 block constants in place of q/scale/mean
  int splits;                   // 64-block ranges of kDecBlocks
  float* partial;               // [splits][M][N]
  int64_t xa_blocks;            // workgroups of X . A^T slices (first in the grid)
  SkinnyJob xa;                 // X . A^T slices (partials only)
};

// The LDS arena of a streaming workgroup starts with the 16 bf16 levels.
constexpr int kDecTab = 64;   // bytes reserved for the table (keeps the rest 16-byte aligned)
constexpr int dec_codes(int W) { return 16 * W * kDecBlocks * 32; }   // the code tile, 16 or 32 KB

// 8 codes (one 32-bit word, code 2j in the low nibble of byte j) -> 8 bf16
// levels as an MFMA operand.  The word is spread into 2 x nibble per byte, the
// byte offset of the level in the table at LDS address 0.
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 levels8(uint32_t c, const uint16_t* tab16) {
  uint32_t lo = (c << 1) & 0x1E1E1E1Eu, hi = (c >> 3) & 0x1E1E1E1Eu;
  asm volatile("" : "+v"(lo), "+v"(hi));   // keep the spread: one extract per lookup
  const char* t = reinterpret_cast<const char*>(tab16);
  uint32_t r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t bl = j == 0 ? (lo & 0xFFu) : (j == 3 ? (lo >> 24) : ((lo >> (8 * j)) & 0xFFu));
    const uint32_t bh = j == 0 ? (hi & 0xFFu) : (j == 3 ? (hi >> 24) : ((hi >> (8 * j)) & 0xFFu));
    u16x2_t v;
    v.x = *reinterpret_cast<const uint16_t*>(t + bl);
    v.y = *reinterpret_cast<const uint16_t*>(t + bh);
    r[j] = __builtin_bit_cast(uint32_t, v);
  }
  return make_uint4(r[0], r[1], r[2], r[3]);
}

template <int W>
__device__ __forceinline__ void decode_rows(const DecodeArgs& a, const uint16_t* tab16,
                                            uint8_t* cs, uint16_t* xs, int64_t b) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j16 = lane & 15, g = lane >> 4;
  const int split = (int)(b % a.splits);
  constexpr int kRows = 16 * W;
  const int64_t n = (b / a.splits) * kRows + 16 * wv + j16;
  const int64_t nl = n < a.N ? n : a.N - 1;
  const int64_t KB = a.K / kBlock;
  const int64_t kb0 = (int64_t)split * kDecBlocks;
  const int nblk = (int)(KB - kb0 < kDecBlocks ? KB - kb0 : kDecBlocks);   // >= 1
  const int64_t qrow = nl * KB + kb0;
  const float mu = a.f32 ? 0.0f : *a.mean;
  // Loads: constants, codes, then X, with no per-lane branch around them
  // (indices past the range are clamped and the values ignored).
  const bool grouped = !a.f32 && (KB & 3) == 0;   // int8 constants four to a word
  uint32_t qw[kDecBlocks / 4];
  float sc[kDecBlocks / 4];
  if (grouped) {
#pragma unroll
    for (int i = 0; i < kDecBlocks / 4; ++i) {
      const int ib = 4 * i < nblk ? 4 * i : (nblk - 1) & ~3;
      qw[i] = *reinterpret_cast<const uint32_t*>(a.q + qrow + ib);
      sc[i] = a.scale[(qrow + ib) / kDqBlock];   // a word never crosses a 256-group
    }
  }
  // The code tile (64 rows x 8 blocks x 32 bytes) into LDS by DMA, each load
  // four whole rows of the tile.  Read back per lane (row, block i, bytes
  // 8 g ..), a row's 16-byte chunks would all sit on the same banks; chunk q
  // of row R is stored at position q ^ (R & 15) instead.  Chunks past the
  // range re-read the last valid one (their blocks meet zero constants).
  {
    const int64_t n0 = (b / a.splits) * kRows;
    constexpr int kLoads = kRows / kDecDmaRows / W;   // per wave
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int jj = kLoads * wv + i, r = kDecDmaRows * jj + lane / kDecRowChunks;
      int64_t nr = n0 + r;
      nr = nr < a.N ? nr : a.N - 1;
      int q = (lane % kDecRowChunks) ^ (r & 15);
      q = q < 2 * nblk ? q : 2 * nblk - 1;
      dma16_nt(a.codes + nr * (a.K / 2) + 32 * kb0 + 16 * q, cs + jj * 1024);
    }
  }
  // X[m][64 kb0 .. 64 (kb0 + 16)) into LDS rows 0..M-1 by DMA: two 1 KB
  // pieces per row, spread over the waves (chunks past the range re-read the
  // last valid one; they meet zero constants)
  const int64_t kx = 64 * kb0;
  const int clim = 64 * nblk - 8;                 // last valid 8-element chunk
#pragma unroll 1
  for (int j = wv; j < kDecXPieces * (int)a.M; j += W) {
    const int m = j / kDecXPieces, pc = j % kDecXPieces, col = 512 * pc + 8 * lane;
    dma16(a.X + m * a.K + kx + (col < clim ? col : clim), xs + m * kDecXStride + 512 * pc);
  }

  // Blocks past the range get a zero constant: they add exactly nothing, and
  // the block loop below has no branch.  Four-to-a-word constants are
  // rebuilt where they are used (fewer live registers).
  float ahat_u[kDecBlocks];
  if (!grouped) {
#pragma unroll
    for (int i = 0; i < kDecBlocks; ++i) {
      const int64_t bi = qrow + (i < nblk ? i : nblk - 1);
      const float v = a.f32 ? a.f32[bi] : absmax_recon(a.q, a.scale, mu, bi);
      ahat_u[i] = i < nblk ? v : 0.f;
    }
  }
  auto ahat = [&](int i) {
    if (!grouped) return ahat_u[i];
    const float v =
        __builtin_fmaf((float)(int8_t)((qw[i / 4] >> (8 * (i & 3))) & 0xFFu), sc[i / 4], mu);
    return i < nblk ? v : 0.f;
  };
  // row M stays zero: the padding token rows of the MFMA read it
  for (int e = tid; e < kDecXStride / 8; e += 64 * W)
    *reinterpret_cast<uint4*>(xs + a.M * kDecXStride + 8 * e) = make_uint4(0u, 0u, 0u, 0u);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's DMA pieces have landed
  __syncthreads();

  const uint16_t* xrow = xs + (j16 < a.M ? j16 : a.M) * kDecXStride + 16 * g;
  const uint8_t* crow = cs + (16 * wv + j16) * kDecRowBytes + 8 * (g & 1);
  auto codes_of = [&](int i) {   // this lane's 8 code bytes of block i
    return *reinterpret_cast<const uint2*>(crow + 16 * ((2 * i + (g >> 1)) ^ j16));
  };
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  // block i: lane group g holds inner indices 16 g .. 16 g + 15 (8 per MFMA).
  // Four blocks at a time (a scheduling barrier between the groups), so that
  // only four MFMA results are live.
#pragma unroll
  for (int i = 0; i < kDecBlocks; ++i) {
    const uint4 x0 = *reinterpret_cast<const uint4*>(xrow + 64 * i);
    const uint4 x1 = *reinterpret_cast<const uint4*>(xrow + 64 * i + 8);
    f32x4_t t = {0.f, 0.f, 0.f, 0.f};
    const uint2 ci = codes_of(i);
    t = mfma16x16x32(x0, levels8(ci.x, tab16), t);
    t = mfma16x16x32(x1, levels8(ci.y, tab16), t);
    const float ah = ahat(i);
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] = __builtin_fmaf(ah, t[v], acc[v]);
    if ((i & 3) == 3) __builtin_amdgcn_sched_barrier(0);
  }
  // D[token 4g + v][row j16]
  float* base = a.partial + (int64_t)split * a.M * a.N;
  if (n < a.N) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t m = 4 * g + v;
      if (m < a.M) base[m * a.N + n] = acc[v];
    }
  }
}

// LoRA down-projection slice `sl` (512 inner indices, one 128-wide step per
// wave): partial[sl][m][j] = sum_k X[m][k] A[j][k], tokens as the 16 MFMA
// rows.  One 16-column tile of A at a time keeps the registers of this
// branch no higher than the streaming branch's.
template <int RT>
__device__ __forceinline__ void xa_slice(const DecodeArgs& a, int r, int64_t sl,
                                         float (*red)[4][64]) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j16 = lane & 15, g = lane >> 4;
  const int64_t K = a.K;
  const int64_t k = sl * (kXaWaves * kSkStep) + (int64_t)wv * kSkStep;
  const bool kwave = wv < kXaWaves;   // further waves only meet the barriers
  const bool tok = j16 < a.M;
  const uint32_t keep = tok ? 0xFFFFFFFFu : 0u;
  const uint16_t* xrow = a.X + (int64_t)(tok ? j16 : 0) * K;
  const uint16_t* A = a.xa.U;
  f32x4_t acc[RT];
#pragma unroll
  for (int jt = 0; jt < RT; ++jt) acc[jt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (kwave && k < K) {
    uint4 x[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
      x[s] = keep_if(load8_bf16(xrow, k + 32 * s + 8 * g, K, true), keep);
    if (a.xa.drop.thr != 0) {   // LoRA dropout of X (element m K + k)
      const uint64_t e = (uint64_t)(tok ? j16 : 0) * (uint64_t)K + k + 8 * g;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t kb = dropout_byte(e + 32 * s, a.xa.drop);
        x[s] = and4(x[s], byte_mask8(kb));
        if (tok && a.xa.drop.bits_out && k + 32 * s + 8 * g < K)
          a.xa.drop.bits_out[(e + 32 * s) >> 3] = (uint8_t)kb;
      }
    }
#pragma unroll
    for (int jt = 0; jt < RT; ++jt) {
      const int u = jt * 16 + j16;
      uint4 bv[4];
#pragma unroll
      for (int s = 0; s < 4; ++s)
        bv[s] = keep_if(load8_bf16(A + (int64_t)(u < r ? u : r - 1) * K, k + 32 * s + 8 * g, K, true),
                        u < r ? 0xFFFFFFFFu : 0u);
#pragma unroll
      for (int s = 0; s < 4; ++s) acc[jt] = mfma16x16x32(x[s], bv[s], acc[jt]);
    }
  }
  // wave partials added in wave order, one 16-column tile at a time
  float* part = a.xa.part + sl * a.M * (RT * 16);
#pragma unroll
  for (int jt = 0; jt < RT; ++jt) {
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (kwave) red[wv][v][lane] = acc[jt][v];
    __syncthreads();
    if (wv == 0) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float sum = red[0][v][lane];
#pragma unroll
        for (int w = 1; w < kXaWaves; ++w) sum += red[w][v][lane];
        const int64_t m = 4 * g + v;
        // (times 1 / (1 - p) under dropout; exactly 1 otherwise)
        if (m < a.M) part[m * (RT * 16) + jt * 16 + j16] = sum * a.xa.drop.inv;
      }
    }
    __syncthreads();
  }
}

// Up to kDecodeBatch independent linears (each its own W, X, adapters and
// output; shared M and rank) in one launch: their workgroups follow one
// another in the grid, and a workgroup finds its job by a scalar search of
// the kernel arguments.
struct DecodeBatch {
  DecodeArgs job[kDecodeBatch];
  int64_t first[kDecodeBatch + 1];   // first workgroup of each job
  int kind[kDecodeBatch];
  int count;
  float level[2][16];                // by kind
};

__device__ __forceinline__ int job_index(const int64_t* first, int count, int64_t item) {
  int lo = 0, hi = count - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (first[mid] <= item) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

template <int RT, int W>
__device__ __forceinline__ void decode_body(const DecodeBatch& bt, int r) {
  // one LDS arena (sized per launch) for either branch: [16 bf16 levels |
  // code tile | X rows 0..M, row M zero] or the 4 KB of XA wave partials
  extern __shared__ __attribute__((aligned(16))) uint8_t arena[];
  const int j = job_index(bt.first, bt.count, blockIdx.x);
  const DecodeArgs& a = bt.job[j];
  const int64_t b = (int64_t)blockIdx.x - bt.first[j];
  if (b < a.xa_blocks) {
    xa_slice<RT>(a, r, b, reinterpret_cast<float (*)[4][64]>(arena));
  } else {
    uint16_t* tab16 = reinterpret_cast<uint16_t*>(arena);
    uint8_t* cs = arena + kDecTab;
    uint16_t* xs = reinterpret_cast<uint16_t*>(arena + kDecTab + dec_codes(W));
    if (threadIdx.x < 16)
      tab16[threadIdx.x] = (uint16_t)(pack_bf16x2(bt.level[bt.kind[j]][threadIdx.x], 0.f) & 0xFFFF);
    decode_rows<W>(a, tab16, cs, xs, b - a.xa_blocks);   // its barrier also covers the table
  }
}

// Two entry points of one body: up to 4 tokens (4 waves), where the arena
// fits 7-8 workgroups per CU, the registers are held to 64 so that as many
// fit (3% faster at one token than the 6 that 74 registers allow); from 5
// tokens (8 waves) the X rows limit the workgroups per CU anyway and the
// registers are left free.
template <int RT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8, 8)))
void k_qlora_decode_narrow(const DecodeBatch bt, int r) {
  decode_body<RT, 4>(bt, r);
}
template <int RT>
__global__ __launch_bounds__(512) void k_qlora_decode(const DecodeBatch bt, int r) {
  decode_body<RT, 8>(bt, r);
}

// src[0] + src[stride] + ... over the first min(count, 16) terms, in order,
// with all of their loads issued first (count >= 1)
__device__ __forceinline__ float sum_first16(const float* src, int64_t stride, int count) {
  float w[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) w[i] = i < count ? src[i * stride] : 0.f;
  float v = w[0];
#pragma unroll
  for (int i = 1; i < 16; ++i)
    if (i < count) v += w[i];
  return v;
}

struct FinishJob {
  const float* partial;   // [splits][M][N]
  int splits;
  int64_t N;
  const float* xa_part;   // [ks][M][rpad]
  int ks;
  const uint16_t* B;
  uint16_t* Y;
  uint16_t* XA_out;
};
struct FinishBatch {
  FinishJob job[kDecodeBatch];
  int64_t first[kDecodeBatch + 1];   // first 256-column block of each job
  int count;
};

// Y[m][n] = bf16( sum_split partial + sum_j bf16(s XA[m][j]) B[n][j] ), with
// XA the slice sum of the down-projection.  Workgroup (n block, token m):
// first the r values of XA[m] (slices added in order, loads unrolled), then
// one output per thread; the n block 0 workgroups also write bf16(XA).
__global__ __launch_bounds__(256) void k_decode_finish(const FinishBatch fb, int64_t M, int rpad,
                                                       int r, float scale) {
  __shared__ float xs[128];
  const int jb = job_index(fb.first, fb.count, blockIdx.x);
  const float* __restrict__ partial = fb.job[jb].partial;
  const int splits = fb.job[jb].splits;
  const int64_t N = fb.job[jb].N;
  const float* __restrict__ xa_part = fb.job[jb].xa_part;
  const int ks = fb.job[jb].ks;
  const uint16_t* __restrict__ B = fb.job[jb].B;
  uint16_t* __restrict__ Y = fb.job[jb].Y;
  uint16_t* __restrict__ XA_out = fb.job[jb].XA_out;
  const int64_t nblock = (int64_t)blockIdx.x - fb.first[jb];
  const int64_t m = blockIdx.y;
  const int t = threadIdx.x;
  if (t < r) {
    const float* src = xa_part + m * rpad + t;
    const int64_t stride = M * rpad;
    float v = sum_first16(src, stride, ks);
    int k = 16;
    for (; k + 8 <= ks; k += 8) {
      float w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = src[(k + i) * stride];
#pragma unroll
      for (int i = 0; i < 8; ++i) v += w[i];
    }
    for (; k < ks; ++k) v += src[k * stride];
    const uint32_t sb = pack_bf16x2(scale * v, 0.f) & 0xFFFFu;
    xs[t] = __builtin_bit_cast(float, sb << 16);
    if (nblock == 0 && XA_out) XA_out[m * r + t] = (uint16_t)(pack_bf16x2(v, 0.f) & 0xFFFF);
  }
  __syncthreads();
  const int64_t n = nblock * 256 + t;
  if (n >= N) return;
  const float* src = partial + m * N + n;
  const int64_t stride = M * N;
  float y = sum_first16(src, stride, splits);
  int k = 16;
  for (; k + 8 <= splits; k += 8) {
    float w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = src[(k + i) * stride];
#pragma unroll
    for (int i = 0; i < 8; ++i) y += w[i];
  }
  for (; k < splits; ++k) y += src[k * stride];
  const uint16_t* brow = B + n * r;
  if ((r & 7) == 0) {
    // 16-byte loads of this row of B (rows are 16-byte aligned when r % 8 == 0)
    for (int j0 = 0; j0 < r; j0 += 8) {
      const uint4 bv = *reinterpret_cast<const uint4*>(brow + j0);
      const uint32_t w[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        y = __builtin_fmaf(xs[j0 + e], bf16_to_f32((uint16_t)(w[e >> 1] >> (16 * (e & 1)))), y);
    }
  } else {
    for (int j = 0; j < r; ++j) y = __builtin_fmaf(xs[j], bf16_to_f32(brow[j]), y);
  }
  Y[m * N + n] = (uint16_t)(pack_bf16x2(y, 0.f) & 0xFFFF);
}

template <int RT>
hipError_t decode_rt(const DecodeBatch& bt, int64_t M, int r, int64_t blocks, hipStream_t s) {
  const int W = dec_waves(M);
  const size_t stream = kDecTab + dec_codes(W) + (size_t)(M + 1) * kDecXStride * 2;
  const size_t xa = (size_t)kXaWaves * 4 * 64 * 4;
  return launch_kernel_lds(W == 4 ? k_qlora_decode_narrow<RT> : k_qlora_decode<RT>,
                           dim3((unsigned)blocks), dim3(64 * W), stream > xa ? stream : xa, s, bt,
                           r);
}

}  // namespace

int gemv_splits(int64_t N, int64_t K) {
  (void)N;
  return (int)ceil_div(K / kBlock, kDecBlocks);   // 64-block ranges of kDecBlocks
}

int decode_xa_slices(int64_t K) {
  // slices of 512 inner indices (one 128-wide step per wave)
  return (int)ceil_div(K, (int64_t)kXaWaves * kSkStep);
}

hipError_t launch_decode(const DecodeJob* jobs, int count, int64_t M, int r, float scale,
                         hipStream_t s) {
  if (count < 1 || count > kDecodeBatch) return hipErrorInvalidValue;
  DecodeBatch bt{};
  FinishBatch fb{};
  std::memcpy(bt.level[kQuantNf4], host_tables(kQuantNf4).level, sizeof(bt.level[0]));
  std::memcpy(bt.level[kQuantInt4], host_tables(kQuantInt4).level, sizeof(bt.level[0]));
  const int rpad = skinny_rpad(r);
  int64_t blocks = 0, nblocks = 0;
  for (int i = 0; i < count; ++i) {
    const DecodeJob& d = jobs[i];
    DecodeArgs& a = bt.job[i];
    a.X = d.X; a.M = M; a.K = d.K; a.N = d.N;
    a.codes = d.W.codes; a.q = d.W.q; a.scale = d.W.scale; a.mean = d.W.mean; a.f32 = d.W.f32;
    a.splits = gemv_splits(d.N, d.K);
    a.partial = d.partial;
    const int ks = decode_xa_slices(d.K);
    a.xa_blocks = ks;                          // one row group of tokens (M <= 16)
    a.xa = SkinnyJob{d.X, d.K, d.K, d.A, d.K, ks, (int64_t)kXaWaves * kSkStep, d.xa_part, scale,
                     nullptr, nullptr, nullptr, 0, 1};
    a.xa.drop = d.drop;
    bt.kind[i] = d.W.kind;
    bt.first[i] = blocks;
    blocks += ks + ceil_div(d.N, (int64_t)16 * dec_waves(M)) * a.splits;
    fb.job[i] = FinishJob{d.partial, a.splits, d.N, d.xa_part, ks, d.B, d.Y, d.XA_out};
    fb.first[i] = nblocks;
    nblocks += ceil_div(d.N, (int64_t)256);
  }
  bt.first[count] = blocks;
  bt.count = count;
  fb.first[count] = nblocks;
  fb.count = count;
  hipError_t e;
  switch (rpad) {
    case 16: e = decode_rt<1>(bt, M, r, blocks, s); break;
    case 32: e = decode_rt<2>(bt, M, r, blocks, s); break;
    case 64: e = decode_rt<4>(bt, M, r, blocks, s); break;
    default: e = decode_rt<8>(bt, M, r, blocks, s); break;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_decode_finish, dim3((unsigned)nblocks, (unsigned)M), dim3(256), 0, s, fb, M,
                     rpad, r, scale);
  return hipGetLastError();
}

}  // namespace qnf4
