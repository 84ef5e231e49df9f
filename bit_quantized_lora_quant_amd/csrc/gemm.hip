// Dequantise-in-register bf16 MFMA GEMMs of the frozen NF4 linear.
//
//   forward  Y  = X . W'^T + (s.XA) . B^T      inner dim K (+ r)
//   backward dX = dY . W'  + (s.G)  . A        inner dim N (+ r)
//
// W' is never materialised: each workgroup reads the 4-bit codes of its W
// tile, rebuilds bf16(level[code] * constant) in registers, and feeds them to
// v_mfma_f32_16x16x32_bf16 as the B operand ("QLoRA: Fine-Tuning a 70B on One
// GPU", section "Double Quantization": NF4 weights are dequantised on the fly
// to the compute dtype for the matmul; section "Practical Implementation":
// bf16 compute dtype).  The LoRA branch rides along as r extra inner columns,
// so one accumulator holds both terms.
//
// Tiling (both kernels): 256 x 256 output tile, 4 waves, each wave owning a
// 256 x 64 slab (16 x 4 MFMA tiles of 16x16, 256 fp32 accumulators per lane).
// Every wave needs all 256 rows of the activation tile, which is staged in
// LDS (double buffered, 16-byte chunks XOR-swizzled by row so the 16-byte
// reads of 8 consecutive rows hit distinct banks).  Each W element is
// dequantised exactly once per workgroup, by the one wave whose columns it
// feeds, so there is no redundant dequant work and no LDS traffic for W.
//
// MFMA 16x16x32 bf16 operands: lane l holds row (l % 16) of A / column
// (l % 16) of B and 8 consecutive inner indices of group (l / 16).  Which
// actual inner indices a group stands for is free as long as A and B agree;
// the kernels use that freedom to give each lane a contiguous run of codes.
#include "launch.h"

namespace qnf4 {
namespace {

constexpr int kTile = 256;     // output rows and columns per workgroup
constexpr int kStep = 64;      // inner indices per main-loop step
constexpr int kThreads = 256;

__device__ __forceinline__ uint4 dequant8(uint32_t c, float a, const float* lvl) {
  uint4 r;
  r.x = pack_bf16x2(lvl[c & 15u] * a, lvl[(c >> 4) & 15u] * a);
  r.y = pack_bf16x2(lvl[(c >> 8) & 15u] * a, lvl[(c >> 12) & 15u] * a);
  r.z = pack_bf16x2(lvl[(c >> 16) & 15u] * a, lvl[(c >> 20) & 15u] * a);
  r.w = pack_bf16x2(lvl[(c >> 24) & 15u] * a, lvl[(c >> 28) & 15u] * a);
  return r;
}

// Activation tile [256 rows][64 cols] bf16 -> LDS, chunk c of row i stored at
// chunk position c ^ (i & 7).  Thread t moves chunk (t & 7) of rows
// (t >> 3) + 32 * it.  Rows >= rows_valid read row rows_valid-1 (results for
// them are never stored); columns >= cols_valid read as zero.
// MODE 0: every chunk in bounds (inner dim a multiple of 64);
// MODE 1: 16-byte chunks either wholly valid or wholly past cols_valid
//         (row stride and cols_valid multiples of 8);
// MODE 2: element-wise bounds (any shape).
template <int MODE>
struct TileLoader {
  uint4 v[8];
  // element offsets of this thread's 8 rows (row * ld), 32-bit: every operand
  // here has fewer than 2^32 elements
  uint32_t roff[8];
  __device__ __forceinline__ void init(int64_t ld, int64_t row0, int64_t rows_valid) {
    const int rr = threadIdx.x >> 3;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      int64_t row = row0 + it * 32 + rr;
      row = row < rows_valid ? row : rows_valid - 1;
      roff[it] = (uint32_t)(row * ld) + (uint32_t)((threadIdx.x & 7) * 8);
    }
  }
  __device__ __forceinline__ void load(const uint16_t* __restrict__ src, uint32_t col0,
                                       uint32_t cols_valid) {
    const uint32_t col = col0 + (threadIdx.x & 7) * 8;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const uint16_t* p = src + col0 + roff[it];
      if (MODE == 0) {
        v[it] = *reinterpret_cast<const uint4*>(p);
      } else if (MODE == 1) {
        v[it] = col < cols_valid ? *reinterpret_cast<const uint4*>(p) : make_uint4(0u, 0u, 0u, 0u);
      } else {
        uint16_t e[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) e[q] = (col + q < cols_valid) ? p[q] : (uint16_t)0;
        v[it].x = e[0] | ((uint32_t)e[1] << 16);
        v[it].y = e[2] | ((uint32_t)e[3] << 16);
        v[it].z = e[4] | ((uint32_t)e[5] << 16);
        v[it].w = e[6] | ((uint32_t)e[7] << 16);
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* lds) const {
    const int c = threadIdx.x & 7, rr = threadIdx.x >> 3;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int row = it * 32 + rr;
      *reinterpret_cast<uint4*>(lds + row * kStep + ((c ^ (row & 7)) * 8)) = v[it];
    }
  }
};

__device__ __forceinline__ uint4 lds_chunk(const uint16_t* lds, int row, int chunk) {
  return *reinterpret_cast<const uint4*>(lds + row * kStep + ((chunk ^ (row & 7)) * 8));
}

// acc += A * B on v_mfma_f32_16x16x32_bf16 with the accumulator tied to its
// AGPRs.  Written as inline asm because, with all 256 AGPRs holding
// accumulators, the register allocator otherwise migrates tiles between
// AGPRs and VGPRs every iteration.  Hazards the compiler cannot see here:
// an AGPR written by VALU must settle before the first MFMA reads it (callers
// run mfma_settle() after zero-filling), and the MFMA result must settle
// before a VALU reads it (mfma_settle() after the last one).  A/B source
// registers are read at issue, so reusing them right after is safe.
typedef uint32_t u32x4v_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void mfma_acc(f32x4_t& acc, const uint4& a, const u32x4v_t& b) {
  const u32x4v_t av = {a.x, a.y, a.z, a.w};
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(av), "v"(b));
}
// Same, for callers whose B operands are assembled by the compiler right
// before the call: a VALU write of a VGPR needs two wait states before an
// MFMA reads it, and the hazard recognizer does not look inside inline asm.
__device__ __forceinline__ void mfma_acc_vw(f32x4_t& acc, const uint4& a, const u32x4v_t& b) {
  const u32x4v_t av = {a.x, a.y, a.z, a.w};
  asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(av), "v"(b));
}
__device__ __forceinline__ void mfma_settle() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"); }
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }


// Global -> LDS copy of an activation tile [256 rows][64 cols] bf16 with the
// LDS-DMA loads (global_load_lds_dwordx4: no VGPRs, no VALU).  Each load
// instruction fills 1 KB = 8 rows; wave w issues loads q = 8w .. 8w+7 for
// rows 8q .. 8q+7.  Lane t lands at row 8q + t/8, chunk position t%8, so it
// fetches global chunk (t%8) ^ (t/8): the XOR swizzle lds_chunk reads back.
template <int WAVES>
struct TileDma {
  static constexpr int kLoads = 32 / WAVES;   // 8-row loads per wave
  uint32_t off[kLoads];   // element offset of this lane's source chunk, per load
  __device__ __forceinline__ void init(int64_t ld, int64_t row0, int64_t rows_valid) {
    const int t = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int c = (t & 7) ^ (t >> 3);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      int64_t row = row0 + 8 * (kLoads * wv + i) + (t >> 3);
      row = row < rows_valid ? row : rows_valid - 1;
      off[i] = (uint32_t)(row * ld) + (uint32_t)(c * 8);
    }
  }
  __device__ __forceinline__ void issue(const uint16_t* __restrict__ src, uint32_t col0,
                                        uint16_t* lds_tile) const {
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) dma16(src + col0 + off[i], lds_tile + (kLoads * wv + i) * 512);
  }
};

__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// The two 32-bit code words of one row for one 64-wide step as used by lane
// group g: sub-step 0 takes inner indices 8g..8g+7 (bytes 4g..4g+3 of the
// row's 32-byte segment), sub-step 1 takes 32+8g.. (bytes 16+4g..).  This is
// the A-operand chunk order 4s + g, which reads LDS without bank conflicts
// (the order 2g + s costs 4 conflict cycles per read on gfx950).
__device__ __forceinline__ uint2 load_codes2(const uint8_t* p) {
  return make_uint2(*reinterpret_cast<const uint32_t*>(p),
                    *reinterpret_cast<const uint32_t*>(p + 16));
}

// Workgroup -> (split, tile): the split slices of one tile are adjacent
// workgroups; tiles are M-fastest as in tile_coords.
__device__ __forceinline__ void tile_coords_split(int64_t tiles_m, int splits, int64_t& tm,
                                                  int64_t& tn, int& split) {
  const int64_t b = blockIdx.x;
  split = (int)(b % splits);
  const int64_t t = b / splits;
  tm = t % tiles_m;
  tn = t / tiles_m;
}

__device__ __forceinline__ void tile_coords(int64_t tiles_m, int64_t& tm, int64_t& tn) {
  // M-fastest: neighbouring workgroups share one W column tile (L2 reuse).
  tm = blockIdx.x % tiles_m;
  tn = blockIdx.x / tiles_m;
}

// ------------------------------------------------------------------ forward
// Every global read of the main loop is an LDS-DMA load, three stages deep:
// at step kt the workgroup streams the X tile of step kt+2 and the code and
// absmax tiles of step kt+3 (codes run one step ahead of X because a step
// already rebuilds the next step's first sub-step).  Per stage:
//   X      [256 rows][64]  bf16, 16-byte chunks XOR-swizzled by row  32 KB
//   codes  [2 halves][256 rows][16 bytes]: half h = code bytes 16h..16h+15
//          of the row's 32-byte step segment (sub-step h)              8 KB
//   absmax [256 rows] fp32 (the block constant of the row at step kt)  1 KB
// Every wave issues the same DMA loads every step (past the slice end they
// re-read its last step into a free stage), so an end-of-step vmcnt(n), n =
// the loads of one step, leaves exactly this step's loads in flight and the
// previous step's have landed.  dX (4 waves): 8 activation, 2 code and 1
// absmax loads per wave; forward (8 waves): 4, 1 and (waves 0-3) 1.
constexpr int kDmaPerStep = 11;

template <int N>
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14)); }

// Two waves per SIMD: 8 waves, each owning a 256 x 32 slab (16 x 2 MFMA
// tiles, 128 accumulators), so that while one wave waits (for LDS data, the
// end-of-step barrier, a busy MFMA pipe) the other wave on its SIMD issues.
// (One wave per SIMD with a 256 x 64 slab runs 6-12% slower: its stalls go
// uncovered, while here every wave reads all 256 activation rows, which
// doubles the A-operand LDS reads.)
// Each W element is still dequantised once per workgroup: a wave rebuilds
// the operands of its own 32 columns.  Group i (0..31) of a step is row tile
// mt = i & 15 of sub-step s = i >> 4: two MFMAs with half a slice of dequant
// work between them (every other group one lookup of a level pair, one
// multiply per group, every other group the convert).  The levels come from
// a 256-entry table of level pairs at LDS address 0, indexed by a code byte
// (both nibbles of a byte feed one operand dword): half the lookups and byte
// extracts of a 16-entry table, bit-identical results, 0.5-2% faster.  A
// wave issues 4 X, 1 code and (waves 0-3) 1 absmax DMA load per step.
constexpr int kThreadsW8 = 512;

__global__ __attribute__((amdgpu_flat_work_group_size(kThreadsW8, kThreadsW8),
                          amdgpu_waves_per_eu(2, 2)))
void k_qlora_fwd_nt(const FwdGemmJob j0, const FwdGemmJob j1, int64_t tn_split, int64_t M,
                    int64_t K, NF4Tables tab, int r, int r32, int splits, int ksteps,
                    float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t xs0[kTile * kStep];
  __shared__ __attribute__((aligned(16))) uint16_t xs1[kTile * kStep];
  __shared__ __attribute__((aligned(16))) uint16_t xs2[kTile * kStep];
  __shared__ __attribute__((aligned(16))) uint32_t cs0[kTile * 8];
  __shared__ __attribute__((aligned(16))) uint32_t cs1[kTile * 8];
  __shared__ __attribute__((aligned(16))) uint32_t cs2[kTile * 8];
  __shared__ __attribute__((aligned(16))) float as0[kTile];
  __shared__ __attribute__((aligned(16))) float as1[kTile];
  __shared__ __attribute__((aligned(16))) float as2[kTile];
  __shared__ __attribute__((aligned(2048))) float2 lvlp[256];   // at LDS address 0
  __shared__ float lvl[16];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // 0..7
  const int j16 = lane & 15, g = lane >> 4;
  int64_t tm, tn;
  int split;
  tile_coords_split(ceil_div(M, kTile), splits, tm, tn, split);
  // two linears in one launch: the column tiles of the second follow the first's
  const bool second = tn >= tn_split;
  if (second) tn -= tn_split;
  const FwdGemmJob& J = second ? j1 : j0;
  const uint16_t* __restrict__ X = J.X;
  const uint8_t* __restrict__ codes = J.codes;
  const int64_t N = J.N;
  const float* __restrict__ ahat_t = J.ahat_t;
  const uint16_t* __restrict__ xas = J.xas;
  const uint16_t* __restrict__ B = J.B;
  uint16_t* __restrict__ Y = J.Y;
  const int64_t m0 = tm * kTile, n0 = tn * kTile;
  if (tid < 16) lvl[tid] = tab.level[tid];
  if (tid < 256) lvlp[tid] = make_float2(tab.level[tid & 15], tab.level[tid >> 4]);

  const uint32_t KTall = (uint32_t)(K / kStep);
  const uint32_t kt0 = (uint32_t)split * (uint32_t)ksteps;
  const uint32_t kt1 = kt0 + (uint32_t)ksteps < KTall ? kt0 + (uint32_t)ksteps : KTall;
  const uint32_t N32 = (uint32_t)N;

  TileDma<8> dma;   // 4 X loads per wave
  dma.init(K, m0, M);
  uint32_t cdma;    // code chunks 64 wv .. 64 wv + 63 of the stage
  {
    int64_t n = n0 + (wv & 3) * 64 + lane;
    n = n < N ? n : N - 1;
    cdma = (uint32_t)(n * (K / 2)) + (uint32_t)(16 * (wv >> 2));
  }
  uint32_t adma;    // absmax rows 64 wv + lane (waves 0-3)
  {
    int64_t n = n0 + 64 * (wv & 3) + lane;
    adma = (uint32_t)(n < N ? n : N - 1);
  }
  auto issue_codes = [&](uint32_t tc, uint32_t* cd, float* ad) {
    dma16(codes + cdma + tc * 32, cd + wv * 256);
    if (wv < 4) dma4(ahat_t + tc * N32 + adma, ad + 64 * wv);
  };
  // this lane's two W rows 32 wv + 16 nt + j16
  auto read_codes = [&](const uint32_t* cs, const float* as, uint2* c, float* a) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int row = 32 * wv + 16 * nt + j16;
      c[nt] = make_uint2(cs[row * 4 + g], cs[(256 + row) * 4 + g]);
      a[nt] = as[row];
    }
  };

  f32x4_t acc[16][2];
#pragma unroll
  for (int mt = 0; mt < 16; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      asm volatile("" : "+a"(acc[mt][nt]));
    }
  mfma_settle();

  const uint32_t tl = kt1 - 1;
  dma.issue(X, kt0 * kStep, xs0);
  issue_codes(kt0, cs0, as0);
  issue_codes(kt0 + 1 < kt1 ? kt0 + 1 : tl, cs1, as1);
  wait_vmem_all();
  __syncthreads();
  uint2 cc[2], cn[2];
  float ac[2], an[2];
  read_codes(cs0, as0, cc, ac);
  read_codes(cs1, as1, cn, an);
  dma.issue(X, (kt0 + 1 < kt1 ? kt0 + 1 : tl) * kStep, xs1);
  issue_codes(kt0 + 2 < kt1 ? kt0 + 2 : tl, cs2, as2);

  uint32_t bop[2][2][4];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int dw = 0; dw < 4; ++dw)
      bop[0][nt][dw] = pack_bf16x2(lvl[(cc[nt].x >> (8 * dw)) & 15u] * ac[nt],
                                   lvl[(cc[nt].x >> (8 * dw + 4)) & 15u] * ac[nt]);

  // Slice j (0..15) of a step rebuilds bop[s ^ 1][nt = (j >> 2) & 1][dw = j & 3]
  // during groups 2j, 2j + 1 (s = j >> 3) from code word k = j >> 2: this
  // step's .y (k < 2), the next step's .x (k < 4), and for the lookahead the
  // next step's .y (k = 4, 5).  Its level pair is looked up four groups
  // earlier (in group 2j - 4).  A code word spreads into two words of 16-bit
  // fields, the byte offsets 8 x byte of bytes 0, 2 and of bytes 1, 3.
  auto pair_at = [&](uint32_t off) { return *reinterpret_cast<const float2*>(
                                         reinterpret_cast<const char*>(lvlp) + off); };
  auto word = [&](int k) -> uint32_t {
    const int nt = k & 1;
    return k < 2 ? cc[nt].y : (k < 4 ? cn[nt].x : cn[nt].y);
  };
  uint32_t wev[2], wod[2];
  auto spread = [&](int k) {
    const uint32_t w = word(k);
    wev[k & 1] = (w & 0x00FF00FFu) << 3;
    wod[k & 1] = (w >> 5) & 0x07F807F8u;
    asm volatile("" : "+v"(wev[k & 1]), "+v"(wod[k & 1]));
  };
  auto pair_lookup = [&](int j) {   // both levels of slice j
    const int k = j >> 2, bsel = j & 3;
    const uint32_t w = (bsel & 1) ? wod[k & 1] : wev[k & 1];
    return pair_at((bsel & 2) ? (w >> 16) : (w & 0xFFFFu));
  };
  constexpr int kD = 4;
  uint4 aq[kD];
  float lq[2][4];   // slice j's levels at [half][j & 3]
  float v0 = 0.f;
  spread(0);
#pragma unroll
  for (int d = 0; d < kD; ++d) {
    aq[d] = lds_chunk(xs0, d * 16 + j16, g);
    if ((d & 1) == 0) {
      const float2 p = pair_lookup(d >> 1);
      lq[0][(d >> 1) & 3] = p.x;
      lq[1][(d >> 1) & 3] = p.y;
    }
  }

  auto step = [&](uint32_t kt, const uint16_t* xb, uint16_t* xd, uint32_t* cd, float* ad,
                  const uint32_t* cr, const float* ar, const uint16_t* xr) {
    const uint32_t tx = kt + 2 < kt1 ? kt + 2 : tl;
    const uint32_t tc = kt + 3 < kt1 ? kt + 3 : tl;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int s = i >> 4, mt = i & 15, q = i % kD;
      const int h = i + kD;
      mfma_acc(acc[mt][0], aq[q], u32x4v_t{bop[s][0][0], bop[s][0][1], bop[s][0][2], bop[s][0][3]});
      __builtin_amdgcn_sched_barrier(0);
      if ((h & 1) == 0) {
        const float2 p = pair_lookup(h >> 1);
        lq[0][(h >> 1) & 3] = p.x;
        lq[1][(h >> 1) & 3] = p.y;
      }
      if ((i & 7) == 0) dma16(X + tx * kStep + dma.off[i >> 3], xd + (4 * wv + (i >> 3)) * 512);
      if (i == 4) issue_codes(tc, cd, ad);
      if ((i & 7) == 0) spread((i >> 3) + 1);
      __builtin_amdgcn_sched_barrier(0);
      mfma_acc(acc[mt][1], aq[q], u32x4v_t{bop[s][1][0], bop[s][1][1], bop[s][1][2], bop[s][1][3]});
      __builtin_amdgcn_sched_barrier(0);
      {
        const int j = i >> 1, nt = (j >> 2) & 1, dw = j & 3;
        const float sc = s ? an[nt] : ac[nt];
        if ((i & 1) == 0) {
          v0 = lq[0][j & 3] * sc;
        } else {
          bop[s ^ 1][nt][dw] = pack_bf16x2(v0, lq[1][j & 3] * sc);
        }
      }
      if (h < 32) aq[q] = lds_chunk(xb, (h & 15) * 16 + j16, 4 * (h >> 4) + g);
      __builtin_amdgcn_sched_barrier(0);
    }
    // X(kt+1) and codes(kt+2) have landed once only this step's loads remain
    if (wv < 4) wait_vmem<6>();
    else wait_vmem<5>();
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) { cc[nt] = cn[nt]; ac[nt] = an[nt]; }
    read_codes(cr, ar, cn, an);
#pragma unroll
    for (int d = 0; d < kD; ++d) aq[d] = lds_chunk(xr, d * 16 + j16, g);
  };
  uint32_t kt = kt0;
  for (; kt + 2 < kt1; kt += 3) {
    step(kt, xs0, xs2, cs0, as0, cs2, as2, xs1);
    step(kt + 1, xs1, xs0, cs1, as1, cs0, as0, xs2);
    step(kt + 2, xs2, xs1, cs2, as2, cs1, as1, xs0);
  }
  if (kt < kt1) step(kt, xs0, xs2, cs0, as0, cs2, as2, xs1);
  if (kt + 1 < kt1) step(kt + 1, xs1, xs0, cs1, as1, cs0, as0, xs2);
  wait_vmem_all();
  mfma_settle();

  // LoRA up-projection as r32 extra inner columns (last K slice only)
  const bool bvec = (r % 8) == 0;
  const int tail = split == splits - 1 ? r32 / 32 : 0;
  for (int ts = 0; ts < tail; ++ts) {
    const int j0 = ts * 32 + g * 8;
    uint4 bb[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      int64_t n = n0 + 32 * wv + 16 * nt + j16;
      n = n < N ? n : N - 1;
      const uint16_t* p = B + n * r + j0;
      if (bvec && j0 + 8 <= r) {
        bb[nt] = *reinterpret_cast<const uint4*>(p);
      } else {
        uint16_t e[8];
        for (int q = 0; q < 8; ++q) e[q] = (j0 + q < r) ? p[q] : (uint16_t)0;
        bb[nt].x = e[0] | ((uint32_t)e[1] << 16);
        bb[nt].y = e[2] | ((uint32_t)e[3] << 16);
        bb[nt].z = e[4] | ((uint32_t)e[5] << 16);
        bb[nt].w = e[6] | ((uint32_t)e[7] << 16);
      }
    }
    uint4 a[16];   // all 16 row tiles' loads in flight at once
#pragma unroll
    for (int mt = 0; mt < 16; ++mt) {
      int64_t m = m0 + mt * 16 + j16;
      m = m < M ? m : M - 1;
      a[mt] = *reinterpret_cast<const uint4*>(xas + m * r32 + j0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mt = 0; mt < 16; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = mfma16x16x32(a[mt], bb[nt], acc[mt][nt]);
    __builtin_amdgcn_sched_barrier(0);
  }

  float* pbase = part + (int64_t)split * M * N;
#pragma unroll
  for (int mt = 0; mt < 16; ++mt) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int64_t n = n0 + 32 * wv + 16 * nt + j16;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t m = m0 + mt * 16 + 4 * g + v;
        if (m < M && n < N) {
          if (splits == 1) Y[m * N + n] = (uint16_t)(pack_bf16x2(acc[mt][nt][v], 0.f) & 0xFFFF);
          else pbase[m * N + n] = acc[mt][nt][v];
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ----------------------------------------------------------------- backward
// LoRA term of dX under dropout of X: the term passes back through the same
// keep / (1 - p) factors as the forward's down-projection input, element by
// element,
//     acc[mt][t][v] = keep(m, kc + t) / (1 - p) * sum_j (s.G)[m][j] A[j][kc + t],
//     m = m0 + 16 mt + 4 g + v,
// so it is computed first, apart from the frozen product, masked, and becomes
// the starting value of the accumulators that the frozen product's MFMAs then
// add to (nothing is added to them by VALU afterwards).  The product runs as
// the unmasked tail does: per 32 adapter indices, A's B operands once and all
// 16 row tiles' (s.G) loads in flight together.  The keep bits come from the
// generator, one block per row and 4 consecutive columns, with the round loop
// rolled over 4 blocks at a time (fully unrolled, the 16 row tiles exceed the
// unroller's budget and the accumulators fall into scratch).  The generator
// is used even where the forward stored the mask: 64 scattered byte loads
// per lane measured slower here than the 64 generator blocks.
__device__ __forceinline__ void dropout_lora_init(f32x4_t (&acc)[16][4],
                                                  const uint16_t* __restrict__ gs,
                                                  const uint16_t* __restrict__ A, int r, int r32,
                                                  int64_t M, int64_t K, int64_t m0, int64_t kcl,
                                                  int j16, int g, const DropoutParams& d) {
#pragma unroll
  for (int mt = 0; mt < 16; ++mt)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[mt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int ts = 0; ts < r32 / 32; ++ts) {
    const int j0 = ts * 32 + g * 8;
    uint2 rows[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = j0 + e;
      rows[e] = (j < r) ? *reinterpret_cast<const uint2*>(A + (int64_t)j * K + kcl)
                        : make_uint2(0u, 0u);
    }
    uint4 bb[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w = (t < 2) ? rows[e].x : rows[e].y;
        h[e] = (t & 1) ? (w >> 16) : (w & 0xFFFFu);
      }
      bb[t].x = h[0] | (h[1] << 16);
      bb[t].y = h[2] | (h[3] << 16);
      bb[t].z = h[4] | (h[5] << 16);
      bb[t].w = h[6] | (h[7] << 16);
    }
    uint4 a[16];
#pragma unroll
    for (int mt = 0; mt < 16; ++mt) {
      int64_t m = m0 + mt * 16 + j16;
      m = m < M ? m : M - 1;
      a[mt] = *reinterpret_cast<const uint4*>(gs + m * r32 + j0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mt = 0; mt < 16; ++mt)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[mt][t] = mfma16x16x32(a[mt], bb[t], acc[mt][t]);
  }
#pragma unroll
  for (int mt = 0; mt < 16; ++mt) {
    uint32_t kn[4];   // keep bits of rows v = 0..3, columns kc .. kc + 3
    uint4 wd[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint64_t c =
          ((uint64_t)(m0 + mt * 16 + 4 * g + v) * (uint64_t)K + (uint64_t)kcl) >> 2;
      wd[v] = make_uint4((uint32_t)c, (uint32_t)(c >> 32), 0u, 0u);
    }
    philox4x32_10_rolled<4>(wd, d.k0, d.k1);
#pragma unroll
    for (int v = 0; v < 4; ++v) kn[v] = keep_nibble(wd[v], d.thr);
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        acc[mt][t][v] = ((kn[v] >> t) & 1u) ? d.inv * acc[mt][t][v] : 0.f;
  }
}

// dX tile 256 (rows m) x 256 (cols k); inner loop over n in steps of 64.
// Lane (j16, g) of wave w owns output columns kc = k0 + 64w + 4*j16 + t,
// t = 0..3, one MFMA per t: so its B operand needs, for each t, 8 consecutive
// W rows of one column -- exactly the 4 codes of a 16-bit load from each of 8
// rows.  All four columns sit in one 64-block of each row.  DROP: the LoRA
// term passes through the dropout of X (dropout_lora_init).
template <int MODE, bool DROP>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(1, 1)))
void k_qlora_dx_nn(const uint16_t* __restrict__ dY, int64_t M, int64_t N,
                   const uint8_t* __restrict__ codes, int64_t K,
                   const float* __restrict__ ahat_t, NF4Tables tab,
                   const uint16_t* __restrict__ gs, const uint16_t* __restrict__ A, int r,
                   int r32, uint16_t* __restrict__ dX, DropoutParams drop) {
  __shared__ __attribute__((aligned(16))) uint16_t ys[2][kTile * kStep];
  __shared__ float lvl[16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int j16 = lane & 15, g = lane >> 4;
  int64_t tm, tn;
  tile_coords(ceil_div(M, kTile), tm, tn);
  const int64_t m0 = tm * kTile, k0 = tn * kTile;
  if (tid < 16) lvl[tid] = tab.level[tid];

  const int64_t kc = k0 + 64 * wv + 4 * j16;      // first of this lane's 4 columns
  const bool kvalid = kc < K;                       // K % 64 == 0: all 4 or none
  const int64_t kcl = kvalid ? kc : K - 4;
  const uint32_t kb = (uint32_t)(kcl / kBlock);
  const uint32_t ldc = (uint32_t)(K / 2);
  const uint32_t N32 = (uint32_t)N;
  const uint32_t NT = (uint32_t)ceil_div(N, kStep);
  const uint32_t ccol = (uint32_t)(kcl / 2);
  const uint32_t abase = kb * N32;

  f32x4_t acc[16][4];
  if constexpr (DROP) {
    dropout_lora_init(acc, gs, A, r, r32, M, K, m0, kcl, j16, g, drop);
#pragma unroll
    for (int mt = 0; mt < 16; ++mt)
#pragma unroll
      for (int t = 0; t < 4; ++t) asm volatile("" : "+a"(acc[mt][t]));
    mfma_settle();
  } else {
#pragma unroll
    for (int mt = 0; mt < 16; ++mt)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[mt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // 16 W rows per step (2 sub-steps x 8): rows n0 + 32s + 8g + e
  auto load_w = [&](uint32_t n0, uint32_t (&c)[16], float (&a)[16]) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t n = n0 + 32 * s + 8 * g + e;
        n = n < N32 ? n : N32 - 1;
        c[s * 8 + e] = *reinterpret_cast<const uint16_t*>(codes + n * ldc + ccol);
        a[s * 8 + e] = ahat_t[abase + n];
      }
  };

  TileLoader<MODE> ld;
  ld.init(N, m0, M);
  uint32_t cc[16];
  float aa[16];
  ld.load(dY, 0, N32);
  ld.store(ys[0]);
  load_w(0, cc, aa);
  __syncthreads();

  for (uint32_t it = 0; it < NT; ++it) {
    const uint32_t nn = it + 1 < NT ? it + 1 : it;   // last step re-reads itself
    ld.load(dY, nn * kStep, N32);
    uint32_t cn[16];
    float an[16];
    load_w(nn * kStep, cn, an);
    const uint16_t* yb = ys[it & 1];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      // B operands of sub-step s: column t, rows e = 0..7 paired (e, e+1)
      uint4 bop[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = lvl[(cc[s * 8 + e] >> (4 * t)) & 15u] * aa[s * 8 + e];
        bop[t].x = pack_bf16x2(v[0], v[1]);
        bop[t].y = pack_bf16x2(v[2], v[3]);
        bop[t].z = pack_bf16x2(v[4], v[5]);
        bop[t].w = pack_bf16x2(v[6], v[7]);
      }
#pragma unroll
      for (int mt = 0; mt < 16; ++mt) {
        const uint4 a = lds_chunk(yb, mt * 16 + j16, 4 * s + g);
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[mt][t] = mfma16x16x32(a, bop[t], acc[mt][t]);
      }
    }
    ld.store(ys[(it + 1) & 1]);
#pragma unroll
    for (int q = 0; q < 16; ++q) { cc[q] = cn[q]; aa[q] = an[q]; }
    __syncthreads();
  }

  // LoRA: + (s.G) . A as r32 extra inner indices (under dropout it went in
  // first, masked)
  for (int ts = 0; ts < (DROP ? 0 : r32 / 32); ++ts) {
    const int j0 = ts * 32 + g * 8;
    uint2 rows[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = j0 + e;
      rows[e] = (j < r) ? *reinterpret_cast<const uint2*>(A + (int64_t)j * K + kcl)
                        : make_uint2(0u, 0u);
    }
    uint4 bb[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w = (t < 2) ? rows[e].x : rows[e].y;
        h[e] = (t & 1) ? (w >> 16) : (w & 0xFFFFu);
      }
      bb[t].x = h[0] | (h[1] << 16);
      bb[t].y = h[2] | (h[3] << 16);
      bb[t].z = h[4] | (h[5] << 16);
      bb[t].w = h[6] | (h[7] << 16);
    }
    uint4 a[16];   // all 16 row tiles' loads in flight at once
#pragma unroll
    for (int mt = 0; mt < 16; ++mt) {
      int64_t m = m0 + mt * 16 + j16;
      m = m < M ? m : M - 1;
      a[mt] = *reinterpret_cast<const uint4*>(gs + m * r32 + j0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mt = 0; mt < 16; ++mt)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[mt][t] = mfma16x16x32(a[mt], bb[t], acc[mt][t]);
  }

  // epilogue: lane holds columns kc..kc+3 of rows 4g + v -> one 8-byte store
  if (kvalid) {
#pragma unroll
    for (int mt = 0; mt < 16; ++mt) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t m = m0 + mt * 16 + 4 * g + v;
        if (m < M) {
          uint2 o;
          o.x = pack_bf16x2(acc[mt][0][v], acc[mt][1][v]);
          o.y = pack_bf16x2(acc[mt][2][v], acc[mt][3][v]);
          *reinterpret_cast<uint2*>(dX + m * K + kc) = o;
        }
      }
    }
  }
}

// Fast dX path for N % 64 == 0 (every step full), built like the forward
// kernel: the dY tile, the code tile and the absmax tile of a step stream into
// three LDS stages by DMA (dY two steps ahead, codes and absmax three), and
// the W' operands of the next sub-step are rebuilt between the MFMAs of the
// current one.  Per stage:
//   dY     [256 rows m][64 n] bf16, chunks XOR-swizzled by row        32 KB
//   codes  8 blocks of 8 W rows x 128 bytes (the tile's 256 columns),
//          block b at b * 1088 bytes (the 64-byte pad puts the four lane
//          groups of a 16-bit code read on disjoint banks)           8.5 KB
//   absmax [4 column blocks][64 rows] fp32                             1 KB
constexpr int kCodeBlk = 1024 + 64;
template <bool DROP>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(1, 1)))
void k_qlora_dx_nn_dma(const uint16_t* __restrict__ dY, int64_t M, int64_t N,
                       const uint8_t* __restrict__ codes, int64_t K,
                       const float* __restrict__ ahat_t, NF4Tables tab,
                       const uint16_t* __restrict__ gs, const uint16_t* __restrict__ A, int r,
                       int r32, uint16_t* __restrict__ dX, int splits, int nsteps,
                       float* __restrict__ part, DropoutParams drop) {
  __shared__ __attribute__((aligned(2048))) float2 lvlp[256];   // at LDS address 0
  __shared__ float lvl[16];
  __shared__ __attribute__((aligned(16))) uint16_t ys0[kTile * kStep];
  __shared__ __attribute__((aligned(16))) uint16_t ys1[kTile * kStep];
  __shared__ __attribute__((aligned(16))) uint16_t ys2[kTile * kStep];
  __shared__ __attribute__((aligned(16))) uint8_t cs0[8 * kCodeBlk];
  __shared__ __attribute__((aligned(16))) uint8_t cs1[8 * kCodeBlk];
  __shared__ __attribute__((aligned(16))) uint8_t cs2[8 * kCodeBlk];
  __shared__ __attribute__((aligned(16))) float as0[kTile];
  __shared__ __attribute__((aligned(16))) float as1[kTile];
  __shared__ __attribute__((aligned(16))) float as2[kTile];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j16 = lane & 15, g = lane >> 4;
  int64_t tm, tn;
  int split;
  tile_coords_split(ceil_div(M, kTile), splits, tm, tn, split);
  const int64_t m0 = tm * kTile, k0 = tn * kTile;
  if (tid < 16) lvl[tid] = tab.level[tid];
  lvlp[tid] = make_float2(tab.level[tid & 15], tab.level[tid >> 4]);

  const int64_t kc = k0 + 64 * wv + 4 * j16;      // first of this lane's 4 columns
  const bool kvalid = kc < K;                       // K % 64 == 0: all 4 or none
  const int64_t kcl = kvalid ? kc : K - 4;
  // this workgroup's inner steps [it0, it1) (split over N)
  const uint32_t NTall = (uint32_t)(N / kStep);
  const uint32_t it0 = (uint32_t)split * (uint32_t)nsteps;
  const uint32_t it1 = it0 + (uint32_t)nsteps < NTall ? it0 + (uint32_t)nsteps : NTall;
  const uint32_t N32 = (uint32_t)N, ldc = (uint32_t)(K / 2);

  // DMA sources of this lane: dY rows (clamped), code block rows (columns
  // clamped into the row; such columns are never stored), absmax rows
  TileDma<4> dma;
  dma.init(N, m0, M);
  uint32_t cdma[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int blk = 2 * wv + i;
    int64_t cb = k0 / 2 + 16 * (lane & 7);
    cb = cb < (int64_t)ldc - 16 ? cb : (int64_t)ldc - 16;
    cdma[i] = (uint32_t)(8 * blk + (lane >> 3)) * ldc + (uint32_t)cb;
  }
  uint32_t adma;
  {
    int64_t kb = k0 / kBlock + wv;
    kb = kb < K / kBlock ? kb : K / kBlock - 1;
    adma = (uint32_t)kb * N32 + (uint32_t)lane;
  }
  auto issue_codes = [&](uint32_t tc, uint8_t* cd, float* ad) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      dma16(codes + cdma[i] + tc * kStep * ldc, cd + (2 * wv + i) * kCodeBlk);
    dma4(ahat_t + adma + tc * kStep, ad + 64 * wv);
  };
  // this lane's W rows of a stage: pair-word 4s + q holds the 16-bit code
  // group (columns kc..kc+3) of rows 32s + 8g + 2q (low half) and +1 (high);
  // a[8s + e] is the block constant of row 32s + 8g + e
  auto read_codes = [&](const uint8_t* cs, const float* as, uint32_t* c, float* a) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint8_t* p = cs + (4 * s2 + g) * kCodeBlk + (2 * q) * 128 + 32 * wv + 2 * j16;
        c[4 * s2 + q] = (uint32_t)*reinterpret_cast<const uint16_t*>(p) |
                        ((uint32_t)*reinterpret_cast<const uint16_t*>(p + 128) << 16);
      }
      const float4 lo = *reinterpret_cast<const float4*>(as + 64 * wv + 32 * s2 + 8 * g);
      const float4 hi = *reinterpret_cast<const float4*>(as + 64 * wv + 32 * s2 + 8 * g + 4);
      a[8 * s2 + 0] = lo.x; a[8 * s2 + 1] = lo.y; a[8 * s2 + 2] = lo.z; a[8 * s2 + 3] = lo.w;
      a[8 * s2 + 4] = hi.x; a[8 * s2 + 5] = hi.y; a[8 * s2 + 6] = hi.z; a[8 * s2 + 7] = hi.w;
    }
  };

  f32x4_t acc[16][4];
  // (under dropout, the last slice starts from the masked LoRA term)
  if (DROP && split == splits - 1) {
    dropout_lora_init(acc, gs, A, r, r32, M, K, m0, kcl, j16, g, drop);
  } else {
#pragma unroll
    for (int mt = 0; mt < 16; ++mt)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[mt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int mt = 0; mt < 16; ++mt)
#pragma unroll
    for (int t = 0; t < 4; ++t) asm volatile("" : "+a"(acc[mt][t]));
  mfma_settle();

  // prologue: dY(it0) and codes(it0), codes(it0+1) resident; then the loads
  // the first step's end-of-step wait is for: dY(it0+1), codes(it0+2)
  const uint32_t itl = it1 - 1;
  dma.issue(dY, it0 * kStep, ys0);
  issue_codes(it0, cs0, as0);
  issue_codes(it0 + 1 < it1 ? it0 + 1 : itl, cs1, as1);
  wait_vmem_all();
  __syncthreads();
  uint32_t cc[8], cn[8];
  float ac[16], an[16];
  read_codes(cs0, as0, cc, ac);
  read_codes(cs1, as1, cn, an);
  dma.issue(dY, (it0 + 1 < it1 ? it0 + 1 : itl) * kStep, ys1);
  issue_codes(it0 + 2 < it1 ? it0 + 2 : itl, cs2, as2);

  // operand set of sub-step s: bop[s][t][q] = bf16 pair of W' rows (2q, 2q+1)
  // at column kc + t
  uint32_t bop[2][4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      bop[0][t][q] = pack_bf16x2(lvl[(cc[q] >> (4 * t)) & 15u] * ac[2 * q],
                                 lvl[(cc[q] >> (16 + 4 * t)) & 15u] * ac[2 * q + 1]);

  // Slice i (0..31) of a step builds bop[s ^ 1][t = i & 3][q = (i >> 2) & 3]
  // from pair-word k = i >> 2 of the step's sequence: this step's sub-step 1
  // (k < 4), the next step's sub-step 0 (k < 8), and for the lookahead the
  // next step's sub-step 1 (k = 8, 9).  Group schedule as in the forward
  // kernel.  Byte 2 hi + c of a pair-word holds row 2q + hi at columns 2c
  // (low nibble) and 2c + 1, so an even slice looks up both rows' level
  // pairs (256-entry table at LDS address 0) for itself and the next slice:
  // half the lookups of a 16-entry table, bit-identical, about 6% faster.
  auto pair_at = [&](uint32_t off) { return *reinterpret_cast<const float2*>(
                                         reinterpret_cast<const char*>(lvlp) + off); };
  auto word = [&](int k) -> uint32_t {
    const int q = k & 3;
    return k < 4 ? cc[4 + q] : (k < 8 ? cn[q] : cn[4 + q]);
  };
  uint32_t wev[2], wod[2];
  auto spread = [&](int k) {
    const uint32_t w = word(k);
    wev[k & 1] = (w & 0x00FF00FFu) << 3;
    wod[k & 1] = (w >> 5) & 0x07F807F8u;
    asm volatile("" : "+v"(wev[k & 1]), "+v"(wod[k & 1]));
  };
  // row (hi) at columns t and t + 1 (t even): byte 2 hi + t / 2 of the pair-word
  auto pair_lookup = [&](int k, int t, int hi) {
    const uint32_t w = (t & 2) ? wod[k & 1] : wev[k & 1];
    return pair_at(hi ? (w >> 16) : (w & 0xFFFFu));
  };
  constexpr int kD = 4;
  uint4 aq[kD];
  float lqa[8], lqb[8];
  spread(0);
  spread(1);
#pragma unroll
  for (int d = 0; d < kD; ++d) {
    aq[d] = lds_chunk(ys0, d * 16 + j16, g);
    if ((d & 1) == 0) {
      const float2 pa = pair_lookup(0, d, 0), pb = pair_lookup(0, d, 1);
      lqa[d] = pa.x; lqa[d + 1] = pa.y;
      lqb[d] = pb.x; lqb[d + 1] = pb.y;
    }
  }

  auto step = [&](uint32_t it, const uint16_t* yb, uint16_t* yd, uint8_t* cd, float* ad,
                  const uint8_t* cr, const float* ar, const uint16_t* yr) {
    const uint32_t ty = it + 2 < it1 ? it + 2 : itl;
    const uint32_t tc = it + 3 < it1 ? it + 3 : itl;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int s = i >> 4, mt = i & 15, qd = i % kD;
      const int ia = i + kD, ka = ia >> 2;
      mfma_acc(acc[mt][0], aq[qd], u32x4v_t{bop[s][0][0], bop[s][0][1], bop[s][0][2], bop[s][0][3]});
      __builtin_amdgcn_sched_barrier(0);
      if ((ia & 1) == 0) {
        const float2 pa = pair_lookup(ka, ia & 3, 0);
        lqa[ia & 7] = pa.x;
        lqa[(ia + 1) & 7] = pa.y;
      }
      if ((i & 7) == 0) {   // dY tile it+2: two of this wave's eight loads
#pragma unroll
        for (int l = 2 * (i >> 3); l < 2 * (i >> 3) + 2; ++l)
          dma16(dY + ty * kStep + dma.off[l], yd + (8 * wv + l) * 512);
      }
      __builtin_amdgcn_sched_barrier(0);
      mfma_acc(acc[mt][1], aq[qd], u32x4v_t{bop[s][1][0], bop[s][1][1], bop[s][1][2], bop[s][1][3]});
      __builtin_amdgcn_sched_barrier(0);
      if ((ia & 1) == 0) {
        const float2 pb = pair_lookup(ka, ia & 3, 1);
        lqb[ia & 7] = pb.x;
        lqb[(ia + 1) & 7] = pb.y;
      }
      if ((i & 3) == 0) spread((i >> 2) + 2);
      if (i == 4) issue_codes(tc, cd, ad);
      __builtin_amdgcn_sched_barrier(0);
      mfma_acc(acc[mt][2], aq[qd], u32x4v_t{bop[s][2][0], bop[s][2][1], bop[s][2][2], bop[s][2][3]});
      __builtin_amdgcn_sched_barrier(0);
      const int k = i >> 2, t = i & 3, q = k & 3;
      const float a0 = k < 4 ? ac[8 + 2 * q] : an[2 * q];
      const float a1 = k < 4 ? ac[9 + 2 * q] : an[2 * q + 1];
      const float v0 = lqa[i & 7] * a0, v1 = lqb[i & 7] * a1;
      __builtin_amdgcn_sched_barrier(0);
      mfma_acc(acc[mt][3], aq[qd], u32x4v_t{bop[s][3][0], bop[s][3][1], bop[s][3][2], bop[s][3][3]});
      __builtin_amdgcn_sched_barrier(0);
      bop[s ^ 1][t][q] = pack_bf16x2(v0, v1);
      if (ia < 32) aq[qd] = lds_chunk(yb, (ia & 15) * 16 + j16, 4 * (ia >> 4) + g);
      __builtin_amdgcn_sched_barrier(0);
    }
    // dY(it+1) and codes(it+2) have landed once only this step's loads remain
    wait_vmem<kDmaPerStep>();
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; ++e) cc[e] = cn[e];
#pragma unroll
    for (int e = 0; e < 16; ++e) ac[e] = an[e];
    read_codes(cr, ar, cn, an);
#pragma unroll
    for (int d = 0; d < kD; ++d) aq[d] = lds_chunk(yr, d * 16 + j16, g);
  };
  // step it lives in dY stage (it - it0) % 3 and code stage (it - it0) % 3
  uint32_t it = it0;
  for (; it + 2 < it1; it += 3) {
    step(it, ys0, ys2, cs0, as0, cs2, as2, ys1);
    step(it + 1, ys1, ys0, cs1, as1, cs0, as0, ys2);
    step(it + 2, ys2, ys1, cs2, as2, cs1, as1, ys0);
  }
  if (it < it1) step(it, ys0, ys2, cs0, as0, cs2, as2, ys1);
  if (it + 1 < it1) step(it + 1, ys1, ys0, cs1, as1, cs0, as0, ys2);
  wait_vmem_all();   // nothing left in flight into LDS at exit
  mfma_settle();

  // LoRA: + (s.G) . A as r32 extra inner indices (last slice only; under
  // dropout it went in first, masked)
  const int tail = !DROP && split == splits - 1 ? r32 / 32 : 0;
  for (int ts = 0; ts < tail; ++ts) {
    const int j0 = ts * 32 + g * 8;
    uint2 rows[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = j0 + e;
      rows[e] = (j < r) ? *reinterpret_cast<const uint2*>(A + (int64_t)j * K + kcl)
                        : make_uint2(0u, 0u);
    }
    uint4 bb[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w = (t < 2) ? rows[e].x : rows[e].y;
        h[e] = (t & 1) ? (w >> 16) : (w & 0xFFFFu);
      }
      bb[t].x = h[0] | (h[1] << 16);
      bb[t].y = h[2] | (h[3] << 16);
      bb[t].z = h[4] | (h[5] << 16);
      bb[t].w = h[6] | (h[7] << 16);
    }
    uint4 a[16];   // all 16 row tiles' loads in flight at once
#pragma unroll
    for (int mt = 0; mt < 16; ++mt) {
      int64_t m = m0 + mt * 16 + j16;
      m = m < M ? m : M - 1;
      a[mt] = *reinterpret_cast<const uint4*>(gs + m * r32 + j0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mt = 0; mt < 16; ++mt)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[mt][t] = mfma16x16x32(a[mt], bb[t], acc[mt][t]);
  }

  // epilogue: lane holds columns kc..kc+3 of rows 4g + v -> one 8-byte
  // store (bf16), or float32 partials [split][M][K] when split
  float* pbase = part + (int64_t)split * M * K;
  if (kvalid) {
#pragma unroll
    for (int mt = 0; mt < 16; ++mt) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t m = m0 + mt * 16 + 4 * g + v;
        if (m < M) {
          if (splits == 1) {
            uint2 o;
            o.x = pack_bf16x2(acc[mt][0][v], acc[mt][1][v]);
            o.y = pack_bf16x2(acc[mt][2][v], acc[mt][3][v]);
            *reinterpret_cast<uint2*>(dX + m * K + kc) = o;
          } else {
            *reinterpret_cast<float4*>(pbase + m * K + kc) =
                make_float4(acc[mt][0][v], acc[mt][1][v], acc[mt][2][v], acc[mt][3][v]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Keep flags (1 kept, 0 dropped) of elements 4c .. 4c + 3 of X, one
// generator block per thread.
__global__ __launch_bounds__(256) void k_dropout_mask(int64_t n, DropoutParams d,
                                                      uint8_t* __restrict__ out) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t e = 4 * c;
  if (e >= n) return;
  const uint4 w = dropout_words((uint64_t)c, d);
  const uint32_t f = (w.x >= d.thr ? 1u : 0u) | (w.y >= d.thr ? 0x100u : 0u) |
                     (w.z >= d.thr ? 0x10000u : 0u) | (w.w >= d.thr ? 0x1000000u : 0u);
  if (e + 4 <= n && (reinterpret_cast<uintptr_t>(out) & 3) == 0) {
    *reinterpret_cast<uint32_t*>(out + e) = f;
  } else {
    const int64_t end = e + 4 < n ? e + 4 : n;
    for (int64_t i = e; i < end; ++i) out[i] = (uint8_t)((f >> (8 * (i - e))) & 1u);
  }
}

// out[i] = bf16(sum over s of part[s][i]), s in order; 4 elements per thread
__global__ __launch_bounds__(256) void k_split_reduce(const float* __restrict__ part, int splits,
                                                      int64_t count,
                                                      uint16_t* __restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= count) return;
  if (i + 4 <= count) {
    float4 acc = *reinterpret_cast<const float4*>(part + i);
    for (int s = 1; s < splits; ++s) {
      const float4 v = *reinterpret_cast<const float4*>(part + (int64_t)s * count + i);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    uint2 o;
    o.x = pack_bf16x2(acc.x, acc.y);
    o.y = pack_bf16x2(acc.z, acc.w);
    *reinterpret_cast<uint2*>(out + i) = o;
  } else {
    for (int64_t j = i; j < count; ++j) {
      float a = part[j];
      for (int s = 1; s < splits; ++s) a += part[(int64_t)s * count + j];
      out[j] = (uint16_t)(pack_bf16x2(a, 0.f) & 0xFFFF);
    }
  }
}

}  // namespace

int fwd_splits(int64_t M, int64_t N, int64_t K) {
  // Split K only when the output tiles cannot fill the chip; keep >= 8 steps
  // per slice, and make every slice non-empty.
  const int64_t tiles = ceil_div(M, kTile) * ceil_div(N, kTile);
  const int64_t steps = K / kStep;
  int64_t s = 1;
  while (s < 8 && tiles * s * 2 <= 256 && steps / (s * 2) >= 8) s *= 2;
  return (int)ceil_div(steps, ceil_div(steps, s));
}

int dx_splits(int64_t M, int64_t N, int64_t K) {
  if (N % kStep != 0) return 1;   // ragged inner dim: single-slice kernel
  return fwd_splits(M, K, N);
}

hipError_t launch_fwd_gemm(const FwdGemmJob* jobs, int count, int64_t M, int64_t K, int r,
                           int r32, int splits, float* part, int kind, hipStream_t s) {
  if (count < 1 || count > 2 || (count == 2 && splits != 1)) return hipErrorInvalidValue;
  const int ksteps = (int)ceil_div(K / kStep, splits);
  const int64_t tn0 = ceil_div(jobs[0].N, kTile);
  const int64_t tn = tn0 + (count == 2 ? ceil_div(jobs[1].N, kTile) : 0);
  const int64_t grid = ceil_div(M, kTile) * tn * splits;
  return launch_kernel(k_qlora_fwd_nt, dim3((unsigned)grid), dim3(kThreadsW8), s, jobs[0],
                       count == 2 ? jobs[1] : jobs[0], tn0, M, K, host_tables(kind), r, r32,
                       splits, ksteps, part);
}

hipError_t launch_dx_gemm(const uint16_t* dY, int64_t M, int64_t N, const uint8_t* codes,
                          int64_t K, const float* ahat_t, const uint16_t* gs, const uint16_t* A,
                          int r, int r32, uint16_t* dX, int splits, float* part, int kind,
                          const DropoutParams* drop, hipStream_t s) {
  const int64_t grid1 = ceil_div(M, kTile) * ceil_div(K, kTile);
  const bool dr = drop && drop->thr != 0 && r32 > 0;
  const DropoutParams dp = dr ? *drop : DropoutParams{};
  if (N % kStep == 0) {
    const int nsteps = (int)ceil_div(N / kStep, splits);
    launch_kernel(dr ? k_qlora_dx_nn_dma<true> : k_qlora_dx_nn_dma<false>,
                  dim3((unsigned)(grid1 * splits)), dim3(kThreads), s, dY, M, N, codes, K, ahat_t,
                  host_tables(kind), gs, A, r, r32, dX, splits, nsteps, part, dp);
  } else if (splits != 1) {
    return hipErrorInvalidValue;
  } else if (N % 8 == 0) {
    launch_kernel(dr ? k_qlora_dx_nn<1, true> : k_qlora_dx_nn<1, false>, dim3((unsigned)grid1),
                  dim3(kThreads), s, dY, M, N, codes, K, ahat_t, host_tables(kind), gs, A, r, r32,
                  dX, dp);
  } else {
    launch_kernel(dr ? k_qlora_dx_nn<2, true> : k_qlora_dx_nn<2, false>, dim3((unsigned)grid1),
                  dim3(kThreads), s, dY, M, N, codes, K, ahat_t, host_tables(kind), gs, A, r, r32,
                  dX, dp);
  }
  return hipGetLastError();
}

hipError_t launch_dropout_mask(int64_t M, int64_t K, const DropoutParams& d, uint8_t* out,
                               hipStream_t s) {
  const int64_t n = M * K;
  if (n == 0) return hipSuccess;
  if (ceil_div(ceil_div(n, 4), 256) > 0x7FFFFFFF) return hipErrorInvalidValue;
  launch_kernel(k_dropout_mask, dim3((unsigned)ceil_div(ceil_div(n, 4), 256)), dim3(256), s, n, d,
                out);
  return hipGetLastError();
}

hipError_t launch_split_reduce(const float* part, int splits, int64_t count, uint16_t* out,
                               hipStream_t s) {
  launch_kernel(k_split_reduce, dim3((unsigned)ceil_div(ceil_div(count, 4), 256)), dim3(256), s,
                part, splits, count, out);
  return hipGetLastError();
}

}  // namespace qnf4
