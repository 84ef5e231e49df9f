// LoRA dropout on the adapter input.  PEFT's LoRA drops elements of the
// layer input X before the down-projection (the lora_dropout knob of the LoRA
// configuration, "QLoRA: Fine-Tuning a 70B on One GPU", section "Practical
// Implementation"):
//
//     D(X)[m][k] = keep(m, k) ? X[m][k] / (1 - p) : 0
//
// and only the adapter path sees D(X).  The keep decision of an element must
// be the same in the forward and in the backward, which regenerates it rather
// than storing a mask, so it comes from a counter-based generator: Philox4x32
// with 10 rounds (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As
// Easy as 1, 2, 3", SC 2011), written here from that definition.
//
// Element e = m K + k of X takes output word e mod 4 of the block whose
// counter is (e div 4 as a 64-bit value in words 0 and 1, words 2 and 3 zero)
// under the key (seed low word, seed high word); it is kept when that word is
// at least thr = floor(p 2^32).  The kernels apply the mask as a bit mask on
// the bf16 operand (dropped elements become +0) and the 1 / (1 - p) factor
// on the float32 sums.
//
// The forward can also leave the mask behind as bits (bit e % 8 of byte
// e / 8 is element e's keep decision, 1/16 of X's bytes), so that the
// backward reads it instead of running the generator again.
#pragma once

#include <cstdint>

namespace qnf4 {

struct DropoutParams {
  uint32_t thr = 0;       // keep iff word >= thr; 0 keeps everything
  float inv = 1.f;        // 1 / (1 - p); 1 without dropout
  uint32_t k0 = 0, k1 = 0;  // key: seed low and high words
  int64_t cols = 0;       // K, the row length of X
  const uint8_t* bits = nullptr;  // keep bits to read instead of the generator
  uint8_t* bits_out = nullptr;    // where a forward writes the keep bits
};

__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    // one round: two 32 x 32 -> 64-bit products of words 0 and 2; their high
    // halves mix with words 1 and 3 and the key, their low halves move over
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    c = make_uint4((uint32_t)(p1 >> 32) ^ c.y ^ k0, (uint32_t)p1,
                   (uint32_t)(p0 >> 32) ^ c.w ^ k1, (uint32_t)p0);
    // key schedule: Weyl sequence steps (golden ratio and sqrt(3) - 1)
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// N blocks at once with the round loop kept rolled: the rounds of the N
// independent blocks interleave, and the code stays small enough to sit in a
// fully unrolled loop over register-resident tiles.
template <int N>
__device__ __forceinline__ void philox4x32_10_rolled(uint4 (&c)[N], uint32_t k0, uint32_t k1) {
#pragma unroll 1
  for (int round = 0; round < 10; ++round) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const uint64_t p0 = (uint64_t)0xD2511F53u * c[i].x;
      const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[i].z;
      c[i] = make_uint4((uint32_t)(p1 >> 32) ^ c[i].y ^ k0, (uint32_t)p1,
                        (uint32_t)(p0 >> 32) ^ c[i].w ^ k1, (uint32_t)p0);
    }
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

// The four output words of block c (elements 4c .. 4c + 3).
__device__ __forceinline__ uint4 dropout_words(uint64_t c, const DropoutParams& d) {
  return philox4x32_10(make_uint4((uint32_t)c, (uint32_t)(c >> 32), 0u, 0u), d.k0, d.k1);
}

// Keep bits of the 4 elements of block c (bit i: element 4c + i).
__device__ __forceinline__ uint32_t keep_nibble(const uint4 w, uint32_t thr) {
  return (w.x >= thr ? 1u : 0u) | (w.y >= thr ? 2u : 0u) | (w.z >= thr ? 4u : 0u) |
         (w.w >= thr ? 8u : 0u);
}

// Keep bits of elements e .. e + 7 of X (e % 8 == 0; bit i: element e + i):
// the forward's stored bits when there are any, else the generator.
__device__ __forceinline__ uint32_t dropout_byte(uint64_t e, const DropoutParams& d) {
  if (d.bits) return d.bits[e >> 3];
  return keep_nibble(dropout_words(e >> 2, d), d.thr) |
         (keep_nibble(dropout_words((e >> 2) + 1, d), d.thr) << 4);
}

// And-masks for 8 bf16 from their keep bits, packed as a uint4 load holds
// them (element 2i in the low half of word i).
__device__ __forceinline__ uint4 byte_mask8(uint32_t b) {
  return make_uint4(((b & 1u) ? 0xFFFFu : 0u) | ((b & 2u) ? 0xFFFF0000u : 0u),
                    ((b & 4u) ? 0xFFFFu : 0u) | ((b & 8u) ? 0xFFFF0000u : 0u),
                    ((b & 16u) ? 0xFFFFu : 0u) | ((b & 32u) ? 0xFFFF0000u : 0u),
                    ((b & 64u) ? 0xFFFFu : 0u) | ((b & 128u) ? 0xFFFF0000u : 0u));
}

// And-masks for the 8 bf16 of elements e .. e + 7 of X (e % 8 == 0).
__device__ __forceinline__ uint4 dropout_keep8(uint64_t e, const DropoutParams& d) {
  return byte_mask8(dropout_byte(e, d));
}

__device__ __forceinline__ uint4 and4(uint4 v, uint4 m) {
  return make_uint4(v.x & m.x, v.y & m.y, v.z & m.z, v.w & m.w);
}

}  // namespace qnf4
