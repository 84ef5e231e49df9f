/*
 * Plain CPU oracle for blockwise NF4 quantisation with double quantisation.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the parity reference for the GPU
 * library: only the tests, the smoke check and the benchmark's CPU-baseline leg
 * may build, load or call it.  It shares no code, header, table or constant
 * generator with the GPU library, and the library never calls it.
 *
 * Everything here is written to be read against the method's description, not
 * to be fast: one loop per step, in the order the method applies them.
 *   - "QLoRA: Fine-Tuning a 70B on One GPU", section "NF4 Quantization": the
 *     4-bit levels form a lookup table built from the normal CDF and each weight
 *     goes to the closest level.
 *   - inquiringlines.com note "QLoRA cuts 65B model finetuning memory ...",
 *     mechanism paragraph: every quantisation bin holds an equal share of a
 *     zero-centred normal distribution; double quantisation then quantises the
 *     quantisation constants themselves.
 *   - "QLoRA: Fine-Tuning a 70B on One GPU", section "Double Quantization": the
 *     block scaling constants are themselves quantised to 8-bit integers.
 * Readings of points the pages leave open (block 64, second-level block 256,
 * tail probability 31/32, tie rule, nibble order, per-tensor mean) are listed
 * in the design notes; each function below states the one it uses.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC
 * (no contraction, so every float operation is one correctly rounded IEEE op
 * except the single explicit fmaf in the absmax reconstruction).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define NF4_BLOCK 64    /* weights per first-level absmax */
#define DQ_BLOCK 256    /* absmax constants per second-level scale */

/* ---------------------------------------------------------------- codebook */

/* Standard normal CDF, Phi(x) = erfc(-x/sqrt(2)) / 2. */
static double phi(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }

/* Inverse normal CDF by bisection on Phi: halve [lo, hi] until the midpoint
 * no longer moves in double precision.  Slow and obviously monotone. */
double oracle_phi_inv(double p) {
  double lo = -40.0, hi = 40.0;
  for (int it = 0; it < 400; ++it) {
    double mid = 0.5 * (lo + hi);
    if (mid == lo || mid == hi) break;
    if (phi(mid) < p) lo = mid; else hi = mid;
  }
  return 0.5 * (lo + hi);
}

/* The 16 NF4 levels.
 * Reading: 7 negative levels, an exact zero and 8 positive levels.  Each half
 * takes normal quantiles at evenly spaced probabilities from 1/2 up to the tail
 * probability P = 1 - 1/32 (the centre of the outermost 1/16 of the mass), and
 * is divided by Phi^-1(P) so the end levels are exactly -1 and +1.  Equal
 * probability steps between neighbouring levels on each side are the "equal
 * share of a zero-centred normal" of the inquiringlines note. */
void oracle_codebook(float out[16]) {
  const double P = 1.0 - 1.0 / 32.0;
  const double z = oracle_phi_inv(P);
  for (int j = 1; j <= 7; ++j)           /* negative half: 7 steps */
    out[7 - j] = (float)(-oracle_phi_inv(0.5 + (P - 0.5) * j / 7.0) / z);
  out[7] = 0.0f;
  for (int j = 1; j <= 8; ++j)           /* positive half: 8 steps */
    out[7 + j] = (float)(oracle_phi_inv(0.5 + (P - 0.5) * j / 8.0) / z);
}

/* --------------------------------------------------------------- quantise */

/* Index of the closest level to x, ties going to the lower index.
 * Brute force over all 16 levels; the distances are taken in double, where
 * the difference of two floats near a midpoint is exact. */
static int nearest_code(float x, const float cb[16]) {
  int best = 0;
  double bestd = fabs((double)x - (double)cb[0]);
  for (int k = 1; k < 16; ++k) {
    double d = fabs((double)x - (double)cb[k]);
    if (d < bestd) { bestd = d; best = k; }
  }
  return best;
}

/* First-level quantisation of a flat (row-major) weight array of n values.
 * Block b holds elements [64b, min(64b+64, n)).
 *   absmax[b] = max |w| over the block (exact)
 *   x = w / absmax[b]   (one IEEE float division; an all-zero block maps to 0)
 *   code = nearest level to x
 * Codes are packed two per byte, element 2i in the low nibble of byte i; a
 * missing last element leaves its high nibble 0. */
void oracle_quantize(const float* w, int64_t n, const float cb[16],
                     uint8_t* codes, float* absmax) {
  int64_t nb = (n + NF4_BLOCK - 1) / NF4_BLOCK;
  memset(codes, 0, (size_t)((n + 1) / 2));
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nb; ++b) {
    int64_t lo = b * NF4_BLOCK, hi = lo + NF4_BLOCK < n ? lo + NF4_BLOCK : n;
    float a = 0.0f;
    for (int64_t i = lo; i < hi; ++i) {
      float m = fabsf(w[i]);
      if (m > a) a = m;
    }
    absmax[b] = a;
    for (int64_t i = lo; i < hi; ++i) {
      float x = (a == 0.0f) ? 0.0f : w[i] / a;
      int c = nearest_code(x, cb);
      /* a block never straddles a byte: 64 is even */
      if (i & 1) codes[i >> 1] |= (uint8_t)(c << 4);
      else       codes[i >> 1] |= (uint8_t)c;
    }
  }
}

/* ------------------------------------------------------ double quantisation */

/* Sum of nb doubles by adjacent pairs, level by level, after padding with
 * +0.0 to a power-of-two length: level l sets v[i] = v[2i] + v[2i+1].  The
 * order is fixed so the mean is one well-defined number. */
static double pairwise_tree_sum(const float* a, int64_t nb, double* scratch) {
  int64_t len = 1;
  while (len < nb) len <<= 1;
  for (int64_t i = 0; i < len; ++i) scratch[i] = i < nb ? (double)a[i] : 0.0;
  while (len > 1) {
    len >>= 1;
    for (int64_t i = 0; i < len; ++i) scratch[i] = scratch[2 * i] + scratch[2 * i + 1];
  }
  return scratch[0];
}

/* Second-level quantisation of the nb first-level constants.
 *   mean  = float( tree_sum(absmax) / nb )            (one value per tensor)
 *   d[b]  = absmax[b] - mean                          (float)
 *   DQ block j holds constants [256j, min(256j+256, nb)):
 *     scale[j] = max |d| over the block / 127          (float division)
 *     q[b]     = scale == 0 ? 0 : clamp(rint(d[b] / scale[j]), -127, 127)
 * rint rounds half to even.  scratch needs next_pow2(nb) doubles. */
void oracle_double_quant(const float* absmax, int64_t nb, int8_t* q, float* scale,
                         float* mean, double* scratch) {
  double total = pairwise_tree_sum(absmax, nb, scratch);
  float mu = (float)(total / (double)nb);
  *mean = mu;
  int64_t nd = (nb + DQ_BLOCK - 1) / DQ_BLOCK;
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < nd; ++j) {
    int64_t lo = j * DQ_BLOCK, hi = lo + DQ_BLOCK < nb ? lo + DQ_BLOCK : nb;
    float s = 0.0f;
    for (int64_t b = lo; b < hi; ++b) {
      float d = fabsf(absmax[b] - mu);
      if (d > s) s = d;
    }
    float S = s / 127.0f;
    scale[j] = S;
    for (int64_t b = lo; b < hi; ++b) {
      float d = absmax[b] - mu;
      float r = (S == 0.0f) ? 0.0f : rintf(d / S);
      if (r > 127.0f) r = 127.0f;
      if (r < -127.0f) r = -127.0f;
      q[b] = (int8_t)r;
    }
  }
}

/* Reconstructed first-level constant: ahat[b] = fma(q[b], scale[b/256], mean),
 * one correctly rounded fused multiply-add. */
void oracle_dequant_absmax(const int8_t* q, const float* scale, float mean, int64_t nb,
                           float* ahat) {
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nb; ++b)
    ahat[b] = fmaf((float)q[b], scale[b / DQ_BLOCK], mean);
}

/* Dequantised weight: w'[i] = level[code[i]] * ahat[i/64]  (one float product). */
void oracle_dequant(const uint8_t* codes, const float* ahat, int64_t n, const float cb[16],
                    float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    int c = (i & 1) ? (codes[i >> 1] >> 4) : (codes[i >> 1] & 15);
    out[i] = cb[c] * ahat[i / NF4_BLOCK];
  }
}

/* Float to bfloat16 bits, round to nearest even (finite inputs). */
void oracle_to_bf16(const float* x, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint32_t u;
    memcpy(&u, &x[i], 4);
    uint32_t lsb = (u >> 16) & 1u;
    out[i] = (uint16_t)((u + 0x7FFFu + lsb) >> 16);
  }
}

int oracle_threads(void) {
  int t = 1;
#pragma omp parallel
  {
#pragma omp single
    {
#ifdef _OPENMP
      extern int omp_get_num_threads(void);
      t = omp_get_num_threads();
#endif
    }
  }
  return t;
}
