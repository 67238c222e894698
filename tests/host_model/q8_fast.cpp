// Host check of the q8_1 block quantizer's fast path (q8.hpp,
// q8_quant_block): the reciprocal-based codes with exact fallback must equal
// roundf(x / d) with the IEEE fp32 quotient, for every value. Compiled for
// the host with QMV_HOST_MODEL (IEEE fp32 arithmetic, no contraction), over
// random blocks at many scales and over values placed within a few ulps of
// the half-integer code boundaries, where an inexact quotient would change
// the code. Prints the number of mismatches and how often the exact
// fallback ran; exits non-zero on any mismatch.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <random>

#include "q8.hpp"

using namespace qmv;

static long mismatches = 0, blocks = 0, values = 0;

static uint32_t bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

// 32 values of one block: the fast block quantizer (8 words of 4) against
// the exact definition, value by value.
static void check_block(const float (&x)[32]) {
  float amax = 0.0f;
  for (float v : x) amax = fmaxf(amax, fabsf(v));
  const float d = q8_scale(amax);
  u32x4 v[8];
  for (int k = 0; k < 8; ++k)
    for (int e = 0; e < 4; ++e) v[k][e] = bits(x[4 * k + e]);
  uint32_t out[8];
  int sum = 0;
  q8_quant_block(v, d, out, sum);
  int ref_sum = 0;
  for (int i = 0; i < 32; ++i) {
    const int ref = d == 0.0f ? 0 : static_cast<int>(roundf(x[i] / d));
    ref_sum += ref;
    // stored as a byte: with a subnormal d a quotient can exceed 127 and
    // wraps the same way on both sides
    const int got = static_cast<int8_t>(out[i / 4] >> (8 * (i % 4)));
    if (got != static_cast<int8_t>(ref)) {
      if (mismatches < 10)
        printf("MISMATCH x=%a d=%a got %d want %d\n", x[i], d, got, ref);
      ++mismatches;
    }
  }
  if (sum != ref_sum) ++mismatches;
  ++blocks;
  values += 32;
}

int main(int argc, char** argv) {
  const long n_random = argc > 1 ? atol(argv[1]) : 200000;
  std::mt19937_64 rng(12345);
  std::normal_distribution<float> nd(0.0f, 1.0f);
  std::uniform_real_distribution<double> ud(0.0, 1.0);
  float x[32];

  // random blocks over scales from subnormal to large
  for (long b = 0; b < n_random; ++b) {
    const float scale = static_cast<float>(pow(2.0, -140.0 + 250.0 * ud(rng)));
    for (float& v : x) v = nd(rng) * scale;
    if (b % 7 == 0) x[b % 32] = 0.0f;
    check_block(x);
  }
  // values within a few ulps of (k + 1/2) * d, for random d and every k
  long near_cases = 0;
  for (long b = 0; b < n_random / 4; ++b) {
    const float amax = static_cast<float>(pow(2.0, -120.0 + 240.0 * ud(rng))) * (1.0f + static_cast<float>(ud(rng)));
    const float d = q8_scale(amax);
    x[0] = (b & 1) ? -amax : amax;
    for (int i = 1; i < 32; ++i) {
      const int k = static_cast<int>(ud(rng) * 127.0);       // 0..126
      float t = (static_cast<float>(k) + 0.5f) * d;
      const int steps = static_cast<int>(ud(rng) * 17.0) - 8;  // -8..8 ulps
      for (int s = 0; s < abs(steps); ++s) t = nextafterf(t, steps > 0 ? INFINITY : 0.0f);
      if (fabsf(t) > amax) t = amax;
      x[i] = (i & 1) ? -t : t;
      ++near_cases;
    }
    check_block(x);
  }
  // exact ties at d = 1 and all-equal blocks
  for (int k = -127; k <= 126; ++k) {
    x[0] = 127.0f;
    for (int i = 1; i < 32; ++i) x[i] = static_cast<float>(k) + 0.5f;
    check_block(x);
    for (float& v : x) v = static_cast<float>(k) * 0.37f;
    check_block(x);
  }
  printf("q8 fast path: %ld blocks, %ld values (%ld near a code boundary), %ld mismatches\n", blocks, values,
         near_cases, mismatches);
  return mismatches ? 1 : 0;
}
