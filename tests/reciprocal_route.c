/* Exhaustive host check of the quantisers' reciprocal route for dynamic scales.
 *
 * FP8-E4M3 and INT8 per-tensor scaling ("Deploying 2:4 Sparsity with FP8 on
 * Hopper", pipeline step 3 and its INT8 W8A8 recipe) code the float32 quotient
 * v / s, s = fp32(amax / D) with D = 448 (E4M3) or 127 (INT8).  The GPU kernels
 * form that quotient as q0 = v * r with r = fp32(1 / s), then one correction
 * with the exact residual: q = copysign(fma(fma(-q0, s, v), r, q0), v).  This
 * program compares the code of that q with the code of the correctly rounded
 * v / s for every finite bf16 amax key in [kmin, 0x7F80) and every bf16 v with
 * |v| <= amax, and prints the number of pairs whose codes differ.
 *
 *   reciprocal_route e4m3|int8 KMIN_HEX
 *
 * Built with -ffp-contract=off and without fast-math, so that every operation
 * is one IEEE float32 operation (fmaf is the fused one), denormals kept.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float bf16(uint32_t h) {
  const uint32_t u = h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* E4M3 (OCP: no infinities, largest finite 448) of v clamped to +-448, round to
 * nearest even, found by comparing with every code's value. */
static uint8_t e4m3(float v) {
  const uint8_t sign = signbit(v) ? 0x80 : 0;
  double a = fabs((double)v);
  if (a > 448.0) a = 448.0;
  double best = 0.0;
  int bc = 0;
  for (int c = 0; c < 0x7F; ++c) {
    const int e = c >> 3, m = c & 7;
    const double val = e == 0 ? m * ldexp(1.0, -9) : (8 + m) * ldexp(1.0, e - 10);
    const double d = fabs(val - a), db = fabs(best - a);
    if (d < db || (d == db && (c & 1) == 0 && (bc & 1) == 1)) {
      best = val;
      bc = c;
    }
  }
  return (uint8_t)(sign | bc);
}

static int i8(float v) { return (int)fminf(fmaxf(rintf(v), -127.0f), 127.0f); }

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s e4m3|int8 KMIN_HEX\n", argv[0]);
    return 2;
  }
  const int int8 = strcmp(argv[1], "int8") == 0;
  const uint32_t kmin = (uint32_t)strtoul(argv[2], NULL, 16);
  const float D = int8 ? 127.0f : 448.0f;
  long long pairs = 0, differ = 0, abnormal = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(+ : pairs, differ, abnormal)
  for (uint32_t key = kmin; key < 0x7F80u; ++key) {
    const float s = bf16(key) / D, r = 1.0f / s;
    if (!(isnormal(s) && isnormal(r))) {
      abnormal++;
      continue;
    }
    for (uint32_t h = 0; h < 0x10000u; ++h) {
      if ((h & 0x7FFFu) > key) continue;
      const float v = bf16(h);
      const float q = v / s;
      const float q0 = v * r;
      const float qf = copysignf(fmaf(fmaf(-q0, s, v), r, q0), v);
      pairs++;
      if (q == qf && signbit(q) == signbit(qf)) continue;
      if (int8 ? i8(q) != i8(qf) : e4m3(q) != e4m3(qf)) differ++;
    }
  }
  printf("%s keys %04x..7f7f: %lld pairs, %lld codes differ, %lld keys with a subnormal scale or reciprocal\n",
         int8 ? "int8" : "e4m3", kmin, pairs, differ, abnormal);
  return 0;
}
