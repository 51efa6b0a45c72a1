/* Enumerates every non-negative finite float x (the product amax*q that an NVFP4 block
 * scale is computed from) and compares two ways of forming x/6 in float arithmetic:
 *   ieee: the correctly rounded quotient x / 6.0f;
 *   fma : q0 = RN(x * RN(1/6)), r = fma(-6, q0, x), s = fma(r, RN(1/6), q0)
 * (one residual correction of the reciprocal product, the form the GPU kernels use).
 * Writes every x whose two results differ as three uint32 (x, fma, ieee bit patterns) to
 * the file named by argv[1] and prints "checked <n> differ <m>".  Built with gcc and
 * -ffp-contract=off so that every operation rounds on its own; fmaf is the C library's
 * correctly rounded fused multiply-add. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float bits_to_float(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t float_to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* The range is split into blocks run in parallel (OpenMP); each block keeps its own list
 * of differing inputs and the lists are written in block order. */
#define NBLOCKS 256
static uint32_t* found[NBLOCKS];
static uint64_t nfound[NBLOCKS];

int main(int argc, char** argv) {
  if (argc != 2) return 2;
  FILE* out = fopen(argv[1], "wb");
  if (!out) return 2;
  const float sixth = 0.16666667163372040f;   /* RN(1/6) */
  const uint64_t total = (uint64_t)0x7F7FFFFFu + 1u;   /* +0 up to the largest finite float */
  const uint64_t per = (total + NBLOCKS - 1) / NBLOCKS;
  int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(|: failed)
  for (int b = 0; b < NBLOCKS; ++b) {
    uint64_t cap = 1024, n = 0;
    uint32_t* buf = malloc(cap * 12);
    const uint64_t lo = (uint64_t)b * per, hi = lo + per < total ? lo + per : total;
    for (uint64_t v = lo; v < hi && buf; ++v) {
      const uint32_t u = (uint32_t)v;
      const float x = bits_to_float(u);
      const float ieee = x / 6.0f;
      const float q0 = x * sixth;
      const float s = fmaf(fmaf(-6.0f, q0, x), sixth, q0);
      if (float_to_bits(s) != float_to_bits(ieee)) {
        if (n == cap) {
          cap *= 2;
          uint32_t* nb = realloc(buf, cap * 12);
          if (!nb) { free(buf); buf = NULL; break; }
          buf = nb;
        }
        buf[3 * n] = u;
        buf[3 * n + 1] = float_to_bits(s);
        buf[3 * n + 2] = float_to_bits(ieee);
        ++n;
      }
    }
    if (!buf) failed = 1;
    found[b] = buf;
    nfound[b] = n;
  }
  if (failed) return 3;
  uint64_t differ = 0;
  for (int b = 0; b < NBLOCKS; ++b) {
    fwrite(found[b], 12, nfound[b], out);
    differ += nfound[b];
    free(found[b]);
  }
  fclose(out);
  printf("checked %llu differ %llu\n", (unsigned long long)total, (unsigned long long)differ);
  return 0;
}
