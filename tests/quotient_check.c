/* Checks, on the host, the division shortcut the NVFP4 quantizer uses for a
 * bf16 magnitude a and a block scale d (a positive fp32):
 *   r = RN(1/d); q = RN(a * r); e = RN(a - q * d) (one fma, exact);
 *   y = RN(q + e * r) (one fma)  ==  RN(a / d).
 * Binary scaling of a or d scales every step exactly while nothing under-
 * or overflows, so it suffices to take a in [1, 2) with each of the 128
 * bf16 significands and d in [1, 2) with its 2^23 fp32 significands.
 * Usage: quotient_check STEP  (d significands 0, STEP, 2 STEP, ...; 1 = all).
 * Prints the number of pairs checked and of mismatches; exit status 1 on a
 * mismatch. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

int main(int argc, char** argv) {
  const uint32_t step = argc > 1 ? (uint32_t)strtoul(argv[1], NULL, 10) : 1u;
  uint64_t checked = 0, bad = 0;
  for (uint32_t ma = 0; ma < 128; ++ma) {
    /* volatile stops the compiler from folding or fusing the steps */
    volatile float a = f_of(0x3F800000u | (ma << 16));
    for (uint32_t md = 0; md < (1u << 23); md += step) {
      volatile float d = f_of(0x3F800000u | md);
      volatile float r = 1.0f / d;
      volatile float q = a * r;
      volatile float e = fmaf(-q, d, a);
      volatile float y = fmaf(e, r, q);
      volatile float ref = a / d;
      ++checked;
      if (u_of(y) != u_of(ref)) {
        if (bad < 5) printf("mismatch a=%a d=%a y=%a ref=%a\n", (double)a, (double)d, (double)y, (double)ref);
        ++bad;
      }
    }
  }
  printf("checked %llu mismatches %llu\n", (unsigned long long)checked, (unsigned long long)bad);
  return bad != 0;
}
