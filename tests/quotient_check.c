/* The writer's span / d for d = 3 and 15: q0 = span * rn(1/d), then
   q0 + (span - q0 d) rn(1/d) with both steps fused (fmaf), compared with the
   IEEE quotient span / d for fp32 spans from 0 to 2^20 (bit patterns
   0 .. 0x49800000, every `stride`-th).  Prints the number of differences. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int main(int argc, char** argv) {
  const uint32_t stride = argc > 1 ? (uint32_t)strtoul(argv[1], NULL, 10) : 1u;
  const float ds[2] = {3.0f, 15.0f};
  unsigned long long bad = 0, n = 0;
  for (int k = 0; k < 2; ++k) {
    const float d = ds[k], r = 1.0f / d;
    for (uint32_t b = 0; b <= 0x49800000u; b += stride) {
      float x;
      memcpy(&x, &b, 4);
      const float q = x / d;
      const float q0 = x * r;
      const float e = fmaf(-q0, d, x);
      const float q1 = fmaf(e, r, q0);
      ++n;
      if (memcmp(&q, &q1, 4) != 0) ++bad;
    }
  }
  printf("%llu %llu\n", bad, n);
  return 0;
}
