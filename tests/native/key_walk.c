/*
 * Exhaustive check of the oracle's order-preserving key over all 2^32 fp32
 * bit patterns, against libm's nextafterf as the independent definition of
 * "the next larger float":
 *   - for every non-NaN x below +inf: key(nextafterf(x, +inf)) > key(x);
 *   - key(+0.0) > key(-0.0) (the reading for signed zeros);
 *   - every +NaN key lies above key(+inf), every -NaN key below key(-inf).
 * The strictly increasing chain from -inf to +inf makes the key injective on
 * all non-NaN patterns and consistent with float order.
 * Usage: key_walk [shard nshards] walks the patterns u with (u >> 24) %
 * nshards == shard (all by default).  Prints "OK <count>" and exits 0 on
 * success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint32_t ets_oracle_order_key(uint32_t bits);

static float as_float(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}
static uint32_t as_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

int main(int argc, char** argv) {
  const uint32_t shard = argc > 2 ? (uint32_t)atoi(argv[1]) : 0;
  const uint32_t nshards = argc > 2 ? (uint32_t)atoi(argv[2]) : 1;
  const uint32_t kinf = ets_oracle_order_key(0x7F800000u);
  const uint32_t kninf = ets_oracle_order_key(0xFF800000u);
  uint64_t checked = 0;
  uint32_t u = 0;
  do {
    if (((u >> 24) % nshards) != shard) {
      u += 1u << 24;
      continue;
    }
    const uint32_t ku = ets_oracle_order_key(u);
    const float x = as_float(u);
    if (isnan(x)) {
      if (!(u & 0x80000000u) && !(ku > kinf)) {
        printf("FAIL +NaN %08x key %08x not above +inf\n", u, ku);
        return 1;
      }
      if ((u & 0x80000000u) && !(ku < kninf)) {
        printf("FAIL -NaN %08x key %08x not below -inf\n", u, ku);
        return 1;
      }
    } else if (!(isinf(x) && x > 0)) {
      const uint32_t v = as_bits(nextafterf(x, INFINITY));
      const uint32_t kv = ets_oracle_order_key(v);
      if (!(kv > ku)) {
        printf("FAIL x=%08x next=%08x keys %08x %08x\n", u, v, ku, kv);
        return 1;
      }
      ++checked;
    }
    ++u;
  } while (u != 0);
  if (!(ets_oracle_order_key(0x00000000u) > ets_oracle_order_key(0x80000000u))) {
    printf("FAIL +0.0 not above -0.0\n");
    return 1;
  }
  printf("OK %llu\n", (unsigned long long)checked);
  return 0;
}
