/*
 * Runs the CPU oracle (oracle/ets_oracle.c, linked in) under AddressSanitizer
 * and UndefinedBehaviorSanitizer over rows of every shape the checks use:
 * empty and one-score rows, rows shorter and longer than k, lengths outside
 * [0, L], heavy ties, special bit patterns, page sizes that are not powers of
 * two, ragged rows with negative lengths, and several thread counts.  Every
 * result is also compared with the rank definition of the selected set
 * (position i is selected iff #{j : key_j > key_i} + #{j < i : key_j =
 * key_i} < k), computed here by brute force; a sanitizer report or a
 * mismatch makes the program exit non-zero.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int ets_oracle_topk_raw(const uint32_t* bits, int64_t row_stride, int32_t B, int32_t L,
                        const int32_t* lens, int32_t k, int32_t* out, int64_t out_stride,
                        int nthreads);
int ets_oracle_topk_paged(const uint32_t* bits, int64_t row_stride, int32_t B, int32_t L,
                          const int32_t* seq_lens, const int32_t* page_table, int64_t pt_stride,
                          int32_t page_size, int32_t k, int32_t* out, int64_t out_stride,
                          int nthreads);
int ets_oracle_topk_ragged(const uint32_t* packed_bits, const int32_t* row_starts,
                           const int32_t* lengths, int32_t B, int32_t k, int32_t* out,
                           int64_t out_stride, int nthreads);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t next32(void) { /* xorshift64* */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}

static uint32_t key_of(uint32_t u) { return (u & 0x80000000u) ? ~u : (u | 0x80000000u); }

static uint32_t draw(int kind) {
  static const uint32_t special[] = {0x00000000u, 0x80000000u, 0x00000001u, 0x807FFFFFu,
                                     0x7F800000u, 0xFF800000u, 0x7FC00000u, 0xFFFFFFFFu,
                                     0x3F800000u, 0xBF800000u};
  switch (kind) {
    case 0: return next32();                               /* any pattern */
    case 1: return 0x3F800000u + (next32() % 5u);          /* heavy ties */
    case 2: return special[next32() % 10u];                /* special values */
    default: return next32() & 0x007FFFFFu;                /* subnormals */
  }
}

/* The selected positions of one row by the rank definition, as a sorted
 * list of row-local positions (m = min(k, n) of them). */
static int32_t brute(const uint32_t* row, int32_t n, int32_t k, int32_t* sel) {
  int32_t m = 0;
  for (int32_t i = 0; i < n; ++i) {
    const uint32_t ki = key_of(row[i]);
    int32_t rank = 0;
    for (int32_t j = 0; j < n; ++j) {
      const uint32_t kj = key_of(row[j]);
      if (kj > ki || (kj == ki && j < i)) ++rank;
    }
    if (rank < k) sel[m++] = i;
  }
  return m;
}

static int cmp_i32(const void* a, const void* b) {
  const int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

static int failures = 0;

/* out row (k slots) against the expected mapped positions want[0..m). */
static void check_row(const char* what, int32_t b, const int32_t* out, int32_t k,
                      int32_t* want, int32_t m) {
  int32_t* got = (int32_t*)malloc(sizeof(int32_t) * (size_t)(k > 0 ? k : 1));
  memcpy(got, out, sizeof(int32_t) * (size_t)k);
  qsort(got, (size_t)k, sizeof(int32_t), cmp_i32);
  qsort(want, (size_t)m, sizeof(int32_t), cmp_i32);
  int32_t pad = 0;
  for (int32_t i = 0; i < k; ++i) pad += got[i] == -1;
  int ok = pad == k - m;
  for (int32_t i = 0; ok && i < m; ++i) ok = got[pad + i] == want[i];
  if (!ok) {
    fprintf(stderr, "%s: row %d differs from the rank definition (m=%d, pad=%d)\n", what, b, m,
            pad);
    ++failures;
  }
  free(got);
}

int main(void) {
  const int32_t Ls[] = {0, 1, 2, 7, 64, 100, 257};
  const int32_t ks[] = {1, 2, 3, 8, 64, 300};
  const int threads[] = {1, 3};
  for (size_t li = 0; li < sizeof(Ls) / sizeof(Ls[0]); ++li) {
    for (int kind = 0; kind < 4; ++kind) {
      const int32_t L = Ls[li], B = 5;
      const int64_t stride = L + 3;
      uint32_t* bits = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)(B * stride + 1));
      for (int64_t i = 0; i < B * stride; ++i) bits[i] = draw(kind);
      int32_t lens[5] = {L, L / 2, 0, -7, L + 50}; /* clamped to [0, L] */
      const int32_t ps = 3;                        /* not a power of two */
      const int32_t npg = (L + ps - 1) / ps + 1;
      int32_t* pt = (int32_t*)malloc(sizeof(int32_t) * (size_t)(B * npg));
      for (int32_t i = 0; i < B * npg; ++i) pt[i] = (int32_t)(next32() % 1000u);
      for (size_t ki = 0; ki < sizeof(ks) / sizeof(ks[0]); ++ki) {
        const int32_t k = ks[ki];
        int32_t* out = (int32_t*)malloc(sizeof(int32_t) * (size_t)(B * k));
        int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)(L + 1));
        for (size_t ti = 0; ti < 2; ++ti) {
          for (int32_t i = 0; i < B * k; ++i) out[i] = 0x5A5A5A5A;
          if (ets_oracle_topk_raw(bits, stride, B, L, lens, k, out, k, threads[ti]) != 0) ++failures;
          for (int32_t b = 0; b < B; ++b) {
            const int32_t n = lens[b] < 0 ? 0 : (lens[b] > L ? L : lens[b]);
            const int32_t m = brute(bits + b * stride, n, k, sel);
            check_row("raw", b, out + b * k, k, sel, m);
          }
          if (ets_oracle_topk_paged(bits, stride, B, L, lens, pt, npg, ps, k, out, k, threads[ti]) != 0)
            ++failures;
          for (int32_t b = 0; b < B; ++b) {
            const int32_t n = lens[b] < 0 ? 0 : (lens[b] > L ? L : lens[b]);
            const int32_t m = brute(bits + b * stride, n, k, sel);
            for (int32_t i = 0; i < m; ++i) sel[i] = pt[b * npg + sel[i] / ps] * ps + sel[i] % ps;
            check_row("paged", b, out + b * k, k, sel, m);
          }
          /* ragged: rows at arbitrary offsets of the same buffer, one negative length */
          int32_t starts[5], rl[5];
          for (int32_t b = 0; b < B; ++b) {
            starts[b] = (int32_t)(b * stride + (L > 0 ? (int32_t)(next32() % (uint32_t)(L + 1)) : 0));
            rl[b] = (int32_t)(stride * B - starts[b]);
            if (rl[b] > L) rl[b] = L;
          }
          rl[3] = -5;
          if (ets_oracle_topk_ragged(bits, starts, rl, B, k, out, k, threads[ti]) != 0) ++failures;
          for (int32_t b = 0; b < B; ++b) {
            const int32_t n = rl[b] < 0 ? 0 : rl[b];
            const int32_t m = brute(bits + starts[b], n, k, sel);
            for (int32_t i = 0; i < m; ++i) sel[i] += starts[b];
            check_row("ragged", b, out + b * k, k, sel, m);
          }
        }
        free(sel);
        free(out);
      }
      free(pt);
      free(bits);
    }
  }
  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("oracle under ASan/UBSan: all rows match the rank definition\n");
  return 0;
}
