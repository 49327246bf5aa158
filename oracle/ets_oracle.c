/*
 * ets_oracle.c -- plain CPU oracle for exact per-row top-k selection.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no code, header, table or
 * helper with the HIP library.
 *
 * What it computes (sglang PR #37591 digest, "Summary" and "Implementation
 * breakdown" item 1: the native ROCm DSA-indexer top-k is exact, i.e. it
 * returns the true top-k of every row, also when most scores share one coarse
 * bucket).  Because the fast method reaches exactly the result of the plain
 * definition, this oracle is that definition written out with no blocking and
 * no shortcut:
 *
 *   1. every fp32 score is mapped to an order-preserving unsigned 32-bit key
 *      (same page, "Key source excerpts", the order_key32 excerpt: a negative
 *      value has all bits inverted, a non-negative value gets its sign bit
 *      set, so unsigned comparison of keys equals float comparison);
 *   2. the valid positions of a row are sorted by (key descending, position
 *      ascending) -- a total order, so the permutation is unique; ties among
 *      equal keys go to the lowest position (the reading taken where the
 *      pages are silent);
 *   3. the first m = min(k, n) positions are the selection;
 *   4. each selected position i is mapped to the output value:
 *        raw    : i
 *        paged  : page_table[b][i / page_size] * page_size + i % page_size
 *                 (sglang PR #36004 digest, "Implementation breakdown" item 4
 *                 and the test excerpt: with an identity page table the
 *                 emitted paged slot equals the token position)
 *        ragged : row_starts[b] + i, the position in the packed buffer
 *                 (PR #37591 digest, the CoopParams excerpt: row_starts and
 *                 lengths address packed rows, and OutMap has a ragged case);
 *   5. the first m output slots receive the mapped selection in sorted order,
 *      and the remaining k - m slots receive -1 (PR #36004 test excerpt: the
 *      output buffer is pre-filled with -1).
 *
 * Row lengths: dense rows use n = clamp(lens[b], 0, L) (lens == NULL means
 * every row is L long); ragged rows use n = max(lengths[b], 0).
 *
 * Rows are independent; a small pthread pool hands out one row per task.  The
 * thread count changes only the wall time, never the result.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ETS_ORACLE_RAW 0
#define ETS_ORACLE_PAGED 1
#define ETS_ORACLE_RAGGED 2

/* Order-preserving key of one fp32 bit pattern (PR #37591, order_key32). */
uint32_t ets_oracle_order_key(uint32_t bits) {
  if (bits & 0x80000000u) return ~bits;
  return bits | 0x80000000u;
}

typedef struct {
  uint32_t key;
  int32_t pos;
} oracle_item;

/* (key descending, position ascending). */
static int oracle_item_cmp(const void* a, const void* b) {
  const oracle_item* x = (const oracle_item*)a;
  const oracle_item* y = (const oracle_item*)b;
  if (x->key != y->key) return (x->key > y->key) ? -1 : 1;
  if (x->pos != y->pos) return (x->pos < y->pos) ? -1 : 1;
  return 0;
}

typedef struct {
  int mode;
  const uint32_t* bits;     /* dense: scores [B, row_stride]; ragged: packed */
  int64_t row_stride;       /* dense only */
  int32_t B;
  int32_t L;                /* dense only */
  const int32_t* lens;      /* dense: per-row valid length, NULL = all L */
  const int32_t* row_starts; /* ragged */
  const int32_t* lengths;   /* ragged */
  const int32_t* page_table; /* paged: [B, pt_stride] */
  int64_t pt_stride;
  int32_t page_size;
  int32_t k;
  int32_t* out;             /* [B, out_stride] */
  int64_t out_stride;
  int64_t next_row;         /* shared work counter */
  int failed;               /* set when a row buffer cannot be allocated */
} oracle_job;

static int oracle_one_row(oracle_job* job, int32_t b) {
  const uint32_t* row;
  int32_t n;
  if (job->mode == ETS_ORACLE_RAGGED) {
    n = job->lengths[b] > 0 ? job->lengths[b] : 0;
    row = job->bits + (int64_t)job->row_starts[b];
  } else {
    n = job->lens ? job->lens[b] : job->L;
    if (n < 0) n = 0;
    if (n > job->L) n = job->L;
    row = job->bits + (int64_t)b * job->row_stride;
  }
  int32_t* out_row = job->out + (int64_t)b * job->out_stride;

  oracle_item* items = NULL;
  if (n > 0) {
    items = (oracle_item*)malloc((size_t)n * sizeof(oracle_item));
    if (!items) return -1;
  }
  for (int32_t i = 0; i < n; ++i) {
    items[i].key = ets_oracle_order_key(row[i]);
    items[i].pos = i;
  }
  if (n > 1) qsort(items, (size_t)n, sizeof(oracle_item), oracle_item_cmp);

  const int32_t m = n < job->k ? n : job->k;
  for (int32_t j = 0; j < m; ++j) {
    const int32_t i = items[j].pos;
    int32_t v = i;
    if (job->mode == ETS_ORACLE_PAGED) {
      const int32_t page = i / job->page_size;
      const int32_t slot = i % job->page_size;
      v = job->page_table[(int64_t)b * job->pt_stride + page] * job->page_size + slot;
    } else if (job->mode == ETS_ORACLE_RAGGED) {
      v = job->row_starts[b] + i;
    }
    out_row[j] = v;
  }
  for (int32_t j = m; j < job->k; ++j) out_row[j] = -1;
  free(items);
  return 0;
}

static void* oracle_worker(void* arg) {
  oracle_job* job = (oracle_job*)arg;
  for (;;) {
    const int64_t b = __atomic_fetch_add(&job->next_row, 1, __ATOMIC_RELAXED);
    if (b >= job->B) break;
    if (oracle_one_row(job, (int32_t)b) != 0) {
      __atomic_store_n(&job->failed, 1, __ATOMIC_RELAXED);
    }
  }
  return NULL;
}

static int oracle_run(oracle_job* job, int nthreads) {
  if (job->B < 0 || job->k < 1) return 1;
  if (job->mode == ETS_ORACLE_PAGED && job->page_size < 1) return 1;
  job->next_row = 0;
  job->failed = 0;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > job->B) nthreads = job->B > 0 ? job->B : 1;
  if (nthreads == 1) {
    oracle_worker(job);
  } else {
    pthread_t* tids = (pthread_t*)malloc((size_t)nthreads * sizeof(pthread_t));
    if (!tids) return 2;
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
      if (pthread_create(&tids[t], NULL, oracle_worker, job) != 0) break;
      ++started;
    }
    if (started == 0) oracle_worker(job); /* no thread could start */
    for (int t = 0; t < started; ++t) pthread_join(tids[t], NULL);
    free(tids);
  }
  return job->failed ? 2 : 0;
}

/* Dense rows, raw output (position within the row). */
int ets_oracle_topk_raw(const uint32_t* bits, int64_t row_stride, int32_t B, int32_t L,
                        const int32_t* lens, int32_t k, int32_t* out, int64_t out_stride,
                        int nthreads) {
  oracle_job job;
  memset(&job, 0, sizeof(job));
  job.mode = ETS_ORACLE_RAW;
  job.bits = bits;
  job.row_stride = row_stride;
  job.B = B;
  job.L = L;
  job.lens = lens;
  job.k = k;
  job.out = out;
  job.out_stride = out_stride;
  return oracle_run(&job, nthreads);
}

/* Dense rows, paged output (slot through the row's page table). */
int ets_oracle_topk_paged(const uint32_t* bits, int64_t row_stride, int32_t B, int32_t L,
                          const int32_t* seq_lens, const int32_t* page_table, int64_t pt_stride,
                          int32_t page_size, int32_t k, int32_t* out, int64_t out_stride,
                          int nthreads) {
  oracle_job job;
  memset(&job, 0, sizeof(job));
  job.mode = ETS_ORACLE_PAGED;
  job.bits = bits;
  job.row_stride = row_stride;
  job.B = B;
  job.L = L;
  job.lens = seq_lens;
  job.page_table = page_table;
  job.pt_stride = pt_stride;
  job.page_size = page_size;
  job.k = k;
  job.out = out;
  job.out_stride = out_stride;
  return oracle_run(&job, nthreads);
}

/* Packed ragged rows, output = position in the packed buffer. */
int ets_oracle_topk_ragged(const uint32_t* packed_bits, const int32_t* row_starts,
                           const int32_t* lengths, int32_t B, int32_t k, int32_t* out,
                           int64_t out_stride, int nthreads) {
  oracle_job job;
  memset(&job, 0, sizeof(job));
  job.mode = ETS_ORACLE_RAGGED;
  job.bits = packed_bits;
  job.B = B;
  job.row_starts = row_starts;
  job.lengths = lengths;
  job.k = k;
  job.out = out;
  job.out_stride = out_stride;
  return oracle_run(&job, nthreads);
}
