/*
 * ets_topk.h -- C ABI of the exact per-row top-k selection library for
 * AMD MI355X (gfx950).
 *
 * What is computed (sglang PR #37591 digest, "Summary" and "Implementation
 * breakdown" item 1): for every row b of fp32 scores, the positions of the k
 * largest scores of the row's valid part, exactly.  Scores are ranked by the
 * order-preserving 32-bit key of their bit pattern (same page, the
 * order_key32 excerpt: negative values have every bit inverted, non-negative
 * values get the sign bit set, and unsigned comparison of keys then equals
 * float comparison).  Consequences of ranking by key:
 *   - +0.0 ranks above -0.0, subnormals are ordered by their bits (no flush
 *     to zero), +NaN ranks above +inf and -NaN below -inf;
 *   - "equal scores" means identical bit patterns; among equal scores the
 *     lowest positions are taken, so the selected set is unique.
 *
 * Output (sglang PR #36004 digest, test excerpt; PR #37591 digest, the
 * CoopParams / OutMap excerpt): each row of `out` receives m = min(k, n)
 * mapped positions followed by k - m entries of -1.  The m entries appear in
 * an unspecified order, which may change from run to run when a row is split
 * over several workgroups (the set never does); compare them as sets.
 * Every one of the k slots is written; prior contents of `out` do not matter.
 * Position maps:
 *   raw    : i                                          (row-local position)
 *   paged  : page_table[b][i / page_size] * page_size + i % page_size
 *   ragged : row_starts[b] + i                          (packed-buffer position)
 *
 * Conventions shared by every call:
 *   - All array pointers are device memory owned by the caller.  The library
 *     allocates nothing on the device and never synchronises the host; work
 *     is enqueued on `stream` (a hipStream_t; NULL = the default stream).
 *   - Arguments are validated on the host before anything is enqueued; a
 *     rejected call enqueues nothing.  Device-side preconditions are not
 *     checked: page ids must be >= 0 with page_id * page_size + page_size - 1
 *     < 2^31, and ragged rows must lie inside the packed buffer.
 *   - Only gfx950 devices are supported; others return ETS_ERR_DEVICE.
 *   - `workspace` is caller-owned device memory of at least the size that
 *     ets_workspace_size() reports for the same (B, max row length, k) on the
 *     current device (0 bytes is valid; then workspace may be NULL).  It is
 *     used when the batch is too small to fill the device and each row is
 *     split over several workgroups that exchange per-row histograms and
 *     counters through it (sglang PR #37591 digest, the topk.hip excerpt:
 *     the caller's allocator provides the row-split workspace).  It must be
 *     zero-filled before its first use (ets_workspace_init, or any zero fill)
 *     and every call returns it to zero (counters, tables and tie lists), so
 *     one workspace serves any number of calls, including replays of a
 *     captured graph.  It must not be
 *     shared by calls that may run concurrently.
 *   - A split row's workgroups wait for one another on the device, and every
 *     such wait is bounded.  The launch plan counts on the device's compute
 *     units: other work only delays the waits, but two split calls that run
 *     at the same time on one device (on different streams, or graphs
 *     replayed concurrently) can each hold compute units that the other's
 *     workgroups need, so such calls must be ordered (one stream, or events).
 *     A wait runs out when that is not done, when other work keeps the
 *     device's compute units for a very long time, or when the workspace was
 *     not zero (a stale ticket); the call has already returned ETS_OK by then,
 *     so the kernel records the failure in the workspace's error word (the
 *     32-bit word at byte offset 128) and that call's output is undefined.
 *     ets_workspace_error() copies and clears that word on the stream without
 *     synchronising; check it after the calls whose results matter.
 */
#ifndef ETS_TOPK_H
#define ETS_TOPK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t ets_status;

#define ETS_OK 0
#define ETS_ERR_INVALID_ARG 1 /* null pointer, negative size, bad stride or page size */
#define ETS_ERR_K_RANGE 2     /* k outside [1, ETS_MAX_K] */
#define ETS_ERR_WORKSPACE 3   /* workspace smaller than ets_workspace_size() */
#define ETS_ERR_DEVICE 4      /* current device is not gfx950 or cannot be queried */
#define ETS_ERR_HIP 5         /* a HIP launch or runtime call failed */
#define ETS_ERR_SCRATCH 6     /* ets_topk_paged_noalloc: the call needs more than its static scratch */

/* Largest supported k (the pages fix k at 1024 for the paged transform,
 * PR #36004 digest, kMaxTopK excerpt, and at 2048 for the DSA top-k,
 * PR #37591 digest, "Implementation breakdown" item 2). */
#define ETS_MAX_K 2048

/*
 * Dense rows, raw output.
 *   scores     fp32 [B, row_stride] (row b starts at scores + b * row_stride);
 *              only the first L entries of a row are ever read.
 *   row_stride elements between consecutive rows, >= L.
 *   B, L       batch size (>= 0) and row capacity (>= 0).
 *   lens       int32 [B] valid length of each row, clamped to [0, L];
 *              NULL means every row is L long.
 *   k          1 <= k <= ETS_MAX_K.
 *   out        int32 [B, out_stride], out_stride >= k; row-local positions.
 */
ets_status ets_topk_raw(const float* scores, int64_t row_stride, int32_t B, int32_t L,
                        const int32_t* lens, int32_t k, int32_t* out, int64_t out_stride,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Dense rows, paged output (PR #36004 digest: the fused top-k + page-table
 * transform, called with scores, seq_lens, page_table, the output and
 * page_size).
 *   seq_lens   int32 [B] valid length of each row (clamped to [0, L]); required.
 *   page_table int32 [B, pt_stride]; row b needs ceil(min(seq_lens[b], L) /
 *              page_size) entries.
 *   page_size  >= 1.
 *   out        int32 [B, out_stride]: page_table[b][i / page_size] *
 *              page_size + i % page_size for each selected position i.
 */
ets_status ets_topk_paged(const float* scores, int64_t row_stride, int32_t B, int32_t L,
                          const int32_t* seq_lens, const int32_t* page_table, int64_t pt_stride,
                          int32_t page_size, int32_t k, int32_t* out, int64_t out_stride,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Dense rows with a window per row, paged output: the decode caller's map
 * when only the last part of each sequence is a candidate (a sliding
 * window).  The pages' row-start offsets (PR #37591 digest, the CoopParams
 * excerpt; its tests cover "variable windows" on all three entry points)
 * address packed ragged rows; this call gives a dense row the same start.
 *   window_starts int32 [B]: row b selects among positions
 *              [w_b, n_b), n_b = seq_lens[b] clamped to [0, L] and w_b =
 *              window_starts[b] clamped to [0, n_b]; NULL = ets_topk_paged.
 *   Every other argument, the result, the padding and the workspace are as
 *   for ets_topk_paged; selected positions are row positions (i >= w_b), so
 *   out holds page_table[b][i / page_size] * page_size + i % page_size.
 *   A window start is not 16-byte aligned in general, so these rows are read
 *   with 4-byte loads.
 */
ets_status ets_topk_paged_window(const float* scores, int64_t row_stride, int32_t B, int32_t L,
                                 const int32_t* window_starts, const int32_t* seq_lens,
                                 const int32_t* page_table, int64_t pt_stride, int32_t page_size,
                                 int32_t k, int32_t* out, int64_t out_stride, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the paged
 * call above with the same arguments and results, but with no workspace
 * argument.  Calls whose rows split over row groups use a static device
 * array of ETS_NOALLOC_SCRATCH_BYTES (4 MiB, one per device, held until the
 * process ends) instead; nothing is allocated or freed, and no memset node is
 * recorded.  A call whose plan needs more workspace than that (a split call
 * with B above 50 on MI355X) returns ETS_ERR_SCRATCH before enqueueing
 * anything; calls that keep one workgroup per row need none and take any B.
 *   - The first call on a device zero-fills the array on `stream` with a
 *     kernel (inside a graph being captured, every replay does, until a call
 *     outside capture has done it once); every call returns the array's
 *     counters and tables to zero.
 *   - All calls on one device share the array: calls that may overlap (on
 *     different streams, or graphs replayed concurrently) race and their
 *     results are undefined.  Serialise them on one stream.
 *   - error_flag (nullable, device int32, caller-owned): when given, the call
 *     also copies the array's error word into error_flag[0] on `stream`
 *     (non-zero: a row group stopped waiting and this call's output is
 *     undefined; see ets_workspace_error) and, if it is set, zero-fills the
 *     array so that the next call starts clean.
 */
#define ETS_NOALLOC_SCRATCH_BYTES (4u << 20)
ets_status ets_topk_paged_noalloc(const float* scores, int64_t row_stride, int32_t B, int32_t L,
                                  const int32_t* seq_lens, const int32_t* page_table,
                                  int64_t pt_stride, int32_t page_size, int32_t k, int32_t* out,
                                  int64_t out_stride, int32_t* error_flag, void* stream);

/*
 * Packed ragged rows (PR #37591 digest, CoopParams excerpt: row_starts and
 * lengths address the rows of one packed buffer).
 *   packed       fp32 buffer holding every row.
 *   row_starts   int32 [B] offset of row b in `packed` (>= 0).
 *   lengths      int32 [B] length of row b (negative counts as 0).
 *   max_len_hint an upper bound of every lengths[b] (the host cannot read
 *                device lengths without a sync); it only steers the launch
 *                shape and the workspace size.  A row longer than the hint
 *                is still handled exactly, only more slowly.
 *   out          int32 [B, out_stride]: row_starts[b] + i per selected i.
 */
ets_status ets_topk_ragged(const float* packed, const int32_t* row_starts,
                           const int32_t* lengths, int32_t B, int64_t max_len_hint, int32_t k,
                           int32_t* out, int64_t out_stride, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * Workspace bytes needed by a call with this batch size, longest row and k on
 * `device` (-1 = the current device).  Writes 0 when the call needs none.
 * The size depends only on B once a workspace is needed at all.
 */
ets_status ets_workspace_size(int32_t B, int64_t max_row_len, int32_t k, int32_t device,
                              size_t* bytes);

/*
 * Zero-fills `bytes` bytes of `workspace` on `stream` (one small kernel), as
 * needed once before a workspace's first use.  workspace must be 16-byte
 * aligned; bytes = 0 is a no-op.
 */
ets_status ets_workspace_init(void* workspace, size_t bytes, void* stream);

/*
 * Enqueues on `stream` a copy of the workspace's error word into flag[0]
 * (device int32, caller-owned) and clears the word, so that the next calls
 * start clean.  Non-zero means a call before it on the stream stopped waiting
 * for the other workgroups of a row, and its output is undefined.  The word
 * is an OR of bits: 2 marks a stale ticket (a workspace that was not zero);
 * the others name the bounded wait that ran out: 1 the exchange of the row's
 * bounds, 4 the poll of the row's coarse histogram, 8 a barrier between
 * radix rounds, 16 the wait for the row's tie-list entries.
 * workspace_bytes = 0 (a call that needed no workspace) writes 0; otherwise
 * workspace must be 16-byte aligned and at least 256 bytes.  Nothing is
 * synchronised: read flag after the stream reaches it.
 */
ets_status ets_workspace_error(void* workspace, size_t workspace_bytes, int32_t* flag, void* stream);

/*
 * The device's compute units, XCDs and the row-group workgroups one compute
 * unit holds (from the HIP occupancy query of the row-group kernels; device =
 * -1: the current device): the inputs of ets_row_split, ets_group_cap and
 * ets_ticket_cap.  A row's members are the workgroups of one XCD when the
 * whole grid fits the device at once, so G is at most one XCD's slots
 * (ets_group_cap).  Larger grids take rows in the order workgroups start when
 * G is at most ets_ticket_cap; a group of G workgroups waits only for its own
 * members, and each XCD hands its workgroups to its shader engines in turn,
 * waiting for the engine whose turn it is, so the waiting members must not
 * fill one engine.  With larger G such a batch runs as several grids on the
 * stream, each over as many rows as fit the device at once.
 */
ets_status ets_device_limits(int32_t device, int32_t* cu_count, int32_t* xcd_count,
                             int32_t* groups_per_cu);

/* The largest row group on a device of these sizes (pure host function; 0 if
 * any input is <= 0): one XCD's row-group slots, min(64, (cu_count /
 * xcd_count) * groups_per_cu), 32 on MI355X. */
int32_t ets_group_cap(int32_t cu_count, int32_t xcd_count, int32_t groups_per_cu);

/* The largest row group a grid that does not fit the device at once takes in
 * one launch (pure host function; 0 if any input is <= 0): one shader
 * engine's row-group slots, min(64, max(1, (cu_count / xcd_count / 4) *
 * groups_per_cu)), 4 shader engines per XCD on gfx950 (8 on MI355X). */
int32_t ets_ticket_cap(int32_t cu_count, int32_t xcd_count, int32_t groups_per_cu);

/*
 * Workgroups per row the library uses for (B, max_row_len) on a device of
 * `cu_count` compute units in `xcd_count` XCDs, each compute unit holding
 * `groups_per_cu` row-group workgroups (ets_device_limits); 0 means one
 * workgroup per row.  Pure host function.
 * Rows that fit one workgroup's 32768-score tile stay whole; longer rows are
 * always split, into chunks of about 16384 scores (g16 = ceil(max_row_len /
 * 16384) members) where one index grid over the batch, xcd_count * G *
 * ceil(B / xcd_count) workgroups, fits the device's slots (cu_count *
 * groups_per_cu) at once; otherwise into the largest G below g16 whose index
 * grid still fits, if its chunks fit one tile; otherwise into the fewest
 * members whose chunks fit one tile (ceil(max_row_len / 32768)).  G is at
 * most ets_group_cap (cu_count, xcd_count or groups_per_cu <= 0: g16, at
 * most 64, the workspace's member slots).
 * The environment variable ETS_ROW_SPLIT, when set to an integer >= 0,
 * overrides the heuristic (0 or 1: one workgroup per row; n: n workgroups per
 * row).  An override above ets_group_cap returns -1, and the selection calls,
 * ets_workspace_size and the floors then return ETS_ERR_INVALID_ARG.  After
 * the pages' row_split heuristic (PR #37591 digest, the topk.hip excerpt),
 * with constants of this library measured on MI355X.
 *
 * A split row of n scores gives each member a chunk of ceil(n / G) scores,
 * rounded up to a multiple of 4, but at least 4096 (enough for a member to
 * bound the row's k-th largest), so a row shorter than G * 4096 leaves its
 * last members empty.  The environment variable ETS_MIN_CHUNK, when set to an
 * integer >= 1, replaces that 4096 (rounded up to a multiple of 4, at most
 * 32768; read at every call).  It changes the work division only, never the
 * result.
 */
int32_t ets_row_split(int32_t B, int64_t max_row_len, int32_t cu_count, int32_t xcd_count,
                      int32_t groups_per_cu);

/*
 * Measurement floors.  Neither selects anything: they give the cost of the
 * parts of a selection call that no selection method avoids, so that a
 * selection's time can be read against them.
 *
 * ets_floor_read: reads the same scores with the same grid, workgroup size,
 * lane layout and loads as a selection call on (B, rows) would, forms the
 * keys, and writes to sink[w] the largest key of the span that workgroup w
 * read (chunk g of row b for w = b * G + g, G = max(1, ets_row_split(...))).
 *   Dense rows (row_starts == NULL): scores, row_stride, B, L and lens
 *   (nullable) as for ets_topk_raw; max_len_hint is ignored.
 *   Ragged rows (row_starts != NULL): scores is the packed buffer, lens the
 *   required lengths and max_len_hint as for ets_topk_ragged; row_stride and
 *   L are ignored.
 *   sink  uint32 [sink_words], sink_words >= B * G.
 *
 * ets_floor_launch: one launch of the grid and workgroup size a selection
 * call on (B, max_row_len) uses, with empty workgroups.
 */
ets_status ets_floor_read(const float* scores, int64_t row_stride, int32_t B, int32_t L,
                          const int32_t* lens, const int32_t* row_starts, int64_t max_len_hint,
                          uint32_t* sink, int64_t sink_words, void* stream);
ets_status ets_floor_launch(int32_t B, int64_t max_row_len, void* stream);

/* Static, human-readable text for a status code. */
const char* ets_status_string(ets_status status);

#ifdef __cplusplus
}
#endif

#endif /* ETS_TOPK_H */
