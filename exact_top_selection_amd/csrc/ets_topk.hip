// ets_topk.hip -- exact per-row top-k selection for gfx950 (CDNA4, wave64).
//
// Method (sglang PR #37591 digest, "Implementation breakdown" item 1): an
// order-preserving 32-bit key, a coarse histogram pass, a threshold-bucket
// search, a scatter pass that emits the winners and stages the threshold
// bucket's members, and an exact resolution of that bucket on the full key.
// This file re-designs each step for one CDNA4 workgroup per row:
//
//  * the row stays in VGPRs (1024 lanes x 32 keys = 32768 scores) after one
//    coalesced HBM pass, so every later pass is register-only;
//  * before the histogram, each lane's largest (or second largest) key is
//    reduced to a provable lower bound of the k-th largest score: the lanes'
//    maxima are k distinct scores, so at least k scores are >= their minimum.
//    Scores below the bound never touch the LDS histogram;
//  * the histogram range adapts to [bound, row max], so one 4096-bin round
//    usually leaves a threshold bucket of a few scores;
//  * ties are resolved on the 64-bit composite (key, ~position), which is
//    unique per score and orders equal keys by lowest position; a bucket
//    that is still large (concentrated scores) is split by further register
//    rounds on the same composite, so no tie buffer can overflow;
//  * a bucket of at most 256 entries is gathered into LDS and ranked by
//    direct comparison; the winners above it are written through one block
//    scan, so the output order is deterministic.
//
// Only integer arithmetic touches the scores.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "ets_topk.h"

namespace ets {

constexpr int kHistBits = 12;
constexpr int kHistBins = 1 << kHistBits;
constexpr int kSmallCap = 128;  // largest bucket ranked by direct comparison
constexpr int kPtCap = 2048;    // page-table entries staged in LDS
constexpr uint32_t kPeelShare = 16;  // lanes of a wave in one bin that switch to merged atomics

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum MapMode : int { kRaw = 0, kPaged = 1, kRagged = 2 };

struct Params {
  const float* scores;
  int64_t row_stride;          // dense rows
  const int32_t* lens;         // dense valid lengths (nullable) or ragged lengths
  const int32_t* row_starts;   // ragged
  const int32_t* page_table;   // paged
  int64_t pt_stride;
  int32_t page_size;
  int32_t page_shift;          // log2(page_size) if a power of two, else -1
  int32_t L;                   // dense row capacity
  int32_t k;
  int32_t* out;
  int64_t out_stride;
};

// Order-preserving key: negative -> all bits inverted, else sign bit set
// (PR #37591 digest, order_key32 excerpt), written branch-free.
__device__ __forceinline__ uint32_t order_key(uint32_t bits) {
  return bits ^ (static_cast<uint32_t>(static_cast<int32_t>(bits) >> 31) | 0x80000000u);
}

// ---------------------------------------------------------------- wave / block primitives
//
// Wave64 scans and reductions use DPP row shifts / permutes inside each
// 16-lane row and v_readlane across rows: no LDS round trip.

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_zero(uint32_t x) {  // out-of-row lanes read 0
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_perm(uint32_t x) {  // full-row permutes
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(static_cast<int>(x), static_cast<int>(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t readlane(uint32_t x, int l) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), l));
}
__device__ __forceinline__ uint32_t readfirstlane(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(x)));
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += dpp_zero<0x111>(x);  // row_shr:1
  x += dpp_zero<0x112>(x);  // row_shr:2
  x += dpp_zero<0x114>(x);  // row_shr:4
  x += dpp_zero<0x118>(x);  // row_shr:8
  const uint32_t r0 = readlane(x, 15), r1 = readlane(x, 31), r2 = readlane(x, 47);
  const int row = __lane_id() >> 4;
  return x + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

struct OpMax { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return max(a, b); } };
struct OpMin { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return min(a, b); } };
struct OpAdd { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; } };

template <class Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t x, Op op) {
  x = op(x, dpp_perm<0xB1>(x));   // quad_perm [1,0,3,2]
  x = op(x, dpp_perm<0x4E>(x));   // quad_perm [2,3,0,1]
  x = op(x, dpp_perm<0x141>(x));  // row_half_mirror
  x = op(x, dpp_perm<0x140>(x));  // row_mirror
  return op(op(readlane(x, 0), readlane(x, 16)), op(readlane(x, 32), readlane(x, 48)));
}

// Sum of the per-wave totals wsum[w] over the waves below (BELOW) or above
// the calling wave: one LDS read per lane and a wave reduction, uniform.
template <int W, bool BELOW>
__device__ __forceinline__ uint32_t sum_other_waves(const uint32_t* wsum) {
  static_assert(W <= 64, "one lane per wave");
  const int lane = static_cast<int>(__lane_id());
  const int wid = static_cast<int>(threadIdx.x >> 6);
  const uint32_t v = wsum[min(lane, W - 1)];
  const bool take = lane < W && (BELOW ? lane < wid : lane > wid);
  return wave_reduce(take ? v : 0u, OpAdd());
}

// Adds one to hist[bin] for every lane with `pred` (call in uniform control
// flow).  Lanes that share lane 0's bin are merged into one LDS atomic issued
// by lane 0, which removes the serialisation when most of a wave lands in one
// bin (concentrated scores); the other lanes add individually.
__device__ __forceinline__ void hist_add_peel(uint32_t* hist, bool pred, uint32_t bin) {
  const uint32_t lead = readfirstlane(bin);
  const bool same = pred && bin == lead;
  const uint64_t m = __ballot(same);
  if (__lane_id() == 0 && m != 0) atomicAdd(&hist[lead], static_cast<uint32_t>(__popcll(m)));
  if (pred && !same) atomicAdd(&hist[bin], 1u);
}

// Finds the histogram bin t with above(t) < kk <= above(t) + hist[t], where
// above(t) counts the entries of all higher bins; bin 0 is read as
// hist[0] - bin0_less.  Two barriers.  Every thread gets (t, above(t),
// hist[t]) in res[0..2].  wsum[] and res[] may be reused after one more
// barrier.
template <int T>
__device__ __forceinline__ void find_threshold_bin(const uint32_t* hist, uint32_t kk,
                                                   uint32_t bin0_less, uint32_t* wsum,
                                                   uint32_t* res) {
  constexpr int BPT = kHistBins / T;  // bins owned by each thread
  constexpr int W = T / 64;
  static_assert(BPT * T == kHistBins && BPT % 4 == 0, "block size must divide the bins by 4");
  const int wid = threadIdx.x >> 6;
  uint32_t h[BPT];
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < BPT; i += 4) {
    const uint4 q = reinterpret_cast<const uint4*>(hist)[threadIdx.x * (BPT / 4) + i / 4];
    h[i] = q.x;
    h[i + 1] = q.y;
    h[i + 2] = q.z;
    h[i + 3] = q.w;
  }
  if (threadIdx.x == 0) h[0] -= bin0_less;
#pragma unroll
  for (int i = 0; i < BPT; ++i) s += h[i];
  const uint32_t incl = wave_incl_scan(s);
  if (__lane_id() == 63) wsum[wid] = incl;
  __syncthreads();
  // higher lanes of this wave, then the waves above
  uint32_t above = readlane(incl, 63) - incl + sum_other_waves<W, false>(wsum);
#pragma unroll
  for (int i = BPT - 1; i >= 0; --i) {
    if (above < kk && kk <= above + h[i]) {
      res[0] = threadIdx.x * BPT + i;
      res[1] = above;
      res[2] = h[i];
    }
    above += h[i];
  }
  __syncthreads();
}

// ---------------------------------------------------------------- row spans

// key[j] for a lane-varying j, as a binary tree of selects (no scratch).
template <int PT>
__device__ __forceinline__ uint32_t select_slot(const uint32_t (&key)[PT], int j) {
  uint32_t v[PT];
#pragma unroll
  for (int i = 0; i < PT; ++i) v[i] = key[i];
#pragma unroll
  for (int w = PT / 2, bit = 0; w >= 1; w /= 2, ++bit) {
    const bool hi = (j >> bit) & 1;
#pragma unroll
    for (int i = 0; i < w; ++i) v[i] = hi ? v[2 * i + 1] : v[2 * i];
  }
  return v[0];
}

// Element layout of one tile held by a thread.  V4: float4 v of thread t holds
// positions base + 4 (v T + t) + c; scalar: slot j of thread t is at
// base + j T + t.  In both layouts a thread's positions increase with j.
template <int T, bool V4>
__device__ __forceinline__ int32_t tile_pos(int j) {
  if constexpr (V4) {
    return 4 * ((j >> 2) * T + static_cast<int>(threadIdx.x)) + (j & 3);
  } else {
    return j * T + static_cast<int>(threadIdx.x);
  }
}

// A contiguous span [start, end) of one row, held tile by tile in the
// caller's key registers.  Slots at positions >= end hold key 0; the passes
// correct for them arithmetically (they all fall into bin 0 while a key range
// starts at 0).
template <int T, int VEC, bool V4>
struct Span {
  static constexpr int PT = 4 * VEC;
  static constexpr int TILE = T * PT;
  using Keys = uint32_t[PT];
  const float* row;  // position 0 of the row (V4: 16-byte aligned, start % 4 == 0)
  int32_t start, end;

  // key-0 slots visited by one pass over the span (all in its last tile)
  __device__ uint32_t pad_slots() const {
    const int32_t len = end - start;
    const int32_t last = len - ((len - 1) / TILE) * TILE;
    return static_cast<uint32_t>(TILE - last);
  }
  // Loads the tile at base.  Every lane issues all of its loads before any
  // key is formed, so the loads overlap; lanes past the end re-read the last
  // in-range word (V4: float4), which keeps each access inside the row (V4
  // rows have a capacity that is a multiple of 4).  Slot groups that lie
  // wholly inside, straddle or lie past the end are told apart per group, the
  // same for all lanes.
  __device__ __forceinline__ void load(Keys& key, int32_t base) const {
    const int32_t tid = static_cast<int32_t>(threadIdx.x);
    if (base >= end) {
#pragma unroll
      for (int j = 0; j < PT; ++j) key[j] = 0u;
      return;
    }
    if constexpr (V4) {
      const int32_t qlast = (end - 1) & ~3;
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        const int32_t q = min(base + 4 * (v * T + tid), qlast);
        const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + q));
        key[4 * v + 0] = w.x;
        key[4 * v + 1] = w.y;
        key[4 * v + 2] = w.z;
        key[4 * v + 3] = w.w;
      }
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        const int32_t g0 = base + 4 * v * T;  // first position of the group
        const int32_t q = g0 + 4 * tid;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          uint32_t& x = key[4 * v + c];
          if (g0 + 4 * T <= end) {
            x = order_key(x);
          } else if (g0 >= end) {
            x = 0u;
          } else {
            x = q + c < end ? order_key(x) : 0u;
          }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < PT; ++j) {
        const int32_t q = min(base + j * T + tid, end - 1);
        key[j] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(row) + q);
      }
#pragma unroll
      for (int j = 0; j < PT; ++j) {
        const int32_t g0 = base + j * T;
        if (g0 + T <= end) {
          key[j] = order_key(key[j]);
        } else if (g0 >= end) {
          key[j] = 0u;
        } else {
          key[j] = g0 + tid < end ? order_key(key[j]) : 0u;
        }
      }
    }
  }
  // f(key, position, slot) over every slot.  RESIDENT: the span is one tile,
  // already in key; otherwise every call streams the span again.
  template <bool RESIDENT, class F>
  __device__ __forceinline__ void for_each(Keys& key, F&& f) const {
    if constexpr (!RESIDENT) {
      for (int32_t base = start; base < end; base += TILE) {
        load(key, base);
#pragma unroll
        for (int j = 0; j < PT; ++j) f(key[j], base + tile_pos<T, V4>(j), j);
      }
    } else {
#pragma unroll
      for (int j = 0; j < PT; ++j) f(key[j], start + tile_pos<T, V4>(j), j);
    }
  }
};

// ---------------------------------------------------------------- threshold refinement

// State of the selection: the threshold bucket and what is still needed.
struct Sel {
  uint32_t lo, hi;    // key range of the bucket
  uint32_t kk;        // entries still to take from the bucket
  uint32_t bucket;    // entries in the bucket (0xFFFFFFFF = not counted yet)
  uint32_t tie;       // 1: the bucket is one key, narrowed by position
  uint32_t dlo, dhi;  // tie: range of d = n - 1 - pos in the bucket
};

struct alignas(16) SelSmem {
  // double-buffered histogram; the 64 words after each buffer are per-lane
  // dummy bins that out-of-range lanes add into
  uint32_t hist[2][kHistBins + 64];
  uint32_t wsum[16];
  uint32_t res[4];
};

template <int T>
__device__ __forceinline__ void hist_clear(uint32_t* hist) {
#pragma unroll
  for (int i = threadIdx.x; i < kHistBins / 4; i += T) {
    reinterpret_cast<uint4*>(hist)[i] = make_uint4(0, 0, 0, 0);
  }
}

// Radix rounds until the bucket holds at most kSmallCap entries: 12-bit
// rounds on the key inside [lo, hi], then (one key left with too many ties)
// rounds on d = n - 1 - pos among the scores equal to it, so that the
// lowest positions win.  Padding slots have pos >= n: their d wraps far
// above any range.  Round r counts into hist[r & 1] and clears the other
// buffer.  Precondition: hist[round & 1] is zero and a barrier has passed.
// Each wave probes (with probe_key) whether its lanes pile into one bin and
// only then merges its LDS atomics.  Returns the refined state.
template <int T, class ForEach>
__device__ __forceinline__ Sel refine(ForEach&& for_each, SelSmem& sm, const Sel in, uint32_t nm1,
                                      uint32_t n_pad, uint32_t probe_key, int& round) {
  uint32_t lo = in.lo, hi = in.hi, kk = in.kk, bucket = in.bucket;
  uint32_t tie = 0, dlo = 0, dhi = nm1;
  while (bucket > static_cast<uint32_t>(kSmallCap) && lo != hi) {
    uint32_t* hist = sm.hist[round & 1];
    hist_clear<T>(sm.hist[(round + 1) & 1]);
    const uint32_t rlo = lo, span = hi - lo;
    const int bl = span ? 32 - __clz(static_cast<int>(span)) : 0;
    const int s = bl > kHistBits ? bl - kHistBits : 0;
    bool peel;
    {
      const uint32_t d = probe_key - rlo;
      const uint32_t bin = d >> s;
      const uint32_t lead = readfirstlane(bin);
      peel = __popcll(__ballot(d <= span && bin == lead)) > kPeelShare;
    }
    if (peel) {
      for_each([&](uint32_t x, int32_t, int) {
        const uint32_t d = x - rlo;
        hist_add_peel(hist, d <= span, d >> s);
      });
    } else {
      const uint32_t dummy = kHistBins + __lane_id();
      for_each([&](uint32_t x, int32_t, int) {
        const uint32_t d = x - rlo;
        atomicAdd(&hist[d <= span ? d >> s : dummy], 1u);
      });
    }
    __syncthreads();
    find_threshold_bin<T>(hist, kk, rlo == 0 ? n_pad : 0u, sm.wsum, sm.res);
    kk -= sm.res[1];
    bucket = sm.res[2];
    lo = rlo + (sm.res[0] << s);
    const uint32_t width = (1u << s) - 1u;
    if (hi - lo > width) hi = lo + width;
    ++round;
  }
  if (bucket > static_cast<uint32_t>(kSmallCap)) {
    tie = 1;
    const uint32_t tkey = lo;
    while (bucket > static_cast<uint32_t>(kSmallCap)) {
      uint32_t* hist = sm.hist[round & 1];
      hist_clear<T>(sm.hist[(round + 1) & 1]);
      const uint32_t rdlo = dlo, span = dhi - dlo;
      const int bl = span ? 32 - __clz(static_cast<int>(span)) : 0;
      const int s = bl > kHistBits ? bl - kHistBits : 0;
      for_each([&](uint32_t x, int32_t pos, int) {
        const uint32_t d = nm1 - static_cast<uint32_t>(pos) - rdlo;
        if (x == tkey && d <= span) atomicAdd(&hist[d >> s], 1u);
      });
      __syncthreads();
      find_threshold_bin<T>(hist, kk, 0u, sm.wsum, sm.res);
      kk -= sm.res[1];
      bucket = sm.res[2];
      dlo = rdlo + (sm.res[0] << s);
      const uint32_t width = (1u << s) - 1u;
      if (dhi - dlo > width) dhi = dlo + width;
      ++round;
    }
  }
  Sel out;
  out.lo = lo;
  out.hi = hi;
  out.kk = kk;
  out.bucket = bucket;
  out.tie = tie;
  out.dlo = dlo;
  out.dhi = dhi;
  return out;
}

// Winner: key above the bucket, or (tie) the bucket's key at a lower
// position than the bucket.  Bucket member: the rest of the bucket.  Slots
// at positions >= end are padding (key 0): they can only match when the
// bucket reaches key 0, so those cases check the position.
__device__ __forceinline__ bool sel_winner(const Sel& s, uint32_t nm1, int32_t end, uint32_t x,
                                           int32_t pos) {
  if (!s.tie) return x > s.hi;
  const uint32_t d = nm1 - static_cast<uint32_t>(pos);
  return x > s.hi || (x == s.hi && d > s.dhi && pos < end);
}
__device__ __forceinline__ bool sel_bucket(const Sel& s, uint32_t nm1, int32_t end, uint32_t x,
                                           int32_t pos) {
  if (!s.tie) return x - s.lo <= s.hi - s.lo && (s.lo != 0 || pos < end);
  return x == s.hi && nm1 - static_cast<uint32_t>(pos) - s.dlo <= s.dhi - s.dlo &&
         (s.hi != 0 || pos < end);
}

// Address-space qualified views: a read through them compiles to an LDS or a
// global load, never to a flat one.
using lds_i32 = __attribute__((address_space(3))) const int32_t;
using glb_i32 = __attribute__((address_space(1))) const int32_t;

// Output value of selected position pos of a row.  Paged: pt_lds is the
// row's page-table staged in LDS, used when use_lds, else pt_row is read.
template <int MODE>
__device__ __forceinline__ int32_t out_value(const Params& p, bool use_lds, const int32_t* pt_lds,
                                             const int32_t* pt_row, int32_t row_start, int32_t pos) {
  if constexpr (MODE == kPaged) {
    int32_t page, off;
    if (p.page_shift >= 0) {
      page = pos >> p.page_shift;
      off = pos & (p.page_size - 1);
    } else {
      page = pos / p.page_size;
      off = pos - page * p.page_size;
    }
    const int32_t id = use_lds ? ((lds_i32*)pt_lds)[page] : ((glb_i32*)pt_row)[page];
    return id * p.page_size + off;
  } else if constexpr (MODE == kRagged) {
    return row_start + pos;
  } else {
    return pos;
  }
}

// Ranks up to kSmallCap bucket entries on (key desc, position asc) and emits
// the kk best at slots first + rank.  G = T / kSmallCap lanes share an entry:
// each compares it with every G-th entry, then row permutes sum the G counts.
// (key, ~position) as one 64-bit word orders the entries the same way.
template <int T, class Emit>
__device__ __forceinline__ void rank_bucket(const uint2* cand, uint32_t nc, uint32_t kk,
                                            uint32_t first, Emit&& emit) {
  constexpr int G = T / kSmallCap;
  static_assert(G == 2 || G == 4 || G == 8, "2, 4 or 8 lanes per bucket entry");
  constexpr int Q = kSmallCap / G;  // entries compared by each lane
  constexpr int QB = 16;            // entries read per batch
  const uint32_t i = threadIdx.x / G;
  const uint32_t part = threadIdx.x % G;
  const uint32_t last = nc > 0 ? nc - 1 : 0;
  const uint2 ci = cand[min(i, last)];
  const uint64_t vi = (static_cast<uint64_t>(ci.x) << 32) | static_cast<uint32_t>(~ci.y);
  uint32_t rank = 0;
#pragma unroll
  for (int q0 = 0; q0 < Q; q0 += QB) {
    if (static_cast<uint32_t>(G * q0) >= nc) break;
    uint2 cj[QB];
#pragma unroll
    for (int q = 0; q < QB; ++q) cj[q] = cand[min(part + G * (q0 + q), last)];
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const uint64_t vj = (static_cast<uint64_t>(cj[q].x) << 32) | static_cast<uint32_t>(~cj[q].y);
      rank += static_cast<uint32_t>((part + G * (q0 + q) < nc) & (vj > vi));
    }
  }
  rank += dpp_perm<0xB1>(rank);                         // quad_perm [1,0,3,2]: pairs
  if constexpr (G >= 4) rank += dpp_perm<0x4E>(rank);   // quad_perm [2,3,0,1]: quads
  if constexpr (G >= 8) rank += dpp_perm<0x141>(rank);  // row_half_mirror: eights
  if (i < nc && part == 0 && rank < kk) emit(first + rank, static_cast<int32_t>(ci.y));
}

// Row geometry shared by every kernel: valid length, base pointer, offsets.
template <int MODE>
struct RowRef {
  int32_t n;
  int32_t row_start;
  const float* row;
  const int32_t* pt_row;
  int32_t* out;
  __device__ RowRef(const Params& p, int b) {
    row_start = 0;
    if constexpr (MODE == kRagged) {
      row_start = p.row_starts[b];
      n = max(p.lens[b], 0);
      row = p.scores + row_start;
    } else {
      n = p.lens ? min(max(p.lens[b], 0), p.L) : p.L;
      row = p.scores + static_cast<int64_t>(b) * p.row_stride;
    }
    pt_row = (MODE == kPaged) ? p.page_table + static_cast<int64_t>(b) * p.pt_stride : nullptr;
    out = p.out + static_cast<int64_t>(b) * p.out_stride;
  }
};

// Rows no longer than k: every position is selected, the rest is padding.
template <int T, int MODE>
__device__ __forceinline__ void emit_whole_row(const Params& p, const RowRef<MODE>& r) {
  for (int32_t i = threadIdx.x; i < p.k; i += T) {
    r.out[i] = (i < r.n) ? out_value<MODE>(p, false, nullptr, r.pt_row, r.row_start, i) : -1;
  }
}

// ---------------------------------------------------------------- single-workgroup row kernel

struct alignas(16) RowSmem {
  SelSmem sel;
  int32_t pt[kPtCap];     // staged page-table row (paged map)
  uint2 cand[kSmallCap];  // threshold bucket: (key, position)
  int32_t pos[ETS_MAX_K]; // selected positions by output slot
  uint32_t red[64];       // per-wave partials (bounds)
  uint32_t ccount;
};

// One exact top-k row on one workgroup.  STREAM = false: the row (n <= one
// tile) is loaded once and every pass runs on registers.  STREAM = true: any
// length; every pass streams the row tile by tile (L2 after the first).
template <int T, int VEC, int MODE, bool V4, bool STREAM>
__device__ __forceinline__ void row_topk(const Params& p, RowSmem& sm, const RowRef<MODE>& r) {
  using SpanT = Span<T, VEC, V4>;
  constexpr int PT = SpanT::PT;
  constexpr int W = T / 64;
  const int tid = threadIdx.x;
  const int wid = tid >> 6;
  const int32_t k = p.k;
  const int32_t n = r.n;

  // Page-table row into LDS: issued before the score loads so its latency
  // hides behind them.
  constexpr int PTV = (MODE == kPaged) ? (kPtCap + T - 1) / T : 1;
  int32_t ptv[PTV];
  bool pt_lds = false;
  int32_t npages = 0;
  if constexpr (MODE == kPaged) {
    npages = p.page_shift >= 0 ? ((n - 1) >> p.page_shift) + 1 : (n - 1) / p.page_size + 1;
    pt_lds = npages <= kPtCap;
    if (pt_lds) {
#pragma unroll
      for (int i = 0; i < PTV; ++i) ptv[i] = (tid + i * T < npages) ? r.pt_row[tid + i * T] : 0;
    }
  }

  const SpanT span{r.row, 0, n};
  uint32_t key[PT];
  if constexpr (!STREAM) span.load(key, 0);
  auto for_each = [&](auto&& f) { span.template for_each<!STREAM>(key, f); };

  hist_clear<T>(sm.sel.hist[0]);
  if (tid == 0) sm.ccount = 0;
  if constexpr (MODE == kPaged) {
    if (pt_lds) {
#pragma unroll
      for (int i = 0; i < PTV; ++i)
        if (tid + i * T < npages) sm.pt[tid + i * T] = ptv[i];
    }
  }

  // ---- bounds: row max and a lower bound of the k-th largest key.  Each
  // thread's jth-largest key, over the nfull threads that hold at least jth
  // scores, gives nfull * jth distinct scores at or above their minimum;
  // jth = ceil(k / threads holding scores) <= 2.  Key-0 padding never raises
  // m1 or m2 of such a thread.  Otherwise the row minimum is the bound.
  const int32_t holders = V4 ? min(T, (n + 3) / 4) : min(T, n);
  const int32_t jth = (k + holders - 1) / holders;
  uint32_t m1 = 0, m2 = 0;
  if (jth == 1) {
    for_each([&](uint32_t x, int32_t, int) { m1 = max(m1, x); });
    m2 = m1;
  } else {
    for_each([&](uint32_t x, int32_t, int) {
      m2 = max(m2, min(m1, x));
      m1 = max(m1, x);
    });
  }
  // threads whose first jth slots hold scores (V4: positions 4t .. 4t+jth-1,
  // scalar: t and t + T)
  const int32_t jpos = V4 ? 4 * tid + jth - 1 : (jth - 1) * T + tid;
  const bool full = jth <= 2 && jpos < n;
  const int32_t nfull = jth > 2 ? 0 : (V4 ? min(T, max(0, (n - jth) / 4 + 1)) : min(T, max(0, n - (jth - 1) * T)));
  Sel sel0{};
  {
    const uint32_t rmax = wave_reduce(m1, OpMax());
    const uint32_t bmin = wave_reduce(full ? m2 : 0xFFFFFFFFu, OpMin());
    if (__lane_id() == 0) {
      sm.red[wid] = rmax;
      sm.red[16 + wid] = bmin;
    }
    __syncthreads();
    uint32_t gmax = 0, gb = 0xFFFFFFFFu;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      gmax = max(gmax, sm.red[w]);
      gb = min(gb, sm.red[16 + w]);
    }
    sel0.hi = gmax;
    if (nfull * jth >= k) {
      sel0.lo = gb;
    } else {
      uint32_t mn = 0xFFFFFFFFu;
      for_each([&](uint32_t x, int32_t pos, int) { mn = min(mn, pos < n ? x : 0xFFFFFFFFu); });
      mn = wave_reduce(mn, OpMin());
      if (__lane_id() == 0) sm.red[32 + wid] = mn;
      __syncthreads();
      sel0.lo = 0xFFFFFFFFu;
#pragma unroll
      for (int w = 0; w < W; ++w) sel0.lo = min(sel0.lo, sm.red[32 + w]);
    }
  }
  sel0.kk = static_cast<uint32_t>(k);
  sel0.bucket = 0xFFFFFFFFu;

  // ---- radix refinement until the bucket is small
  const uint32_t nm1 = static_cast<uint32_t>(n - 1);
  int round = 0;
  const Sel sel = refine<T>(for_each, sm.sel, sel0, nm1, span.pad_slots(), key[0], round);

  // ---- scatter: append the bucket to LDS, count the winners, place them by
  // one block scan (whose barrier also publishes the bucket) into the
  // position list.
  const uint32_t first = static_cast<uint32_t>(k) - sel.kk;  // number of winners
  // the page-table source is chosen once per row, so that each emitting loop
  // reads only LDS (or only global memory) and never waits on its stores
  auto emitter = [&](auto lds) {
    return [&](uint32_t slot, int32_t pos) {
      r.out[slot] = out_value<MODE>(p, decltype(lds)::value, sm.pt, r.pt_row, r.row_start, pos);
    };
  };
  auto with_emit = [&](auto&& body) {
    if (MODE != kPaged || pt_lds) {
      body(emitter(std::true_type()));
    } else {
      body(emitter(std::false_type()));
    }
  };
  auto append = [&](uint32_t x, int32_t pos) {
    const uint32_t slot = atomicAdd(&sm.ccount, 1u);
    if (slot < static_cast<uint32_t>(kSmallCap)) sm.cand[slot] = make_uint2(x, static_cast<uint32_t>(pos));
  };
  if constexpr (!STREAM) {
    // bit PT-1-j of wmask / cmask: slot j is a winner / in the bucket
    static_assert(PT <= 32, "slot masks are 32 bits");
    uint32_t wmask = 0, cmask = 0;
    if (!sel.tie) {
      const uint32_t khi = sel.hi, klo = sel.lo, kspan = sel.hi - sel.lo;
      if (klo != 0) {
        for_each([&](uint32_t x, int32_t, int) {
          wmask = wmask + wmask + (x > khi ? 1u : 0u);
          cmask = cmask + cmask + (x - klo <= kspan ? 1u : 0u);
        });
      } else {
        for_each([&](uint32_t x, int32_t pos, int) {
          wmask = wmask + wmask + (x > khi ? 1u : 0u);
          cmask = cmask + cmask + (x - klo <= kspan && pos < n ? 1u : 0u);
        });
      }
    } else {
      for_each([&](uint32_t x, int32_t pos, int) {
        wmask = wmask + wmask + (sel_winner(sel, nm1, span.end, x, pos) ? 1u : 0u);
        cmask = cmask + cmask + (sel_bucket(sel, nm1, n, x, pos) ? 1u : 0u);
      });
    }
    if (__ballot(cmask != 0) != 0) {
      while (cmask != 0) {
        const int j = PT - __ffs(static_cast<int>(cmask));
        cmask &= cmask - 1u;
        append(select_slot<PT>(key, j), tile_pos<T, V4>(j));
      }
    }
    const uint32_t nwin = static_cast<uint32_t>(__popc(wmask));
    const uint32_t incl = wave_incl_scan(nwin);
    if (__lane_id() == 63) sm.sel.wsum[wid] = incl;
    __syncthreads();
    uint32_t off = incl - nwin + sum_other_waves<W, true>(sm.sel.wsum);
    // the bound only guards the row against a broken invariant
    while (wmask != 0) {
      const int j = PT - __ffs(static_cast<int>(wmask));
      wmask &= wmask - 1u;
      if (off < first) sm.pos[off] = tile_pos<T, V4>(j);
      ++off;
    }
  } else {
    uint32_t nwin = 0;
    for_each([&](uint32_t x, int32_t pos, int) {
      nwin += sel_winner(sel, nm1, span.end, x, pos) ? 1u : 0u;
      const bool c = sel_bucket(sel, nm1, n, x, pos);
      if (__ballot(c) != 0 && c) append(x, pos);
    });
    const uint32_t incl = wave_incl_scan(nwin);
    if (__lane_id() == 63) sm.sel.wsum[wid] = incl;
    __syncthreads();
    uint32_t off = incl - nwin + sum_other_waves<W, true>(sm.sel.wsum);
    for_each([&](uint32_t x, int32_t pos, int) {
      if (sel_winner(sel, nm1, span.end, x, pos)) {
        if (off < first) sm.pos[off] = pos;
        ++off;
      }
    });
  }

  // ---- the bucket's best kk, placed by rank
  rank_bucket<T>(sm.cand, min(sm.ccount, static_cast<uint32_t>(kSmallCap)), sel.kk, first,
                 [&](uint32_t slot, int32_t pos) { sm.pos[slot] = pos; });
  __syncthreads();

  // ---- emit the k selected positions through the output map, coalesced
  with_emit([&](auto emit) {
    for (int32_t i = tid; i < k; i += T) emit(static_cast<uint32_t>(i), sm.pos[i]);
  });
}

// One workgroup per row.  STREAM = false: rows fit one tile (the host
// guarantees it for dense rows; a ragged row longer than its length hint
// falls back to the streamed passes).  STREAM = true: any row length.
template <int T, int VEC, int MODE, bool V4, bool STREAM>
__global__ __launch_bounds__(T) void row_topk_kernel(Params p) {
  constexpr int TILE = T * 4 * VEC;
  __shared__ RowSmem sm;
  const RowRef<MODE> r(p, blockIdx.x);
  if (r.n <= p.k) {
    emit_whole_row<T, MODE>(p, r);
    return;
  }
  if constexpr (STREAM) {
    row_topk<T, VEC, MODE, V4, true>(p, sm, r);
  } else {
    if constexpr (MODE == kRagged) {
      if (r.n > TILE) {
        row_topk<T, VEC, MODE, V4, true>(p, sm, r);
        return;
      }
    }
    row_topk<T, VEC, MODE, V4, false>(p, sm, r);
  }
}

// ---------------------------------------------------------------- row-split path
//
// Long rows are cut into G chunks of `chunk` scores, one workgroup each
// (after the pages' row-split path, PR #37591 topk.hip excerpt: histogram,
// scatter and refine kernels over a workspace, the kernel boundaries acting
// as the barriers between the chunks of a row).  Six launches:
//   split_zero     clears the per-row records and histograms;
//   split_bounds   per chunk: max, min of lane maxima, holders, min;
//   split_hist     per chunk: the row's range from all chunks' bounds, a LDS
//                  histogram of the chunk, merged into the row's histogram;
//   split_select   per row: the threshold bin; a bucket still above
//                  kSmallCap is refined by this workgroup streaming the row;
//   split_scatter  per chunk: winners to the output and the bucket to the
//                  workspace, placed through one 64-bit cursor per row;
//   split_finish   per row: rank the bucket, emit; rows with n <= k.
// Workspace (u32 words): rec[B][16] | part[B][G][4] | hist[B][4096] | cand[B][kSmallCap][2].

constexpr int kRec = 16;
enum RecField : int { kRecLo = 0, kRecHi, kRecKk, kRecTie, kRecDlo, kRecDhi, kRecShift, kRecPad,
                      kRecCursor = 8 /* u64: winners << 32 | bucket entries */ };

struct SplitWs {
  uint32_t* rec;
  uint32_t* part;
  uint32_t* hist;
  uint2* cand;
  __device__ SplitWs(uint32_t* ws, int32_t B, int32_t G) {
    rec = ws;
    part = rec + static_cast<int64_t>(B) * kRec;
    hist = part + static_cast<int64_t>(B) * G * 4;
    cand = reinterpret_cast<uint2*>(hist + static_cast<int64_t>(B) * kHistBins);
  }
};

__global__ __launch_bounds__(256) void split_zero(uint32_t* ws, int32_t B, int32_t G) {
  const SplitWs w(ws, B, G);
  const int64_t nrec = static_cast<int64_t>(B) * kRec;
  const int64_t nhist = static_cast<int64_t>(B) * kHistBins;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < nrec + nhist; i += 256ll * gridDim.x) {
    if (i < nrec) w.rec[i] = 0u;
    else w.hist[i - nrec] = 0u;
  }
}

// Chunk g of a row: [g chunk, (g+1) chunk), the last chunk running to the
// row's end (a ragged row may be longer than the length hint).
__device__ __forceinline__ int32_t chunk_end(int32_t g, int32_t G, int32_t chunk, int32_t n) {
  return g == G - 1 ? n : min(g * chunk + chunk, n);
}

// Runs body(std::true_type) when the span fits one tile (loaded once, kept
// in registers), else body(std::false_type) (streamed per pass).
template <class SpanT, class Body>
__device__ __forceinline__ void with_span(const SpanT& span, typename SpanT::Keys& key, Body&& body) {
  if (span.end - span.start <= SpanT::TILE) {
    span.load(key, span.start);
    body(std::true_type());
  } else {
    body(std::false_type());
  }
}

template <int T, int VEC, int MODE, bool V4>
__global__ __launch_bounds__(T) void split_bounds(Params p, uint32_t* ws, int32_t B, int32_t G,
                                                  int32_t chunk) {
  constexpr int W = T / 64;
  __shared__ uint32_t red[4 * 16];
  const int b = blockIdx.x / G, g = blockIdx.x % G;
  const RowRef<MODE> r(p, b);
  if (r.n <= p.k) return;
  const SplitWs w(ws, B, G);
  uint32_t* part = w.part + (static_cast<int64_t>(b) * G + g) * 4;
  const Span<T, VEC, V4> span{r.row, g * chunk, chunk_end(g, G, chunk, r.n)};
  uint32_t key[4 * VEC];
  if (span.start >= span.end) {
    if (threadIdx.x == 0) {
      part[0] = 0u;
      part[1] = 0xFFFFFFFFu;
      part[2] = 0u;
      part[3] = 0xFFFFFFFFu;
    }
    return;
  }
  uint32_t m1 = 0, mn = 0xFFFFFFFFu;
  with_span(span, key, [&](auto res) {
    span.template for_each<decltype(res)::value>(key, [&](uint32_t x, int32_t pos, int) {
      m1 = max(m1, x);
      mn = min(mn, pos < span.end ? x : 0xFFFFFFFFu);
    });
  });
  // a thread holds a score iff its first slot does
  const int32_t first_pos = span.start + (V4 ? 4 * static_cast<int32_t>(threadIdx.x) : static_cast<int32_t>(threadIdx.x));
  const bool holds = first_pos < span.end;
  const uint32_t vmax = wave_reduce(m1, OpMax());
  const uint32_t vmm = wave_reduce(holds ? m1 : 0xFFFFFFFFu, OpMin());
  const uint32_t vh = wave_reduce(holds ? 1u : 0u, OpAdd());
  const uint32_t vmin = wave_reduce(mn, OpMin());
  const int wid = threadIdx.x >> 6;
  if (__lane_id() == 0) {
    red[wid] = vmax;
    red[16 + wid] = vmm;
    red[32 + wid] = vh;
    red[48 + wid] = vmin;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0, bm = 0xFFFFFFFFu, c = 0, d = 0xFFFFFFFFu;
    for (int i = 0; i < W; ++i) {
      a = max(a, red[i]);
      bm = min(bm, red[16 + i]);
      c += red[32 + i];
      d = min(d, red[48 + i]);
    }
    part[0] = a;
    part[1] = bm;
    part[2] = c;
    part[3] = d;
  }
}

// The row's key range from all chunks: [lower bound, max].  The lanes'
// maxima over all chunks are `holders` distinct scores, so if they number at
// least k their minimum bounds the k-th largest from below; otherwise the
// row minimum does.
template <int T>
__device__ __forceinline__ void split_range(const uint32_t* part, int32_t G, int32_t k,
                                            uint32_t* red, uint32_t& lo, uint32_t& hi) {
  constexpr int W = T / 64;
  uint32_t a = 0, bm = 0xFFFFFFFFu, c = 0, d = 0xFFFFFFFFu;
  for (int g = threadIdx.x; g < G; g += T) {
    const uint4 q = reinterpret_cast<const uint4*>(part)[g];
    a = max(a, q.x);
    bm = min(bm, q.y);
    c += q.z;
    d = min(d, q.w);
  }
  a = wave_reduce(a, OpMax());
  bm = wave_reduce(bm, OpMin());
  c = wave_reduce(c, OpAdd());
  d = wave_reduce(d, OpMin());
  const int wid = threadIdx.x >> 6;
  if (__lane_id() == 0) {
    red[wid] = a;
    red[16 + wid] = bm;
    red[32 + wid] = c;
    red[48 + wid] = d;
  }
  __syncthreads();
  a = 0, bm = 0xFFFFFFFFu, c = 0, d = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    a = max(a, red[i]);
    bm = min(bm, red[16 + i]);
    c += red[32 + i];
    d = min(d, red[48 + i]);
  }
  hi = a;
  lo = c >= static_cast<uint32_t>(k) ? bm : d;
}

template <int T, int VEC, int MODE, bool V4>
__global__ __launch_bounds__(T) void split_hist(Params p, uint32_t* ws, int32_t B, int32_t G,
                                                int32_t chunk) {
  __shared__ __align__(16) uint32_t hist[kHistBins + 64];
  __shared__ uint32_t red[4 * 16];
  const int b = blockIdx.x / G, g = blockIdx.x % G;
  const RowRef<MODE> r(p, b);
  if (r.n <= p.k) return;
  const SplitWs w(ws, B, G);
  const Span<T, VEC, V4> span{r.row, g * chunk, chunk_end(g, G, chunk, r.n)};
  uint32_t key[4 * VEC];
  hist_clear<T>(hist);
  uint32_t lo, hi;
  split_range<T>(w.part + static_cast<int64_t>(b) * G * 4, G, p.k, red, lo, hi);
  const uint32_t span_k = hi - lo;
  const int bl = span_k ? 32 - __clz(static_cast<int>(span_k)) : 0;
  const int s = bl > kHistBits ? bl - kHistBits : 0;
  uint32_t* rec = w.rec + static_cast<int64_t>(b) * kRec;
  if (g == 0 && threadIdx.x == 0) {
    rec[kRecLo] = lo;
    rec[kRecHi] = hi;
    rec[kRecShift] = static_cast<uint32_t>(s);
  }
  if (span.start >= span.end) return;
  with_span(span, key, [&](auto res) {
    constexpr bool RES = decltype(res)::value;
    bool peel = false;
    if (RES) {
      const uint32_t d = key[0] - lo;
      const uint32_t bin = d >> s;
      const uint32_t lead = readfirstlane(bin);
      peel = __popcll(__ballot(d <= span_k && bin == lead)) > kPeelShare;
    }
    if (peel) {
      span.template for_each<RES>(key, [&](uint32_t x, int32_t, int) {
        const uint32_t d = x - lo;
        hist_add_peel(hist, d <= span_k, d >> s);
      });
    } else {
      const uint32_t dummy = kHistBins + __lane_id();
      span.template for_each<RES>(key, [&](uint32_t x, int32_t, int) {
        const uint32_t d = x - lo;
        atomicAdd(&hist[d <= span_k ? d >> s : dummy], 1u);
      });
    }
  });
  __syncthreads();
  if (lo == 0 && threadIdx.x == 0) hist[0] -= span.pad_slots();
  __syncthreads();
  uint32_t* ghist = w.hist + static_cast<int64_t>(b) * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += T) {
    const uint32_t c = hist[i];
    if (c) __hip_atomic_fetch_add(&ghist[i], c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

struct alignas(16) SelectSmem {
  SelSmem sel;
};

// Per row: threshold bin of the merged histogram; a bucket still above
// kSmallCap is refined by this workgroup streaming the whole row.
template <int T, int VEC, int MODE, bool V4>
__global__ __launch_bounds__(T) void split_select(Params p, uint32_t* ws, int32_t B, int32_t G) {
  __shared__ SelectSmem sm;
  const int b = blockIdx.x;
  const RowRef<MODE> r(p, b);
  if (r.n <= p.k) return;
  const SplitWs w(ws, B, G);
  uint32_t* rec = w.rec + static_cast<int64_t>(b) * kRec;
  const uint32_t lo = rec[kRecLo], hi = rec[kRecHi];
  const int s = static_cast<int>(rec[kRecShift]);
  const uint32_t* ghist = w.hist + static_cast<int64_t>(b) * kHistBins;
  for (int i = threadIdx.x; i < kHistBins / 4; i += T) {
    reinterpret_cast<uint4*>(sm.sel.hist[0])[i] = reinterpret_cast<const uint4*>(ghist)[i];
  }
  hist_clear<T>(sm.sel.hist[1]);
  __syncthreads();
  find_threshold_bin<T>(sm.sel.hist[0], static_cast<uint32_t>(p.k), 0u, sm.sel.wsum, sm.sel.res);
  Sel sel{};
  sel.kk = static_cast<uint32_t>(p.k) - sm.sel.res[1];
  sel.bucket = sm.sel.res[2];
  sel.lo = lo + (sm.sel.res[0] << s);
  sel.hi = hi;
  sel.dhi = static_cast<uint32_t>(r.n - 1);
  const uint32_t width = (1u << s) - 1u;
  if (sel.hi - sel.lo > width) sel.hi = sel.lo + width;
  if (sel.bucket > static_cast<uint32_t>(kSmallCap)) {
    const Span<T, VEC, V4> span{r.row, 0, r.n};
    uint32_t key[4 * VEC];
    int round = 1;
    sel = refine<T>([&](auto&& f) { span.template for_each<false>(key, f); }, sm.sel, sel,
                    static_cast<uint32_t>(r.n - 1), span.pad_slots(), 0u, round);
  }
  if (threadIdx.x == 0) {
    rec[kRecLo] = sel.lo;
    rec[kRecHi] = sel.hi;
    rec[kRecKk] = sel.kk;
    rec[kRecTie] = sel.tie;
    rec[kRecDlo] = sel.dlo;
    rec[kRecDhi] = sel.dhi;
  }
}

template <int T, int VEC, int MODE, bool V4>
__global__ __launch_bounds__(T) void split_scatter(Params p, uint32_t* ws, int32_t B, int32_t G,
                                                   int32_t chunk) {
  constexpr int W = T / 64;
  __shared__ uint32_t wsum[16];
  __shared__ uint32_t base[2];
  const int b = blockIdx.x / G, g = blockIdx.x % G;
  const RowRef<MODE> r(p, b);
  if (r.n <= p.k) return;
  const SplitWs w(ws, B, G);
  uint32_t* rec = w.rec + static_cast<int64_t>(b) * kRec;
  const Span<T, VEC, V4> span{r.row, g * chunk, chunk_end(g, G, chunk, r.n)};
  uint32_t key[4 * VEC];
  if (span.start >= span.end) return;
  Sel sel{};
  sel.lo = rec[kRecLo];
  sel.hi = rec[kRecHi];
  sel.kk = rec[kRecKk];
  sel.tie = rec[kRecTie];
  sel.dlo = rec[kRecDlo];
  sel.dhi = rec[kRecDhi];
  const uint32_t nm1 = static_cast<uint32_t>(r.n - 1);
  const uint32_t first = static_cast<uint32_t>(p.k) - sel.kk;
  uint2* cand = w.cand + static_cast<int64_t>(b) * kSmallCap;
  with_span(span, key, [&](auto res) {
    constexpr bool RES = decltype(res)::value;
    uint32_t nw = 0, nc = 0;
    span.template for_each<RES>(key, [&](uint32_t x, int32_t pos, int) {
      nw += sel_winner(sel, nm1, span.end, x, pos) ? 1u : 0u;
      nc += sel_bucket(sel, nm1, span.end, x, pos) ? 1u : 0u;
    });
    // one scan of (winners | bucket << 16): a chunk has fewer than 2^16 of each
    const uint32_t packed = nw | (nc << 16);
    const uint32_t incl = wave_incl_scan(packed);
    const int wid = threadIdx.x >> 6;
    if (__lane_id() == 63) wsum[wid] = incl;
    __syncthreads();
    uint32_t off = incl - packed, tot = 0;
#pragma unroll
    for (int i = 0; i < W; ++i) {
      off += (i < wid) ? wsum[i] : 0u;
      tot += wsum[i];
    }
    if (threadIdx.x == 0) {
      const uint64_t add = (static_cast<uint64_t>(tot & 0xFFFFu) << 32) | (tot >> 16);
      const uint64_t old = __hip_atomic_fetch_add(reinterpret_cast<uint64_t*>(rec + kRecCursor), add,
                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      base[0] = static_cast<uint32_t>(old >> 32);
      base[1] = static_cast<uint32_t>(old);
    }
    __syncthreads();
    uint32_t wo = base[0] + (off & 0xFFFFu);
    uint32_t co = base[1] + (off >> 16);
    span.template for_each<RES>(key, [&](uint32_t x, int32_t pos, int) {
      if (sel_winner(sel, nm1, span.end, x, pos)) {
        if (wo < first) r.out[wo] = out_value<MODE>(p, false, nullptr, r.pt_row, r.row_start, pos);
        ++wo;
      }
      if (sel_bucket(sel, nm1, span.end, x, pos)) {
        if (co < static_cast<uint32_t>(kSmallCap)) cand[co] = make_uint2(x, static_cast<uint32_t>(pos));
        ++co;
      }
    });
  });
}

template <int T, int MODE>
__global__ __launch_bounds__(T) void split_finish(Params p, uint32_t* ws, int32_t B, int32_t G) {
  __shared__ uint2 cand[kSmallCap];
  const int b = blockIdx.x;
  const RowRef<MODE> r(p, b);
  if (r.n <= p.k) {
    emit_whole_row<T, MODE>(p, r);
    return;
  }
  const SplitWs w(ws, B, G);
  const uint32_t* rec = w.rec + static_cast<int64_t>(b) * kRec;
  const uint32_t kk = rec[kRecKk];
  const uint32_t nc = min(rec[kRecCursor], static_cast<uint32_t>(kSmallCap));
  const uint2* gc = w.cand + static_cast<int64_t>(b) * kSmallCap;
  for (uint32_t i = threadIdx.x; i < nc; i += T) cand[i] = gc[i];
  __syncthreads();
  rank_bucket<T>(cand, nc, kk, static_cast<uint32_t>(p.k) - kk, [&](uint32_t slot, int32_t pos) {
    r.out[slot] = out_value<MODE>(p, false, nullptr, r.pt_row, r.row_start, pos);
  });
}

}  // namespace ets

// ==================================================================== host side

namespace {

struct DeviceInfo {
  bool queried = false;
  bool supported = false;
  int cu_count = 0;
};

constexpr int kMaxDevices = 64;
std::mutex g_dev_mutex;
DeviceInfo g_dev[kMaxDevices];

ets_status current_device(int* dev_out, DeviceInfo* info_out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ETS_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_dev_mutex);
  DeviceInfo& d = g_dev[dev];
  if (!d.queried) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ETS_ERR_DEVICE;
    d.supported = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.cu_count = prop.multiProcessorCount;
    d.queried = true;
  }
  if (!d.supported) return ETS_ERR_DEVICE;
  *dev_out = dev;
  *info_out = d;
  return ETS_OK;
}

int32_t page_shift_of(int32_t ps) {
  if (ps <= 0 || (ps & (ps - 1)) != 0) return -1;
  int32_t s = 0;
  while ((1 << s) < ps) ++s;
  return s;
}

constexpr int kRowThreads = 1024;
constexpr int kRowVec = 8;  // 8 x float4 per lane -> 32768 scores per tile
constexpr int64_t kRowTile = static_cast<int64_t>(kRowThreads) * 4 * kRowVec;

// row-split path: chunk workgroups of 256 lanes x 16 scores, per-row kernels of 1024 lanes
constexpr int kSplitThreads = 256;
constexpr int kSplitVec = 4;
constexpr int64_t kSplitChunk = static_cast<int64_t>(kSplitThreads) * 4 * kSplitVec;  // 4096
constexpr int kSelThreads = 1024;
constexpr int kSelVec = 8;

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// Chunks per row (0 = one workgroup per row).  A row that fits one resident
// tile stays on one workgroup; longer rows are cut into kSplitChunk chunks.
// ETS_ROW_SPLIT = 0 disables splitting; a positive value forces that many
// chunks per row.
int32_t split_plan(int32_t B, int64_t max_len) {
  (void)B;
  if (const char* e = std::getenv("ETS_ROW_SPLIT"); e != nullptr && *e != '\0') {
    char* end = nullptr;
    const long v = std::strtol(e, &end, 10);
    if (end != e && *end == '\0' && v >= 0 && v <= 65536) {
      if (v == 0 || max_len <= 0) return 0;
      return static_cast<int32_t>(std::min<int64_t>(v, (max_len + 3) / 4));
    }
  }
  if (max_len <= kRowTile) return 0;
  return static_cast<int32_t>((max_len + kSplitChunk - 1) / kSplitChunk);
}

int32_t split_chunk(int64_t max_len, int32_t G) {
  const int64_t c = (max_len + G - 1) / G;
  return static_cast<int32_t>((c + 3) / 4 * 4);
}

size_t split_ws_bytes(int32_t B, int32_t G) {
  const size_t words = static_cast<size_t>(B) *
                       (ets::kRec + 4 * static_cast<size_t>(G) + ets::kHistBins + 2 * ets::kSmallCap);
  return (words * 4 + 255) / 256 * 256;
}

// Host-side check of the split path's workspace, before any HIP call.
ets_status check_workspace(int32_t B, int64_t max_len, const void* ws, size_t ws_bytes) {
  const int32_t G = split_plan(B, max_len);
  if (G == 0) return ETS_OK;
  if (static_cast<int64_t>(B) * G > INT32_MAX) return ETS_ERR_INVALID_ARG;
  if (!ws || ws_bytes < split_ws_bytes(B, G) || !aligned16(ws)) return ETS_ERR_WORKSPACE;
  return ETS_OK;
}

template <int MODE, bool V4, int T, int VEC, bool STREAM>
void launch_rows(const ets::Params& p, int32_t B, hipStream_t stream) {
  hipLaunchKernelGGL((ets::row_topk_kernel<T, VEC, MODE, V4, STREAM>), dim3(B), dim3(T), 0, stream,
                     p);
}

template <int MODE, bool V4>
ets_status launch(const ets::Params& p, int32_t B, int64_t max_len, void* ws, size_t ws_bytes,
                  hipStream_t stream) {
  const int32_t G = split_plan(B, max_len);
  if (G == 0) {
    // the smallest resident tile (1024 lanes x 4 VEC scores) that holds the row
    // the smallest resident tile that holds the row, with as few scores per
    // lane as the lane count allows: the passes are latency bound, and more
    // waves with shorter slot loops hide more of it
    if (max_len <= 2048) {
      launch_rows<MODE, V4, 512, 1, false>(p, B, stream);
    } else if (max_len <= 4096) {
      launch_rows<MODE, V4, kRowThreads, 1, false>(p, B, stream);
    } else if (max_len <= kRowTile / 4) {
      launch_rows<MODE, V4, kRowThreads, kRowVec / 4, false>(p, B, stream);
    } else if (max_len <= kRowTile / 2) {
      launch_rows<MODE, V4, kRowThreads, kRowVec / 2, false>(p, B, stream);
    } else if (max_len <= kRowTile) {
      launch_rows<MODE, V4, kRowThreads, kRowVec, false>(p, B, stream);
    } else {
      launch_rows<MODE, V4, kRowThreads, kRowVec, true>(p, B, stream);
    }
    return hipGetLastError() == hipSuccess ? ETS_OK : ETS_ERR_HIP;
  }
  // (workspace already validated by check_workspace)
  const int32_t chunk = split_chunk(max_len, G);
  auto* w = static_cast<uint32_t*>(ws);
  const int64_t zero_words = static_cast<int64_t>(B) * (ets::kRec + ets::kHistBins);
  const int zero_blocks = static_cast<int>(std::min<int64_t>(1024, (zero_words + 255) / 256));
  const dim3 chunks(static_cast<uint32_t>(B) * G), rows(B);
  hipLaunchKernelGGL(ets::split_zero, dim3(zero_blocks), dim3(256), 0, stream, w, B, G);
  hipLaunchKernelGGL((ets::split_bounds<kSplitThreads, kSplitVec, MODE, V4>), chunks,
                     dim3(kSplitThreads), 0, stream, p, w, B, G, chunk);
  hipLaunchKernelGGL((ets::split_hist<kSplitThreads, kSplitVec, MODE, V4>), chunks,
                     dim3(kSplitThreads), 0, stream, p, w, B, G, chunk);
  hipLaunchKernelGGL((ets::split_select<kSelThreads, kSelVec, MODE, V4>), rows, dim3(kSelThreads),
                     0, stream, p, w, B, G);
  hipLaunchKernelGGL((ets::split_scatter<kSplitThreads, kSplitVec, MODE, V4>), chunks,
                     dim3(kSplitThreads), 0, stream, p, w, B, G, chunk);
  hipLaunchKernelGGL((ets::split_finish<kSelThreads, MODE>), rows, dim3(kSelThreads), 0, stream, p,
                     w, B, G);
  return hipGetLastError() == hipSuccess ? ETS_OK : ETS_ERR_HIP;
}

}  // namespace

extern "C" {

const char* ets_status_string(ets_status status) {
  switch (status) {
    case ETS_OK: return "ok";
    case ETS_ERR_INVALID_ARG: return "invalid argument";
    case ETS_ERR_K_RANGE: return "k outside [1, ETS_MAX_K]";
    case ETS_ERR_WORKSPACE: return "workspace too small";
    case ETS_ERR_DEVICE: return "unsupported or unavailable device (gfx950 required)";
    case ETS_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int32_t ets_row_split(int32_t B, int64_t max_row_len, int32_t cu_count) {
  (void)cu_count;
  return split_plan(B, max_row_len);
}

ets_status ets_workspace_size(int32_t B, int64_t max_row_len, int32_t k, int32_t device,
                              size_t* bytes) {
  if (!bytes || B < 0 || max_row_len < 0) return ETS_ERR_INVALID_ARG;
  if (k < 1 || k > ETS_MAX_K) return ETS_ERR_K_RANGE;
  (void)device;
  const int32_t G = split_plan(B, max_row_len);
  *bytes = (G == 0 || B == 0) ? 0 : split_ws_bytes(B, G);
  return ETS_OK;
}

ets_status ets_topk_raw(const float* scores, int64_t row_stride, int32_t B, int32_t L,
                        const int32_t* lens, int32_t k, int32_t* out, int64_t out_stride,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (k < 1 || k > ETS_MAX_K) return ETS_ERR_K_RANGE;
  if (B < 0 || L < 0 || row_stride < L || out_stride < k) return ETS_ERR_INVALID_ARG;
  if (B == 0) return ETS_OK;
  if (!out || (L > 0 && !scores)) return ETS_ERR_INVALID_ARG;
  if (ets_status st = check_workspace(B, L, workspace, workspace_bytes); st != ETS_OK) return st;
  int dev;
  DeviceInfo info;
  if (ets_status st = current_device(&dev, &info); st != ETS_OK) return st;
  ets::Params p{};
  p.scores = scores;
  p.row_stride = row_stride;
  p.lens = lens;
  p.L = L;
  p.k = k;
  p.out = out;
  p.out_stride = out_stride;
  p.page_shift = -1;
  const bool v4 = aligned16(scores) && (row_stride % 4 == 0) && (L % 4 == 0);
  auto s = static_cast<hipStream_t>(stream);
  return v4 ? launch<ets::kRaw, true>(p, B, L, workspace, workspace_bytes, s)
            : launch<ets::kRaw, false>(p, B, L, workspace, workspace_bytes, s);
}

ets_status ets_topk_paged(const float* scores, int64_t row_stride, int32_t B, int32_t L,
                          const int32_t* seq_lens, const int32_t* page_table, int64_t pt_stride,
                          int32_t page_size, int32_t k, int32_t* out, int64_t out_stride,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (k < 1 || k > ETS_MAX_K) return ETS_ERR_K_RANGE;
  if (B < 0 || L < 0 || row_stride < L || out_stride < k || page_size < 1 || pt_stride < 0)
    return ETS_ERR_INVALID_ARG;
  if (B == 0) return ETS_OK;
  if (!out || !seq_lens || !page_table || (L > 0 && !scores)) return ETS_ERR_INVALID_ARG;
  if (ets_status st = check_workspace(B, L, workspace, workspace_bytes); st != ETS_OK) return st;
  int dev;
  DeviceInfo info;
  if (ets_status st = current_device(&dev, &info); st != ETS_OK) return st;
  ets::Params p{};
  p.scores = scores;
  p.row_stride = row_stride;
  p.lens = seq_lens;
  p.page_table = page_table;
  p.pt_stride = pt_stride;
  p.page_size = page_size;
  p.page_shift = page_shift_of(page_size);
  p.L = L;
  p.k = k;
  p.out = out;
  p.out_stride = out_stride;
  const bool v4 = aligned16(scores) && (row_stride % 4 == 0) && (L % 4 == 0);
  auto s = static_cast<hipStream_t>(stream);
  return v4 ? launch<ets::kPaged, true>(p, B, L, workspace, workspace_bytes, s)
            : launch<ets::kPaged, false>(p, B, L, workspace, workspace_bytes, s);
}

ets_status ets_topk_ragged(const float* packed, const int32_t* row_starts,
                           const int32_t* lengths, int32_t B, int64_t max_len_hint, int32_t k,
                           int32_t* out, int64_t out_stride, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (k < 1 || k > ETS_MAX_K) return ETS_ERR_K_RANGE;
  if (B < 0 || max_len_hint < 0 || out_stride < k) return ETS_ERR_INVALID_ARG;
  if (B == 0) return ETS_OK;
  if (!out || !row_starts || !lengths || !packed) return ETS_ERR_INVALID_ARG;
  if (ets_status st = check_workspace(B, max_len_hint, workspace, workspace_bytes); st != ETS_OK)
    return st;
  int dev;
  DeviceInfo info;
  if (ets_status st = current_device(&dev, &info); st != ETS_OK) return st;
  ets::Params p{};
  p.scores = packed;
  p.lens = lengths;
  p.row_starts = row_starts;
  p.k = k;
  p.out = out;
  p.out_stride = out_stride;
  p.page_shift = -1;
  return launch<ets::kRagged, false>(p, B, max_len_hint, workspace, workspace_bytes,
                                     static_cast<hipStream_t>(stream));
}

}  // extern "C"
