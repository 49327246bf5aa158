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

template <int MODE>
__device__ __forceinline__ int32_t map_position(const Params& p, const int32_t* pt_row,
                                                int32_t row_start, int32_t pos) {
  if constexpr (MODE == kPaged) {
    int32_t page, slot;
    if (p.page_shift >= 0) {
      page = pos >> p.page_shift;
      slot = pos & (p.page_size - 1);
    } else {
      page = pos / p.page_size;
      slot = pos - page * p.page_size;
    }
    return pt_row[page] * p.page_size + slot;
  } else if constexpr (MODE == kRagged) {
    return row_start + pos;
  } else {
    return pos;
  }
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

// Exclusive prefix sum over the block in thread order; `total` gets the sum.
// Uses s_wave[0 .. T/64); ends with a barrier so s_wave may be reused.
template <int T>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* s_wave, uint32_t& total) {
  constexpr int W = T / 64;
  const int wid = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan(v);
  if (__lane_id() == 63) s_wave[wid] = incl;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const uint32_t s = s_wave[w];
    tot += s;
    before += (w < wid) ? s : 0u;
  }
  __syncthreads();
  total = tot;
  return before + incl - v;
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
// above(t) counts the entries of all higher bins.  Every thread gets
// (t, above(t), hist[t]) in s_res[0..2] after the final barrier.
template <int T>
__device__ __forceinline__ void find_threshold_bin(const uint32_t* hist, uint32_t kk,
                                                   uint32_t* s_wave, uint32_t* s_res) {
  constexpr int BPT = kHistBins / T;  // bins owned by each thread
  static_assert(BPT * T == kHistBins && BPT % 4 == 0, "block size must divide the bins by 4");
  uint32_t h[BPT];
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < BPT; i += 4) {
    const uint4 q = reinterpret_cast<const uint4*>(hist)[threadIdx.x * (BPT / 4) + i / 4];
    h[i] = q.x;
    h[i + 1] = q.y;
    h[i + 2] = q.z;
    h[i + 3] = q.w;
    s += q.x + q.y + q.z + q.w;
  }
  uint32_t total;
  const uint32_t excl = block_excl_scan<T>(s, s_wave, total);
  uint32_t above = total - excl - s;  // entries in bins of higher threads
#pragma unroll
  for (int i = BPT - 1; i >= 0; --i) {
    if (above < kk && kk <= above + h[i]) {
      s_res[0] = threadIdx.x * BPT + i;
      s_res[1] = above;
      s_res[2] = h[i];
    }
    above += h[i];
  }
  __syncthreads();
}

// ---------------------------------------------------------------- single-workgroup row kernel

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

struct alignas(16) RowSmem {
  uint32_t hist[kHistBins];    // LDS histogram (16 KiB)
  int32_t pt[kPtCap];          // staged page-table row (paged map)
  uint2 cand[kSmallCap];       // threshold bucket: (key, position)
  uint32_t wave[64];
  uint32_t res[4];
  uint32_t ccount;
};

// Element layout of one tile held by a thread.  V4: float4 v of thread t holds
// positions 4 (v T + t) + c; scalar: element j of thread t is at j T + t.
// In both layouts a thread's positions increase with j.
template <int T, bool V4>
__device__ __forceinline__ int32_t tile_pos(int j) {
  if constexpr (V4) {
    return 4 * ((j >> 2) * T + static_cast<int>(threadIdx.x)) + (j & 3);
  } else {
    return j * T + static_cast<int>(threadIdx.x);
  }
}

// Loads one tile of keys.  Slots at positions >= n get key 0 and are never
// counted: the passes below correct for them arithmetically (see row_topk).
template <int T, int VEC, bool V4>
__device__ __forceinline__ void load_tile(uint32_t (&key)[4 * VEC], const float* row, int32_t n,
                                             int64_t cap, int32_t base) {
  const int32_t tid = static_cast<int32_t>(threadIdx.x);
  if constexpr (V4) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      const int32_t q = base + 4 * (v * T + tid);
      if (q + 3 < n) {
        const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + q));
        key[4 * v + 0] = order_key(w.x);
        key[4 * v + 1] = order_key(w.y);
        key[4 * v + 2] = order_key(w.z);
        key[4 * v + 3] = order_key(w.w);
      } else if (q < n) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          key[4 * v + c] = (q + c < n) ? order_key(__float_as_uint(row[q + c])) : 0u;
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) key[4 * v + c] = 0u;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4 * VEC; ++j) {
      const int32_t q = base + j * T + tid;
      key[j] = (q < n) ? order_key(__builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(row) + q)) : 0u;
    }
  }
  (void)cap;
}

// Clears the histogram (call between barriers).
template <int T>
__device__ __forceinline__ void hist_clear(uint32_t* hist) {
#pragma unroll
  for (int i = threadIdx.x; i < kHistBins / 4; i += T) {
    reinterpret_cast<uint4*>(hist)[i] = make_uint4(0, 0, 0, 0);
  }
}

// One exact top-k row on one workgroup.  STREAM = false: the row (n <= one
// tile) is loaded once and every pass runs on registers.  STREAM = true: any
// length; every pass streams the row tile by tile.
//
// Slots beyond the row hold key 0.  They can only matter while the key range
// starts at 0, where all of them fall into bin 0: that bin is corrected by
// their known count, and the passes that emit positions check pos < n.
template <int T, int VEC, int MODE, bool V4, bool STREAM>
__device__ __forceinline__ void row_topk(const Params& p, RowSmem& sm, int32_t n, const float* row,
                                         int64_t cap, int32_t row_start, const int32_t* pt_row,
                                         int32_t* out) {
  constexpr int PT = 4 * VEC;
  constexpr int TILE = T * PT;
  constexpr int W = T / 64;
  const int tid = threadIdx.x;
  const int wid = tid >> 6;
  const int32_t k = p.k;
  // Slots a thread uses in a tile of nt scores: whole float4 groups (V4) or
  // whole strides (scalar) that hold at least one score.  Uniform per block.
  auto slots_for = [](int32_t nt) -> int32_t {
    return V4 ? min(4 * ((nt + 4 * T - 1) / (4 * T)), PT) : min((nt + T - 1) / T, PT);
  };
  const int32_t ntiles = STREAM ? (n + TILE - 1) / TILE : 1;
  const int32_t last_n = n - (ntiles - 1) * TILE;  // scores in the last tile
  const int32_t jlim = slots_for(last_n);           // resident rows: used slots
  // key-0 slots inside the used slots (only the last tile has any)
  const uint32_t n_pad = static_cast<uint32_t>(jlim * T - last_n);

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
      for (int i = 0; i < PTV; ++i) ptv[i] = (tid + i * T < npages) ? pt_row[tid + i * T] : 0;
    }
  }

  uint32_t key[PT];
  if constexpr (!STREAM) load_tile<T, VEC, V4>(key, row, n, cap, 0);

  if constexpr (MODE == kPaged) {
    if (pt_lds) {
#pragma unroll
      for (int i = 0; i < PTV; ++i)
        if (tid + i * T < npages) sm.pt[tid + i * T] = ptv[i];
    }
  }

  // f(key, position) over every used slot of the row this thread holds;
  // slots past the row's end are skipped block-uniformly.
  auto for_each = [&](auto&& f) {
    if constexpr (STREAM) {
      for (int32_t base = 0; base < n; base += TILE) {
        load_tile<T, VEC, V4>(key, row, n, cap, base);
        const int32_t jl = slots_for(n - base);
#pragma unroll
        for (int j = 0; j < PT; ++j)
          if (j < jl) f(key[j], base + tile_pos<T, V4>(j));
      }
    } else {
#pragma unroll
      for (int j = 0; j < PT; ++j)
        if (j < jlim) f(key[j], tile_pos<T, V4>(j));
    }
  };

  // ---- bounds: row max and a lower bound of the k-th largest key.  Each
  // thread's jth-largest key, over the nfull threads that hold at least jth
  // scores, gives nfull * jth distinct scores at or above their minimum;
  // jth = ceil(k / threads holding scores) <= 2.  Key-0 padding never raises
  // m1 or m2 of such a thread.  Otherwise the row minimum is the bound.
  const int32_t holders = V4 ? min(T, (n + 3) / 4) : min(T, n);
  const int32_t jth = (k + holders - 1) / holders;
  uint32_t m1 = 0, m2 = 0;
  for_each([&](uint32_t x, int32_t) {
    m2 = max(m2, min(m1, x));
    m1 = max(m1, x);
  });
  uint32_t lo, hi;
  {
    // this thread's first jth slots are positions 4 tid .. (V4) or tid, tid + T (scalar)
    const int32_t jpos = V4 ? 4 * tid + jth - 1 : (jth - 1) * T + tid;
    const bool full = jth <= 2 && jpos < n;
    const uint32_t rmax = wave_reduce(m1, OpMax());
    const uint32_t bmin = wave_reduce(full ? (jth == 1 ? m1 : m2) : 0xFFFFFFFFu, OpMin());
    const uint32_t nfull = wave_reduce(full ? 1u : 0u, OpAdd());
    if (__lane_id() == 0) {
      sm.wave[wid] = rmax;
      sm.wave[16 + wid] = bmin;
      sm.wave[32 + wid] = nfull;
    }
    __syncthreads();
    uint32_t gmax = 0, gb = 0xFFFFFFFFu, gfull = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      gmax = max(gmax, sm.wave[w]);
      gb = min(gb, sm.wave[16 + w]);
      gfull += sm.wave[32 + w];
    }
    __syncthreads();
    hi = gmax;
    if (jth <= 2 && gfull * static_cast<uint32_t>(jth) >= static_cast<uint32_t>(k)) {
      lo = gb;
    } else {
      uint32_t mn = 0xFFFFFFFFu;
      for_each([&](uint32_t x, int32_t pos) { mn = min(mn, pos < n ? x : 0xFFFFFFFFu); });
      mn = wave_reduce(mn, OpMin());
      if (__lane_id() == 0) sm.wave[wid] = mn;
      __syncthreads();
      lo = 0xFFFFFFFFu;
#pragma unroll
      for (int w = 0; w < W; ++w) lo = min(lo, sm.wave[w]);
      __syncthreads();
    }
  }

  // ---- radix rounds on the key inside [lo, hi] until the threshold bucket is
  // small, or a single key.  Each round first probes how many lanes of a wave
  // share one bin; only then is the merging (peeled) LDS atomic worth its cost.
  uint32_t kk = static_cast<uint32_t>(k);
  uint32_t bucket = 0;
  for (;;) {
    const uint32_t span = hi - lo;
    const int bl = span ? 32 - __clz(static_cast<int>(span)) : 0;
    const int s = bl > kHistBits ? bl - kHistBits : 0;
    {
      const uint32_t d = key[0] - lo;
      const uint32_t bin = d >> s;
      const uint32_t lead = readfirstlane(bin);
      const uint32_t share = static_cast<uint32_t>(__popcll(__ballot(d <= span && bin == lead)));
      if (__lane_id() == 0) sm.wave[48 + wid] = share;
    }
    hist_clear<T>(sm.hist);
    __syncthreads();
    uint32_t max_share = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) max_share = max(max_share, sm.wave[48 + w]);
    if (max_share > kPeelShare) {
      for_each([&](uint32_t x, int32_t) {
        const uint32_t d = x - lo;
        hist_add_peel(sm.hist, d <= span, d >> s);
      });
    } else {
      for_each([&](uint32_t x, int32_t) {
        const uint32_t d = x - lo;
        if (d <= span) atomicAdd(&sm.hist[d >> s], 1u);
      });
    }
    __syncthreads();
    if (lo == 0) {
      if (tid == 0) sm.hist[0] -= n_pad;
      __syncthreads();
    }
    find_threshold_bin<T>(sm.hist, kk, sm.wave, sm.res);
    const uint32_t t = sm.res[0];
    kk -= sm.res[1];
    bucket = sm.res[2];
    lo += t << s;
    const uint32_t width = (1u << s) - 1u;
    if (hi - lo > width) hi = lo + width;
    __syncthreads();  // sm.res is rewritten by the next round
    if (bucket <= static_cast<uint32_t>(kSmallCap) || s == 0) break;
  }

  // ---- a single key with too many ties: radix rounds on d = n - 1 - pos
  // among the scores equal to it (the largest d is the lowest position).
  // Padding slots have pos >= n, so their d wraps far above any range.
  // Positions are distinct, so these histograms never pile onto one bin.
  const bool tie_stage = bucket > static_cast<uint32_t>(kSmallCap);
  uint32_t dlo = 0, dhi = static_cast<uint32_t>(n - 1);
  const uint32_t nm1 = static_cast<uint32_t>(n - 1);
  if (tie_stage) {
    const uint32_t tkey = lo;
    for (;;) {
      const uint32_t span = dhi - dlo;
      const int bl = span ? 32 - __clz(static_cast<int>(span)) : 0;
      const int sd = bl > kHistBits ? bl - kHistBits : 0;
      hist_clear<T>(sm.hist);
      __syncthreads();
      for_each([&](uint32_t x, int32_t pos) {
        const uint32_t d = nm1 - static_cast<uint32_t>(pos) - dlo;
        if (x == tkey && d <= span) atomicAdd(&sm.hist[d >> sd], 1u);
      });
      __syncthreads();
      find_threshold_bin<T>(sm.hist, kk, sm.wave, sm.res);
      const uint32_t t = sm.res[0];
      kk -= sm.res[1];
      bucket = sm.res[2];
      dlo += t << sd;
      const uint32_t width = (1u << sd) - 1u;
      if (dhi - dlo > width) dhi = dlo + width;
      __syncthreads();
      if (bucket <= static_cast<uint32_t>(kSmallCap)) break;
    }
  }

  // Winners: key above the bucket, or (tie stage) the bucket's key at a
  // lower position than the bucket.  Bucket: the remaining candidates.
  const uint32_t klo = lo, khi = hi, kspan = hi - lo, dspan = dhi - dlo;
  // output value of a selected position
  auto emit = [&](uint32_t slot, int32_t pos) {
    int32_t v;
    if constexpr (MODE == kPaged) {
      int32_t page, off;
      if (p.page_shift >= 0) {
        page = pos >> p.page_shift;
        off = pos & (p.page_size - 1);
      } else {
        page = pos / p.page_size;
        off = pos - page * p.page_size;
      }
      v = (pt_lds ? sm.pt[page] : pt_row[page]) * p.page_size + off;
    } else if constexpr (MODE == kRagged) {
      v = row_start + pos;
    } else {
      v = pos;
    }
    out[slot] = v;
  };

  if (tid == 0) sm.ccount = 0;
  __syncthreads();
  // Count winners, gather the bucket into LDS (rare: skipped per wave), and
  // emit the winners in thread order.  TIE selects the tie-stage tests.
  auto scatter = [&](auto tie_tag) -> uint32_t {
    constexpr bool TIE = decltype(tie_tag)::value;
    auto is_winner = [&](uint32_t x, int32_t pos) {
      if constexpr (!TIE) {
        return x > khi;
      } else {
        const uint32_t d = nm1 - static_cast<uint32_t>(pos);
        return x > khi || (x == khi && d > dhi && d <= nm1);
      }
    };
    auto in_bucket = [&](uint32_t x, int32_t pos) {
      if constexpr (!TIE) {
        return x - klo <= kspan && pos < n;
      } else {
        return x == khi && nm1 - static_cast<uint32_t>(pos) - dlo <= dspan;
      }
    };
    auto gather = [&](uint32_t x, int32_t pos) {
      const bool c = in_bucket(x, pos);
      if (__ballot(c) != 0 && c) {
        const uint32_t slot = atomicAdd(&sm.ccount, 1u);
        if (slot < static_cast<uint32_t>(kSmallCap)) sm.cand[slot] = make_uint2(x, static_cast<uint32_t>(pos));
      }
    };
    const uint32_t first = static_cast<uint32_t>(k) - kk;  // number of winners
    if constexpr (!STREAM) {
      // bit j of wmask / cmask: slot j is a winner / a bucket candidate.  One
      // block scan of (winners | candidates << 16) places both, in thread order.
      uint32_t wmask = 0, cmask = 0;
#pragma unroll
      for (int j = 0; j < PT; ++j) {
        if (j < jlim) {
          const int32_t pos = tile_pos<T, V4>(j);
          wmask |= (is_winner(key[j], pos) ? 1u : 0u) << j;
          cmask |= (in_bucket(key[j], pos) ? 1u : 0u) << j;
        }
      }
      const uint32_t packed = static_cast<uint32_t>(__popc(wmask)) |
                              (static_cast<uint32_t>(__popc(cmask)) << 16);
      uint32_t total;
      const uint32_t excl = block_excl_scan<T>(packed, sm.wave, total);  // ends with a barrier
      uint32_t off = excl & 0xFFFFu;
      uint32_t coff = excl >> 16;
      if (tid == 0) sm.ccount = total >> 16;
      while (cmask != 0) {
        const int j = __ffs(static_cast<int>(cmask)) - 1;
        cmask &= cmask - 1u;
        const int32_t pos = V4 ? 4 * ((j >> 2) * T + tid) + (j & 3) : j * T + tid;
        if (coff < static_cast<uint32_t>(kSmallCap))
          sm.cand[coff] = make_uint2(select_slot<PT>(key, j), static_cast<uint32_t>(pos));
        ++coff;
      }
      __syncthreads();  // candidates visible; no global store is pending here
      // winners straight to the output; the bound only guards a broken invariant
      while (wmask != 0) {
        const int j = __ffs(static_cast<int>(wmask)) - 1;
        wmask &= wmask - 1u;
        const int32_t pos = V4 ? 4 * ((j >> 2) * T + tid) + (j & 3) : j * T + tid;
        if (off < first) emit(off, pos);
        ++off;
      }
    } else {
      uint32_t nwin = 0;
      for_each([&](uint32_t x, int32_t pos) {
        nwin += is_winner(x, pos) ? 1u : 0u;
        gather(x, pos);
      });
      uint32_t total_win;
      uint32_t off = block_excl_scan<T>(nwin, sm.wave, total_win);  // ends with a barrier
      for_each([&](uint32_t x, int32_t pos) {
        if (is_winner(x, pos)) {
          if (off < first) emit(off, pos);
          ++off;
        }
      });
    }
    return first;
  };
  const uint32_t first = tie_stage ? scatter(std::true_type()) : scatter(std::false_type());

  // ---- the bucket's best kk, placed by rank.  Eight lanes share a
  // candidate: each compares it with every eighth entry, then the lanes'
  // counts are summed with row permutes.
  {
    const uint32_t nc = min(sm.ccount, static_cast<uint32_t>(kSmallCap));
    static_assert(T >= 8 * kSmallCap, "eight lanes per bucket entry");
    const uint32_t i = tid >> 3;
    const uint32_t part = tid & 7;
    uint32_t rank = 0;
    uint2 ci = make_uint2(0, 0);
    if (i < nc) {
      ci = sm.cand[i];
#pragma unroll
      for (uint32_t q = 0; q < kSmallCap / 8; ++q) {
        const uint32_t j = part + 8 * q;
        const uint2 cj = sm.cand[min(j, nc - 1)];
        const bool before = cj.x > ci.x || (cj.x == ci.x && static_cast<int32_t>(cj.y) < static_cast<int32_t>(ci.y));
        rank += (j < nc && before) ? 1u : 0u;
      }
    }
    rank += dpp_perm<0xB1>(rank);   // quad_perm [1,0,3,2]
    rank += dpp_perm<0x4E>(rank);   // quad_perm [2,3,0,1]
    rank += dpp_perm<0x141>(rank);  // row_half_mirror: the other quad of the eight
    if (i < nc && part == 0 && rank < kk) emit(first + rank, static_cast<int32_t>(ci.y));
  }
}

// One workgroup per row.  STREAM = false: rows fit one tile (the host
// guarantees it for dense rows; a ragged row longer than its length hint
// falls back to the streamed passes).  STREAM = true: any row length.
template <int T, int VEC, int MODE, bool V4, bool STREAM>
__global__ __launch_bounds__(T) void row_topk_kernel(Params p) {
  constexpr int TILE = T * 4 * VEC;
  __shared__ RowSmem sm;
  const int b = blockIdx.x;

  int32_t n;
  int32_t row_start = 0;
  int64_t cap;  // readable scores from the row base
  const float* row;
  if constexpr (MODE == kRagged) {
    row_start = p.row_starts[b];
    n = max(p.lens[b], 0);
    row = p.scores + row_start;
    cap = n;
  } else {
    n = p.lens ? min(max(p.lens[b], 0), p.L) : p.L;
    row = p.scores + static_cast<int64_t>(b) * p.row_stride;
    cap = p.L;
  }
  const int32_t* pt_row = nullptr;
  if constexpr (MODE == kPaged) pt_row = p.page_table + static_cast<int64_t>(b) * p.pt_stride;
  int32_t* out = p.out + static_cast<int64_t>(b) * p.out_stride;

  if (n <= p.k) {
    // every position is selected, the rest is padding
    for (int32_t i = threadIdx.x; i < p.k; i += T) {
      out[i] = (i < n) ? map_position<MODE>(p, pt_row, row_start, i) : -1;
    }
    return;
  }
  if constexpr (STREAM) {
    row_topk<T, VEC, MODE, V4, true>(p, sm, n, row, cap, row_start, pt_row, out);
  } else {
    if constexpr (MODE == kRagged) {
      if (n > TILE) {
        row_topk<T, VEC, MODE, V4, true>(p, sm, n, row, cap, row_start, pt_row, out);
        return;
      }
    }
    row_topk<T, VEC, MODE, V4, false>(p, sm, n, row, cap, row_start, pt_row, out);
  }
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

template <int MODE, bool V4>
ets_status launch_rows(const ets::Params& p, int32_t B, int64_t max_len, hipStream_t stream) {
  if (max_len > kRowTile) {
    hipLaunchKernelGGL((ets::row_topk_kernel<kRowThreads, kRowVec, MODE, V4, true>), dim3(B),
                       dim3(kRowThreads), 0, stream, p);
  } else {
    hipLaunchKernelGGL((ets::row_topk_kernel<kRowThreads, kRowVec, MODE, V4, false>), dim3(B),
                       dim3(kRowThreads), 0, stream, p);
  }
  return hipGetLastError() == hipSuccess ? ETS_OK : ETS_ERR_HIP;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

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
  if (const char* e = std::getenv("ETS_ROW_SPLIT"); e != nullptr && *e != '\0') {
    char* end = nullptr;
    const long v = std::strtol(e, &end, 10);
    if (end != e && *end == '\0' && v >= 0 && v <= 1024) return static_cast<int32_t>(v);
  }
  (void)B;
  (void)max_row_len;
  (void)cu_count;
  return 0;
}

ets_status ets_workspace_size(int32_t B, int64_t max_row_len, int32_t k, int32_t device,
                              size_t* bytes) {
  if (!bytes || B < 0 || max_row_len < 0) return ETS_ERR_INVALID_ARG;
  if (k < 1 || k > ETS_MAX_K) return ETS_ERR_K_RANGE;
  (void)device;
  *bytes = 0;
  return ETS_OK;
}

ets_status ets_topk_raw(const float* scores, int64_t row_stride, int32_t B, int32_t L,
                        const int32_t* lens, int32_t k, int32_t* out, int64_t out_stride,
                        void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (k < 1 || k > ETS_MAX_K) return ETS_ERR_K_RANGE;
  if (B < 0 || L < 0 || row_stride < L || out_stride < k) return ETS_ERR_INVALID_ARG;
  if (B == 0) return ETS_OK;
  if (!out || (L > 0 && !scores)) return ETS_ERR_INVALID_ARG;
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
  return v4 ? launch_rows<ets::kRaw, true>(p, B, L, s) : launch_rows<ets::kRaw, false>(p, B, L, s);
}

ets_status ets_topk_paged(const float* scores, int64_t row_stride, int32_t B, int32_t L,
                          const int32_t* seq_lens, const int32_t* page_table, int64_t pt_stride,
                          int32_t page_size, int32_t k, int32_t* out, int64_t out_stride,
                          void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (k < 1 || k > ETS_MAX_K) return ETS_ERR_K_RANGE;
  if (B < 0 || L < 0 || row_stride < L || out_stride < k || page_size < 1 || pt_stride < 0)
    return ETS_ERR_INVALID_ARG;
  if (B == 0) return ETS_OK;
  if (!out || !seq_lens || !page_table || (L > 0 && !scores)) return ETS_ERR_INVALID_ARG;
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
  return v4 ? launch_rows<ets::kPaged, true>(p, B, L, s) : launch_rows<ets::kPaged, false>(p, B, L, s);
}

ets_status ets_topk_ragged(const float* packed, const int32_t* row_starts,
                           const int32_t* lengths, int32_t B, int64_t max_len_hint, int32_t k,
                           int32_t* out, int64_t out_stride, void* workspace,
                           size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (k < 1 || k > ETS_MAX_K) return ETS_ERR_K_RANGE;
  if (B < 0 || max_len_hint < 0 || out_stride < k) return ETS_ERR_INVALID_ARG;
  if (B == 0) return ETS_OK;
  if (!out || !row_starts || !lengths || !packed) return ETS_ERR_INVALID_ARG;
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
  return launch_rows<ets::kRagged, false>(p, B, max_len_hint, static_cast<hipStream_t>(stream));
}

}  // extern "C"
