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
//    Scores below the bound count into per-lane dummy bins past the
//    histogram, never into its bins;
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
constexpr int kSmallCap = 128;  // bucket ranked by direct comparison, 8 lanes per entry (1024 lanes)
// A one-workgroup row ranks buckets of up to kRankCap entries directly, with
// half as many lanes per entry above kSmallCap: one more radix round on a
// resident row costs a pass over every slot, a histogram search and the later
// rounds' histogram copies (up to 5.7 us, measured on rows whose first round
// left 129 to 256 entries), the wider ranking about 0.5 us.
constexpr int kRankCap = 256;
constexpr int kPtCap = 2048;    // page-table entries staged in LDS
constexpr uint32_t kPeelShare = 16;  // lanes of a wave in one bin that switch to merged atomics
// Radix rounds needed at most: 12 + 12 + 8 key bits, then 12 + 12 + 7 position
// bits; loops stop there even on inconsistent counts, so every kernel ends.
constexpr int kMaxRounds = 8;
constexpr int kSubCopies = 4;  // histogram copies of a row's later rounds (lane % 4)
// words between copies: a bin of two copies falls in different LDS banks
constexpr int kSubStride = (1 << 12) + 8;
// a resident row of at least kEarlyMinFill quarters of its tile takes the
// bounds of its first round from the waves whose loads arrive first, unless
// the range they leave puts up to 2^(s + log2 n - 23) > 2^(kEarlyMaxSpread -
// 23) of its n scores into one octave's bin of 2^s keys (measured on MI355X:
// rows below half a tile lost more to coarse bins than they gained)
constexpr int kEarlyMinFill = 2;
constexpr int kEarlyMaxSpread = 32;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum MapMode : int { kRaw = 0, kPaged = 1, kRagged = 2 };

struct Params {
  const float* scores;
  int64_t row_stride;          // dense rows
  const int32_t* lens;         // dense valid lengths (nullable) or ragged lengths
  const int32_t* row_starts;   // ragged
  const int32_t* win_starts;   // dense windows (nullable): row b selects among [win_starts[b], n_b)
  const int32_t* page_table;   // paged
  int64_t pt_stride;
  int32_t page_size;
  int32_t page_shift;          // log2(page_size) if a power of two, else -1
  int32_t L;                   // dense row capacity
  int32_t k;
  int32_t* out;
  int64_t out_stride;
  int32_t min_chunk;           // row groups: fewest scores in a member's chunk (see member_chunk)
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

// Slot masks: mask = 2 * mask + (a < b), resp. (a <= b), as one compare into
// VCC and one add with carry-in (the compiler's form takes a select and a
// shifted add on top of the compare).
__device__ __forceinline__ uint32_t shift_in_lt(uint32_t mask, uint32_t a, uint32_t b) {
  asm("v_cmp_lt_u32 vcc, %1, %2\n\tv_addc_co_u32 %0, vcc, %0, %0, vcc" : "+v"(mask) : "v"(a), "v"(b) : "vcc");
  return mask;
}
__device__ __forceinline__ uint32_t shift_in_le(uint32_t mask, uint32_t a, uint32_t b) {
  asm("v_cmp_le_u32 vcc, %1, %2\n\tv_addc_co_u32 %0, vcc, %0, %0, vcc" : "+v"(mask) : "v"(a), "v"(b) : "vcc");
  return mask;
}
__device__ __forceinline__ uint32_t shift_in_eq(uint32_t mask, uint32_t a, uint32_t b) {
  asm("v_cmp_eq_u32 vcc, %1, %2\n\tv_addc_co_u32 %0, vcc, %0, %0, vcc" : "+v"(mask) : "v"(a), "v"(b) : "vcc");
  return mask;
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

// One histogram pass over the keys of for_each into hist (bins of d =
// x - lo, d <= span, shifted by s; out-of-range keys go to the lane's dummy
// bin) for a wave whose lanes pile into one `hot` bin: each lane counts its
// hot keys in a register and sends them to its dummy bin instead, and the
// wave adds the hot count once, so that the pile causes no serialised LDS
// atomics (and no per-key scalar work).  Call in uniform control flow.
template <class ForEach>
__device__ __forceinline__ void hist_pass_hot(ForEach&& for_each, uint32_t* hist, uint32_t lo,
                                              uint32_t span, int s, uint32_t hot) {
  const uint32_t dummy = kHistBins + __lane_id();
  uint32_t cnt = 0;
  for_each([&](uint32_t x, int32_t, int) {
    const uint32_t d = x - lo;
    const uint32_t b = d <= span ? d >> s : dummy;
    const bool h = b == hot;
    cnt += h ? 1u : 0u;
    atomicAdd(&hist[h ? dummy : b], 1u);
  });
  cnt = wave_reduce(cnt, OpAdd());
  if (__lane_id() == 0 && cnt != 0) atomicAdd(&hist[hot], cnt);
}

// The wave's hot bin for a round: of the bins of lanes 0, 16, 32 and 48 (one
// probe slot each), the one most lanes share, with that lane count.  One
// probe lane holding an outlier no longer hides a bin that the rest of the
// wave piles into.
__device__ __forceinline__ uint2 wave_hot_bin(bool pred, uint32_t bin) {
  uint32_t best = 0, count = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t cand = readlane(bin, 16 * c);
    const uint32_t n = static_cast<uint32_t>(__popcll(__ballot(pred && bin == cand)));
    if (n > count) {
      count = n;
      best = cand;
    }
  }
  return make_uint2(best, count);
}

// Finds the histogram bin t with above(t) < kk <= above(t) + hist[t], where
// above(t) counts the entries of all higher bins; bin 0 is read as
// hist[0] - bin0_less.  Two barriers.  Every thread gets (t, above(t),
// hist[t]) in res[0..2].  wsum[] and res[] may be reused after one more
// barrier.
template <int T>
__device__ __forceinline__ void find_threshold_regs(uint32_t (&h)[kHistBins / T], uint32_t kk,
                                                   uint32_t* wsum, uint32_t* res);

template <int T>
__device__ __forceinline__ void find_threshold_bin(const uint32_t* hist, uint32_t kk,
                                                   uint32_t bin0_less, uint32_t* wsum,
                                                   uint32_t* res) {
  constexpr int BPT = kHistBins / T;  // bins owned by each thread
  static_assert(BPT * T == kHistBins && BPT % 4 == 0, "block size must divide the bins by 4");
  uint32_t h[BPT];
#pragma unroll
  for (int i = 0; i < BPT; i += 4) {
    const uint4 q = reinterpret_cast<const uint4*>(hist)[threadIdx.x * (BPT / 4) + i / 4];
    h[i] = q.x;
    h[i + 1] = q.y;
    h[i + 2] = q.z;
    h[i + 3] = q.w;
  }
  if (threadIdx.x == 0) h[0] -= bin0_less;
  find_threshold_regs<T>(h, kk, wsum, res);
}

// The search of find_threshold_bin on bins already in registers: thread t
// holds bins [t * BPT, (t + 1) * BPT).
template <int T>
__device__ __forceinline__ void find_threshold_regs(uint32_t (&h)[kHistBins / T], uint32_t kk,
                                                   uint32_t* wsum, uint32_t* res) {
  constexpr int BPT = kHistBins / T;
  constexpr int W = T / 64;
  const int wid = threadIdx.x >> 6;
  uint32_t s = 0;
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

// The search of find_threshold_bin by wave 0 alone, one barrier: lane l sums
// bins [64 l, 64 l + 64); a wave scan from the top finds the lane whose
// range holds the threshold; that range's 64 bins, one per lane, are scanned
// the same way.  res[0..2] as find_threshold_bin; the other waves wait at the
// barrier.
__device__ __forceinline__ void find_threshold_w0(const uint32_t* hist, uint32_t kk,
                                                  uint32_t bin0_less, uint32_t* res) {
  static_assert(kHistBins == 64 * 64, "64 bins per lane");
  if (threadIdx.x < 64) {
    const uint32_t l = threadIdx.x;
    const uint4* q = reinterpret_cast<const uint4*>(hist) + l * 16;
    // lanes 256 bytes apart would all meet the same banks: lane l visits its
    // 16-byte groups in the order i ^ (l % 16), so the lanes that the LDS
    // serves together read different banks
    const uint32_t rot = l & 15u;
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint4 v = q[static_cast<uint32_t>(i) ^ rot];
      sum += (v.x + v.y) + (v.z + v.w);
    }
    if (l == 0) sum -= bin0_less;
    uint32_t incl = wave_incl_scan(sum);
    const uint32_t total = readlane(incl, 63);
    uint32_t above = total - incl;  // entries in higher lanes' ranges
    const uint64_t hit = __ballot(above < kk && kk <= above + sum);
    const int L = hit ? __ffsll(static_cast<unsigned long long>(hit)) - 1 : 0;
    const uint32_t base = readlane(above, L);
    uint32_t h = hist[64 * L + l];
    if (L == 0 && l == 0) h -= bin0_less;
    incl = wave_incl_scan(h);
    above = base + readlane(incl, 63) - incl;
    const uint64_t hit2 = __ballot(above < kk && kk <= above + h);
    const int j = hit2 ? __ffsll(static_cast<unsigned long long>(hit2)) - 1 : 0;
    if (l == static_cast<uint32_t>(j)) {
      res[0] = 64 * L + j;
      res[1] = above;
      res[2] = h;
    }
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
    if (base >= end) {
#pragma unroll
      for (int j = 0; j < PT; ++j) key[j] = 0u;
      return;
    }
    if constexpr (V4) {
      issue(key, base);
      form(key, base);
    } else {
      const int32_t tid = static_cast<int32_t>(threadIdx.x);
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
  // V4, base < end: the loads of load(), bit patterns into key; form() then
  // waits for them and turns them into keys.  Between the two a wave may do
  // other work (a barrier included) while its loads are in flight.
  __device__ __forceinline__ void issue(Keys& key, int32_t base) const {
    static_assert(V4, "float4 layout");
    const int32_t tid = static_cast<int32_t>(threadIdx.x);
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
  }
  __device__ __forceinline__ void form(Keys& key, int32_t base) const {
    static_assert(V4, "float4 layout");
    const int32_t tid = static_cast<int32_t>(threadIdx.x);
    {
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        const int32_t g0 = base + 4 * v * T;  // first position of the group
        const int32_t q = g0 + 4 * tid;
        if (g0 + 4 * T <= end) {
#pragma unroll
          for (int c = 0; c < 4; ++c) key[4 * v + c] = order_key(key[4 * v + c]);
        } else if (g0 >= end) {
#pragma unroll
          for (int c = 0; c < 4; ++c) key[4 * v + c] = 0u;
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c) key[4 * v + c] = q + c < end ? order_key(key[4 * v + c]) : 0u;
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

// The threshold search of a row's round: by wave 0 alone for 1024-lane
// workgroups (measured faster there: one barrier instead of two, the other
// 15 waves idle meanwhile), by the whole block for 512 lanes.
template <int T>
__device__ __forceinline__ void find_threshold(const uint32_t* hist, uint32_t kk, uint32_t bin0_less,
                                               SelSmem& sm) {
  if constexpr (T >= 1024) {
    find_threshold_w0(hist, kk, bin0_less, sm.res);
  } else {
    find_threshold_bin<T>(hist, kk, bin0_less, sm.wsum, sm.res);
  }
}

template <int T>
__device__ __forceinline__ void hist_clear(uint32_t* hist) {
#pragma unroll
  for (int i = threadIdx.x; i < kHistBins / 4; i += T) {
    reinterpret_cast<uint4*>(hist)[i] = make_uint4(0, 0, 0, 0);
  }
}

// Radix rounds until the bucket holds at most CAP entries: 12-bit
// rounds on the key inside [lo, hi], then (one key left with too many ties)
// rounds on d = n - 1 - pos among the scores equal to it, so that the
// lowest positions win.  Padding slots have pos >= n: their d wraps far
// above any range.  Round r counts into hist[r & 1] and clears the other
// buffer.  Precondition: hist[round & 1] is zero and a barrier has passed.
// Each wave probes (with probe_key) whether its lanes pile into one hot bin
// and only then merges the atomics into it.  Without tie_rounds, a key left
// with too many ties is returned as is (tie = 1, bucket = its count) for the
// caller to resolve by position.  above_free: no key that for_each visits
// lies above in.hi (otherwise keys above the range go to the dummy bins by a
// range test in every round).  Returns the refined state.
template <int T, int CAP = kSmallCap, class ForEach>
__device__ __forceinline__ Sel refine(ForEach&& for_each, SelSmem& sm, const Sel in, uint32_t nm1,
                                      uint32_t n_pad, uint32_t probe_key, int& round,
                                      bool tie_rounds = true, bool above_free = true,
                                      uint32_t* sub = nullptr) {
  uint32_t lo = in.lo, hi = in.hi, kk = in.kk, bucket = in.bucket;
  uint32_t tie = 0, dlo = 0, dhi = nm1;
  const int first_round = round;
  bool sub_clear = false;  // the copies are zero (cleared before their first use)
  while (bucket > static_cast<uint32_t>(CAP) && lo != hi && round < kMaxRounds) {
    uint32_t* hist = sm.hist[round & 1];
    hist_clear<T>(sm.hist[(round + 1) & 1]);
    if (sub != nullptr && round > 0 && !sub_clear) {
#pragma unroll
      for (int c = 0; c < kSubCopies; ++c) hist_clear<T>(sub + c * kSubStride);
      sub_clear = true;
      __syncthreads();
    }
    const uint32_t rlo = lo, span = hi - lo;
    const int bl = span ? 32 - __clz(static_cast<int>(span)) : 0;
    const int s = bl > kHistBits ? bl - kHistBits : 0;
    const uint32_t pd = probe_key - rlo;
    const uint2 hot = wave_hot_bin(pd <= span, pd >> s);
    if (hot.y > kPeelShare) {
      hist_pass_hot(for_each, hist, rlo, span, s, hot.x);
    } else if (above_free && round == first_round && rlo != 0 && ((0u - rlo) >> s) >= kHistBins + 64) {
      // First round: nothing lies above hi, and a key under lo wraps to a
      // difference whose bin lies past every lane's dummy, so a min picks the
      // dummy without a range test (in-range bins are the same as below).
      const uint32_t dummy = kHistBins + __lane_id();
      for_each([&](uint32_t x, int32_t, int) {
        atomicAdd(&hist[min((x - rlo) >> s, dummy)], 1u);
      });
    } else if (sub != nullptr && round > 0) {
      // A later round, where a row's keys crowd into few bins: lane l counts
      // into copy l % kSubCopies of the histogram, so one wave's LDS atomics
      // meet a quarter as many lanes per address and bank; the copies are
      // merged into hist below.
      uint32_t* base = sub + (__lane_id() % kSubCopies) * kSubStride;
      uint32_t* dummy = hist + kHistBins + __lane_id();
      for_each([&](uint32_t x, int32_t, int) {
        const uint32_t d = x - rlo;
        atomicAdd(d <= span ? base + (d >> s) : dummy, 1u);
      });
    } else {
      const uint32_t dummy = kHistBins + __lane_id();
      for_each([&](uint32_t x, int32_t, int) {
        const uint32_t d = x - rlo;
        atomicAdd(&hist[d <= span ? d >> s : dummy], 1u);
      });
    }
    __syncthreads();
    if (sub != nullptr && round > 0) {
      // merge the copies into hist and return them to zero (each wave chose
      // its own path; copies a wave did not touch hold zeros)
      for (int i = threadIdx.x; i < kHistBins / 4; i += T) {
        uint4 a = reinterpret_cast<uint4*>(hist)[i];
#pragma unroll
        for (int c = 0; c < kSubCopies; ++c) {
          uint4* q = reinterpret_cast<uint4*>(sub + c * kSubStride) + i;
          const uint4 b = *q;
          *q = make_uint4(0u, 0u, 0u, 0u);
          a.x += b.x;
          a.y += b.y;
          a.z += b.z;
          a.w += b.w;
        }
        reinterpret_cast<uint4*>(hist)[i] = a;
      }
      __syncthreads();
    }
    find_threshold<T>(hist, kk, rlo == 0 ? n_pad : 0u, sm);
    kk -= sm.res[1];
    bucket = sm.res[2];
    lo = rlo + (sm.res[0] << s);
    const uint32_t width = (1u << s) - 1u;
    if (hi - lo > width) hi = lo + width;
    ++round;
  }
  if (bucket > static_cast<uint32_t>(CAP)) {
    tie = 1;
    const uint32_t tkey = lo;
    while (tie_rounds && bucket > static_cast<uint32_t>(CAP) && round < kMaxRounds) {
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
      find_threshold<T>(hist, kk, 0u, sm);
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

// Output value of selected position pos of a row: pos counts from the row's
// first candidate, row_start is that candidate's position (dense rows: the
// window start, 0 without windows; ragged rows: the row's offset in the
// packed buffer).  Paged: pt_lds is the row's page-table staged in LDS, used
// when use_lds, else pt_row is read.
template <int MODE>
__device__ __forceinline__ int32_t out_value(const Params& p, bool use_lds, const int32_t* pt_lds,
                                             const int32_t* pt_row, int32_t row_start, int32_t pos) {
  if constexpr (MODE == kPaged) {
    const int32_t a = row_start + pos;  // position in the row
    int32_t page, off;
    if (p.page_shift >= 0) {
      page = a >> p.page_shift;
      off = a & (p.page_size - 1);
    } else {
      page = a / p.page_size;
      off = a - page * p.page_size;
    }
    const int32_t id = use_lds ? ((lds_i32*)pt_lds)[page] : ((glb_i32*)pt_row)[page];
    return id * p.page_size + off;
  } else {
    return row_start + pos;
  }
}

// A bucket entry: key and position as one 64-bit word, (key << 32) |
// ~position, whose unsigned order is the order on (key desc, position asc).
// A zero word is no entry: it ranks below every entry.
__device__ __forceinline__ uint64_t bucket_entry(uint32_t key, int32_t pos) {
  return (static_cast<uint64_t>(key) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(pos));
}

// Ranks up to CAP bucket entries on (key desc, position asc) and emits
// the kk best at slots first + rank.  G = T / CAP lanes share an entry:
// each compares it with every G-th entry, then row permutes sum the G counts.
// cand holds the nc entries followed by zero words up to CAP, so no
// read is clamped and no comparison tests an index.
template <int T, int CAP = kSmallCap, class Emit>
__device__ __forceinline__ void rank_bucket(const uint64_t* cand, uint32_t nc, uint32_t kk,
                                            uint32_t first, Emit&& emit) {
  constexpr int G = T / CAP;
  static_assert(G == 2 || G == 4 || G == 8, "2, 4 or 8 lanes per bucket entry");
  constexpr int Q = CAP / G;  // entries compared by each lane
  constexpr int QB = 4;             // entries read per batch: small buckets read little
  static_assert(Q % QB == 0, "whole batches");
  const uint32_t i = threadIdx.x / G;
  const uint32_t part = threadIdx.x % G;
  // a wave whose entries all lie past the bucket has nothing to rank
  if ((threadIdx.x & ~63u) / G >= nc) return;
  const uint64_t vi = cand[i];
  uint32_t rank = 0;
#pragma unroll
  for (int q0 = 0; q0 < Q; q0 += QB) {
    if (static_cast<uint32_t>(G * q0) >= nc) break;
    uint64_t vj[QB];
#pragma unroll
    for (int q = 0; q < QB; ++q) vj[q] = cand[part + G * (q0 + q)];
#pragma unroll
    for (int q = 0; q < QB; ++q) rank += vj[q] > vi ? 1u : 0u;
  }
  rank += dpp_perm<0xB1>(rank);                         // quad_perm [1,0,3,2]: pairs
  if constexpr (G >= 4) rank += dpp_perm<0x4E>(rank);   // quad_perm [2,3,0,1]: quads
  if constexpr (G >= 8) rank += dpp_perm<0x141>(rank);  // row_half_mirror: eights
  if (i < nc && part == 0 && rank < kk) emit(first + rank, static_cast<int32_t>(~static_cast<uint32_t>(vi)));
}

// Row geometry shared by every kernel: the candidates of row b are the n
// scores from `row` on; row_start is the position of the first of them (see
// out_value).  Dense rows: n_b = their length clamped to [0, L]; with windows,
// the candidates start at the window start clamped to [0, n_b].
template <int MODE>
struct RowRef {
  int32_t n;
  int32_t row_start;
  const float* row;
  const int32_t* pt_row;
  int32_t* out;
  __device__ __forceinline__ RowRef(const Params& p, int b) {
    row_start = 0;
    if constexpr (MODE == kRagged) {
      row_start = p.row_starts[b];
      n = max(p.lens[b], 0);
      row = p.scores + row_start;
    } else {
      const int32_t nb = p.lens ? min(max(p.lens[b], 0), p.L) : p.L;
      row_start = p.win_starts ? min(max(p.win_starts[b], 0), nb) : 0;
      n = nb - row_start;
      row = p.scores + static_cast<int64_t>(b) * p.row_stride + row_start;
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

// First round of a resident float4 row (T = 1024) whose loads were issued
// and formed into keys only by the first WB = W / 2 waves.  Bounds from
// those waves' keys: their largest (hi), and a lower bound (lo) of the row's
// k-th largest from the jth-largest keys of their lanes (jth = ceil(k /
// lanes), at most 4), as in the whole-row bounds; 0 if too few lanes hold
// jth scores.  Keys of the other waves may lie above hi, so the 12-bit
// histogram of [lo, hi] keeps its last bin for every key from
// lo + (kHistBins - 1) << s up.  The other waves form their keys in this
// pass.  Returns the state after the round (a bucket of the last bin
// reaches up to the largest key); hist[0] has been used, hist[1] is zero.
template <int T, int VEC, class SpanT>
__device__ __forceinline__ Sel early_round(const SpanT& span, uint32_t (&key)[4 * VEC], SelSmem& sm,
                                           uint32_t* red, int32_t k, int32_t n) {
  constexpr int PT = 4 * VEC;
  constexpr int W = T / 64;
  constexpr int WB = W / 2;
  constexpr int LB = 64 * WB;  // lanes of the bounding waves
  const int tid = threadIdx.x;
  const int wid = tid >> 6;
  const int32_t jth = (k + LB - 1) / LB;  // 1 .. 4 for k <= ETS_MAX_K
  static_assert(ETS_MAX_K <= 4 * LB, "at most the 4th-largest key of a lane");
  uint32_t m1 = 0, mj = 0;
  if (wid < WB) {
    if (jth <= 2) {
      uint32_t m2 = 0;
#pragma unroll
      for (int j = 0; j < PT; ++j) {
        m2 = max(m2, min(m1, key[j]));
        m1 = max(m1, key[j]);
      }
      mj = jth == 1 ? m1 : m2;
    } else {
      uint32_t m2 = 0, m3 = 0, m4 = 0;
#pragma unroll
      for (int j = 0; j < PT; ++j) {
        const uint32_t x = key[j];
        m4 = max(m4, min(m3, x));
        m3 = max(m3, min(m2, x));
        m2 = max(m2, min(m1, x));
        m1 = max(m1, x);
      }
      mj = jth == 3 ? m3 : m4;
    }
    // lanes whose first jth slots (positions 4t .. 4t + jth - 1) hold scores
    const bool full = 4 * tid + jth - 1 < n;
    const uint32_t wmax = wave_reduce(m1, OpMax());
    const uint32_t wlb = wave_reduce(full ? mj : 0xFFFFFFFFu, OpMin());
    if (__lane_id() == 0) {
      red[wid] = wmax;
      red[16 + wid] = wlb;
    }
  }
  hist_clear<T>(sm.hist[1]);
  __syncthreads();
  uint32_t hi = 0, lb = 0xFFFFFFFFu;
#pragma unroll
  for (int w = 0; w < WB; ++w) {
    hi = max(hi, red[w]);
    lb = min(lb, red[16 + w]);
  }
  const int32_t nfull = n >= jth ? min(LB, (n - jth) / 4 + 1) : 0;
  uint32_t lo = nfull * jth >= k ? lb : 0u;
  auto shift_of = [](uint32_t span) {
    int sh = span ? 32 - __clz(static_cast<int>(span)) : 0;
    sh = sh > kHistBits ? sh - kHistBits : 0;
    if ((span >> sh) >= static_cast<uint32_t>(kHistBins - 1)) ++sh;  // [lo, hi] in bins below the last
    return sh;
  };
  int s = shift_of(hi - lo);
  bool formed = wid < WB;
  if (s + (31 - __clz(n)) > kEarlyMaxSpread) {
    // Too wide a range for the row (bins of 2^s keys, 2^(23 - s) to an
    // octave of floats: with n >= 2^(kEarlyMaxSpread - s) scores a bin near
    // the threshold may outgrow the bucket that is ranked directly; the
    // range then reaches down many octaves, across zero say): take the
    // whole-row bounds as well, the minimum over all lanes of their j2-th largest key, j2 =
    // ceil(k / T) <= 2 (every lane holds two: n >= 4 T), and the largest key.
    if (!formed) span.form(key, 0);
    formed = true;
    uint32_t a = 0, b2 = 0;
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      b2 = max(b2, min(a, key[j]));
      a = max(a, key[j]);
    }
    static_assert(ETS_MAX_K <= 2 * T, "two keys per lane bound the k-th largest");
    const uint32_t wmax = wave_reduce(a, OpMax());
    const uint32_t wmin = wave_reduce(k <= T ? a : b2, OpMin());
    if (__lane_id() == 0) {
      red[32 + wid] = wmax;
      red[48 + wid] = wmin;
    }
    __syncthreads();
    uint32_t lo2 = 0xFFFFFFFFu;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      hi = max(hi, red[32 + w]);
      lo2 = min(lo2, red[48 + w]);
    }
    lo = max(lo, lo2);
    s = shift_of(hi - lo);
  }
  const uint64_t top = static_cast<uint64_t>(lo) + (static_cast<uint64_t>(kHistBins - 1) << s);
  const uint32_t clampv = top > 0xFFFFFFFFull ? 0xFFFFFFFFu : static_cast<uint32_t>(top);
  // keys under lo wrap past every lane's dummy bin, or are tested
  const bool wrap = lo != 0 && ((0u - lo) >> s) >= static_cast<uint32_t>(kHistBins + 64);
  const uint32_t dummy = kHistBins + __lane_id();

  if (!formed) span.form(key, 0);
  uint32_t* hist = sm.hist[0];
  auto bin = [&](uint32_t x) {
    const uint32_t b = (min(x, clampv) - lo) >> s;
    return wrap ? min(b, dummy) : (x >= lo ? b : dummy);
  };
  const uint32_t pb = bin(key[0]);
  const uint2 hot = wave_hot_bin(pb < static_cast<uint32_t>(kHistBins), pb);
  if (hot.y > kPeelShare) {
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      const uint32_t b = bin(key[j]);
      const bool h = b == hot.x;
      cnt += h ? 1u : 0u;
      atomicAdd(&hist[h ? dummy : b], 1u);
    }
    cnt = wave_reduce(cnt, OpAdd());
    if (__lane_id() == 0 && cnt != 0) atomicAdd(&hist[hot.x], cnt);
  } else if (wrap) {
#pragma unroll
    for (int j = 0; j < PT; ++j) atomicAdd(&hist[min((min(key[j], clampv) - lo) >> s, dummy)], 1u);
  } else {
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      const uint32_t x = key[j];
      atomicAdd(&hist[x >= lo ? (min(x, clampv) - lo) >> s : dummy], 1u);
    }
  }
  __syncthreads();
  find_threshold<T>(hist, static_cast<uint32_t>(k), lo == 0 ? span.pad_slots() : 0u, sm);
  Sel out{};
  out.kk = static_cast<uint32_t>(k) - sm.res[1];
  out.bucket = sm.res[2];
  out.lo = lo + (sm.res[0] << s);
  out.hi = sm.res[0] == static_cast<uint32_t>(kHistBins - 1) ? 0xFFFFFFFFu : out.lo + ((1u << s) - 1u);
  out.dhi = static_cast<uint32_t>(n - 1);
  return out;
}

// NSUB histogram copies for later rounds (1024-lane rows; none for 512).
template <int NSUB>
struct alignas(16) RowSmem {
  SelSmem sel;
  uint32_t sub[NSUB > 0 ? NSUB : 1][NSUB > 0 ? kSubStride : 1];  // a later round's histogram copies
  int32_t pt[kPtCap];     // staged page-table row (paged map)
  uint64_t cand[kRankCap];  // threshold bucket (bucket_entry words, zero past the bucket)
  int32_t pos[ETS_MAX_K]; // selected positions by output slot
  uint32_t red[64];       // per-wave partials (bounds)
  uint32_t ccount;
};

// One exact top-k row on one workgroup.  STREAM = false: the row (n <= one
// tile) is loaded once and every pass runs on registers.  STREAM = true: any
// length; every pass streams the row tile by tile (L2 after the first).
template <int T, int VEC, int MODE, bool V4, bool STREAM>
__device__ __forceinline__ void row_topk(const Params& p, RowSmem<T >= 1024 ? kSubCopies : 0>& sm,
                                         const RowRef<MODE>& r) {
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
    // pages of positions [0, row_start + n): with a window, those before it too
    const int32_t last = r.row_start + n - 1;
    npages = p.page_shift >= 0 ? (last >> p.page_shift) + 1 : last / p.page_size + 1;
    pt_lds = npages <= kPtCap;
    if (pt_lds) {
#pragma unroll
      for (int i = 0; i < PTV; ++i) ptv[i] = (tid + i * T < npages) ? r.pt_row[tid + i * T] : 0;
    }
  }

  const SpanT span{r.row, 0, n};
  uint32_t key[PT];
  // A resident float4 row takes the bounds of its first round from the
  // first WB waves, whose loads the compute unit serves first, and the
  // other waves form their keys only in the histogram pass: the bounds and
  // part of that pass overlap the loads still in flight.
  constexpr bool kEarly = V4 && !STREAM && T == 1024 && VEC >= 2;
  constexpr int WB = W / 2;
  bool early = false;
  if constexpr (kEarly) {
    early = n >= kEarlyMinFill * SpanT::TILE / 4;
    if (early) {
      span.issue(key, 0);
      if (wid < WB) span.form(key, 0);
    } else {
      span.load(key, 0);
    }
  } else if constexpr (!STREAM) {
    span.load(key, 0);
  }
  auto for_each = [&](auto&& f) { span.template for_each<!STREAM>(key, f); };

  hist_clear<T>(sm.sel.hist[0]);
  if (tid == 0) sm.ccount = 0;
  for (int i = tid; i < kRankCap; i += T) sm.cand[i] = 0ull;
  if constexpr (MODE == kPaged) {
    if (pt_lds) {
#pragma unroll
      for (int i = 0; i < PTV; ++i)
        if (tid + i * T < npages) sm.pt[tid + i * T] = ptv[i];
    }
  }

  const uint32_t nm1 = static_cast<uint32_t>(n - 1);
  int round = 0;
  // a resident row in float4 layout resolves a key with too many ties by the
  // positions' prefix counts instead of radix rounds on positions
  constexpr bool kPrefixTies = V4 && !STREAM;
  Sel sel{};
  if constexpr (kEarly) {
    if (early) {
      sel = early_round<T, VEC>(span, key, sm.sel, sm.red, k, n);
      round = 1;
      sel = refine<T, kRankCap>(for_each, sm.sel, sel, nm1, span.pad_slots(), key[0], round, !kPrefixTies, false,
                      T >= 1024 ? &sm.sub[0][0] : nullptr);
    }
  }
  if (!early) {
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
  const int32_t nfull = jth > 2 ? 0 : (V4 ? (n >= jth ? min(T, (n - jth) / 4 + 1) : 0) : min(T, max(0, n - (jth - 1) * T)));
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
    static_assert(W % 4 == 0, "per-wave partials are read four at a time");
#pragma unroll
    for (int w = 0; w < W; w += 4) {
      const uint4 a = *reinterpret_cast<const uint4*>(&sm.red[w]);
      const uint4 c = *reinterpret_cast<const uint4*>(&sm.red[16 + w]);
      gmax = max(gmax, max(max(a.x, a.y), max(a.z, a.w)));
      gb = min(gb, min(min(c.x, c.y), min(c.z, c.w)));
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
  sel = refine<T, kRankCap>(for_each, sm.sel, sel0, nm1, span.pad_slots(), key[0], round, !kPrefixTies, true,
                  T >= 1024 ? &sm.sub[0][0] : nullptr);
  }
  const bool prefix_ties = kPrefixTies && sel.tie && sel.bucket > static_cast<uint32_t>(kRankCap);

  // ---- scatter: append the bucket to LDS, count the winners, place them by
  // one block scan (whose barrier also publishes the bucket) into the
  // position list.
  // number of winners placed by the scatter (the rest come from the bucket)
  const uint32_t first = prefix_ties ? static_cast<uint32_t>(k) : static_cast<uint32_t>(k) - sel.kk;
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
    if (slot < static_cast<uint32_t>(kRankCap)) sm.cand[slot] = bucket_entry(x, pos);
  };
  if constexpr (!STREAM) {
    // bit PT-1-j of wmask / cmask: slot j is a winner / in the bucket
    static_assert(PT <= 32, "slot masks are 32 bits");
    uint32_t wmask = 0, cmask = 0;
    if (prefix_ties) {
      // One key T with more than kRankCap copies: its sel.kk copies at the
      // lowest positions win.  Positions grow with (group v of four slots,
      // lane, slot c in the group).  Block totals per group name the group
      // v* that holds the kk-th copy; one block scan of that group's counts
      // over the lanes then tells each lane how many of its copies there
      // win.  Copies in lower groups all win.  Padding lies past every
      // position, hence after every copy.
      static_assert(PT == 4 * VEC && W <= 16, "float4 groups, at most 16 waves");
      constexpr int NW = (VEC + 1) / 2;
      const uint32_t tkey = sel.hi;
      uint32_t emask = 0;
      for_each([&](uint32_t x, int32_t, int) {
        wmask = shift_in_lt(wmask, tkey, x);
        emask = shift_in_eq(emask, x, tkey);
      });
      // group v's slot c sits at bit 3 - c of its nibble
      auto nib = [&](int v) { return (emask >> (PT - 4 - 4 * v)) & 0xFu; };
      if (tid < NW) sm.red[tid] = 0u;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        const uint32_t c0 = static_cast<uint32_t>(__popc(nib(2 * i)));
        const uint32_t c1 = 2 * i + 1 < VEC ? static_cast<uint32_t>(__popc(nib(2 * i + 1))) : 0u;
        // two 16-bit fields: a block holds at most 4 * T <= 4096 copies per group
        const uint32_t ws = wave_reduce(c0 | (c1 << 16), OpAdd());
        if (__lane_id() == 0 && ws != 0) atomicAdd(&sm.red[i], ws);
      }
      __syncthreads();
      uint32_t need = sel.kk, vstar = 0;
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        const uint32_t tot = (sm.red[v / 2] >> (16 * (v & 1))) & 0xFFFFu;
        if (vstar == static_cast<uint32_t>(v) && need > tot) {
          need -= tot;
          ++vstar;
        }
      }
      // vstar < VEC: the bucket holds kk or more copies
      const uint32_t shift = PT - 4 - 4 * vstar;
      const uint32_t e = (emask >> shift) & 0xFu;
      const uint32_t cnt = static_cast<uint32_t>(__popc(e));
      const uint32_t incl = wave_incl_scan(cnt);
      if (__lane_id() == 63) sm.sel.wsum[wid] = incl;
      __syncthreads();
      const uint32_t ex = incl - cnt + sum_other_waves<W, true>(sm.sel.wsum);
      const uint32_t r = need > ex ? min(need - ex, cnt) : 0u;  // this lane's winning copies in v*
      uint32_t top = e;  // its r highest set bits: drop the lowest cnt - r
#pragma unroll
      for (int q = 1; q <= 4; ++q)
        if (cnt - r >= static_cast<uint32_t>(q)) top &= top - 1u;
      const uint32_t lower = vstar == 0 ? 0u : ~0u << (PT - 4 * vstar);  // groups below v*
      wmask |= (emask & lower) | (top << shift);
      __syncthreads();  // sm.red and wsum are free again
    } else if (!sel.tie) {
      const uint32_t khi = sel.hi, klo = sel.lo, kspan = sel.hi - sel.lo;
      if (klo != 0) {
        // bucket = at least lo and not a winner
        for_each([&](uint32_t x, int32_t, int) {
          wmask = shift_in_lt(wmask, khi, x);
          cmask = shift_in_le(cmask, klo, x);
        });
        cmask &= ~wmask;
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
  {
    const uint32_t nc = min(sm.ccount, static_cast<uint32_t>(kRankCap));
    auto place = [&](uint32_t slot, int32_t pos) { sm.pos[slot] = pos; };
    if (nc <= static_cast<uint32_t>(kSmallCap)) {
      rank_bucket<T>(sm.cand, nc, sel.kk, first, place);
    } else {
      rank_bucket<T, kRankCap>(sm.cand, nc, sel.kk, first, place);
    }
  }
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
  __shared__ RowSmem<T >= 1024 ? kSubCopies : 0> sm;
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

// ---------------------------------------------------------------- row-group path
//
// When the batch alone cannot fill the device, each row is cut into G
// chunks, one workgroup each, and the G workgroups of a row run the
// method's rounds together inside one launch (the pages' row-split path,
// PR #37591 topk.hip excerpt, carries each row's histogram through a
// workspace between separate kernels; here the kernel boundaries are
// replaced by waits inside the kernel):
//
//  * bounds: every member stores its chunk's largest key and a lower bound
//    of the row's k-th largest (from its lanes' jth-largest keys) in its own
//    slot, one 64-bit store that also marks the slot written; the members
//    poll the row's G slots and take the largest key and the best bound;
//  * round 0: every member builds a 12-bit LDS histogram of its chunk over
//    [lower bound, largest key], merges 8 fine bins to one and adds the
//    512 coarse bins into the row's table, and the count of its scores
//    under the lower bound into one more word; one wave of every member
//    polls the table until it and that word hold all n scores of the row
//    (no barrier: the total reaches n only once every member's adds have
//    landed) and finds the same threshold bin.  A bucket
//    larger than the tie list (scores concentrated in a few bins) is
//    narrowed by further rounds of 12-bit digits of the key, then of the
//    position among equal keys;
//  * every member writes its winners to the output and appends its bucket
//    members to the row's tie list, both placed through one 64-bit cursor
//    whose top byte also counts the members that have taken it;
//  * the last member to take the cursor waits for each tie-list entry (an
//    entry is never 0 once written), ranks the list exactly (LDS radix
//    rounds, then direct comparison), emits the rest of the row and returns
//    the row's workspace to zero.
//
// Members are assigned by workgroup index, a row's G members on one XCD,
// when the whole grid fits the device's row-group slots at once; otherwise
// groups are formed in the order workgroups start (a ticket counter), or the
// batch is cut into several such index grids.  How workgroups reach the
// compute units (measured on MI355X): workgroup i goes to XCD i % 8, and each
// XCD deals its own workgroups, in order, to its 4 shader engines in a fixed
// rotation, waiting for a slot on the engine whose turn it is even while the
// other engines have free ones.  An index grid that fits the device is
// resident at once: no engine is dealt more than ceil(grid / 32) <= 8 of it,
// so no member ever waits for a workgroup that has not started.  Why a
// ticketed grid always finishes when G is at most one engine's row-group
// slots (its compute units times the workgroups one compute unit holds; the
// host derives that cap from the device): tickets are consecutive, so every
// group whose G tickets are all taken has all of its members started, waits
// only for them and finishes; only the group holding the newest ticket can be
// incomplete, with at most G - 1 started members waiting.  They cannot fill
// an engine, so on every XCD the engine whose turn it is holds a member of a
// complete group or a free slot, and that XCD goes on starting workgroups,
// which take the next tickets.  With G above one engine's slots the
// incomplete group can fill the engine whose turn it is on the only XCD still
// starting workgroups, its missing members queued behind it there: a wait
// then runs to its bound (seen at G = 32 and 64 on grids of thousands of
// workgroups).  Both arguments count on the device's row-group slots: other
// work only delays a member's start, but two row-group launches running at
// once on one device (on different streams) can each hold slots that the
// other's missing members need.  Every wait is bounded; on expiry the
// workspace's error word gets the bit of that wait (bounds exchange, coarse
// table, round barrier or tie list), the call's output is undefined, and the
// kernel still ends.

// Data crosses workgroups only through agent-scope relaxed atomics, with each
// wave's memory counter drained before a round barrier's arrival is counted
// (or, for the coarse table and the tie list, completion read from the data
// itself).  Why this is
// enough on gfx942/gfx950 (LLVM AMDGPU usage guide, "Memory Model GFX942",
// which gfx950 follows): an agent-scope atomic load, store or
// read-modify-write is issued with the sc1 bit, so it is performed at the
// device's point of coherence rather than in one XCD's L2 or a compute
// unit's L1, and two workgroups on different XCDs see one value per
// location.  What an agent-scope release adds on top of that is a write-back
// of the L2 (for ordinary stores) and the s_waitcnt vmcnt(0) that waits for
// the completion of every earlier memory access; the acquire side adds an L1
// and L2 invalidate (for ordinary loads).  Here every word that one
// workgroup writes and another reads (slots, tables, counters, cursor, tie
// list) is written and read by such atomics, so no ordinary access needs the
// write-back or the invalidate, and the completion wait is drain_vmem()
// before the arrival that publishes the data.  Two hand-offs need no such
// wait, because the reader sees completion in the data itself: the coarse
// table, whose total reaches n only once every add has landed, and the tie
// list, whose entries are never 0 once written.  The output rows are written
// with ordinary stores but never read inside the kernel.
//
// Workspace (u32 words): hdr[64], then per row rec[192] (counters, then one
// u64 slot per member) | hist[3][4096] | ties[kTieCap] (u64).  It must be
// zero before its first use; every call returns all of it to zero.

constexpr int kTieCap = 4096;      // tie-list entries per row
// Scores per member of a split row: n / G rounded up to a multiple of 4
// (float4 groups), but at least min_chunk (a multiple of 4; by default
// kMinChunk), so that a member's lanes hold at least 4096 scores and their
// two largest keys each give a lower bound of the row's k-th largest
// (k <= 2048 = 1024 lanes x 2).  A row shorter than G * min_chunk leaves its
// last members empty.  Measured on MI355X (raw rows, k = 2048, N(0,1),
// lengths U[32768, 262144], B = 4, G = 16): 16.7 us per call, against 23.2
// with chunks of n / G, where the shorter rows got no bound at all and their
// first round spanned the whole key range.
constexpr int32_t kMinChunk = 4096;
__host__ __device__ __forceinline__ int64_t member_chunk(int64_t n, int32_t G, int32_t min_chunk) {
  const int64_t c = ((n + G - 1) / G + 3) & ~static_cast<int64_t>(3);
  return c > min_chunk ? c : min_chunk;
}
// Round 0 exchanges 2^kCoarseBits bins per row.  Measured on MI355X (HIP
// graph of 300 calls): 512 bins against 256 cut the banded ragged rows of
// 65536 to 262144 scores (B = 4, k = 2048) from 14.97 to 14.10 us, and N(0,1)
// rows at B = 1, L = 262144 and B = 4, L = 65536 by about 1 us, with B = 16
// and 64 unchanged: the threshold's coarse bin then holds under 128 scores,
// so the last member ranks the tie list directly; 1024 bins cost 6 to 12 us
// more on the N(0,1) rows (more device atomics and a longer poll).
constexpr int kCoarseBits = 9;
constexpr int kCoarseBins = 1 << kCoarseBits;
constexpr int kFinePerCoarse = kHistBins / kCoarseBins;
constexpr int kGroupPtCap = 1024;  // chunk page-table entries staged in LDS
constexpr int kRecWords = 64 + 2 * 64;  // per-row record (a 256-byte line) and one u64 slot per member
constexpr int kHdrWords = 64;
constexpr uint32_t kSpinLimit = 1u << 20;

enum HdrField : int { kHdrTicket = 0, kHdrFinished = 16, kHdrError = 32 };
// Bits of the error word: which bounded wait ran out, or a stale ticket.
enum ErrBit : uint32_t { kErrBounds = 1u, kErrStale = 2u, kErrCoarse = 4u, kErrBarrier = 8u, kErrTies = 16u };
enum GroupRecField : int { kRecBarrier = 0, kRecCursor = 32 /* u64 */,
                          kRecBelow = 48, kRecSlots = 64 /* u64 per member */ };

__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class U>
__device__ __forceinline__ U add_dev(U* p, U v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void or_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Waits until every global access this wave issued has completed.
__device__ __forceinline__ void drain_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// A tie-list entry: the key in the high word, the complement of the position
// (never 0, as positions are below 2^31) in the low word, so that an entry
// still in flight reads as 0 in a list that every call returns to zero.
__device__ __forceinline__ uint64_t tie_word(uint32_t key, uint32_t pos) {
  return (static_cast<uint64_t>(key) << 32) | static_cast<uint32_t>(~pos);
}

// Arrives at a row's barrier and returns once `target` arrivals are counted.
// Every thread calls it; what each thread wrote before has completed by the
// time any member leaves.
__device__ __forceinline__ void group_sync(uint32_t* ctr, uint32_t target, uint32_t* err) {
  drain_vmem();
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t seen = add_dev(ctr, 1u) + 1u;
    uint32_t spins = 0;
    while (seen < target) {
      __builtin_amdgcn_s_sleep(1);
      seen = ld_dev(ctr);
      if (++spins > kSpinLimit) {
        or_dev(err, kErrBarrier);
        break;
      }
    }
  }
  __syncthreads();
}

// Per-row block: record | three histogram tables | tie list.  The layout of a
// row does not depend on the batch size, so calls of different shapes can
// share one workspace: the tie lists, the only words left non-zero, never
// overlap another call's counters or tables.
constexpr int64_t kRowWords = kRecWords + 3 * kHistBins + 2 * kTieCap;

struct GroupWs {
  uint32_t* hdr;
  __device__ explicit GroupWs(uint32_t* ws) : hdr(ws) {}
  __device__ uint32_t* rec(int b) const { return hdr + kHdrWords + b * kRowWords; }
  __device__ uint32_t* hist(int b) const { return rec(b) + kRecWords; }
  __device__ uint64_t* ties(int b) const {
    return reinterpret_cast<uint64_t*>(hist(b) + 3 * kHistBins);
  }
};

// Adds the LDS bins >= from that are not zero into dst (device atomics) and
// clears every LDS bin of the calling thread.
template <int T>
__device__ __forceinline__ void push_bins(uint32_t* lh, uint32_t from, uint32_t* dst) {
  constexpr int BPT = kHistBins / T;
#pragma unroll
  for (int i = 0; i < BPT; i += 4) {
    const uint32_t b0 = threadIdx.x * BPT + i;
    uint4* q = reinterpret_cast<uint4*>(lh + b0);
    const uint4 c = *q;
    *q = make_uint4(0u, 0u, 0u, 0u);
    if (c.x != 0 && b0 >= from) add_dev(dst + b0, c.x);
    if (c.y != 0 && b0 + 1 >= from) add_dev(dst + b0 + 1, c.y);
    if (c.z != 0 && b0 + 2 >= from) add_dev(dst + b0 + 2, c.z);
    if (c.w != 0 && b0 + 3 >= from) add_dev(dst + b0 + 3, c.w);
  }
}

// Reads the row histogram src and finds its threshold bin for kk (res).
template <int T>
__device__ __forceinline__ void read_bins(const uint32_t* src, uint32_t kk, SelSmem& ss) {
  constexpr int BPT = kHistBins / T;
  uint32_t h[BPT];
#pragma unroll
  for (int i = 0; i < BPT; i += 2) {
    const uint64_t v = ld_dev(reinterpret_cast<const uint64_t*>(src + threadIdx.x * BPT + i));
    h[i] = static_cast<uint32_t>(v);
    h[i + 1] = static_cast<uint32_t>(v >> 32);
  }
  find_threshold_regs<T>(h, kk, ss.wsum, ss.res);
}

template <int T>
__device__ __forceinline__ void clear_bins(uint32_t* buf, uint32_t count) {
  for (uint32_t i = threadIdx.x; i < count; i += T) st_dev(buf + i, 0u);
}

// Adds the LDS histogram, merged kFinePerCoarse bins at a time, into the
// coarse table dst (device atomics; zero bins are skipped) and clears it.
// Returns the count of the calling thread's four bins.
template <int T>
__device__ __forceinline__ uint32_t push_coarse(uint32_t* lh, uint32_t* dst) {
  constexpr int LPC = kFinePerCoarse / 4;  // lanes per coarse bin
  static_assert(kHistBins / T == 4 && (LPC == 1 || LPC == 2 || LPC == 4 || LPC == 16), "lanes per coarse bin");
  uint4* q = reinterpret_cast<uint4*>(lh) + threadIdx.x;
  const uint4 c = *q;
  *q = make_uint4(0u, 0u, 0u, 0u);
  const uint32_t own = (c.x + c.y) + (c.z + c.w);
  uint32_t v = own;
  if constexpr (LPC >= 2) v += dpp_perm<0xB1>(v);  // quad_perm [1,0,3,2]
  if constexpr (LPC >= 4) v += dpp_perm<0x4E>(v);  // quad_perm [2,3,0,1]
  if constexpr (LPC >= 16) {
    v += dpp_perm<0x141>(v);  // row_half_mirror
    v += dpp_perm<0x140>(v);  // row_mirror
  }
  if ((threadIdx.x % LPC) == 0 && v != 0) add_dev(dst + threadIdx.x / LPC, v);
  return own;
}

// One wave polls the row's coarse table src, and the count below of the
// row's scores under the round's range, until together they hold all n
// scores: each member adds its bins and its count under the range, every
// word only grows, so the total reaches n exactly when every member's adds
// have landed, and then every word is final.  Then finds the threshold bin
// for kk: (bin, entries above it, entries in it), the same in every lane.  A
// wait past kSpinLimit polls sets kErrCoarse in the error word and returns
// what it read.
__device__ __forceinline__ uint3 poll_coarse(const uint32_t* src, const uint32_t* below, uint32_t n,
                                             uint32_t kk, uint32_t* err) {
  constexpr int C = kCoarseBins / 64;  // coarse bins per lane
  static_assert(C * 64 == kCoarseBins && (C == 1 || C % 2 == 0), "coarse bins per lane");
  const uint32_t l = __lane_id();
  uint32_t h[C];
  uint32_t sum = 0;
  for (uint32_t spins = 0;; ++spins) {
    if constexpr (C >= 2) {
#pragma unroll
      for (int i = 0; i < C; i += 2) {
        const uint64_t a = ld_dev(reinterpret_cast<const uint64_t*>(src + C * l + i));
        h[i] = static_cast<uint32_t>(a);
        h[i + 1] = static_cast<uint32_t>(a >> 32);
      }
    } else {
      h[0] = ld_dev(src + l);
    }
    const uint32_t b = __builtin_amdgcn_readfirstlane(ld_dev(below));
    sum = 0;
#pragma unroll
    for (int i = 0; i < C; ++i) sum += h[i];
    const uint32_t total = wave_reduce(sum, OpAdd()) + b;
    if (total == n) break;
    if (spins > kSpinLimit) {
      if (l == 0) or_dev(err, kErrCoarse);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  const uint32_t incl = wave_incl_scan(sum);
  uint32_t above = readlane(incl, 63) - incl;  // entries in higher lanes' bins
  uint32_t t = 0, ta = 0, th = 0;
  bool hit = false;
#pragma unroll
  for (int i = C - 1; i >= 0; --i) {
    if (!hit && above < kk && kk <= above + h[i]) {
      hit = true;
      t = C * l + i;
      ta = above;
      th = h[i];
    }
    above += h[i];
  }
  const uint64_t m = __ballot(hit);
  const int src_lane = m ? __ffsll(static_cast<unsigned long long>(m)) - 1 : 0;
  return make_uint3(readlane(t, src_lane), readlane(ta, src_lane), readlane(th, src_lane));
}

// Shift that maps a range of span + 1 values onto at most kHistBins bins.
__device__ __forceinline__ int digit_shift(uint32_t span) {
  const int bl = span ? 32 - __clz(static_cast<int>(span)) : 0;
  return bl > kHistBits ? bl - kHistBits : 0;
}

// The selection state after a round over digit (x - lo) >> s (keys) or
// (n - 1 - pos - dlo) >> s (positions among equal keys) found bin res[0]
// with res[1] entries above it and res[2] in it.
__device__ __forceinline__ void narrow(Sel& sel, const uint32_t* res, int s) {
  sel.kk -= res[1];
  sel.bucket = res[2];
  const uint32_t width = (1u << s) - 1u;
  if (!sel.tie) {
    sel.lo += res[0] << s;
    if (sel.hi - sel.lo > width) sel.hi = sel.lo + width;
  } else {
    sel.dlo += res[0] << s;
    if (sel.dhi - sel.dlo > width) sel.dhi = sel.dlo + width;
  }
}

struct alignas(16) GroupSmem {
  SelSmem sel;              // histograms (hist[0] is zero between rounds) and scan scratch
  int32_t pt[kGroupPtCap];  // the chunk's page-table entries (paged map)
  uint64_t cand[kSmallCap];  // final bucket of the tie list (bucket_entry words, zero past it)
  union {
    int32_t pos[ETS_MAX_K];  // this workgroup's winners, in slot order
    uint2 ties[kTieCap];     // the last workgroup: the row's tie list
  } u;
  uint32_t wsum2[16];
  uint32_t ticket, last, wcount, ccount;
  uint32_t base[3];
};

// One chunk [span.start, span.end) of row b as member g of its row's group.
// RES: the chunk fits one tile and stays in registers; otherwise every pass
// streams it.
template <int T, int VEC, int MODE, bool V4, bool RES>
__device__ __forceinline__ void group_row(const Params& p, GroupSmem& sm, const GroupWs& w,
                                          const RowRef<MODE>& r, int b, int g, int G,
                                          const Span<T, VEC, V4>& span) {
  constexpr int PT = Span<T, VEC, V4>::PT;
  constexpr int W = T / 64;
  const int tid = threadIdx.x;
  const int wid = tid >> 6;
  const int32_t k = p.k;
  const int32_t n = r.n;
  const uint32_t nm1 = static_cast<uint32_t>(n - 1);
  uint32_t* rec = w.rec(b);
  uint64_t* slots = reinterpret_cast<uint64_t*>(rec + kRecSlots);
  uint32_t* ghist = w.hist(b);
  uint64_t* gties = w.ties(b);
  uint32_t* err = w.hdr + kHdrError;
  uint32_t* lh = sm.sel.hist[0];  // cleared below, then zero again after every push

  uint32_t key[PT];
  if constexpr (RES) span.load(key, span.start);
  auto for_each = [&](auto&& f) { span.template for_each<RES>(key, f); };
  // the chunk's page ids, fetched after the scores and kept in registers
  // until the winners are emitted, so that no wait on them delays the rounds
  constexpr int PTV = (MODE == kPaged) ? (kGroupPtCap + T - 1) / T : 1;
  int32_t ptv[PTV];
  int32_t p0 = 0, np = 0;
  bool pt_lds = false;
  if constexpr (MODE == kPaged) {
    if (p.page_shift >= 0 && span.end > span.start) {
      p0 = (r.row_start + span.start) >> p.page_shift;
      np = ((r.row_start + span.end - 1) >> p.page_shift) - p0 + 1;
      pt_lds = np <= kGroupPtCap;
      if (pt_lds) {
#pragma unroll
        for (int i = 0; i < PTV; ++i) ptv[i] = (tid + i * T < np) ? r.pt_row[p0 + tid + i * T] : 0;
      }
    }
  }
  hist_clear<T>(lh);
  __syncthreads();
  const uint32_t pad = span.pad_slots();
  const int32_t nc = span.end - span.start;

  // ---- bounds of the row, in one exchange: its largest key, and a lower
  // bound of its k-th largest.  A chunk whose lanes' jth-largest keys are at
  // least k distinct scores bounds the row's k-th largest by their minimum
  // (jth = ceil(k / lanes holding scores) <= 2); other chunks offer 0.
  {
    uint32_t m1 = 0, m2 = 0;
    for_each([&](uint32_t x, int32_t, int) {
      m2 = max(m2, min(m1, x));
      m1 = max(m1, x);
    });
    const int32_t holders = V4 ? min(T, (nc + 3) / 4) : min(T, nc);
    const int32_t jth = holders > 0 ? (k + holders - 1) / holders : 3;
    const int32_t jpos = V4 ? 4 * tid + jth - 1 : (jth - 1) * T + tid;
    const bool full = jth <= 2 && span.start + jpos < span.end;
    // lanes whose first jth slots hold scores: float4 lane t holds positions
    // 4t .. 4t + 3 of the chunk, so 4t + jth - 1 < nc; none when nc < jth
    const int32_t nfull = jth > 2 ? 0 : (V4 ? (nc >= jth ? min(T, (nc - jth) / 4 + 1) : 0) : min(T, max(0, nc - (jth - 1) * T)));
    const uint32_t vmax = wave_reduce(m1, OpMax());
    const uint32_t vlb = wave_reduce(full ? (jth == 1 ? m1 : m2) : 0xFFFFFFFFu, OpMin());
    if (__lane_id() == 0) {
      sm.sel.wsum[wid] = vmax;
      sm.wsum2[wid] = vlb;
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t cmax = 0, clb = 0xFFFFFFFFu;
      for (int w = 0; w < W; ++w) {
        cmax = max(cmax, sm.sel.wsum[w]);
        clb = min(clb, sm.wsum2[w]);
      }
      // one store carries the member's bounds and marks them written:
      // the high word is the largest key plus one (saturated; 1 for an
      // empty chunk), never 0
      const uint32_t hi_enc = nc > 0 ? (cmax == 0xFFFFFFFFu ? cmax : cmax + 1u) : 1u;
      const uint32_t lbv = nfull * jth >= k ? clb : 0u;
      st_dev(slots + g, (static_cast<uint64_t>(hi_enc) << 32) | lbv);
    }
  }
  // every member's slot, read by the lanes of wave 0: the row's largest key
  // and the best of the offered lower bounds
  if (tid < 64) {
    uint64_t v = 0;
    if (tid < G) {
      v = ld_dev(slots + tid);
      uint32_t spins = 0;
      while (v == 0) {
        __builtin_amdgcn_s_sleep(1);
        v = ld_dev(slots + tid);
        if (++spins > kSpinLimit) {
          or_dev(err, kErrBounds);
          break;
        }
      }
    }
    const uint32_t he = static_cast<uint32_t>(v >> 32);
    const uint32_t hi = wave_reduce(he == 0xFFFFFFFFu ? he : (he ? he - 1u : 0u), OpMax());
    const uint32_t lb = wave_reduce(static_cast<uint32_t>(v), OpMax());
    if (tid == 0) {
      sm.base[0] = hi;
      sm.base[1] = lb;
    }
  }
  __syncthreads();
  uint32_t nbar = 0;  // group barriers passed
  Sel sel{};
  sel.lo = sm.base[1];
  sel.hi = sm.base[0];
  sel.kk = static_cast<uint32_t>(k);
  sel.dlo = 0u;
  sel.dhi = nm1;

  // ---- round 0: a 12-bit histogram of [lo, hi]
  int s0;
  {
    const uint32_t lo = sel.lo, span_k = sel.hi - sel.lo;
    s0 = digit_shift(span_k);
    const int s = s0;
    const uint32_t pd = (RES ? key[0] : 0u) - lo;
    const uint2 hot = wave_hot_bin(pd <= span_k, pd >> s);
    const uint32_t dummy = kHistBins + __lane_id();
    if (hot.y > kPeelShare) {
      hist_pass_hot(for_each, lh, lo, span_k, s, hot.x);
    } else if (lo != 0 && ((0u - lo) >> s) >= kHistBins + 64) {
      // nothing lies above hi, and a key under lo wraps past every dummy
      for_each([&](uint32_t x, int32_t, int) { atomicAdd(&lh[min((x - lo) >> s, dummy)], 1u); });
    } else {
      for_each([&](uint32_t x, int32_t, int) {
        const uint32_t d = x - lo;
        atomicAdd(&lh[d <= span_k ? d >> s : dummy], 1u);
      });
    }
    __syncthreads();
    if (lo == 0 && tid == 0) lh[0] -= pad;  // padding slots hold key 0
    __syncthreads();
  }
  // the row's histogram, 8 bins to one: few device atomics per member, and a
  // coarse threshold bucket that the tie list absorbs; with it the count of
  // the chunk's scores under lo, so that the table tells when it is whole
  {
    const uint32_t win = wave_reduce(push_coarse<T>(lh, ghist), OpAdd());
    if (__lane_id() == 0) sm.wsum2[wid] = win;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t in_range = 0;
    for (int w = 0; w < W; ++w) in_range += sm.wsum2[w];
    const uint32_t under = static_cast<uint32_t>(nc) - in_range;
    if (under != 0) add_dev(rec + kRecBelow, under);
  }
  if (tid < 64) {
    const uint3 c = poll_coarse(ghist, rec + kRecBelow, static_cast<uint32_t>(n), sel.kk, err);
    if (tid == 0) {
      sm.sel.res[0] = c.x;
      sm.sel.res[1] = c.y;
      sm.sel.res[2] = c.z;
    }
  }
  __syncthreads();
  {
    const uint32_t res[3] = {sm.sel.res[0], sm.sel.res[1], sm.sel.res[2]};
    narrow(sel, res, s0 + (kHistBits - kCoarseBits));
  }

  // ---- further rounds while the bucket exceeds the tie list
  int round = 1;
  while (sel.bucket > static_cast<uint32_t>(kTieCap) && round < kMaxRounds) {
    uint32_t* buf = ghist + (round % 3) * kHistBins;
    if (!sel.tie && sel.lo == sel.hi) sel.tie = 1;
    int s;
    if (!sel.tie) {
      const uint32_t lo = sel.lo, span_k = sel.hi - sel.lo;
      s = digit_shift(span_k);
      const uint32_t pd = (RES ? key[0] : 0u) - lo;
      const uint2 hot = wave_hot_bin(pd <= span_k, pd >> s);
      if (hot.y > kPeelShare) {
        hist_pass_hot(for_each, lh, lo, span_k, s, hot.x);
      } else {
        const uint32_t dummy = kHistBins + __lane_id();
        for_each([&](uint32_t x, int32_t, int) {
          const uint32_t d = x - lo;
          atomicAdd(&lh[d <= span_k ? d >> s : dummy], 1u);
        });
      }
      __syncthreads();
      if (lo == 0 && tid == 0) lh[0] -= pad;
    } else {
      const uint32_t tkey = sel.hi, dlo = sel.dlo, span_d = sel.dhi - sel.dlo;
      s = digit_shift(span_d);
      const int32_t end = span.end;
      for_each([&](uint32_t x, int32_t pos, int) {
        const uint32_t d = nm1 - static_cast<uint32_t>(pos) - dlo;
        if (x == tkey && pos < end && d <= span_d) atomicAdd(&lh[d >> s], 1u);
      });
    }
    __syncthreads();
    push_bins<T>(lh, 0u, buf);
    group_sync(rec + kRecBarrier, static_cast<uint32_t>(G) * ++nbar, err);
    if (g == 0) {
      // the previous round's table is read by every member by now and is next
      // used two rounds on, after this member's next arrival
      const int prev = round - 1;
      clear_bins<T>(ghist + (prev % 3) * kHistBins, prev == 0 ? kCoarseBins : kHistBins);
    }
    read_bins<T>(buf, sel.kk, sm.sel);
    narrow(sel, sm.sel.res, s);
    ++round;
  }

  // ---- scatter: winners to the output, bucket members to the tie list
  if constexpr (MODE == kPaged) {
    if (pt_lds) {
#pragma unroll
      for (int i = 0; i < PTV; ++i)
        if (tid + i * T < np) sm.pt[tid + i * T] = ptv[i];
    }
  }
  const uint32_t first = static_cast<uint32_t>(k) - sel.kk;  // winners of the whole row
  const int32_t cend = span.end;
  uint32_t nw = 0, nb = 0;
  uint32_t wmask = 0, cmask = 0;  // RES: bit PT-1-j marks slot j
  if constexpr (RES) {
    static_assert(PT <= 32, "slot masks are 32 bits");
    if (!sel.tie && sel.lo != 0) {
      // padding (key 0) lies below lo: the plain range tests hold
      const uint32_t khi = sel.hi, klo = sel.lo;
      // bucket = at least lo and not a winner
      for_each([&](uint32_t x, int32_t, int) {
        wmask = shift_in_lt(wmask, khi, x);
        cmask = shift_in_le(cmask, klo, x);
      });
      cmask &= ~wmask;
    } else {
      for_each([&](uint32_t x, int32_t pos, int) {
        wmask = wmask + wmask + (sel_winner(sel, nm1, cend, x, pos) ? 1u : 0u);
        cmask = cmask + cmask + (sel_bucket(sel, nm1, cend, x, pos) ? 1u : 0u);
      });
    }
    nw = static_cast<uint32_t>(__popc(wmask));
    nb = static_cast<uint32_t>(__popc(cmask));
  } else {
    for_each([&](uint32_t x, int32_t pos, int) {
      nw += sel_winner(sel, nm1, cend, x, pos) ? 1u : 0u;
      nb += sel_bucket(sel, nm1, cend, x, pos) ? 1u : 0u;
    });
  }
  const uint32_t iw = wave_incl_scan(nw);
  const uint32_t ib = wave_incl_scan(nb);
  if (__lane_id() == 63) {
    sm.sel.wsum[wid] = iw;
    sm.wsum2[wid] = ib;
  }
  __syncthreads();
  uint32_t ow = iw - nw + sum_other_waves<W, true>(sm.sel.wsum);
  uint32_t ob = ib - nb + sum_other_waves<W, true>(sm.wsum2);
  if (tid == T - 1) {
    // one atomic places this member's winners (bits 32..55: at most k of a
    // row) and bucket members (bits 0..31), and counts its arrival (bits
    // 56..63): the member that takes it last resolves the tie list
    static_assert(ETS_MAX_K < (1 << 24), "a row's winners fit 24 bits");
    static_assert((kRecWords - kRecSlots) / 2 < 256, "a row's member slots fit 8 bits");
    const uint64_t add = (1ull << 56) | (static_cast<uint64_t>(ow + nw) << 32) | (ob + nb);
    const uint64_t old = add_dev(reinterpret_cast<uint64_t*>(rec + kRecCursor), add);
    sm.base[0] = static_cast<uint32_t>(old >> 32) & 0xFFFFFFu;
    sm.base[1] = static_cast<uint32_t>(old);
    sm.base[2] = static_cast<uint32_t>(old) + ob + nb;  // the row's bucket total, if last
    sm.last = static_cast<uint32_t>(old >> 56) == static_cast<uint32_t>(G - 1) ? 1u : 0u;
    sm.wcount = ow + nw;
  }
  // the winners' chunk-local slots need no cursor: placed while it returns
  if constexpr (RES) {
    while (wmask != 0) {
      const int j = PT - __ffs(static_cast<int>(wmask));
      wmask &= wmask - 1u;
      if (ow < static_cast<uint32_t>(ETS_MAX_K)) sm.u.pos[ow] = span.start + tile_pos<T, V4>(j);
      ++ow;
    }
  } else {
    for_each([&](uint32_t x, int32_t pos, int) {
      if (sel_winner(sel, nm1, cend, x, pos)) {
        if (ow < static_cast<uint32_t>(ETS_MAX_K)) sm.u.pos[ow] = pos;
        ++ow;
      }
    });
  }
  __syncthreads();
  const uint32_t wbase = sm.base[0];
  const uint32_t wtot = sm.wcount;
  ob += sm.base[1];
  if constexpr (RES) {
    while (cmask != 0) {
      const int j = PT - __ffs(static_cast<int>(cmask));
      cmask &= cmask - 1u;
      const uint32_t pos = static_cast<uint32_t>(span.start + tile_pos<T, V4>(j));
      if (ob < static_cast<uint32_t>(kTieCap))
        st_dev(gties + ob, tie_word(select_slot<PT>(key, j), pos));
      ++ob;
    }
  } else {
    for_each([&](uint32_t x, int32_t pos, int) {
      if (sel_bucket(sel, nm1, cend, x, pos)) {
        if (ob < static_cast<uint32_t>(kTieCap))
          st_dev(gties + ob, tie_word(x, static_cast<uint32_t>(pos)));
        ++ob;
      }
    });
  }
  // winners through the output map, contiguous stores
  auto map_any = [&](int32_t pos) {
    return out_value<MODE>(p, false, nullptr, r.pt_row, r.row_start, pos);
  };
  if (MODE == kPaged && pt_lds) {
    const int32_t ps = p.page_size, sh = p.page_shift;
    for (uint32_t i = tid; i < wtot; i += T) {
      const uint32_t slot = wbase + i;
      if (slot < first && i < static_cast<uint32_t>(ETS_MAX_K)) {
        const int32_t pos = r.row_start + sm.u.pos[i];  // position in the row
        r.out[slot] = ((lds_i32*)sm.pt)[(pos >> sh) - p0] * ps + (pos & (ps - 1));
      }
    }
  } else {
    for (uint32_t i = tid; i < wtot; i += T) {
      const uint32_t slot = wbase + i;
      if (slot < first && i < static_cast<uint32_t>(ETS_MAX_K)) r.out[slot] = map_any(sm.u.pos[i]);
    }
  }

  // ---- the group's last workgroup (the last to take the cursor) resolves
  // the tie list.  No wave waits for its stores: the output is not read
  // here, and the last workgroup waits for each tie-list entry itself.  The
  // barrier: every wave is done with this workgroup's winners in LDS.
  __syncthreads();
  if (!sm.last) return;
  const uint32_t m = min(sm.base[2], static_cast<uint32_t>(kTieCap));
  // every entry below m was stored, or is being stored, by a member that has
  // taken the cursor; one still in flight reads as 0.  A wait past
  // kSpinLimit polls sets kErrTies and takes the entry as padding (key 0 at
  // position n), which selects nothing.
  for (uint32_t i = tid; i < m; i += T) {
    uint64_t v = ld_dev(gties + i);
    uint32_t spins = 0;
    while (static_cast<uint32_t>(v) == 0u && spins <= kSpinLimit) {
      __builtin_amdgcn_s_sleep(1);
      v = ld_dev(gties + i);
      ++spins;
    }
    if (static_cast<uint32_t>(v) == 0u) {
      or_dev(err, kErrTies);
      sm.u.ties[i] = make_uint2(0u, static_cast<uint32_t>(n));
    } else {
      sm.u.ties[i] = make_uint2(static_cast<uint32_t>(v >> 32), ~static_cast<uint32_t>(v));
    }
  }
  if (tid == 0) {
    sm.wcount = 0;
    sm.ccount = 0;
  }
  if (tid < kSmallCap) sm.cand[tid] = 0ull;
  __syncthreads();
  // ---- return the row's workspace to zero before the tie list is resolved,
  // so that the stores land meanwhile: every member has taken the cursor,
  // after its last read of the slots, the tables and the record, and every
  // tie-list entry has landed (read above).  The last round's table (round
  // 0: its coarse bins; earlier rounds were cleared on the way) and the
  // record.
  {
    const int lastr = round - 1;
    clear_bins<T>(ghist + (lastr % 3) * kHistBins, lastr == 0 ? kCoarseBins : kHistBins);
    for (uint32_t i = tid; i < m; i += T) st_dev(gties + i, 0ull);  // entries this thread read
    if (tid < G) st_dev(slots + tid, 0ull);
    if (tid == 0) {
      st_dev(rec + kRecBarrier, 0u);
      st_dev(rec + kRecBelow, 0u);
      st_dev(reinterpret_cast<uint64_t*>(rec + kRecCursor), 0ull);
    }
  }
  const int trips = static_cast<int>((m + T - 1) / T);
  const uint32_t tpad = static_cast<uint32_t>(trips) * T - m;
  // every lane visits the same number of slots (the radix rounds vote per wave);
  // slots past the list read as key 0 at position n
  auto for_ties = [&](auto&& f) {
    for (int j = 0; j < trips; ++j) {
      const uint32_t i = static_cast<uint32_t>(j * T + tid);
      const bool v = i < m;
      const uint2 e = sm.u.ties[v ? i : 0u];
      f(v ? e.x : 0u, v ? static_cast<int32_t>(e.y) : n, j);
    }
  };
  int lround = 0;
  const Sel fin = refine<T>(for_ties, sm.sel, sel, nm1, tpad, sm.u.ties[min(static_cast<uint32_t>(tid), m > 0 ? m - 1 : 0u)].x,
                            lround);
  const uint32_t first2 = first + (sel.kk - fin.kk);
  for_ties([&](uint32_t x, int32_t pos, int) {
    if (pos >= n) return;
    if (sel_winner(fin, nm1, n, x, pos)) {
      const uint32_t slot = first + atomicAdd(&sm.wcount, 1u);
      if (slot < first2) r.out[slot] = map_any(pos);
    } else if (sel_bucket(fin, nm1, n, x, pos)) {
      const uint32_t c = atomicAdd(&sm.ccount, 1u);
      if (c < static_cast<uint32_t>(kSmallCap)) sm.cand[c] = bucket_entry(x, pos);
    }
  });
  __syncthreads();
  rank_bucket<T>(sm.cand, min(sm.ccount, static_cast<uint32_t>(kSmallCap)), fin.kk, first2,
                 [&](uint32_t slot, int32_t pos) { r.out[slot] = map_any(pos); });

}

// G workgroups per row.  TICKET: B * G workgroups take rows in the order
// they start (a device counter), so that a group only waits for members that
// have started or start next; progress needs G within one shader engine's
// row-group slots (checked by the host).  Otherwise members are assigned by
// workgroup index over rows [b0, B): the dispatcher deals workgroup i to XCD
// i % nx, and the grid (nx * G * ceil((B - b0) / nx) workgroups, the padding
// idle) gives each row the G workgroups of one XCD, so that its exchanges
// wait only for that XCD's starts (XCDs start a launch up to 2 us apart; on
// MI355X, C5 13.4 us against 14.1 with rows spread over every XCD).  The
// placement only affects speed.  The host launches such a grid only when it
// fits the device's row-group slots at once, where waiting members can never
// keep the rest of the grid from starting, wherever they run (work of other
// streams that holds compute units only delays them, until it ends).
template <int T, int VEC, int MODE, bool V4, bool TICKET>
__global__ __launch_bounds__(T) void group_topk_kernel(Params p, uint32_t* ws, int32_t B, int32_t G,
                                                       int32_t nx, int32_t b0) {
  __shared__ GroupSmem sm;
  const GroupWs w(ws);
  int b, g;
  if constexpr (TICKET) {
    if (threadIdx.x == 0) sm.ticket = add_dev(w.hdr + kHdrTicket, 1u);
    __syncthreads();
    b = static_cast<int>(sm.ticket / static_cast<uint32_t>(G));
    g = static_cast<int>(sm.ticket % static_cast<uint32_t>(G));
  } else {
    // workgroup i starts on XCD i % nx: row b's members are the workgroups
    // of XCD b % nx, so that a row's exchanges wait for one XCD's starts only
    const uint32_t x = blockIdx.x % static_cast<uint32_t>(nx), s = blockIdx.x / static_cast<uint32_t>(nx);
    b = b0 + static_cast<int>(x + static_cast<uint32_t>(nx) * (s / static_cast<uint32_t>(G)));
    g = static_cast<int>(s % static_cast<uint32_t>(G));
    if (b >= B) return;  // the grid's padding
  }
  if (b >= B) {
    // only a workspace that was not zero (a stale ticket) gets here: this
    // workgroup's chunk goes unselected, so the call's output is undefined
    if (threadIdx.x == 0) or_dev(w.hdr + kHdrError, kErrStale);
  } else {
    const RowRef<MODE> r(p, b);
    if (r.n <= p.k) {
      if (g == 0) emit_whole_row<T, MODE>(p, r);
    } else {
      using SpanT = Span<T, VEC, V4>;
      const int64_t chunk = member_chunk(r.n, G, p.min_chunk);
      const int32_t start = static_cast<int32_t>(min(static_cast<int64_t>(g) * chunk, static_cast<int64_t>(r.n)));
      const int32_t end = (g == G - 1) ? r.n : static_cast<int32_t>(min(start + chunk, static_cast<int64_t>(r.n)));
      const SpanT span{r.row, start, end};
      if (end - start <= SpanT::TILE) {
        group_row<T, VEC, MODE, V4, true>(p, sm, w, r, b, g, G, span);
      } else {
        group_row<T, VEC, MODE, V4, false>(p, sm, w, r, b, g, G, span);
      }
    }
  }
  // the last workgroup to finish re-arms the ticket counter for the next call
  if constexpr (TICKET) {
    drain_vmem();
    __syncthreads();
    if (threadIdx.x == 0 && add_dev(w.hdr + kHdrFinished, 1u) == gridDim.x - 1) {
      st_dev(w.hdr + kHdrTicket, 0u);
      st_dev(w.hdr + kHdrFinished, 0u);
    }
  }
}

// Zero-fills a workspace (words of 4 bytes).
__global__ __launch_bounds__(256) void workspace_clear(uint32_t* ws, int64_t words) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < words; i += 256ll * gridDim.x) ws[i] = 0u;
}

// Copies a workspace's error word to flag[0] and clears it (ws may be null:
// flag[0] = 0).  One lane; ordered after earlier work on the same stream.
__global__ __launch_bounds__(64) void workspace_error_take(uint32_t* ws, int32_t* flag) {
  if (threadIdx.x != 0) return;
  uint32_t e = 0;
  if (ws != nullptr) {
    e = ld_dev(ws + kHdrError);
    st_dev(ws + kHdrError, 0u);
  }
  flag[0] = static_cast<int32_t>(e);
}

// ---------------------------------------------------------------- measurement floors

// The read alone: the grid, lane layout and loads of a selection launch.
// Workgroup blockIdx.x takes chunk g of row b (G = 1: the whole row), forms
// the keys and writes the chunk's largest key to sink[blockIdx.x]; nothing
// else.
template <int T, int VEC, int MODE, bool V4>
__global__ __launch_bounds__(T) void floor_read_kernel(Params p, uint32_t* sink, int32_t G) {
  using SpanT = Span<T, VEC, V4>;
  __shared__ uint32_t red[T / 64];
  const int b = static_cast<int>(blockIdx.x / static_cast<uint32_t>(G));
  const int g = static_cast<int>(blockIdx.x % static_cast<uint32_t>(G));
  const RowRef<MODE> r(p, b);
  const int64_t chunk = member_chunk(r.n, G, p.min_chunk);
  const int32_t start = static_cast<int32_t>(min(static_cast<int64_t>(g) * chunk, static_cast<int64_t>(r.n)));
  const int32_t end = (g == G - 1) ? r.n : static_cast<int32_t>(min(start + chunk, static_cast<int64_t>(r.n)));
  const SpanT span{r.row, start, end};
  uint32_t key[SpanT::PT];
  uint32_t m = 0;
  span.template for_each<false>(key, [&](uint32_t x, int32_t, int) { m = max(m, x); });
  m = wave_reduce(m, OpMax());
  if (__lane_id() == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 1; w < T / 64; ++w) m = max(m, red[w]);
    sink[blockIdx.x] = m;
  }
}

// The launch alone: a selection launch's grid and workgroup size, no work.
template <int T>
__global__ __launch_bounds__(T) void floor_launch_kernel() {}

// Row-group workspace for callers that cannot allocate (ets_topk_paged_noalloc):
// static device storage of kScratchBytes, one copy per device, held until
// the process ends.  Host code never uses this name as an address: it takes
// the device address once per device with hipGetSymbolAddress.
constexpr size_t kScratchBytes = ETS_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte lines");
static __device__ __align__(256) uint32_t scratch[kScratchBytes / 4];

// Copies the error word of workspace ws (words) to flag[0]; if it is set,
// zero-fills the whole workspace so that the next call starts clean.
__global__ __launch_bounds__(1024) void scratch_error_take(uint32_t* ws, int64_t words, int32_t* flag) {
  __shared__ uint32_t e;
  if (threadIdx.x == 0) {
    e = ld_dev(ws + kHdrError);
    flag[0] = static_cast<int32_t>(e);
  }
  __syncthreads();
  if (e == 0) return;
  for (int64_t i = threadIdx.x; i < words; i += 1024) st_dev(ws + i, 0u);
}

}  // namespace ets

// ==================================================================== host side

namespace {

struct DeviceInfo {
  bool queried = false;
  bool supported = false;
  int cu_count = 0;
  int xcd_count = 0;   // XCDs (dies with their own L2 and workgroup dispatcher)
  int group_occ = 0;   // row-group workgroups one compute unit holds at once
  int group_cap = 0;   // largest row group whose members fit the slots of one XCD
  int ticket_cap = 0;  // largest row group a ticketed grid takes: one shader engine's slots
};

constexpr int kMaxDevices = 64;
std::mutex g_dev_mutex;
DeviceInfo g_dev[kMaxDevices];

int group_kernel_occupancy();  // fewest resident workgroups per CU over the row-group kernels

// Slots in a row's workspace record: the most members a row group can have.
constexpr int kGroupSlotCap = 64;

// The largest row group: an index grid places a row's G members on one XCD,
// so G is at most the row-group slots of one XCD (its compute units times the
// workgroups one compute unit holds).  Ticketed grids take the smaller cap
// of ticket_cap_of.
int32_t group_cap_of(int32_t cu_count, int32_t xcd_count, int32_t per_cu) {
  if (cu_count <= 0 || xcd_count <= 0 || per_cu <= 0) return 0;
  const int64_t slots = static_cast<int64_t>(cu_count / xcd_count) * per_cu;
  return static_cast<int32_t>(std::min<int64_t>(slots, kGroupSlotCap));
}

// Shader engines per XCD on gfx950.  Each XCD deals its workgroups to its
// engines in a fixed rotation and waits, in order, for a slot on the engine
// whose turn it is (measured on MI355X: workgroups that held one engine's
// compute units 40 times longer than the others still received exactly a
// quarter of each XCD's workgroups, and the rest of the XCD waited for them).
constexpr int kEnginesPerXcd = 4;

// The largest row group a ticketed grid may take.  Its waiting members (at
// most G - 1, all in the group holding the newest ticket) must leave a slot
// on every engine, or the engine whose turn it is can hold only waiting
// members and its XCD stops starting workgroups; near the end of the grid
// no other XCD may be left to start the group's missing members.  So G is at
// most one engine's row-group slots: its compute units times the workgroups
// one compute unit holds (8 on MI355X).
int32_t ticket_cap_of(int32_t cu_count, int32_t xcd_count, int32_t per_cu) {
  if (cu_count <= 0 || xcd_count <= 0 || per_cu <= 0) return 0;
  const int64_t slots = static_cast<int64_t>(cu_count / xcd_count / kEnginesPerXcd) * per_cu;
  return static_cast<int32_t>(std::min<int64_t>(std::max<int64_t>(slots, 1), kGroupSlotCap));
}

ets_status device_info(int dev, DeviceInfo* info_out) {
  if (dev < 0 || dev >= kMaxDevices) return ETS_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_dev_mutex);
  DeviceInfo& d = g_dev[dev];
  if (!d.queried) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ETS_ERR_DEVICE;
    d.supported = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.cu_count = prop.multiProcessorCount;
    int xcc = 0;
    if (hipDeviceGetAttribute(&xcc, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || xcc <= 0)
      return ETS_ERR_DEVICE;
    d.xcd_count = xcc;
    if (d.supported) {
      // occupancy queries refer to the current device
      int cur = -1;
      if (hipGetDevice(&cur) != hipSuccess) return ETS_ERR_DEVICE;
      if (cur != dev && hipSetDevice(dev) != hipSuccess) return ETS_ERR_DEVICE;
      d.group_occ = group_kernel_occupancy();
      if (cur != dev) (void)hipSetDevice(cur);
      if (d.group_occ <= 0) return ETS_ERR_DEVICE;
      d.group_cap = group_cap_of(d.cu_count, d.xcd_count, d.group_occ);
      d.ticket_cap = ticket_cap_of(d.cu_count, d.xcd_count, d.group_occ);
    }
    d.queried = true;
  }
  if (!d.supported) return ETS_ERR_DEVICE;
  *info_out = d;
  return ETS_OK;
}

ets_status current_device(int* dev_out, DeviceInfo* info_out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ETS_ERR_DEVICE;
  *dev_out = dev;
  return device_info(dev, info_out);
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

// row-group path: 1024-lane workgroups, each holding up to VEC float4 per lane
constexpr int kGroupThreads = 1024;
constexpr int64_t kGroupChunk = 16384;  // scores per workgroup of a split row

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

template <int MODE, bool V4, int VEC, bool TICKET>
int occupancy_of() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, reinterpret_cast<const void*>(&ets::group_topk_kernel<kGroupThreads, VEC, MODE, V4, TICKET>),
          kGroupThreads, 0) != hipSuccess)
    return 0;
  return n;
}
template <int MODE, bool V4, bool TICKET>
int occupancy_vecs() {
  return std::min(std::min(occupancy_of<MODE, V4, 1, TICKET>(), occupancy_of<MODE, V4, 2, TICKET>()),
                  std::min(occupancy_of<MODE, V4, 4, TICKET>(), occupancy_of<MODE, V4, 8, TICKET>()));
}
int group_kernel_occupancy() {
  int m = occupancy_vecs<ets::kRagged, false, false>();
  m = std::min(m, occupancy_vecs<ets::kRagged, false, true>());
  m = std::min(m, occupancy_vecs<ets::kRaw, false, false>());
  m = std::min(m, occupancy_vecs<ets::kRaw, false, true>());
  m = std::min(m, occupancy_vecs<ets::kRaw, true, false>());
  m = std::min(m, occupancy_vecs<ets::kRaw, true, true>());
  m = std::min(m, occupancy_vecs<ets::kPaged, false, false>());
  m = std::min(m, occupancy_vecs<ets::kPaged, false, true>());
  m = std::min(m, occupancy_vecs<ets::kPaged, true, false>());
  m = std::min(m, occupancy_vecs<ets::kPaged, true, true>());
  return m;
}

// Workgroups per row (0 = one workgroup per row on the row kernel; -1 = an
// ETS_ROW_SPLIT override above max_group, which the calls reject).  A row
// that fits one resident 32768-score tile stays on one workgroup: measured on
// MI355X, the group's exchanges cost more than the work they spread.  Longer
// rows are always split, and the choice is between two member counts: g16,
// chunks of at most kGroupChunk (16384) scores, and g32, the fewest members
// whose chunks still fit one resident tile.  A sweep on MI355X (raw rows,
// k = 2048, B from 1 to 512, L = 65536, 131072 and 262144, G from 2 to 32)
// placed the best G at:
//  * the largest G <= g16 whose index grid fits the device at once (one XCD
//    per row, no member waiting for a workgroup that has not started), as
//    long as that keeps chunks resident (G >= g32): B = 48, L = 131072 took
//    17.6 us at G = 5 against 27.9 at G = 8 on a ticketed grid;
//  * otherwise g32, on a ticketed grid or several index grids, also once the
//    rows alone fill the compute units: B = 256, L = 262144 took 122 us at
//    G = 8 against 182 us with one workgroup per row streaming its tiles, and
//    B = 192, L = 65536 33.5 us at G = 2 against 45.9.
// The device is given by its compute units, XCDs and the row-group
// workgroups one compute unit holds: G is at most one XCD's slots
// (group_cap_of); rows longer than that many tiles stream their chunks.
// Unknown device facts (<= 0) leave g16 within the workspace's slot count.
// ETS_ROW_SPLIT overrides: 0 or 1 = one workgroup per row, n >= 2 = n
// workgroups per row, n at most the cap.
// Fewest scores per member chunk of a split row: ets::kMinChunk, or the
// environment variable ETS_MIN_CHUNK (read at every call) when it is an
// integer >= 1, rounded up to a multiple of 4 and capped at one 32768-score
// tile.
int32_t min_chunk_setting() {
  if (const char* e = std::getenv("ETS_MIN_CHUNK"); e != nullptr && *e != '\0') {
    char* end = nullptr;
    const long v = std::strtol(e, &end, 10);
    if (end != e && *end == '\0' && v >= 1) {
      const int64_t c = (std::min<int64_t>(v, kRowTile) + 3) & ~static_cast<int64_t>(3);
      return static_cast<int32_t>(c);
    }
  }
  return ets::kMinChunk;
}

int32_t split_plan(int32_t B, int64_t max_len, int32_t cu_count, int32_t xcd_count, int32_t per_cu) {
  if (B <= 0 || max_len <= 0) return 0;
  const bool known = cu_count > 0 && xcd_count > 0 && per_cu > 0;
  const int64_t cap = known ? std::max(group_cap_of(cu_count, xcd_count, per_cu), 1) : kGroupSlotCap;
  if (const char* e = std::getenv("ETS_ROW_SPLIT"); e != nullptr && *e != '\0') {
    char* end = nullptr;
    const long v = std::strtol(e, &end, 10);
    if (end != e && *end == '\0' && v >= 0) {
      if (v <= 1) return 0;
      return v <= cap ? static_cast<int32_t>(v) : -1;
    }
  }
  if (max_len <= kRowTile) return 0;
  const int64_t g16 = std::min((max_len + kGroupChunk - 1) / kGroupChunk, cap);
  const int64_t g32 = std::min((max_len + kRowTile - 1) / kRowTile, cap);
  if (!known) return static_cast<int32_t>(g16);
  // the largest G whose index grid (padded to whole rows per XCD) fits the
  // device's row-group slots at once
  const int64_t slots = static_cast<int64_t>(cu_count) * per_cu;
  const int64_t rows_per_xcd = (static_cast<int64_t>(B) + xcd_count - 1) / xcd_count;
  const int64_t g_index = std::min(g16, slots / (static_cast<int64_t>(xcd_count) * rows_per_xcd));
  const int64_t G = g_index >= g32 ? g_index : g32;
  return G >= 2 ? static_cast<int32_t>(G) : 0;
}

size_t group_ws_bytes(int32_t B) {
  const size_t per_row = ets::kRecWords + 3 * static_cast<size_t>(ets::kHistBins) + 2 * static_cast<size_t>(ets::kTieCap);
  return (ets::kHdrWords + static_cast<size_t>(B) * per_row) * 4;
}

// Host-side check of a call's launch plan and of the row-group path's
// workspace, before anything is enqueued.
ets_status check_workspace(int32_t B, int64_t max_len, const DeviceInfo& info, const void* ws,
                           size_t ws_bytes) {
  const int32_t G = split_plan(B, max_len, info.cu_count, info.xcd_count, info.group_occ);
  if (G < 0) return ETS_ERR_INVALID_ARG;
  if (G == 0) return ETS_OK;
  if (static_cast<int64_t>(B) * G > INT32_MAX) return ETS_ERR_INVALID_ARG;
  if (!ws || ws_bytes < group_ws_bytes(B) || !aligned16(ws)) return ETS_ERR_WORKSPACE;
  return ETS_OK;
}

template <int MODE, bool V4, int T, int VEC, bool STREAM>
void launch_rows(const ets::Params& p, int32_t B, hipStream_t stream) {
  hipLaunchKernelGGL((ets::row_topk_kernel<T, VEC, MODE, V4, STREAM>), dim3(B), dim3(T), 0, stream,
                     p);
}

// Members are assigned by workgroup index, one XCD per row, when the whole
// padded grid fits the device's row-group slots at once (each compute unit
// holds group_occ of them); otherwise by ticket in start order (see
// group_topk_kernel) when G is within ticket_cap; otherwise in several index
// grids on the stream, each over as many whole rows per XCD as fit the
// device at once.
template <int MODE, bool V4, int VEC>
void launch_group(const ets::Params& p, int32_t B, int32_t G, const DeviceInfo& info, void* ws,
                  hipStream_t stream) {
  const int64_t slots = static_cast<int64_t>(info.cu_count) * info.group_occ;
  const int32_t nx = std::max(info.xcd_count, 1);
  auto index_grid = [&](int32_t b0, int32_t rows) {
    // nx * G workgroups per nx rows, padded to whole rows per XCD
    const int64_t padded = static_cast<int64_t>(nx) * G * ((rows + nx - 1) / nx);
    hipLaunchKernelGGL((ets::group_topk_kernel<kGroupThreads, VEC, MODE, V4, false>),
                       dim3(static_cast<uint32_t>(padded)), dim3(kGroupThreads), 0, stream, p,
                       static_cast<uint32_t*>(ws), b0 + rows, G, nx, b0);
  };
  const int64_t padded = static_cast<int64_t>(nx) * G * ((B + nx - 1) / nx);
  if (padded <= slots) {
    index_grid(0, B);
  } else if (G <= info.ticket_cap) {
    const uint32_t grid = static_cast<uint32_t>(B) * static_cast<uint32_t>(G);
    hipLaunchKernelGGL((ets::group_topk_kernel<kGroupThreads, VEC, MODE, V4, true>), dim3(grid),
                       dim3(kGroupThreads), 0, stream, p, static_cast<uint32_t*>(ws), B, G, nx, 0);
  } else {
    // G <= group_cap, so at least one row per XCD fits
    const int32_t per_xcd = static_cast<int32_t>(std::max<int64_t>(1, slots / nx / G));
    const int32_t rows = nx * per_xcd;
    for (int32_t b0 = 0; b0 < B; b0 += rows) index_grid(b0, std::min(rows, B - b0));
  }
}

// Launch shape of a selection call: workgroups per row (1 = one per row on
// the row kernel), lanes per workgroup, float4 per lane per tile, and whether
// a one-workgroup row is streamed tile by tile instead of held in registers.
// A row on one workgroup gets the smallest resident tile that holds it, with
// as few scores per lane as the lane count allows: the passes are latency
// bound, and more waves with shorter slot loops hide more of it.
struct Shape {
  int32_t groups, threads, vec;
  bool stream;
};

Shape launch_shape(int32_t B, int64_t max_len, const DeviceInfo& info) {
  const int32_t G = split_plan(B, max_len, info.cu_count, info.xcd_count, info.group_occ);
  if (G <= 0) {
    if (max_len <= 2048) return {1, 512, 1, false};
    if (max_len <= 4096) return {1, kRowThreads, 1, false};
    if (max_len <= kRowTile / 4) return {1, kRowThreads, kRowVec / 4, false};
    if (max_len <= kRowTile / 2) return {1, kRowThreads, kRowVec / 2, false};
    return {1, kRowThreads, kRowVec, max_len > kRowTile};
  }
  const int64_t chunk = ets::member_chunk(max_len, G, min_chunk_setting());
  const int32_t vec = chunk <= kGroupThreads * 4 ? 1 : chunk <= kGroupThreads * 8 ? 2
                    : chunk <= kGroupThreads * 16 ? 4 : 8;
  return {G, kGroupThreads, vec, false};
}

template <int MODE, bool V4>
ets_status launch(const ets::Params& params, int32_t B, int64_t max_len, const DeviceInfo& info,
                  void* ws, hipStream_t stream) {
  ets::Params p = params;
  p.min_chunk = min_chunk_setting();
  const Shape sh = launch_shape(B, max_len, info);
  if (sh.groups == 1) {
    if (sh.threads == 512) {
      launch_rows<MODE, V4, 512, 1, false>(p, B, stream);
    } else if (sh.stream) {
      launch_rows<MODE, V4, kRowThreads, kRowVec, true>(p, B, stream);
    } else if (sh.vec == 1) {
      launch_rows<MODE, V4, kRowThreads, 1, false>(p, B, stream);
    } else if (sh.vec == 2) {
      launch_rows<MODE, V4, kRowThreads, 2, false>(p, B, stream);
    } else if (sh.vec == 4) {
      launch_rows<MODE, V4, kRowThreads, 4, false>(p, B, stream);
    } else {
      launch_rows<MODE, V4, kRowThreads, 8, false>(p, B, stream);
    }
    return hipGetLastError() == hipSuccess ? ETS_OK : ETS_ERR_HIP;
  }
  // (workspace already validated by check_workspace)
  if (sh.vec == 1) {
    launch_group<MODE, V4, 1>(p, B, sh.groups, info, ws, stream);
  } else if (sh.vec == 2) {
    launch_group<MODE, V4, 2>(p, B, sh.groups, info, ws, stream);
  } else if (sh.vec == 4) {
    launch_group<MODE, V4, 4>(p, B, sh.groups, info, ws, stream);
  } else {
    launch_group<MODE, V4, 8>(p, B, sh.groups, info, ws, stream);
  }
  return hipGetLastError() == hipSuccess ? ETS_OK : ETS_ERR_HIP;
}

// Per-device address of ets::scratch (hipGetSymbolAddress once per device,
// with that device current) and whether it has been zero-filled by a launch
// that ran outside graph capture.
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};
bool g_scratch_zeroed[kMaxDevices] = {};

ets_status scratch_setup(int dev, hipStream_t stream, void** ptr_out) {
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(ets::scratch)) != hipSuccess || ptr == nullptr)
      return ETS_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  if (!g_scratch_zeroed[dev]) {
    // zero-fill on the caller's stream with a kernel (no memset node if the
    // stream is being captured: the graph then zero-fills on every replay
    // until an eager call has done it once)
    const int64_t words = static_cast<int64_t>(ets::kScratchBytes / 4);
    hipLaunchKernelGGL(ets::workspace_clear, dim3(1024), dim3(256), 0, stream,
                       static_cast<uint32_t*>(g_scratch_ptr[dev]), words);
    if (hipGetLastError() != hipSuccess) return ETS_ERR_HIP;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return ETS_ERR_HIP;
    if (cs == hipStreamCaptureStatusNone) g_scratch_zeroed[dev] = true;
  }
  *ptr_out = g_scratch_ptr[dev];
  return ETS_OK;
}

template <int MODE, bool V4, int T, int VEC>
void launch_floor_read(const ets::Params& p, uint32_t grid, uint32_t* sink, int32_t G, hipStream_t s) {
  hipLaunchKernelGGL((ets::floor_read_kernel<T, VEC, MODE, V4>), dim3(grid), dim3(T), 0, s, p, sink, G);
}

template <int MODE, bool V4>
void floor_read(const ets::Params& p, const Shape& sh, uint32_t grid, uint32_t* sink, hipStream_t s) {
  if (sh.threads == 512) {
    launch_floor_read<MODE, V4, 512, 1>(p, grid, sink, sh.groups, s);
  } else if (sh.vec == 1) {
    launch_floor_read<MODE, V4, 1024, 1>(p, grid, sink, sh.groups, s);
  } else if (sh.vec == 2) {
    launch_floor_read<MODE, V4, 1024, 2>(p, grid, sink, sh.groups, s);
  } else if (sh.vec == 4) {
    launch_floor_read<MODE, V4, 1024, 4>(p, grid, sink, sh.groups, s);
  } else {
    launch_floor_read<MODE, V4, 1024, 8>(p, grid, sink, sh.groups, s);
  }
}

}  // namespace

extern "C" {

ets_status ets_floor_read(const float* scores, int64_t row_stride, int32_t B, int32_t L,
                          const int32_t* lens, const int32_t* row_starts, int64_t max_len_hint,
                          uint32_t* sink, int64_t sink_words, void* stream) {
  const bool ragged = row_starts != nullptr;
  if (B < 0 || (ragged ? (max_len_hint < 0 || !lens) : (L < 0 || row_stride < L)))
    return ETS_ERR_INVALID_ARG;
  if (B == 0) return ETS_OK;
  if (!sink || !scores) return ETS_ERR_INVALID_ARG;
  int dev;
  DeviceInfo info;
  if (ets_status st = current_device(&dev, &info); st != ETS_OK) return st;
  const int64_t max_len = ragged ? max_len_hint : L;
  if (split_plan(B, max_len, info.cu_count, info.xcd_count, info.group_occ) < 0) return ETS_ERR_INVALID_ARG;
  const Shape sh = launch_shape(B, max_len, info);
  const int64_t grid = static_cast<int64_t>(B) * sh.groups;
  if (grid > INT32_MAX || sink_words < grid) return ETS_ERR_INVALID_ARG;
  ets::Params p{};
  p.scores = scores;
  p.row_stride = row_stride;
  p.lens = lens;
  p.row_starts = row_starts;
  p.L = L;
  p.min_chunk = min_chunk_setting();
  auto s = static_cast<hipStream_t>(stream);
  const uint32_t g = static_cast<uint32_t>(grid);
  if (ragged) {
    floor_read<ets::kRagged, false>(p, sh, g, sink, s);
  } else if (aligned16(scores) && row_stride % 4 == 0 && L % 4 == 0) {
    floor_read<ets::kRaw, true>(p, sh, g, sink, s);
  } else {
    floor_read<ets::kRaw, false>(p, sh, g, sink, s);
  }
  return hipGetLastError() == hipSuccess ? ETS_OK : ETS_ERR_HIP;
}

ets_status ets_floor_launch(int32_t B, int64_t max_row_len, void* stream) {
  if (B < 0 || max_row_len < 0) return ETS_ERR_INVALID_ARG;
  if (B == 0) return ETS_OK;
  int dev;
  DeviceInfo info;
  if (ets_status st = current_device(&dev, &info); st != ETS_OK) return st;
  if (split_plan(B, max_row_len, info.cu_count, info.xcd_count, info.group_occ) < 0) return ETS_ERR_INVALID_ARG;
  const Shape sh = launch_shape(B, max_row_len, info);
  const int64_t grid = static_cast<int64_t>(B) * sh.groups;
  if (grid > INT32_MAX) return ETS_ERR_INVALID_ARG;
  auto s = static_cast<hipStream_t>(stream);
  if (sh.threads == 512) {
    hipLaunchKernelGGL(ets::floor_launch_kernel<512>, dim3(static_cast<uint32_t>(grid)), dim3(512), 0, s);
  } else {
    hipLaunchKernelGGL(ets::floor_launch_kernel<1024>, dim3(static_cast<uint32_t>(grid)), dim3(1024), 0, s);
  }
  return hipGetLastError() == hipSuccess ? ETS_OK : ETS_ERR_HIP;
}

const char* ets_status_string(ets_status status) {
  switch (status) {
    case ETS_OK: return "ok";
    case ETS_ERR_INVALID_ARG: return "invalid argument";
    case ETS_ERR_K_RANGE: return "k outside [1, ETS_MAX_K]";
    case ETS_ERR_WORKSPACE: return "workspace too small";
    case ETS_ERR_DEVICE: return "unsupported or unavailable device (gfx950 required)";
    case ETS_ERR_HIP: return "HIP runtime error";
    case ETS_ERR_SCRATCH: return "call needs more row-group workspace than the library's static scratch";
    default: return "unknown status";
  }
}

int32_t ets_row_split(int32_t B, int64_t max_row_len, int32_t cu_count, int32_t xcd_count,
                      int32_t groups_per_cu) {
  return split_plan(B, max_row_len, cu_count, xcd_count, groups_per_cu);
}

ets_status ets_workspace_size(int32_t B, int64_t max_row_len, int32_t k, int32_t device,
                              size_t* bytes) {
  if (!bytes || B < 0 || max_row_len < 0) return ETS_ERR_INVALID_ARG;
  if (k < 1 || k > ETS_MAX_K) return ETS_ERR_K_RANGE;
  DeviceInfo info;
  int dev = device;
  if (dev < 0 && hipGetDevice(&dev) != hipSuccess) return ETS_ERR_DEVICE;
  if (ets_status st = device_info(dev, &info); st != ETS_OK) return st;
  const int32_t G = split_plan(B, max_row_len, info.cu_count, info.xcd_count, info.group_occ);
  if (G < 0) return ETS_ERR_INVALID_ARG;
  *bytes = (G == 0 || B == 0) ? 0 : group_ws_bytes(B);
  return ETS_OK;
}

ets_status ets_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (workspace_bytes == 0) return ETS_OK;
  if (!workspace || !aligned16(workspace)) return ETS_ERR_INVALID_ARG;
  const int64_t words = static_cast<int64_t>(workspace_bytes / 4);
  const int blocks = static_cast<int>(std::min<int64_t>(1024, (words + 255) / 256));
  hipLaunchKernelGGL(ets::workspace_clear, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint32_t*>(workspace), words);
  return hipGetLastError() == hipSuccess ? ETS_OK : ETS_ERR_HIP;
}

ets_status ets_workspace_error(void* workspace, size_t workspace_bytes, int32_t* flag, void* stream) {
  if (!flag) return ETS_ERR_INVALID_ARG;
  if (workspace_bytes != 0 && (!workspace || !aligned16(workspace) ||
                               workspace_bytes < static_cast<size_t>(ets::kHdrWords) * 4))
    return ETS_ERR_INVALID_ARG;
  hipLaunchKernelGGL(ets::workspace_error_take, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                     workspace_bytes != 0 ? static_cast<uint32_t*>(workspace) : nullptr, flag);
  return hipGetLastError() == hipSuccess ? ETS_OK : ETS_ERR_HIP;
}

ets_status ets_device_limits(int32_t device, int32_t* cu_count, int32_t* xcd_count,
                             int32_t* groups_per_cu) {
  if (!cu_count || !xcd_count || !groups_per_cu) return ETS_ERR_INVALID_ARG;
  int dev = device;
  if (dev < 0 && hipGetDevice(&dev) != hipSuccess) return ETS_ERR_DEVICE;
  DeviceInfo info;
  if (ets_status st = device_info(dev, &info); st != ETS_OK) return st;
  *cu_count = info.cu_count;
  *xcd_count = info.xcd_count;
  *groups_per_cu = info.group_occ;
  return ETS_OK;
}

int32_t ets_group_cap(int32_t cu_count, int32_t xcd_count, int32_t groups_per_cu) {
  return group_cap_of(cu_count, xcd_count, groups_per_cu);
}

int32_t ets_ticket_cap(int32_t cu_count, int32_t xcd_count, int32_t groups_per_cu) {
  return ticket_cap_of(cu_count, xcd_count, groups_per_cu);
}

ets_status ets_topk_raw(const float* scores, int64_t row_stride, int32_t B, int32_t L,
                        const int32_t* lens, int32_t k, int32_t* out, int64_t out_stride,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (k < 1 || k > ETS_MAX_K) return ETS_ERR_K_RANGE;
  if (B < 0 || L < 0 || row_stride < L || out_stride < k) return ETS_ERR_INVALID_ARG;
  if (B == 0) return ETS_OK;
  if (!out || (L > 0 && !scores)) return ETS_ERR_INVALID_ARG;
  int dev;
  DeviceInfo info;
  if (ets_status st = current_device(&dev, &info); st != ETS_OK) return st;
  if (ets_status st = check_workspace(B, L, info, workspace, workspace_bytes); st != ETS_OK)
    return st;
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
  return v4 ? launch<ets::kRaw, true>(p, B, L, info, workspace, s)
            : launch<ets::kRaw, false>(p, B, L, info, workspace, s);
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
  int dev;
  DeviceInfo info;
  if (ets_status st = current_device(&dev, &info); st != ETS_OK) return st;
  if (ets_status st = check_workspace(B, L, info, workspace, workspace_bytes); st != ETS_OK)
    return st;
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
  return v4 ? launch<ets::kPaged, true>(p, B, L, info, workspace, s)
            : launch<ets::kPaged, false>(p, B, L, info, workspace, s);
}

ets_status ets_topk_paged_window(const float* scores, int64_t row_stride, int32_t B, int32_t L,
                                 const int32_t* window_starts, const int32_t* seq_lens,
                                 const int32_t* page_table, int64_t pt_stride, int32_t page_size,
                                 int32_t k, int32_t* out, int64_t out_stride, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (window_starts == nullptr)
    return ets_topk_paged(scores, row_stride, B, L, seq_lens, page_table, pt_stride, page_size, k, out,
                          out_stride, workspace, workspace_bytes, stream);
  if (k < 1 || k > ETS_MAX_K) return ETS_ERR_K_RANGE;
  if (B < 0 || L < 0 || row_stride < L || out_stride < k || page_size < 1 || pt_stride < 0)
    return ETS_ERR_INVALID_ARG;
  if (B == 0) return ETS_OK;
  if (!out || !seq_lens || !page_table || (L > 0 && !scores)) return ETS_ERR_INVALID_ARG;
  int dev;
  DeviceInfo info;
  if (ets_status st = current_device(&dev, &info); st != ETS_OK) return st;
  if (ets_status st = check_workspace(B, L, info, workspace, workspace_bytes); st != ETS_OK)
    return st;
  ets::Params p{};
  p.scores = scores;
  p.row_stride = row_stride;
  p.lens = seq_lens;
  p.win_starts = window_starts;
  p.page_table = page_table;
  p.pt_stride = pt_stride;
  p.page_size = page_size;
  p.page_shift = page_shift_of(page_size);
  p.L = L;
  p.k = k;
  p.out = out;
  p.out_stride = out_stride;
  // a window start moves a row's first score off the 16-byte grid: dword loads
  return launch<ets::kPaged, false>(p, B, L, info, workspace, static_cast<hipStream_t>(stream));
}

ets_status ets_topk_paged_noalloc(const float* scores, int64_t row_stride, int32_t B, int32_t L,
                                  const int32_t* seq_lens, const int32_t* page_table,
                                  int64_t pt_stride, int32_t page_size, int32_t k, int32_t* out,
                                  int64_t out_stride, int32_t* error_flag, void* stream) {
  if (k < 1 || k > ETS_MAX_K) return ETS_ERR_K_RANGE;
  if (B < 0 || L < 0 || row_stride < L || out_stride < k || page_size < 1 || pt_stride < 0)
    return ETS_ERR_INVALID_ARG;
  if (B == 0) return ETS_OK;
  if (!out || !seq_lens || !page_table || (L > 0 && !scores)) return ETS_ERR_INVALID_ARG;
  int dev;
  DeviceInfo info;
  if (ets_status st = current_device(&dev, &info); st != ETS_OK) return st;
  const int32_t G = split_plan(B, L, info.cu_count, info.xcd_count, info.group_occ);
  if (G < 0 || static_cast<int64_t>(B) * G > INT32_MAX) return ETS_ERR_INVALID_ARG;
  const size_t need = G == 0 ? 0 : group_ws_bytes(B);
  if (need > ets::kScratchBytes) return ETS_ERR_SCRATCH;
  auto s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (need > 0 || error_flag != nullptr) {
    if (ets_status st = scratch_setup(dev, s, &ws); st != ETS_OK) return st;
  }
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
  const ets_status st = v4 ? launch<ets::kPaged, true>(p, B, L, info, ws, s)
                           : launch<ets::kPaged, false>(p, B, L, info, ws, s);
  if (st != ETS_OK || error_flag == nullptr) return st;
  hipLaunchKernelGGL(ets::scratch_error_take, dim3(1), dim3(1024), 0, s, static_cast<uint32_t*>(ws),
                     static_cast<int64_t>(ets::kScratchBytes / 4), error_flag);
  return hipGetLastError() == hipSuccess ? ETS_OK : ETS_ERR_HIP;
}

ets_status ets_topk_ragged(const float* packed, const int32_t* row_starts,
                           const int32_t* lengths, int32_t B, int64_t max_len_hint, int32_t k,
                           int32_t* out, int64_t out_stride, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (k < 1 || k > ETS_MAX_K) return ETS_ERR_K_RANGE;
  if (B < 0 || max_len_hint < 0 || out_stride < k) return ETS_ERR_INVALID_ARG;
  if (B == 0) return ETS_OK;
  if (!out || !row_starts || !lengths || !packed) return ETS_ERR_INVALID_ARG;
  int dev;
  DeviceInfo info;
  if (ets_status st = current_device(&dev, &info); st != ETS_OK) return st;
  if (ets_status st = check_workspace(B, max_len_hint, info, workspace, workspace_bytes);
      st != ETS_OK)
    return st;
  ets::Params p{};
  p.scores = packed;
  p.lens = lengths;
  p.row_starts = row_starts;
  p.k = k;
  p.out = out;
  p.out_stride = out_stride;
  p.page_shift = -1;
  return launch<ets::kRagged, false>(p, B, max_len_hint, info, workspace,
                                     static_cast<hipStream_t>(stream));
}

}  // extern "C"
