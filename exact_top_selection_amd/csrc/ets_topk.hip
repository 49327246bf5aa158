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

#include "ets_topk.h"

namespace ets {

constexpr int kHistBits = 12;
constexpr int kHistBins = 1 << kHistBits;
constexpr int kSmallCap = 256;  // largest bucket ranked by direct comparison

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

__device__ __forceinline__ uint64_t composite(uint32_t key, int32_t pos) {
  return (static_cast<uint64_t>(key) << 32) | static_cast<uint32_t>(~pos);
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

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  const int lane = __lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = max(x, static_cast<uint32_t>(__shfl_xor(x, o, 64)));
  return x;
}
__device__ __forceinline__ uint32_t wave_min(uint32_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = min(x, static_cast<uint32_t>(__shfl_xor(x, o, 64)));
  return x;
}
__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += static_cast<uint32_t>(__shfl_xor(x, o, 64));
  return x;
}

// Exclusive prefix sum over the block in thread order; `total` gets the sum.
// Uses s_wave[0 .. T/64); ends with a barrier so s_wave may be reused.
template <int T>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* s_wave, uint32_t& total) {
  constexpr int W = T / 64;
  const int lane = __lane_id();
  const int wid = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan(v);
  if (lane == 63) s_wave[wid] = incl;
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

// Adds one to hist[bin] for every lane with `pred`.  Lanes that share the
// first active lane's bin are merged into one LDS atomic, which removes the
// serialisation when most of a wave lands in one bin (concentrated scores).
__device__ __forceinline__ void hist_add(uint32_t* hist, bool pred, uint32_t bin) {
  if (pred) {
    const uint32_t lead = __builtin_amdgcn_readfirstlane(bin);
    const uint64_t same = __ballot(bin == lead);
    if (bin == lead) {
      if (__lane_id() == __builtin_amdgcn_readfirstlane(__lane_id())) {
        atomicAdd(&hist[lead], static_cast<uint32_t>(__popcll(same)));
      }
    } else {
      atomicAdd(&hist[bin], 1u);
    }
  }
}

// Finds the histogram bin t with above(t) < kk <= above(t) + hist[t], where
// above(t) counts the entries of all higher bins.  Results land in s_res[0..2]
// = (t, above(t), hist[t]) for every thread after the final barrier.
template <int T>
__device__ __forceinline__ void find_threshold_bin(const uint32_t* hist, uint32_t kk,
                                                   uint32_t* s_wave, uint32_t* s_res) {
  constexpr int BPT = kHistBins / T;  // bins owned by each thread
  static_assert(BPT * T == kHistBins, "block size must divide the bin count");
  uint32_t h[BPT];
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    h[i] = hist[threadIdx.x * BPT + i];
    s += h[i];
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

// Element layout of one tile held by a thread.  V4: float4 v of thread t holds
// positions 4 (v T + t) + c; scalar: element j of thread t is at j T + t.
template <int T, int PT, bool V4>
__device__ __forceinline__ int32_t tile_pos(int j) {
  if constexpr (V4) {
    return 4 * ((j >> 2) * T + static_cast<int>(threadIdx.x)) + (j & 3);
  } else {
    return j * T + static_cast<int>(threadIdx.x);
  }
}

template <int T, int VEC, int MODE, bool V4>
__global__ __launch_bounds__(T) void row_topk_kernel(Params p) {
  constexpr int PT = VEC * 4;     // keys per thread per tile
  constexpr int TILE = T * PT;    // scores per tile
  constexpr int W = T / 64;

  __shared__ __align__(16) uint32_t s_hist[kHistBins];
  __shared__ uint32_t s_ckey[kSmallCap];
  __shared__ int32_t s_cpos[kSmallCap];
  __shared__ uint32_t s_wave[4 * W];
  __shared__ uint32_t s_res[4];
  __shared__ uint32_t s_ccount;

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = __lane_id();
  const int wid = tid >> 6;

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
  const int32_t k = p.k;

  // Rows no longer than k: every position is selected, the rest is padding.
  if (n <= k) {
    for (int32_t i = tid; i < k; i += T) {
      out[i] = (i < n) ? map_position<MODE>(p, pt_row, row_start, i) : -1;
    }
    return;
  }

  const int ntiles = (n + TILE - 1) / TILE;
  uint32_t key[PT];

  auto load_tile = [&](int tile) {
    const int32_t base = tile * TILE;
    if constexpr (V4) {
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        const int32_t q = base + 4 * (v * T + tid);
        if (q >= n) {
#pragma unroll
          for (int c = 0; c < 4; ++c) key[4 * v + c] = 0u;
        } else if (q + 3 < cap) {
          const uint4 w = *reinterpret_cast<const uint4*>(row + q);
          key[4 * v + 0] = order_key(w.x);
          key[4 * v + 1] = order_key(w.y);
          key[4 * v + 2] = order_key(w.z);
          key[4 * v + 3] = order_key(w.w);
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            key[4 * v + c] = (q + c < n) ? order_key(__float_as_uint(row[q + c])) : 0u;
          }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < PT; ++j) {
        const int32_t q = base + j * T + tid;
        key[j] = (q < n) ? order_key(__float_as_uint(row[q])) : 0u;
      }
    }
  };
  // Applies f(key, pos) to every valid score of the row, tile by tile.  A
  // row that fits one tile is loaded once and then reused from registers.
  auto for_each = [&](auto&& f) {
    for (int tile = 0; tile < ntiles; ++tile) {
      if (ntiles > 1) load_tile(tile);
      const int32_t base = tile * TILE;
      if (base + TILE <= n) {
#pragma unroll
        for (int j = 0; j < PT; ++j) f(key[j], base + tile_pos<T, PT, V4>(j), true);
      } else {
#pragma unroll
        for (int j = 0; j < PT; ++j) {
          const int32_t pos = base + tile_pos<T, PT, V4>(j);
          f(key[j], pos, pos < n);
        }
      }
    }
  };

  if (ntiles == 1) load_tile(0);

  // ---- bounds: row max, and a lower bound of the k-th largest key.
  const int32_t jth = (k + T - 1) / T;  // 1 or 2 for T = 1024, k <= 2048
  uint32_t m1 = 0, m2 = 0, mn = 0xFFFFFFFFu, cnt = 0;
  for_each([&](uint32_t x, int32_t, bool valid) {
    if (valid) {
      m2 = max(m2, min(m1, x));
      m1 = max(m1, x);
      mn = min(mn, x);
      ++cnt;
    }
  });
  {
    const bool full = (jth <= 2) && (cnt >= static_cast<uint32_t>(jth));
    uint32_t cand = full ? (jth == 1 ? m1 : m2) : 0xFFFFFFFFu;
    uint32_t rmax = wave_max(cnt ? m1 : 0u);
    uint32_t rmin = wave_min(mn);
    uint32_t bmin = wave_min(cand);
    uint32_t nfull = wave_sum(full ? 1u : 0u);
    if (lane == 0) {
      s_wave[wid] = rmax;
      s_wave[W + wid] = rmin;
      s_wave[2 * W + wid] = bmin;
      s_wave[3 * W + wid] = nfull;
    }
    __syncthreads();
    rmax = 0;
    rmin = 0xFFFFFFFFu;
    bmin = 0xFFFFFFFFu;
    nfull = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      rmax = max(rmax, s_wave[w]);
      rmin = min(rmin, s_wave[W + w]);
      bmin = min(bmin, s_wave[2 * W + w]);
      nfull += s_wave[3 * W + w];
    }
    __syncthreads();
    // nfull * jth distinct scores are >= bmin; if that is not k of them the
    // row minimum is the (trivially valid) bound.
    const uint32_t lo_key = (jth <= 2 && nfull * static_cast<uint32_t>(jth) >= static_cast<uint32_t>(k))
                                ? bmin : rmin;
    m1 = rmax;
    mn = lo_key;
  }

  // ---- radix rounds on the composite (key, ~pos) inside [lo, hi].
  uint64_t lo = static_cast<uint64_t>(mn) << 32;
  uint64_t hi = (static_cast<uint64_t>(m1) << 32) | 0xFFFFFFFFull;
  uint32_t kk = static_cast<uint32_t>(k);
  uint32_t bucket = 0;
  for (;;) {
    const uint64_t span = hi - lo;
    const int bl = span ? 64 - __clzll(span) : 0;
    const int s = bl > kHistBits ? bl - kHistBits : 0;
    for (int i = tid; i < kHistBins / 4; i += T) reinterpret_cast<uint4*>(s_hist)[i] = make_uint4(0, 0, 0, 0);
    __syncthreads();
    if (s >= 32) {
      // key-aligned range: bins depend on the key only
      const uint32_t lk = static_cast<uint32_t>(lo >> 32), hk = static_cast<uint32_t>(hi >> 32);
      const int sk = s - 32;
      for_each([&](uint32_t x, int32_t, bool valid) {
        const bool in = valid && x >= lk && x <= hk;
        hist_add(s_hist, in, (x - lk) >> sk);
      });
    } else {
      for_each([&](uint32_t x, int32_t pos, bool valid) {
        const uint64_t c = composite(x, pos);
        const bool in = valid && c >= lo && c <= hi;
        hist_add(s_hist, in, static_cast<uint32_t>((c - lo) >> s));
      });
    }
    __syncthreads();
    find_threshold_bin<T>(s_hist, kk, s_wave, s_res);
    const uint32_t t = s_res[0];
    const uint32_t above = s_res[1];
    bucket = s_res[2];
    const uint64_t nlo = lo + (static_cast<uint64_t>(t) << s);
    const uint64_t width = (s >= 64) ? ~0ull : ((1ull << s) - 1ull);
    const uint64_t nhi = (hi - nlo > width) ? nlo + width : hi;
    lo = nlo;
    hi = nhi;
    kk -= above;
    __syncthreads();  // s_res is rewritten by the next round
    if (bucket <= static_cast<uint32_t>(kSmallCap)) break;
  }

  // ---- scatter: count winners (composite > hi), gather the bucket into LDS.
  if (tid == 0) s_ccount = 0;
  __syncthreads();
  uint32_t nwin = 0;
  for_each([&](uint32_t x, int32_t pos, bool valid) {
    const uint64_t c = composite(x, pos);
    nwin += (valid && c > hi) ? 1u : 0u;
    const bool cand = valid && c >= lo && c <= hi;
    const uint64_t m = __ballot(cand);
    if (m) {
      uint32_t base = 0;
      if (lane == __ffsll(static_cast<unsigned long long>(m)) - 1) {
        base = atomicAdd(&s_ccount, static_cast<uint32_t>(__popcll(m)));
      }
      base = __shfl(base, __ffsll(static_cast<unsigned long long>(m)) - 1, 64);
      const uint32_t slot = base + static_cast<uint32_t>(__popcll(m & ((1ull << lane) - 1ull)));
      if (cand && slot < static_cast<uint32_t>(kSmallCap)) {
        s_ckey[slot] = x;
        s_cpos[slot] = pos;
      }
    }
  });
  uint32_t total_win;
  uint32_t off = block_excl_scan<T>(nwin, s_wave, total_win);  // ends with a barrier
  // winners: k - kk of them, written in thread order (the bound only guards
  // the output row against a broken invariant)
  const uint32_t first = static_cast<uint32_t>(k) - kk;
  for_each([&](uint32_t x, int32_t pos, bool valid) {
    if (valid && composite(x, pos) > hi) {
      if (off < first) out[off] = map_position<MODE>(p, pt_row, row_start, pos);
      ++off;
    }
  });
  // bucket: rank by direct comparison, keep the kk best, place them by rank
  const uint32_t nc = min(s_ccount, static_cast<uint32_t>(kSmallCap));
  for (uint32_t i = tid; i < nc; i += T) {
    const uint64_t ci = composite(s_ckey[i], s_cpos[i]);
    uint32_t rank = 0;
    for (uint32_t j = 0; j < nc; ++j) rank += composite(s_ckey[j], s_cpos[j]) > ci ? 1u : 0u;
    if (rank < kk) out[first + rank] = map_position<MODE>(p, pt_row, row_start, s_cpos[i]);
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

template <int MODE, bool V4>
ets_status launch_rows(const ets::Params& p, int32_t B, hipStream_t stream) {
  hipLaunchKernelGGL((ets::row_topk_kernel<kRowThreads, kRowVec, MODE, V4>), dim3(B),
                     dim3(kRowThreads), 0, stream, p);
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
  return v4 ? launch_rows<ets::kRaw, true>(p, B, s) : launch_rows<ets::kRaw, false>(p, B, s);
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
  return v4 ? launch_rows<ets::kPaged, true>(p, B, s) : launch_rows<ets::kPaged, false>(p, B, s);
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
  return launch_rows<ets::kRagged, false>(p, B, static_cast<hipStream_t>(stream));
}

}  // extern "C"
