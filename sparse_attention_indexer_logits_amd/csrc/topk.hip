// Deterministic per-row top-k of the indexer logits (gfx950).
//
// Result (pages "xkernels #28 -- DeepSeek-V4 serving support": top-512 Flash /
// top-1024 Pro per query; "DeepSeek V4 Flash on a single AMD MI300X":
// deterministic sparse top-k with a tie-break, canonical order of the
// selection): among the n = clamp(limit+1, 0, K) valid keys of a row, the
// min(k, n) largest scores ordered by (score desc, j asc), then -1 padding.
//
// Many short rows (at least 1024 rows of at most 4096 keys, k <= 512) run
// one wave per row (topk_wave_kernel, below); otherwise one workgroup per
// row. Rows up to 16384 keys are read from HBM once and
// stay in VGPRs (V values per thread, j = tid + BLOCK*v); longer rows keep a
// 16384-key prefix in VGPRs and stream the rest once (topk_long_kernel).
// Scores become order-preserving u32 keys (-0.0 folded to +0.0); key 0 marks
// a slot past the row's end.
//
// Bucket path (every row in practice):
//  1. The block's finite score range [lo, hi] gives 2048 bins linear in the
//     score; an LDS histogram of the row, and one wave's descending scan of
//     it, give each bin's first output slot and the bin b* that holds the
//     k-th largest score.
//  2. Every entry in a bin >= b* is scattered to its bin's slots (atomic
//     cursors); its final position is the bin's first slot plus the number
//     of entries of its bin that precede it in (score desc, j asc) order,
//     counted by comparison, so the result does not depend on atomic order.
//     Positions below k are the output.
// Bins linear in the score spread logits over hundreds of bins, so the
// histogram atomics rarely collide and b* holds a handful of entries.
//
// Radix path (fallback when the bins at or above b* hold more than 2048
// entries: scores crowded into one bin by heavy ties or far outliers):
//  A. An LDS histogram of the top 11 key bits (sign, exponent, 2 mantissa
//     bits) and one wave's scan give the bucket b* that holds the k-th
//     largest key, the count above it and the count in it.
//  B. One sweep appends every key above b* to the selection and every key
//     in b* to an LDS candidate list; slots come from wave ballots and one
//     block-wide scan of the wave totals (no per-element atomics).
//  C. The rest of the threshold is found on the short candidate list only:
//     radix passes over key bits 20..10 and 9..0, then, for ties on the full
//     key, over j ascending (lower j wins). Histogram counts do not depend on
//     atomic order, so the selected SET is fixed.
//     If b* holds more keys than the list can take (heavy ties), the same
//     passes run over the row instead.
//  D. The selection is sorted by (key << 32 | ~j), descending, with a
//     counting sort on 2048 bins spanning its key range, then an exact rank
//     among the entries that share a bin.
#include <algorithm>
#include <type_traits>

#include "tile16.h"

namespace xk {
namespace {

constexpr int kBins = 2048;  // 11-bit digits
constexpr int kRefreshRoom = 2048;  // list entries kept free for the chunks after a refresh check

__device__ __forceinline__ int lane_id() { return int(threadIdx.x & 63); }

// DPP controls (GFX9 encoding).
constexpr int kDppQuadSwap1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppRowShr = 0x110;      // row_shr:n = kDppRowShr + n
constexpr int kDppRowMirror = 0x140;   // lane i <- 15 - i within a row of 16
constexpr int kDppHalfMirror = 0x141;  // lane i <- 7 - i within 8 lanes
constexpr int kDppBcast15 = 0x142;     // lane 15 of each row -> next row
constexpr int kDppBcast31 = 0x143;     // lane 31 -> rows 2 and 3

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp0(int v) {  // lanes without a source read 0
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4, 8
// inside each row of 16 lanes, then the row totals carried across rows by
// the broadcasts of lanes 15 and 31. All VALU, no LDS round trip.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp0<kDppRowShr + 1>(v);
  v += dpp0<kDppRowShr + 2>(v);
  v += dpp0<kDppRowShr + 4>(v);
  v += dpp0<kDppRowShr + 8>(v);
  v += dpp0<kDppBcast15, 0xA>(v);
  v += dpp0<kDppBcast31, 0xC>(v);
  return v;
}

// Minimum and maximum over the wave, uniform result: butterflies inside
// each row of 16 lanes, then the four row results read as scalars.
__device__ __forceinline__ void wave_min_max(uint32_t& mn, uint32_t& mx) {
#define XK_STEP(C)                                                           \
  mn = min(mn, uint32_t(__builtin_amdgcn_update_dpp(int(mn), int(mn), C, 0xF, 0xF, false))); \
  mx = max(mx, uint32_t(__builtin_amdgcn_update_dpp(int(mx), int(mx), C, 0xF, 0xF, false)));
  XK_STEP(kDppQuadSwap1)
  XK_STEP(kDppQuadSwap2)
  XK_STEP(kDppHalfMirror)
  XK_STEP(kDppRowMirror)
#undef XK_STEP
  uint32_t a = min(uint32_t(__builtin_amdgcn_readlane(int(mn), 0)), uint32_t(__builtin_amdgcn_readlane(int(mn), 16)));
  uint32_t b = min(uint32_t(__builtin_amdgcn_readlane(int(mn), 32)), uint32_t(__builtin_amdgcn_readlane(int(mn), 48)));
  mn = min(a, b);
  a = max(uint32_t(__builtin_amdgcn_readlane(int(mx), 0)), uint32_t(__builtin_amdgcn_readlane(int(mx), 16)));
  b = max(uint32_t(__builtin_amdgcn_readlane(int(mx), 32)), uint32_t(__builtin_amdgcn_readlane(int(mx), 48)));
  mx = max(a, b);
}

// LDS of one row. sel holds entries key << 32 | ~j (larger = better): the
// radix path's selection, or the bucket path's bin slots. ckey / cj is a
// candidate list: keys of the radix threshold bucket, or a long row's
// candidates.
template <int BLOCK, int CAP>
struct TopkShared {
  __attribute__((aligned(16))) uint32_t hist[kBins];
  uint64_t sel[kMaxTopk];
  uint32_t ckey[CAP];
  uint32_t cj[CAP];
  int wsel[BLOCK / 64], wcand[BLOCK / 64];
  uint32_t wlo[BLOCK / 64], whi[BLOCK / 64];  // per-wave finite key range
  int wtot[BLOCK / 64];                        // per-wave bin totals of the block scan
  float wsum[2][2][BLOCK / 64];                // long rows: per-wave sums of the threshold search
  int digit, above, at;
  int ccount;    // candidate list: entries claimed so far
  int overflow;  // 1 if the candidate list ran out of room
  uint32_t tau;  // long rows: smallest prefix key in a bin >= b*
};

// Wave 0: find the bin that holds the `need`-th element of hist[0..NBINS),
// counted from the top bin down (descending) or from bin 0 up. Each lane
// loads its NBINS/64 consecutive bins with 128-bit LDS reads, so the scan
// costs a few LDS round trips.
template <int NBINS, int BLOCK, int CAP>
__device__ __forceinline__ void find_bin(TopkShared<BLOCK, CAP>& sh, int need, bool descending) {
  constexpr int PER = NBINS / 64;
  static_assert(PER % 4 == 0, "bins per lane");
  const int lane = lane_id();
  // lane L covers scan positions [L*PER, L*PER+PER); descending scan position
  // p is bin NBINS-1-p, so lane L's bins are the block ending at NBINS-L*PER
  const int base = descending ? NBINS - (lane + 1) * PER : lane * PER;
  uint32_t c[PER];
#pragma unroll
  for (int i = 0; i < PER / 4; ++i) {
    const u32x4 q4 = *reinterpret_cast<const u32x4*>(&sh.hist[base + 4 * i]);
    c[4 * i] = q4[0];
    c[4 * i + 1] = q4[1];
    c[4 * i + 2] = q4[2];
    c[4 * i + 3] = q4[3];
  }
  int s = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) s += int(c[i]);
  const int incl = wave_incl_scan(s);
  int before = incl - s;
  if (before < need && incl >= need) {
    int found = -1, f_above = 0, f_at = 0;
#pragma unroll
    for (int o = 0; o < PER; ++o) {  // scan order within the lane's block
      const int i = descending ? PER - 1 - o : o;
      const int cnt = int(c[i]);
      if (found < 0 && before + cnt >= need) {
        found = base + i;
        f_above = before;
        f_at = cnt;
      }
      before += cnt;
    }
    sh.digit = found;
    sh.above = f_above;
    sh.at = f_at;
  }
}

template <int BLOCK, int CAP>
__device__ __forceinline__ void clear_hist(TopkShared<BLOCK, CAP>& sh, int nbins) {
  for (int i = threadIdx.x; i < nbins; i += BLOCK) sh.hist[i] = 0u;
}

// Append entries of a chunk (U per thread) to the selection (pred == 1) or
// to the candidate list (pred == 2). Each thread counts its hits, one wave
// scan of the packed counts plus per-wave totals in LDS give every thread
// its first slot, and each thread then writes only its own hits. key_at(u)
// / j_at(u) give entry u; the predicate is evaluated once, into a 2-bit
// class per entry. The running totals nsel / ncand stay in registers
// (uniform across the block).
template <int BLOCK, int CAP, int U, typename KeyAt, typename JAt, typename Pred>
__device__ __forceinline__ void compact(TopkShared<BLOCK, CAP>& sh, KeyAt key_at, JAt j_at,
                                        Pred pred, int& nsel, int& ncand) {
  constexpr int NW = BLOCK / 64;
  const int lane = lane_id(), wave = int(threadIdx.x) >> 6;
  static_assert(U <= 32, "2-bit class mask holds 32 entries");
  using Mask = typename std::conditional<(U > 16), uint64_t, uint32_t>::type;
  int packed = 0;  // selection hits in the low 16 bits, candidate hits above
  Mask cls = 0u;   // 2 bits per entry: 1 = selection, 2 = candidate list
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = pred(key_at(u), j_at(u));
    cls |= Mask(c) << (2 * u);
    packed += c == 1 ? 1 : (c == 2 ? 0x10000 : 0);
  }
  const int incl = wave_incl_scan(packed);
  if (lane == 63) {
    sh.wsel[wave] = incl & 0xFFFF;
    sh.wcand[wave] = incl >> 16;
  }
  __syncthreads();
  int bs = nsel + ((incl - packed) & 0xFFFF), bc = ncand + ((incl - packed) >> 16);
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int a = sh.wsel[w], c = sh.wcand[w];
    if (w < wave) {
      bs += a;
      bc += c;
    }
    nsel += a;
    ncand += c;
  }
  if (cls != 0u) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t c = uint32_t(cls >> (2 * u)) & 3u;
      if (c == 1u) {
        if (bs < kMaxTopk) sh.sel[bs] = (uint64_t(key_at(u)) << 32) | uint64_t(~j_at(u));
        ++bs;
      } else if (c == 2u) {
        if (bc < CAP) {
          sh.ckey[bc] = key_at(u);
          sh.cj[bc] = j_at(u);
        }
        ++bc;
      }
    }
  }
  __syncthreads();  // wsel / wcand are rewritten by the next call
}

// Running threshold: a key is taken when (key >> shift) > thr, or equals thr
// with j <= jcut. `need` is how many of the keys equal to thr (at this
// resolution) are still to be taken.
struct Cut {
  int shift;
  uint32_t thr;
  uint32_t jcut;
  int need;
  bool settled;
};

// One radix pass over a source of (key, j): histogram of key bits
// [sft, sft+width) among keys whose bits above sft+width equal cut.thr,
// then refine the cut. `each(f)` calls f(key, j) for every element.
template <int BLOCK, int CAP, typename Each>
__device__ __forceinline__ void key_pass(TopkShared<BLOCK, CAP>& sh, Cut& cut, int sft, int width, Each each) {
  const uint32_t hi_thr = cut.thr;
  const int hi_shift = sft + width;
  const uint32_t mask = (1u << width) - 1u;
  clear_hist(sh, kBins);
  __syncthreads();
  each([&](uint32_t key, uint32_t) {
    if (key != 0u && (hi_shift >= 32 || (key >> hi_shift) == hi_thr))
      atomicAdd(&sh.hist[(key >> sft) & mask], 1u);
  });
  __syncthreads();
  if (threadIdx.x < 64) {
    if (width == 11)
      find_bin<2048>(sh, cut.need, true);
    else
      find_bin<1024>(sh, cut.need, true);
  }
  __syncthreads();
  cut.thr = (hi_shift >= 32 ? 0u : (hi_thr << width)) | uint32_t(sh.digit);
  cut.shift = sft;
  cut.need -= sh.above;
  cut.settled = sh.at == cut.need;
  __syncthreads();
}

// Radix pass over j (ascending) among keys equal to `full` (shift 0).
template <int BLOCK, int CAP, typename Each>
__device__ __forceinline__ void j_pass(TopkShared<BLOCK, CAP>& sh, uint32_t full, uint32_t& jpre, int& need,
                       int sft, int width, Each each) {
  const int hi_shift = sft + width;
  const uint32_t mask = (1u << width) - 1u;
  clear_hist(sh, kBins);
  __syncthreads();
  each([&](uint32_t key, uint32_t j) {
    if (key == full && (hi_shift >= 32 || (j >> hi_shift) == jpre))
      atomicAdd(&sh.hist[(j >> sft) & mask], 1u);
  });
  __syncthreads();
  if (threadIdx.x < 64) {
    if (width == 11)
      find_bin<2048>(sh, need, false);
    else
      find_bin<1024>(sh, need, false);
  }
  __syncthreads();
  jpre = (hi_shift >= 32 ? 0u : (jpre << width)) | uint32_t(sh.digit);
  need -= sh.above;
  __syncthreads();
}

// Finish a cut over a source: remaining key bits below cut.shift, then j.
template <int BLOCK, int CAP, typename Each>
__device__ __forceinline__ void finish_cut(TopkShared<BLOCK, CAP>& sh, Cut& cut, Each each) {
  if (!cut.settled && cut.shift == 21) key_pass(sh, cut, 10, 11, each);
  if (!cut.settled && cut.shift == 10) key_pass(sh, cut, 0, 10, each);
  if (!cut.settled) {  // ties on the full key: the `need` lowest j
    uint32_t jpre = 0u;
    int need = cut.need;
    j_pass(sh, cut.thr, jpre, need, 21, 11, each);
    j_pass(sh, cut.thr, jpre, need, 10, 11, each);
    j_pass(sh, cut.thr, jpre, need, 0, 10, each);
    cut.jcut = jpre;
  }
}

__device__ __forceinline__ bool taken(const Cut& c, uint32_t key, uint32_t j) {
  const uint32_t h = key >> c.shift;
  return key != 0u && (h > c.thr || (h == c.thr && j <= c.jcut));
}

// Select the winners of a row into sh.sel, unsorted; nsel counts them. That
// is min(k, n) entries, or, when the whole threshold bucket fits, every
// entry at or above it (at least k), to be cut to k by the sort.
// `chunks(g)` calls g(key_at, j_at) per chunk of BLOCK*U entries, with
// key_at(u) / j_at(u) giving this thread's entry u (key 0 = no entry) and
// the same number of chunks on every thread.
template <int BLOCK, int CAP, int U, typename Chunks>
__device__ __forceinline__ void select_row(TopkShared<BLOCK, CAP>& sh, int n, int k, Chunks chunks,
                                           int& nsel) {
  auto each_src = [&](auto f) {
    chunks([&](auto key_at, auto j_at) {
#pragma unroll
      for (int u = 0; u < U; ++u) f(key_at(u), j_at(u));
    });
  };
  const int tid = threadIdx.x;
  int ncand = 0;
  if (n > k) {
    // A: top 11 bits over the whole row
    Cut cut{32, 0u, 0xFFFFFFFFu, k, false};
    key_pass(sh, cut, 21, 11, each_src);
    const int above = k - cut.need, at = sh.at;
    if (!cut.settled && above + at <= kMaxTopk) {
      // B': everything at or above b* goes to the selection; the sort orders
      // it by (key desc, j asc) and the row keeps the first k, which is
      // exactly the cut C would find
      const uint32_t b = cut.thr;
      chunks([&](auto key_at, auto j_at) {
        compact<BLOCK, CAP, U>(sh, key_at, j_at,
                               [&](uint32_t kv, uint32_t) { return kv != 0u && (kv >> 21) >= b ? 1 : 0; },
                               nsel, ncand);
      });
      return;
    }
    if (cut.settled || at <= CAP) {
      // B: above b* -> selection, in b* -> candidate list
      const Cut bucket = cut;
      chunks([&](auto key_at, auto j_at) {
        compact<BLOCK, CAP, U>(sh, key_at, j_at, [&](uint32_t kv, uint32_t) {
          const uint32_t h = kv >> 21;
          if (kv == 0u) return 0;
          if (h > bucket.thr || (bucket.settled && h == bucket.thr)) return 1;
          return (!bucket.settled && h == bucket.thr) ? 2 : 0;
        }, nsel, ncand);
      });
      if (!cut.settled) {
        // C: finish the cut on the candidate list
        const int nc = ncand;
        auto each_cand = [&](auto f) {
          for (int i = tid; i < nc; i += BLOCK) f(sh.ckey[i], sh.cj[i]);
        };
        finish_cut(sh, cut, each_cand);
        for (int base = 0; base < nc; base += BLOCK) {
          const int i = base + tid;
          const bool in = i < nc;
          const uint32_t ck = in ? sh.ckey[i] : 0u, cj = in ? sh.cj[i] : 0u;
          int dummy = 0;
          compact<BLOCK, CAP, 1>(sh, [&](int) { return ck; }, [&](int) { return cj; },
                                 [&](uint32_t kv, uint32_t jv) { return taken(cut, kv, jv) ? 1 : 0; },
                                 nsel, dummy);
        }
      }
    } else {
      // heavy ties in b*: finish the cut over the whole row, then select
      finish_cut(sh, cut, each_src);
      chunks([&](auto key_at, auto j_at) {
        compact<BLOCK, CAP, U>(sh, key_at, j_at,
                               [&](uint32_t kv, uint32_t jv) { return taken(cut, kv, jv) ? 1 : 0; },
                               nsel, ncand);
      });
    }
  } else {
    __syncthreads();
    chunks([&](auto key_at, auto j_at) {
      compact<BLOCK, CAP, U>(sh, key_at, j_at, [](uint32_t kv, uint32_t) { return kv != 0u ? 1 : 0; },
                             nsel, ncand);
    });
  }
}

// ---------------------------------------------------------------------------
// Bucket path: one histogram both finds the threshold and orders the winners.

// Keys of finite scores (-inf maps to 0x007FFFFF, +inf to 0xFF800000).
__device__ __forceinline__ bool finite_key(uint32_t key) {
  return key > 0x007FFFFFu && key < 0xFF800000u;
}

// Bin of a key, linear in the score over the row's finite range [lo, hi]
// (s = NB / (hi - lo)); +-inf clamp to the end bins. Subtraction,
// multiplication by s >= 0 and truncation all preserve order, so a larger
// key never lands in a lower bin, which is all the selection relies on.
// s = 0 (no finite range) sends every finite key to bin 0.
template <int NB>
struct LinearBins {
  float lo, s;
  __device__ __forceinline__ int operator()(uint32_t key) const {
    const float t = (key_value(key) - lo) * s;
    return t >= float(NB - 1) ? NB - 1 : (t > 0.f ? int(t) : 0);
  }
};
using ValueBins = LinearBins<kBins>;

// Turn the bin counts in hist into descending exclusive starts (entries in
// higher bins) in place, and find the threshold bin b*: the bin holding the
// need-th largest entry, need = min(k, entries). Leaves sh.digit = b* and
// sh.at = entries in bins >= b* (b* = kBins and 0 when there are no
// entries). Run by the whole block (every thread calls it): thread t holds
// kBins/BLOCK consecutive bins, thread 0 the top ones; a wave prefix sum, one
// barrier and the totals of the waves above give each thread its first
// start. Exactly one thread holds b*.
template <int BLOCK, int CAP>
__device__ __forceinline__ void scan_desc_block(TopkShared<BLOCK, CAP>& sh, int k) {
  constexpr int NW = BLOCK / 64;
  constexpr int PER = kBins / BLOCK;
  static_assert(PER >= 1 && kBins % BLOCK == 0, "bins per thread");
  const int tid = threadIdx.x, wave = tid >> 6;
  const int base = kBins - (tid + 1) * PER;  // thread 0 holds the top bins
  uint32_t c[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) c[i] = sh.hist[base + i];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) sum += int(c[i]);
  const int incl = wave_incl_scan(sum);
  if (lane_id() == 63) sh.wtot[wave] = incl;
  __syncthreads();
  int above = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int t = sh.wtot[w];
    above += w < wave ? t : 0;
    total += t;
  }
  const int need = min(k, total);
  int run = above + incl - sum, found = -1, upto = 0;
#pragma unroll
  for (int o = 0; o < PER; ++o) {  // descending bin order within the thread
    const int i = PER - 1 - o;
    const int cnt = int(c[i]);
    c[i] = uint32_t(run);
    run += cnt;
    if (found < 0 && run - cnt < need && run >= need) {
      found = base + i;
      upto = run;
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) sh.hist[base + i] = c[i];
  if (found >= 0) {
    sh.digit = found;
    sh.at = upto;
  }
  if (need == 0 && tid == 0) {
    sh.digit = kBins;
    sh.at = 0;
  }
}

// Range, histogram and scan over U entries per thread (key_at(u), key 0 =
// no entry; entries u >= nu, a uniform count, are all empty and skipped).
// Returns the bin map and each entry's bin in bin[u] (-1 for none);
// afterwards hist holds the bins' descending starts and sh.digit / sh.at
// the threshold bin and the number of entries at or above it.
template <int BLOCK, int CAP, int U, typename KeyAt>
__device__ __forceinline__ ValueBins bucket_threshold(TopkShared<BLOCK, CAP>& sh, KeyAt key_at, int k, int nu,
                                                      int (&bin)[U]) {
  constexpr int NW = BLOCK / 64;
  const int lane = lane_id(), wave = int(threadIdx.x) >> 6;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (u >= nu) break;
    const uint32_t kv = key_at(u);
    if (finite_key(kv)) {
      mn = min(mn, kv);
      mx = max(mx, kv);
    }
  }
  wave_min_max(mn, mx);
  if (lane == 0) {
    sh.wlo[wave] = mn;
    sh.whi[wave] = mx;
  }
  clear_hist(sh, kBins);
  __syncthreads();
  mn = 0xFFFFFFFFu;
  mx = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    mn = min(mn, sh.wlo[w]);
    mx = max(mx, sh.whi[w]);
  }
  ValueBins bins{0.f, 0.f};
  if (mn <= mx) {
    bins.lo = key_value(mn);
    const float range = key_value(mx) - bins.lo;
    bins.s = range > 0.f ? float(kBins) / range : 0.f;  // an overflowed range gives 0
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    bin[u] = -1;
    if (u >= nu) continue;
    const uint32_t kv = key_at(u);
    if (kv != 0u) {
      bin[u] = bins(kv);
      atomicAdd(&sh.hist[bin[u]], 1u);
    }
  }
  __syncthreads();
  scan_desc_block(sh, k);
  __syncthreads();
  return bins;
}

// Exact top-k of entries held U per thread (key_at(u), j_at(u), key 0 = no
// entry), written to orow in (score desc, j asc) order, -1 past the last
// entry. Every entry in a bin at or above b* is scattered to its bin's
// slots (b*'s bins hold the k-th largest, so these are the winners plus the
// rest of b*), hist[b] serving as bin b's cursor: afterwards hist[b] is the
// end of bin b and hist[b + 1] its start (bins above b* are all filled).
// An entry's rank inside its bin is counted by comparison, so the result
// does not depend on the order of the atomics. Returns false,
// having written nothing, when those bins hold more than kMaxTopk entries
// (scores crowded into a few bins: heavy ties, far outliers).
template <int BLOCK, int CAP, int U, typename KeyAt, typename JAt>
__device__ __forceinline__ bool bucket_topk(TopkShared<BLOCK, CAP>& sh, KeyAt key_at, JAt j_at,
                                            int k, int32_t* __restrict__ orow, int nu = U) {
  const int tid = threadIdx.x;
  int bin[U];
  const ValueBins bins = bucket_threshold<BLOCK, CAP, U>(sh, key_at, k, nu, bin);
  const int bstar = sh.digit, m = sh.at;
  if (m > kMaxTopk) return false;  // uniform
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (bin[u] >= bstar) {
      const uint32_t pos = atomicAdd(&sh.hist[bin[u]], 1u);
      sh.sel[pos] = (uint64_t(key_at(u)) << 32) | uint64_t(~j_at(u));
    }
  }
  __syncthreads();
  for (int p = tid; p < m; p += BLOCK) {
    const uint64_t e = sh.sel[p];
    const int b = bins(uint32_t(e >> 32));
    const int start = b == kBins - 1 ? 0 : int(sh.hist[b + 1]);
    const int end = int(sh.hist[b]);
    int rank = 0;
    for (int q = start; q < end; ++q) rank += sh.sel[q] > e ? 1 : 0;
    if (start + rank < k) orow[start + rank] = int32_t(~uint32_t(e & 0xFFFFFFFFull));
  }
  for (int p = m + tid; p < k; p += BLOCK) orow[p] = -1;
  return true;
}

// Append a list (entries [0, nc) of ckey/cj) to the selection: the k winners
// when nc > k, else all of them.
template <int BLOCK, int CAP>
__device__ __forceinline__ void select_list(TopkShared<BLOCK, CAP>& sh, int nc, int k, int& nsel) {
  const int tid = threadIdx.x;
  auto each_list = [&](auto f) {
    for (int i = tid; i < nc; i += BLOCK) f(sh.ckey[i], sh.cj[i]);
  };
  Cut cut{0, 0u, 0xFFFFFFFFu, 0, true};  // takes every entry
  if (nc > k) {
    cut = Cut{32, 0u, 0xFFFFFFFFu, k, false};
    key_pass(sh, cut, 21, 11, each_list);
    finish_cut(sh, cut, each_list);
  }
  for (int base = 0; base < nc; base += BLOCK) {
    const int i = base + tid;
    const bool in = i < nc;
    const uint32_t ck = in ? sh.ckey[i] : 0u, cj = in ? sh.cj[i] : 0u;
    int dummy = 0;
    compact<BLOCK, CAP, 1>(sh, [&](int) { return ck; }, [&](int) { return cj; },
                           [&](uint32_t kv, uint32_t jv) { return in && taken(cut, kv, jv) ? 1 : 0; },
                           nsel, dummy);
  }
}

// Row scores through a range-checked buffer descriptor (make_rsrc over the
// row's first `len` scores): a load past the end reads 0 with no memory
// access and no branch, so every load of a loop is issued unconditionally
// and the compiler's wait counts stay exact (a load inside a branch is
// waited for right there, which serialises a row's loads).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const float* row, int len) {
  return make_rsrc(row, len * 4);
}

__device__ __forceinline__ float load_score(__amdgpu_buffer_rsrc_t rs, int j) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, j * 4, 0, 0));
}

// Entry u of this thread in the chunk of BLOCK*U entries starting at base:
// base + BLOCK*u + tid, or with Q4 (16-byte loads: 4 consecutive entries per
// load) base + 4*BLOCK*(u/4) + 4*tid + u%4.
template <int BLOCK, bool Q4>
__device__ __forceinline__ int chunk_j(int base, int u) {
  return Q4 ? base + 4 * BLOCK * (u >> 2) + 4 * int(threadIdx.x) + (u & 3) : base + BLOCK * u + int(threadIdx.x);
}

// Loads of the chunk of BLOCK*U entries starting at base (entry u at
// chunk_j). Q4 needs the row 16-byte aligned, base a multiple of 4 and rs
// covering whole quads.
template <int BLOCK, int U, bool Q4 = false>
__device__ __forceinline__ void load_chunk(__amdgpu_buffer_rsrc_t rs, int base, float (&c)[U]) {
  if constexpr (Q4) {
    static_assert(U % 4 == 0, "whole quads");
#pragma unroll
    for (int i = 0; i < U / 4; ++i) {
      // Non-temporal: each score is read once; caching it only evicts lines still in use.
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, chunk_j<BLOCK, true>(base, 4 * i) * 4, 0, 2);
#pragma unroll
      for (int e = 0; e < 4; ++e) c[4 * i + e] = __uint_as_float(v[e]);
    }
  } else {
#pragma unroll
    for (int u = 0; u < U; ++u) c[u] = load_score(rs, chunk_j<BLOCK, false>(base, u));
  }
}

// g(scores, base) over chunks of entries [j_lo, j_hi) of the row streamed
// from memory (entry u of this thread is j = base + BLOCK*u + tid; the
// caller masks j >= j_hi), BLOCK*U per chunk, three register buffers in
// rotation: two chunks' loads are in flight while one is processed. `c0`
// and `c1` hold the first two chunks' loads (load_chunk at j_lo and
// j_lo + BLOCK*U), issued by the caller as early as it likes; rs covers at
// least [0, j_hi) (and reads 0 past its end). Each iteration processes
// three chunks unconditionally (entries past j_hi are masked): with no exit
// between a load and its use, the compiler issues the loads where they
// stand instead of next to their use.
template <int BLOCK, int U, int NBUF, bool Q4, typename G>
__device__ __forceinline__ void stream_chunks(__amdgpu_buffer_rsrc_t rs, int j_lo, int j_hi, float (&c0)[U],
                                              float (&c1)[U], G g) {
  static_assert(NBUF == 2 || NBUF == 3, "two or three buffers");
  constexpr int C = BLOCK * U;
  if constexpr (NBUF == 3) {
    float c2[U];
    for (int base = j_lo; base < j_hi; base += 3 * C) {
      load_chunk<BLOCK, U, Q4>(rs, base + 2 * C, c2);
      g(c0, base);
      load_chunk<BLOCK, U, Q4>(rs, base + 3 * C, c0);
      g(c1, base + C);
      load_chunk<BLOCK, U, Q4>(rs, base + 4 * C, c1);
      g(c2, base + 2 * C);
    }
  } else {  // c1 unused: one chunk in flight while one is processed
    float nxt[U];
    for (int base = j_lo; base < j_hi; base += 2 * C) {
      load_chunk<BLOCK, U, Q4>(rs, base + C, nxt);
      g(c0, base);
      load_chunk<BLOCK, U, Q4>(rs, base + 2 * C, c0);
      g(nxt, base + C);
    }
  }
}

// Order the selection sh.sel[0..nsel) (at most kMaxTopk entries, at least
// min(k, valid keys)) and write the first k: the entries move to registers
// and go through the bucket path, which always succeeds on so few entries.
template <int BLOCK, int CAP>
__device__ __forceinline__ void sort_selection(TopkShared<BLOCK, CAP>& sh, int nsel, int k,
                                               int32_t* __restrict__ orow) {
  constexpr int PER = kMaxTopk / BLOCK;
  const int tid = threadIdx.x;
  uint32_t sk[PER], sj[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int p = tid + BLOCK * i;
    const uint64_t e = p < nsel ? sh.sel[p] : 0ull;
    sk[i] = uint32_t(e >> 32);
    sj[i] = ~uint32_t(e & 0xFFFFFFFFull);
  }
  bucket_topk<BLOCK, CAP, PER>(sh, [&](int i) { return sk[i]; }, [&](int i) { return sj[i]; }, k, orow);
}

// Radix path over the whole row, re-read from memory chunk by chunk (rows
// whose scores crowd into a few bins, where the bucket path gives up). It
// is rare, so it is kept lean in registers rather than fast.
template <int BLOCK, int CAP>
__device__ __forceinline__ void radix_topk(TopkShared<BLOCK, CAP>& sh, const float* __restrict__ x,
                                           int n, int k, int32_t* __restrict__ orow) {
  constexpr int U = 2;
  const auto rs = row_rsrc(x, n);
  auto all_chunks = [&](auto g) {
    for (int base = 0; base < n; base += BLOCK * U) {
      uint32_t kv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = base + BLOCK * u + int(threadIdx.x);
        kv[u] = j < n ? order_key(load_score(rs, j)) : 0u;
      }
      g([&](int u) { return kv[u]; }, [&](int u) { return uint32_t(base + BLOCK * u + int(threadIdx.x)); });
    }
  };
  int nsel = 0;
  select_row<BLOCK, CAP, U>(sh, n, k, all_chunks, nsel);
  sort_selection(sh, nsel, k, orow);
}

// Rows of at most BLOCK*V keys: the row is read once into V registers per
// thread (j = tid + BLOCK*v). Rows run last to first: under a causal limit
// the longest rows are the last ones, and starting them first leaves the
// short rows to fill the end of the grid.
template <int BLOCK, int V, int CAP>
__global__ __launch_bounds__(BLOCK) void topk_kernel(const float* __restrict__ logits,
                                                     const int32_t* __restrict__ limit,
                                                     int32_t* __restrict__ idx, int R, int K, int k) {
  __shared__ TopkShared<BLOCK, CAP> sh;
  const int tid = threadIdx.x;
  // Row r runs on XCD r % 8 (workgroup i runs on XCD i % 8), where the
  // gather of its selection runs too, so the indices it reads are in that
  // XCD's L2; groups of eight rows go last to first (the longest rows first
  // under a causal limit). The grid is R rounded up to whole groups.
  const int64_t row = (int64_t(gridDim.x / 8) - 1 - blockIdx.x / 8) * 8 + blockIdx.x % 8;
  if (row >= R) return;  // uniform
  const float* x = logits + row * K;
  float raw[V];  // issued before the limit arrives; keys past it are masked below
  load_chunk<BLOCK, V>(row_rsrc(x, K), 0, raw);
  const int n = limit ? max(0, min(limit[row], K - 1) + 1) : K;
  uint32_t key[V];
#pragma unroll
  for (int v = 0; v < V; ++v) key[v] = tid + BLOCK * v < n ? order_key(raw[v]) : 0u;
  auto key_at = [&](int v) { return key[v]; };
  auto j_at = [&](int v) { return uint32_t(tid + BLOCK * v); };
  // register chunks wholly past the row's end are skipped (causal rows)
  if (bucket_topk<BLOCK, CAP, V>(sh, key_at, j_at, k, idx + row * k, (n + BLOCK - 1) / BLOCK)) return;
  radix_topk<BLOCK, CAP>(sh, x, n, k, idx + row * k);
}

// ---------------------------------------------------------------------------
// Many short rows (prefill under a causal limit): one wave per row and no
// barrier on the common path. The row sits in V registers per lane (16-byte
// loads, j = 256*i + 4*lane + c). A wave64 VALU instruction holds its SIMD
// for four cycles and LDS atomics contend across the CU, so the wave first
// narrows the row in registers:
//  1. A bound tau with C(tau) = #{scores >= tau} >= min(k, n). The first
//     probe is the normal quantile, at the wanted tail fraction, of the mean
//     and variance of every fourth key; further probes are false position on the exact
//     counts (one compare and add per entry and a wave sum), until C(tau) is
//     a little above k. Every winner scores >= the k-th largest >= tau.
//  2. The C(tau) candidates go to a wave-private LDS list (raw score bits
//     and ~j), each lane's run placed by a wave prefix sum of the lanes'
//     counts, with no atomics.
//  3. The bucket path on the list: kWaveBins bins linear in the score over
//     the candidates' range, a histogram and one descending scan in
//     registers give the bin b* that holds the k-th largest; the entries of
//     bins >= b* are scattered to their bins' slots through atomic cursors
//     (issued back to back: lanes without an entry count into a private
//     dummy) and ranked inside their bin by comparison, so the output does
//     not depend on atomic order.
// LDS operations of one wave complete in program order, so the phases need
// no barrier. A row with more than kWaveCand candidates after the search
// (scores crowded by heavy ties, infinities) is left to the radix path,
// which the whole workgroup runs on it after one barrier, in the same LDS.
constexpr int kWaveBins = 512;
constexpr int kWaveCand = 896;   // candidate entries per wave
constexpr int kWaveRows = 4;     // rows (waves) per workgroup
constexpr int kWaveMaxK = 512;   // k for which the wave path is used
constexpr int kWaveFallbackCap = 256;
constexpr int kWaveSearchSteps = 6;

struct WaveRowShared {
  __attribute__((aligned(16))) uint32_t hist[kWaveBins + 64];  // + a dummy counter per lane
  uint64_t cand[kWaveCand];  // the candidates, then the bin slots of the selection
};
constexpr size_t kWaveSmem = std::max(sizeof(WaveRowShared) * kWaveRows,
                                      sizeof(TopkShared<64 * kWaveRows, kWaveFallbackCap>));

__device__ __forceinline__ int wave_sum(int v) { return __builtin_amdgcn_readlane(wave_incl_scan(v), 63); }

// Sum over the wave, uniform result (butterflies in each row of 16 lanes,
// then the four row sums read as scalars).
__device__ __forceinline__ float wave_fsum(float v) {
#define XK_ADD_DPP(C) v += __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), C, 0xF, 0xF, false));
  XK_ADD_DPP(kDppQuadSwap1)
  XK_ADD_DPP(kDppQuadSwap2)
  XK_ADD_DPP(kDppHalfMirror)
  XK_ADD_DPP(kDppRowMirror)
#undef XK_ADD_DPP
  const auto at = [&](int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); };
  return (at(0) + at(16)) + (at(32) + at(48));
}

// Upper-tail normal quantile: z with P(Z > z) = p, 0 < p < 1, by the
// rational approximation of Abramowitz and Stegun (Handbook of Mathematical
// Functions, formula 26.2.23; absolute error below 4.5e-4). It only seeds
// the threshold search, so its accuracy affects speed, not results.
__device__ __forceinline__ float normal_upper_quantile(float p) {
  const bool upper = p <= 0.5f;
  const float q = upper ? p : 1.f - p;
  const float t = sqrtf(-2.f * __logf(q));
  const float num = fmaf(fmaf(0.010328f, t, 0.802853f), t, 2.515517f);
  const float den = fmaf(fmaf(fmaf(0.001308f, t, 0.189269f), t, 1.432788f), t, 1.f);
  const float z = t - num / den;
  return upper ? z : -z;
}

// Descending exclusive starts of the bins in place (entries in higher bins),
// the threshold bin b* (holding the need-th largest entry, need = min(k,
// entries)) and m, the entries in bins >= b*; b* = kWaveBins and m = 0 for
// a row with no entry. Lane 0 holds the top bins.
__device__ __forceinline__ void wave_scan_desc(uint32_t* hist, int k, int& bstar, int& m) {
  constexpr int PER = kWaveBins / 64;
  static_assert(PER % 4 == 0, "bins per lane");
  const int lane = lane_id();
  const int base = kWaveBins - (lane + 1) * PER;
  uint32_t c[PER];
#pragma unroll
  for (int i = 0; i < PER / 4; ++i) {
    const u32x4 q4 = *reinterpret_cast<const u32x4*>(&hist[base + 4 * i]);
#pragma unroll
    for (int e = 0; e < 4; ++e) c[4 * i + e] = q4[e];
  }
  int sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) sum += int(c[i]);
  const int incl = wave_incl_scan(sum);
  const int need = min(k, __builtin_amdgcn_readlane(incl, 63));
  int run = incl - sum, found = -1, upto = 0;
#pragma unroll
  for (int o = 0; o < PER; ++o) {
    const int i = PER - 1 - o;
    const int cnt = int(c[i]);
    c[i] = uint32_t(run);
    run += cnt;
    if (found < 0 && run - cnt < need && run >= need) {
      found = base + i;
      upto = run;
    }
  }
#pragma unroll
  for (int i = 0; i < PER / 4; ++i)
    *reinterpret_cast<u32x4*>(&hist[base + 4 * i]) = u32x4{c[4 * i], c[4 * i + 1], c[4 * i + 2], c[4 * i + 3]};
  const uint64_t fm = __ballot(found >= 0);
  if (fm == 0ull) {
    bstar = kWaveBins;
    m = 0;
  } else {
    const int src = __builtin_ctzll(fm);
    bstar = __builtin_amdgcn_readlane(found, src);
    m = __builtin_amdgcn_readlane(upto, src);
  }
}

// One row by one wave; returns false, having written nothing, when the
// row keeps more than kWaveCand candidates. K % 4 == 0 and the row 16-byte
// aligned (the launcher checks).
template <int V>
__device__ __forceinline__ bool wave_row_topk(WaveRowShared& sh, const float* __restrict__ x, int n, int k,
                                              int32_t* __restrict__ orow) {
  constexpr int G = V / 4;                   // 16-byte loads per lane
  constexpr int U = (kWaveCand + 63) / 64;   // list entries per lane
  const int lane = lane_id();
  const auto rs = make_rsrc(x, ((n + 3) & ~3) * 4);  // whole quads: reads stay inside the row
  float xs[V];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const u32x4 r = __builtin_amdgcn_raw_buffer_load_b128(rs, (256 * i + 4 * lane) * 4, 0, 2);  // read once: non-temporal
#pragma unroll
    for (int c = 0; c < 4; ++c) xs[4 * i + c] = __uint_as_float(r[c]);
  }
  // Every loop below runs over all G groups with a uniform test, so xs stays
  // in registers: groups >= ng hold no entry and are skipped, and the one
  // group straddling the row's end tests each entry's index. (Writing NaN
  // into that group instead made the compiler copy row registers across the
  // uniform branches and spill four of them, reloaded in every search probe.)
  // The mean and variance only seed the search's first probe, so they come
  // from every fourth key (j % 4 == 0): half the VALU of the full sums
  // (measured 25.4 -> 24.2 us on the causal 4096-key rows, same indices).
  const int ng = (n + 255) >> 8, nfull = n >> 8;
  float mn = INFINITY, mx = -INFINITY, s1 = 0.f, s2 = 0.f;
#pragma unroll
  for (int i = 0; i < G; ++i) {
    if (i < nfull) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float v = xs[4 * i + c];
        mn = fminf(mn, v);
        mx = fmaxf(mx, v);
        if (c == 0) {
          s1 += v;
          s2 = fmaf(v, v, s2);
        }
      }
    } else if (i < ng) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bool in = 256 * i + 4 * lane + c < n;
        const float v = in ? xs[4 * i + c] : 0.f;
        if (in) {
          mn = fminf(mn, v);
          mx = fmaxf(mx, v);
        }
        if (c == 0) {
          s1 += v;
          s2 = fmaf(v, v, s2);
        }
      }
    }
  }
  const float n_sampled = float((n + 3) >> 2);  // keys j < n with j % 4 == 0
  auto count_lane = [&](float t) {
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      if (i < nfull) {
#pragma unroll
        for (int c = 0; c < 4; ++c) cnt += xs[4 * i + c] >= t ? 1 : 0;
      } else if (i < ng) {
#pragma unroll
        for (int c = 0; c < 4; ++c) cnt += xs[4 * i + c] >= t && 256 * i + 4 * lane + c < n ? 1 : 0;
      }
    }
    return cnt;
  };
  // 1. the bound tau (c = C(tau), mine = this lane's part of it)
  const int need = min(k, n);
  const int goal = min(need + (need >> 2) + 32, kWaveCand);
  float tau = -INFINITY;
  int c = n, mine = -1;
  uint32_t kmn = order_key(mn), kmx = order_key(mx);
  wave_min_max(kmn, kmx);
  if (c > goal && finite_key(kmn) && finite_key(kmx) && kmn < kmx) {
    float lo = key_value(kmn), hi = key_value(kmx);
    int clo = n, chi = 1;  // estimates until measured; they only steer the probes
    const float aim = float((need + goal) >> 1);
    const float mean = wave_fsum(s1) / n_sampled;
    const float var = fmaxf(wave_fsum(s2) / n_sampled - mean * mean, 0.f);
    float t = fmaf(sqrtf(var), normal_upper_quantile(aim / float(n)), mean);
#pragma unroll 1
    for (int step = 0; step < kWaveSearchSteps; ++step) {
      if (step > 0 || !(t > lo && t < hi)) {
        // false position on the count, kept inside [1/8, 7/8] of the bracket
        float f = (float(clo) - aim) / float(max(clo - chi, 1));
        f = fminf(fmaxf(f, 0.125f), 0.875f);
        t = fmaf(f, hi, fmaf(-f, lo, lo));  // lo + f (hi - lo), no overflow
        if (!(t > lo && t < hi)) break;     // the bracket cannot shrink
      }
      const int cl = count_lane(t);
      const int ct = wave_sum(cl);
      if (ct >= need) {
        lo = t;
        clo = ct;
        tau = t;
        c = ct;
        mine = cl;
        if (c <= goal) break;
      } else {
        hi = t;
        chi = ct;
      }
    }
  }
  if (c > kWaveCand) return false;  // uniform
  if (mine < 0) mine = count_lane(tau);  // uniform test (tau = -inf: the valid entries)
  // 2. the candidates into the list, each lane's run from a wave prefix sum
  {
    int at = wave_incl_scan(mine) - mine;
#pragma unroll
    for (int i = 0; i < G; ++i)
      if (i < ng) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (xs[4 * i + e] >= tau && (i < nfull || 256 * i + 4 * lane + e < n))
            sh.cand[at++] = (uint64_t(__float_as_uint(xs[4 * i + e])) << 32) |
                            uint64_t(~uint32_t(256 * i + 4 * lane + e));
      }
  }
  // 3. bucket path on the list, held U entries per lane as key << 32 | ~j.
  // The bins span [tau, row maximum] (the row's finite range without a
  // search), which holds every finite candidate; infinities clamp to the end
  // bins. The reads are unconditional (U * 64 == kWaveCand), so no load
  // waits inside a branch.
  static_assert(U * 64 == kWaveCand, "the list fills whole lane rows");
  LinearBins<kWaveBins> bins{0.f, 0.f};
  if (finite_key(kmn) && finite_key(kmx)) {
    bins.lo = tau > -INFINITY ? tau : key_value(kmn);
    const float range = key_value(kmx) - bins.lo;
    bins.s = range > 0.f && range < INFINITY ? float(kWaveBins) / range : 0.f;
  }
  uint64_t ent[U];
  int bin[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint64_t e = sh.cand[64 * u + lane];
    const float f = __uint_as_float(uint32_t(e >> 32));
    const float t = (f - bins.lo) * bins.s;
    ent[u] = (uint64_t(order_key(f)) << 32) | (e & 0xFFFFFFFFull);
    bin[u] = 64 * u + lane < c ? (t >= float(kWaveBins - 1) ? kWaveBins - 1 : (t > 0.f ? int(t) : 0)) : -1;
  }
  static_assert(kWaveBins % 256 == 0, "clear with 16-byte stores");
#pragma unroll
  for (int i = 0; i < kWaveBins / 256; ++i)
    *reinterpret_cast<u32x4*>(&sh.hist[256 * i + 4 * lane]) = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (64 * u < c) atomicAdd(&sh.hist[bin[u] >= 0 ? bin[u] : kWaveBins + lane], 1u);  // uniform test
  int bstar, m;
  wave_scan_desc(sh.hist, k, bstar, m);
  // scatter (the list is in registers, its LDS now holds the bin slots):
  // hist[b] is bin b's cursor; afterwards its end, and hist[b + 1] its start
  // (every bin above b* is full)
  uint32_t pos[U];
#pragma unroll
  for (int u = 0; u < U; ++u)
    pos[u] = 64 * u < c ? atomicAdd(&sh.hist[bin[u] >= bstar ? bin[u] : kWaveBins + lane], 1u) : 0u;
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (64 * u < c && bin[u] >= bstar) sh.cand[pos[u]] = ent[u];
  // each lane ranks its own scattered entries inside their bins (pos now
  // holds each bin's end, start its first slot)
  int start[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int b = max(bin[u], 0);
    pos[u] = sh.hist[b];
    start[u] = b == kWaveBins - 1 ? 0 : int(sh.hist[b + 1]);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (64 * u < c && bin[u] >= bstar) {
      int rank = 0;
      if (int(pos[u]) - start[u] > 1)  // a bin of one entry holds only this one
        for (int q = start[u]; q < int(pos[u]); ++q) rank += sh.cand[q] > ent[u] ? 1 : 0;
      if (start[u] + rank < k) orow[start[u] + rank] = int32_t(~uint32_t(ent[u] & 0xFFFFFFFFull));
    }
  }
  for (int p = m + lane; p < k; p += 64) orow[p] = -1;
  return true;
}

// kWaveRows rows per workgroup, last to first (the longest rows first under
// a causal limit); rows the wave path gives back are finished by the
// workgroup's radix path.
template <int V>
__global__ __launch_bounds__(64 * kWaveRows, 4) void topk_wave_kernel(const float* __restrict__ logits,
                                                                   const int32_t* __restrict__ limit,
                                                                   int32_t* __restrict__ idx, int R, int K,
                                                                   int k) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kWaveSmem];
  __shared__ int redo[kWaveRows];
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
  const int64_t row = int64_t(R) - 1 - (int64_t(blockIdx.x) * kWaveRows + wave);
  int n = 0;
  bool done = true;
  if (row >= 0) {
    n = limit ? max(0, min(limit[row], K - 1) + 1) : K;
    n = __builtin_amdgcn_readfirstlane(n);
    done = wave_row_topk<V>(reinterpret_cast<WaveRowShared*>(smem)[wave], logits + row * K, n, k, idx + row * k);
  }
  if (lane_id() == 0) redo[wave] = done ? -1 : n;
  __syncthreads();
  auto& sh = *reinterpret_cast<TopkShared<64 * kWaveRows, kWaveFallbackCap>*>(smem);
#pragma unroll 1
  for (int w = 0; w < kWaveRows; ++w) {
    const int nw = redo[w];  // uniform over the workgroup
    if (nw < 0) continue;
    const int64_t rw = int64_t(R) - 1 - (int64_t(blockIdx.x) * kWaveRows + w);
    radix_topk<64 * kWaveRows, kWaveFallbackCap>(sh, logits + rw * K, nw, k, idx + rw * k);
    __syncthreads();
  }
}

// Sum of a and of b over the block, uniform (per-wave sums through LDS; the
// two slots of sh.wsum alternate between consecutive calls, so one barrier
// per call suffices).
template <int BLOCK, int CAP>
__device__ __forceinline__ void block_fsum2(TopkShared<BLOCK, CAP>& sh, int slot, float& a, float& b) {
  constexpr int NW = BLOCK / 64;
  const int wave = int(threadIdx.x) >> 6;
  a = wave_fsum(a);
  b = wave_fsum(b);
  if (lane_id() == 0) {
    sh.wsum[slot][0][wave] = a;
    sh.wsum[slot][1][wave] = b;
  }
  __syncthreads();
  a = 0.f;
  b = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    a += sh.wsum[slot][0][w];
    b += sh.wsum[slot][1][w];
  }
}

// A bound tau on V register-held scores per thread (m valid scores in all,
// entry v valid when valid(v)) with C(tau) = #{scores >= tau} in
// [need, goal]: tau is then at most the need-th largest score. The first
// probe is the normal quantile of the scores' mean and variance at the
// wanted tail fraction, later ones false position on the exact counts (as
// in the one-wave-per-row path), at most kSteps probes. Returns false when
// no such tau was found (non-finite or crowded scores).
template <int BLOCK, int CAP, int V, typename Valid>
__device__ __forceinline__ bool count_threshold(TopkShared<BLOCK, CAP>& sh, const float (&x)[V], Valid valid, int m,
                                                int need, int goal, float& tau) {
  constexpr int kSteps = 8;
  float s1 = 0.f, s2 = 0.f;
  uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const uint32_t kv = order_key(x[v]);
    if (valid(v) && finite_key(kv)) {
      s1 += x[v];
      s2 = fmaf(x[v], x[v], s2);
      kmn = min(kmn, kv);
      kmx = max(kmx, kv);
    }
  }
  wave_min_max(kmn, kmx);
  {
    const int wave = int(threadIdx.x) >> 6;
    if (lane_id() == 0) {
      sh.wlo[wave] = kmn;
      sh.whi[wave] = kmx;
    }
  }
  block_fsum2(sh, 0, s1, s2);  // its barrier also publishes wlo / whi
#pragma unroll
  for (int w = 0; w < BLOCK / 64; ++w) {
    kmn = min(kmn, sh.wlo[w]);
    kmx = max(kmx, sh.whi[w]);
  }
  if (!(finite_key(kmn) && finite_key(kmx) && kmn < kmx)) return false;
  float lo = key_value(kmn), hi = key_value(kmx);
  int clo = m, chi = 1;
  const float aim = float((need + goal) >> 1);
  const float mean = s1 / float(m);
  const float var = fmaxf(s2 / float(m) - mean * mean, 0.f);
  float t = fmaf(sqrtf(var), normal_upper_quantile(aim / float(m)), mean);
#pragma unroll 1
  for (int step = 0; step < kSteps; ++step) {
    if (step > 0 || !(t > lo && t < hi)) {
      float f = (float(clo) - aim) / float(max(clo - chi, 1));
      f = fminf(fmaxf(f, 0.125f), 0.875f);
      t = fmaf(f, hi, fmaf(-f, lo, lo));
      if (!(t > lo && t < hi)) return false;  // uniform: the bracket cannot shrink
    }
    float cl = 0.f, unused = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v) cl += valid(v) && x[v] >= t ? 1.f : 0.f;
    block_fsum2(sh, 1 - (step & 1), cl, unused);
    const int ct = int(cl);
    if (ct >= need) {
      lo = t;
      clo = ct;
      if (ct <= goal) {
        tau = t;
        return true;
      }
    } else {
      hi = t;
      chi = ct;
    }
  }
  return false;
}

// count_threshold for entries that all lie inside the row (a long row's
// prefix): no validity test per entry, the range from float min / max
// (v_min3 / v_max3), and the first probe's mean and variance from every
// fourth entry. A prefix with a non-finite score (or NaN) goes through
// count_threshold, which keeps such scores out of the range and moments.
template <int BLOCK, int CAP, int V>
__device__ __forceinline__ bool count_threshold_dense(TopkShared<BLOCK, CAP>& sh, const float (&x)[V], int m,
                                                      int need, int goal, float& tau) {
  constexpr int kSteps = 8;
  static_assert(V % 4 == 0, "sampled moments take entries 0, 4, 8, ...");
  float mn = INFINITY, mx = -INFINITY, s1 = 0.f, s2 = 0.f;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    mn = fminf(mn, x[v]);
    mx = fmaxf(mx, x[v]);
    if (v % 4 == 0) {
      s1 += x[v];
      s2 = fmaf(x[v], x[v], s2);
    }
  }
  // NaN (outside the contract) or infinities: the careful search
  const bool odd = !(fabsf(mn) < INFINITY && fabsf(mx) < INFINITY && s2 < INFINITY);
  uint32_t kmn = order_key(mn), kmx = order_key(mx);
  wave_min_max(kmn, kmx);
  {
    const int wave = int(threadIdx.x) >> 6;
    const uint64_t any_odd = __ballot(odd);
    if (lane_id() == 0) {
      sh.wlo[wave] = any_odd ? 0u : kmn;  // 0 (below every finite key) flags the wave
      sh.whi[wave] = kmx;
    }
  }
  block_fsum2(sh, 0, s1, s2);  // its barrier also publishes wlo / whi
#pragma unroll
  for (int w = 0; w < BLOCK / 64; ++w) {
    kmn = min(kmn, sh.wlo[w]);
    kmx = max(kmx, sh.whi[w]);
  }
  if (!(finite_key(kmn) && finite_key(kmx))) {
    __syncthreads();  // every thread has read wlo / whi before the careful search rewrites them
    return count_threshold<BLOCK, CAP, V>(sh, x, [](int) { return true; }, m, need, goal, tau);
  }
  if (!(kmn < kmx)) return false;
  float lo = key_value(kmn), hi = key_value(kmx);
  int clo = m, chi = 1;
  const float aim = float((need + goal) >> 1);
  const float ms = float(m >> 2);  // entries sampled per row (m = BLOCK * V)
  const float mean = s1 / ms;
  const float var = fmaxf(s2 / ms - mean * mean, 0.f);
  float t = fmaf(sqrtf(var), normal_upper_quantile(aim / float(m)), mean);
#pragma unroll 1
  for (int step = 0; step < kSteps; ++step) {
    if (step > 0 || !(t > lo && t < hi)) {
      float f = (float(clo) - aim) / float(max(clo - chi, 1));
      f = fminf(fmaxf(f, 0.125f), 0.875f);
      t = fmaf(f, hi, fmaf(-f, lo, lo));
      if (!(t > lo && t < hi)) return false;  // uniform: the bracket cannot shrink
    }
    int cnt = 0;
#pragma unroll
    for (int v = 0; v < V; ++v) cnt += x[v] >= t ? 1 : 0;
    float cl = float(cnt), unused = 0.f;
    block_fsum2(sh, 1 - (step & 1), cl, unused);
    const int ct = int(cl);
    if (ct >= need) {
      lo = t;
      clo = ct;
      if (ct <= goal) {
        tau = t;
        return true;
      }
    } else {
      hi = t;
      chi = ct;
    }
  }
  return false;
}

// Append the entries u of a chunk with take(u) to the LDS list ckey / cj
// (key_at / j_at are evaluated for taken entries only). The wave takes all
// U ballots first and claims room for all its entries with one LDS atomic,
// so the per-entry-index chain is only SALU counting. The list order
// depends on the atomics, which nothing downstream relies on.
template <int BLOCK, int CAP, int U, typename KeyAt, typename JAt, typename Take>
__device__ __forceinline__ void append_list(TopkShared<BLOCK, CAP>& sh, KeyAt key_at, JAt j_at,
                                            Take take_it) {
  uint64_t mask[U];
  int total = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    mask[u] = __builtin_amdgcn_ballot_w64(take_it(u));  // the compare's own lane mask
    total += __popcll(mask[u]);
  }
  if (total == 0) return;  // uniform
  int base = 0;
  if (lane_id() == 0) base = atomicAdd(&sh.ccount, total);
  base = __builtin_amdgcn_readlane(base, 0);
  if (base + total > CAP) {  // uniform: the list is full, the row goes to the radix path
    if (lane_id() == 0) sh.overflow = 1;
    return;
  }
  // take_it is evaluated again rather than kept: U lane masks held as
  // booleans would not fit the scalar registers
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (take_it(u)) {
      const int pos = base + int(__builtin_amdgcn_mbcnt_hi(uint32_t(mask[u] >> 32),
                                                           __builtin_amdgcn_mbcnt_lo(uint32_t(mask[u]), 0u)));
      sh.ckey[pos] = key_at(u);
      sh.cj[pos] = j_at(u);
    }
    base += __popcll(mask[u]);
  }
}

// Raise a long row's bound and shrink its candidate list in place. The
// list holds every key >= tau_f seen so far (raw score bits), at least k of
// them; a count search over the list finds t with k <= C(t) <= k + k/8 + 64
// list entries >= t, so the row's k-th largest key is >= t and every winner
// seen so far stays in the list, and later keys below t can be dropped.
// Called by the whole block with the list complete (after a barrier), when
// it has filled past its refresh mark. Returns false (list untouched) when
// the search finds no such t (non-finite or crowded scores).
template <int BLOCK, int CAP>
__device__ __forceinline__ bool refresh_list(TopkShared<BLOCK, CAP>& sh, int k, float& tau_f) {
  constexpr int LR = CAP / BLOCK;
  const int tid = threadIdx.x;
  const int nc = sh.ccount;  // uniform: read after a barrier
  float lx[LR];
  uint32_t lj[LR];
#pragma unroll
  for (int u = 0; u < LR; ++u) {
    const int i = tid + BLOCK * u;
    lx[u] = i < nc ? __uint_as_float(sh.ckey[i]) : 0.f;
    lj[u] = i < nc ? sh.cj[i] : 0u;
  }
  auto valid = [&](int u) { return tid + BLOCK * u < nc; };
  float t = 0.f;
  // every thread's list reads above come before the search's first barrier
  if (!count_threshold<BLOCK, CAP, LR>(sh, lx, valid, nc, k, k + (k >> 3) + 64, t)) return false;
  if (tid == 0) sh.ccount = 0;
  __syncthreads();
  append_list<BLOCK, CAP, LR>(sh, [&](int u) { return __float_as_uint(lx[u]); }, [&](int u) { return lj[u]; },
                              [&](int u) { return valid(u) && lx[u] >= t; });
  tau_f = fmaxf(tau_f, t);
  return true;
}

// Longer rows. The first BLOCK*V keys are held in registers; their
// histogram gives the bin b* that holds the prefix's k-th largest key, and
// tau, the smallest prefix key in a bin >= b*, is at most that key. The
// row's k-th largest key is at least the prefix's (the prefix is part of
// the row), so every winner of the row is >= tau: the prefix keys in bins
// >= b* and the keys >= tau of the rest of the row (streamed once) form an
// LDS candidate list, from which the winners are selected exactly. If the list runs out of room (scores
// crowded into b*), the row falls back to multi-pass streaming selection.
// REFRESH: a list that fills past CAP - kRefreshRoom entries during the
// stream is shrunk by refresh_list, which also raises the bound; this lets
// a list of CAP entries serve rows whose first bound admits more keys than
// that.
template <int BLOCK, int V, int CAP, int NBUF, bool Q4 = false, bool REFRESH = false>
__device__ __forceinline__ void long_row_topk(TopkShared<BLOCK, CAP>& sh, const float* __restrict__ x, int n,
                                              int k, int32_t* __restrict__ orow) {
  constexpr int U = 16;           // streamed entries per thread per chunk
  constexpr int L = CAP / BLOCK;  // list entries per thread
  static_assert(CAP % BLOCK == 0, "list spread evenly over the block");
  static_assert(!Q4 || V % 4 == 0, "whole quads");
  const int tid = threadIdx.x;
  const int prefix = min(n, BLOCK * V);
  // Q4: whole quads, so a 16-byte load never straddles the range's end (the
  // entries of the last quad past n are row data, masked by index below)
  const auto rs = Q4 ? make_rsrc(x, ((n + 3) & ~3) * 4) : row_rsrc(x, n);
  float raw[V];
  load_chunk<BLOCK, V, Q4>(rs, 0, raw);
  float first[U], second[U];  // the streamed part's first chunks, in flight during the prefix's threshold
  load_chunk<BLOCK, U, Q4>(rs, prefix, first);
  if constexpr (NBUF == 3) load_chunk<BLOCK, U, Q4>(rs, prefix + BLOCK * U, second);
  // order keys of the prefix (0 = past the row's end); held in registers
  // unless the prefix is wide (REFRESH kernels), where they are recomputed
  uint32_t key[REFRESH ? 1 : V];
  if constexpr (!REFRESH) {
#pragma unroll
    for (int v = 0; v < V; ++v) key[v] = chunk_j<BLOCK, Q4>(0, v) < prefix ? order_key(raw[v]) : 0u;
  }
  auto key_at = [&](int v) -> uint32_t {
    if constexpr (REFRESH) return chunk_j<BLOCK, Q4>(0, v) < prefix ? order_key(raw[v]) : 0u;
    else return key[v];
  };
  auto j_at = [&](int v) { return uint32_t(chunk_j<BLOCK, Q4>(0, v)); };
  if (n <= prefix) {
    // entries u >= nu lie past n for every thread
    const int nu = Q4 ? 4 * ((n + 4 * BLOCK - 1) / (4 * BLOCK)) : (n + BLOCK - 1) / BLOCK;
    if (!bucket_topk<BLOCK, CAP, V>(sh, key_at, j_at, k, orow, nu))
      radix_topk<BLOCK, CAP>(sh, x, n, k, orow);
    return;
  }
  if (tid == 0) {
    sh.ccount = 0;
    sh.overflow = 0;
    sh.tau = 0xFFFFFFFFu;
  }
  // The bound tau. Rows of at least four prefixes (every row past the
  // prefix with REFRESH): a count search over the prefix (compares and
  // block sums only) for C(tau) between k and k + k/8 + 64. Otherwise, or
  // if it finds none, the prefix's histogram gives b* and tau is the
  // smallest prefix key in a bin >= b* (REFRESH: the radix path instead). Either way
  // tau is at most the prefix's k-th largest key. (Measured on the long fp8
  // rows, ~96K keys: 187.5 -> 183.2 us; on 16K-64K rows the search's looser
  // bound lets through more candidates than its cheaper start saves, and a
  // tighter window costs more probes than it saves on either.) The list
  // holds raw score bits until the stream ends (one dense pass then turns
  // them into order keys), so the stream's masked writes carry no
  // conversion.
  float tau_f = 0.f;
  bool can_refresh = true;  // uniform: cleared when a refresh finds no bound
  bool counted;
  if constexpr (REFRESH)  // n > prefix: every prefix entry lies inside the row
    counted = count_threshold_dense<BLOCK, CAP, V>(sh, raw, prefix, min(k, prefix),
                                                   min(k, prefix) + (min(k, prefix) >> 3) + 64, tau_f);
  else
    counted = n >= 4 * prefix &&
              count_threshold<BLOCK, CAP, V>(sh, raw, [&](int v) { return key_at(v) != 0u; }, prefix, min(k, prefix),
                                             min(k, prefix) + (min(k, prefix) >> 3) + 64, tau_f);
  if (counted) {
    if constexpr (REFRESH) {
      // in two halves: 32 lane masks would not fit the scalar registers
      static_assert(V % 8 == 0, "halves of whole quads");
      constexpr int H2 = V / 2;
      append_list<BLOCK, CAP, H2>(sh, [&](int v) { return __float_as_uint(raw[v]); }, j_at,
                                  [&](int v) { return raw[v] >= tau_f; });
      append_list<BLOCK, CAP, H2>(sh, [&](int v) { return __float_as_uint(raw[H2 + v]); },
                                  [&](int v) { return j_at(H2 + v); }, [&](int v) { return raw[H2 + v] >= tau_f; });
    } else {
      append_list<BLOCK, CAP, V>(sh, [&](int v) { return __float_as_uint(raw[v]); }, j_at,
                                 [&](int v) { return key_at(v) != 0u && raw[v] >= tau_f; });
    }
  } else if constexpr (REFRESH) {
    // no bound from the search (non-finite or crowded scores): the radix
    // path (the prefix histogram's registers would not fit beside a wide
    // prefix)
    __syncthreads();  // the search's last LDS reads come before the radix path's writes
    radix_topk<BLOCK, CAP>(sh, x, n, k, orow);
    return;
  } else {
    __syncthreads();  // the search may return right after reading wlo / whi, which the histogram rewrites
    int bin[V];
    bucket_threshold<BLOCK, CAP, V>(sh, key_at, k, V, bin);
    auto bin_at = [&](int v) { return bin[v]; };
    const int bstar = sh.digit;
    // prefix keys in bins >= b* join the list; tau, the smallest of them, is
    // at most the prefix's k-th largest key
    uint32_t mn = 0xFFFFFFFFu, unused = 0u;
    append_list<BLOCK, CAP, V>(sh, [&](int v) { return __float_as_uint(key_value(key_at(v))); }, j_at, [&](int v) {
      const bool t = bin_at(v) >= bstar;
      if (t) mn = min(mn, key_at(v));
      return t;
    });
    wave_min_max(mn, unused);
    if (lane_id() == 0) atomicMin(&sh.tau, mn);
    __syncthreads();
    tau_f = key_value(sh.tau);
  }
  // streamed keys >= tau join too (one float compare per key; only joining
  // keys are converted)
  // Only the last chunk needs the range test: past the range a load reads
  // 0.0, which can pass only when tau_f <= 0, and with Q4 the rest of the
  // last quad holds row data.
  stream_chunks<BLOCK, U, NBUF, Q4>(rs, prefix, n, first, second, [&](const float (&c)[U], int base) {
    auto key_of = [&](int u) { return __float_as_uint(c[u]); };
    auto j_of = [&](int u) { return uint32_t(chunk_j<BLOCK, Q4>(base, u)); };
    if (base + BLOCK * U <= n || (!Q4 && tau_f > 0.f))  // uniform
      append_list<BLOCK, CAP, U>(sh, key_of, j_of, [&](int u) { return c[u] >= tau_f; });
    else
      append_list<BLOCK, CAP, U>(sh, key_of, j_of,
                                 [&](int u) { return chunk_j<BLOCK, Q4>(base, u) < n && c[u] >= tau_f; });
    if constexpr (REFRESH) {
      __syncthreads();  // the chunk's appends are in: the count is uniform
      if (can_refresh && !sh.overflow && sh.ccount > CAP - kRefreshRoom) {
        can_refresh = refresh_list<BLOCK, CAP>(sh, k, tau_f);
        __syncthreads();  // the shrunk list is complete before the next chunk appends
      }
    }
  });
  __syncthreads();
  if (!sh.overflow) {
    const int nc = sh.ccount;
    for (int i = tid; i < nc; i += BLOCK) sh.ckey[i] = order_key(__uint_as_float(sh.ckey[i]));
    __syncthreads();
    uint32_t lkey[L], lj[L];
#pragma unroll
    for (int u = 0; u < L; ++u) {
      const int i = tid + BLOCK * u;
      lkey[u] = i < nc ? sh.ckey[i] : 0u;
      lj[u] = i < nc ? sh.cj[i] : 0u;
    }
    if (bucket_topk<BLOCK, CAP, L>(sh, [&](int u) { return lkey[u]; }, [&](int u) { return lj[u]; },
                                   k, orow))
      return;
    int nsel = 0;
    select_list(sh, nc, k, nsel);
    sort_selection(sh, nsel, k, orow);
    return;
  }
  radix_topk<BLOCK, CAP>(sh, x, n, k, orow);
}

// The second bound keeps 4 waves per SIMD (128 VGPRs): two 512-thread
// workgroups per CU, or one of 1024.
template <int BLOCK, int V, int CAP, int NBUF = 2, bool Q4 = false, bool REFRESH = false>
__global__ __launch_bounds__(BLOCK, 4) void topk_long_kernel(const float* __restrict__ logits,
                                                          const int32_t* __restrict__ limit,
                                                          int32_t* __restrict__ idx, int K, int k) {
  __shared__ TopkShared<BLOCK, CAP> sh;
  const int64_t row = blockIdx.x;
  const int n = limit ? max(0, min(limit[row], K - 1) + 1) : K;
  long_row_topk<BLOCK, V, CAP, NBUF, Q4, REFRESH>(sh, logits + row * K, n, k, idx + row * k);
}

// ---------------------------------------------------------------------------
// Fused logits -> top-k, second half. The candidate pass (the prefill
// logits kernel with its candidate epilogue) leaves, per row, nch regions
// of capc (order key, j) entries that hold every key of the row's top-k.
// One workgroup per row selects the top-k of those entries exactly (the
// bucket path). A row whose regions overflowed, or whose candidates crowd
// the bucket path's threshold bin, is queued for the recompute kernel.

constexpr int kSelBlock = 1024;

template <int L>  // region slots per thread: nch * capc <= kSelBlock * L
__global__ __launch_bounds__(kSelBlock) void fused_select_kernel(const uint2* __restrict__ cand,
                                                                 const int* __restrict__ count, int nch,
                                                                 int capc, int k, int32_t* __restrict__ idx,
                                                                 int* __restrict__ ctrl, int* __restrict__ over) {
  __shared__ TopkShared<kSelBlock, 64> sh;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int* crow = count + row * nch;
  const int slots = nch * capc;
  const auto rs = make_rsrc(cand + row * slots, slots * 8);
  u32x2 e[L];  // slots past a region's count read (0, 0) without a memory access
#pragma unroll
  for (int u = 0; u < L; ++u) {
    const int s = tid + kSelBlock * u;
    const int c = s / capc;
    const bool valid = c < nch && s - c * capc < crow[min(c, nch - 1)];
    e[u] = __builtin_amdgcn_raw_buffer_load_b64(rs, valid ? s * 8 : slots * 8, 0, 0);
  }
  const bool spill = __syncthreads_or(tid < nch && crow[tid] > capc);
  int32_t* orow = idx + row * k;
  if (!spill && bucket_topk<kSelBlock, 64, L>(
                    sh, [&](int u) { return e[u][0]; }, [&](int u) { return e[u][1]; }, k, orow))
    return;
  if (tid == 0) over[atomicAdd(&ctrl[0], 1)] = int(row);
}

// Rows the selection could not finish: a work queue over the listed rows
// (ctrl[0] rows, claimed through ctrl[1]) for a fixed grid of workgroups,
// each with a scratch row of K scores. The row's scores are recomputed with
// the logits kernels' tile arithmetic (Query16 and subtile_total on the
// same fragments, so the same bits), then the long-row selection runs on
// them. Every workgroup leaves once the queue is drained.
constexpr int kRecBlock = 1024;

// Scores of row `row` (n valid keys) into x, 64-key tiles spread over the
// block's waves. Kept out of line: its fragments and the selection's
// registers are then allocated separately instead of competing.
template <bool FP8>
__device__ __attribute__((noinline)) void score_row(const uint8_t* __restrict__ q, const float* __restrict__ q_scale,
                                                    const uint8_t* __restrict__ kmat, const float* __restrict__ k_scale,
                                                    const float* __restrict__ w, int64_t row, int64_t b, int K, int n,
                                                    float* __restrict__ x) {
  using M = Mma16<FP8>;
  using Frag = typename M::Frag;
  constexpr int kRowBytes = kHeadDim * M::kElemBytes;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, r = lane & 15;
  // fp8 scores on 32x32 tiles, bf16 on 16x16 tiles: the prefill kernel's forms
  std::conditional_t<FP8, Query32, Query16<false>> qr;
  qr.load(q + row * (kHeads * kRowBytes), w + row * kHeads, FP8 ? q_scale + row * kHeads : nullptr, lane);
  const auto krs = make_rsrc(kmat + b * int64_t(K) * kRowBytes, n * kRowBytes);
  const auto srs = make_rsrc(FP8 ? k_scale + b * int64_t(K) : nullptr, FP8 ? n * 4 : 0);
  const auto xrs = make_rsrc(x, n * 4);
  for (int j0 = 64 * wave; j0 < n; j0 += 64 * int(blockDim.x / 64)) {
    float tot;
    if constexpr (FP8) {
      // block blk, step s: lane (l % 32, l / 32) takes bytes [64s + 32(l/32), +32) of key j0 + 32 blk + l % 32
      float p[2];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        i32x8 bf[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int off = (j0 + 32 * blk + (lane & 31)) * kRowBytes + 64 * s + 32 * (lane >> 5);
          const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0);
          const u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(krs, off + 16, 0, 0);
          bf[s] = i32x8{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
        }
        p[blk] = qr.partial(bf);
      }
      tot = tile_total32(p[0], p[1]);
    } else {
      float p[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        Frag bf[M::kSteps];
        const int base = (j0 + 16 * st + r) * kRowBytes;
#pragma unroll
        for (int s = 0; s < M::kSteps; ++s)
          bf[s] = __builtin_bit_cast(Frag, __builtin_amdgcn_raw_buffer_load_b128(krs, base + M::dofs(s, g) * M::kElemBytes, 0, 0));
        p[st] = qr.partial(bf);
      }
      tot = subtile_total(p, lane);
    }
    const float sk =
        FP8 ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srs, (j0 + lane) * 4, 0, 0)) : 1.f;
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, qr.finish(tot, sk)), xrs, (j0 + lane) * 4,
                                          0, 0);
  }
}

template <bool FP8>
__global__ __launch_bounds__(kRecBlock) void fused_recompute_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale, const uint8_t* __restrict__ kmat,
    const float* __restrict__ k_scale, const float* __restrict__ w, const int32_t* __restrict__ limit, int T,
    int K, int ktop, int32_t* __restrict__ idx, int* __restrict__ ctrl, const int* __restrict__ over,
    float* __restrict__ scratch) {
  __shared__ TopkShared<kRecBlock, 8192> sh;
  __shared__ int claimed;
  float* x = scratch + int64_t(blockIdx.x) * K;
  for (;;) {
    if (threadIdx.x == 0) claimed = atomicAdd(&ctrl[1], 1);
    __syncthreads();
    const int i = claimed;
    const int queued = ctrl[0];
    __syncthreads();
    if (i >= queued) break;  // uniform
    const int64_t row = over[i];
    const int n = limit ? max(0, min(limit[row], K - 1) + 1) : K;
    score_row<FP8>(q, q_scale, kmat, k_scale, w, row, row / T, K, n, x);
    // the row's scores, written by every wave, are read back by every wave
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    long_row_topk<kRecBlock, 8, 8192, 2>(sh, x, n, ktop, idx + row * ktop);
    __syncthreads();  // the scratch row and LDS are reused by the next claim
  }
}

template <int BLOCK, int V, int CAP>
hipError_t launch_one(const float* logits, const int32_t* limit, int32_t* idx, int R, int K, int k,
                      hipStream_t stream) {
  hipLaunchKernelGGL((topk_kernel<BLOCK, V, CAP>), dim3(unsigned((R + 7) / 8 * 8)), dim3(BLOCK), 0, stream,
                     logits, limit, idx, R, K, k);
  return hipGetLastError();
}

template <int V>
hipError_t launch_wave(const float* logits, const int32_t* limit, int32_t* idx, int R, int K, int k,
                       hipStream_t stream) {
  hipLaunchKernelGGL(topk_wave_kernel<V>, dim3(unsigned((R + kWaveRows - 1) / kWaveRows)), dim3(64 * kWaveRows),
                     0, stream, logits, limit, idx, R, K, k);
  return hipGetLastError();
}

constexpr int kWaveMinRows = 1024;  // fewer rows leave most SIMDs idle: a workgroup per row instead
constexpr int kLongPairRows = 512;  // rows for two long-row workgroups per CU

}  // namespace

hipError_t launch_topk(const float* logits, const int32_t* limit, int32_t* idx, int R, int K,
                       int k, hipStream_t stream) {
  const bool wave_path = R >= kWaveMinRows && k <= kWaveMaxK && K % 4 == 0 &&
                         reinterpret_cast<uintptr_t>(logits) % 16 == 0;
  if (wave_path && K <= 1024) return launch_wave<16>(logits, limit, idx, R, K, k, stream);
  if (wave_path && K <= 2048) return launch_wave<32>(logits, limit, idx, R, K, k, stream);
  if (wave_path && K <= 4096) return launch_wave<64>(logits, limit, idx, R, K, k, stream);
  if (K <= 256 * 4) return launch_one<256, 4, 256>(logits, limit, idx, R, K, k, stream);
  if (K <= 256 * 16) return launch_one<256, 16, 256>(logits, limit, idx, R, K, k, stream);
  if (K <= 1024 * 8) return launch_one<1024, 8, 1024>(logits, limit, idx, R, K, k, stream);
  if (K <= 1024 * 16) return launch_one<1024, 16, 1024>(logits, limit, idx, R, K, k, stream);
  // 16-byte loads when every row starts 16-byte aligned. With enough rows
  // for two workgroups per CU, 512-thread workgroups (same 16K-key prefix,
  // 6K-entry list refreshed when it fills): one row's selection phases then
  // overlap the other's streaming.
  const bool q4 = K % 4 == 0 && reinterpret_cast<uintptr_t>(logits) % 16 == 0;
  if (q4 && R >= kLongPairRows)
    hipLaunchKernelGGL((topk_long_kernel<512, 32, 6144, 2, true, true>), dim3(unsigned(R)), dim3(512), 0, stream,
                       logits, limit, idx, K, k);
  else if (q4)
    hipLaunchKernelGGL((topk_long_kernel<1024, 16, 8192, 2, true>), dim3(unsigned(R)), dim3(1024), 0, stream,
                       logits, limit, idx, K, k);
  else
    hipLaunchKernelGGL((topk_long_kernel<1024, 16, 8192>), dim3(unsigned(R)), dim3(1024), 0, stream,
                       logits, limit, idx, K, k);
  return hipGetLastError();
}

hipError_t launch_fused_select(const FusedPlan& p, const CandidateOut& co, int R, int k, int32_t* idx,
                               int* ctrl, int* over, hipStream_t stream) {
  const int slots = p.nch * p.capc;
  if (slots <= kSelBlock * 4)
    hipLaunchKernelGGL(fused_select_kernel<4>, dim3(unsigned(R)), dim3(kSelBlock), 0, stream, co.cand, co.count,
                       p.nch, p.capc, k, idx, ctrl, over);
  else
    hipLaunchKernelGGL(fused_select_kernel<16>, dim3(unsigned(R)), dim3(kSelBlock), 0, stream, co.cand, co.count,
                       p.nch, p.capc, k, idx, ctrl, over);
  return hipGetLastError();
}

hipError_t launch_fused_recompute(const void* q, const float* q_scale, const void* k, const float* k_scale,
                                  const float* w, const int32_t* limit, const FusedPlan& p, int T, int K,
                                  int ktop, bool fp8, int32_t* idx, int* ctrl, const int* over, float* scratch,
                                  hipStream_t stream) {
  const auto* q8 = static_cast<const uint8_t*>(q);
  const auto* k8 = static_cast<const uint8_t*>(k);
  const dim3 grid(unsigned(p.fallback_blocks));
  if (fp8)
    hipLaunchKernelGGL(fused_recompute_kernel<true>, grid, dim3(kRecBlock), 0, stream, q8, q_scale, k8, k_scale,
                       w, limit, T, K, ktop, idx, ctrl, over, scratch);
  else
    hipLaunchKernelGGL(fused_recompute_kernel<false>, grid, dim3(kRecBlock), 0, stream, q8, q_scale, k8, k_scale,
                       w, limit, T, K, ktop, idx, ctrl, over, scratch);
  return hipGetLastError();
}

}  // namespace xk
