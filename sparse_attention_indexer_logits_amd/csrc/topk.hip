// Deterministic per-row top-k of the indexer logits (gfx950).
//
// Result (pages "xkernels #28 -- DeepSeek-V4 serving support": top-512 Flash /
// top-1024 Pro per query; "DeepSeek V4 Flash on a single AMD MI300X":
// deterministic sparse top-k with a tie-break, canonical order of the
// selection): among the n = clamp(limit+1, 0, K) valid keys of a row, the
// min(k, n) largest scores ordered by (score desc, j asc), then -1 padding.
//
// One workgroup per row. Rows up to 16384 keys are read from HBM once and
// stay in VGPRs (V values per thread, j = tid + BLOCK*v); longer rows keep a
// 32768-key prefix in VGPRs and stream the rest once (topk_long_kernel).
// Scores become order-preserving u32 keys (-0.0 folded to +0.0); key 0 marks
// a slot past the row's end.
//
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
//     passes run over the registers instead.
//  D. The selection is sorted by (key << 32 | ~j), descending: 64-entry runs
//     by a bitonic network across the lanes of a wave, then pairwise merges
//     in which each entry's slot comes from a binary search in the other run.
#include <algorithm>

#include "xk_internal.h"

namespace xk {
namespace {

constexpr int kBins = 2048;  // 11-bit digits

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0.0 ties with +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lane_id() { return int(threadIdx.x & 63); }

__device__ __forceinline__ int prefix_in_wave(uint64_t mask) {
  return __popcll(mask & ((uint64_t(1) << lane_id()) - 1));
}

template <int BLOCK, int CAP>
struct TopkShared {
  __attribute__((aligned(16))) uint32_t hist[kBins];
  uint64_t sel[kMaxTopk];
  union {
    struct {
      uint32_t ckey[CAP];  // candidate list: keys in the threshold bucket
      uint32_t cj[CAP];    // ... and their positions
    };
    uint64_t sel2[kMaxTopk];  // merge-round buffer (the list is dead by then)
  };
  int wsel[BLOCK / 64], wcand[BLOCK / 64];
  int digit, above, at;
  int ccount;       // streamed candidate list: entries claimed so far
  int overflow;     // 1 if the streamed list ran out of room
  uint32_t tau;     // smallest key of the prefix selection
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
  int incl = s;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(incl, d);
    if (lane >= d) incl += t;
  }
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
// to the candidate list (pred == 2) with one block-wide scan: per-wave
// ballots give each lane its slot, per-wave totals in LDS give each wave its
// base. key_at(u) / j_at(u) give entry u; the predicate is evaluated again
// in the writing sweep instead of being stored. The running totals nsel /
// ncand stay in registers (uniform across the block).
template <int BLOCK, int CAP, int U, typename KeyAt, typename JAt, typename Pred>
__device__ __forceinline__ void compact(TopkShared<BLOCK, CAP>& sh, KeyAt key_at, JAt j_at,
                                        Pred pred, int& nsel, int& ncand) {
  constexpr int NW = BLOCK / 64;
  const int lane = lane_id(), wave = int(threadIdx.x) >> 6;
  int ts = 0, tc = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = pred(key_at(u), j_at(u));
    ts += __popcll(__ballot(c == 1));
    tc += __popcll(__ballot(c == 2));
  }
  if (lane == 0) {
    sh.wsel[wave] = ts;
    sh.wcand[wave] = tc;
  }
  __syncthreads();
  int bs = nsel, bc = ncand;
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
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t kv = key_at(u), jv = j_at(u);
    const int c = pred(kv, jv);
    const uint64_t ms = __ballot(c == 1), mc = __ballot(c == 2);
    if (c == 1) {
      const int pos = bs + prefix_in_wave(ms);
      if (pos < kMaxTopk) sh.sel[pos] = (uint64_t(kv) << 32) | uint64_t(~jv);
    } else if (c == 2) {
      const int pos = bc + prefix_in_wave(mc);
      if (pos < CAP) {
        sh.ckey[pos] = kv;
        sh.cj[pos] = jv;
      }
    }
    bs += __popcll(ms);
    bc += __popcll(mc);
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

// Sorts one 64-entry run held one per lane, descending (bitonic network
// across the lanes of a wave).
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t x) {
  const int lane = lane_id();
#pragma unroll
  for (int sz = 2; sz <= 64; sz <<= 1) {
#pragma unroll
    for (int s = sz >> 1; s > 0; s >>= 1) {
      const uint64_t o = __shfl_xor(x, s);
      const bool desc = (lane & sz) == 0;
      const bool lower = (lane & s) == 0;
      const uint64_t hi = x > o ? x : o, lo = x > o ? o : x;
      x = (lower == desc) ? hi : lo;
    }
  }
  return x;
}

// Number of entries of the descending run a[0..L) that are > x (or >= x).
template <bool OR_EQUAL>
__device__ __forceinline__ int count_before(const uint64_t* a, int L, uint64_t x) {
  int pos = 0;
  for (int step = L >> 1; step > 0; step >>= 1) {
    const uint64_t y = a[pos + step - 1];
    if (OR_EQUAL ? y >= x : y > x) pos += step;
  }
  const uint64_t last = a[L - 1];
  if (pos == L - 1 && (OR_EQUAL ? last >= x : last > x)) pos = L;
  return pos;
}

// Sort sh.sel[0..m) descending (m <= kMaxTopk) and write the row:
// 64-entry runs are sorted inside waves, then runs are merged pairwise; in a
// merge every entry finds its slot as (its index in its run) + (entries of
// the partner run that precede it), by binary search. Entries are distinct
// except the zero padding, which the left run places first.
template <int BLOCK, int CAP>
__device__ __forceinline__ void sort_and_store(TopkShared<BLOCK, CAP>& sh, int m, int32_t* orow,
                                               int k) {
  constexpr int NW = BLOCK / 64;
  const int lane = lane_id(), wave = int(threadIdx.x) >> 6;
  int runs = (m + 63) >> 6;
  int P = 1;
  while (P < runs) P <<= 1;  // runs padded to a power of two
  const int N = P * 64;
  for (int r = wave; r < P; r += NW) {
    const int i = r * 64 + lane;
    const uint64_t x = i < m ? sh.sel[i] : 0ull;
    sh.sel[i] = wave_sort_desc(x);
  }
  __syncthreads();
  uint64_t* src = sh.sel;
  uint64_t* dst = sh.sel2;
  for (int L = 64; L < N; L <<= 1) {
    for (int i = threadIdx.x; i < N; i += BLOCK) {
      const uint64_t x = src[i];
      const int run = i / L, own = i % L;
      const int base = (run & ~1) * L;
      const uint64_t* partner = src + (run ^ 1) * L;
      const int c = (run & 1) ? count_before<true>(partner, L, x)
                              : count_before<false>(partner, L, x);
      dst[base + own + c] = x;
    }
    __syncthreads();
    uint64_t* t = src;
    src = dst;
    dst = t;
  }
  for (int p = threadIdx.x; p < k; p += BLOCK)
    orow[p] = p < m ? int32_t(~uint32_t(src[p] & 0xFFFFFFFFull)) : -1;
}

// Select the min(k, n) winners of a row into sh.sel (unsorted; nsel counts
// them). `chunks(g)` calls g(key_at, j_at) per chunk of BLOCK*U entries,
// with key_at(u) / j_at(u) giving this thread's entry u (key 0 = no entry)
// and the same number of chunks on every thread.
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
  auto one = [](int) { return 0; };
  if (n > k) {
    // A: top 11 bits over the whole row
    Cut cut{32, 0u, 0xFFFFFFFFu, k, false};
    key_pass(sh, cut, 21, 11, each_src);
    if (cut.settled || sh.at <= CAP) {
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
  (void)one;
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

// chunks(g) over entries [j_lo, j_hi) of x streamed from memory, BLOCK*U per
// chunk, the next chunk's loads in flight while this one is processed.
template <int BLOCK, int U, typename G>
__device__ __forceinline__ void stream_chunks(const float* __restrict__ x, int j_lo, int j_hi, G g) {
  const int tid = threadIdx.x;
  uint32_t kv[U];
  float cur[U], nxt[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = j_lo + BLOCK * u + tid;
    cur[u] = j < j_hi ? x[j] : 0.f;
    nxt[u] = 0.f;
  }
  for (int base = j_lo; base < j_hi; base += BLOCK * U) {
    const int nb = base + BLOCK * U;
    if (nb < j_hi) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = nb + BLOCK * u + tid;
        nxt[u] = j < j_hi ? x[j] : 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = base + BLOCK * u + tid;
      kv[u] = j < j_hi ? order_key(cur[u]) : 0u;
    }
    g([&](int u) { return kv[u]; }, [&](int u) { return uint32_t(base + BLOCK * u + tid); });
#pragma unroll
    for (int u = 0; u < U; ++u) cur[u] = nxt[u];
  }
}

// Rows of at most BLOCK*V keys: the row is read once into V registers per
// thread (j = tid + BLOCK*v).
template <int BLOCK, int V, int CAP>
__global__ __launch_bounds__(BLOCK) void topk_kernel(const float* __restrict__ logits,
                                                     const int32_t* __restrict__ limit,
                                                     int32_t* __restrict__ idx, int K, int k) {
  __shared__ TopkShared<BLOCK, CAP> sh;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int n = limit ? max(0, min(limit[row], K - 1) + 1) : K;
  const float* x = logits + row * K;
  uint32_t key[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int j = tid + BLOCK * v;
    key[v] = j < n ? order_key(x[j]) : 0u;
  }
  auto chunks = [&](auto g) {
    g([&](int v) { return key[v]; }, [&](int v) { return uint32_t(tid + BLOCK * v); });
  };
  int nsel = 0;
  select_row<BLOCK, CAP, V>(sh, n, k, chunks, nsel);
  sort_and_store(sh, min(k, n), idx + row * k, k);
}

// Longer rows. The first BLOCK*V keys are held in registers and selected
// exactly; the smallest selected key tau is a lower bound of the row's k-th
// largest key (a prefix's k-th largest cannot exceed the row's). The rest of
// the row is streamed once and only keys > tau join an LDS candidate list
// (a key equal to tau arrives with a larger j than every kept one, so it can
// never win). The winners are then selected exactly from prefix-selection +
// candidates. If the list runs out of room (only for adversarial rows), the
// row falls back to multi-pass streaming selection over the whole row.
template <int BLOCK, int V, int CAP>
__global__ __launch_bounds__(BLOCK) void topk_long_kernel(const float* __restrict__ logits,
                                                          const int32_t* __restrict__ limit,
                                                          int32_t* __restrict__ idx, int K, int k) {
  constexpr int U = 8;  // streamed entries per thread per chunk
  __shared__ TopkShared<BLOCK, CAP> sh;
  const int tid = threadIdx.x, lane = lane_id();
  const int64_t row = blockIdx.x;
  const int n = limit ? max(0, min(limit[row], K - 1) + 1) : K;
  const int prefix = min(n, BLOCK * V);
  const float* x = logits + row * K;
  uint32_t key[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int j = tid + BLOCK * v;
    key[v] = j < prefix ? order_key(x[j]) : 0u;
  }
  auto reg_chunks = [&](auto g) {
    g([&](int v) { return key[v]; }, [&](int v) { return uint32_t(tid + BLOCK * v); });
  };
  int nsel = 0;
  select_row<BLOCK, CAP, V>(sh, prefix, k, reg_chunks, nsel);

  if (n > prefix) {
    // move the prefix winners into the candidate list; tau = their smallest key
    if (tid == 0) {
      sh.tau = 0xFFFFFFFFu;
      sh.ccount = nsel;
      sh.overflow = 0;
    }
    __syncthreads();
    uint32_t mn = 0xFFFFFFFFu;
    for (int i = tid; i < nsel; i += BLOCK) {
      const uint64_t e = sh.sel[i];
      const uint32_t kv = uint32_t(e >> 32);
      sh.ckey[i] = kv;
      sh.cj[i] = ~uint32_t(e & 0xFFFFFFFFull);
      mn = min(mn, kv);
    }
    for (int d = 32; d > 0; d >>= 1) mn = min(mn, uint32_t(__shfl_xor(int(mn), d)));
    if (lane == 0) atomicMin(&sh.tau, mn);
    __syncthreads();
    const uint32_t tau = nsel == k ? sh.tau : 0u;  // fewer than k so far: take every key
    // stream the rest once; keys above tau join the list (one atomic per wave)
    stream_chunks<BLOCK, U>(x, prefix, n, [&](auto key_at, auto j_at) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t kv = key_at(u);
        const bool take = kv > tau;
        const uint64_t m = __ballot(take);
        if (m == 0) continue;
        const int leader = __ffsll((unsigned long long)m) - 1;
        int base = 0;
        if (lane == leader) base = atomicAdd(&sh.ccount, __popcll(m));
        base = __shfl(base, leader);
        if (take) {
          const int pos = base + prefix_in_wave(m);
          if (pos < CAP) {
            sh.ckey[pos] = kv;
            sh.cj[pos] = j_at(u);
          } else {
            sh.overflow = 1;
          }
        }
      }
    });
    __syncthreads();
    nsel = 0;
    if (!sh.overflow) {
      // exact selection over prefix winners + streamed candidates
      select_list(sh, sh.ccount, k, nsel);
    } else {
      // fallback: multi-pass selection streaming the whole row
      auto all_chunks = [&](auto g) { stream_chunks<BLOCK, U>(x, 0, n, g); };
      select_row<BLOCK, CAP, U>(sh, n, k, all_chunks, nsel);
    }
  }
  sort_and_store(sh, min(k, n), idx + row * k, k);
}

template <int BLOCK, int V, int CAP>
hipError_t launch_one(const float* logits, const int32_t* limit, int32_t* idx, int R, int K, int k,
                      hipStream_t stream) {
  hipLaunchKernelGGL((topk_kernel<BLOCK, V, CAP>), dim3(unsigned(R)), dim3(BLOCK), 0, stream,
                     logits, limit, idx, K, k);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(const float* logits, const int32_t* limit, int32_t* idx, int R, int K,
                       int k, hipStream_t stream) {
  if (K <= 256 * 4) return launch_one<256, 4, 2048>(logits, limit, idx, R, K, k, stream);
  if (K <= 256 * 16) return launch_one<256, 16, 2048>(logits, limit, idx, R, K, k, stream);
  if (K <= 1024 * 8) return launch_one<1024, 8, 4096>(logits, limit, idx, R, K, k, stream);
  if (K <= 1024 * 16) return launch_one<1024, 16, 4096>(logits, limit, idx, R, K, k, stream);
  hipLaunchKernelGGL((topk_long_kernel<1024, 32, 6144>), dim3(unsigned(R)), dim3(1024), 0, stream,
                     logits, limit, idx, K, k);
  return hipGetLastError();
}

}  // namespace xk
