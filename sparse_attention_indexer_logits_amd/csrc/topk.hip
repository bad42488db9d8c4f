// Deterministic per-row top-k of the indexer logits (gfx950).
//
// Result (pages "xkernels #28 -- DeepSeek-V4 serving support": top-512 Flash /
// top-1024 Pro per query; "DeepSeek V4 Flash on a single AMD MI300X":
// deterministic sparse top-k with a tie-break, canonical order of the
// selection): among the n = clamp(limit+1, 0, K) valid keys of a row, the
// min(k, n) largest scores ordered by (score desc, j asc), then -1 padding.
//
// One workgroup per row; the row is read from HBM once and stays in VGPRs
// (V values per thread, j = tid + BLOCK*v).
//  1. Scores become order-preserving u32 keys (-0.0 first folded to +0.0);
//     key 0 marks an invalid slot (every valid float maps above it).
//  2. Radix select, 8 bits per pass from the top: an LDS histogram of the
//     next digit over the keys still matching the prefix, then one wave finds
//     the digit holding the k-th largest key with a suffix scan. A pass stops
//     early when that digit's bucket is exactly what is still needed.
//  3. If the threshold bucket holds more keys than needed, the lowest j win:
//     a second radix select over j (ascending) inside that bucket gives the
//     cut. Histogram counts are order independent, so the selected SET is
//     fixed regardless of atomic ordering.
//  4. The k winners go to LDS as 64-bit (key << 32 | ~j) and a bitonic sort
//     (descending) puts them in the canonical order, which is unique.
#include <algorithm>

#include "xk_internal.h"

namespace xk {
namespace {

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;                     // -0.0 ties with +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct TopkShared {
  uint32_t hist[256];
  uint64_t cand[kMaxTopk];
  int digit;       // digit found by the scan
  int above;       // count of matching keys in digits past `digit`
  int at;          // count of matching keys in `digit`
  int cnt;         // compaction cursor
};

// Wave 0 scans hist[] for the bucket holding the `need`-th element, counting
// from the top digit down (descending) or from digit 0 up (ascending).
__device__ void find_digit(TopkShared& sh, int need, bool descending) {
  const int lane = threadIdx.x;  // only wave 0 calls this
  int c[4];
  int s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int bin = descending ? 255 - (4 * lane + i) : 4 * lane + i;
    c[i] = int(sh.hist[bin]);
    s += c[i];
  }
  // exclusive prefix over lanes in scan order
  int incl = s;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(incl, d);
    if (lane >= d) incl += t;
  }
  int before = incl - s;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (before < need && before + c[i] >= need) {
      sh.digit = descending ? 255 - (4 * lane + i) : 4 * lane + i;
      sh.above = before;
      sh.at = c[i];
    }
    before += c[i];
  }
}

template <int BLOCK, int V>
__global__ __launch_bounds__(BLOCK) void topk_kernel(const float* __restrict__ logits,
                                                     const int32_t* __restrict__ limit,
                                                     int32_t* __restrict__ idx, int K, int k) {
  __shared__ TopkShared sh;
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

  const int m = min(k, n);
  // selection rule: (key >> shift) > thr, or == thr with j <= jcut
  int shift = 0;
  uint32_t thr = 0u;  // with shift 0 and jcut max: take every valid key (n <= k)
  int jcut = 0x7FFFFFFF;
  if (n > k) {
    uint32_t prefix = 0u;
    int need = k;
    bool settled = false;
    for (int pass = 0; pass < 4 && !settled; ++pass) {
      const int sft = 24 - 8 * pass;
      const uint32_t hi_mask = pass == 0 ? 0u : (0xFFFFFFFFu << (sft + 8));
      for (int i = tid; i < 256; i += BLOCK) sh.hist[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (key[v] != 0u && (key[v] & hi_mask) == prefix)
          atomicAdd(&sh.hist[(key[v] >> sft) & 255u], 1u);
      __syncthreads();
      if (tid < 64) find_digit(sh, need, true);
      __syncthreads();
      prefix |= uint32_t(sh.digit) << sft;
      need -= sh.above;
      shift = sft;
      thr = prefix >> sft;
      settled = sh.at == need;  // the whole bucket is taken
      __syncthreads();          // sh.* read by all before the next pass rewrites it
    }
    if (!settled) {
      // ties on the full key: the `need` lowest j among key == prefix
      uint32_t jprefix = 0u;
      for (int pass = 0; pass < 4; ++pass) {
        const int sft = 24 - 8 * pass;
        const uint32_t hi_mask = pass == 0 ? 0u : (0xFFFFFFFFu << (sft + 8));
        for (int i = tid; i < 256; i += BLOCK) sh.hist[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int v = 0; v < V; ++v) {
          const uint32_t j = uint32_t(tid + BLOCK * v);
          if (key[v] == prefix && (j & hi_mask) == jprefix)
            atomicAdd(&sh.hist[(j >> sft) & 255u], 1u);
        }
        __syncthreads();
        if (tid < 64) find_digit(sh, need, false);
        __syncthreads();
        jprefix |= uint32_t(sh.digit) << sft;
        need -= sh.above;
        __syncthreads();
      }
      jcut = int(jprefix);
    }
  }

  if (tid == 0) sh.cnt = 0;
  __syncthreads();
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int j = tid + BLOCK * v;
    const uint32_t kk = key[v] >> shift;
    if (key[v] != 0u && (kk > thr || (kk == thr && j <= jcut))) {
      const int pos = atomicAdd(&sh.cnt, 1);
      if (pos < kMaxTopk) sh.cand[pos] = (uint64_t(key[v]) << 32) | uint64_t(~uint32_t(j));
    }
  }
  __syncthreads();

  // bitonic sort (descending) of the m winners, padded to a power of two
  int P = 1;
  while (P < m) P <<= 1;
  for (int i = m + tid; i < P; i += BLOCK) sh.cand[i] = 0ull;
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < (P >> 1); i += BLOCK) {
        const int lo = 2 * stride * (i / stride) + (i % stride);
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const uint64_t a = sh.cand[lo], c = sh.cand[hi];
        if (desc ? (a < c) : (a > c)) {
          sh.cand[lo] = c;
          sh.cand[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  int32_t* orow = idx + row * k;
  for (int s = tid; s < k; s += BLOCK)
    orow[s] = s < m ? int32_t(~uint32_t(sh.cand[s] & 0xFFFFFFFFull)) : -1;
}

template <int BLOCK, int V>
hipError_t launch_one(const float* logits, const int32_t* limit, int32_t* idx, int R, int K, int k,
                      hipStream_t stream) {
  hipLaunchKernelGGL((topk_kernel<BLOCK, V>), dim3(unsigned(R)), dim3(BLOCK), 0, stream, logits,
                     limit, idx, K, k);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(const float* logits, const int32_t* limit, int32_t* idx, int R, int K,
                       int k, hipStream_t stream) {
  if (K <= 256 * 4) return launch_one<256, 4>(logits, limit, idx, R, K, k, stream);
  if (K <= 256 * 8) return launch_one<256, 8>(logits, limit, idx, R, K, k, stream);
  if (K <= 256 * 16) return launch_one<256, 16>(logits, limit, idx, R, K, k, stream);
  if (K <= 1024 * 8) return launch_one<1024, 8>(logits, limit, idx, R, K, k, stream);
  if (K <= 1024 * 16) return launch_one<1024, 16>(logits, limit, idx, R, K, k, stream);
  if (K <= 1024 * 32) return launch_one<1024, 32>(logits, limit, idx, R, K, k, stream);
  if (K <= 1024 * 64) return launch_one<1024, 64>(logits, limit, idx, R, K, k, stream);
  return launch_one<1024, 96>(logits, limit, idx, R, K, k, stream);
}

}  // namespace xk
