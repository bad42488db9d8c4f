// Fused indexer logits -> top-k (gfx950): the top-k of every query's scores
// without writing the [B,T,K] score matrix.
//
//  1. candidates the prefill logits kernel with its candidate epilogue: one
//                wave streams a query's whole row and appends every key that
//                scores >= its running lower bound on the row's k-th largest
//                score (expected ~ k (1 + ln(n/k)) times a small factor)
//  2. select     one workgroup per row: exact top-k of the row's candidates
//                (bucket path); rows it cannot finish are queued
//  3. recompute  a fixed grid drains the queue: rescore the row into a
//                scratch row with the same tile arithmetic and run the
//                long-row selection on it
// The queue counters are cleared by the candidate pass (no memset, so the
// call can be captured in a HIP graph). Calls where filtering cannot pay
// (fewer than 16 keys per selected index, or too few query blocks to give
// every CU one) write the scores to the workspace and run the plain top-k.
#include <algorithm>

#include "xk_internal.h"

namespace xk {
namespace {

constexpr int kMaxSlots = 16384;     // candidate slots per row (the select kernel's registers)
constexpr int kMinKeysPerIndex = 16;  // K / k below this: filtering keeps most keys
constexpr int kMinQueryBlocks = 256;  // one workgroup per CU at least
constexpr int kMaxRecomputeBlocks = 64;
constexpr int kMaxRowKeys = 1 << 22;  // one chunk's key bytes stay in a buffer descriptor's range

size_t align256(size_t x) { return (x + 255) / 256 * 256; }
int round_up(int x, int m) { return (x + m - 1) / m * m; }

}  // namespace

FusedPlan plan_fused(int B, int T, int K, int k, bool fp8) {
  FusedPlan p{};
  const int64_t R = int64_t(B) * T;
  const int QB = fp8 ? 8 : 4;  // queries per workgroup of the prefill kernel
  p.nqb = (T + QB - 1) / QB;
  const int64_t qblocks = int64_t(p.nqb) * B;
  p.fused = T >= 8 && qblocks >= kMinQueryBlocks && int64_t(K) >= int64_t(kMinKeysPerIndex) * k &&
            K <= kMaxRowKeys;
  if (!p.fused) {
    p.off_logits = 0;
    p.bytes = align256(size_t(R) * size_t(K) * 4);
    return p;
  }
  // one chunk per row: a wave's bound then covers every key of its row seen
  // so far (separate chunks would each admit ~k ln(chunk/k) on their own)
  p.kpw = round_up(K, 64);
  p.nch = 1;
  p.capc = std::min(p.kpw, kMaxSlots);
  p.nl = k <= 256 ? 4 : k <= 512 ? 8 : k <= 1024 ? 16 : 32;
  p.fallback_blocks = int(std::min<int64_t>(R, kMaxRecomputeBlocks));
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  p.off_ctrl = take(2 * sizeof(int));
  p.off_count = take(size_t(R) * p.nch * 4);
  p.off_over = take(size_t(R) * 4);
  p.off_cand = take(size_t(R) * p.nch * p.capc * 8);
  p.off_scratch = take(size_t(p.fallback_blocks) * K * 4);
  p.bytes = off;
  return p;
}

hipError_t launch_logits_topk(const void* q, const float* q_scale, const void* k, const float* k_scale,
                              const float* w, const int32_t* limit, int32_t* idx, int B, int T, int K,
                              int ktop, bool fp8, void* workspace, hipStream_t stream) {
  const FusedPlan p = plan_fused(B, T, K, ktop, fp8);
  auto* base = static_cast<uint8_t*>(workspace);
  const int R = B * T;
  hipError_t e;
  if (!p.fused) {
    auto* scores = reinterpret_cast<float*>(base + p.off_logits);
    e = launch_logits(q, q_scale, k, k_scale, w, limit, scores, B, T, K, fp8, stream);
    if (e != hipSuccess) return e;
    return launch_topk(scores, limit, idx, R, K, ktop, stream);
  }
  int* ctrl = reinterpret_cast<int*>(base + p.off_ctrl);  // [0] rows queued, [1] rows claimed
  CandidateOut co{reinterpret_cast<uint2*>(base + p.off_cand), reinterpret_cast<int*>(base + p.off_count), ctrl,
                  p.capc};
  int* over = reinterpret_cast<int*>(base + p.off_over);
  auto* scratch = reinterpret_cast<float*>(base + p.off_scratch);
  e = launch_logits_candidates(q, q_scale, k, k_scale, w, limit, p, co, B, T, K, fp8, stream);
  if (e != hipSuccess) return e;
  e = launch_fused_select(p, co, R, ktop, idx, ctrl, over, stream);
  if (e != hipSuccess) return e;
  return launch_fused_recompute(q, q_scale, k, k_scale, w, limit, p, T, K, ktop, fp8, idx, ctrl, over, scratch,
                                stream);
}

}  // namespace xk
