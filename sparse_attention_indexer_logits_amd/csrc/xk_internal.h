// Internal declarations shared by the HIP translation units of libxk.
// (Device code only; the CPU oracle shares nothing with this file.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xk {

constexpr int kHeads = 64;     // DeepSeek-V4 index_n_heads
constexpr int kHeadDim = 128;  // DeepSeek-V4 index_head_dim
constexpr int kMaxTopk = 2048;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short s16x4;  // four bf16 bit patterns
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

// Raw buffer resource over [base, base + bytes): the hardware range check
// makes loads at or past `bytes` return 0 and drops such stores, with no
// branch and no memory access (dword 3 = 0x00020000: 32-bit data format,
// the raw-buffer setting of gfx9-family parts).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// Order key of a score: an unsigned integer that sorts like the score
// (-0.0 folded to +0.0, which it equals); key 0 is below every score and
// marks "no entry".
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Score of an order key (inverse of order_key).
__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Candidate output of the fused logits -> top-k pass.
struct CandidateOut {
  uint2* cand;  // [rows][n_chunks][capc] (order key, j)
  int* count;   // [rows][n_chunks] entries each region received (may exceed capc)
  int* ctrl;    // the recompute queue's two counters, cleared by the candidate pass
  int capc;     // entries per region
};

// Shapes and workspace layout of the fused logits -> top-k call (host).
struct FusedPlan {
  bool fused;           // false: scores go to the workspace and the plain top-k reads them
  int nqb, nch, kpw;    // query blocks, key chunks per row, keys per chunk
  int capc, nl;         // entries per (row, chunk) region; per-lane list length (64*nl >= k)
  int fallback_blocks;  // workgroups (and scratch rows) of the recompute path
  size_t off_count, off_ctrl, off_over, off_cand, off_scratch, off_logits, bytes;
};
FusedPlan plan_fused(int B, int T, int K, int k, bool fp8);

// Host-side launchers (one per translation unit). Arguments are validated by
// the C ABI layer before these run; they only enqueue work and return the
// launch status.
hipError_t launch_logits(const void* q, const float* q_scale, const void* k,
                         const float* k_scale, const float* w, const int32_t* limit,
                         float* logits, int B, int T, int K, bool fp8, hipStream_t stream);
hipError_t launch_logits_paged(const void* q, const float* q_scale, const float* w,
                               const int32_t* limit, const void* k_cache, const void* k_scale,
                               const int32_t* block_table, float* logits, int B, int T, int K,
                               int MB, int bs, bool mxfp4, hipStream_t stream);
hipError_t launch_quant_fp8_rows(const void* x, bool bf16, uint8_t* out, float* scale, int64_t N,
                                 hipStream_t stream);
hipError_t launch_mxfp4_write(const void* x, bool bf16, const int64_t* slots, uint8_t* kv_fp4,
                              uint8_t* kv_scale, int64_t N, int64_t n_slots, hipStream_t stream);
hipError_t launch_topk(const float* logits, const int32_t* limit, int32_t* idx, int R,
                       int K, int k, hipStream_t stream);
hipError_t launch_logits_candidates(const void* q, const float* q_scale, const void* k,
                                    const float* k_scale, const float* w, const int32_t* limit,
                                    const FusedPlan& plan, const CandidateOut& co, int B, int T, int K,
                                    bool fp8, hipStream_t stream);
hipError_t launch_fused_select(const FusedPlan& plan, const CandidateOut& co, int R, int k,
                               int32_t* idx, int* ctrl, int* over, hipStream_t stream);
hipError_t launch_fused_recompute(const void* q, const float* q_scale, const void* k,
                                  const float* k_scale, const float* w, const int32_t* limit,
                                  const FusedPlan& plan, int T, int K, int ktop, bool fp8, int32_t* idx,
                                  int* ctrl, const int* over, float* scratch, hipStream_t stream);
hipError_t launch_logits_topk(const void* q, const float* q_scale, const void* k,
                              const float* k_scale, const float* w, const int32_t* limit,
                              int32_t* idx, int B, int T, int K, int ktop, bool fp8, void* workspace,
                              hipStream_t stream);
hipError_t launch_sparse_attention(const uint16_t* q, const uint8_t* kv_fp4, const uint8_t* kv_scale,
                                   const int32_t* block_table, const int32_t* sel_pos, const int32_t* row_seq,
                                   const float* sink, float scale, float* out, int R, int H, int k, int MB, int bs,
                                   hipStream_t stream);
hipError_t launch_gather(const uint8_t* kv_fp4, const uint8_t* kv_scale,
                         const int32_t* block_table, const int32_t* sel_pos,
                         const int32_t* row_seq, uint16_t* out, int R, int k, int MB,
                         int bs, hipStream_t stream);

}  // namespace xk
