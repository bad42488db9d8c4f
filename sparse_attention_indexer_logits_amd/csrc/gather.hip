// mxfp4 paged KV gather -> bf16 (gfx950).
//
// Semantics (page "xkernels #28 -- DeepSeek-V4 serving support", comment
// shipping mxfp4_paged_gather): per (row, top-k slot) look up the block
// table, decode E2M1 nibbles times the E8M0 group scale 2^(b-127) with
// 0xFF -> 0, write bf16; a slot with sel_pos < 0 gets a zero row.
//
// Decode: decode8 (mxfp4.h), exact, no rounding.
//
// Work split: a 16-byte piece of output (8 elements) per thread and step; 16
// consecutive lanes write one 256-byte row, so stores are fully coalesced.
// The store stream (256 B per slot) is ~80% of the bytes, so the kernel is
// HBM-write bound; output uses non-temporal stores.
#include "mxfp4.h"

namespace xk {
namespace {

// A wave owns 4*STEPS consecutive slots. Lane l fetches sel_pos of slot l
// and resolves it to a physical token (two dependent loads for the whole
// wave); then STEPS steps each cover 4 slots x 16 pieces: the token index is
// broadcast from its lane, all steps' nibble/scale loads are issued
// together, and each step ends in one contiguous 1 KB store.
template <int STEPS>
__global__ __launch_bounds__(256) void mxfp4_gather_kernel(
    const uint32_t* __restrict__ kv_fp4,   // [NB*bs, 16] dwords (64 B per token)
    const uint8_t* __restrict__ kv_scale,  // [NB*bs, 4]
    const int32_t* __restrict__ block_table, int MB,
    const int32_t* __restrict__ sel_pos, const int32_t* __restrict__ row_seq,
    u32x4* __restrict__ out, int64_t n_slots, int k, int bs_log2, int bpr) {
  static_assert(4 * STEPS <= 64, "one lane resolves each slot of the wave");
  const int lane = threadIdx.x & 63;
  // bpr > 0 (a row is bpr whole workgroups): the workgroups of row r run on
  // XCD r % 8 (workgroup i runs on XCD i % 8). The one-workgroup-per-row
  // top-k kernels run row r there too, so the row's sel_pos loads hit that
  // XCD's L2 (a placement for speed only; any sel_pos gives the same output)
  int64_t blk = blockIdx.x;
  if (bpr > 0) {
    const int64_t m = blockIdx.x / 8;
    blk = ((m / bpr) * 8 + blockIdx.x % 8) * bpr + m % bpr;
  }
  const int64_t slot0 = (blk * 4 + (threadIdx.x >> 6)) * (4 * STEPS);
  if (slot0 >= n_slots) return;  // uniform per wave

  // 1. this lane's slot -> physical token (-1: padded slot or past the end)
  const int64_t s = slot0 + lane;
  int tok = -1;
  if (lane < 4 * STEPS && s < n_slots) {
    // the row's sequence does not depend on sel_pos: both loads go out
    // together, leaving two dependent hops (table, then data)
    const int64_t row = s / k;
    const int seq = row_seq ? row_seq[row] : int(row);
    const int p = sel_pos[s];
    if (p >= 0) {
      const int blk = block_table[int64_t(seq) * MB + (p >> bs_log2)];
      tok = (blk << bs_log2) + (p & ((1 << bs_log2) - 1));
    }
  }
  // 2. step `it` covers slots slot0 + 4*it + lane/16, piece lane%16
  const int piece = lane & 15;
  uint32_t nib[STEPS], sc[STEPS];
  int tk[STEPS];
#pragma unroll
  for (int it = 0; it < STEPS; ++it) {
    tk[it] = __shfl(tok, 4 * it + (lane >> 4));
    nib[it] = 0u;
    sc[it] = 0u;
    if (tk[it] >= 0) {
      nib[it] = kv_fp4[int64_t(tk[it]) * 16 + piece];
      sc[it] = kv_scale[int64_t(tk[it]) * 4 + (piece >> 2)];
    }
  }
#pragma unroll
  for (int it = 0; it < STEPS; ++it) {
    const int64_t slot = slot0 + 4 * it + (lane >> 4);
    if (slot >= n_slots) break;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (tk[it] >= 0) v = decode8(nib[it], sc[it]);
    __builtin_nontemporal_store(v, out + slot * 16 + piece);
  }
}

}  // namespace

hipError_t launch_gather(const uint8_t* kv_fp4, const uint8_t* kv_scale,
                         const int32_t* block_table, const int32_t* sel_pos,
                         const int32_t* row_seq, uint16_t* out, int R, int k, int MB,
                         int bs, hipStream_t stream) {
  const int64_t n_slots = int64_t(R) * k;
  const int bs_log2 = __builtin_ctz(unsigned(bs));
  // Two steps (8 slots) per wave at every size: measured against 1, 4, 8
  // and 16 steps, 2 gave the shortest gathers on the Flash and long prefill
  // shapes (2M slots: 90 us against 106 us for 16 steps) and matched the best
  // on the decode shapes. Shorter waves keep more independent
  // sel_pos -> table -> data chains in flight; a single step leaves most
  // lanes of the resolving load idle.
  constexpr int kSteps = 2;
  constexpr int64_t per_block = 4 * 4 * kSteps;  // 4 waves x 4*kSteps slots
  // rows of whole workgroups go to XCDs by row (the grid rounded up to eight
  // rows); otherwise workgroups take consecutive slots
  const int bpr = k % per_block == 0 ? int(k / per_block) : 0;
  const int64_t blocks = bpr ? (int64_t(R) + 7) / 8 * 8 * bpr : (n_slots + per_block - 1) / per_block;
  hipLaunchKernelGGL(mxfp4_gather_kernel<kSteps>, dim3(unsigned(blocks)), dim3(256), 0, stream,
                     reinterpret_cast<const uint32_t*>(kv_fp4), kv_scale, block_table, MB, sel_pos, row_seq,
                     reinterpret_cast<u32x4*>(out), n_slots, k, bs_log2, bpr);
  return hipGetLastError();
}

}  // namespace xk
