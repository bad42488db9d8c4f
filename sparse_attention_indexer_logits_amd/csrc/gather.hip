// mxfp4 paged KV gather -> bf16 (gfx950).
//
// Semantics (page "xkernels #28 -- DeepSeek-V4 serving support", comment
// shipping mxfp4_paged_gather): per (row, top-k slot) look up the block
// table, decode E2M1 nibbles times the E8M0 group scale 2^(b-127) with
// 0xFF -> 0, write bf16; a slot with sel_pos < 0 gets a zero row.
//
// The decode builds the bf16 bit pattern with integer ops: an E2M1 magnitude
// is 0.5, or (1 + m/2) * 2^(e-1), so times 2^(b-127) it is a bf16 with
// biased exponent e-1+b (b-1 for code 1) and one mantissa bit; the only
// non-normal outcomes are the two subnormal exponents (b <= 1) and overflow
// to inf (exponent >= 255). No rounding ever happens.
//
// Work split: a 16-byte piece of output (8 elements) per thread and step; 16
// consecutive threads write one 256-byte row, so stores are fully coalesced.
// The store stream (256 B per slot) is ~80% of the bytes, so the kernel is
// HBM-write bound; output uses non-temporal stores.
#include "xk_internal.h"

namespace xk {
namespace {

__device__ __forceinline__ uint32_t e2m1_e8m0_to_bf16(uint32_t code, uint32_t scale) {
  const uint32_t sign = (code & 8u) << 12;
  const uint32_t mag = code & 7u;
  if (mag == 0u || scale == 0xFFu) return sign;  // +-0 * s, or x * 0
  const bool normal_code = mag >= 2u;            // codes 2..7: e >= 1
  const int biased = normal_code ? int(mag >> 1) - 1 + int(scale) : int(scale) - 1;
  const uint32_t mant = normal_code ? (mag & 1u) : 0u;
  if (biased >= 255) return sign | 0x7F80u;                       // overflow -> inf
  if (biased >= 1) return sign | (uint32_t(biased) << 7) | (mant << 6);
  // biased in {-1, 0}: subnormal, value (2 + mant) * 2^(biased-128) = field * 2^-133
  return sign | ((2u + mant) << (biased + 5));
}

// Each thread owns kPer pieces spaced one grid apart and runs their
// dependent loads (sel_pos -> block table -> nibbles + scale) side by side,
// so kPer independent chains are in flight per thread.
constexpr int kPer = 4;

__global__ __launch_bounds__(256) void mxfp4_gather_kernel(
    const uint32_t* __restrict__ kv_fp4,   // [NB*bs, 16] dwords (64 B per token)
    const uint8_t* __restrict__ kv_scale,  // [NB*bs, 4]
    const int32_t* __restrict__ block_table, int MB,
    const int32_t* __restrict__ sel_pos, const int32_t* __restrict__ row_seq,
    u32x4* __restrict__ out, int64_t n_pieces, int k, int bs_log2) {
  const int64_t stride = int64_t(gridDim.x) * 256;
  const int64_t first = int64_t(blockIdx.x) * 256 + threadIdx.x;
  int p[kPer];
  int64_t blk[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int64_t piece = first + i * stride;
    p[i] = piece < n_pieces ? sel_pos[piece >> 4] : -1;
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    blk[i] = 0;
    if (p[i] >= 0) {
      const int64_t row = ((first + i * stride) >> 4) / k;
      const int seq = row_seq ? row_seq[row] : int(row);
      blk[i] = block_table[int64_t(seq) * MB + (p[i] >> bs_log2)];
    }
  }
  uint32_t nib[kPer], sc[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    nib[i] = 0u;
    sc[i] = 0u;
    if (p[i] >= 0) {
      const int part = int((first + i * stride) & 15);  // elements [8*part, 8*part+8)
      const int64_t token = (blk[i] << bs_log2) + (p[i] & ((1 << bs_log2) - 1));
      nib[i] = kv_fp4[token * 16 + part];
      sc[i] = kv_scale[token * 4 + (part >> 2)];
    }
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int64_t piece = first + i * stride;
    if (piece >= n_pieces) break;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (p[i] >= 0) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t byte = (nib[i] >> (8 * b)) & 0xFFu;
        v[b] = e2m1_e8m0_to_bf16(byte & 0xFu, sc[i]) | (e2m1_e8m0_to_bf16(byte >> 4, sc[i]) << 16);
      }
    }
    __builtin_nontemporal_store(v, out + piece);
  }
}

}  // namespace

hipError_t launch_gather(const uint8_t* kv_fp4, const uint8_t* kv_scale,
                         const int32_t* block_table, const int32_t* sel_pos,
                         const int32_t* row_seq, uint16_t* out, int R, int k, int MB,
                         int bs, hipStream_t stream) {
  const int64_t n_pieces = int64_t(R) * k * 16;
  const int bs_log2 = __builtin_ctz(unsigned(bs));
  const int64_t blocks = (n_pieces + 256 * kPer - 1) / (256 * kPer);
  hipLaunchKernelGGL(mxfp4_gather_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream,
                     reinterpret_cast<const uint32_t*>(kv_fp4), kv_scale, block_table, MB,
                     sel_pos, row_seq, reinterpret_cast<u32x4*>(out), n_pieces, k, bs_log2);
  return hipGetLastError();
}

}  // namespace xk
