// Producers of the path's quantized inputs (gfx950).
//
//  * Per-row OCP fp8 (pages "DeepSeek V4 Flash on a single AMD MI300X", "FP8
//    format" fix: the indexer's fp8 cache is OCP e4m3 with FP8_MAX 448; "DeepSeek-
//    V4 on ATOM" tracker, "Quantization & Transform": act_quant BF16 -> FP8
//    e4m3 per 1x128): scale = amax / 448 (1 for an all-zero row), code =
//    e4m3 round-to-nearest-even of the float32 quotient x / scale. A key is
//    one row (per-token scale); q is T*H rows (per-(token, head) scale).
//  * mxfp4 cache writer, the inverse of the mxfp4 paged gather (page
//    "xkernels #28 -- DeepSeek-V4 serving support", comment shipping
//    mxfp4_paged_gather): per 32-element group the OCP MX rule, exponent e =
//    floor(log2 amax) - 2 clamped to [-127, 127] (-127 for an all-zero
//    group), E8M0 byte e + 127, element = E2M1 round-to-nearest-even of
//    x * 2^-e saturated to +-6, element 2i in the low nibble.
//
// One wave per 128-element row, two elements per lane: lane l holds
// elements 2l and 2l+1, so a row of 16 lanes is one 32-element group and a
// lane's two nibbles are one cache byte. Integer codes are decided from
// float32 values exactly as the definitions state them (IEEE division,
// power-of-two scaling, rint = round-to-nearest-even).
#include <math.h>

#include "xk_internal.h"

namespace xk {
namespace {

constexpr int kQuantWaves = 4;  // rows per 256-thread workgroup

// max over the 16 lanes of a DPP row (quad swaps, half mirror, mirror)
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x140, 0xF, 0xF, false)));
  return v;
}

// max over the wave (row maxima read as scalars)
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  const float a = fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)),
                        __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16)));
  const float b = fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)),
                        __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48)));
  return fmaxf(a, b);
}

// OCP e4m3 code of v: round to nearest even, saturated to +-448.
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t sign = __float_as_uint(v) >> 31 << 7;
  const float a = fminf(fabsf(v), 448.f);
  uint32_t code;
  if (a < 0.015625f) {  // below 2^-6: subnormal, quantum 2^-9 (8 rounds up to the least normal)
    code = uint32_t(rintf(a * 512.f));
  } else {
    int e = int((__float_as_uint(a) >> 23) & 0xFF) - 127;  // a is a normal float here
    float m = rintf(ldexpf(a, 3 - e));                       // 3 mantissa bits: m in [8, 16]
    if (m == 16.f) {
      m = 8.f;
      ++e;
    }
    code = (uint32_t(e + 7) << 3) | (uint32_t(m) - 8u);
  }
  return sign | code;
}

// E2M1 code of v: round to nearest even (ties to the code with mantissa 0),
// saturated to +-6. Magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 are codes 0..7.
__device__ __forceinline__ uint32_t e2m1_rne(float v) {
  const uint32_t sign = __float_as_uint(v) >> 31 << 3;
  const float a = fabsf(v);
  uint32_t m = a > 5.f ? 7u : a >= 3.5f ? 6u : a > 2.5f ? 5u : a >= 1.75f ? 4u
             : a > 1.25f ? 3u : a >= 0.75f ? 2u : a > 0.25f ? 1u : 0u;
  return sign | m;
}

template <bool BF16>
__device__ __forceinline__ void load_pair(const void* x, int64_t row, int lane, float& x0, float& x1) {
  if constexpr (BF16) {
    const uint32_t w = reinterpret_cast<const uint32_t*>(x)[row * 64 + lane];  // two bf16
    x0 = __uint_as_float(w << 16);
    x1 = __uint_as_float(w & 0xFFFF0000u);
  } else {
    const float2 f = reinterpret_cast<const float2*>(x)[row * 64 + lane];
    x0 = f.x;
    x1 = f.y;
  }
}

template <bool BF16>
__global__ __launch_bounds__(kQuantWaves * 64) void quant_fp8_rows_kernel(
    const void* __restrict__ x, uint8_t* __restrict__ out, float* __restrict__ scale, int64_t N) {
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * kQuantWaves + (threadIdx.x >> 6);
  if (row >= N) return;  // whole wave
  float x0, x1;
  load_pair<BF16>(x, row, lane, x0, x1);
  const float amax = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
  const float s = amax > 0.f ? amax / 448.f : 1.f;
  const uint32_t c = e4m3_rne(x0 / s) | (e4m3_rne(x1 / s) << 8);
  reinterpret_cast<uint16_t*>(out)[row * 64 + lane] = uint16_t(c);
  if (lane == 0) scale[row] = s;
}

template <bool BF16>
__global__ __launch_bounds__(kQuantWaves * 64) void mxfp4_write_kernel(
    const void* __restrict__ x, const int64_t* __restrict__ slots, uint8_t* __restrict__ kv_fp4,
    uint8_t* __restrict__ kv_scale, int64_t N, int64_t n_slots) {
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * kQuantWaves + (threadIdx.x >> 6);
  if (row >= N) return;
  const int64_t slot = slots[row];
  if (slot < 0 || slot >= n_slots) return;  // skipped row (whole wave)
  float x0, x1;
  load_pair<BF16>(x, row, lane, x0, x1);
  const float amax = row16_max(fmaxf(fabsf(x0), fabsf(x1)));  // this lane's 32-element group
  int e = -127;
  if (amax > 0.f) {
    int ex;
    frexpf(amax, &ex);  // amax = m * 2^ex, m in [0.5, 1): floor(log2 amax) = ex - 1
    e = min(max(ex - 1 - 2, -127), 127);
  }
  const uint32_t b = e2m1_rne(ldexpf(x0, -e)) | (e2m1_rne(ldexpf(x1, -e)) << 4);
  kv_fp4[slot * 64 + lane] = uint8_t(b);
  if ((lane & 15) == 0) kv_scale[slot * 4 + (lane >> 4)] = uint8_t(e + 127);
}

}  // namespace

hipError_t launch_quant_fp8_rows(const void* x, bool bf16, uint8_t* out, float* scale, int64_t N,
                                 hipStream_t stream) {
  const dim3 grid(unsigned((N + kQuantWaves - 1) / kQuantWaves));
  if (bf16)
    hipLaunchKernelGGL(quant_fp8_rows_kernel<true>, grid, dim3(kQuantWaves * 64), 0, stream, x, out, scale, N);
  else
    hipLaunchKernelGGL(quant_fp8_rows_kernel<false>, grid, dim3(kQuantWaves * 64), 0, stream, x, out, scale, N);
  return hipGetLastError();
}

hipError_t launch_mxfp4_write(const void* x, bool bf16, const int64_t* slots, uint8_t* kv_fp4,
                              uint8_t* kv_scale, int64_t N, int64_t n_slots, hipStream_t stream) {
  const dim3 grid(unsigned((N + kQuantWaves - 1) / kQuantWaves));
  if (bf16)
    hipLaunchKernelGGL(mxfp4_write_kernel<true>, grid, dim3(kQuantWaves * 64), 0, stream, x, slots, kv_fp4,
                       kv_scale, N, n_slots);
  else
    hipLaunchKernelGGL(mxfp4_write_kernel<false>, grid, dim3(kQuantWaves * 64), 0, stream, x, slots, kv_fp4,
                       kv_scale, N, n_slots);
  return hipGetLastError();
}

}  // namespace xk
