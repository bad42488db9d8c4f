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
// Sixteen lanes per 128-element row, eight consecutive elements per lane
// (one 16- or 32-byte load): a DPP row of 16 lanes is one data row, four
// lanes one 32-element group, and a lane's eight nibbles one 32-bit word
// of the cache row. A wave takes 4 rows per pass and issues the loads of
// its passes before any arithmetic, to keep enough bytes in flight.
// Integer codes are decided from float32 values exactly as the definitions
// state them (IEEE division, power-of-two scaling, rint = round to nearest
// even).
#include <math.h>

#include <type_traits>

#include "xk_internal.h"

namespace xk {
namespace {

constexpr int kQuantWaves = 4;  // waves per workgroup; a wave takes 4 rows per pass
// Passes per wave (rows 4 * P): one below kManyRows rows, four above.
// Measured on the long-prefill shapes (0.1 M rows: one pass 10-15% faster)
// and the Pro decode keys (2.6 M rows: four passes 9% faster for the mxfp4
// writer, equal for the fp8 rows).
constexpr int64_t kManyRows = int64_t(1) << 20;

template <int CTRL>
__device__ __forceinline__ float dpp_max(float v) {
  return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xF, 0xF,
                                                             false)));
}

// max over each quad of lanes (a 32-element group), then over each row of 16 (a data row)
__device__ __forceinline__ float quad_max(float v) { return dpp_max<0x4E>(dpp_max<0xB1>(v)); }
__device__ __forceinline__ float row16_max(float v) { return dpp_max<0x140>(dpp_max<0x141>(quad_max(v))); }

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

// Eight consecutive elements of a row: lane (row % 4 in the pass, l % 16)
// holds elements 8*(l % 16) .. +7.
struct Eight {
  u32x4 w[2];  // bf16: w[0] holds eight bf16; fp32: w[0], w[1] hold eight floats
};

template <bool BF16>
__device__ __forceinline__ Eight load8(const void* x, int64_t row, int col) {
  Eight e;
  if constexpr (BF16) {
    e.w[0] = reinterpret_cast<const u32x4*>(x)[row * 16 + col];
    e.w[1] = u32x4{0u, 0u, 0u, 0u};
  } else {
    e.w[0] = reinterpret_cast<const u32x4*>(x)[row * 32 + 2 * col];
    e.w[1] = reinterpret_cast<const u32x4*>(x)[row * 32 + 2 * col + 1];
  }
  return e;
}

template <bool BF16>
__device__ __forceinline__ float elem(const Eight& e, int i) {
  if constexpr (BF16) {
    const uint32_t w = e.w[0][i >> 1];
    return __uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
  } else {
    return __uint_as_float(e.w[i >> 2][i & 3]);
  }
}

template <bool BF16, int P>
__global__ __launch_bounds__(kQuantWaves * 64) void quant_fp8_rows_kernel(
    const void* __restrict__ x, uint8_t* __restrict__ out, float* __restrict__ scale, int64_t N) {
  const int lane = threadIdx.x & 63, col = lane & 15;
  const int64_t base = (int64_t(blockIdx.x) * kQuantWaves + (threadIdx.x >> 6)) * (4 * P) + (lane >> 4);
  Eight v[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {  // all loads first (rows past N read row N-1)
    const int64_t row = min(base + 4 * p, N - 1);
    v[p] = load8<BF16>(x, row, col);
  }
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int64_t row = base + 4 * p;
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(elem<BF16>(v[p], i)));
    amax = row16_max(amax);
    const float s = amax > 0.f ? amax / 448.f : 1.f;
    uint32_t lo = 0u, hi = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= e4m3_rne(elem<BF16>(v[p], i) / s) << (8 * i);
      hi |= e4m3_rne(elem<BF16>(v[p], 4 + i) / s) << (8 * i);
    }
    if (row < N) {
      reinterpret_cast<uint2*>(out)[row * 16 + col] = make_uint2(lo, hi);
      if (col == 0) scale[row] = s;
    }
  }
}

template <bool BF16, int P>
__global__ __launch_bounds__(kQuantWaves * 64) void mxfp4_write_kernel(
    const void* __restrict__ x, const int64_t* __restrict__ slots, uint8_t* __restrict__ kv_fp4,
    uint8_t* __restrict__ kv_scale, int64_t N, int64_t n_slots) {
  const int lane = threadIdx.x & 63, col = lane & 15;
  const int64_t base = (int64_t(blockIdx.x) * kQuantWaves + (threadIdx.x >> 6)) * (4 * P) + (lane >> 4);
  Eight v[P];
  int64_t slot[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int64_t row = min(base + 4 * p, N - 1);
    v[p] = load8<BF16>(x, row, col);
    slot[p] = base + 4 * p < N ? slots[row] : -1;
  }
#pragma unroll
  for (int p = 0; p < P; ++p) {
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(elem<BF16>(v[p], i)));
    amax = quad_max(amax);  // this lane's 32-element group
    int e = -127;
    if (amax > 0.f) {
      int ex;
      frexpf(amax, &ex);  // amax = m * 2^ex, m in [0.5, 1): floor(log2 amax) = ex - 1
      e = min(max(ex - 1 - 2, -127), 127);
    }
    uint32_t word = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) word |= e2m1_rne(ldexpf(elem<BF16>(v[p], i), -e)) << (4 * i);
    const int64_t sl = slot[p];
    if (sl >= 0 && sl < n_slots) {
      reinterpret_cast<uint32_t*>(kv_fp4)[sl * 16 + col] = word;
      if ((col & 3) == 0) kv_scale[sl * 4 + (col >> 2)] = uint8_t(e + 127);
    }
  }
}

}  // namespace

hipError_t launch_quant_fp8_rows(const void* x, bool bf16, uint8_t* out, float* scale, int64_t N,
                                 hipStream_t stream) {
  auto go = [&](auto bf16_tag, auto p_tag) {
    constexpr bool F = decltype(bf16_tag)::value;
    constexpr int P = decltype(p_tag)::value;
    const dim3 grid(unsigned((N + kQuantWaves * 4 * P - 1) / (kQuantWaves * 4 * P)));
    hipLaunchKernelGGL((quant_fp8_rows_kernel<F, P>), grid, dim3(kQuantWaves * 64), 0, stream, x, out, scale, N);
  };
  auto by_p = [&](auto bf16_tag) {
    if (N >= kManyRows)
      go(bf16_tag, std::integral_constant<int, 4>{});
    else
      go(bf16_tag, std::integral_constant<int, 1>{});
  };
  if (bf16)
    by_p(std::true_type{});
  else
    by_p(std::false_type{});
  return hipGetLastError();
}

hipError_t launch_mxfp4_write(const void* x, bool bf16, const int64_t* slots, uint8_t* kv_fp4,
                              uint8_t* kv_scale, int64_t N, int64_t n_slots, hipStream_t stream) {
  auto go = [&](auto bf16_tag, auto p_tag) {
    constexpr bool F = decltype(bf16_tag)::value;
    constexpr int P = decltype(p_tag)::value;
    const dim3 grid(unsigned((N + kQuantWaves * 4 * P - 1) / (kQuantWaves * 4 * P)));
    hipLaunchKernelGGL((mxfp4_write_kernel<F, P>), grid, dim3(kQuantWaves * 64), 0, stream, x, slots, kv_fp4,
                       kv_scale, N, n_slots);
  };
  auto by_p = [&](auto bf16_tag) {
    if (N >= kManyRows)
      go(bf16_tag, std::integral_constant<int, 4>{});
    else
      go(bf16_tag, std::integral_constant<int, 1>{});
  };
  if (bf16)
    by_p(std::true_type{});
  else
    by_p(std::false_type{});
  return hipGetLastError();
}

}  // namespace xk
