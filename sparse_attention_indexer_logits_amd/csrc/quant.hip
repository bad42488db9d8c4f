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
// Integer codes are decided from the same float32 values the definitions
// give (the correctly rounded quotient x / scale, power-of-two scaling), and
// the rounding to e4m3 or E2M1 is the hardware conversion, which rounds to
// nearest even as both formats specify.
#include <math.h>

#include <type_traits>

#include "xk_internal.h"

namespace xk {
namespace {

constexpr int kQuantWaves = 4;  // waves per workgroup; a wave takes 4 rows per pass
// Passes per wave (rows 4 * P) of the fp8 rows: one below kManyRows rows, two
// above. Measured on the Pro decode keys (2.5 M rows): two passes 6% faster
// than one or four; on the long-prefill shapes (0.1 M rows) one to eight
// passes time alike. The mxfp4 writer takes one pass at every size (8%
// faster than two or four on the Pro decode keys).
constexpr int64_t kManyRows = int64_t(1) << 20;

template <int CTRL>
__device__ __forceinline__ float dpp_max(float v) {
  return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xF, 0xF,
                                                             false)));
}

// max over each quad of lanes (a 32-element group), then over each row of 16 (a data row)
__device__ __forceinline__ float quad_max(float v) { return dpp_max<0x4E>(dpp_max<0xB1>(v)); }
__device__ __forceinline__ float row16_max(float v) { return dpp_max<0x140>(dpp_max<0x141>(quad_max(v))); }

// Four OCP e4m3 codes (element i in byte i) of values already clamped to
// [-448, 448]; the conversion rounds to nearest even.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true));
}

// The float32 quotient x / s rounded to nearest even, as an IEEE division
// gives it, wherever |x / s| >= 2^-10 (below that the e4m3 code is a zero of
// x's sign, and the sign is kept). rs is the double reciprocal of s (relative
// error 2^-53), so x * rs is within 2^-52 (relative) of the exact quotient.
// A quotient of two float32 numbers lies more than 2^-49 (relative) from any
// float32 rounding midpoint M: M has 25 significant bits with the last one
// set, so x never equals M * s, and x - M * s is a nonzero multiple of the
// smaller of x's last-bit weight and the product of M's and s's, at least
// 2^-49 of M * s. One rounding of x * rs to float32 therefore lands where the
// exact quotient's does.
__device__ __forceinline__ float quotient(float x, double rs) { return float(double(x) * rs); }

// Two E2M1 codes into byte sel of old, a in the low nibble and b in the high
// one, of values in (-8, 8): round to nearest even, magnitudes beyond 6
// saturate.
__device__ __forceinline__ uint32_t e2m1x2(uint32_t old, float a, float b, int sel) {
  switch (sel) {  // the byte select is an immediate of the instruction
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.f, 3);
  }
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
    const double rs = 1.0 / double(s);
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = __builtin_amdgcn_fmed3f(quotient(elem<BF16>(v[p], i), rs), -448.f, 448.f);
    const uint32_t lo = e4m3x4(q[0], q[1], q[2], q[3]), hi = e4m3x4(q[4], q[5], q[6], q[7]);
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
    for (int i = 0; i < 4; ++i)  // |x * 2^-e| < 8 by the choice of e
      word = e2m1x2(word, ldexpf(elem<BF16>(v[p], 2 * i), -e), ldexpf(elem<BF16>(v[p], 2 * i + 1), -e), i);
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
      go(bf16_tag, std::integral_constant<int, 2>{});
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
  if (bf16)
    go(std::true_type{}, std::integral_constant<int, 1>{});
  else
    go(std::false_type{}, std::integral_constant<int, 1>{});
  return hipGetLastError();
}

}  // namespace xk
