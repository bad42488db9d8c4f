// The 16x16 MFMA score tile shared by the logits kernels and by the fused
// top-k's recompute path (gfx950). Every kernel that scores a key goes
// through Query16::partial and subtile_total with the same operands, so a
// key's score has the same bits whichever kernel computes it.
#pragma once

#include "xk_internal.h"

namespace xk {

// For one query the 64 heads are four 16-row
// M-tiles and 16 keys the N dimension; a 16x16 fp32 accumulator gives lane l
// rows 4*(l/16)+i (i < 4) of column l%16, i.e. 16 heads of one key per lane
// across the four M-tiles. That keeps the per-query state small (16 head
// weights + 16 accumulators per lane) so a wave can own QW queries and each
// B fragment read from LDS feeds 4*QW MFMAs. After the four 16-key subtiles
// of a 64-key tile, three lane swaps and adds leave lane l with the full
// score of key l, so stores are 64 consecutive floats.
template <bool FP8>
struct Mma16;

template <>
struct Mma16<false> {  // bf16: v_mfma_f32_16x16x32_bf16, 4 steps over D = 128
  using Frag = bf16x8;
  static constexpr int kSteps = 4;
  static constexpr int kElemBytes = 2;
  __device__ static int dofs(int s, int g) { return 32 * s + 8 * g; }  // g = lane / 16
  __device__ static Frag load(const uint8_t* p) { return *reinterpret_cast<const Frag*>(p); }
  __device__ static f32x4 mma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mma16<true> {  // OCP e4m3: v_mfma_scale_f32_16x16x128_f8f6f4, 1 step
  using Frag = i32x8;
  static constexpr int kSteps = 1;
  static constexpr int kElemBytes = 1;
  __device__ static int dofs(int, int g) { return 32 * g; }
  __device__ static Frag load(const uint8_t* p) {
    const i32x4 lo = *reinterpret_cast<const i32x4*>(p);
    const i32x4 hi = *reinterpret_cast<const i32x4*>(p + 16);
    return Frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  __device__ static f32x4 mma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
};

template <bool FP8>
struct Query16 {
  using M = Mma16<FP8>;
  typename M::Frag a[4][M::kSteps];  // [M-tile][step]
  float wr[4][4];                    // head 16*mt + 4*(lane/16) + i

  __device__ void load(const uint8_t* qrow, const float* wrow, const float* sqrow, int lane) {
    const int g = lane >> 4, r = lane & 15;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int s = 0; s < M::kSteps; ++s)
        a[mt][s] = M::load(qrow + ((16 * mt + r) * kHeadDim + M::dofs(s, g)) * M::kElemBytes);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 16 * mt + 4 * g + i;
        wr[mt][i] = FP8 ? wrow[h] * sqrow[h] : wrow[h];
      }
  }
  __device__ void zero() {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int s = 0; s < M::kSteps; ++s) a[mt][s] = typename M::Frag{};
#pragma unroll
      for (int i = 0; i < 4; ++i) wr[mt][i] = 0.f;
    }
  }
  // the four M-tiles' accumulators of a 16-key subtile (steps outermost, so
  // consecutive MFMAs are independent)
  __device__ void mma(const typename M::Frag (&b)[M::kSteps], f32x4 (&acc)[4]) const {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < M::kSteps; ++s)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[mt] = M::mma(a[mt][s], b[s], acc[mt]);
  }
  // this lane's 16-head partial score (ReLU, head weight, sum) of key
  // (lane % 16) from the subtile's accumulators
  __device__ float epilogue(const f32x4 (&acc)[4]) const {
    float p0 = 0.f, p1 = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      p0 = fmaf(wr[mt][0], fmaxf(acc[mt][0], 0.f), p0);
      p1 = fmaf(wr[mt][1], fmaxf(acc[mt][1], 0.f), p1);
      p0 = fmaf(wr[mt][2], fmaxf(acc[mt][2], 0.f), p0);
      p1 = fmaf(wr[mt][3], fmaxf(acc[mt][3], 0.f), p1);
    }
    return p0 + p1;
  }
  // this lane's 16-head partial score of key (lane % 16) of a 16-key subtile
  __device__ float partial(const typename M::Frag (&b)[M::kSteps]) const {
    f32x4 acc[4];
    mma(b, acc);
    return epilogue(acc);
  }
};

// p[st] = this lane's partial for key 16*st + lane%16; returns the full score
// of key `lane` (sum over the four lane groups).
__device__ __forceinline__ float subtile_total(const float (&p)[4], int lane) {
  // v_permlane32_swap: lanes 32-63 of the first operand trade places with
  // lanes 0-31 of the second. After swapping (p0, p2) the lower half holds
  // subtile 0 of both halves and the upper half subtile 2 of both, so one add
  // sums each key over the two halves (likewise p1, p3).
  const auto x02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[0]), __float_as_uint(p[2]), false, false);
  const auto x13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[1]), __float_as_uint(p[3]), false, false);
  const float a0 = __uint_as_float(x02[0]) + __uint_as_float(x02[1]);
  const float a1 = __uint_as_float(x13[0]) + __uint_as_float(x13[1]);
  // v_permlane16_swap does the same for 16-lane groups within each half:
  // even groups end with a0 of both groups, odd groups with a1
  const auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(a0), __float_as_uint(a1), false, false);
  (void)lane;
  return __uint_as_float(y[0]) + __uint_as_float(y[1]);
}

}  // namespace xk
