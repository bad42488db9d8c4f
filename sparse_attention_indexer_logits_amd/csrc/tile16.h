// The MFMA score tiles shared by the logits kernels and by the fused
// top-k's recompute path (gfx950). Every kernel that scores a key of a given
// call goes through the same scorer with the same operands, so the key's
// score has the same bits whichever kernel computes it: bf16 queries (and
// fp8 decode queries) through Query16 and subtile_total on 16x16 tiles, fp8
// prefill queries through Query32 and tile_total32 on 32x32 tiles.
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
  // A block scale 2^-25 (E8M0 byte 102), B scale 1: every e4m3 score
  // |q8 . k8| <= 128 * 448 * 448 < 2^25 arrives in (-1, 1), so the epilogue
  // can take the ReLU with an output clamp to [0, 1]. Scaling by a power of
  // two changes no rounding, so the sum equals the unit-scaled one * 2^-25.
  static constexpr int kScaleShift = 25;
  __device__ static f32x4 mma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127 - kScaleShift, 0, 127);
  }
};

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// ReLU of two fp8-path scores (each in (-1, 1)) rounded to nearest-even f16:
// the compiler folds the clamp to [0, 1] into v_cvt_pk_f16_f32 (one VALU op
// for two heads). Measured on gfx950: that instruction's clamp bit clamps,
// while v_cvt_pkrtz_f16_f32 ignores its own (negative values pass), so the
// round-toward-zero convert must not be used here.
__device__ __forceinline__ f16x2 relu_pk_f16(float x0, float x1) {
  const f16x2 h = __builtin_convertvector(f32x2{x0, x1}, f16x2);
  return __builtin_elementwise_min(__builtin_elementwise_max(h, f16x2{0, 0}), f16x2{1, 1});
}

// acc + x * w on both f16 halves, one rounding each (v_pk_fma_f16).
// Measured on gfx950: packed f16 FMAs issue alongside the 32x32x64 fp8
// MFMAs, while v_dot2_f32_f16 / v_dot2c_f32_f16 do not overlap them at all
// (even when independent of them), so the epilogue avoids the dot
// instructions.
__device__ __forceinline__ f16x2 pk_fma(f16x2 x, f16x2 w, f16x2 acc) { return __builtin_elementwise_fma(x, w, acc); }
// lo + hi of a packed f16 pair as an fp32 (one rounding of the exact sum,
// the same bits as converting both and adding) in one v_fma_mix_f32
// (lo * 1.0 + hi, f16 sources): the compiler otherwise converts each half
// and adds, three VALU ops. An ALU-only asm, not volatile, so it is
// scheduled like any arithmetic.
__device__ __forceinline__ float pair_sum(f16x2 h) {
  float r;
  asm("v_fma_mix_f32 %0, %1, 1.0, %1 op_sel:[0,0,1] op_sel_hi:[1,0,1]" : "=v"(r) : "v"(h));
  return r;
}
// the fp32 sum of two packed f16 partial sums (measured on the long fp8
// prefill logits: 1145.7 -> 1133.6 us, identical outputs)
__device__ __forceinline__ float sum4(f16x2 a, f16x2 b) { return pair_sum(a) + pair_sum(b); }

// The head weights in the form the epilogue takes.
//  bf16: fp32 weights; per head one v_max (ReLU) and one fma.
//  fp8:  the scores arrive scaled into (-1, 1) (Mma16<true>), so one clamped
//        f16 convert takes the ReLU of two heads, and one v_pk_fma_f16
//        multiplies both by their f16 weights and adds them to two f16
//        partial sums: one VALU op per head instead of two. Each partial sum
//        takes 8 heads (4 on 16x16 tiles), and the partial sums are added in
//        fp32. The weights are w * sq * 2^e rounded to nearest f16, with e
//        putting the query's largest |w * sq| in [2^11, 2^12): every term is
//        then below 2^12 and every partial sum below 2^15, inside the f16
//        range. `post` = 2^(25 - e) undoes both scalings exactly on the
//        finished score. Each f16 rounding is a relative error of at most
//        2^-11 (the fp8 inputs themselves carry 2^-4).
template <bool FP8>
struct Query16 {
  using M = Mma16<FP8>;
  typename M::Frag a[4][M::kSteps];  // [M-tile][step]
  float wr[4][4];                    // bf16: weight of head 16*mt + 4*(lane/16) + i
  f16x2 wh[4][2];                    // fp8: f16 weights of heads (i = 0, 1) and (2, 3)
  float post;                        // fp8: 2^(25 - e); bf16: 1

  // wf[mt][i]: the weight (times the fp8 q scale) of head 16*mt + 4*(lane/16) + i.
  // Every lane of the wave must call this (fp8 takes a maximum across lanes).
  __device__ void set_weights(const float (&wf)[4][4]) {
    if constexpr (FP8) {
      float m = 0.f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(wf[mt][i]));
      // lanes l, l^16, l^32, l^48 hold the four head groups
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      // m = f * 2^x with f in [0.5, 1): m * 2^(12 - x) lies in [2^11, 2^12)
      const int e = m > 0.f ? min(max(12 - __builtin_amdgcn_frexp_expf(m), -100), 140) : 0;
      post = __builtin_ldexpf(1.f, M::kScaleShift - e);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 2; ++i)
          wh[mt][i] = f16x2{_Float16(__builtin_ldexpf(wf[mt][2 * i], e)),
                            _Float16(__builtin_ldexpf(wf[mt][2 * i + 1], e))};
    } else {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) wr[mt][i] = wf[mt][i];
      post = 1.f;
    }
  }

  __device__ void load(const uint8_t* qrow, const float* wrow, const float* sqrow, int lane) {
    const int g = lane >> 4, r = lane & 15;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int s = 0; s < M::kSteps; ++s)
        a[mt][s] = M::load(qrow + ((16 * mt + r) * kHeadDim + M::dofs(s, g)) * M::kElemBytes);
    float wf[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 16 * mt + 4 * g + i;
        wf[mt][i] = FP8 ? wrow[h] * sqrow[h] : wrow[h];
      }
    set_weights(wf);
  }
  __device__ void zero() {
    float wf[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int s = 0; s < M::kSteps; ++s) a[mt][s] = typename M::Frag{};
#pragma unroll
      for (int i = 0; i < 4; ++i) wf[mt][i] = 0.f;
    }
    set_weights(wf);
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
    if constexpr (FP8) {
      f16x2 h0 = {0, 0}, h1 = {0, 0};
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        h0 = pk_fma(relu_pk_f16(acc[mt][0], acc[mt][1]), wh[mt][0], h0);
        h1 = pk_fma(relu_pk_f16(acc[mt][2], acc[mt][3]), wh[mt][1], h1);
      }
      return sum4(h0, h1);
    } else {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        p0 = fmaf(wr[mt][0], fmaxf(acc[mt][0], 0.f), p0);
        p1 = fmaf(wr[mt][1], fmaxf(acc[mt][1], 0.f), p1);
        p0 = fmaf(wr[mt][2], fmaxf(acc[mt][2], 0.f), p0);
        p1 = fmaf(wr[mt][3], fmaxf(acc[mt][3], 0.f), p1);
      }
    }
    return p0 + p1;
  }
  // this lane's 16-head partial score of key (lane % 16) of a 16-key subtile
  __device__ float partial(const typename M::Frag (&b)[M::kSteps]) const {
    f32x4 acc[4];
    mma(b, acc);
    return epilogue(acc);
  }
  // the finished score of a key from its head sum (subtile_total) and, for
  // fp8, the key's dequant scale
  __device__ float finish(float tot, float sk) const { return FP8 ? tot * post * sk : tot; }
};

// fp8 queries on 32x32 tiles (v_mfma_scale_f32_32x32x64_f8f6f4): the prefill
// kernel and the fused path's rescoring, so both give a key the same bits.
// The 64 heads are two 32-row M-tiles, 32 keys the N dimension and D = 128
// two 64-deep steps. Measured on gfx950: this MFMA (16 passes) leaves most of
// the issue slots of its run to VALU work, where the 16x16x128 form (8
// passes) hides about half, and that is what the epilogue needs (one VALU op
// per head and key). Accumulator layout (measured): lane l, element e holds
// column l % 32 and row 8*(e/4) + 4*(l/32) + e%4, so a lane holds 16 heads of
// one key per M-tile and lanes l, l^32 together hold all 64. A lane (r, g)
// = (l % 32, l / 32) of either operand supplies bytes [64s + 32g, +32) of its
// row (q head row or key row) in step s; both 8-bit operands follow one K
// order, so the pairing is consistent whatever that order is.
struct Query32 {
  using M = Mma16<true>;                 // the e4m3 scale shift (2^-25) and the epilogue's ranges
  i32x8 a[2][2];                         // [M-tile][step]
  f16x2 wh[2][8];                        // [M-tile][2*i + p]: heads 32*mt + 8*i + 4*(lane/32) + 2*p + {0, 1}
  float post;                            // 2^(25 - e)

  __device__ static i32x8 load32(const uint8_t* p) {
    const i32x4 lo = *reinterpret_cast<const i32x4*>(p);
    const i32x4 hi = *reinterpret_cast<const i32x4*>(p + 16);
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  __device__ static int head(int mt, int e, int lane) { return 32 * mt + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3); }

  // wf[mt][e]: weight (times the q scale) of head(mt, e, lane); every lane
  // of the wave calls this (the largest |weight| is taken across lanes)
  __device__ void set_weights(const float (&wf)[2][16]) {
    float m = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(wf[mt][e]));
    m = fmaxf(m, __shfl_xor(m, 32));  // lanes l and l^32 hold the two halves of the heads
    const int e2 = m > 0.f ? min(max(12 - __builtin_amdgcn_frexp_expf(m), -100), 140) : 0;
    post = __builtin_ldexpf(1.f, M::kScaleShift - e2);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        wh[mt][i] = f16x2{_Float16(__builtin_ldexpf(wf[mt][2 * i], e2)), _Float16(__builtin_ldexpf(wf[mt][2 * i + 1], e2))};
  }
  __device__ void load(const uint8_t* qrow, const float* wrow, const float* sqrow, int lane) {
    const int r = lane & 31, g = lane >> 5;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int s = 0; s < 2; ++s) a[mt][s] = load32(qrow + (32 * mt + r) * kHeadDim + 64 * s + 32 * g);
    float wf[2][16];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int h = head(mt, e, lane);
        wf[mt][e] = wrow[h] * sqrow[h];
      }
    set_weights(wf);
  }
  __device__ void zero() {
    float wf[2][16];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int s = 0; s < 2; ++s) a[mt][s] = i32x8{};
#pragma unroll
      for (int e = 0; e < 16; ++e) wf[mt][e] = 0.f;
    }
    set_weights(wf);
  }
  // this lane's 32-head partial score (ReLU, weight, sum) of key lane % 32 of
  // a 32-key block whose B fragments (steps 0, 1) are b. The two M-tiles'
  // MFMAs alternate, so each step's MFMA has the other tile's in between
  // before its result is needed.
  __device__ float partial(const i32x8 (&b)[2]) const {
    constexpr int kSa = 127 - M::kScaleShift;
    f32x16 acc0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[0][0], b[0], f32x16{}, 0, 0, 0, kSa, 0, 127);
    f32x16 acc1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[1][0], b[0], f32x16{}, 0, 0, 0, kSa, 0, 127);
    acc0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[0][1], b[1], acc0, 0, 0, 0, kSa, 0, 127);
    acc1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[1][1], b[1], acc1, 0, 0, 0, kSa, 0, 127);
    // keep all four MFMAs ahead of the epilogue (left alone, the scheduler
    // runs the two M-tiles one after the other through one accumulator)
    __builtin_amdgcn_sched_barrier(0);
    f16x2 h0 = {0, 0}, h1 = {0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i) h0 = pk_fma(relu_pk_f16(acc0[2 * i], acc0[2 * i + 1]), wh[0][i], h0);
#pragma unroll
    for (int i = 0; i < 8; ++i) h1 = pk_fma(relu_pk_f16(acc1[2 * i], acc1[2 * i + 1]), wh[1][i], h1);
    return sum4(h0, h1);
  }
  __device__ float finish(float tot, float sk) const { return tot * post * sk; }
};

// Full scores of a 64-key tile from the partials of its two 32-key blocks:
// lane l ends with key l of the tile (block l / 32, key l % 32), the sum of
// that key's partials in lanes l % 32 and l % 32 + 32. (v_permlane32_swap
// trades the upper half of the first operand for the lower half of the
// second.)
__device__ __forceinline__ float tile_total32(float p_lo, float p_hi) {
  const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(p_lo), __float_as_uint(p_hi), false, false);
  return __uint_as_float(x[0]) + __uint_as_float(x[1]);
}

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
