// DSA indexer logits on gfx950 MFMA.
//
// Computes (page "xkernels #27 -- [AMD/MI300A] DeepSeek-V4 DSA indexer +
// attention", comment announcing dsa_indexer_logits):
//   logits[b,t,j] = sum_h w[b,t,h] * relu(q[b,t,h,:] . k[b,j,:]),  j <= limit[b,t]
//   logits[b,t,j] = -inf                                             otherwise
// with H = 64 heads, D = 128, one shared key per position (MQA).
//
// Mapping onto the matrix cores: for one query the 64 heads are the M
// dimension, keys the N dimension and D the contraction. Because the
// accumulator layout puts several rows (heads) of ONE column (key) in each
// lane, the ReLU, the head weight and most of the head sum run in registers
// of that lane and only a few cross-lane adds finish the 64-head sum; the
// score never leaves registers until it is final.
//
// The dequant scales of fp8 inputs are positive, so relu(sq*sk*x) =
// sq*sk*relu(x): sq folds into the head weight and sk multiplies the
// finished score. fp8 operands use the f8f6f4 MFMAs with OCP e4m3 on both
// sides; the A block scale 2^-25 brings every e4m3 score into (-1, 1), so the
// ReLU and the rounding to f16 take one clamped packed convert per two
// heads, and the weighted head sum one v_fma_mix_f32 per head (tile16.h).
//
// Two kernels:
//  * decode  (few queries, long rows; HBM bound; 16x16 tiles). A workgroup
//    owns one query and a key chunk; each wave streams its own keys with B
//    fragments loaded from HBM straight into registers, 16 KB in flight.
//  * prefill (many queries; MFMA bound). A workgroup owns 4 (bf16) or 8
//    (fp8) queries, one per wave, and a key chunk; three rotating LDS key
//    tiles (64 bf16 or 128 fp8 keys) are shared by all its waves. bf16 runs
//    on 16x16 tiles, fp8 on 32x32 tiles (v_mfma_scale_f32_32x32x64_f8f6f4),
//    whose longer MFMAs leave more issue slots to the epilogue's VALU work.
// Causal tiles that lie wholly past a query's limit are skipped and filled
// with -inf.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "tile16.h"

namespace xk {
namespace {

__device__ __forceinline__ int clamp_limit(const int32_t* limit, int64_t bt, int K) {
  return limit ? min(limit[bt], K - 1) : K - 1;
}

// ---------------------------------------------------------------------------
// decode: 1-D grid over (B*T rows) x (key chunks); a workgroup owns one query
// and a key chunk, split into one contiguous range per wave. q and its head
// weights are staged once in LDS and then held by every wave as A fragments
// in registers. Each wave streams its keys as 16-key subtiles whose B
// fragments are loaded from HBM straight into registers (lane l: key l%16,
// the 16-byte pieces of d named by Mma16::dofs), 16 KB in flight per wave;
// 64 keys (four subtiles) make one coalesced 256-byte store. No LDS traffic
// and no barrier inside the key loop.
constexpr int kDecWaves = 2;    // dense keys: two waves x a 256- or 384-key chunk
constexpr int kPagedWaves = 4;  // paged keys: four waves (the paged kernel below)
constexpr int kDecGroup = 64;  // keys per store: four 16-key subtiles

template <bool FP8>
__global__ __launch_bounds__(kDecWaves * 64, 2) void logits_decode_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale,
    const uint8_t* __restrict__ k, const float* __restrict__ k_scale,
    const float* __restrict__ w, const int32_t* __restrict__ limit,
    float* __restrict__ out, int T, int K, int keys_per_wg, int n_chunks) {
  using M = Mma16<FP8>;
  using Frag = typename M::Frag;
  constexpr int kRowBytes = kHeadDim * M::kElemBytes;  // 256 or 128
  constexpr int kPitch = kRowBytes + 16;               // padded LDS row
  constexpr int kLanesPerRow = kRowBytes / 16;
  constexpr int kDecRing = 16 * 1024 / (16 * kRowBytes);  // subtiles in flight: 4 or 8
  __shared__ __attribute__((aligned(16))) uint8_t q_lds[kHeads * kPitch];
  __shared__ __attribute__((aligned(16))) float w_lds[kHeads];

  // the wave index in a scalar register: per-wave values derived from it
  // (rows, buffer descriptors) then stay scalar
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, r = lane & 15;
  const int64_t bt = blockIdx.x / n_chunks;  // all chunks of a row are adjacent
  const int chunk = int(blockIdx.x % n_chunks);
  const int64_t b = bt / T;
  const int lim = clamp_limit(limit, bt, K);
  const int j_begin = chunk * keys_per_wg;
  const int j_end = min(j_begin + keys_per_wg, K);
  float* orow = out + bt * K;

  for (int j = max(j_begin, lim + 1) + int(threadIdx.x); j < j_end; j += kDecWaves * 64)
    orow[j] = -INFINITY;
  const int c_end = min(j_end, lim + 1);  // keys [j_begin, c_end) are scored
  if (c_end <= j_begin) return;           // uniform over the workgroup

  const int per_wave = keys_per_wg / kDecWaves;  // a multiple of kDecGroup
  const int w_begin = j_begin + wave * per_wave;
  const int n_keys = max(0, min(w_begin + per_wave, c_end) - w_begin);  // this wave's keys
  // the wave's keys, key scales and outputs as range-checked buffers: loads
  // past the wave's last key read 0 and stores there are dropped, so the
  // prefetch ring and the ragged tail need no branch (a fixed count of
  // memory operations per iteration keeps the waits exact)
  const auto krs = make_rsrc(k + (b * int64_t(K) + w_begin) * kRowBytes, n_keys * kRowBytes);
  const auto srs = make_rsrc(FP8 ? k_scale + b * int64_t(K) + w_begin : nullptr, FP8 ? n_keys * 4 : 0);
  const auto ors = make_rsrc(orow + w_begin, n_keys * 4);

  // q chunks and head weights first, so that waiting for them does not wait
  // for the key ring issued after them
  constexpr int kQLoads = kHeads * kLanesPerRow / (kDecWaves * 64);
  const uint8_t* qsrc = q + bt * (kHeads * kRowBytes);
  u32x4 qv[kQLoads];
#pragma unroll
  for (int i = 0; i < kQLoads; ++i) {
    const int c = int(threadIdx.x) + kDecWaves * 64 * i;
    qv[i] = *reinterpret_cast<const u32x4*>(qsrc + (c / kLanesPerRow) * kRowBytes + (c % kLanesPerRow) * 16);
  }
  float wv = 0.f;
  if (threadIdx.x < kHeads) {
    const int h = threadIdx.x;
    wv = FP8 ? w[bt * kHeads + h] * q_scale[bt * kHeads + h] : w[bt * kHeads + h];
  }

  // B fragments of the subtile whose first key is jj (relative to w_begin)
  Frag buf[kDecRing][M::kSteps];
  auto gload = [&](int jj, Frag (&f)[M::kSteps]) {
    const int base = (jj + r) * kRowBytes;
#pragma unroll
    for (int s = 0; s < M::kSteps; ++s) {
      const int off = base + M::dofs(s, g) * M::kElemBytes;
      if constexpr (FP8) {
        const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0);
        const u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(krs, off + 16, 0, 0);
        f[s] = Frag{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]),
                    int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
      } else {
        f[s] = __builtin_bit_cast(Frag, __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0));
      }
    }
  };
  float sk[kDecRing / 4];  // fp8: scale of key (group start + lane)
  auto sload = [&](int jg) {
    return FP8 ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srs, (jg + lane) * 4, 0, 0))
               : 1.f;
  };
#pragma unroll
  for (int i = 0; i < kDecRing; ++i) gload(16 * i, buf[i]);
#pragma unroll
  for (int i = 0; i < kDecRing / 4; ++i) sk[i] = sload(kDecGroup * i);

#pragma unroll
  for (int i = 0; i < kQLoads; ++i) {
    const int c = int(threadIdx.x) + kDecWaves * 64 * i;
    *reinterpret_cast<u32x4*>(q_lds + (c / kLanesPerRow) * kPitch + (c % kLanesPerRow) * 16) = qv[i];
  }
  if (threadIdx.x < kHeads) w_lds[threadIdx.x] = wv;
  __syncthreads();
  // the query's A fragments and head weights, in the form every scoring
  // kernel uses (Query16), so a key's score has the same bits here as in the
  // prefill kernel
  Query16<FP8> qr;
  float wf[4][4];  // head 16*mt + 4*g + i
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int s = 0; s < M::kSteps; ++s)
      qr.a[mt][s] = M::load(q_lds + (16 * mt + r) * kPitch + M::dofs(s, g) * M::kElemBytes);
    const f32x4 w4 = *reinterpret_cast<const f32x4*>(&w_lds[16 * mt + 4 * g]);
#pragma unroll
    for (int i = 0; i < 4; ++i) wf[mt][i] = w4[i];
  }
  qr.set_weights(wf);

  for (int j0 = 0; j0 < n_keys; j0 += 16 * kDecRing) {
#pragma unroll
    for (int grp = 0; grp < kDecRing / 4; ++grp) {
      const int jg = j0 + kDecGroup * grp;
      float p[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int slot = 4 * grp + st;
        p[st] = qr.partial(buf[slot]);
        gload(jg + 16 * st + 16 * kDecRing, buf[slot]);  // the slot's next subtile
        // keep the refill here: sunk to the end of the loop, all refills
        // would be waited for together and the ring would not overlap
        __builtin_amdgcn_sched_barrier(0);
      }
      const float s_key = sk[grp];
      sk[grp] = sload(jg + 16 * kDecRing);
      const float tot = subtile_total(p, lane);
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, qr.finish(tot, s_key)), ors,
                                            (jg + lane) * 4, 0, 0);
    }
  }
}

// ---------------------------------------------------------------------------
// paged keys: the decode kernel's structure with keys read through a block
// table from a quantized cache (fp8 q; mxfp4 or fp8 keys). A workgroup owns
// one query and a chunk of positions; its block-table entries are staged in
// LDS. Pages hold at least 16 positions, so a 16-key subtile lies in one
// page: each subtile gets a range-checked buffer descriptor over its valid
// keys, so positions past the limit read 0 without a branch.
//  * mxfp4 keys (v_mfma_scale_f32_16x16x128_f8f6f4 with B in E2M1). Lane
//    layouts measured on gfx950 (K = the contraction index the block scales
//    follow): an E2M1 operand's lane group g holds K in [32g, 32g+32) in
//    nibble order and lane group g's scale byte scales K-block g; an 8-bit
//    operand's lane group g holds K in [16g, 16g+16) in bytes 0..15 and K
//    64 higher in bytes 16..31. With K = d, a key lane (r, g) takes the 16
//    bytes of nibbles of d in [32g, 32g+32) and its E8M0 byte g, exactly the
//    cache layout, and a q lane takes bytes [16g, 16g+16) and [64+16g, ...)
//    of its head row. (The dense fp8 path pairs two 8-bit operands in one
//    consistent order with unit scales, so its order does not matter.) The
//    hardware reads scale 0xFF as NaN where the cache means 0, so such a
//    group's nibbles are zeroed in registers (scale 127).
//  * fp8 keys: 32-byte fragments with unit block scales; the per-token fp32
//    scale multiplies the finished score, as in the dense fp8 path.
constexpr int kPagedTab = 72;  // staged table entries per workgroup (chunk / 16 + 1)

template <bool MXFP4, int kRing = 8>  // kRing: subtiles in flight per wave
__global__ __launch_bounds__(kPagedWaves * 64, 2) void logits_paged_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale,
    const uint8_t* __restrict__ kc, const uint8_t* __restrict__ kcs,
    const int32_t* __restrict__ block_table, const float* __restrict__ w,
    const int32_t* __restrict__ limit, float* __restrict__ out, int T, int K, int MB, int bs_log2,
    int keys_per_wg, int n_chunks) {
  using M = Mma16<true>;  // fp8 A fragments (q): one 128-deep step per M-tile
  using Frag = M::Frag;
  constexpr int kRowBytes = MXFP4 ? 64 : 128;  // cache bytes per key
  constexpr int kQRow = kHeadDim;              // fp8 q bytes per head
  constexpr int kPitch = kQRow + 16;
  constexpr int kLanesPerRow = kQRow / 16;
  static_assert(kRing % 4 == 0, "whole 64-key groups in flight");
  __shared__ __attribute__((aligned(16))) uint8_t q_lds[kHeads * kPitch];
  __shared__ __attribute__((aligned(16))) float w_lds[kHeads];
  __shared__ int32_t tab_lds[kPagedTab];

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, r = lane & 15;
  const int64_t bt = blockIdx.x / n_chunks;
  const int chunk = int(blockIdx.x % n_chunks);
  const int64_t b = bt / T;
  const int lim = clamp_limit(limit, bt, K);
  const int j_begin = chunk * keys_per_wg;
  const int j_end = min(j_begin + keys_per_wg, K);
  float* orow = out + bt * K;

  for (int j = max(j_begin, lim + 1) + int(threadIdx.x); j < j_end; j += kPagedWaves * 64)
    orow[j] = -INFINITY;
  const int c_end = min(j_end, lim + 1);
  if (c_end <= j_begin) return;  // uniform over the workgroup

  const int per_wave = keys_per_wg / kPagedWaves;
  const int w_begin = j_begin + wave * per_wave;
  const int w_end = max(w_begin, min(w_begin + per_wave, c_end));
  const int tab0 = j_begin >> bs_log2;                      // first staged page index
  const int n_tab = ((c_end - 1) >> bs_log2) - tab0 + 1;   // pages with a scored key
  const auto ors = make_rsrc(orow + w_begin, (w_end - w_begin) * 4);

  // q chunks, head weights (times the q scale) and the chunk's table entries
  constexpr int kQLoads = kHeads * kLanesPerRow / (kPagedWaves * 64);
  const uint8_t* qsrc = q + bt * (kHeads * kQRow);
  u32x4 qv[kQLoads];
#pragma unroll
  for (int i = 0; i < kQLoads; ++i) {
    const int c = int(threadIdx.x) + kPagedWaves * 64 * i;
    qv[i] = *reinterpret_cast<const u32x4*>(qsrc + (c / kLanesPerRow) * kQRow + (c % kLanesPerRow) * 16);
  }
  float wv = 0.f;
  if (threadIdx.x < kHeads) wv = w[bt * kHeads + threadIdx.x] * q_scale[bt * kHeads + threadIdx.x];
  int32_t tv = 0;
  if (int(threadIdx.x) < n_tab) tv = block_table[b * MB + tab0 + int(threadIdx.x)];
#pragma unroll
  for (int i = 0; i < kQLoads; ++i) {
    const int c = int(threadIdx.x) + kPagedWaves * 64 * i;
    *reinterpret_cast<u32x4*>(q_lds + (c / kLanesPerRow) * kPitch + (c % kLanesPerRow) * 16) = qv[i];
  }
  if (threadIdx.x < kHeads) w_lds[threadIdx.x] = wv;
  if (int(threadIdx.x) < n_tab) tab_lds[threadIdx.x] = tv;
  __syncthreads();

  Frag a[4];
  float wr[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const uint8_t* qrow = q_lds + (16 * mt + r) * kPitch;
    if constexpr (MXFP4) {  // the 8-bit operand's K order (see above)
      const i32x4 lo = *reinterpret_cast<const i32x4*>(qrow + 16 * g);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(qrow + 64 + 16 * g);
      a[mt] = Frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
      a[mt] = M::load(qrow + M::dofs(0, g));
    }
    const f32x4 w4 = *reinterpret_cast<const f32x4*>(&w_lds[16 * mt + 4 * g]);
#pragma unroll
    for (int i = 0; i < 4; ++i) wr[mt][i] = w4[i];
  }

  // one subtile: B fragment and (mxfp4) block scale of key jj + r, group g;
  // (fp8) the scale of key jj + (lane % 16), kept by the lanes whose store
  // slot it is (lane / 16 == subtile index in its group)
  struct Sub {
    Frag b;
    uint32_t sc;
  };
  Sub buf[kRing];
  float sk[kRing / 4];
  auto gload = [&](int jj, int st, Sub& dst, float& skk) {
    const int valid = max(0, min(16, w_end - jj));
    const int page = min(max((jj >> bs_log2) - tab0, 0), n_tab - 1);
    const int64_t slot = (int64_t(tab_lds[page]) << bs_log2) | (jj & ((1 << bs_log2) - 1));
    const auto rs = make_rsrc(kc + slot * kRowBytes, valid * kRowBytes);
    if constexpr (MXFP4) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, r * kRowBytes + 16 * g, 0, 0);
      dst.b = Frag{int(v[0]), int(v[1]), int(v[2]), int(v[3]), 0, 0, 0, 0};
      const auto ss = make_rsrc(kcs + slot * 4, valid * 4);
      dst.sc = __builtin_amdgcn_raw_buffer_load_b32(ss, r * 4, 0, 0);
    } else {
      const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(rs, r * kRowBytes + 32 * g, 0, 0);
      const u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(rs, r * kRowBytes + 32 * g + 16, 0, 0);
      dst.b = Frag{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
      const auto ss = make_rsrc(kcs + slot * 4, valid * 4);
      const float v = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ss, r * 4, 0, 0));
      skk = (lane >> 4) == st ? v : skk;
    }
  };
  auto partial = [&](const Sub& sub) {
    Frag bf = sub.b;
    int sb = 127;
    if constexpr (MXFP4) {
      sb = int((sub.sc >> (8 * g)) & 0xFFu);
      if (sb == 0xFF) {  // E8M0 0xFF means 0 here: zero the group
        bf = Frag{0, 0, 0, 0, 0, 0, 0, 0};
        sb = 127;
      }
    }
    f32x4 acc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      // operand formats: A fp8 e4m3 (0), B E2M1 (4) or e4m3 (0); A scale 1.0
      acc[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[mt], bf, f32x4{0.f, 0.f, 0.f, 0.f},
                                                                 0, MXFP4 ? 4 : 0, 0, 127, 0, sb);
    }
    float p0 = 0.f, p1 = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      p0 = fmaf(wr[mt][0], fmaxf(acc[mt][0], 0.f), p0);
      p1 = fmaf(wr[mt][1], fmaxf(acc[mt][1], 0.f), p1);
      p0 = fmaf(wr[mt][2], fmaxf(acc[mt][2], 0.f), p0);
      p1 = fmaf(wr[mt][3], fmaxf(acc[mt][3], 0.f), p1);
    }
    return p0 + p1;
  };

#pragma unroll
  for (int i = 0; i < kRing; ++i) gload(w_begin + 16 * i, i & 3, buf[i], sk[i >> 2]);
  for (int j0 = w_begin; j0 < w_end; j0 += 16 * kRing) {
#pragma unroll
    for (int grp = 0; grp < kRing / 4; ++grp) {
      const int jg = j0 + kDecGroup * grp;
      float p[4];
      const float s_key = sk[grp];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int slot = 4 * grp + st;
        p[st] = partial(buf[slot]);
        gload(jg + 16 * st + 16 * kRing, st, buf[slot], sk[grp]);
        __builtin_amdgcn_sched_barrier(0);
      }
      const float tot = subtile_total(p, lane);
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, MXFP4 ? tot : tot * s_key), ors,
                                            (jg - w_begin + lane) * 4, 0, 0);
    }
  }
}

// prefill grid: 1-D over (query blocks, longest causal rows first) x B x
// (key chunks). NW waves, one query each, share 64-key tiles that the
// buffer unit writes straight into LDS (buffer_load ... lds, 16 bytes per
// lane): three tile buffers rotate, so while a tile is scored the next one
// has landed and the one after it is in flight, with one barrier per tile
// and no tile data passing through registers. The LDS rows are unpadded;
// each 16-byte piece is stored at its index XOR a row-dependent mask, so a
// fragment read (16 keys x one 16-byte piece) still hits 16 distinct
// 16-byte bank groups. Within a tile the next subtile's B fragments are
// read before the current subtile's MFMAs, and a subtile's ReLU/weight
// epilogue is issued alongside the next subtile's MFMAs.
//
// With NL > 0 the kernel writes no logits: it is the first half of the
// fused logits -> top-k path, one query per wave. Each lane keeps the NL
// largest scores it has seen in a sorted register list (one med3 per entry
// and key). The wave's 64 lists hold 64*NL >= k distinct scores of the
// row, so their minimum, the bound tau, is at most the row's k-th largest
// score. Keys scoring >= tau are appended to the (row, chunk) candidate
// region as (order key, j): every key of the row's top-k scores >= the
// k-th largest >= tau, so the candidates hold the whole top-k, ties
// included. The count written at the end may exceed the region's capacity
// (entries past it are dropped); the selection kernel then has the row
// recomputed.
constexpr int kPrefillTile = 64;     // bf16 keys per LDS tile
constexpr int kPrefillBufsFp8 = 4;    // fp8 key-tile buffers in rotation
constexpr int kPrefillTileFp8 = 128;  // fp8 keys per LDS tile (16 KB, one barrier per two 64-key groups)
// keys per prefill workgroup chunk are capped so that a chunk's key bytes
// fit a buffer descriptor's 32-bit range
constexpr int kPrefillMaxChunk = 1 << 22;
constexpr int kXcds = 8;  // MI355X: workgroups are dealt round-robin to 8 XCDs

// minimum over the wave, uniform result (DPP butterflies in each row of 16
// lanes, then the four rows read as scalars)
__device__ __forceinline__ float wave_min(float v) {
#define XK_MIN_DPP(C) \
  v = fminf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), C, 0xF, 0xF, false)));
  XK_MIN_DPP(0xB1)   // quad_perm [1,0,3,2]
  XK_MIN_DPP(0x4E)   // quad_perm [2,3,0,1]
  XK_MIN_DPP(0x141)  // row_half_mirror
  XK_MIN_DPP(0x140)  // row_mirror
#undef XK_MIN_DPP
  const auto lane_v = [&](int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); };
  return fminf(fminf(lane_v(0), lane_v(16)), fminf(lane_v(32), lane_v(48)));
}

// -inf over orow[j0, j1) by one wave: 16-byte non-temporal stores over the
// 16-byte aligned body when the row starts 16-byte aligned (vec), single
// stores at the ragged ends
__device__ __forceinline__ void fill_neg_inf(float* orow, int j0, int j1, int lane, bool vec) {
  if (j0 >= j1) return;  // uniform
  if (!vec) {
    for (int j = j0 + lane; j < j1; j += 64) orow[j] = -INFINITY;
    return;
  }
  const int a0 = min(j1, (j0 + 3) & ~3), a1 = max(a0, j1 & ~3);
  if (lane < a0 - j0) orow[j0 + lane] = -INFINITY;
  if (lane < j1 - a1) orow[a1 + lane] = -INFINITY;
  const f32x4 ninf = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  for (int j = a0 + 4 * lane; j < a1; j += 256) __builtin_nontemporal_store(ninf, reinterpret_cast<f32x4*>(orow + j));
}

// waits until at most N vector-memory operations of this wave are
// outstanding, then joins the workgroup barrier; the asm's memory clobber
// keeps the compiler from moving memory accesses across it
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt field (6 bits)");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// N loads of 16 bytes per lane from `rs` (at this lane's offsets) straight
// into LDS: load i fills the 1 KB at dst + i*1024, lane l its 16 bytes at l*16.
// (The 16-byte form is a gfx950 instruction that the host pass's view of the
// device target lacks, so the host pass sees an empty body.)
template <int N>
__device__ __forceinline__ void lds_load_1k(__amdgpu_buffer_rsrc_t rs, uint8_t* dst, const int (&voff)[N]) {
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
  for (int i = 0; i < N; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + i * 1024), 16,
                                             voff[i], 0, 0, 0);
#endif
}

template <bool FP8, int NW, int NL>
// The second bound is the minimum number of waves per SIMD: fp8 workgroups
// of 8 waves need 4 (128 VGPRs) for two workgroups per CU; bf16 workgroups
// of 4 waves run three per CU. The candidate form (NL > 0) runs one
// workgroup per query block with whole rows, one per CU at the fused
// shapes, so it takes 2: its lists then fit without spilling (fp8 NL = 16:
// 56 bytes of scratch at 128 VGPRs; measured 1554 -> 1444 us for the fused
// call on the long fp8 prefill).
__global__ __launch_bounds__(NW * 64, NL > 0 ? 2 : (FP8 ? 4 : 3)) void logits_prefill_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale,
    const uint8_t* __restrict__ k, const float* __restrict__ k_scale,
    const float* __restrict__ w, const int32_t* __restrict__ limit,
    float* __restrict__ out, CandidateOut co, int B, int T, int K, int n_chunks, int n_qblocks) {
  using M = Mma16<FP8>;
  using Frag = typename M::Frag;
  constexpr bool kCand = NL > 0;
  constexpr int QB = NW;  // queries per workgroup, one per wave
  constexpr int kRowBytes = kHeadDim * M::kElemBytes;        // 256 (bf16) or 128 (fp8)
  constexpr int kTile = FP8 ? kPrefillTileFp8 : kPrefillTile;  // keys per LDS tile
  constexpr int kGroups = kTile / 64;                          // 64-key score groups per tile
  constexpr int kTileBytes = kTile * kRowBytes;
  constexpr int kDma = kTileBytes / (NW * 64 * 16);           // 16-byte LDS loads per lane per tile
  static_assert(kDma >= 1 && kTileBytes % (NW * 64 * 16) == 0, "tile split");
  // Tile buffers in rotation: while tile t is scored, tiles t+1 .. t+kBufs-1
  // are landing. fp8 (two workgroups per CU, 16 KB tiles) takes four, bf16
  // (three workgroups per CU) three.
  constexpr int kBufs = FP8 ? kPrefillBufsFp8 : 3;
  static_assert(kBufs >= 2 && kBufs <= 4, "two to four tile buffers");
  // vector-memory operations a wave may still have outstanding at the end
  // of step t once tile t+1 has landed: those issued after tile t+1's
  // loads, i.e. the score stores of the step that issued them and, in each
  // later step, the key scales (fp8), the next tile's loads and the stores
  constexpr int kAfter = kGroups + (kBufs - 2) * (kDma + kGroups + (FP8 ? kGroups : 0));
  constexpr int kTauEvery = 512 / kTile;  // candidates: tiles between bound updates
  // tile buffers as separate arrays, so the compiler can tell the buffer
  // being read from the ones being written
  __shared__ __attribute__((aligned(16))) uint8_t tile0[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t tile1[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t tile2[kBufs >= 3 ? kTileBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t tile3[kBufs == 4 ? kTileBytes : 16];

  // the wave index in a scalar register: per-wave values derived from it
  // (rows, buffer descriptors) then stay scalar
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, r = lane & 15;
  // Workgroup i runs on XCD i % 8. Eight consecutive workgroups take the
  // same key chunk of eight consecutive (sequence, query block) units, so
  // every XCD gets an equal share of each chunk; units run longest causal
  // rows first.
  const int x8 = int(blockIdx.x % kXcds), grp = int(blockIdx.x / kXcds);
  const int chunk = grp % n_chunks;
  const int unit = (grp / n_chunks) * kXcds + x8;
  if (unit >= n_qblocks * B) return;  // uniform: the grid is rounded up to whole groups
  const int64_t b = unit % B;
  const int qb = n_qblocks - 1 - unit / B;
  int blk_lim = -1;
#pragma unroll
  for (int i = 0; i < QB; ++i) {
    const int ti = qb * QB + i;
    if (ti < T) blk_lim = max(blk_lim, clamp_limit(limit, b * T + ti, K));
  }
  // The block's own scored range [0, row_end) is split into n_chunks parts
  // of equal tile counts: under a causal limit the parts shrink with the
  // row, so no workgroup is left with an empty fixed key range and long and
  // short rows are cut alike. The last part also covers the keys past the
  // block's limit (their -inf fill).
  const int row_end = min(K, blk_lim + 1);
  const int nt_all = (max(row_end, 0) + kTile - 1) / kTile;
  const int t_lo = int(int64_t(nt_all) * chunk / n_chunks), t_hi = int(int64_t(nt_all) * (chunk + 1) / n_chunks);
  const int j_begin = t_lo * kTile;
  const int j_end = chunk == n_chunks - 1 ? K : min(K, t_hi * kTile);
  const int c_end = min(j_end, blk_lim + 1);

  const int t_q = qb * QB + wave;
  const bool qvalid = t_q < T;
  const int64_t bt = b * T + (qvalid ? t_q : 0);
  const int lim = qvalid ? clamp_limit(limit, bt, K) : -1;
  const int q_end = min(j_end, lim + 1);
  // this query's keys of the chunk past its limit are -inf; a workgroup with
  // keys to score issues these stores once tile 0 has landed, so no early
  // wait (vector-memory counts complete in issue order) waits for them
  const bool vec = (K & 3) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0;
  auto fill = [&]() {
    if (!kCand && qvalid) fill_neg_inf(out + bt * K, max(j_begin, lim + 1), j_end, lane, vec);
  };
  if (kCand && blockIdx.x == 0 && threadIdx.x < 2) co.ctrl[threadIdx.x] = 0;  // queue counters
  if (c_end <= j_begin) {  // uniform over the workgroup
    fill();
    if (kCand && qvalid && lane == 0) co.count[bt * n_chunks + chunk] = 0;
    return;
  }

  // the chunk's scored keys: loads at or past c_end read 0 without a memory
  // access (those keys' scores are never stored)
  const int n_tiles = (c_end - j_begin + kTile - 1) / kTile;
  const int valid_bytes = (c_end - j_begin) * kRowBytes;
  const uint8_t* kchunk = k + (b * int64_t(K) + j_begin) * kRowBytes;
  const auto srs = make_rsrc(FP8 ? k_scale + b * int64_t(K) + j_begin : nullptr, FP8 ? (c_end - j_begin) * 4 : 0);
  // piece p of LDS row `row` holds the row's 16-byte piece p ^ swz(row),
  // so a fragment read (one piece of 16 or 32 consecutive rows per lane
  // group) spreads over the banks. Measured with SQ_LDS_BANK_CONFLICT on
  // gfx950: bf16 16x16 reads with row % 16 and fp8 32x32 reads with
  // (row / 2) % 8 take no conflict cycles ((row / 4) % 8 takes one per read,
  // no swizzle about six).
  auto swz = [](int row) { return FP8 ? (row >> 1) & 7 : row & 15; };
  constexpr int kPieces = kRowBytes / 16;
  // this lane's source offset (within a tile) for each of its LDS loads;
  // load i of wave w fills LDS bytes [(w*kDma + i)*1024, +1024), lane l
  // the 16 bytes at l*16 of that range
  int voff[kDma];
#pragma unroll
  for (int i = 0; i < kDma; ++i) {
    const int o = (wave * kDma + i) * 1024 + lane * 16;
    const int row = o / kRowBytes, p = (o % kRowBytes) / 16;
    voff[i] = row * kRowBytes + (p ^ swz(row)) * 16;
  }
  auto dma = [&](uint8_t* dst, int tix) {
    const int off = tix * kTileBytes;  // scalar
    lds_load_1k<kDma>(make_rsrc(kchunk + off, max(0, valid_bytes - off)), dst + wave * kDma * 1024, voff);
  };
  // LDS offsets of this lane's fragment pieces.
  //  bf16 (16x16 tiles): key r of a 16-key subtile, pieces named by Mma16::dofs.
  //  fp8 (32x32 tiles): key l % 32 of a 32-key block, bytes [64s + 32g, +32)
  //  of step s (g = l / 32): pieces 4s + 2g and 4s + 2g + 1.
  constexpr int kRd = FP8 ? 4 : M::kSteps;
  int rd[kRd];
#pragma unroll
  for (int i = 0; i < kRd; ++i) {
    const int row = FP8 ? (lane & 31) : r;
    const int piece = FP8 ? 4 * (i >> 1) + 2 * (lane >> 5) + (i & 1) : (M::dofs(i, g) * M::kElemBytes) / 16;
    rd[i] = row * kRowBytes + ((piece ^ swz(row)) % kPieces) * 16;
  }
  auto frag_load = [&](const uint8_t* buf, int st, Frag (&f)[M::kSteps]) {  // bf16 subtile st
    const uint8_t* base = buf + st * 16 * kRowBytes;
#pragma unroll
    for (int s = 0; s < M::kSteps; ++s) f[s] = M::load(base + rd[s]);
  };
  auto frag32 = [&](const uint8_t* buf, int blk, i32x8 (&f)[2]) {  // fp8 32-key block blk
    const uint8_t* base = buf + blk * 32 * kRowBytes;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const i32x4 lo = *reinterpret_cast<const i32x4*>(base + rd[2 * s]);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(base + rd[2 * s + 1]);
      f[s] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  };

  // logits: this query's outputs of the chunk, up to its limit;
  // candidates: the (row, chunk) region
  const auto ors = kCand ? make_rsrc(co.cand + (bt * n_chunks + chunk) * int64_t(co.capc), co.capc * 8)
                         : make_rsrc(out + bt * K + j_begin, max(0, q_end - j_begin) * 4);
  float best[kCand ? NL : 1];  // descending; -inf until the lane has seen NL keys
#pragma unroll
  for (int i = 0; i < (kCand ? NL : 1); ++i) best[i] = -INFINITY;
  float tau = -INFINITY;  // the row bound (uniform)
  int cnt = 0;            // candidates this wave has emitted (uniform)

  // q fragments and head weights are loaded before the key tiles: memory
  // waits count in issue order, so waiting for them (at their first use)
  // must not also wait for tiles in flight
  std::conditional_t<FP8, Query32, Query16<false>> qr;
  if (qvalid)
    qr.load(q + bt * (kHeads * kRowBytes), w + bt * kHeads, FP8 ? q_scale + bt * kHeads : nullptr, lane);
  else
    qr.zero();
  dma(tile0, 0);
  if constexpr (kBufs >= 3) dma(tile1, 1);
  if constexpr (kBufs == 4) dma(tile2, 2);
  // tile 0 has landed (this wave's part), then all waves' parts
  wait_vm_barrier<(kBufs - 2) * kDma>();
  fill();

  // score tile tix (in `cur`) after starting tile tix + kBufs - 1 (into
  // `nxt`, the buffer every wave finished reading before the last barrier)
  auto step = [&](const uint8_t* cur, uint8_t* nxt, int tix) {
    if (kCand && (tix % kTauEvery) == kTauEvery - 2) tau = fmaxf(tau, wave_min(best[kCand ? NL - 1 : 0]));
    float sk[kGroups];  // fp8: scale of key (group start + lane)
#pragma unroll
    for (int h = 0; h < kGroups; ++h)
      sk[h] = FP8 ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                  srs, (tix * kTile + 64 * h + lane) * 4, 0, 0))
                  : 1.f;
    // the scale loads stay ahead of the tile loads: waiting for them then
    // leaves the tile loads in flight
    __builtin_amdgcn_sched_barrier(0);
    dma(nxt, tix + kBufs - 1);
#pragma unroll
    for (int h = 0; h < kGroups; ++h) {
      const uint8_t* grp = cur + h * 64 * kRowBytes;
      float tot;
      if constexpr (FP8) {
        i32x8 bf[2][2];  // [block][step]
        frag32(grp, 0, bf[0]);
        frag32(grp, 1, bf[1]);
        const float p0 = qr.partial(bf[0]);
        const float p1 = qr.partial(bf[1]);
        tot = tile_total32(p0, p1);
      } else {
        Frag bf[2][M::kSteps];
        f32x4 acc[2][4];
        float p[4];
        frag_load(grp, 0, bf[0]);
        qr.mma(bf[0], acc[0]);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          if (st < 3) {
            frag_load(grp, st + 1, bf[(st + 1) & 1]);
            qr.mma(bf[(st + 1) & 1], acc[(st + 1) & 1]);
          }
          p[st] = qr.epilogue(acc[st & 1]);
        }
        tot = subtile_total(p, lane);
      }
      const float sc = qr.finish(tot, sk[h]);
      const int jo = tix * kTile + 64 * h + lane;  // this lane's key, relative to j_begin
      if constexpr (kCand) {
        const int j = j_begin + jo;
        const bool valid = j < q_end;
        const float sv = valid ? sc : -INFINITY;
#pragma unroll
        for (int i = NL - 1; i > 0; --i) best[i] = __builtin_amdgcn_fmed3f(best[i], best[i - 1], sv);
        best[0] = fmaxf(best[0], sv);
        const bool pass = valid && sc >= tau;
        const uint64_t m = __ballot(pass);
        const int rank = __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u));
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{order_key(sc), uint32_t(j)}, ors,
                                              pass ? (cnt + rank) * 8 : co.capc * 8, 0, 0);
        cnt += __popcll(m);
      } else {
        // Non-temporal (cache policy 2): the score matrix is written once and read once by
        // the selection; keeping it out of L2/MALL leaves those to the key tiles and lets the
        // following top-k's reads stream (measured 55 us less per step at 8 Ki x 96 Ki).
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sc), ors, jo * 4, 0, 2);
      }
    }
    // tile tix + 1 has landed: this wave's part, then all waves'
    wait_vm_barrier<kAfter>();
  };
  // Candidates: every eighth tile the wave raises tau to its lists' minimum.
  for (int tix = 0;;) {
    if constexpr (kBufs == 2) {
      step(tile0, tile1, tix);
      if (++tix >= n_tiles) break;
      step(tile1, tile0, tix);
      if (++tix >= n_tiles) break;
    } else {
      step(tile0, kBufs == 4 ? tile3 : tile2, tix);
      if (++tix >= n_tiles) break;
      step(tile1, tile0, tix);
      if (++tix >= n_tiles) break;
      step(tile2, tile1, tix);
      if (++tix >= n_tiles) break;
      if constexpr (kBufs == 4) {
        step(tile3, tile2, tix);
        if (++tix >= n_tiles) break;
      }
    }
  }
  // no LDS load may still be in flight when the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(0);
  if (kCand && qvalid && lane == 0) co.count[bt * n_chunks + chunk] = cnt;
}

int round_up(int x, int m) { return (x + m - 1) / m * m; }
int64_t round_up64(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

}  // namespace

hipError_t launch_logits_paged(const void* q, const float* q_scale, const float* w,
                               const int32_t* limit, const void* k_cache, const void* k_scale,
                               const int32_t* block_table, float* logits, int B, int T, int K,
                               int MB, int bs, bool mxfp4, hipStream_t stream) {
  // 512 to 1024 positions per workgroup (a quarter of the bytes of a bf16
  // key per position, so longer chunks than the dense decode kernel's;
  // measured on the Flash and Pro decode shapes)
  const int64_t rows = int64_t(B) * T;
  const int64_t per = (int64_t(K) * rows + 2047) / 2048;
  int kpw = int(std::min<int64_t>(std::max<int64_t>(per, 2 * kPagedWaves * kDecGroup), 4 * kPagedWaves * kDecGroup));
  kpw = std::min(round_up(kpw, kPagedWaves * kDecGroup), round_up(K, kPagedWaves * kDecGroup));
  const int nch = (K + kpw - 1) / kpw;
  int bs_log2 = 0;
  while ((1 << bs_log2) < bs) ++bs_log2;
  const dim3 grid(unsigned(rows * nch));
  const auto* q8 = static_cast<const uint8_t*>(q);
  const auto* kc = static_cast<const uint8_t*>(k_cache);
  const auto* ks = static_cast<const uint8_t*>(k_scale);
  if (mxfp4)
    hipLaunchKernelGGL(logits_paged_kernel<true>, grid, dim3(kPagedWaves * 64), 0, stream, q8, q_scale, kc, ks,
                       block_table, w, limit, logits, T, K, MB, bs_log2, kpw, nch);
  else
    hipLaunchKernelGGL(logits_paged_kernel<false>, grid, dim3(kPagedWaves * 64), 0, stream, q8, q_scale, kc, ks,
                       block_table, w, limit, logits, T, K, MB, bs_log2, kpw, nch);
  return hipGetLastError();
}

hipError_t launch_logits(const void* q, const float* q_scale, const void* k,
                         const float* k_scale, const float* w, const int32_t* limit,
                         float* logits, int B, int T, int K, bool fp8, hipStream_t stream) {
  const auto* q8 = static_cast<const uint8_t*>(q);
  const auto* k8 = static_cast<const uint8_t*>(k);
  if (T < 8) {
    // one query per workgroup; chunks of 256 or 384 keys (a multiple of two
    // waves x 64). Short chunks keep a workgroup's life short next to the
    // kernel's, so ragged rows balance across CUs (measured on the Flash
    // and Pro decode shapes: two waves x 128 keys beat four x 128 by 2-3%,
    // and beat 8 x 64, 8 x 128, 2 x 64 and 1 x 128)
    const int64_t rows = int64_t(B) * T;
    const int64_t per = (int64_t(K) * rows + 2047) / 2048;
    int kpw = int(std::min<int64_t>(std::max<int64_t>(per, 2 * kDecWaves * kDecGroup), 3 * kDecWaves * kDecGroup));
    kpw = std::min(round_up(kpw, kDecWaves * kDecGroup), round_up(K, kDecWaves * kDecGroup));
    const int nch = (K + kpw - 1) / kpw;
    const dim3 grid(unsigned(rows * nch));
    if (fp8)
      hipLaunchKernelGGL(logits_decode_kernel<true>, grid, dim3(kDecWaves * 64), 0, stream, q8, q_scale, k8,
                         k_scale, w, limit, logits, T, K, kpw, nch);
    else
      hipLaunchKernelGGL(logits_decode_kernel<false>, grid, dim3(kDecWaves * 64), 0, stream, q8, q_scale, k8,
                         k_scale, w, limit, logits, T, K, kpw, nch);
  } else {
    // One query per wave (64 VGPRs of A fragments): 4 waves for bf16 (three
    // workgroups per CU), 8 for fp8 (half the A bytes, so a workgroup's LDS
    // tile is shared by more queries). Shapes measured on the flash-prefill
    // and long-context configs.
    const int QB = fp8 ? 8 : 4;
    const int nqb = (T + QB - 1) / QB;
    const int64_t qblocks = int64_t(nqb) * B;
    // every block's row in at least two parts (under a causal limit rows
    // of 1 to K/64 tiles then give workgroups of half those sizes, which
    // balance better; both parts of a block run on one XCD, so its second q
    // read hits that XCD's L2); more parts only when there are fewer than
    // ~1024 query blocks, since each part re-reads q
    const int nch = int(std::max<int64_t>({2, (1024 + qblocks - 1) / qblocks,
                                           (int64_t(K) + kPrefillMaxChunk - 1) / kPrefillMaxChunk}));
    const dim3 grid(unsigned(int64_t(nch) * round_up64(qblocks, kXcds)));
    if (fp8)
      hipLaunchKernelGGL((logits_prefill_kernel<true, 8, 0>), grid, dim3(8 * 64), 0, stream, q8,
                         q_scale, k8, k_scale, w, limit, logits, CandidateOut{}, B, T, K, nch, nqb);
    else
      hipLaunchKernelGGL((logits_prefill_kernel<false, 4, 0>), grid, dim3(4 * 64), 0, stream, q8,
                         q_scale, k8, k_scale, w, limit, logits, CandidateOut{}, B, T, K, nch, nqb);
  }
  return hipGetLastError();
}

hipError_t launch_logits_candidates(const void* q, const float* q_scale, const void* k,
                                    const float* k_scale, const float* w, const int32_t* limit,
                                    const FusedPlan& p, const CandidateOut& co, int B, int T, int K,
                                    bool fp8, hipStream_t stream) {
  const auto* q8 = static_cast<const uint8_t*>(q);
  const auto* k8 = static_cast<const uint8_t*>(k);
  const dim3 grid(unsigned(int64_t(p.nch) * round_up64(int64_t(p.nqb) * B, kXcds)));
  auto go = [&](auto fp8_tag, auto nl_tag) {
    constexpr bool F = decltype(fp8_tag)::value;
    constexpr int NL = decltype(nl_tag)::value;
    constexpr int NW = F ? 8 : 4;
    hipLaunchKernelGGL((logits_prefill_kernel<F, NW, NL>), grid, dim3(NW * 64), 0, stream, q8, q_scale,
                       k8, k_scale, w, limit, nullptr, co, B, T, K, p.nch, p.nqb);
  };
  using T4 = std::integral_constant<int, 4>;
  using T8 = std::integral_constant<int, 8>;
  using T16 = std::integral_constant<int, 16>;
  using T32 = std::integral_constant<int, 32>;
  auto by_nl = [&](auto fp8_tag) {
    switch (p.nl) {
      case 4: go(fp8_tag, T4{}); break;
      case 8: go(fp8_tag, T8{}); break;
      case 16: go(fp8_tag, T16{}); break;
      default: go(fp8_tag, T32{}); break;
    }
  };
  if (fp8)
    by_nl(std::true_type{});
  else
    by_nl(std::false_type{});
  return hipGetLastError();
}

}  // namespace xk
