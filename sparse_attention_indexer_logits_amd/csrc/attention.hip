// Sparse attention over the indexer's selection, reading the paged mxfp4
// cache directly (gfx950): the consumer of the top-k indices.
//
// Semantics (page "DeepSeek-V4 on ATOM" tracker, "CSA": index gather, online
// softmax, attention-sink bias; the rows are the cache rows the mxfp4 paged
// gather of page "xkernels #28 -- DeepSeek-V4 serving support" decodes): for
// row r with selected positions sel_pos[r, :] and head h,
//   s_j = scale * (q[r,h,:] . v_j)   over slots j with sel_pos >= 0
//   out[r,h,:] = sum_j exp(s_j) v_j / (sum_j exp(s_j) + exp(sink[h]))
// where v_j, the decoded cache row, is both key and value (MQA over the
// latent row). A row with no valid slot gives 0.
//
// One workgroup per (row, 64 heads), one wave per 16 heads. The row's slots
// are resolved to cache tokens once (sel_pos -> block table) into LDS.
// Then per chunk of 64 slots:
//  * 256 threads decode the chunk's mxfp4 rows (exact, as the gather does)
//    into one tile [slot][d] in LDS, read as K and, through gfx950's
//    transposing LDS load, as V^T; the next chunk's nibbles are loaded into
//    registers meanwhile;
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (keys as rows, this wave's 16
//    heads as columns): lane l holds head l%16's scores of keys 4(l/16)+i of
//    each 16-key subtile;
//  * online softmax in base 2 per head (max and sum across the four lane
//    groups of a head by two shuffles), accumulators rescaled;
//  * O^T += V^T P^T on the same MFMA: P^T is the B operand straight from the
//    S^T registers (rounded to bf16). The contraction over keys only needs A
//    and B to agree on the key order, so K-slot 8g+e of a 32-key step is key
//    4g+e of its first subtile (e < 4) or of its second (e >= 4), and the V^T
//    fragment holds the same keys: two ds_read_b64_tr_b16 from the [slot][d]
//    tile. Measured lane mapping of that load: in each 16-lane group, lane
//    i = 4a + b receives element b of the 8-byte reads of lanes a, a + 4,
//    a + 8 and a + 12; so when lane j reads row base + (j & 15) / 4 at
//    columns 16 mt + 4 (j & 3), lane i gets d = 16 mt + i of rows base ..
//    base + 3.
// At the end the sink joins the denominator and lane l stores 4 consecutive
// outputs of head l%16 per 16-dim tile (attention_rows_kernel). Decode
// batches, with fewer (row, 64-head) workgroups than CUs, run
// sparse_attention_split_kernel: 16 heads per workgroup and the chunk's keys
// split over its four waves, merged at the end.
#include "mxfp4.h"

namespace xk {
namespace {

constexpr int kAttnHeads = 64;              // heads per workgroup
constexpr int kKPitch = kHeadDim + 16;      // bf16 per tile row: 72 dwords

// Element offset of (row, col) in a [slot][d] tile, col a multiple of 4. The
// 16-byte piece col/8 is stored at piece ^ (row bit 3). With the 72-dword
// pitch (8 banks per row) the three access patterns then take no bank
// conflicts: 16-byte reads and writes of 16 consecutive rows (rows r and
// r + 8 land 4 banks apart) and the transposing 8-byte reads of 4
// consecutive rows times 4 column pairs per 16-lane group (8 banks per row,
// one swizzle bit per group). A 68-dword pitch suits the first pattern only:
// measured, its bank-conflict cycles exceeded its LDS cycles.
__device__ __forceinline__ int tile_at(int row, int col) {
  return row * kKPitch + (((col >> 3) ^ ((row >> 3) & 1)) << 3) + (col & 7);
}
constexpr int kMaxAttnSlots = 2048;         // tokens resolved in LDS
constexpr int kRowsHeadTiles = 1;           // 16-head tiles per wave in attention_rows_kernel
constexpr int kRowsChunk = 64;              // slots per chunk in attention_rows_kernel
constexpr int kSplitWaves = 8;              // waves (16-slot key subtiles per chunk) in sparse_attention_split_kernel

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;

// V^T fragment half: d = 16 mt + (lane & 15) of tile rows base .. base + 3
// (the transposing load's mapping above). `kt` points into LDS.
__device__ __forceinline__ uint2 vt_frag4(const uint16_t* kt, int base, int mt, int lane) {
  const uint16_t* p = kt + tile_at(base + ((lane & 15) >> 2), 16 * mt + 4 * (lane & 3));
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(uint2, v);
}

__device__ __forceinline__ float shfl_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}
__device__ __forceinline__ float shfl_sum(float v) {
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

// Decode batches (fewer (row, 64-head) workgroups than CUs): the workgroup
// takes 16 heads and its NW waves split every chunk of 16*NW slots (wave w
// keys 16w..16w+15), each wave running its own online softmax over its keys
// of every chunk; the NW partial states are merged at the end in a fixed
// order, so the result does not depend on timing. More waves mean fewer
// chunks per row, i.e. fewer dependent decode -> score -> accumulate rounds
// for the few workgroups of a decode batch. The chunk tile and the merge
// buffers share the LDS.
template <int NW>
__global__ __launch_bounds__(64 * NW) void sparse_attention_split_kernel(
    const uint16_t* __restrict__ q, const uint32_t* __restrict__ kv_fp4, const uint8_t* __restrict__ kv_scale,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ sel_pos,
    const int32_t* __restrict__ row_seq, const float* __restrict__ sink, float scale_log2,
    float* __restrict__ out, int H, int k, int MB, int bs_log2) {
  using Frag = bf16x8;
  constexpr int NT = 64 * NW;   // threads
  constexpr int C = 16 * NW;    // slots per chunk
  constexpr int kHeadsPerWg = 16;
  constexpr int DPT = kHeadDim * kHeadsPerWg / NT;  // merged outputs per thread
  static_assert(DPT >= 2 && DPT % 2 == 0, "merge split");
  struct Loop {
    uint16_t kt[C * kKPitch];
    float sbias[C];
  };
  struct Merge {
    float cm[NW][kHeadsPerWg], cl[NW][kHeadsPerWg];
    float co[NW][kHeadsPerWg][kHeadDim];
  };
  __shared__ __attribute__((aligned(16))) uint8_t lds[sizeof(Loop) > sizeof(Merge) ? sizeof(Loop) : sizeof(Merge)];
  __shared__ int tok[kMaxAttnSlots];
  auto& L = *reinterpret_cast<Loop*>(lds);
  uint16_t* kt = L.kt;
  float* sbias = L.sbias;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int groups = H / kHeadsPerWg;
  const int64_t r = blockIdx.x / groups;
  const int head = (blockIdx.x % groups) * kHeadsPerWg + c;  // this lane's head column

  // 1. the row's slots -> cache tokens (-1: padded slot)
  const int seq = row_seq ? row_seq[r] : int(r);
  for (int j = tid; j < k; j += NT) {
    const int p = sel_pos[r * k + j];
    int t = -1;
    if (p >= 0) {
      const int blk = block_table[int64_t(seq) * MB + (p >> bs_log2)];
      t = (blk << bs_log2) + (p & ((1 << bs_log2) - 1));
    }
    tok[j] = t;
  }
  // this wave's 16 heads as B fragments (column = head, K = d in [32s+8g, +8))
  Frag qb[4];
  const uint16_t* qrow = q + (r * H + head) * int64_t(kHeadDim);
#pragma unroll
  for (int s = 0; s < 4; ++s) qb[s] = *reinterpret_cast<const Frag*>(qrow + 32 * s + 8 * g);
  __syncthreads();

  // chunk loads: thread -> slot tid%C of the chunk, dims [32*(tid/C), +32)
  const int lslot = tid % C, quarter = tid / C;
  auto fetch = [&](int c0, u32x4& nib, uint32_t& sc, int& t) {
    const int j = c0 + lslot;
    t = j < k ? tok[j] : -1;
    nib = u32x4{0u, 0u, 0u, 0u};
    sc = 0u;
    if (t >= 0) {
      nib = reinterpret_cast<const u32x4*>(kv_fp4)[int64_t(t) * 4 + quarter];
      sc = kv_scale[int64_t(t) * 4 + quarter];
    }
  };
  u32x4 nib;
  uint32_t sc;
  int t;
  fetch(0, nib, sc, t);

  f32x4 o[8];  // O^T tile mt: dims 16mt + 4g + i of head c
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;  // running max (base-2 scaled) and sum of head c

  for (int c0 = 0; c0 < k; c0 += C) {
    // 2. decode the chunk into the tile
    {
      u32x4 d[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) d[w] = t >= 0 ? decode8(nib[w], sc) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int w = 0; w < 4; ++w) *reinterpret_cast<u32x4*>(kt + tile_at(lslot, 32 * quarter + 8 * w)) = d[w];
      if (quarter == 0) sbias[lslot] = t >= 0 ? 0.f : -INFINITY;
    }
    __syncthreads();
    if (c0 + C < k) fetch(c0 + C, nib, sc, t);  // in flight during the MFMAs

    // 3. S^T = K Q^T for this wave's 16 keys
    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
    {
#pragma unroll
      for (int s = 0; s < 4; ++s)
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            *reinterpret_cast<const Frag*>(kt + tile_at(16 * wave + c, 8 * g + 32 * s)), qb[s], sacc, 0, 0, 0);
    }
    // 4. online softmax (base 2), head c
    float x[4], cmax = -INFINITY;
    {
      const f32x4 b4 = *reinterpret_cast<const f32x4*>(&sbias[16 * wave + 4 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = fmaf(sacc[i], scale_log2, b4[i]);
        cmax = fmaxf(cmax, x[i]);
      }
    }
    cmax = shfl_max(cmax);
    const float m_new = fmaxf(m, cmax);
    const bool any = m_new > -INFINITY;
    const float alpha = any ? __builtin_amdgcn_exp2f(m - m_new) : 1.f;
    float psum = 0.f;
    s16x4 pq;  // this lane's probabilities (bf16 bits) of keys 4g..4g+3 of the wave's subtile
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = any ? __builtin_amdgcn_exp2f(x[i] - m_new) : 0.f;
      psum += p;
      pq[i] = __builtin_bit_cast(short, __bf16(p));
    }
    l = fmaf(l, alpha, shfl_sum(psum));
    m = m_new;
    // 5. O^T = O^T * alpha + V^T P^T: one 16-key step on
    // v_mfma_f32_16x16x16_bf16; a lane group's K slots are keys 4g..4g+3 of
    // the wave's subtile on both operands
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) o[mt] *= alpha;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const uint2 v = vt_frag4(kt, 16 * wave + 4 * g, mt, lane);
      o[mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, v), pq, o[mt], 0, 0, 0);
    }
    __syncthreads();  // the tiles are rewritten by the next chunk (and by the merge)
  }

  {
    // 6. merge the NW waves' states of the 16 heads, then the sink
    auto& M = *reinterpret_cast<Merge*>(lds);
    if (g == 0) {
      M.cm[wave][c] = m;
      M.cl[wave][c] = l;
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) *reinterpret_cast<f32x4*>(&M.co[wave][c][16 * mt + 4 * g]) = o[mt];
    __syncthreads();
    constexpr int TPH = NT / kHeadsPerWg;   // threads per head
    const int hc = tid / TPH, d0 = DPT * (tid % TPH);
    float mw[NW], mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      mw[w] = M.cm[w][hc];
      mm = fmaxf(mm, mw[w]);
    }
    float lsum = 0.f, acc[DPT];
#pragma unroll
    for (int e = 0; e < DPT; ++e) acc[e] = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float a = mw[w] > -INFINITY ? __builtin_amdgcn_exp2f(mw[w] - mm) : 0.f;
      lsum = fmaf(M.cl[w][hc], a, lsum);
#pragma unroll
      for (int e = 0; e < DPT; ++e) acc[e] = fmaf(M.co[w][hc][d0 + e], a, acc[e]);
    }
    const int hd = (blockIdx.x % groups) * kHeadsPerWg + hc;
    const float s2 = sink ? sink[hd] * 1.4426950408889634f : -INFINITY;
    const float mf = fmaxf(mm, s2);
    float f = 0.f;
    if (mf > -INFINITY) {
      const float a = __builtin_amdgcn_exp2f(mm - mf);
      f = a / (lsum * a + __builtin_amdgcn_exp2f(s2 - mf));
    }
    float* orow = out + (r * H + hd) * int64_t(kHeadDim) + d0;
#pragma unroll
    for (int e = 0; e < DPT; e += 2) *reinterpret_cast<f32x2*>(orow + e) = f32x2{acc[e], acc[e + 1]} * f;
  }
}

// Rows with many (row, 64-head) workgroups: HT 16-head tiles per wave,
// 4 / HT waves per workgroup. Each K-tile or V^T fragment read from LDS
// feeds HT MFMAs, so two tiles per wave halve the LDS reads per row; the
// price is registers (233 VGPRs, two waves per SIMD), and measured on the
// long prefill rows that is slower (139 against 110 us), so one tile per
// wave (113 VGPRs, four waves per SIMD) is the launched form.
template <int HT, int C>
__global__ __launch_bounds__(64 * (4 / HT), HT == 2 && C == 64 ? 2 : (HT == 2 ? 3 : 4)) void attention_rows_kernel(
    const uint16_t* __restrict__ q, const uint32_t* __restrict__ kv_fp4, const uint8_t* __restrict__ kv_scale,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ sel_pos,
    const int32_t* __restrict__ row_seq, const float* __restrict__ sink, float scale_log2,
    float* __restrict__ out, int H, int k, int MB, int bs_log2) {
  using Frag = bf16x8;
  constexpr int NW = 4 / HT;           // waves per workgroup (64 heads)
  constexpr int NT = 64 * NW;          // threads
  constexpr int NST = C / 16;          // 16-slot subtiles per chunk
  constexpr int SPP = NT / C;          // threads per slot in the decode
  constexpr int NQ = 4 / SPP;          // 32-dim groups each thread decodes per slot
  static_assert(NQ >= 1 && NQ * SPP == 4, "decode split");
  __shared__ __attribute__((aligned(16))) uint16_t kt[C * kKPitch];
  __shared__ __attribute__((aligned(16))) float sbias[C];
  __shared__ int tok[kMaxAttnSlots];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int groups = H / kAttnHeads;
  const int64_t r = blockIdx.x / groups;
  const int hbase = (blockIdx.x % groups) * kAttnHeads + 16 * HT * wave;  // head column c of tile ht: hbase + 16 ht + c

  // 1. the row's slots -> cache tokens (-1: padded slot)
  const int seq = row_seq ? row_seq[r] : int(r);
  for (int j = tid; j < k; j += NT) {
    const int p = sel_pos[r * k + j];
    int t = -1;
    if (p >= 0) {
      const int blk = block_table[int64_t(seq) * MB + (p >> bs_log2)];
      t = (blk << bs_log2) + (p & ((1 << bs_log2) - 1));
    }
    tok[j] = t;
  }
  // the wave's heads as B fragments (column = head, K = d in [32s+8g, +8))
  Frag qb[HT][4];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const uint16_t* qrow = q + (r * H + hbase + 16 * ht + c) * int64_t(kHeadDim);
#pragma unroll
    for (int s = 0; s < 4; ++s) qb[ht][s] = *reinterpret_cast<const Frag*>(qrow + 32 * s + 8 * g);
  }
  __syncthreads();

  // chunk loads: thread -> slot tid%C of the chunk, dims [32*NQ*part, +32*NQ)
  const int lslot = tid % C, part = tid / C;
  u32x4 nib[NQ];
  uint32_t sc[NQ];
  int t;
  auto fetch = [&](int c0) {
    const int j = c0 + lslot;
    t = j < k ? tok[j] : -1;
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq) {
      nib[qq] = u32x4{0u, 0u, 0u, 0u};
      sc[qq] = 0u;
      if (t >= 0) {
        nib[qq] = reinterpret_cast<const u32x4*>(kv_fp4)[int64_t(t) * 4 + NQ * part + qq];
        sc[qq] = kv_scale[int64_t(t) * 4 + NQ * part + qq];
      }
    }
  };
  fetch(0);

  f32x4 o[HT][8];  // O^T tile mt of head tile ht: dims 16mt + 4g + i of head c
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) o[ht][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[HT], l[HT];  // running max (base-2 scaled) and sum of head c of each tile
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    m[ht] = -INFINITY;
    l[ht] = 0.f;
  }

  for (int c0 = 0; c0 < k; c0 += C) {
    // 2. decode the chunk into the tile
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq) {
#pragma unroll
      for (int w = 0; w < 4; ++w)
        *reinterpret_cast<u32x4*>(kt + tile_at(lslot, 32 * (NQ * part + qq) + 8 * w)) =
            t >= 0 ? decode8(nib[qq][w], sc[qq]) : u32x4{0u, 0u, 0u, 0u};
    }
    if (part == 0) sbias[lslot] = t >= 0 ? 0.f : -INFINITY;
    __syncthreads();
    if (c0 + C < k) fetch(c0 + C);  // in flight during the MFMAs

    // 3. S^T = K Q^T: each K fragment feeds the wave's HT head tiles
    f32x4 sacc[HT][NST];
#pragma unroll
    for (int st = 0; st < NST; ++st) {
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) sacc[ht][st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const Frag a = *reinterpret_cast<const Frag*>(kt + tile_at(16 * st + c, 8 * g + 32 * s));
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
          sacc[ht][st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[ht][s], sacc[ht][st], 0, 0, 0);
      }
    }
    // 4. online softmax (base 2), head c of each tile
    Frag pb[HT][C / 32];
    float alpha[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      float x[NST][4], cmax = -INFINITY;
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        const f32x4 b4 = *reinterpret_cast<const f32x4*>(&sbias[16 * st + 4 * g]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[st][i] = fmaf(sacc[ht][st][i], scale_log2, b4[i]);
          cmax = fmaxf(cmax, x[st][i]);
        }
      }
      cmax = shfl_max(cmax);
      const float m_new = fmaxf(m[ht], cmax);
      const bool any = m_new > -INFINITY;
      alpha[ht] = any ? __builtin_amdgcn_exp2f(m[ht] - m_new) : 1.f;
      float psum = 0.f;
#pragma unroll
      for (int st = 0; st < NST; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = any ? __builtin_amdgcn_exp2f(x[st][i] - m_new) : 0.f;
          psum += p;
          pb[ht][st >> 1][4 * (st & 1) + i] = __bf16(p);
        }
      l[ht] = fmaf(l[ht], alpha[ht], shfl_sum(psum));
      m[ht] = m_new;
    }
    // 5. O^T = O^T * alpha + V^T P^T: each V^T fragment feeds HT tiles
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) o[ht][mt] *= alpha[ht];
#pragma unroll
    for (int ks = 0; ks < C / 32; ++ks) {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const uint2 lo = vt_frag4(kt, 32 * ks + 4 * g, mt, lane);
        const uint2 hi = vt_frag4(kt, 32 * ks + 16 + 4 * g, mt, lane);
        const Frag a = __builtin_bit_cast(Frag, u32x4{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
          o[ht][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[ht][ks], o[ht][mt], 0, 0, 0);
      }
    }
    __syncthreads();  // the tile is rewritten by the next chunk
  }

  // 6. the sink joins the denominator; store head c's outputs of each tile
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int head = hbase + 16 * ht + c;
    const float s2 = sink ? sink[head] * 1.4426950408889634f : -INFINITY;
    const float mf = fmaxf(m[ht], s2);
    float f = 0.f;
    if (mf > -INFINITY) {
      const float a = __builtin_amdgcn_exp2f(m[ht] - mf);
      f = a / (l[ht] * a + __builtin_amdgcn_exp2f(s2 - mf));
    }
    float* orow = out + (r * H + head) * int64_t(kHeadDim);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) *reinterpret_cast<f32x4*>(orow + 16 * mt + 4 * g) = o[ht][mt] * f;
  }
}

}  // namespace

hipError_t launch_sparse_attention(const uint16_t* q, const uint8_t* kv_fp4, const uint8_t* kv_scale,
                                   const int32_t* block_table, const int32_t* sel_pos, const int32_t* row_seq,
                                   const float* sink, float scale, float* out, int R, int H, int k, int MB, int bs,
                                   hipStream_t stream) {
  const int bs_log2 = __builtin_ctz(unsigned(bs));
  const float scale_log2 = float(double(scale) * 1.4426950408889634);  // softmax in base 2
  // Fewer (row, 64-head) workgroups than CUs (decode): 16 heads per workgroup
  // with the keys split across its waves, four times the workgroups.
  if (int64_t(R) * (H / kAttnHeads) < 256)
    hipLaunchKernelGGL((sparse_attention_split_kernel<kSplitWaves>), dim3(unsigned(int64_t(R) * (H / 16))),
                       dim3(64 * kSplitWaves), 0, stream, q, reinterpret_cast<const uint32_t*>(kv_fp4), kv_scale,
                       block_table, sel_pos, row_seq, sink, scale_log2, out, H, k, MB, bs_log2);
  else
    hipLaunchKernelGGL((attention_rows_kernel<kRowsHeadTiles, kRowsChunk>), dim3(unsigned(int64_t(R) * (H / kAttnHeads))),
                       dim3(64 * (4 / kRowsHeadTiles)), 0, stream, q, reinterpret_cast<const uint32_t*>(kv_fp4), kv_scale,
                       block_table, sel_pos, row_seq, sink, scale_log2, out, H, k, MB, bs_log2);
  return hipGetLastError();
}

}  // namespace xk
