// DSA indexer logits on gfx950 MFMA.
//
// Computes (page "xkernels #27 -- [AMD/MI300A] DeepSeek-V4 DSA indexer +
// attention", comment announcing dsa_indexer_logits):
//   logits[b,t,j] = sum_h w[b,t,h] * relu(q[b,t,h,:] . k[b,j,:]),  j <= limit[b,t]
//   logits[b,t,j] = -inf                                             otherwise
// with H = 64 heads, D = 128, one shared key per position (MQA).
//
// Mapping onto the matrix cores: for one query the 64 heads are the M
// dimension (two 32-row MFMA tiles), 32 keys are the N dimension and D the
// contraction. With a 32x32 fp32 accumulator a lane holds 16 rows (heads) of
// ONE column (key), so the ReLU, the head weight and most of the head sum run
// in registers of that lane; one cross-lane add (lane l with l^32) finishes
// the 64-head sum. The score never leaves registers until it is final.
//
// bf16: v_mfma_f32_32x32x16_bf16, 8 steps over D.
// fp8 : v_mfma_scale_f32_32x32x64_f8f6f4 with both operands OCP e4m3 and unit
//       block scales, 2 steps over D. The dequant scales are positive, so
//       relu(sq*sk*x) = sq*sk*relu(x): sq folds into the head weight and sk
//       multiplies the finished score.
//
// Two kernels share that core:
//  * decode  (few queries, long rows; HBM bound): a workgroup owns one query
//    and a key chunk; each wave streams its own 32-key tiles straight from
//    HBM into MFMA B registers, prefetching one tile ahead.
//  * prefill (many queries; MFMA bound): a workgroup owns 8 queries (one per
//    wave) and a key chunk; 64-key tiles are staged once in LDS and read by
//    all 8 waves, so each key byte fetched from L2 feeds 8 queries.
// Causal tiles that lie wholly past a query's limit are skipped and filled
// with -inf.
#include <math.h>

#include <algorithm>

#include "xk_internal.h"

namespace xk {
namespace {

// Row (head) held in register i of lane `lane` by a 32x32 fp32 MFMA result;
// the column (key) is lane % 32.
__device__ __forceinline__ int acc_row(int i, int lane) {
  return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

template <bool FP8>
struct Mma;

template <>
struct Mma<false> {  // bf16 operands
  using Frag = bf16x8;                 // 8 bf16 = 16 bytes per lane
  static constexpr int kSteps = 8;     // 8 x K16 = 128
  static constexpr int kElemBytes = 2;
  // First d of the fragment of step s held by lane half hf (A and B alike).
  __device__ static int dofs(int s, int hf) { return 16 * s + 8 * hf; }
  __device__ static Frag load(const uint8_t* p) { return *reinterpret_cast<const Frag*>(p); }
  __device__ static f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mma<true> {  // OCP e4m3 operands
  using Frag = i32x8;                  // 32 fp8 = 32 bytes per lane
  static constexpr int kSteps = 2;     // 2 x K64 = 128
  static constexpr int kElemBytes = 1;
  __device__ static int dofs(int s, int hf) { return 64 * s + 32 * hf; }
  __device__ static Frag load(const uint8_t* p) {
    const i32x4 lo = *reinterpret_cast<const i32x4*>(p);
    const i32x4 hi = *reinterpret_cast<const i32x4*>(p + 16);
    return Frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  __device__ static f32x16 mma(Frag a, Frag b, f32x16 c) {
    // operand formats 0/0 = fp8 e4m3 (OCP); E8M0 block scales 127 = 1.0
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
};

// Everything one wave keeps for its query: the 64x128 q block as MFMA A
// fragments and the head weights laid out like the accumulator rows.
template <bool FP8>
struct QueryRegs {
  using M = Mma<FP8>;
  typename M::Frag a[2][M::kSteps];
  float wr[2][16];

  __device__ void load(const uint8_t* qrow, const float* wrow, const float* sqrow, int lane) {
    const int hf = lane >> 5, col = lane & 31;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int s = 0; s < M::kSteps; ++s)
        a[mt][s] = M::load(qrow + ((32 * mt + col) * kHeadDim + M::dofs(s, hf)) * M::kElemBytes);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int h = 32 * mt + acc_row(i, lane);
        wr[mt][i] = FP8 ? wrow[h] * sqrow[h] : wrow[h];
      }
  }

  __device__ void zero() {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int s = 0; s < M::kSteps; ++s) a[mt][s] = typename M::Frag{};
#pragma unroll
      for (int i = 0; i < 16; ++i) wr[mt][i] = 0.f;
    }
  }

  // Score of key (lane % 32) of a 32-key tile whose B fragments are `b`.
  // Returned in both lane halves.
  __device__ float score(const typename M::Frag (&b)[M::kSteps]) const {
    f32x16 acc0 = {}, acc1 = {};
#pragma unroll
    for (int s = 0; s < M::kSteps; ++s) {
      acc0 = M::mma(a[0][s], b[s], acc0);
      acc1 = M::mma(a[1][s], b[s], acc1);
    }
    float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      p0 = fmaf(wr[0][i], fmaxf(acc0[i], 0.f), p0);
      p1 = fmaf(wr[0][i + 1], fmaxf(acc0[i + 1], 0.f), p1);
      p2 = fmaf(wr[1][i], fmaxf(acc1[i], 0.f), p2);
      p3 = fmaf(wr[1][i + 1], fmaxf(acc1[i + 1], 0.f), p3);
    }
    float p = (p0 + p1) + (p2 + p3);
    p += __shfl_xor(p, 32);  // the other 32 heads of this key live in lane ^ 32
    return p;
  }
};

__device__ __forceinline__ int clamp_limit(const int32_t* limit, int64_t bt, int K) {
  return limit ? min(limit[bt], K - 1) : K - 1;
}

// ---------------------------------------------------------------------------
// decode: 1-D grid over (B*T rows) x (key chunks); 4 waves, each streaming its own 32-key tiles.
template <bool FP8>
__global__ __launch_bounds__(256, 2) void logits_decode_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale,
    const uint8_t* __restrict__ k, const float* __restrict__ k_scale,
    const float* __restrict__ w, const int32_t* __restrict__ limit,
    float* __restrict__ out, int T, int K, int keys_per_wg, int n_chunks) {
  using M = Mma<FP8>;
  constexpr int kRowBytes = kHeadDim * M::kElemBytes;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hf = lane >> 5, col = lane & 31;
  const int64_t bt = blockIdx.x / n_chunks;  // all chunks of a row are adjacent
  const int chunk = int(blockIdx.x % n_chunks);
  const int64_t b = bt / T;
  const int lim = clamp_limit(limit, bt, K);
  const int j_begin = chunk * keys_per_wg;
  const int j_end = min(j_begin + keys_per_wg, K);
  float* orow = out + bt * K;

  for (int j = max(j_begin, lim + 1) + int(threadIdx.x); j < j_end; j += 256) orow[j] = -INFINITY;
  const int c_end = min(j_end, lim + 1);  // keys [j_begin, c_end) are scored
  if (c_end <= j_begin) return;

  QueryRegs<FP8> qr;
  qr.load(q + bt * (kHeads * kRowBytes), w + bt * kHeads, FP8 ? q_scale + bt * kHeads : nullptr,
          lane);
  const uint8_t* kseq = k + b * int64_t(K) * kRowBytes;
  const float* skseq = FP8 ? k_scale + b * int64_t(K) : nullptr;

  typename M::Frag nxt[M::kSteps];
  auto load_tile = [&](int j0) {
    const int row = min(j0 + col, K - 1);  // ragged tail: clamp, result discarded
    const uint8_t* krow = kseq + int64_t(row) * kRowBytes;
#pragma unroll
    for (int s = 0; s < M::kSteps; ++s) nxt[s] = M::load(krow + M::dofs(s, hf) * M::kElemBytes);
  };
  int j0 = j_begin + 32 * wave;
  if (j0 < c_end) load_tile(j0);
  for (; j0 < c_end; j0 += 128) {
    typename M::Frag cur[M::kSteps];
#pragma unroll
    for (int s = 0; s < M::kSteps; ++s) cur[s] = nxt[s];
    if (j0 + 128 < c_end) load_tile(j0 + 128);
    float p = qr.score(cur);
    const int j = j0 + col;
    if (hf == 0 && j < c_end) {
      if (FP8) p *= skseq[j];
      orow[j] = p;
    }
  }
}

// ---------------------------------------------------------------------------
// prefill: 1-D grid over (query blocks of 8, longest causal rows first) x B x
// (key chunks); 8 waves = 8 queries.
constexpr int kPrefillQ = 8;
constexpr int kPrefillTile = 64;

template <bool FP8>
__global__ __launch_bounds__(512, 2) void logits_prefill_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale,
    const uint8_t* __restrict__ k, const float* __restrict__ k_scale,
    const float* __restrict__ w, const int32_t* __restrict__ limit,
    float* __restrict__ out, int B, int T, int K, int keys_per_wg, int n_chunks, int n_qblocks) {
  using M = Mma<FP8>;
  constexpr int kRowBytes = kHeadDim * M::kElemBytes;
  constexpr int kPitch = kRowBytes + 16;  // 16-byte pad: conflict-free fragment reads
  constexpr int kChunks = kRowBytes / 16;
  __shared__ __attribute__((aligned(16))) uint8_t tile[kPrefillTile * kPitch];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hf = lane >> 5, col = lane & 31;
  const int chunk = int(blockIdx.x % n_chunks);
  const int rest = int(blockIdx.x / n_chunks);
  const int64_t b = rest % B;
  const int qb = n_qblocks - 1 - rest / B;  // longest causal rows first
  const int t = qb * kPrefillQ + wave;
  const bool qvalid = t < T;
  const int64_t bt = b * T + t;
  const int lim = qvalid ? clamp_limit(limit, bt, K) : -1;
  int blk_lim = -1;
#pragma unroll
  for (int i = 0; i < kPrefillQ; ++i) {
    const int ti = qb * kPrefillQ + i;
    if (ti < T) blk_lim = max(blk_lim, clamp_limit(limit, b * T + ti, K));
  }
  const int j_begin = chunk * keys_per_wg;
  const int j_end = min(j_begin + keys_per_wg, K);
  float* orow = out + bt * K;
  if (qvalid)
    for (int j = max(j_begin, lim + 1) + lane; j < j_end; j += 64) orow[j] = -INFINITY;
  const int c_end = min(j_end, blk_lim + 1);
  if (c_end <= j_begin) return;  // uniform over the workgroup

  QueryRegs<FP8> qr;
  if (qvalid)
    qr.load(q + bt * (kHeads * kRowBytes), w + bt * kHeads,
            FP8 ? q_scale + bt * kHeads : nullptr, lane);
  else
    qr.zero();
  const uint8_t* kseq = k + b * int64_t(K) * kRowBytes;
  const float* skseq = FP8 ? k_scale + b * int64_t(K) : nullptr;
  const int q_end = min(j_end, lim + 1);  // this wave's scored keys end

  for (int j0 = j_begin; j0 < c_end; j0 += kPrefillTile) {
    __syncthreads();  // previous tile fully consumed
    for (int c = threadIdx.x; c < kPrefillTile * kChunks; c += 512) {
      const int r = c / kChunks, cc = c % kChunks;
      const int row = min(j0 + r, K - 1);
      const u32x4 v = *reinterpret_cast<const u32x4*>(kseq + int64_t(row) * kRowBytes + cc * 16);
      *reinterpret_cast<u32x4*>(tile + r * kPitch + cc * 16) = v;
    }
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < kPrefillTile / 32; ++nt) {
      const int jt = j0 + 32 * nt;
      if (jt >= q_end) break;  // uniform per wave
      typename M::Frag bf[M::kSteps];
      const uint8_t* lrow = tile + (32 * nt + col) * kPitch;
#pragma unroll
      for (int s = 0; s < M::kSteps; ++s) bf[s] = M::load(lrow + M::dofs(s, hf) * M::kElemBytes);
      float p = qr.score(bf);
      const int j = jt + col;
      if (hf == 0 && j < q_end) {
        if (FP8) p *= skseq[j];
        orow[j] = p;
      }
    }
  }
}

int round_up(int x, int m) { return (x + m - 1) / m * m; }

}  // namespace

hipError_t launch_logits(const void* q, const float* q_scale, const void* k,
                         const float* k_scale, const float* w, const int32_t* limit,
                         float* logits, int B, int T, int K, bool fp8, hipStream_t stream) {
  const auto* q8 = static_cast<const uint8_t*>(q);
  const auto* k8 = static_cast<const uint8_t*>(k);
  if (T < kPrefillQ) {
    // one query per workgroup; ~1024 workgroups, chunks a multiple of 4 waves x 32 keys
    const int64_t rows = int64_t(B) * T;
    int64_t per = (int64_t(K) * rows + 1023) / 1024;
    int kpw = int(std::min<int64_t>(std::max<int64_t>(per, 256), K));
    kpw = round_up(kpw, 128);
    const int nch = (K + kpw - 1) / kpw;
    const dim3 grid(unsigned(rows * nch));
    if (fp8)
      hipLaunchKernelGGL(logits_decode_kernel<true>, grid, dim3(256), 0, stream, q8, q_scale, k8,
                         k_scale, w, limit, logits, T, K, kpw, nch);
    else
      hipLaunchKernelGGL(logits_decode_kernel<false>, grid, dim3(256), 0, stream, q8, q_scale, k8,
                         k_scale, w, limit, logits, T, K, kpw, nch);
  } else {
    const int nqb = (T + kPrefillQ - 1) / kPrefillQ;
    const int64_t qblocks = int64_t(nqb) * B;
    const int nkc = int(std::max<int64_t>(1, (2048 + qblocks - 1) / qblocks));
    const int kpw = round_up((K + nkc - 1) / nkc, kPrefillTile);
    const int nch = (K + kpw - 1) / kpw;
    const dim3 grid(unsigned(int64_t(nch) * qblocks));
    if (fp8)
      hipLaunchKernelGGL(logits_prefill_kernel<true>, grid, dim3(512), 0, stream, q8, q_scale, k8,
                         k_scale, w, limit, logits, B, T, K, kpw, nch, nqb);
    else
      hipLaunchKernelGGL(logits_prefill_kernel<false>, grid, dim3(512), 0, stream, q8, q_scale, k8,
                         k_scale, w, limit, logits, B, T, K, kpw, nch, nqb);
  }
  return hipGetLastError();
}

}  // namespace xk
