// C ABI of libxk: argument validation, device check and kernel dispatch.
// Every check that needs no device runs before the first HIP call, so a bad
// argument is reported without touching the GPU.
#include <math.h>
#include <string.h>

#include <map>
#include <mutex>
#include <string>

#include "../../include/xk.h"
#include "xk_internal.h"

#define XK_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

xk_status fail(xk_status s, const std::string& why) {
  g_last_error = why;
  return s;
}

xk_status ok() {
  g_last_error.clear();
  return XK_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// The code objects in this library are built for gfx950 only.
xk_status check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(XK_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  static std::mutex mu;
  static std::map<int, bool> is_gfx950;
  std::lock_guard<std::mutex> lock(mu);
  auto it = is_gfx950.find(dev);
  if (it == is_gfx950.end()) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return fail(XK_ERR_HIP, std::string("hipGetDeviceProperties: ") + hipGetErrorString(e));
    it = is_gfx950.emplace(dev, strncmp(prop.gcnArchName, "gfx950", 6) == 0).first;
  }
  if (!it->second) return fail(XK_ERR_UNSUPPORTED, "device is not gfx950 (MI355X)");
  return XK_OK;
}

xk_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(XK_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return ok();
}

// Checks shared by xk_indexer_logits and xk_indexer_logits_topk.
xk_status check_logits_args(const void* q, const float* q_scale, const void* k, const float* k_scale,
                            const float* w, const void* out, int B, int T, int K, int H, int D, int dtype) {
  if (!q || !k || !w || !out) return fail(XK_ERR_INVALID_ARGUMENT, "null q, k, w or output");
  if (B < 1 || T < 1 || K < 1 || H < 1 || D < 1)
    return fail(XK_ERR_INVALID_ARGUMENT, "B, T, K, H, D must be >= 1");
  if (dtype != XK_BF16 && dtype != XK_FP8_E4M3_OCP) return fail(XK_ERR_INVALID_ARGUMENT, "unknown dtype");
  const bool fp8 = dtype == XK_FP8_E4M3_OCP;
  if (fp8 && (!q_scale || !k_scale)) return fail(XK_ERR_INVALID_ARGUMENT, "fp8 needs q_scale and k_scale");
  if (!fp8 && (q_scale || k_scale)) return fail(XK_ERR_INVALID_ARGUMENT, "bf16 takes no scales");
  if (H != xk::kHeads || D != xk::kHeadDim)
    return fail(XK_ERR_UNSUPPORTED, "only H=64, D=128 (DeepSeek-V4 indexer) is implemented");
  if (!aligned(q, 16) || !aligned(k, 16)) return fail(XK_ERR_INVALID_ARGUMENT, "q and k must be 16-byte aligned");
  if (int64_t(B) * T > (int64_t(1) << 30)) return fail(XK_ERR_UNSUPPORTED, "B*T above 2^30");
  // 1 TB of fp32 logits; keeps every launch grid (rows x key chunks) below 2^31
  if (int64_t(B) * T * K > (int64_t(1) << 38)) return fail(XK_ERR_UNSUPPORTED, "B*T*K above 2^38");
  return XK_OK;
}

}  // namespace

XK_EXPORT const char* xk_status_string(xk_status s) {
  switch (s) {
    case XK_OK: return "XK_OK";
    case XK_ERR_INVALID_ARGUMENT: return "XK_ERR_INVALID_ARGUMENT";
    case XK_ERR_UNSUPPORTED: return "XK_ERR_UNSUPPORTED";
    case XK_ERR_HIP: return "XK_ERR_HIP";
  }
  return "XK_UNKNOWN_STATUS";
}

XK_EXPORT const char* xk_last_error(void) { return g_last_error.c_str(); }

XK_EXPORT xk_status xk_indexer_logits(const void* q, const float* q_scale, const void* k,
                                      const float* k_scale, const float* w, const int32_t* limit,
                                      float* logits, int B, int T, int K, int H, int D, xk_qk_dtype dtype,
                                      hipStream_t stream) {
  xk_status s = check_logits_args(q, q_scale, k, k_scale, w, logits, B, T, K, H, D, dtype);
  if (s != XK_OK) return s;
  const bool fp8 = dtype == XK_FP8_E4M3_OCP;
  s = check_device();
  if (s != XK_OK) return s;
  return launched(xk::launch_logits(q, q_scale, k, k_scale, w, limit, logits, B, T, K, fp8,
                                    static_cast<hipStream_t>(stream)),
                  "xk_indexer_logits launch");
}

XK_EXPORT xk_status xk_indexer_logits_paged(const void* q, const float* q_scale, const float* w,
                                            const int32_t* limit, const void* k_cache,
                                            const void* k_scale, const int32_t* block_table,
                                            float* logits, int B, int T, int K, int H, int D, int MB,
                                            int NB, int bs, xk_kcache_format kformat, hipStream_t stream) {
  if (!q || !q_scale || !w || !k_cache || !k_scale || !block_table || !logits)
    return fail(XK_ERR_INVALID_ARGUMENT,
                "null q, q_scale, w, k_cache, k_scale, block_table or logits");
  if (B < 1 || T < 1 || K < 1 || H < 1 || D < 1 || MB < 1 || NB < 1 || bs < 1)
    return fail(XK_ERR_INVALID_ARGUMENT, "B, T, K, H, D, MB, NB, bs must be >= 1");
  if (kformat != XK_KCACHE_MXFP4 && kformat != XK_KCACHE_FP8_E4M3_OCP)
    return fail(XK_ERR_INVALID_ARGUMENT, "unknown key cache format");
  if (H != xk::kHeads || D != xk::kHeadDim)
    return fail(XK_ERR_UNSUPPORTED, "only H=64, D=128 (DeepSeek-V4 indexer) is implemented");
  if ((bs & (bs - 1)) != 0) return fail(XK_ERR_INVALID_ARGUMENT, "block size must be a power of two");
  if (bs < 16) return fail(XK_ERR_UNSUPPORTED, "block size must be >= 16 (a 16-key tile within one page)");
  if (int64_t(K) > int64_t(MB) * bs)
    return fail(XK_ERR_INVALID_ARGUMENT, "K exceeds the positions the block table maps (MB*bs)");
  if (int64_t(NB) * bs > (int64_t(1) << 31) - 1)
    return fail(XK_ERR_UNSUPPORTED, "NB*bs (cache positions) above 2^31-1");
  if (int64_t(B) * T > (int64_t(1) << 30)) return fail(XK_ERR_UNSUPPORTED, "B*T above 2^30");
  if (int64_t(B) * T * K > (int64_t(1) << 38)) return fail(XK_ERR_UNSUPPORTED, "B*T*K above 2^38");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(k_scale, 4))
    return fail(XK_ERR_INVALID_ARGUMENT, "q and k_cache must be 16-byte, k_scale 4-byte aligned");
  xk_status s = check_device();
  if (s != XK_OK) return s;
  return launched(xk::launch_logits_paged(q, q_scale, w, limit, k_cache, k_scale, block_table, logits,
                                          B, T, K, MB, bs, kformat == XK_KCACHE_MXFP4,
                                          static_cast<hipStream_t>(stream)),
                  "xk_indexer_logits_paged launch");
}

XK_EXPORT xk_status xk_quant_fp8_rows(const void* x, xk_in_dtype x_dtype, uint8_t* out, float* scale,
                                      int64_t N, int D, hipStream_t stream) {
  if (!x || !out || !scale) return fail(XK_ERR_INVALID_ARGUMENT, "null x, out or scale");
  if (N < 1 || D < 1) return fail(XK_ERR_INVALID_ARGUMENT, "N, D must be >= 1");
  if (x_dtype != XK_IN_FP32 && x_dtype != XK_IN_BF16)
    return fail(XK_ERR_INVALID_ARGUMENT, "unknown x dtype");
  if (D != xk::kHeadDim) return fail(XK_ERR_UNSUPPORTED, "only D=128 is implemented");
  if (N > (int64_t(1) << 34)) return fail(XK_ERR_UNSUPPORTED, "N above 2^34");  // grid: N / 16 workgroups
  if (!aligned(x, 16) || !aligned(out, 8) || !aligned(scale, 4))
    return fail(XK_ERR_INVALID_ARGUMENT, "x, out or scale misaligned (16, 8, 4 bytes)");
  xk_status s = check_device();
  if (s != XK_OK) return s;
  return launched(xk::launch_quant_fp8_rows(x, x_dtype == XK_IN_BF16, out, scale, N,
                                            static_cast<hipStream_t>(stream)),
                  "xk_quant_fp8_rows launch");
}

XK_EXPORT xk_status xk_mxfp4_cache_write(const void* x, xk_in_dtype x_dtype, const int64_t* slots,
                                         uint8_t* kv_fp4, uint8_t* kv_scale, int64_t N, int NB,
                                         int bs, int D, hipStream_t stream) {
  if (!x || !slots || !kv_fp4 || !kv_scale)
    return fail(XK_ERR_INVALID_ARGUMENT, "null x, slots, kv_fp4 or kv_scale");
  if (N < 1 || NB < 1 || bs < 1 || D < 1)
    return fail(XK_ERR_INVALID_ARGUMENT, "N, NB, bs, D must be >= 1");
  if (x_dtype != XK_IN_FP32 && x_dtype != XK_IN_BF16)
    return fail(XK_ERR_INVALID_ARGUMENT, "unknown x dtype");
  if (D != xk::kHeadDim) return fail(XK_ERR_UNSUPPORTED, "only D=128 is implemented");
  if (N > (int64_t(1) << 34)) return fail(XK_ERR_UNSUPPORTED, "N above 2^34");  // grid: N / 16 workgroups
  if (!aligned(x, 16) || !aligned(slots, 8) || !aligned(kv_fp4, 4))
    return fail(XK_ERR_INVALID_ARGUMENT, "x, slots or kv_fp4 misaligned (16, 8, 4 bytes)");
  xk_status s = check_device();
  if (s != XK_OK) return s;
  return launched(xk::launch_mxfp4_write(x, x_dtype == XK_IN_BF16, slots, kv_fp4, kv_scale, N,
                                         int64_t(NB) * bs, static_cast<hipStream_t>(stream)),
                  "xk_mxfp4_cache_write launch");
}

XK_EXPORT size_t xk_indexer_topk_workspace_size(int R, int K, int k) {
  (void)R;
  (void)K;
  (void)k;
  return 0;  // rows are selected entirely on chip
}

XK_EXPORT xk_status xk_indexer_topk(const float* logits, const int32_t* limit, int32_t* idx, int R,
                                    int K, int k, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  if (!logits || !idx) return fail(XK_ERR_INVALID_ARGUMENT, "null logits or idx");
  if (R < 1 || K < 1 || k < 1) return fail(XK_ERR_INVALID_ARGUMENT, "R, K, k must be >= 1");
  if (k > xk::kMaxTopk) return fail(XK_ERR_UNSUPPORTED, "k above 2048");
  const size_t need = xk_indexer_topk_workspace_size(R, K, k);
  if (workspace_bytes < need || (need && !workspace))
    return fail(XK_ERR_INVALID_ARGUMENT, "workspace too small");
  xk_status s = check_device();
  if (s != XK_OK) return s;
  return launched(xk::launch_topk(logits, limit, idx, R, K, k, static_cast<hipStream_t>(stream)),
                  "xk_indexer_topk launch");
}

XK_EXPORT size_t xk_indexer_logits_topk_workspace_size(int B, int T, int K, int k, xk_qk_dtype dtype) {
  if (B < 1 || T < 1 || K < 1 || k < 1 || k > xk::kMaxTopk) return 0;
  if (dtype != XK_BF16 && dtype != XK_FP8_E4M3_OCP) return 0;
  if (int64_t(B) * T > (int64_t(1) << 30)) return 0;
  return xk::plan_fused(B, T, K, k, dtype == XK_FP8_E4M3_OCP).bytes;
}

XK_EXPORT xk_status xk_indexer_logits_topk(const void* q, const float* q_scale, const void* k,
                                           const float* k_scale, const float* w, const int32_t* limit,
                                           int32_t* idx, int B, int T, int K, int H, int D, int topk, xk_qk_dtype dtype,
                                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  xk_status s = check_logits_args(q, q_scale, k, k_scale, w, idx, B, T, K, H, D, dtype);
  if (s != XK_OK) return s;
  if (topk < 1) return fail(XK_ERR_INVALID_ARGUMENT, "topk must be >= 1");
  if (topk > xk::kMaxTopk) return fail(XK_ERR_UNSUPPORTED, "topk above 2048");
  if (int64_t(B) * T * topk > (int64_t(1) << 31) - 1) return fail(XK_ERR_UNSUPPORTED, "B*T*topk above 2^31-1");
  const size_t need = xk_indexer_logits_topk_workspace_size(B, T, K, topk, dtype);
  if (!workspace || workspace_bytes < need) return fail(XK_ERR_INVALID_ARGUMENT, "workspace too small");
  if (!aligned(workspace, 256)) return fail(XK_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  s = check_device();
  if (s != XK_OK) return s;
  return launched(xk::launch_logits_topk(q, q_scale, k, k_scale, w, limit, idx, B, T, K, topk,
                                         dtype == XK_FP8_E4M3_OCP, workspace, static_cast<hipStream_t>(stream)),
                  "xk_indexer_logits_topk launch");
}

// ---------------------------------------------------------------------------
// Fused logits -> top-k for callers that cannot allocate: the workspace is
// this file-scope device array (one per GPU, alive until the process ends).
// Host code never passes the array's name to a kernel: its host-side symbol
// is not a device address. The device address comes from
// hipGetSymbolAddress, once per device with that device current.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`.
xk_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(XK_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(XK_ERR_UNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(XK_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return XK_OK;
}

// Fewest near-equal parts (sizes n / parts and its ceiling) of n items with
// every part at least min_size and fits(size) true; 0 if there is none.
template <class F>
int64_t split_parts(int64_t n, int64_t min_size, F fits) {
  for (int64_t parts = 1; parts <= n;) {
    const int64_t lo = n / parts, hi = (n + parts - 1) / parts;
    if (lo < min_size) return 0;
    if (fits(lo) && fits(hi)) return parts;
    parts += parts / 8 + 1;
  }
  return 0;
}

}  // namespace

XK_EXPORT xk_status xk_indexer_logits_topk_noalloc(const void* q, const float* q_scale, const void* k,
                                                   const float* k_scale, const float* w, const int32_t* limit,
                                                   int32_t* idx, int B, int T, int K, int H, int D, int topk,
                                                   xk_qk_dtype dtype, hipStream_t stream) {
  xk_status s = check_logits_args(q, q_scale, k, k_scale, w, idx, B, T, K, H, D, dtype);
  if (s != XK_OK) return s;
  if (topk < 1) return fail(XK_ERR_INVALID_ARGUMENT, "topk must be >= 1");
  if (topk > xk::kMaxTopk) return fail(XK_ERR_UNSUPPORTED, "topk above 2048");
  if (int64_t(B) * T * topk > (int64_t(1) << 31) - 1) return fail(XK_ERR_UNSUPPORTED, "B*T*topk above 2^31-1");
  const bool fp8 = dtype == XK_FP8_E4M3_OCP;
  auto fits = [&](int64_t b, int64_t t) {
    return xk::plan_fused(int(b), int(t), K, topk, fp8).bytes <= kNoAllocScratchBytes;
  };
  // Slices: groups of whole sequences when one sequence fits, else one
  // sequence's queries in ranges of at least 8 (queries of a call with T >= 8
  // are always scored by the prefill kernels, so every slice gives each row
  // the bits the whole call would).
  int64_t b_parts = split_parts(B, 1, [&](int64_t bc) { return fits(bc, T); });
  int64_t t_parts = 1;
  if (b_parts == 0) {
    if (T >= 8) t_parts = split_parts(T, 8, [&](int64_t tc) { return fits(1, tc); });
    if (T < 8 || t_parts == 0)
      return fail(XK_ERR_UNSUPPORTED, "a slice of these sizes needs more than the " +
                                          std::to_string(kNoAllocScratchBytes >> 20) +
                                          " MiB of built-in scratch; use xk_indexer_logits_topk with a workspace");
    b_parts = B;
  }
  s = check_device();
  if (s != XK_OK) return s;
  void* ws = nullptr;
  s = scratch_address(&ws);
  if (s != XK_OK) return s;
  const size_t eb = fp8 ? 1 : 2;
  const auto* q8 = static_cast<const uint8_t*>(q);
  const auto* k8 = static_cast<const uint8_t*>(k);
  for (int64_t bi = 0; bi < b_parts; ++bi) {
    const int64_t b0 = B * bi / b_parts, b1 = B * (bi + 1) / b_parts;
    for (int64_t ti = 0; ti < t_parts; ++ti) {
      const int64_t t0 = T * ti / t_parts, t1 = T * (ti + 1) / t_parts;
      const int64_t Bs = b1 - b0, Ts = t_parts == 1 ? T : t1 - t0;
      const int64_t row0 = b0 * T + t0;  // first (b, t) row of the slice
      const hipError_t e = xk::launch_logits_topk(
          q8 + row0 * H * D * eb, fp8 ? q_scale + row0 * H : nullptr, k8 + b0 * int64_t(K) * D * eb,
          fp8 ? k_scale + b0 * int64_t(K) : nullptr, w + row0 * H, limit ? limit + row0 : nullptr,
          idx + row0 * topk, int(Bs), int(Ts), K, topk, fp8, ws, static_cast<hipStream_t>(stream));
      if (e != hipSuccess) return launched(e, "xk_indexer_logits_topk_noalloc launch");
    }
  }
  return ok();
}

XK_EXPORT xk_status xk_mxfp4_paged_gather(const uint8_t* kv_fp4, const uint8_t* kv_scale,
                                          const int32_t* block_table, const int32_t* sel_pos,
                                          const int32_t* row_seq, uint16_t* out, int R, int k,
                                          int S, int MB, int NB, int bs, int D, hipStream_t stream) {
  if (!kv_fp4 || !kv_scale || !block_table || !sel_pos || !out)
    return fail(XK_ERR_INVALID_ARGUMENT, "null kv_fp4, kv_scale, block_table, sel_pos or out");
  if (R < 1 || k < 1 || S < 1 || MB < 1 || NB < 1 || bs < 1 || D < 1)
    return fail(XK_ERR_INVALID_ARGUMENT, "R, k, S, MB, NB, bs, D must be >= 1");
  if (D != xk::kHeadDim) return fail(XK_ERR_UNSUPPORTED, "only D=128 is implemented");
  if ((bs & (bs - 1)) != 0) return fail(XK_ERR_INVALID_ARGUMENT, "block size must be a power of two");
  if (!row_seq && R > S) return fail(XK_ERR_INVALID_ARGUMENT, "row_seq NULL needs R <= S");
  if (!aligned(kv_fp4, 4) || !aligned(out, 16))
    return fail(XK_ERR_INVALID_ARGUMENT, "kv_fp4 must be 4-byte and out 16-byte aligned");
  if (int64_t(R) * k > (int64_t(1) << 31) - 1)
    return fail(XK_ERR_UNSUPPORTED, "R*k above 2^31-1");
  if (int64_t(NB) * bs > (int64_t(1) << 31) - 1)
    return fail(XK_ERR_UNSUPPORTED, "NB*bs (cache tokens) above 2^31-1");
  xk_status s = check_device();
  if (s != XK_OK) return s;
  return launched(xk::launch_gather(kv_fp4, kv_scale, block_table, sel_pos, row_seq, out, R, k,
                                    MB, bs, static_cast<hipStream_t>(stream)),
                  "xk_mxfp4_paged_gather launch");
}

XK_EXPORT xk_status xk_sparse_attention_mxfp4(const void* q, const uint8_t* kv_fp4, const uint8_t* kv_scale,
                                              const int32_t* block_table, const int32_t* sel_pos,
                                              const int32_t* row_seq, const float* sink, float scale, float* out,
                                              int R, int H, int k, int S, int MB, int NB, int bs, int D,
                                              hipStream_t stream) {
  if (!q || !kv_fp4 || !kv_scale || !block_table || !sel_pos || !out)
    return fail(XK_ERR_INVALID_ARGUMENT, "null q, kv_fp4, kv_scale, block_table, sel_pos or out");
  if (R < 1 || H < 1 || k < 1 || S < 1 || MB < 1 || NB < 1 || bs < 1 || D < 1)
    return fail(XK_ERR_INVALID_ARGUMENT, "R, H, k, S, MB, NB, bs, D must be >= 1");
  if (!(scale == scale) || scale == INFINITY || scale == -INFINITY)
    return fail(XK_ERR_INVALID_ARGUMENT, "scale must be finite");
  if (D != xk::kHeadDim) return fail(XK_ERR_UNSUPPORTED, "only D=128 is implemented");
  if (H % 64 != 0) return fail(XK_ERR_UNSUPPORTED, "H must be a multiple of 64");
  if (k > 2048) return fail(XK_ERR_UNSUPPORTED, "k above 2048");
  if ((bs & (bs - 1)) != 0) return fail(XK_ERR_INVALID_ARGUMENT, "block size must be a power of two");
  if (!row_seq && R > S) return fail(XK_ERR_INVALID_ARGUMENT, "row_seq NULL needs R <= S");
  if (int64_t(NB) * bs > (int64_t(1) << 31) - 1)
    return fail(XK_ERR_UNSUPPORTED, "NB*bs (cache tokens) above 2^31-1");
  if (int64_t(R) * (H / 64) > (int64_t(1) << 31) - 1) return fail(XK_ERR_UNSUPPORTED, "R*H/64 above 2^31-1");
  if (!aligned(q, 16) || !aligned(kv_fp4, 16) || !aligned(out, 16))
    return fail(XK_ERR_INVALID_ARGUMENT, "q, kv_fp4 and out must be 16-byte aligned");
  xk_status s = check_device();
  if (s != XK_OK) return s;
  return launched(xk::launch_sparse_attention(static_cast<const uint16_t*>(q), kv_fp4, kv_scale, block_table,
                                              sel_pos, row_seq, sink, scale, out, R, H, k, MB, bs,
                                              static_cast<hipStream_t>(stream)),
                  "xk_sparse_attention_mxfp4 launch");
}
