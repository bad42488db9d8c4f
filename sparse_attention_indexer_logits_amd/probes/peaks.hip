// Achievable-rate probes for the benchmark, next to the spec peaks it
// quotes: dense MFMA issue (fp8 32x32x64 and bf16 16x16x32, the tile shapes
// of the prefill logits kernels) and an HBM read stream. Not part of the
// indexer library; bench.py loads this one on its own.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Four independent accumulator chains per wave, 4 waves per SIMD: the matrix
// core never waits on a result. `in` holds 64 words of operand bits.
__global__ __launch_bounds__(256, 4) void mfma_fp8_loop(const int* __restrict__ in, float* __restrict__ out,
                                                        int iters) {
  const int l = threadIdx.x & 63;
  i32x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = in[(l + i) & 63];
    b[i] = in[(l + 3 * i) & 63];
  }
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 0, 0, 0, 127, 0, 127);
  }
  float t = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c) t += acc[c][0] + acc[c][15];
  out[blockIdx.x * 256 + threadIdx.x] = t;
}

__global__ __launch_bounds__(256, 4) void mfma_bf16_loop(const int* __restrict__ in, float* __restrict__ out,
                                                         int iters) {
  const int l = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = __bf16(float(in[(l + i) & 63] & 7));
    b[i] = __bf16(float(in[(l + 5 * i) & 63] & 3));
  }
  f32x4 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = f32x4{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
  }
  float t = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c) t += acc[c][0] + acc[c][3];
  out[blockIdx.x * 256 + threadIdx.x] = t;
}

// Grid-stride read of n16 16-byte words with non-temporal loads; one sum per thread.
__global__ __launch_bounds__(256) void read_stream(const u32x4* __restrict__ src, int64_t n16,
                                                   uint32_t* __restrict__ out) {
  uint32_t s = 0;
  const int64_t stride = int64_t(gridDim.x) * 256;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    s += v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// CU count and peak engine / memory clocks (kHz) of `dev`; 0 on success.
__attribute__((visibility("default"))) int xkp_device_info(int dev, int* cus, int* clock_khz, int* mem_clock_khz) {
  if (hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 1;
  if (hipDeviceGetAttribute(clock_khz, hipDeviceAttributeClockRate, dev) != hipSuccess) return 1;
  if (hipDeviceGetAttribute(mem_clock_khz, hipDeviceAttributeMemoryClockRate, dev) != hipSuccess) return 1;
  return 0;
}

// fp8 (kind 0) or bf16 (kind 1) MFMA loop: `blocks` workgroups of 4 waves,
// each wave 4 * iters MFMAs. in: 64 ints; out: blocks * 256 floats.
__attribute__((visibility("default"))) int xkp_mfma_loop(int kind, const int* in, float* out, int blocks, int iters,
                                                         hipStream_t stream) {
  if (blocks <= 0 || iters <= 0 || !in || !out) return 1;
  if (kind == 0)
    hipLaunchKernelGGL(mfma_fp8_loop, dim3(blocks), dim3(256), 0, stream, in, out, iters);
  else
    hipLaunchKernelGGL(mfma_bf16_loop, dim3(blocks), dim3(256), 0, stream, in, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// Read n16 16-byte words at src (16-byte aligned); out: blocks * 256 words.
__attribute__((visibility("default"))) int xkp_read_stream(const void* src, int64_t n16, uint32_t* out, int blocks,
                                                           hipStream_t stream) {
  if (blocks <= 0 || n16 < 0 || !src || !out || (reinterpret_cast<uintptr_t>(src) & 15)) return 1;
  hipLaunchKernelGGL(read_stream, dim3(blocks), dim3(256), 0, stream, static_cast<const u32x4*>(src), n16, out);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // extern "C"
