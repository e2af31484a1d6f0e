// probe.hip -- measurement probes: the measured ceilings that the benchmark
// reports beside MI355X's spec peaks (the TSO paper measures its MAC and DRAM
// roofs next to the theoretical ones, because the rest of the machine keeps
// either from being reached; roofline evaluation, Figure 11). Not part of the
// convolution path.
//
//   * mfma_peak_kernel: back-to-back independent v_mfma_f32_16x16x32_bf16
//     (or v_mfma_i32_16x16x64_i8) on every SIMD, operands that vary per lane
//     (varying data draws more power than constants, which sets the clock).
//     The instructions are written out with their accumulators tied to one
//     register quad each: the compiler's own selection moves accumulators
//     between register files around every instruction of such a loop, and
//     those moves, not the matrix cores, would set the rate.
//   * stream_copy_kernel: a read + write stream, 16 bytes per lane, four
//     chunks per lane in flight, stores that do not stay in the caches.
#include <hip/hip_runtime.h>

#include "../../include/conv_probe.h"
#include "device_common.h"

namespace convnhwc {
namespace {

constexpr int kChains = 8;  // independent accumulators per wave

template <int ESZ>
__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  const uint32_t h = (uint32_t)(blockIdx.x * 256 + threadIdx.x) * 2654435761u;
  i32x4 a, b;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    // bf16 pairs with exponents near 1 and pseudo-random mantissas (int8:
    // pseudo-random bytes)
    const uint32_t m = (h >> (r * 3)) ^ (0x9E3779B9u * (r + 1));
    a[r] = (int)(ESZ == 2 ? ((m & 0x007F007Fu) | 0x3F003F00u) : m);
    b[r] = (int)(ESZ == 2 ? (((m >> 7) & 0x007F007Fu) | 0x3E803E80u) : (m * 0x01000193u));
  }
  if constexpr (ESZ == 2) {
    f32x4 c[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j) c[j] = f32x4{0, 0, 0, 0};
    // wait states between the VALU writes of the accumulators and the first
    // MFMA that reads them, and between the last MFMA and the VALU reads
#pragma unroll
    for (int j = 0; j < kChains; ++j) asm volatile("s_nop 4" : "+v"(c[j]));
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < kChains; ++j)
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c[j]) : "v"(a), "v"(b));
    }
#pragma unroll
    for (int j = 0; j < kChains; ++j) asm volatile("s_nop 7\n\ts_nop 7" : "+v"(c[j]));
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kChains; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
    if (lane == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
  } else {
    i32x4 c[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j) c[j] = i32x4{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < kChains; ++j) asm volatile("s_nop 4" : "+v"(c[j]));
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < kChains; ++j)
        asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+v"(c[j]) : "v"(a), "v"(b));
    }
#pragma unroll
    for (int j = 0; j < kChains; ++j) asm volatile("s_nop 7\n\ts_nop 7" : "+v"(c[j]));
    int s = 0;
#pragma unroll
    for (int j = 0; j < kChains; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
    if (lane == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = (float)s;
  }
}

// n16 16-byte chunks from src to dst. Each lane moves four chunks per step,
// 256 chunks apart, so a wave keeps four 1 KiB requests in flight.
__global__ __launch_bounds__(256) void stream_copy_kernel(const i32x4* __restrict__ src, i32x4* __restrict__ dst,
                                                          int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 1024;
  int64_t i = (int64_t)blockIdx.x * 1024 + threadIdx.x;
  for (; i + 768 < n16; i += stride) {
    const i32x4 v0 = src[i], v1 = src[i + 256], v2 = src[i + 512], v3 = src[i + 768];
    __builtin_nontemporal_store(v0, dst + i);
    __builtin_nontemporal_store(v1, dst + i + 256);
    __builtin_nontemporal_store(v2, dst + i + 512);
    __builtin_nontemporal_store(v3, dst + i + 768);
  }
  for (int k = 0; k < 4; ++k, i += 256)
    if (i < n16) dst[i] = src[i];
}

}  // namespace
}  // namespace convnhwc

using namespace convnhwc;

extern "C" {

conv_status conv_probe_mfma(int32_t dtype, int32_t iters, float* out, double* ops, void* stream) {
  if (!out || !ops) return CONV_E_NULL;
  if ((dtype != CONV_BF16 && dtype != CONV_I8) || iters <= 0) return CONV_E_UNSUPPORTED;
  if ((uintptr_t)out & 3) return CONV_E_ALIGN;
  const int wgs = kProbeMfmaWorkgroups;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == CONV_BF16)
    hipLaunchKernelGGL(mfma_peak_kernel<2>, dim3(wgs), dim3(256), 0, s, iters, out);
  else
    hipLaunchKernelGGL(mfma_peak_kernel<1>, dim3(wgs), dim3(256), 0, s, iters, out);
  if (hipGetLastError() != hipSuccess) return CONV_E_HIP;
  // 16x16 outputs x K (32 bf16 or 64 int8) multiply-adds per MFMA
  const double per_mfma = 2.0 * 16 * 16 * (dtype == CONV_BF16 ? 32 : 64);
  *ops = per_mfma * kChains * (double)iters * wgs * 4;
  return CONV_OK;
}

conv_status conv_probe_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (!src || !dst) return CONV_E_NULL;
  if (bytes <= 0 || bytes % 16) return CONV_E_SHAPE;
  if (((uintptr_t)src | (uintptr_t)dst) & 15) return CONV_E_ALIGN;
  const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
  if (a < b + (uintptr_t)bytes && b < a + (uintptr_t)bytes) return CONV_E_ALIAS;
  const int64_t n16 = bytes / 16;
  int64_t wgs = (n16 + 1023) / 1024;
  if (wgs > 256 * 16) wgs = 256 * 16;
  hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)wgs), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const i32x4*>(src), static_cast<i32x4*>(dst), n16);
  return hipGetLastError() == hipSuccess ? CONV_OK : CONV_E_HIP;
}

}  // extern "C"
