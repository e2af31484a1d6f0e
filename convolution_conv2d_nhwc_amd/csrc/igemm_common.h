// igemm_common.h -- device helpers shared by the implicit-GEMM kernels:
// buffer loads with out-of-range-reads-zero semantics, the MFMA wrappers, the
// swizzled LDS row layout, and the split-K reduction.
#pragma once

#include <algorithm>

#include "device_common.h"
#include "mfma_epilogue.h"
#include "plan.h"

namespace convnhwc {
namespace {

constexpr int kBKB = 128;         // bytes of K per tile row
constexpr uint32_t kOOB = 0x80000000u;  // buffer offset past any tensor: reads 0
constexpr int kMaxSplits = 8;     // split-K: at most this many K ranges (plan_split_k)


template <int ESZ>
struct Mfma;

template <>
struct Mfma<2> {
  typedef f32x4 acc_t;
  static __device__ __forceinline__ acc_t run(i32x4 a, i32x4 b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

template <>
struct Mfma<1> {
  typedef i32x4 acc_t;
  static __device__ __forceinline__ acc_t run(i32x4 a, i32x4 b, acc_t c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
  }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}

__device__ __forceinline__ i32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

// Same with a wave-uniform byte offset added by the buffer unit (soffset).
__device__ __forceinline__ i32x4 bload16s(__amdgpu_buffer_rsrc_t r, uint32_t off, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, soff, 0);
}

template <int ESZ>
__device__ __forceinline__ uint32_t bload_elem(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (ESZ == 2)
    return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
  else
    return __builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
}

// q = n / d and r = n % d for 0 <= n < 2^24 and 1 <= d < 2^24 through an fp32
// reciprocal (rcp_d = 1.0f / d): the float quotient is off by at most one,
// and one correction step each way makes it exact.
__device__ __forceinline__ void divmod_small(int n, int d, float rcp_d, int& q, int& r) {
  q = (int)((float)n * rcp_d);
  r = n - q * d;
  if (r < 0) {
    --q;
    r += d;
  }
  if (r >= d) {
    ++q;
    r -= d;
  }
}

// LDS byte offset of chunk c of row r (128-byte rows, XOR-swizzled chunks).
__device__ __forceinline__ int lds_off(int r, int c) { return r * kBKB + ((c ^ (r & 7)) << 4); }

// Sum of the K-split partials in split order (the same order on every run),
// then the fused epilogue. One lane per output quad (4 channels).
template <int ESZ>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const void* ws, int ksplit, int m, int cout, Epi e,
                                                            int out_kind, void* y) {
  typedef typename Mfma<ESZ>::acc_t acc_t;
  const int nq = cout / 4;
  const long total = (long)m * nq;
  const acc_t* w = reinterpret_cast<const acc_t*>(ws);
  const OutRef o = out_ref(y, m, cout, ESZ == 2 ? 2 : (out_kind == OUT_I32 ? 4 : 1), e.res);
  with_epilogue<ESZ>(out_kind, e.act, [&](auto oc, auto ac) {
    constexpr int OUT = decltype(oc)::value, ACT = decltype(ac)::value;
    for (long q = (long)blockIdx.x * blockDim.x + threadIdx.x; q < total; q += (long)gridDim.x * blockDim.x) {
      // every split's quad is loaded before the first add (one memory
      // latency, not ksplit of them); the adds keep split order
      acc_t part[kMaxSplits];
#pragma unroll
      for (int s = 0; s < kMaxSplits; ++s)
        if (s < ksplit) part[s] = w[(size_t)s * total + q];
      acc_t acc = part[0];
#pragma unroll
      for (int s = 1; s < kMaxSplits; ++s)
        if (s < ksplit) acc += part[s];
      const int px = (int)(q / nq);
      const int co = (int)(q - (long)px * nq) * 4;
      store_quad_t<ESZ, OUT, ACT>(acc, load_quad_consts_t<ESZ>(e, co, cout), co, px, o);
    }
  });
}

}  // namespace

// The K-split partial sums [ksplit][m][cout] of plan p summed in split order,
// then the fused epilogue into y.
inline hipError_t launch_splitk_reduce(const conv_plan* p, const Epi& e, void* y, hipStream_t s) {
  if (p->ksplit > kMaxSplits) return hipErrorInvalidValue;  // plan_split_k never makes more
  const long quads = (long)p->g.m * (p->g.cout / 4);
  const int blocks = (int)std::min<long>((quads + 255) / 256, 256L * 8);
  if (p->in_esz == 2)
    hipLaunchKernelGGL(splitk_reduce_kernel<2>, dim3(blocks), dim3(256), 0, s, p->ws, p->ksplit, p->g.m,
                       p->g.cout, e, p->out_kind, y);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<1>, dim3(blocks), dim3(256), 0, s, p->ws, p->ksplit, p->g.m,
                       p->g.cout, e, p->out_kind, y);
  return hipGetLastError();
}

}  // namespace convnhwc
