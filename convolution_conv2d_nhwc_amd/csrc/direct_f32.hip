// direct_f32.hip -- true-fp32 dense convolution on the vector ALUs.
//
// fp32 layers are computed with fp32 fused multiply-adds and an fp32
// accumulator; no reduced-precision matrix mode is involved (the nanoinfer
// README reports a vendor library silently switching fp32 convolution to a
// 10-bit-mantissa tensor-core mode, 7.76e-3 relative error; this path cannot
// do that). The fp32 workload (a 28x28x1 -> 8 channel MNIST layer) is far
// below any throughput roof, so the kernel is a plain direct convolution:
// one lane per (output pixel, group of 4 output channels), the input value of
// a tap is loaded once and reused for the 4 channels; weights are read
// through the cache.
#include "device_common.h"
#include "plan.h"

namespace convnhwc {
namespace {

struct F32Args {
  const float* x;
  const float* w;
  float* y;
  Epi e;
  Geometry g;
  int cog;     // groups of 4 output channels
  long total;  // m * cog
};

__global__ __launch_bounds__(256) void conv_f32_kernel(F32Args a) {
  const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= a.total) return;
  const Geometry& g = a.g;
  const int cg = (int)(t % a.cog);
  const int px = (int)(t / a.cog);
  const int hw = g.ho * g.wo;
  const int n = px / hw;
  const int rem = px - n * hw;
  const int ho = rem / g.wo;
  const int wo = rem - ho * g.wo;
  const int co0 = cg * 4;
  const int nco = min(4, g.cout - co0);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int kh = 0; kh < g.kh; ++kh) {
    const int hi = ho * g.sh - g.ph + kh;
    if ((unsigned)hi >= (unsigned)g.h) continue;
    for (int kw = 0; kw < g.kw; ++kw) {
      const int wi = wo * g.sw - g.pw + kw;
      if ((unsigned)wi >= (unsigned)g.w) continue;
      const float* xp = a.x + ((size_t)(n * g.h + hi) * g.w + wi) * g.c;
      const size_t wtap = (size_t)(kh * g.kw + kw) * g.c;
      for (int ci = 0; ci < g.c; ++ci) {
        const float xv = xp[ci];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (r < nco) acc[r] = __builtin_fmaf(xv, a.w[(size_t)(co0 + r) * g.k + wtap + ci], acc[r]);
      }
    }
  }
  float* yp = a.y + (size_t)px * g.cout + co0;
  const float* rp = a.e.res ? static_cast<const float*>(a.e.res) + (size_t)px * g.cout + co0 : nullptr;
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (r < nco) yp[r] = apply_act(acc[r] + (a.e.bias ? a.e.bias[co0 + r] : 0.0f), a.e.act) + (rp ? rp[r] : 0.0f);
}

}  // namespace

hipError_t launch_f32(const conv_plan* p, const void* x, const void* w, const Epi& e, void* y,
                      hipStream_t s) {
  F32Args a;
  a.x = static_cast<const float*>(x);
  a.w = static_cast<const float*>(w);
  a.y = static_cast<float*>(y);
  a.e = e;
  a.g = p->g;
  a.cog = (p->g.cout + 3) / 4;
  a.total = (long)p->g.m * a.cog;
  const long blocks = (a.total + 255) / 256;
  hipLaunchKernelGGL(conv_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace convnhwc
