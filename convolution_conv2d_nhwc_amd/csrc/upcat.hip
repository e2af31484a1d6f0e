// upcat.hip -- nearest-neighbour 2x upsampling and channel concatenation of
// two maps, written straight into the NHWC input of the next convolution
// (zerolat.eu YOLOv4 report, section 9 "Four custom Tensix kernels", K4: the neck gathers
// two feature maps, repeats one 2x in rows and columns and joins them along
// channels in the layout the following convolution reads).
//
// A pure copy, bound by HBM: each lane moves 16-byte chunks of output
// pixels. Consecutive lanes take consecutive chunks of one output row, so
// every store is part of a contiguous run and the loads of one source pixel
// are contiguous too; the four output pixels an upsampled source pixel feeds
// read it from L2 after the first. Grid: x over the chunks of an output row,
// y over the rows of the batch.
#include "device_common.h"
#include "plan.h"

namespace convnhwc {
namespace {

struct UpcatArgs {
  const char* s0;
  const char* s1;
  char* y;
  int k0, kt;          // 16-byte chunks per pixel: of source 0, of the output
  int up0, up1;        // source s is repeated 2x when up_s = 1
  int ho, wo;          // output size
  int chunks_row;      // wo * kt
  float inv_kt;        // 1 / kt
  int s0_bytes, s1_bytes, y_bytes;
};

// Each lane moves CPT chunks of the row, 256 chunks apart: all loads are
// issued before the first store, so CPT loads per lane are in flight.
#ifndef UPCAT_ST_AUX
#define UPCAT_ST_AUX 2  // non-temporal output stores
#endif
#ifndef UPCAT_CPT
#define UPCAT_CPT 2
#endif
constexpr int CPT = UPCAT_CPT;

__global__ __launch_bounds__(256) void upcat_kernel(UpcatArgs a) {
  const int row = blockIdx.y;  // n * ho + i
  const int n = row / a.ho;
  const int i = row - n * a.ho;
  const __amdgpu_buffer_rsrc_t r0 = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(a.s0), 0, a.s0_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t r1 = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(a.s1), 0, a.s1_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(a.y, 0, a.y_bytes, 0x00020000);
  const uint32_t ybase = (uint32_t)row * (uint32_t)a.chunks_row * 16u;
  i32x4 v[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int t = (blockIdx.x * CPT + c) * 256 + threadIdx.x;
    // output pixel j of the row and chunk k of the pixel (t + 1/2 keeps the
    // quotient at least 1/(2 kt) away from an integer; t < 2^22)
    const int j = (int)(((float)t + 0.5f) * a.inv_kt);
    const int k = t - j * a.kt;
    const bool first = k < a.k0;
    const int up = first ? a.up0 : a.up1;
    const int kc = first ? a.k0 : a.kt - a.k0;  // chunks per pixel of this source
    const int hs = a.ho >> up, ws = a.wo >> up;
    uint32_t src = (uint32_t)((((n * hs + (i >> up)) * ws + (j >> up)) * kc + (first ? k : k - a.k0)) * 16);
    if (t >= a.chunks_row) src = 0x80000000u;  // past the row: reads zero, the store below is dropped
    v[c] = __builtin_amdgcn_raw_buffer_load_b128(first ? r0 : r1, (int)src, 0, 0);
  }
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int t = (blockIdx.x * CPT + c) * 256 + threadIdx.x;
    const uint32_t dst = t < a.chunks_row ? ybase + (uint32_t)t * 16u : 0x80000000u;
    __builtin_amdgcn_raw_buffer_store_b128(v[c], ry, (int)dst, 0, UPCAT_ST_AUX);
  }
}

}  // namespace

hipError_t launch_upcat(const void* s0, int64_t c0_bytes, int up0, const void* s1, int64_t c1_bytes, int up1, void* y,
                        int64_t n, int64_t ho, int64_t wo, hipStream_t s) {
  UpcatArgs a;
  a.s0 = static_cast<const char*>(s0);
  a.s1 = static_cast<const char*>(s1);
  a.y = static_cast<char*>(y);
  a.k0 = (int)(c0_bytes / 16);
  a.kt = (int)((c0_bytes + c1_bytes) / 16);
  a.up0 = up0;
  a.up1 = up1;
  a.ho = (int)ho;
  a.wo = (int)wo;
  a.chunks_row = (int)(wo * a.kt);
  a.inv_kt = 1.0f / (float)a.kt;
  a.s0_bytes = (int)(n * (ho >> up0) * (wo >> up0) * c0_bytes);
  a.s1_bytes = (int)(n * (ho >> up1) * (wo >> up1) * c1_bytes);
  a.y_bytes = (int)(n * ho * wo * (c0_bytes + c1_bytes));
  const dim3 grid((unsigned)((a.chunks_row + 256 * CPT - 1) / (256 * CPT)), (unsigned)(n * ho));
  hipLaunchKernelGGL(upcat_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace convnhwc
