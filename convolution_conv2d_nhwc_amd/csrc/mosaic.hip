// mosaic.hip -- four-tile mosaic packing (YOLOv4 on Tenstorrent Wormhole,
// section 4, the m640 layout: four 320x320 photos placed 2x2 in one 640x640
// canvas, A top-left, B top-right, C bottom-left, D bottom-right), with the
// conversion to the network's input type fused into the copy.
//
// Every canvas row is two contiguous half-rows, each a copy of one tile row.
// When no channel padding is requested (c_pad == c) and a half-row holds a
// multiple of 8 values, each lane converts 8 consecutive values with 16- and
// 32-byte vector accesses. A bf16 canvas padded to 8 channels (16 bytes per
// pixel, the input of the window stem kernel) gets one 16-byte store per
// pixel; otherwise one lane writes one canvas pixel value by value.
#include "device_common.h"
#include "plan.h"

namespace convnhwc {
namespace {

struct MosArgs {
  const char* tiles;
  char* canvas;
  int in_f32, out_f32;
  int m, th, tw, c, c_pad;
  long total;
};

__device__ __forceinline__ float load_in(const char* base, long idx, int in_f32) {
  if (in_f32) return reinterpret_cast<const float*>(base)[idx];
  return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
}

__device__ __forceinline__ void store_out(char* base, long idx, float v, int out_f32) {
  if (out_f32)
    reinterpret_cast<float*>(base)[idx] = v;
  else
    reinterpret_cast<uint16_t*>(base)[idx] = f32_to_bf16_bits(v);
}

// One lane per canvas pixel (any c, c_pad).
__global__ __launch_bounds__(256) void mosaic_pixel_kernel(MosArgs a) {
  const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= a.total) return;
  const int cw = 2 * a.tw, chh = 2 * a.th;
  const int x = (int)(t % cw);
  long r = t / cw;
  const int y = (int)(r % chh);
  const int i = (int)(r / chh);
  const int quad = 2 * (y >= a.th) + (x >= a.tw);
  const int ty = y >= a.th ? y - a.th : y;
  const int tx = x >= a.tw ? x - a.tw : x;
  const long src = (((long)(4 * i + quad) * a.th + ty) * a.tw + tx) * a.c;
  const long dst = t * a.c_pad;
  for (int ch = 0; ch < a.c_pad; ++ch)
    store_out(a.canvas, dst + ch, ch < a.c ? load_in(a.tiles, src + ch, a.in_f32) : 0.0f, a.out_f32);
}

// One lane per 8 consecutive values of a half-row (c_pad == c, tw*c % 8 == 0).
__global__ __launch_bounds__(256) void mosaic_vec8_kernel(MosArgs a) {
  const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= a.total) return;
  const int hrow = a.tw * a.c;  // values per half-row
  const int per = hrow / 8;     // lanes per half-row
  const int v8 = (int)(t % per);
  long r = t / per;
  const int half = (int)(r % 2);
  r /= 2;
  const int y = (int)(r % (2 * a.th));
  const int i = (int)(r / (2 * a.th));
  const int quad = 2 * (y >= a.th) + half;
  const int ty = y >= a.th ? y - a.th : y;
  const long src = ((long)(4 * i + quad) * a.th + ty) * hrow + v8 * 8;
  const long dst = ((long)(i * 2 * a.th + y) * 2 + half) * hrow + v8 * 8;
  float v[8];
  if (a.in_f32) {
    const f32x4* p = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(a.tiles) + src);
    const f32x4 lo = p[0], hi = p[1];
    for (int e = 0; e < 4; ++e) {
      v[e] = lo[e];
      v[4 + e] = hi[e];
    }
  } else {
    const i32x4 q = *reinterpret_cast<const i32x4*>(reinterpret_cast<const uint16_t*>(a.tiles) + src);
    for (int e = 0; e < 8; ++e) {
      const uint32_t wd = (uint32_t)q[e >> 1];
      v[e] = bf16_bits_to_f32((e & 1) ? (wd >> 16) : (wd & 0xffffu));
    }
  }
  if (a.out_f32) {
    f32x4* p = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.canvas) + dst);
    p[0] = f32x4{v[0], v[1], v[2], v[3]};
    p[1] = f32x4{v[4], v[5], v[6], v[7]};
  } else {
    uint32_t wd[4];
    for (int q = 0; q < 4; ++q)
      wd[q] = bf16x2_bits(v[2 * q], v[2 * q + 1]);
    *reinterpret_cast<i32x4*>(reinterpret_cast<uint16_t*>(a.canvas) + dst) =
        i32x4{(int)wd[0], (int)wd[1], (int)wd[2], (int)wd[3]};
  }
}

// One lane per canvas pixel of a bf16 canvas with c_pad == 8 (c <= 8): the
// pixel's c values, zero-filled to 8, as one 16-byte store.
__global__ __launch_bounds__(256) void mosaic_px16_kernel(MosArgs a) {
  const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= a.total) return;
  const int cw = 2 * a.tw, chh = 2 * a.th;
  const int x = (int)(t % cw);
  long r = t / cw;
  const int y = (int)(r % chh);
  const int i = (int)(r / chh);
  const int quad = 2 * (y >= a.th) + (x >= a.tw);
  const int ty = y >= a.th ? y - a.th : y;
  const int tx = x >= a.tw ? x - a.tw : x;
  const long src = (((long)(4 * i + quad) * a.th + ty) * a.tw + tx) * a.c;
  uint32_t wd[4] = {0, 0, 0, 0};
  for (int ch = 0; ch < a.c; ++ch)
    wd[ch >> 1] |= (uint32_t)f32_to_bf16_bits(load_in(a.tiles, src + ch, a.in_f32)) << (16 * (ch & 1));
  *reinterpret_cast<i32x4*>(a.canvas + t * 16) = i32x4{(int)wd[0], (int)wd[1], (int)wd[2], (int)wd[3]};
}

}  // namespace

hipError_t launch_mosaic(const void* tiles, int in_f32, void* canvas, int out_f32, int m, int th,
                         int tw, int c, int c_pad, hipStream_t s) {
  MosArgs a;
  a.tiles = static_cast<const char*>(tiles);
  a.canvas = static_cast<char*>(canvas);
  a.in_f32 = in_f32;
  a.out_f32 = out_f32;
  a.m = m;
  a.th = th;
  a.tw = tw;
  a.c = c;
  a.c_pad = c_pad;
  if (!out_f32 && c_pad == 8) {
    a.total = (long)m * 2 * th * 2 * tw;
    const long blocks = (a.total + 255) / 256;
    hipLaunchKernelGGL(mosaic_px16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  } else if (c_pad == c && ((long)tw * c) % 8 == 0) {
    a.total = (long)m * 2 * th * 2 * ((long)tw * c / 8);
    const long blocks = (a.total + 255) / 256;
    hipLaunchKernelGGL(mosaic_vec8_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  } else {
    a.total = (long)m * 2 * th * 2 * tw;
    const long blocks = (a.total + 255) / 256;
    hipLaunchKernelGGL(mosaic_pixel_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace convnhwc
