// dwconv.hip -- depthwise 3x3 convolution (groups == Cin == Cout), NHWC.
//
// A depthwise layer has no reduction across channels, so there is nothing
// for a matrix core to do: per output element it is 9 multiply-adds against
// 2 bytes (bf16) of output, i.e. bandwidth-bound (nanoinfer README: the
// depthwise layer is almost entirely epilogue and memory; NHWC is the layout
// where one vector load covers many channels of one pixel). The kernel
// therefore runs on the vector ALUs:
//   * a lane owns one 16-byte channel vector (8 bf16, 16 int8, 4 fp32) of
//     PW horizontally adjacent output pixels, so every global load and store
//     is a full 16-byte vector and a wave covers 64 contiguous vectors;
//   * consecutive lanes take consecutive channel vectors, then consecutive
//     pixel groups: a wave's loads of one tap are contiguous in memory and
//     the 3x3 halo re-reads of neighbouring lanes hit in L1/L2;
//   * the PW outputs of a lane share their input rows: for stride 1 a lane
//     loads PW+2 columns per row instead of 3*PW;
//   * the 9 taps of the lane's channels are 9*VE contiguous weights
//     ([C][3][3] layout), read as nine 16-byte loads;
//   * accumulation is fp32 (fp32/bf16) or exact int32 (int8), then the same
//     fused epilogue as the dense kernels.
#include "device_common.h"
#include "plan.h"

namespace convnhwc {
namespace {

struct DwArgs {
  const char* x;
  const char* w;
  void* y;
  Epi e;
  Geometry g;
  int out_kind;
  int cv;      // channel vectors per pixel
  int wgrp;    // pixel groups per output row
  long total;  // threads doing work
};

// Element loads/stores for the three input types, widened to the
// accumulator type.
template <typename T>
struct Elt;
template <>
struct Elt<float> {
  typedef float acc_t;
  static __device__ __forceinline__ acc_t get(const i32x4& v, int e) {
    // copy the element to a scalar first: bit_cast of an ext-vector
    // subscript would reinterpret the vector's first element instead
    const int bits = v[e];
    return __builtin_bit_cast(float, bits);
  }
  static __device__ __forceinline__ acc_t get1(const char* p) {
    return *reinterpret_cast<const float*>(p);
  }
};
template <>
struct Elt<uint16_t> {  // bf16 bits
  typedef float acc_t;
  static __device__ __forceinline__ acc_t get(const i32x4& v, int e) {
    const uint32_t wd = (uint32_t)v[e >> 1];
    return bf16_bits_to_f32((e & 1) ? (wd >> 16) : (wd & 0xffffu));
  }
  static __device__ __forceinline__ acc_t get1(const char* p) {
    return bf16_bits_to_f32(*reinterpret_cast<const uint16_t*>(p));
  }
};
template <>
struct Elt<int8_t> {
  typedef int acc_t;
  static __device__ __forceinline__ acc_t get(const i32x4& v, int e) {
    return (int)(int8_t)(((uint32_t)v[e >> 2]) >> (8 * (e & 3)));
  }
  static __device__ __forceinline__ acc_t get1(const char* p) {
    return *reinterpret_cast<const int8_t*>(p);
  }
};

// VE = channels per lane (16 bytes worth, or 1 for the scalar fallback).
template <typename T, int VE, int PW>
__global__ __launch_bounds__(256) void dw3x3_kernel(DwArgs a) {
  typedef typename Elt<T>::acc_t acc_t;
  constexpr int ESZ = sizeof(T);
  const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= a.total) return;
  const Geometry& g = a.g;
  const int cvi = (int)(t % a.cv);
  long r = t / a.cv;
  const int wgi = (int)(r % a.wgrp);
  r /= a.wgrp;
  const int ho = (int)(r % g.ho);
  const int n = (int)(r / g.ho);
  const int c0 = cvi * VE;
  const int wo0 = wgi * PW;

  // weights of channels c0..c0+VE-1: [VE][9] contiguous
  acc_t wr[VE][9];
  if constexpr (VE * ESZ == 16) {
    const char* wp = a.w + (size_t)c0 * 9 * ESZ;
#pragma unroll
    for (int q = 0; q < 9; ++q) {
      const i32x4 v = *reinterpret_cast<const i32x4*>(wp + 16 * q);
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        const int flat = q * VE + e;  // element index within [VE][9]
        wr[flat / 9][flat % 9] = Elt<T>::get(v, e);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < VE; ++e)
#pragma unroll
      for (int q = 0; q < 9; ++q) wr[e][q] = Elt<T>::get1(a.w + ((size_t)(c0 + e) * 9 + q) * ESZ);
  }

  acc_t acc[PW][VE];
#pragma unroll
  for (int p = 0; p < PW; ++p)
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[p][e] = 0;

  const int wi_first = wo0 * g.sw - g.pw;
#pragma unroll
  for (int kh = 0; kh < 3; ++kh) {
    const int hi = ho * g.sh - g.ph + kh;
    if ((unsigned)hi >= (unsigned)g.h) continue;
    const char* rowp = a.x + ((size_t)(n * g.h + hi) * g.w) * g.c * ESZ;
    if (g.sw == 1) {
      // PW + 2 input columns feed PW outputs
#pragma unroll
      for (int col = 0; col < PW + 2; ++col) {
        const int wi = wi_first + col;
        if ((unsigned)wi >= (unsigned)g.w) continue;
        const char* px = rowp + ((size_t)wi * g.c + c0) * ESZ;
        acc_t xv[VE];
        if constexpr (VE * ESZ == 16) {
          const i32x4 v = *reinterpret_cast<const i32x4*>(px);
#pragma unroll
          for (int e = 0; e < VE; ++e) xv[e] = Elt<T>::get(v, e);
        } else {
#pragma unroll
          for (int e = 0; e < VE; ++e) xv[e] = Elt<T>::get1(px + e * ESZ);
        }
#pragma unroll
        for (int p = 0; p < PW; ++p) {
          const int kw = col - p;
          if (kw < 0 || kw > 2) continue;
#pragma unroll
          for (int e = 0; e < VE; ++e) acc[p][e] += xv[e] * wr[e][kh * 3 + kw];
        }
      }
    } else {
#pragma unroll
      for (int p = 0; p < PW; ++p) {
#pragma unroll
        for (int kw = 0; kw < 3; ++kw) {
          const int wi = wi_first + p * g.sw + kw;
          if ((unsigned)wi >= (unsigned)g.w) continue;
          const char* px = rowp + ((size_t)wi * g.c + c0) * ESZ;
          if constexpr (VE * ESZ == 16) {
            const i32x4 v = *reinterpret_cast<const i32x4*>(px);
#pragma unroll
            for (int e = 0; e < VE; ++e) acc[p][e] += Elt<T>::get(v, e) * wr[e][kh * 3 + kw];
          } else {
#pragma unroll
            for (int e = 0; e < VE; ++e) acc[p][e] += Elt<T>::get1(px + e * ESZ) * wr[e][kh * 3 + kw];
          }
        }
      }
    }
  }

  // fused epilogue
#pragma unroll
  for (int p = 0; p < PW; ++p) {
    const int wo = wo0 + p;
    if (wo >= g.wo) break;
    const size_t off = ((size_t)(n * g.ho + ho) * g.wo + wo) * g.cout + c0;
    if constexpr (sizeof(T) == 1) {
      int rv[VE];
#pragma unroll
      for (int e = 0; e < VE; ++e) rv[e] = acc[p][e] + (a.e.ibias ? a.e.ibias[c0 + e] : 0);
      if (a.out_kind == OUT_I32) {
        int32_t* yp = reinterpret_cast<int32_t*>(a.y) + off;
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          int v = rv[e];
          if (a.e.act == ACT_RELU) v = v > 0 ? v : 0;
          yp[e] = v;
        }
      } else {
        int8_t* yp = reinterpret_cast<int8_t*>(a.y) + off;
        if constexpr (VE == 16) {
          uint32_t wd[4] = {0, 0, 0, 0};
#pragma unroll
          for (int e = 0; e < VE; ++e)
            wd[e >> 2] |= ((uint32_t)requant_i8(rv[e], a.e.scale[c0 + e], a.e.act) & 0xffu) << (8 * (e & 3));
          *reinterpret_cast<i32x4*>(yp) = i32x4{(int)wd[0], (int)wd[1], (int)wd[2], (int)wd[3]};
        } else {
#pragma unroll
          for (int e = 0; e < VE; ++e) yp[e] = (int8_t)requant_i8(rv[e], a.e.scale[c0 + e], a.e.act);
        }
      }
    } else {
      float v[VE];
#pragma unroll
      for (int e = 0; e < VE; ++e)
        v[e] = apply_act(acc[p][e] + (a.e.bias ? a.e.bias[c0 + e] : 0.0f), a.e.act);
      if constexpr (sizeof(T) == 4) {
        float* yp = reinterpret_cast<float*>(a.y) + off;
        if constexpr (VE == 4) {
          *reinterpret_cast<f32x4*>(yp) = f32x4{v[0], v[1], v[2], v[3]};
        } else {
#pragma unroll
          for (int e = 0; e < VE; ++e) yp[e] = v[e];
        }
      } else {
        uint16_t* yp = reinterpret_cast<uint16_t*>(a.y) + off;
        if constexpr (VE == 8) {
          uint32_t wd[4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            wd[q] = (uint32_t)f32_to_bf16_bits(v[2 * q]) | ((uint32_t)f32_to_bf16_bits(v[2 * q + 1]) << 16);
          *reinterpret_cast<i32x4*>(yp) = i32x4{(int)wd[0], (int)wd[1], (int)wd[2], (int)wd[3]};
        } else {
#pragma unroll
          for (int e = 0; e < VE; ++e) yp[e] = f32_to_bf16_bits(v[e]);
        }
      }
    }
  }
}

template <typename T, int VE, int PW>
hipError_t launch_dw_t(const DwArgs& base, hipStream_t s) {
  DwArgs a = base;
  a.cv = a.g.c / VE;
  a.wgrp = (a.g.wo + PW - 1) / PW;
  a.total = (long)a.g.n * a.g.ho * a.wgrp * a.cv;
  const long blocks = (a.total + 255) / 256;
  hipLaunchKernelGGL((dw3x3_kernel<T, VE, PW>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dw(const conv_plan* p, const void* x, const void* w, const Epi& e, void* y,
                     hipStream_t s) {
  DwArgs a;
  a.x = static_cast<const char*>(x);
  a.w = static_cast<const char*>(w);
  a.y = y;
  a.e = e;
  a.g = p->g;
  a.out_kind = p->out_kind;
  const bool vec = p->loader == LOAD_VEC;
  switch (p->in_esz) {
    case 4: return vec ? launch_dw_t<float, 4, 4>(a, s) : launch_dw_t<float, 1, 4>(a, s);
    case 2: return vec ? launch_dw_t<uint16_t, 8, 4>(a, s) : launch_dw_t<uint16_t, 1, 4>(a, s);
    default: return vec ? launch_dw_t<int8_t, 16, 2>(a, s) : launch_dw_t<int8_t, 1, 4>(a, s);
  }
}

}  // namespace convnhwc
