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
  int x_bytes;
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
// ACT and OUT (the int8 output kind) are compile-time: the epilogue runs once
// per output vector and a per-element branch on them would cost more than it.
template <typename T, int VE, int PW, int ACT, int OUT>
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
      if constexpr (OUT == OUT_I32) {
        int32_t* yp = reinterpret_cast<int32_t*>(a.y) + off;
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          int v = rv[e];
          if constexpr (ACT == ACT_RELU) v = v > 0 ? v : 0;
          yp[e] = v;
        }
      } else {
        int8_t* yp = reinterpret_cast<int8_t*>(a.y) + off;
        if constexpr (VE == 16) {
          uint32_t wd[4] = {0, 0, 0, 0};
#pragma unroll
          for (int e = 0; e < VE; ++e)
            wd[e >> 2] |= ((uint32_t)requant_i8_t<ACT>(rv[e], a.e.scale[c0 + e]) & 0xffu) << (8 * (e & 3));
          *reinterpret_cast<i32x4*>(yp) = i32x4{(int)wd[0], (int)wd[1], (int)wd[2], (int)wd[3]};
        } else {
#pragma unroll
          for (int e = 0; e < VE; ++e) yp[e] = (int8_t)requant_i8_t<ACT>(rv[e], a.e.scale[c0 + e]);
        }
      }
    } else {
      float v[VE];
#pragma unroll
      for (int e = 0; e < VE; ++e)
        v[e] = act_t<ACT>(acc[p][e] + (a.e.bias ? a.e.bias[c0 + e] : 0.0f));
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

// ---------------------------------------------------------------------------
// Stride-1 kernel with a sliding row window. A lane owns VE channels of PW
// adjacent output columns and walks TH output rows down the image: the three
// input rows it needs sit in registers already widened to the accumulator
// type, each new input row is loaded (PW+2 vectors) and widened once, and the
// next row's loads are in flight during the current row's multiply-adds, so
// memory latency overlaps arithmetic. The lane shapes
// (channels, columns, rows) were chosen by timing the depthwise probe on
// MI355X: bf16 4x2x8, int8 4x4x4, fp32 4x2x8. Loads are buffer loads: rows and
// columns outside the image read zero (the zero padding). Weights are widened
// once per lane.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dw_rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}

constexpr uint32_t kDwOOB = 0x80000000u;

// raw vector of VE elements of T
template <typename T, int VE>
struct RawVec {
  static constexpr int kBytes = VE * (int)sizeof(T);
  static constexpr int kWords = kBytes / 4;
  uint32_t w[kWords];
};

template <typename T, int VE>
__device__ __forceinline__ RawVec<T, VE> load_raw(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  RawVec<T, VE> v;
  if constexpr (RawVec<T, VE>::kBytes == 16) {
    const i32x4 q = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    v.w[0] = q[0];
    v.w[1] = q[1];
    v.w[2] = q[2];
    v.w[3] = q[3];
  } else if constexpr (RawVec<T, VE>::kBytes == 4) {
    v.w[0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
  } else {
    typedef int i32x2 __attribute__((ext_vector_type(2)));
    const i32x2 q = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
    v.w[0] = q[0];
    v.w[1] = q[1];
  }
  return v;
}

template <typename T>
__device__ __forceinline__ typename Elt<T>::acc_t widen_word(uint32_t wd, int e) {
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(float, wd);
  } else if constexpr (sizeof(T) == 2) {
    return bf16_bits_to_f32((e & 1) ? (wd >> 16) : (wd & 0xffffu));
  } else {
    return (int)(int8_t)(wd >> (8 * (e & 3)));
  }
}

template <typename T, int VE, int PW, int TH, int ACT, int OUT>
__global__ __launch_bounds__(256) void dw3x3_rows_kernel(DwArgs a) {
  typedef typename Elt<T>::acc_t acc_t;
  constexpr int ESZ = sizeof(T);
  constexpr int PER = 4 / ESZ;  // elements per 32-bit word
  constexpr int NC = PW + 2;    // input columns per row
  const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= a.total) return;
  const Geometry& g = a.g;
  const int cvi = (int)(t % a.cv);
  long r = t / a.cv;
  const int wgi = (int)(r % a.wgrp);
  r /= a.wgrp;
  const int nhb = (g.ho + TH - 1) / TH;
  const int hb = (int)(r % nhb);
  const int n = (int)(r / nhb);
  const int c0 = cvi * VE;
  const int wo0 = wgi * PW;
  const int ho0 = hb * TH;
  const __amdgpu_buffer_rsrc_t rx = dw_rsrc(a.x, a.x_bytes);

  acc_t wr[VE][9];
#pragma unroll
  for (int e = 0; e < VE; ++e)
#pragma unroll
    for (int q = 0; q < 9; ++q) wr[e][q] = Elt<T>::get1(a.w + ((size_t)(c0 + e) * 9 + q) * ESZ);

  // byte offsets of this lane's input columns within one input row
  const int rowbytes = g.w * g.c * ESZ;
  uint32_t coff[NC];
  bool cok[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int wi = wo0 - g.pw + j;
    cok[j] = (unsigned)wi < (unsigned)g.w;
    coff[j] = (uint32_t)((wi * g.c + c0) * ESZ);
  }
  auto fetch_row = [&](int hi, RawVec<T, VE> (&raw)[NC]) {
    const bool rok = (unsigned)hi < (unsigned)g.h;
    const uint32_t rbase = (uint32_t)((n * g.h + hi) * rowbytes);
#pragma unroll
    for (int j = 0; j < NC; ++j) raw[j] = load_raw<T, VE>(rx, (rok && cok[j]) ? rbase + coff[j] : kDwOOB);
  };
  auto widen_row = [&](const RawVec<T, VE> (&raw)[NC], acc_t (&row)[NC][VE]) {
#pragma unroll
    for (int j = 0; j < NC; ++j)
#pragma unroll
      for (int e = 0; e < VE; ++e) row[j][e] = widen_word<T>(raw[j].w[e / PER], e);
  };

  acc_t rows[3][NC][VE];
  RawVec<T, VE> nxt[NC];
  {
    const int hi0 = ho0 - g.ph;
    fetch_row(hi0, nxt);
    widen_row(nxt, rows[0]);
    fetch_row(hi0 + 1, nxt);
    widen_row(nxt, rows[1]);
    fetch_row(hi0 + 2, nxt);
  }

  float bsf[VE];
  int bsi[VE];
  float scl[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) {
    if constexpr (ESZ == 1) {
      bsi[e] = a.e.ibias ? a.e.ibias[c0 + e] : 0;
      scl[e] = a.e.scale ? a.e.scale[c0 + e] : 0.f;
    } else {
      bsf[e] = a.e.bias ? a.e.bias[c0 + e] : 0.f;
    }
  }

#pragma unroll
  for (int i = 0; i < TH; ++i) {
    const int ho = ho0 + i;
    if (ho >= g.ho) break;
    // the row loaded last becomes window row (i + 2) % 3, then the next
    // row's loads go out before this row's multiply-adds
    widen_row(nxt, rows[(i + 2) % 3]);
    if (i + 1 < TH) fetch_row(ho - g.ph + 3, nxt);
    acc_t acc[PW][VE];
#pragma unroll
    for (int p = 0; p < PW; ++p)
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[p][e] = 0;
#pragma unroll
    for (int kh = 0; kh < 3; ++kh)
#pragma unroll
      for (int kw = 0; kw < 3; ++kw)
#pragma unroll
        for (int p = 0; p < PW; ++p)
#pragma unroll
          for (int e = 0; e < VE; ++e) acc[p][e] += rows[(i + kh) % 3][p + kw][e] * wr[e][kh * 3 + kw];
    // fused epilogue, VE channels of PW pixels
#pragma unroll
    for (int p = 0; p < PW; ++p) {
      const int wo = wo0 + p;
      if (wo >= g.wo) break;
      const size_t off = ((size_t)(n * g.ho + ho) * g.wo + wo) * g.cout + c0;
      if constexpr (ESZ == 1) {
        if constexpr (OUT == OUT_I32) {
          int32_t* yp = reinterpret_cast<int32_t*>(a.y) + off;
#pragma unroll
          for (int e = 0; e < VE; ++e) {
            int v = acc[p][e] + bsi[e];
            if constexpr (ACT == ACT_RELU) v = v > 0 ? v : 0;
            yp[e] = v;
          }
        } else {
          uint32_t wd[VE / 4];
#pragma unroll
          for (int q = 0; q < VE / 4; ++q) wd[q] = 0;
#pragma unroll
          for (int e = 0; e < VE; ++e)
            wd[e >> 2] |= ((uint32_t)requant_i8_t<ACT>(acc[p][e] + bsi[e], scl[e]) & 0xffu) << (8 * (e & 3));
          if constexpr (VE == 4)
            *reinterpret_cast<uint32_t*>(reinterpret_cast<int8_t*>(a.y) + off) = wd[0];
          else if constexpr (VE == 8)
            *reinterpret_cast<uint2*>(reinterpret_cast<int8_t*>(a.y) + off) = uint2{wd[0], wd[1]};
          else
            *reinterpret_cast<i32x4*>(reinterpret_cast<int8_t*>(a.y) + off) =
                i32x4{(int)wd[0], (int)wd[1], (int)wd[2], (int)wd[3]};
        }
      } else {
        float v[VE];
#pragma unroll
        for (int e = 0; e < VE; ++e) v[e] = act_t<ACT>(acc[p][e] + bsf[e]);
        if constexpr (ESZ == 4) {
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.y) + off) = f32x4{v[0], v[1], v[2], v[3]};
        } else {
          uint32_t wd[VE / 2];
#pragma unroll
          for (int q = 0; q < VE / 2; ++q)
            wd[q] = (uint32_t)f32_to_bf16_bits(v[2 * q]) | ((uint32_t)f32_to_bf16_bits(v[2 * q + 1]) << 16);
          uint16_t* yp = reinterpret_cast<uint16_t*>(a.y) + off;
          if constexpr (VE == 8)
            *reinterpret_cast<i32x4*>(yp) = i32x4{(int)wd[0], (int)wd[1], (int)wd[2], (int)wd[3]};
          else
            *reinterpret_cast<uint2*>(yp) = uint2{wd[0], wd[1]};
        }
      }
    }
  }
}

// f(OUT, ACT) as compile-time constants for a layer's output kind and
// activation (the int32 checkpoint allows NONE and RELU only).
template <class F>
hipError_t with_act(int out_kind, int act, F&& f) {
  using std::integral_constant;
  if (out_kind == OUT_I32) {
    if (act == ACT_RELU) return f(integral_constant<int, OUT_I32>{}, integral_constant<int, ACT_RELU>{});
    return f(integral_constant<int, OUT_I32>{}, integral_constant<int, ACT_NONE>{});
  }
  switch (act) {
    case ACT_RELU: return f(integral_constant<int, OUT_I8>{}, integral_constant<int, ACT_RELU>{});
    case ACT_RELU6: return f(integral_constant<int, OUT_I8>{}, integral_constant<int, ACT_RELU6>{});
    case ACT_MISH: return f(integral_constant<int, OUT_I8>{}, integral_constant<int, ACT_MISH>{});
    default: return f(integral_constant<int, OUT_I8>{}, integral_constant<int, ACT_NONE>{});
  }
}

template <typename T, int VE, int PW, int TH>
hipError_t launch_rows_t(const DwArgs& base, hipStream_t s) {
  DwArgs a = base;
  a.cv = a.g.c / VE;
  a.wgrp = (a.g.wo + PW - 1) / PW;
  a.total = (long)a.g.n * ((a.g.ho + TH - 1) / TH) * a.wgrp * a.cv;
  const long blocks = (a.total + 255) / 256;
  return with_act(a.out_kind, a.e.act, [&](auto oc, auto ac) {
    hipLaunchKernelGGL((dw3x3_rows_kernel<T, VE, PW, TH, decltype(ac)::value, decltype(oc)::value>),
                       dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
  });
}

template <typename T, int VE, int PW>
hipError_t launch_dw_t(const DwArgs& base, hipStream_t s) {
  DwArgs a = base;
  a.cv = a.g.c / VE;
  a.wgrp = (a.g.wo + PW - 1) / PW;
  a.total = (long)a.g.n * a.g.ho * a.wgrp * a.cv;
  const long blocks = (a.total + 255) / 256;
  return with_act(a.out_kind, a.e.act, [&](auto oc, auto ac) {
    hipLaunchKernelGGL((dw3x3_kernel<T, VE, PW, decltype(ac)::value, decltype(oc)::value>), dim3((unsigned)blocks),
                       dim3(256), 0, s, a);
    return hipGetLastError();
  });
}

}  // namespace

// Lane shape of a depthwise plan: th > 0 selects the sliding-window kernel.
void dw_shape(const conv_plan* p, int* ve, int* pw, int* th) {
  const int c = p->g.c;
  const bool s1 = p->g.sh == 1 && p->g.sw == 1;
  const bool vec = p->loader == LOAD_VEC;
  *th = 0;
  if (s1 && c % 4 == 0) {
    *ve = 4;
    *pw = p->in_esz == 1 ? 4 : 2;
    *th = p->in_esz == 1 ? 4 : 8;
    return;
  }
  *ve = vec ? 16 / p->in_esz : 1;
  *pw = (p->in_esz == 1 && vec) ? 2 : 4;
}

hipError_t launch_dw(const conv_plan* p, const void* x, const void* w, const Epi& e, void* y,
                     hipStream_t s) {
  DwArgs a;
  a.x = static_cast<const char*>(x);
  a.w = static_cast<const char*>(w);
  a.y = y;
  a.e = e;
  a.g = p->g;
  a.out_kind = p->out_kind;
  a.x_bytes = (int)p->x_bytes;
  int ve, pw, th;
  dw_shape(p, &ve, &pw, &th);
  if (th) {
    switch (p->in_esz) {
      case 4: return launch_rows_t<float, 4, 2, 8>(a, s);
      case 2: return launch_rows_t<uint16_t, 4, 2, 8>(a, s);
      default: return launch_rows_t<int8_t, 4, 4, 4>(a, s);
    }
  }
  const bool vec = ve > 1;
  switch (p->in_esz) {
    case 4: return vec ? launch_dw_t<float, 4, 4>(a, s) : launch_dw_t<float, 1, 4>(a, s);
    case 2: return vec ? launch_dw_t<uint16_t, 8, 4>(a, s) : launch_dw_t<uint16_t, 1, 4>(a, s);
    default: return vec ? launch_dw_t<int8_t, 16, 2>(a, s) : launch_dw_t<int8_t, 1, 4>(a, s);
  }
}

}  // namespace convnhwc
