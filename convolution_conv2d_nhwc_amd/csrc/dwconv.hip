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

// Lane shape of the row-window kernels (timed on the depthwise probe on
// MI355X): input rows in flight per lane, bf16 output columns per lane, and
// the lane count (per CU) below which a lane walks fewer rows.
#ifndef DW_PF
#define DW_PF 2
#endif
#ifndef DW_BF16_PW
#define DW_BF16_PW 4
#endif
// Cache policy of the row-window kernels' output stores: non-temporal (the
// output streams out; measured on the N=16 probe: 4 % faster for bf16,
// 10 % for int8). A chained network that wants the next layer to find its
// input in the caches can build with 0.
#ifndef DW_ST_AUX
#define DW_ST_AUX 2
#endif
#ifndef DW_MIN_LANES_PER_CU
#define DW_MIN_LANES_PER_CU 256
#endif

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
  int y_bytes;
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

// int8 output of one element, with the residual (an int8 tensor of y's shape,
// element idx) added after the activation when res is not null; the low
// byte of the result is the output.
template <int ACT>
__device__ __forceinline__ int dw_q8(int r, float s, const void* res, size_t idx) {
  if (res) return requant_i8_res_t<ACT>(r, s, static_cast<const int8_t*>(res)[idx]);
  return (int)requant_i8_word_t<ACT>(r, s);
}

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
            wd[e >> 2] |= ((uint32_t)dw_q8<ACT>(rv[e], a.e.scale[c0 + e], a.e.res, off + e) & 0xffu) << (8 * (e & 3));
          *reinterpret_cast<i32x4*>(yp) = i32x4{(int)wd[0], (int)wd[1], (int)wd[2], (int)wd[3]};
        } else {
#pragma unroll
          for (int e = 0; e < VE; ++e) yp[e] = (int8_t)dw_q8<ACT>(rv[e], a.e.scale[c0 + e], a.e.res, off + e);
        }
      }
    } else {
      float v[VE];
#pragma unroll
      for (int e = 0; e < VE; ++e)
        v[e] = (sizeof(T) == 4 ? act_t<ACT>(acc[p][e] + (a.e.bias ? a.e.bias[c0 + e] : 0.0f))
                               : act_t<ACT>(acc[p][e] + (a.e.bias ? a.e.bias[c0 + e] : 0.0f)));
      if (a.e.res) {
#pragma unroll
        for (int e = 0; e < VE; ++e) v[e] += Elt<T>::get1(static_cast<const char*>(a.e.res) + (off + e) * sizeof(T));
      }
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
            wd[q] = bf16x2_bits(v[2 * q], v[2 * q + 1]);
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
// memory latency overlaps arithmetic. Loads and stores are buffer accesses
// with 32-bit offsets: rows and columns outside the image read zero (the
// zero padding) and stores past the last column are dropped. Weights are
// widened once per lane and the accumulators start at the bias.
//
// Per output element the work is 9 multiply-adds, the activation and the
// conversion, against 2 (bf16) or 1 (int8) bytes of HBM traffic each way, so
// on MI355X these kernels are bounded by vector-ALU issue about as much as by
// HBM (Mish alone is two transcendental and seven plain operations): the
// kernels therefore minimise operations per output, not only bytes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dw_rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}

constexpr uint32_t kDwOOB = 0x80000000u;
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Buffer offsets as a row part plus a column part, each 2^31 or more when its
// row or column lies outside the image (or past the output's last column).
// Their saturating sum is then out of range whenever either part is, and the
// exact offset otherwise (every valid offset is below 2^31): one instruction
// per access instead of a select.
__device__ __forceinline__ uint32_t dw_add_sat(uint32_t a, uint32_t b) { return __builtin_elementwise_add_sat(a, b); }
__device__ __forceinline__ uint32_t dw_col_off(int wi, const Geometry& g, int cbyte0, int esz) {
  return (unsigned)wi < (unsigned)g.w ? (uint32_t)(wi * g.c * esz + cbyte0) : kDwOOB;
}
__device__ __forceinline__ uint32_t dw_row_off(int hi, int n, const Geometry& g, int rowbytes) {
  return (unsigned)hi < (unsigned)g.h ? (uint32_t)((n * g.h + hi) * rowbytes) : kDwOOB;
}

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


// Lane decomposition shared by the row-window kernels: channel vector
// fastest, then the group of PW columns, then the block of TH rows, then the
// image.
struct DwLane {
  int c0, wo0, ho0, n;
};
// 32-bit arithmetic: the lane count is below the output's element count,
// itself below 2^31.
template <int VE, int PW, int TH>
__device__ __forceinline__ DwLane dw_lane(const DwArgs& a, uint32_t t) {
  const Geometry& g = a.g;
  DwLane l;
  const uint32_t cv = (uint32_t)a.cv, wgrp = (uint32_t)a.wgrp, nhb = (uint32_t)((g.ho + TH - 1) / TH);
  uint32_t r = t / cv;
  l.c0 = (int)(t - r * cv) * VE;
  uint32_t r2 = r / wgrp;
  l.wo0 = (int)(r - r2 * wgrp) * PW;
  r = r2 / nhb;
  l.ho0 = (int)(r2 - r * nhb) * TH;
  l.n = (int)r;
  return l;
}

template <typename T, int VE, int PW, int TH, int ACT, int OUT, int PF>
__global__ __launch_bounds__(256) void dw3x3_rows_kernel(DwArgs a) {
  typedef typename Elt<T>::acc_t acc_t;
  constexpr int ESZ = sizeof(T);
  constexpr int PER = 4 / ESZ;  // elements per 32-bit word
  constexpr int NC = PW + 2;    // input columns per row
  static_assert(ESZ != 1, "int8 layers run dw3x3_i8_kernel");
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  if (t >= (uint32_t)a.total) return;
  const Geometry& g = a.g;
  const DwLane l = dw_lane<VE, PW, TH>(a, t);
  const int c0 = l.c0, wo0 = l.wo0, ho0 = l.ho0, n = l.n;
  const __amdgpu_buffer_rsrc_t rx = dw_rsrc(a.x, a.x_bytes);
  const __amdgpu_buffer_rsrc_t ry = dw_rsrc(a.y, a.y_bytes);
  const bool has_res = a.e.res != nullptr;  // residual of y's type and shape, added after the activation
  const __amdgpu_buffer_rsrc_t rr = dw_rsrc(a.e.res, has_res ? a.y_bytes : 0);

  // the 9 * VE weights of this lane's channels are contiguous ([VE][3][3])
  // and 4-byte aligned (VE * 9 * ESZ is a multiple of 4): whole-word loads
  static_assert(VE * 9 * ESZ % 4 == 0, "weight block of whole words");
  constexpr int WW = VE * 9 * ESZ / 4;
  uint32_t wraw[WW];
  const uint32_t* wp = reinterpret_cast<const uint32_t*>(a.w + (size_t)c0 * 9 * ESZ);
#pragma unroll
  for (int q = 0; q < WW; ++q) wraw[q] = wp[q];
  acc_t wr[VE][9];
#pragma unroll
  for (int e = 0; e < VE; ++e)
#pragma unroll
    for (int q = 0; q < 9; ++q) wr[e][q] = widen_word<T>(wraw[(e * 9 + q) / PER], e * 9 + q);

  // byte offsets of this lane's input columns within one input row
  const int rowbytes = g.w * g.c * ESZ;
  uint32_t coff[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) coff[j] = dw_col_off(wo0 - g.pw + j, g, c0 * ESZ, ESZ);
  auto fetch_row = [&](int hi, RawVec<T, VE> (&raw)[NC]) {
    const uint32_t rb = dw_row_off(hi, n, g, rowbytes);
#pragma unroll
    for (int j = 0; j < NC; ++j) raw[j] = load_raw<T, VE>(rx, dw_add_sat(rb, coff[j]));
  };
  auto widen_row = [&](const RawVec<T, VE> (&raw)[NC], acc_t (&row)[NC][VE]) {
#pragma unroll
    for (int j = 0; j < NC; ++j)
#pragma unroll
      for (int e = 0; e < VE; ++e) row[j][e] = widen_word<T>(raw[j].w[e / PER], e);
  };

  // window rows in registers, widened; the next PF input rows in flight
  acc_t rows[3][NC][VE];
  RawVec<T, VE> nxt[PF][NC];
  {
    const int hi0 = ho0 - g.ph;
    fetch_row(hi0, nxt[0]);
    widen_row(nxt[0], rows[0]);
    fetch_row(hi0 + 1, nxt[0]);
    widen_row(nxt[0], rows[1]);
#pragma unroll
    for (int f = 0; f < PF && f < TH; ++f) fetch_row(hi0 + 2 + f, nxt[f]);
  }

  acc_t bias[VE];
  float scl[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) {
    if constexpr (ESZ == 1) {
      bias[e] = a.e.ibias ? a.e.ibias[c0 + e] : 0;
      scl[e] = OUT == OUT_I8 ? a.e.scale[c0 + e] : 0.f;
    } else {
      bias[e] = a.e.bias ? a.e.bias[c0 + e] : 0.f;
    }
  }
  // byte offset of (ho0, wo0, c0) in y; one row further is wo * cout
  const int out_esz = ESZ == 1 ? (OUT == OUT_I32 ? 4 : 1) : ESZ;
  uint32_t yoff = (uint32_t)((((n * g.ho + ho0) * g.wo + wo0) * g.cout + c0) * out_esz);
  const uint32_t yrow = (uint32_t)(g.wo * g.cout * out_esz);
  uint32_t poff[PW];  // output column p, or out of range past the last column
#pragma unroll
  for (int p = 0; p < PW; ++p) poff[p] = wo0 + p < g.wo ? (uint32_t)(p * g.cout * out_esz) : kDwOOB;

#pragma unroll
  for (int i = 0; i < TH; ++i) {
    const int ho = ho0 + i;
    if (ho >= g.ho) break;
    // input row ho - ph + 2 becomes window row (i + 2) % 3, then the loads
    // of the row PF further go out before this row's multiply-adds
    widen_row(nxt[i % PF], rows[(i + 2) % 3]);
    if (i + PF < TH) fetch_row(ho - g.ph + 2 + PF, nxt[i % PF]);
    acc_t acc[PW][VE];
#pragma unroll
    for (int p = 0; p < PW; ++p)
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[p][e] = bias[e];
#pragma unroll
    for (int kh = 0; kh < 3; ++kh)
#pragma unroll
      for (int kw = 0; kw < 3; ++kw)
#pragma unroll
        for (int p = 0; p < PW; ++p)
#pragma unroll
          for (int e = 0; e < VE; ++e) acc[p][e] += rows[(i + kh) % 3][p + kw][e] * wr[e][kh * 3 + kw];
    // fused epilogue, VE channels of PW pixels; columns past the edge drop
#pragma unroll
    for (int p = 0; p < PW; ++p) {
      const uint32_t off = dw_add_sat(yoff, poff[p]);
      if constexpr (ESZ == 4) {
        float v[VE];
#pragma unroll
        for (int e = 0; e < VE; ++e) v[e] = act_t<ACT>(acc[p][e]);
        if (has_res) {
#pragma unroll
          for (int q = 0; q < VE / 4; ++q) {
            const i32x4 rv = __builtin_amdgcn_raw_buffer_load_b128(rr, (int)(off + 16 * q), 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int bits = rv[e];  // a scalar copy: bit_cast of the subscript would read element 0
              v[4 * q + e] += __builtin_bit_cast(float, bits);
            }
          }
        }
#pragma unroll
        for (int q = 0; q < VE / 4; ++q)
          __builtin_amdgcn_raw_buffer_store_b128(
              i32x4{__builtin_bit_cast(int, v[4 * q]), __builtin_bit_cast(int, v[4 * q + 1]),
                    __builtin_bit_cast(int, v[4 * q + 2]), __builtin_bit_cast(int, v[4 * q + 3])},
              ry, (int)(off + 16 * q), 0, DW_ST_AUX);
      } else {
        float v[VE];
#pragma unroll
        for (int e = 0; e < VE; ++e) v[e] = act_t<ACT>(acc[p][e]);
        if (has_res) {
          RawVec<T, VE> rv = load_raw<T, VE>(rr, off);
#pragma unroll
          for (int e = 0; e < VE; ++e) v[e] += widen_word<T>(rv.w[e / PER], e);
        }
        uint32_t wd[VE / 2];
#pragma unroll
        for (int q = 0; q < VE / 2; ++q) wd[q] = bf16x2_bits(v[2 * q], v[2 * q + 1]);
        if constexpr (VE == 8)
          __builtin_amdgcn_raw_buffer_store_b128(i32x4{(int)wd[0], (int)wd[1], (int)wd[2], (int)wd[3]}, ry, (int)off, 0, DW_ST_AUX);
        else
          __builtin_amdgcn_raw_buffer_store_b64(u32x2{wd[0], wd[1]}, ry, (int)off, 0, DW_ST_AUX);
      }
    }
    yoff += yrow;
  }
}
// ---------------------------------------------------------------------------
// int8, stride 1: four channels per lane (one 32-bit word per pixel) and the
// three window rows of each (column, channel) packed into one word, bytes
// (row r-2, row r-1, row r, 0). A new row enters every word with one byte
// permute, and each output then costs one 4-way int8 dot product per kernel
// column against the word (w[c][0][kw], w[c][1][kw], w[c][2][kw], 0): three
// instructions for the nine multiply-adds, exact in int32.
template <int PW, int TH, int ACT, int OUT, int PF>
__global__ __launch_bounds__(256) void dw3x3_i8_kernel(DwArgs a) {
  constexpr int NC = PW + 2;
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  if (t >= (uint32_t)a.total) return;
  const Geometry& g = a.g;
  const DwLane l = dw_lane<4, PW, TH>(a, t);
  const int c0 = l.c0, wo0 = l.wo0, ho0 = l.ho0, n = l.n;
  const __amdgpu_buffer_rsrc_t rx = dw_rsrc(a.x, a.x_bytes);
  const __amdgpu_buffer_rsrc_t ry = dw_rsrc(a.y, a.y_bytes);
  const bool has_res = a.e.res != nullptr;  // residual of y's type and shape, added after the activation
  const __amdgpu_buffer_rsrc_t rr = dw_rsrc(a.e.res, has_res ? a.y_bytes : 0);

  // weights of channels c0..c0+3 are 36 contiguous bytes ([4][3][3]),
  // 4-byte aligned because c0 is a multiple of 4
  uint32_t wb[9];
  const uint32_t* wp = reinterpret_cast<const uint32_t*>(a.w + (size_t)c0 * 9);
#pragma unroll
  for (int q = 0; q < 9; ++q) wb[q] = wp[q];
  auto wbyte = [&](int i) { return (wb[i >> 2] >> (8 * (i & 3))) & 0xffu; };
  int wk[3][4];  // wk[kw][e] = (w[e][0][kw], w[e][1][kw], w[e][2][kw], 0)
#pragma unroll
  for (int kw = 0; kw < 3; ++kw)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      wk[kw][e] = (int)(wbyte(9 * e + kw) | (wbyte(9 * e + 3 + kw) << 8) | (wbyte(9 * e + 6 + kw) << 16));

  const int rowbytes = g.w * g.c;
  uint32_t coff[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) coff[j] = dw_col_off(wo0 - g.pw + j, g, c0, 1);
  auto fetch_row = [&](int hi, uint32_t (&raw)[NC]) {
    const uint32_t rb = dw_row_off(hi, n, g, rowbytes);
#pragma unroll
    for (int j = 0; j < NC; ++j)
      raw[j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rx, (int)dw_add_sat(rb, coff[j]), 0, 0);
  };
  // window words: shift out the oldest row, byte e of the new row's word in
  // as byte 2 (selector bytes 4..7 pick the first operand, 0..3 the second,
  // 12 gives zero)
  uint32_t win[NC][4];
  auto push_row = [&](const uint32_t (&raw)[NC]) {
#pragma unroll
    for (int j = 0; j < NC; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) win[j][e] = __builtin_amdgcn_perm(win[j][e], raw[j], 0x0C000605u | ((uint32_t)e << 16));
  };
#pragma unroll
  for (int j = 0; j < NC; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) win[j][e] = 0;

  uint32_t nxt[PF][NC];  // the next PF input rows in flight
  {
    const int hi0 = ho0 - g.ph;
    fetch_row(hi0, nxt[0]);
    push_row(nxt[0]);
    fetch_row(hi0 + 1, nxt[0]);
    push_row(nxt[0]);
#pragma unroll
    for (int f = 0; f < PF && f < TH; ++f) fetch_row(hi0 + 2 + f, nxt[f]);
  }
  int bias[4];
  float scl[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    bias[e] = a.e.ibias ? a.e.ibias[c0 + e] : 0;
    scl[e] = OUT == OUT_I8 ? a.e.scale[c0 + e] : 0.f;
  }
  const int out_esz = OUT == OUT_I32 ? 4 : 1;
  uint32_t yoff = (uint32_t)((((n * g.ho + ho0) * g.wo + wo0) * g.cout + c0) * out_esz);
  const uint32_t yrow = (uint32_t)(g.wo * g.cout * out_esz);
  uint32_t poff[PW];
#pragma unroll
  for (int p = 0; p < PW; ++p) poff[p] = wo0 + p < g.wo ? (uint32_t)(p * g.cout * out_esz) : kDwOOB;

#pragma unroll
  for (int i = 0; i < TH; ++i) {
    if (ho0 + i >= g.ho) break;
    push_row(nxt[i % PF]);
    if (i + PF < TH) fetch_row(ho0 + i - g.ph + 2 + PF, nxt[i % PF]);
#pragma unroll
    for (int p = 0; p < PW; ++p) {
      int acc[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] = bias[e];
#pragma unroll
        for (int kw = 0; kw < 3; ++kw) acc[e] = __builtin_amdgcn_sdot4((int)win[p + kw][e], wk[kw][e], acc[e], false);
      }
      const uint32_t off = dw_add_sat(yoff, poff[p]);
      if constexpr (OUT == OUT_I32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = ACT == ACT_RELU ? max(acc[e], 0) : acc[e];
        __builtin_amdgcn_raw_buffer_store_b128(i32x4{acc[0], acc[1], acc[2], acc[3]}, ry, (int)off, 0, DW_ST_AUX);
      } else {
        uint32_t q[4];
        if (has_res) {
          const uint32_t rv = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rr, (int)off, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) q[e] = (uint32_t)requant_i8_res_t<ACT>(acc[e], scl[e], (int)(int8_t)(rv >> (8 * e)));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) q[e] = requant_i8_word_t<ACT>(acc[e], scl[e]);
        }
        // low bytes of q0..q3 into one word
        const uint32_t lo = __builtin_amdgcn_perm(q[1], q[0], 0x0C0C0400u);
        const uint32_t hi = __builtin_amdgcn_perm(q[3], q[2], 0x0C0C0400u);
        __builtin_amdgcn_raw_buffer_store_b32((int)__builtin_amdgcn_perm(hi, lo, 0x05040100u), ry, (int)off, 0, DW_ST_AUX);
      }
    }
    yoff += yrow;
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
    if constexpr (sizeof(T) == 1)
      hipLaunchKernelGGL((dw3x3_i8_kernel<PW, TH, decltype(ac)::value, decltype(oc)::value, DW_PF>),
                         dim3((unsigned)blocks), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((dw3x3_rows_kernel<T, VE, PW, TH, decltype(ac)::value, decltype(oc)::value, DW_PF>),
                         dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
  });
}

template <typename T, int VE, int PW>
hipError_t launch_rows_th(int th, const DwArgs& a, hipStream_t s) {
  switch (th) {
    case 8: return launch_rows_t<T, VE, PW, 8>(a, s);
    case 4: return launch_rows_t<T, VE, PW, 4>(a, s);
    case 2: return launch_rows_t<T, VE, PW, 2>(a, s);
    default: return launch_rows_t<T, VE, PW, 1>(a, s);
  }
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

int dw_prefetch_rows() { return DW_PF; }

// Lane shape of a depthwise plan: th > 0 selects the sliding-window kernels.
// A lane walks th output rows; th is the largest of 8, 4, 2 that still gives
// the chip DW_MIN_LANES_PER_CU lanes per CU (fewer rows per lane re-read more
// input rows from cache and repeat the lane's set-up, too few lanes leave CUs
// idle), else 1.
void dw_shape(const conv_plan* p, int* ve, int* pw, int* th) {
  const int c = p->g.c;
  const bool s1 = p->g.sh == 1 && p->g.sw == 1;
  const bool vec = p->loader == LOAD_VEC;
  *th = 0;
  if (s1 && c % 4 == 0) {
    *ve = 4;
    *pw = p->in_esz == 1 ? 4 : p->in_esz == 2 ? DW_BF16_PW : 2;
    if (p->tile > 0) {
      *th = p->tile;
      return;
    }
    const long lanes_per_row = (long)p->g.n * ((p->g.wo + *pw - 1) / *pw) * (c / 4);
    *th = 1;
    for (int t = 8; t >= 2; t /= 2)
      if (lanes_per_row * ((p->g.ho + t - 1) / t) >= 256L * DW_MIN_LANES_PER_CU) {
        *th = t;
        break;
      }
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
  a.y_bytes = (int)p->y_bytes;
  int ve, pw, th;
  dw_shape(p, &ve, &pw, &th);
  if (th) {
    switch (p->in_esz) {
      case 4: return launch_rows_th<float, 4, 2>(th, a, s);
      case 2: return launch_rows_th<uint16_t, 4, DW_BF16_PW>(th, a, s);
      default: return launch_rows_th<int8_t, 4, 4>(th, a, s);
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
