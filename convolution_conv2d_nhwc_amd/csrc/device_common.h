// device_common.h -- types and the fused epilogue shared by the gfx950 kernels.
//
// The epilogue is the per-output-element tail of every conv kernel: bias add,
// activation, and the conversion to the output type, done in registers so the
// output tensor is written exactly once (nanoinfer README, GPU section: the
// fused bias/ReLU epilogue removes two extra passes over the output).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace convnhwc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

enum Act { ACT_NONE = 0, ACT_RELU = 1, ACT_RELU6 = 2, ACT_MISH = 3 };

// Output kinds of a kernel instance.
enum OutKind {
  OUT_F32 = 0,   // float out (fp32 layers)
  OUT_BF16 = 1,  // bf16 out, one RNE rounding
  OUT_I8 = 2,    // int8 out through the per-channel requantisation
  OUT_I32 = 3    // int32 checkpoint (acc + bias, optional ReLU)
};

// Mish(v) = v * tanh(ln(1 + e^v)) (YOLOv4 on Tenstorrent Wormhole, section 7
// function table). With t = e^v, tanh(ln(1+t)) = ((1+t)^2 - 1)/((1+t)^2 + 1)
// = n/(n + 2) where n = t*(t + 2). This form has no cancellation for v << 0
// (the K1 form v - 2v/((1+t)^2+1) of section 9 subtracts two nearly equal
// numbers there). The exponent is clamped at 20: beyond it n/(n+2) rounds to
// 1 in fp32, so Mish(v) = v, and e^v cannot overflow. The quotient uses the
// hardware reciprocal (1 ulp) instead of an IEEE division.
__device__ __forceinline__ float mish_f32(float v) {
  const float t = __expf(fminf(v, 20.0f));
  const float n = t * (t + 2.0f);
  return v * (n * __builtin_amdgcn_rcpf(n + 2.0f));
}

// Mish for outputs that are rounded to bf16 or to an integer afterwards, in
// seven instructions (two of them transcendental) instead of nine: the same
// function written as v - 2v / ((1 + e^v)^2 + 1), the section 9 form. No
// clamp is needed: e^v = inf gives v, e^v = 0 gives 0. For v < 0 the
// subtraction loses relative accuracy (the absolute error stays about
// |v| * 2^-22), which is far below the rounding of a bf16 output at the scale
// of its layer, and an int8 output never rounds near there (|Mish(v)| < 0.31
// for v < 0). For v > 0 the quotient is at most 0.2 and there is no
// cancellation.
__device__ __forceinline__ float mish_lo(float v) {
  const float u = __builtin_amdgcn_exp2f(v * 1.44269504088896341f) + 1.0f;
  const float r = __builtin_amdgcn_rcpf(__builtin_fmaf(u, u, 1.0f));
  return __builtin_fmaf(-2.0f * v, r, v);
}

__device__ __forceinline__ float apply_act(float v, int act) {
  switch (act) {
    case ACT_RELU: return fmaxf(v, 0.0f);
    case ACT_RELU6: return fminf(fmaxf(v, 0.0f), 6.0f);
    case ACT_MISH: return mish_f32(v);
    default: return v;
  }
}

// int8 requantisation of one int32 value r = acc + bias: an RNE int->float
// conversion, one RNE float multiply (never fused), the activation, then
// round-half-to-even and saturation to [-127, 127].
__device__ __forceinline__ int requant_i8(int r, float s, int act) {
  const float v = __fmul_rn((float)r, s);
  const float m = apply_act(v, act);
  const float q = fminf(fmaxf(__builtin_rintf(m), -127.0f), 127.0f);
  return (int)q;
}

// With a residual rr added after the activation (see requant_i8_res_t).
__device__ __forceinline__ int requant_i8_res(int r, float s, int act, int rr) {
  const float v = __fmul_rn((float)r, s);
  const float m = fminf(fmaxf(apply_act(v, act), -1048576.0f), 1048576.0f);
  const int q = (int)__builtin_rintf(m);
  return min(max(q + rr, -127), 127);
}

// Compile-time loop: f(std::integral_constant<int, i>) for i = I .. N-1.
// Unlike `#pragma unroll` it does not depend on the unroller's size limit, so
// register arrays indexed by i stay in registers however long the body is.
template <int I, int N>
struct StaticFor {
  template <class F>
  __device__ __forceinline__ static void run(F&& f) {
    f(std::integral_constant<int, I>{});
    StaticFor<I + 1, N>::run(f);
  }
};
template <int N>
struct StaticFor<N, N> {
  template <class F>
  __device__ __forceinline__ static void run(F&&) {}
};

// The same with the activation and, for requant_i8_t, the clamp fixed at
// compile time (no per-element branch).
template <int ACT>
__device__ __forceinline__ float act_t(float v) {
  if constexpr (ACT == ACT_RELU)
    return fmaxf(v, 0.0f);
  else if constexpr (ACT == ACT_RELU6)
    return fminf(fmaxf(v, 0.0f), 6.0f);
  else if constexpr (ACT == ACT_MISH)
    return mish_f32(v);
  else
    return v;
}

// act_t with mish_lo: for bf16 and int8 outputs
template <int ACT>
__device__ __forceinline__ float act_lo_t(float v) {
  if constexpr (ACT == ACT_MISH)
    return mish_lo(v);
  else
    return act_t<ACT>(v);
}

// The int8 requantisation with the activation fixed at compile time. The
// saturation comes first (the bounds are integers, so clamping before or
// after rounding is the same); adding 1.5 * 2^23 then rounds half to even in
// the adder and leaves the integer in the low mantissa bits. The low byte of
// the returned word is the int8 result (two's complement); requant_i8_t
// gives it as an int.
template <int ACT>
__device__ __forceinline__ uint32_t requant_i8_word_t(int r, float s) {
  const float v = __fmul_rn((float)r, s);
  float c;  // the activation and the saturation, one clamp where they merge
  if constexpr (ACT == ACT_RELU)
    c = __builtin_amdgcn_fmed3f(v, 0.0f, 127.0f);
  else if constexpr (ACT == ACT_RELU6)
    c = __builtin_amdgcn_fmed3f(v, 0.0f, 6.0f);
  else
    c = __builtin_amdgcn_fmed3f(act_lo_t<ACT>(v), -127.0f, 127.0f);
  return __builtin_bit_cast(uint32_t, c + 12582912.0f);
}
// The same with a residual rr (an int8 value in the output's units) added
// after the activation: Q = clamp(rne(act(v) + rr), -127, 127). rr is an
// integer, so rne(m + rr) = rne(m) + rr exactly: the activation's value is
// rounded first (clamped to +-2^20 so that the adder rounds it; beyond that
// it saturates either way), then rr is added in integers before the
// saturation.
template <int ACT>
__device__ __forceinline__ int requant_i8_res_t(int r, float s, int rr) {
  const float v = __fmul_rn((float)r, s);
  float m;
  if constexpr (ACT == ACT_RELU)
    m = fmaxf(v, 0.0f);
  else if constexpr (ACT == ACT_RELU6)
    m = __builtin_amdgcn_fmed3f(v, 0.0f, 6.0f);
  else
    m = act_lo_t<ACT>(v);
  const float c = __builtin_amdgcn_fmed3f(m, -1048576.0f, 1048576.0f);
  const int q = (int)(__builtin_bit_cast(uint32_t, c + 12582912.0f) - 0x4B400000u);
  return min(max(q + rr, -127), 127);
}

template <int ACT>
__device__ __forceinline__ int requant_i8_t(int r, float s) {
  return (int)(requant_i8_word_t<ACT>(r, s) - 0x4B400000u);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
  __bf16 h = (__bf16)v;  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

// Per-layer epilogue constants. For fp32/bf16 layers `bias` is float[c_out]
// (or null); for int8 layers `ibias` is int32[c_out] (or null) and `scale`
// float[c_out] (null only for the int32 checkpoint output).
struct Epi {
  const float* bias;
  const int32_t* ibias;
  const float* scale;
  const void* res;  // residual of the output's type and shape, added after the activation, or null
  int act;
};

}  // namespace convnhwc
