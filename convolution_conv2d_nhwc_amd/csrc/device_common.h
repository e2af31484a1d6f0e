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

// Q = clamp(round_half_even(m + rr), -127, 127) for a float m and an
// integer rr, with one rounding of the exact sum (a plain float add of m and
// rr can round before the integer rounding does). With q0 = rne(m) and the
// remainder d = m - q0 (exact: |d| <= 1/2, and m and q0 are within a factor
// of two of each other unless q0 = 0), m + rr = (q0 + rr) + d. For |d| < 1/2
// the nearest integer is q0 + rr. For d = +-1/2 the sum is a tie between
// q0 + rr and q0 + rr + 2d; q0 is even (it is itself a tie broken to even),
// so the even neighbour is q0 + rr when rr is even and q0 + rr + 2d when rr
// is odd. m is first clamped to +-2^20, beyond which the result saturates
// either way; adding 1.5 * 2^23 then rounds half to even in the adder.
__device__ __forceinline__ int round_add_sat_i8(float m, int rr) {
  const float c = __builtin_amdgcn_fmed3f(m, -1048576.0f, 1048576.0f);
  const float t = c + 12582912.0f;
  const int q0 = (int)(__builtin_bit_cast(uint32_t, t) - 0x4B400000u);
  const float d = c - (t - 12582912.0f);
  const int tie = (rr & 1) && __builtin_fabsf(d) == 0.5f ? (d > 0.0f ? 1 : -1) : 0;
  return min(max(q0 + rr + tie, -127), 127);
}

// With a residual rr added after the activation: Q = clamp(rne(act(v) + rr),
// -127, 127).
__device__ __forceinline__ int requant_i8_res(int r, float s, int act, int rr) {
  const float v = __fmul_rn((float)r, s);
  return round_add_sat_i8(apply_act(v, act), rr);
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
    c = __builtin_amdgcn_fmed3f(act_t<ACT>(v), -127.0f, 127.0f);
  return __builtin_bit_cast(uint32_t, c + 12582912.0f);
}
// The same with a residual rr (an int8 value in the output's units) added
// after the activation: Q = clamp(rne(act(v) + rr), -127, 127), the sum
// rounded once (round_add_sat_i8).
template <int ACT>
__device__ __forceinline__ int requant_i8_res_t(int r, float s, int rr) {
  const float v = __fmul_rn((float)r, s);
  float m;
  if constexpr (ACT == ACT_RELU)
    m = fmaxf(v, 0.0f);
  else if constexpr (ACT == ACT_RELU6)
    m = __builtin_amdgcn_fmed3f(v, 0.0f, 6.0f);
  else
    m = act_t<ACT>(v);
  return round_add_sat_i8(m, rr);
}

template <int ACT>
__device__ __forceinline__ int requant_i8_t(int r, float s) {
  return (int)(requant_i8_word_t<ACT>(r, s) - 0x4B400000u);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
  __bf16 h = (__bf16)v;  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

// Two floats to a packed pair of bf16 (lo in the low half), each rounded to
// nearest even exactly as f32_to_bf16_bits rounds it: one v_cvt_pk_bf16_f32
// for the pair.
__device__ __forceinline__ uint32_t bf16x2_bits(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
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
