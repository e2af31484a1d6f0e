// mfma_epilogue.h -- the fused epilogue of one 16x16 MFMA output fragment.
//
// After v_mfma_*_16x16x* with weights as the A operand and pixels as the B
// operand, lane l holds four consecutive output channels co..co+3 of one
// pixel px. This writes them once, to NHWC, after bias, activation and the
// output conversion: bf16 (one RNE rounding), int8 (requantisation), or the
// int32 checkpoint (acc + bias, optional ReLU).
#pragma once

#include <type_traits>

#include "device_common.h"

namespace convnhwc {

// Per-channel constants of the four channels a lane owns.
struct QuadConsts {
  float bsf[4];
  int bsi[4];
  float scl[4];
};

template <int ESZ>
__device__ __forceinline__ QuadConsts load_quad_consts(const Epi& e, int co, int cout) {
  QuadConsts q;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    q.bsf[r] = 0.f;
    q.bsi[r] = 0;
    q.scl[r] = 0.f;
    if (co + r < cout) {
      if constexpr (ESZ == 2) {
        if (e.bias) q.bsf[r] = e.bias[co + r];
      } else {
        if (e.ibias) q.bsi[r] = e.ibias[co + r];
        if (e.scale) q.scl[r] = e.scale[co + r];
      }
    }
  }
  return q;
}

// Store the quad v (channels co..co+3 of pixel px). The caller guarantees
// px < m and co < cout; channels at or beyond cout are not written. res is
// the residual (y's type and shape) added after the activation, or null.
template <int ESZ, typename acc_t>
__device__ __forceinline__ void store_quad(const acc_t& v, const QuadConsts& q, int co, int px, int cout,
                                           int out_kind, int act, void* y, const void* res) {
  const size_t off = (size_t)px * cout + co;
  const bool vec4 = (cout & 3) == 0;
  if constexpr (ESZ == 2) {
    uint32_t h[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float f = apply_act(v[r] + q.bsf[r], act);
      if (res && co + r < cout) f += bf16_bits_to_f32(static_cast<const uint16_t*>(res)[off + r]);
      h[r] = f32_to_bf16_bits(f);
    }
    uint16_t* yp = reinterpret_cast<uint16_t*>(y) + off;
    if (vec4) {
      uint2 w;
      w.x = h[0] | (h[1] << 16);
      w.y = h[2] | (h[3] << 16);
      *reinterpret_cast<uint2*>(yp) = w;
    } else {
      for (int r = 0; r < 4; ++r)
        if (co + r < cout) yp[r] = (uint16_t)h[r];
    }
  } else if (out_kind == OUT_I32) {
    int w[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      w[r] = v[r] + q.bsi[r];
      if (act == ACT_RELU) w[r] = w[r] > 0 ? w[r] : 0;
    }
    int32_t* yp = reinterpret_cast<int32_t*>(y) + off;
    if (vec4) {
      *reinterpret_cast<i32x4*>(yp) = i32x4{w[0], w[1], w[2], w[3]};
    } else {
      for (int r = 0; r < 4; ++r)
        if (co + r < cout) yp[r] = w[r];
    }
  } else {
    uint32_t b[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      b[r] = (uint32_t)((res ? requant_i8_res(v[r] + q.bsi[r], q.scl[r], act,
                                              co + r < cout ? static_cast<const int8_t*>(res)[off + r] : 0)
                             : requant_i8(v[r] + q.bsi[r], q.scl[r], act)) &
                        0xff);
    int8_t* yp = reinterpret_cast<int8_t*>(y) + off;
    if (vec4) {
      *reinterpret_cast<uint32_t*>(yp) = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
    } else {
      for (int r = 0; r < 4; ++r)
        if (co + r < cout) yp[r] = (int8_t)b[r];
    }
  }
}

// ---- compile-time epilogue ------------------------------------------------
// The per-element form above decides the activation and the output kind at
// run time for every element; across the 64-256 accumulator quads of a
// large tile those uniform branches cost more than the arithmetic. The forms
// below take both as template arguments (with_epilogue turns the layer's run
// time values into them once per tile) and store through buffer
// instructions, whose out-of-range offsets are dropped, so a ragged tile
// needs no branch either.

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// f(out_kind, act) with both as std::integral_constant, for the output kinds
// and activations an element size supports (bf16 -> bf16; int8 -> int8, or
// the int32 checkpoint with NONE/RELU).
template <int ESZ, class F>
__device__ __forceinline__ void with_epilogue(int out_kind, int act, F&& f) {
  using std::integral_constant;
  if constexpr (ESZ == 2) {
    switch (act) {
      case ACT_RELU: f(integral_constant<int, OUT_BF16>{}, integral_constant<int, ACT_RELU>{}); break;
      case ACT_RELU6: f(integral_constant<int, OUT_BF16>{}, integral_constant<int, ACT_RELU6>{}); break;
      case ACT_MISH: f(integral_constant<int, OUT_BF16>{}, integral_constant<int, ACT_MISH>{}); break;
      default: f(integral_constant<int, OUT_BF16>{}, integral_constant<int, ACT_NONE>{}); break;
    }
  } else if (out_kind == OUT_I32) {
    if (act == ACT_RELU)
      f(integral_constant<int, OUT_I32>{}, integral_constant<int, ACT_RELU>{});
    else
      f(integral_constant<int, OUT_I32>{}, integral_constant<int, ACT_NONE>{});
  } else {
    switch (act) {
      case ACT_RELU: f(integral_constant<int, OUT_I8>{}, integral_constant<int, ACT_RELU>{}); break;
      case ACT_RELU6: f(integral_constant<int, OUT_I8>{}, integral_constant<int, ACT_RELU6>{}); break;
      case ACT_MISH: f(integral_constant<int, OUT_I8>{}, integral_constant<int, ACT_MISH>{}); break;
      default: f(integral_constant<int, OUT_I8>{}, integral_constant<int, ACT_NONE>{}); break;
    }
  }
}

// The output tensor as a buffer: y, its size in bytes, m pixels x cout
// channels (cout % 4 == 0 for store_quad_t), and the residual added after the
// activation (same type and shape as y; has_res is uniform, so the test is a
// scalar branch).
struct OutRef {
  __amdgpu_buffer_rsrc_t r;
  __amdgpu_buffer_rsrc_t rr;
  int m, cout;
  bool has_res;
};

__device__ __forceinline__ OutRef out_ref(void* y, int m, int cout, int out_esz, const void* res) {
  OutRef o;
  o.r = __builtin_amdgcn_make_buffer_rsrc(y, 0, m * cout * out_esz, 0x00020000);
  o.rr = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(res), 0, res ? m * cout * out_esz : 0, 0x00020000);
  o.m = m;
  o.cout = cout;
  o.has_res = res != nullptr;
  return o;
}

// Per-channel constants of channels co..co+3 for store_quad_t (cout % 4 ==
// 0, co % 4 == 0): one 16-byte buffer load per array; a NULL array or a quad
// past cout reads as zeros.
template <int ESZ>
__device__ __forceinline__ QuadConsts load_quad_consts_t(const Epi& e, int co, int cout) {
  QuadConsts q;
  const uint32_t off = (uint32_t)co * 4u;
  if constexpr (ESZ == 2) {
    const __amdgpu_buffer_rsrc_t rb =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(e.bias), 0, e.bias ? cout * 4 : 0, 0x00020000);
    const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      q.bsf[r] = __builtin_bit_cast(float, (uint32_t)b[r]);
      q.bsi[r] = 0;
      q.scl[r] = 0.0f;
    }
  } else {
    const __amdgpu_buffer_rsrc_t rb =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(e.ibias), 0, e.ibias ? cout * 4 : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(e.scale), 0, e.scale ? cout * 4 : 0, 0x00020000);
    const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0);
    const u32x4 sc = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      q.bsf[r] = 0.0f;
      q.bsi[r] = (int)b[r];
      q.scl[r] = __builtin_bit_cast(float, (uint32_t)sc[r]);
    }
  }
  return q;
}

// bf16(act(v + bias) [+ residual]) of channels co..co+3 of pixel px, packed
// as one 8-byte quad (the residual quad is read only when px < m and
// co < cout), for kernels that store through LDS or delay their stores.
template <int ACT>
__device__ __forceinline__ u32x2 pack_quad_bf16(const f32x4& v, const QuadConsts& q, int co, int px, const OutRef& o) {
  float f[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) f[r] = act_t<ACT>(v[r] + q.bsf[r]);
  if (o.has_res) {
    const bool in = px < o.m && co < o.cout;
    const u32x2 rv =
        __builtin_amdgcn_raw_buffer_load_b64(o.rr, in ? (uint32_t)(px * o.cout + co) * 2u : 0x80000000u, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) f[r] += bf16_bits_to_f32((r & 1) ? (rv[r >> 1] >> 16) : (rv[r >> 1] & 0xffffu));
  }
  return u32x2{bf16x2_bits(f[0], f[1]), bf16x2_bits(f[2], f[3])};
}

// Store quad v (channels co..co+3 of pixel px); nothing is written when
// px >= m or co >= cout. Requires cout % 4 == 0.
template <int ESZ, int OUT, int ACT, typename acc_t>
__device__ __forceinline__ void store_quad_t(const acc_t& v, const QuadConsts& q, int co, int px, const OutRef& o) {
  constexpr uint32_t kNowhere = 0x80000000u;  // past any output buffer
  const bool in = px < o.m && co < o.cout;
  const uint32_t idx = (uint32_t)(px * o.cout + co);
  if constexpr (ESZ == 2) {
    float f[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) f[r] = act_t<ACT>(v[r] + q.bsf[r]);
    if (o.has_res) {
      const u32x2 rv = __builtin_amdgcn_raw_buffer_load_b64(o.rr, in ? idx * 2u : kNowhere, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) f[r] += bf16_bits_to_f32((r & 1) ? (rv[r >> 1] >> 16) : (rv[r >> 1] & 0xffffu));
    }
    const u32x2 d = {bf16x2_bits(f[0], f[1]), bf16x2_bits(f[2], f[3])};
    __builtin_amdgcn_raw_buffer_store_b64(d, o.r, in ? idx * 2u : kNowhere, 0, 0);
  } else if constexpr (OUT == OUT_I32) {
    u32x4 d;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int w = v[r] + q.bsi[r];
      if constexpr (ACT == ACT_RELU) w = w > 0 ? w : 0;
      d[r] = (uint32_t)w;
    }
    __builtin_amdgcn_raw_buffer_store_b128(d, o.r, in ? idx * 4u : kNowhere, 0, 0);
  } else {
    uint32_t b = 0;
    if (o.has_res) {
      const uint32_t rv = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(o.rr, in ? idx : kNowhere, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        b |= ((uint32_t)requant_i8_res_t<ACT>(v[r] + q.bsi[r], q.scl[r], (int)(int8_t)(rv >> (8 * r))) & 0xffu)
             << (8 * r);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) b |= (requant_i8_word_t<ACT>(v[r] + q.bsi[r], q.scl[r]) & 0xffu) << (8 * r);
    }
    __builtin_amdgcn_raw_buffer_store_b32(b, o.r, in ? idx : kNowhere, 0, 0);
  }
}

}  // namespace convnhwc
