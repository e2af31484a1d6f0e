// mfma_epilogue.h -- the fused epilogue of one 16x16 MFMA output fragment.
//
// After v_mfma_*_16x16x* with weights as the A operand and pixels as the B
// operand, lane l holds four consecutive output channels co..co+3 of one
// pixel px. This writes them once, to NHWC, after bias, activation and the
// output conversion: bf16 (one RNE rounding), int8 (requantisation), or the
// int32 checkpoint (acc + bias, optional ReLU).
#pragma once

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
// px < m and co < cout; channels at or beyond cout are not written.
template <int ESZ, typename acc_t>
__device__ __forceinline__ void store_quad(const acc_t& v, const QuadConsts& q, int co, int px, int cout,
                                           int out_kind, int act, void* y) {
  const size_t off = (size_t)px * cout + co;
  const bool vec4 = (cout & 3) == 0;
  if constexpr (ESZ == 2) {
    uint32_t h[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) h[r] = f32_to_bf16_bits(apply_act(v[r] + q.bsf[r], act));
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
    for (int r = 0; r < 4; ++r) b[r] = (uint32_t)(requant_i8(v[r] + q.bsi[r], q.scl[r], act) & 0xff);
    int8_t* yp = reinterpret_cast<int8_t*>(y) + off;
    if (vec4) {
      *reinterpret_cast<uint32_t*>(yp) = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
    } else {
      for (int r = 0; r < 4; ++r)
        if (co + r < cout) yp[r] = (int8_t)b[r];
    }
  }
}

}  // namespace convnhwc
