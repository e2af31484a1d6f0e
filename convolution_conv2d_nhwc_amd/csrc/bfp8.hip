// bfp8.hip -- encoding of OHWI weights into the library's block-floating-point
// (bfp8) image, the storage the implicit-GEMM kernel decodes (YOLOv4 on
// Tenstorrent Wormhole, the table "Precision in the selected m640 graph":
// weights in block floating point, 16 values sharing one exponent).
//
// One thread per block of 16 consecutive weights of a row (K zero-padded to
// Kp): the block's largest magnitude A gives e = max(floor(log2 A), -126);
// each mantissa is round_half_even(w * 2^(6 - e)), and if one reaches 128
// the block is rounded again with e + 1; the exponent byte is e + 127 (0 for
// an all-zero block). The scaling by a power of two is exact in fp32 (or
// the scaled value is far below one half, which rounds to 0 either way), so
// the fp32 arithmetic gives the exact mantissas of the definition. Output:
// int8 mantissas [rows][Kp] (one 16-byte store per block), then uint8
// exponents [rows][Kp / 16].
#include "device_common.h"
#include "plan.h"

namespace convnhwc {
namespace {

struct Bfp8Args {
  const void* w;
  int w_f32;  // weights are fp32 (else bf16)
  int rows, k, kp;
  unsigned char* out;
};

__global__ __launch_bounds__(256) void bfp8_pack_kernel(Bfp8Args a) {
  const int nb = a.kp >> 4;
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= a.rows * nb) return;
  const int r = t / nb, b = t - r * nb;
  float v[16];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int kk = b * 16 + i;
    float x = 0.0f;
    if (kk < a.k) {
      const size_t idx = (size_t)r * a.k + kk;
      x = a.w_f32 ? static_cast<const float*>(a.w)[idx]
                  : __builtin_bit_cast(float, (uint32_t)static_cast<const unsigned short*>(a.w)[idx] << 16);
    }
    v[i] = x;
    amax = fmaxf(amax, __builtin_fabsf(x));
  }
  uint32_t mw[4] = {0, 0, 0, 0};
  uint32_t ebyte = 0;
  if (amax > 0.0f) {
    // amax = f * 2^x with f in [0.5, 1): floor(log2 amax) = x - 1
    int e = max(__builtin_amdgcn_frexp_expf(amax) - 1, -126);
    int q[16];
    int qmax = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      q[i] = (int)__builtin_rintf(__builtin_ldexpf(v[i], 6 - e));
      qmax = max(qmax, abs(q[i]));
    }
    if (qmax > 127) {
      ++e;
#pragma unroll
      for (int i = 0; i < 16; ++i) q[i] = (int)__builtin_rintf(__builtin_ldexpf(v[i], 6 - e));
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) mw[i >> 2] |= ((uint32_t)q[i] & 0xffu) << (8 * (i & 3));
    ebyte = (uint32_t)(e + 127);
  }
  *reinterpret_cast<i32x4*>(a.out + (size_t)r * a.kp + b * 16) =
      i32x4{(int)mw[0], (int)mw[1], (int)mw[2], (int)mw[3]};
  a.out[(size_t)a.rows * a.kp + (size_t)r * nb + b] = (unsigned char)ebyte;
}

}  // namespace

hipError_t launch_bfp8_pack(const void* w, int w_f32, int rows, int k, void* packed, hipStream_t s) {
  Bfp8Args a;
  a.w = w;
  a.w_f32 = w_f32;
  a.rows = rows;
  a.k = k;
  a.kp = (k + 15) / 16 * 16;
  a.out = static_cast<unsigned char*>(packed);
  const long blocks = ((long)rows * (a.kp / 16) + 255) / 256;
  hipLaunchKernelGGL(bfp8_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace convnhwc
