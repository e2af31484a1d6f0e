// spp.hip -- SPP max-pool block: the 13x13, 9x9 and 5x5 stride-1 max pools
// of an NHWC map and the map itself, concatenated along channels (zerolat.eu
// YOLOv4 report, section 9 "Four custom Tensix kernels", K3; section 3 names SPP as the
// block that widens the context with those three windows).
//
// The larger windows come from cascaded 5x5 pools, the identity the report's
// kernel uses: with positions outside the image ignored, the 5x5 max of a 5x5
// max is the 9x9 max and a third pass gives the 13x13 one (every element of
// the larger window is reached through an intermediate position that lies
// inside both the image and the smaller window), and a 5x5 pool is a 5-wide
// row max followed by a 5-tall column max. A workgroup keeps one image of a
// slice of channels in LDS and runs the six passes there, so global memory
// sees one read of x and one write of y: the block is bound by HBM, and for
// the small maps SPP runs on, by launch and latency.
//
// Values are compared through an order-preserving integer key: bf16 and fp32
// bit patterns become two's-complement integers of the same order (negative
// values get their magnitude bits flipped), int8 widens to int16. One packed
// 16-bit max then handles two bf16 or int8 values, and the keys convert back
// to the exact input bits. -0 orders below +0.
#include "device_common.h"
#include "plan.h"

namespace convnhwc {
namespace {

typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef signed char s8x8 __attribute__((ext_vector_type(8)));
typedef int i32x2v __attribute__((ext_vector_type(2)));

struct SppArgs {
  const char* x;
  char* y;
  int h, w, c;     // map size
  int nch;         // 16-byte key chunks per pixel in one workgroup (a power of two)
  int nch_log2;
  int nblk_c;      // workgroups per image
  float inv_w;     // 1 / w
  int x_bytes, y_bytes;
};

// DT: 0 fp32 (4 channels per chunk), 1 bf16 (8), 2 int8 (8, 8 bytes in memory)
template <int DT>
struct SppType {
  static constexpr int kEsz = DT == 0 ? 4 : DT == 1 ? 2 : 1;
  static constexpr int kPer = DT == 0 ? 4 : 8;  // channels per chunk
  static constexpr int kGlobal = kPer * kEsz;   // bytes per chunk in memory
};

template <int DT>
__device__ __forceinline__ i32x4 spp_load_key(__amdgpu_buffer_rsrc_t r, uint32_t off, i32x4* raw) {
  if constexpr (DT == 2) {
    const i32x2v b = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
    *raw = i32x4{b[0], b[1], 0, 0};
    const s16x8 k = __builtin_convertvector(__builtin_bit_cast(s8x8, b), s16x8);
    return __builtin_bit_cast(i32x4, k);
  } else {
    const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    *raw = v;
    if constexpr (DT == 1) {
      const s16x8 b = __builtin_bit_cast(s16x8, v);
      return __builtin_bit_cast(i32x4, b ^ ((b >> 15) & (short)0x7fff));
    } else {
      return v ^ ((v >> 31) & 0x7fffffff);
    }
  }
}

// AUX: cache policy of the stores (2 = non-temporal, for outputs that
// stream past the caches)
template <int DT, int AUX>
__device__ __forceinline__ void spp_store_raw(i32x4 raw, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (DT == 2)
    __builtin_amdgcn_raw_buffer_store_b64(i32x2v{raw[0], raw[1]}, r, (int)off, 0, AUX);
  else
    __builtin_amdgcn_raw_buffer_store_b128(raw, r, (int)off, 0, AUX);
}

template <int DT, int AUX>
__device__ __forceinline__ void spp_store_key(i32x4 k, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (DT == 2) {
    const s8x8 b = __builtin_convertvector(__builtin_bit_cast(s16x8, k), s8x8);
    const i32x2v v = __builtin_bit_cast(i32x2v, b);
    spp_store_raw<DT, AUX>(i32x4{v[0], v[1], 0, 0}, r, off);
  } else if constexpr (DT == 1) {
    const s16x8 b = __builtin_bit_cast(s16x8, k);
    spp_store_raw<DT, AUX>(__builtin_bit_cast(i32x4, b ^ ((b >> 15) & (short)0x7fff)), r, off);
  } else {
    spp_store_raw<DT, AUX>(k ^ ((k >> 31) & 0x7fffffff), r, off);
  }
}

template <int DT>
__device__ __forceinline__ i32x4 spp_max(i32x4 a, i32x4 b) {
  if constexpr (DT == 0)
    return __builtin_elementwise_max(a, b);
  else
    return __builtin_bit_cast(i32x4, __builtin_elementwise_max(__builtin_bit_cast(s16x8, a),
                                                                __builtin_bit_cast(s16x8, b)));
}

template <int DT, int AUX>
__global__ __launch_bounds__(256) void spp_kernel(SppArgs a) {
  typedef SppType<DT> Ty;
  extern __shared__ i32x4 spp_lds[];
  const int nch = a.nch;
  const int npx = a.h * a.w;
  const int items = npx * nch;
  i32x4* const A = spp_lds;
  i32x4* const B = spp_lds + items;
  const int n = blockIdx.x / a.nblk_c;
  const int c0 = (blockIdx.x - n * a.nblk_c) * nch * Ty::kPer;  // first channel of the slice
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(a.x), 0, a.x_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(a.y, 0, a.y_bytes, 0x00020000);
  const uint32_t xpix = (uint32_t)a.c * Ty::kEsz;  // bytes per pixel of x
  const uint32_t ypix = 4 * xpix;                  // of y
  const uint32_t x0 = (uint32_t)(n * npx) * xpix + (uint32_t)c0 * Ty::kEsz;
  const uint32_t y0 = (uint32_t)(n * npx) * ypix + (uint32_t)c0 * Ty::kEsz;
  // item i = (pixel i >> nch_log2, chunk i & (nch - 1)); the row of a pixel
  // by a float reciprocal (pixel + 1/2 keeps the quotient at least 1/(2w)
  // away from an integer, far beyond the rounding error)
  auto split = [&](int i, int& px, int& ch, int& hh, int& ww) {
    px = i >> a.nch_log2;
    ch = i & (nch - 1);
    hh = (int)(((float)px + 0.5f) * a.inv_w);
    ww = px - hh * a.w;
  };

  for (int i = threadIdx.x; i < items; i += 256) {
    int px, ch, hh, ww;
    split(i, px, ch, hh, ww);
    i32x4 raw;
    A[i] = spp_load_key<DT>(rx, x0 + px * xpix + ch * Ty::kGlobal, &raw);
    spp_store_raw<DT, AUX>(raw, ry, y0 + px * ypix + 3 * xpix + ch * Ty::kGlobal);  // block 3: the map
  }
  __syncthreads();
  // pass p turns A = the (4p+1)-window max into the (4p+5)-window max and
  // writes it to block 2 - p (5x5 -> 2, 9x9 -> 1, 13x13 -> 0). Indices clamp
  // to the image: the clamped position lies between the centre and the
  // requested one, so it is inside the window and the max is unchanged.
  for (int p = 0; p < 3; ++p) {
    for (int i = threadIdx.x; i < items; i += 256) {
      int px, ch, hh, ww;
      split(i, px, ch, hh, ww);
      i32x4 m = A[i];
#pragma unroll
      for (int d = -2; d <= 2; ++d) {
        if (d == 0) continue;
        const int w2 = min(max(ww + d, 0), a.w - 1);
        m = spp_max<DT>(m, A[((hh * a.w + w2) << a.nch_log2) + ch]);
      }
      B[i] = m;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < items; i += 256) {
      int px, ch, hh, ww;
      split(i, px, ch, hh, ww);
      i32x4 m = B[i];
#pragma unroll
      for (int d = -2; d <= 2; ++d) {
        if (d == 0) continue;
        const int h2 = min(max(hh + d, 0), a.h - 1);
        m = spp_max<DT>(m, B[((h2 * a.w + ww) << a.nch_log2) + ch]);
      }
      A[i] = m;
      spp_store_key<DT, AUX>(m, ry, y0 + px * ypix + (2 - p) * xpix + ch * Ty::kGlobal);
    }
    __syncthreads();
  }
}

}  // namespace

// Chunks per pixel and workgroup: the largest power of two that divides the
// map's chunk count, keeps the two LDS copies of the slice within 64 KiB
// and still gives 256 workgroups when the batch allows (on the 16 x 20x20x512
// batch, 256 workgroups of four chunks ran in 18 us, 1024 of one in 33 us:
// more items per thread between the barriers pays); 0 if one chunk per pixel
// does not fit (more than 2048 pixels).
int spp_chunks(int64_t n, int64_t h, int64_t w, int64_t c, int dtype) {
  const int per = dtype == CONV_F32 ? 4 : 8;
  const int64_t npx = h * w;
  if (c % per || npx * 32 > 65536) return 0;
  const int64_t kc = c / per;
  int nch = 1;
  while (kc % (2 * nch) == 0 && npx * 32 * (2 * nch) <= 65536 && n * (kc / (2 * nch)) >= 256) nch *= 2;
  return nch;
}

hipError_t launch_spp(const void* x, int dtype, void* y, int64_t n, int64_t h, int64_t w, int64_t c, int64_t x_bytes,
                      hipStream_t s) {
  const int nch = spp_chunks(n, h, w, c, dtype);
  if (nch == 0) return hipErrorInvalidValue;
  const int per = dtype == CONV_F32 ? 4 : 8;
  SppArgs a;
  a.x = static_cast<const char*>(x);
  a.y = static_cast<char*>(y);
  a.h = (int)h;
  a.w = (int)w;
  a.c = (int)c;
  a.nch = nch;
  a.nch_log2 = __builtin_ctz((unsigned)nch);
  a.nblk_c = (int)(c / per / nch);
  a.inv_w = 1.0f / (float)w;
  a.x_bytes = (int)x_bytes;
  a.y_bytes = (int)(4 * x_bytes);
  const dim3 grid((unsigned)(n * a.nblk_c));
  const size_t lds = (size_t)32 * h * w * nch;
  // outputs of 8 MB and more stream out with non-temporal stores (measured
  // on 16 x 20x20x512 bf16: 18.1 -> 14.4 us; on one 10x10x512 map they cost
  // 0.6 us)
  const bool nt = 4 * x_bytes >= (8 << 20);
  switch (dtype) {
    case CONV_F32:
      if (nt) hipLaunchKernelGGL((spp_kernel<0, 2>), grid, dim3(256), lds, s, a);
      else hipLaunchKernelGGL((spp_kernel<0, 0>), grid, dim3(256), lds, s, a);
      break;
    case CONV_BF16:
      if (nt) hipLaunchKernelGGL((spp_kernel<1, 2>), grid, dim3(256), lds, s, a);
      else hipLaunchKernelGGL((spp_kernel<1, 0>), grid, dim3(256), lds, s, a);
      break;
    default:
      if (nt) hipLaunchKernelGGL((spp_kernel<2, 2>), grid, dim3(256), lds, s, a);
      else hipLaunchKernelGGL((spp_kernel<2, 0>), grid, dim3(256), lds, s, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace convnhwc
