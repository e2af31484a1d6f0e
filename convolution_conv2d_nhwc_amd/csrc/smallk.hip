// smallk.hip -- convolution with a short reduction (KH*KW*Cin*elem_size <= 128
// bytes) and a channel count that does not fill 16-byte vectors: the stems of
// the workloads (3x3 on 3-channel images, the 10x4 keyword-spotting stem on a
// 1-channel spectrogram).
//
// Such a layer is one or a few MFMA K-steps per output tile, so staging tiles
// through LDS buys nothing: every wave builds its MFMA operands straight from
// global memory and needs no barrier.
//   * A (weights): each lane gathers its 16 bytes of K for the output channels
//     of its fragment rows once, at the start, and keeps them in registers.
//   * B (pixels): for each 64-pixel tile, lane l gathers, for the pixel
//     (l % 16) of each of the four 16-pixel fragments, the K elements
//     8*(l/16) .. (16 for int8) of its receptive field. The decomposition of
//     those K indices into (kh, kw, ci) depends only on the lane, so it is
//     done once; each element is a buffer load whose offset is forced out of
//     range (reads 0) outside the image or past K. All loads of a tile are
//     issued before any is used.
//   * Waves walk the 64-pixel tiles with a grid stride, at most four
//     workgroups per CU, so that the set-up above serves several tiles.
//   * Such a layer is bound by instruction issue, not by memory: on the
//     640x640x3 -> 32 stem (bf16, Mish) the wave-level VALU instructions
//     alone (about 7 M, four cycles each on a 16-lane SIMD: ~12 us) are
//     more than half of the kernel's time, most of them in the epilogue.
//     Staging the input rows in LDS with 16-byte loads, tried in place of
//     the element gathers, measured no faster (20.3 against 19.8 us).
// The output quads go through the same fused epilogue as the implicit GEMM.
#include <algorithm>

#include "device_common.h"
#include "mfma_epilogue.h"
#include "plan.h"

namespace convnhwc {
namespace {

constexpr uint32_t kOOB = 0x80000000u;

struct SkArgs {
  const char* x;
  const char* w;
  void* y;
  Epi e;
  Geometry g;
  int out_kind;
  int x_bytes;
  int w_bytes;
  float rcp_c;
  float rcp_kw;
  float rcp_wo;
  float rcp_ho;
  int npx_tiles;  // ceil(m / 64)
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}

template <int ESZ>
__device__ __forceinline__ uint32_t bload_elem(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (ESZ == 2)
    return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
  else
    return __builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
}

__device__ __forceinline__ void divmod_small(int n, int d, float rcp_d, int& q, int& r) {
  q = (int)((float)n * rcp_d);
  r = n - q * d;
  if (r < 0) {
    --q;
    r += d;
  }
  if (r >= d) {
    ++q;
    r -= d;
  }
}

template <int ESZ, int VE>
__device__ __forceinline__ i32x4 pack16(const uint32_t (&v)[VE]) {
  uint32_t wd[4] = {0, 0, 0, 0};
#pragma unroll
  for (int e = 0; e < VE; ++e) wd[e * ESZ / 4] |= v[e] << (8 * ((e * ESZ) & 3));
  return i32x4{(int)wd[0], (int)wd[1], (int)wd[2], (int)wd[3]};
}

template <int ESZ>
struct Mfma;
template <>
struct Mfma<2> {
  typedef f32x4 acc_t;
  static __device__ __forceinline__ acc_t run(i32x4 a, i32x4 b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <>
struct Mfma<1> {
  typedef i32x4 acc_t;
  static __device__ __forceinline__ acc_t run(i32x4 a, i32x4 b, acc_t c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
  }
};

// FCO fragments of 16 output channels per wave; KS MFMA K-steps of 64 bytes.
template <int ESZ, int FCO, int KS>
__global__ __launch_bounds__(256) void smallk_kernel(SkArgs a) {
  constexpr int VE = 16 / ESZ;  // K elements per lane per step
  constexpr int KE = 64 / ESZ;  // K elements per step
  typedef typename Mfma<ESZ>::acc_t acc_t;
  const Geometry g = a.g;
  const int lane = threadIdx.x & 63;
  const int kg = lane >> 4;
  const int lr = lane & 15;
  const int co0 = blockIdx.y * (16 * FCO);
  const __amdgpu_buffer_rsrc_t rx = rsrc(a.x, a.x_bytes);
  const __amdgpu_buffer_rsrc_t rw = rsrc(a.w, a.w_bytes);

  // this lane's K indices: k = ks*KE + kg*VE + e -> (kh, kw, ci)
  int kofs[KS][VE], khs[KS][VE], kws[KS][VE];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      const int k = ks * KE + kg * VE + e;
      int tap, ci, kh, kw;
      divmod_small(k, g.c, a.rcp_c, tap, ci);
      divmod_small(tap, g.kw, a.rcp_kw, kh, kw);
      const bool kin = k < g.k;
      kofs[ks][e] = (kh * g.w + kw) * g.c + ci;
      khs[ks][e] = kin ? kh : -0x40000000;  // fails every bounds test
      kws[ks][e] = kw;
    }

  // weights of rows co0 + 16 i + lr
  i32x4 af[FCO][KS];
#pragma unroll
  for (int i = 0; i < FCO; ++i) {
    const int co = co0 + 16 * i + lr;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint32_t v[VE];
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        const int k = ks * KE + kg * VE + e;
        v[e] = bload_elem<ESZ>(rw, (co < g.cout && k < g.k) ? (uint32_t)(co * g.k + k) * ESZ : kOOB);
      }
      af[i][ks] = pack16<ESZ, VE>(v);
    }
  }

  QuadConsts q[FCO];
#pragma unroll
  for (int i = 0; i < FCO; ++i) q[i] = load_quad_consts<ESZ>(a.e, co0 + 16 * i + 4 * kg, g.cout);

  const int hw_o = g.ho * g.wo;
  const OutRef o = out_ref(a.y, g.m, g.cout, ESZ == 2 ? 2 : (a.out_kind == OUT_I32 ? 4 : 1), a.e.res);
  const int nwaves = gridDim.x * 4;
  // The K elements of the four 16-pixel fragments of 64-pixel tile pt. The
  // tile's first pixel is decomposed once (wave-uniform); the pixels of the
  // fragments follow by small divisions, exact here (< 2^24).
  auto gather = [&](int pt, uint32_t (&v)[4][KS][VE]) __attribute__((always_inline)) {
    const int pbase = __builtin_amdgcn_readfirstlane(pt) * 64;
    const int nb = pbase / hw_o;
    const int rb = pbase - nb * hw_o;
    const int hob = rb / g.wo;
    const int wob = rb - hob * g.wo;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int p = pbase + 16 * j + lr;
      int base = 0, hi0 = -0x40000000, wi0 = 0;
      if (p < g.m) {
        int q, wo, q2, ho;
        divmod_small(wob + 16 * j + lr, g.wo, a.rcp_wo, q, wo);
        divmod_small(hob + q, g.ho, a.rcp_ho, q2, ho);
        const int n = nb + q2;
        hi0 = ho * g.sh - g.ph;
        wi0 = wo * g.sw - g.pw;
        base = ((n * g.h + hi0) * g.w + wi0) * g.c;
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          const bool ok = (unsigned)(hi0 + khs[ks][e]) < (unsigned)g.h && (unsigned)(wi0 + kws[ks][e]) < (unsigned)g.w;
          v[j][ks][e] = bload_elem<ESZ>(rx, ok ? (uint32_t)(base + kofs[ks][e]) * ESZ : kOOB);
        }
    }
  };
  // Each wave walks its tiles. (Loading the next tile's elements while the
  // current one is multiplied and stored measured slower on the 640x640
  // stem, 19.4 against 18.5 us: the second set of registers costs waves.)
  int pt = blockIdx.x * 4 + (threadIdx.x >> 6);
  uint32_t v[4][KS][VE];
  for (; pt < a.npx_tiles; pt += nwaves) {
    const int pbase = pt * 64;
    gather(pt, v);
    acc_t acc[FCO][4];
#pragma unroll
    for (int i = 0; i < FCO; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = acc_t{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const i32x4 bf = pack16<ESZ, VE>(v[j][ks]);
#pragma unroll
        for (int i = 0; i < FCO; ++i) acc[i][j] = Mfma<ESZ>::run(af[i][ks], bf, acc[i][j]);
      }
    if ((g.cout & 3) == 0) {
      with_epilogue<ESZ>(a.out_kind, a.e.act, [&](auto oc, auto ac) {
        constexpr int OUT = decltype(oc)::value, ACT = decltype(ac)::value;
#pragma unroll
        for (int i = 0; i < FCO; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            store_quad_t<ESZ, OUT, ACT>(acc[i][j], q[i], co0 + 16 * i + 4 * kg, pbase + 16 * j + lr, o);
      });
      continue;
    }
#pragma unroll
    for (int i = 0; i < FCO; ++i) {
      const int co = co0 + 16 * i + 4 * kg;
      if (co >= g.cout) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int px = pbase + 16 * j + lr;
        if (px < g.m) store_quad<ESZ>(acc[i][j], q[i], co, px, g.cout, a.out_kind, a.e.act, a.y, a.e.res);
      }
    }
  }
}

template <int ESZ, int FCO>
hipError_t launch_fco(int ks, const SkArgs& args, dim3 grid, hipStream_t s) {
  switch (ks) {
    case 1: hipLaunchKernelGGL((smallk_kernel<ESZ, FCO, 1>), grid, dim3(256), 0, s, args); break;
    default: hipLaunchKernelGGL((smallk_kernel<ESZ, FCO, 2>), grid, dim3(256), 0, s, args); break;
  }
  return hipGetLastError();
}

template <int ESZ>
hipError_t launch_esz(int fco, int ks, const SkArgs& args, dim3 grid, hipStream_t s) {
  switch (fco) {
    case 1: return launch_fco<ESZ, 1>(ks, args, grid, s);
    case 2: return launch_fco<ESZ, 2>(ks, args, grid, s);
    default: return launch_fco<ESZ, 4>(ks, args, grid, s);
  }
}

}  // namespace

// Output-channel fragments per wave and K-steps of a small-K layer.
void smallk_shape(const Geometry& g, int esz, int* fco, int* ks) {
  const int f = (g.cout + 15) / 16;
  *fco = f <= 1 ? 1 : f <= 2 ? 2 : 4;
  *ks = (g.k * esz + 63) / 64;
}

hipError_t launch_smallk(const conv_plan* p, const void* x, const void* w, const Epi& e, void* y,
                         hipStream_t s) {
  SkArgs a;
  a.x = static_cast<const char*>(x);
  a.w = static_cast<const char*>(w);
  a.y = y;
  a.e = e;
  a.g = p->g;
  a.out_kind = p->out_kind;
  a.x_bytes = (int)p->x_bytes;
  a.w_bytes = (int)p->w_bytes;
  a.rcp_c = 1.0f / (float)p->g.c;
  a.rcp_kw = 1.0f / (float)p->g.kw;
  a.rcp_wo = 1.0f / (float)p->g.wo;
  a.rcp_ho = 1.0f / (float)p->g.ho;
  a.npx_tiles = (p->g.m + 63) / 64;
  int fco, ks;
  smallk_shape(p->g, p->in_esz, &fco, &ks);
  const int nco = (p->g.cout + 16 * fco - 1) / (16 * fco);
  // at most four workgroups (16 waves) per CU, each wave walking several
  // 64-pixel tiles (measured on the 640x640 stem: 18.9 us at four per CU
  // against 21.4 us at one tile per wave)
  const int wgs = std::min((a.npx_tiles + 3) / 4, 4 * p->cus);
  const dim3 grid(wgs, nco);
  if (p->in_esz == 2) return launch_esz<2>(fco, ks, a, grid, s);
  return launch_esz<1>(fco, ks, a, grid, s);
}

}  // namespace convnhwc
