// igemm_ws.hip -- weight-stationary implicit GEMM for short reductions
// (K * elem_size <= 256 bytes: the 1x1 layers over up to 128 bf16 / 256 int8
// channels), NHWC activations, OHWI weights, fused epilogue.
//
// On such layers the output-stationary kernel (igemm.hip) streams both
// operands of every 64x64 tile through LDS, and its time goes to that
// traffic: per 128-byte K-tile a workgroup loads 16 KiB through the vector
// memory path, writes 16 KiB to LDS and reads 32 KiB back, for 32 MFMAs.
// Here a workgroup keeps the weights of its 64 output channels in registers
// for the whole reduction (each wave: its 32 channels x K, as MFMA A
// fragments, loaded once) and walks pixel tiles with a grid stride; only the
// activations go through LDS (8 KiB loaded and written, 16 KiB read per
// K-tile), so the bytes per MFMA on each path are halved. This is the
// weight-stationary schedule of the three TSO compares (tensor slicing and
// tiling for multicore NPUs, dataflow discussion); it pays here because the
// reduction is short enough for a wave's weights to fit its registers.
//
// Measured on MI355X (640x640 stack, N=1): the 1x1 layers gain (320x320
// 64 -> 64: 8.6 -> 7.4 us; 160x160 128 -> 64: 3.7 -> 3.1 us); the 3x3 layers
// over 64 channels (1152-byte reductions, 220 registers, two waves per SIMD)
// lose against the output-stationary kernel's five (29 against 21 us), so
// the kernel is limited to reductions of at most 256 bytes.
//
//   * workgroup: 4 wave64s as 2 (channels) x 2 (pixels), tile 64 x 64, each
//     wave a 32 x 32 block: 2 x 2 fragments of v_mfma_f32_16x16x32_bf16 /
//     v_mfma_i32_16x16x64_i8, the same operand layout as igemm.hip;
//   * A: af[i][s] = 16 bytes of K (K-step s, lane group l/16) of channel
//     row (lane & 15) of fragment i, straight from global memory;
//   * B: the 64 pixel rows of each K-tile through two LDS buffers with the
//     XOR-swizzled 128-byte rows of igemm.hip, loaded by the same `tap`,
//     `1x1` and `vec16` gathers; the first K-tile of the next pixel tile is
//     loaded while the current one is stored;
//   * the K-tile loop is unrolled (KS, the K-steps of 64 bytes: 2 or 4, is a
//     template argument), so the weight fragments are indexed statically.
#include "igemm_common.h"

namespace convnhwc {
namespace {

struct WsArgs {
  const char* x;
  const char* w;
  void* y;
  Epi e;
  Geometry g;
  int out_kind;
  int x_bytes;
  int w_bytes;
  float rcp_c;   // 1.0f / Cin
  float rcp_kw;  // 1.0f / KW
  int x_shift;   // LOAD_TAP: bytes the x descriptor starts before x
  int npx_tiles; // ceil(m / 64)
};

// Two waves per SIMD: the register allocator keeps the weights, the
// accumulators and two B stages within 256 VGPRs.
template <int ESZ, int LOADER, int KS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void igemm_ws_kernel(WsArgs a) {
  constexpr int TCO = 64, TPX = 64, FCO = 2, FPX = 2, BCH = TPX / 32;
  constexpr int NKT = (KS + 1) / 2;  // K-tiles of 128 bytes
  constexpr int VE = 16 / ESZ;
  constexpr int BKE = kBKB / ESZ;
  static_assert(LOADER != LOAD_GENERIC, "16-byte loaders only");
  typedef typename Mfma<ESZ>::acc_t acc_t;

  __shared__ __attribute__((aligned(16))) char Bs[2 * TPX * kBKB];

  const Geometry g = a.g;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wco = wave >> 1, wpx = wave & 1;
  const int co0 = blockIdx.y * TCO;
  const int kbytes = g.k * ESZ;
  const int nkt = (kbytes + kBKB - 1) / kBKB;  // <= NKT
  const int cbytes = g.c * ESZ;
  const int hw_o = g.ho * g.wo;
  const __amdgpu_buffer_rsrc_t rx = rsrc(a.x, a.x_bytes);
  const __amdgpu_buffer_rsrc_t rw = rsrc(a.w, a.w_bytes);
  const __amdgpu_buffer_rsrc_t rxt = LOADER == LOAD_TAP ? rsrc(a.x - a.x_shift, a.x_bytes + a.x_shift) : rx;

  // ---- this wave's weights: channels co0 + 32 wco + 16 i + (lane & 15)
  i32x4 af[FCO][KS];
#pragma unroll
  for (int i = 0; i < FCO; ++i) {
    const int co = co0 + 32 * wco + 16 * i + (lane & 15);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int kb = 64 * s + 16 * (lane >> 4);
      af[i][s] = bload16(rw, (co < g.cout && kb < kbytes) ? (uint32_t)(co * kbytes + kb) : kOOB);
    }
  }

  // ---- per pixel tile: the gather state of this thread's B rows
  // (row (tid >> 3) + 32 j, 16-byte column tid & 7)
  const int c16 = (tid & 7) * 16;
  int b_base[BCH], b_hi0[BCH], b_wi0[BCH];
  uint32_t voff_b[BCH], tmask[BCH];
  auto setup_rows = [&](int px0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < BCH; ++j) {
      const int p = px0 + (tid >> 3) + 32 * j;
      b_base[j] = 0;
      b_hi0[j] = -0x40000000;  // every bounds test fails
      b_wi0[j] = 0;
      if (p < g.m) {
        const int n = p / hw_o;
        const int r = p - n * hw_o;
        const int ho = r / g.wo;
        const int wo = r - ho * g.wo;
        if constexpr (LOADER == LOAD_1X1) {
          b_base[j] = p * g.c;
          b_hi0[j] = 0;
        } else {
          b_hi0[j] = ho * g.sh - g.ph;
          b_wi0[j] = wo * g.sw - g.pw;
          b_base[j] = ((n * g.h + b_hi0[j]) * g.w + b_wi0[j]) * g.c;
        }
      }
      if constexpr (LOADER == LOAD_TAP) {
        voff_b[j] = (uint32_t)(b_base[j] * ESZ + a.x_shift + c16);
        uint32_t m = 0;
        for (int kh = 0, tap = 0; kh < g.kh; ++kh)
          for (int kw = 0; kw < g.kw; ++kw, ++tap) {
            const int hi = b_hi0[j] + kh, wi = b_wi0[j] + kw;
            if ((unsigned)hi < (unsigned)g.h && (unsigned)wi < (unsigned)g.w) m |= 1u << tap;
          }
        tmask[j] = m;
      } else if constexpr (LOADER == LOAD_1X1) {
        voff_b[j] = b_hi0[j] == 0 ? (uint32_t)(b_base[j] * ESZ + c16) : kOOB;
      }
    }
  };
  // the B chunks of K-tile kt (zero past K or outside the image)
  auto fetch = [&](int kt, i32x4 (&rb)[BCH]) __attribute__((always_inline)) {
    const int kb0 = kt * kBKB;
    if constexpr (LOADER == LOAD_TAP) {
      // Cin * ESZ % 128 == 0: the K-tile is one 128-byte channel block of one tap
      const bool live = kt < nkt;
      const int tap = kb0 / cbytes;
      const int cb = kb0 - tap * cbytes;
      const int kh = tap / g.kw, kw = tap - kh * g.kw;
      const int soff = (kh * g.w + kw) * cbytes + cb;
#pragma unroll
      for (int j = 0; j < BCH; ++j) {
        const bool ok = live && ((tmask[j] >> (tap & 31)) & 1u);
        rb[j] = bload16s(rxt, ok ? voff_b[j] : kOOB, ok ? soff : 0);
      }
    } else if constexpr (LOADER == LOAD_1X1) {
      const bool cin_ok = c16 < cbytes - kb0;
#pragma unroll
      for (int j = 0; j < BCH; ++j) rb[j] = bload16s(rx, cin_ok ? voff_b[j] : kOOB, cin_ok ? kb0 : 0);
    } else {
      const int kc = kt * BKE + (tid & 7) * VE;  // first element of this thread's chunk
      int tap, ci, kh, kw;
      divmod_small(kc, g.c, a.rcp_c, tap, ci);
      divmod_small(tap, g.kw, a.rcp_kw, kh, kw);
      const int tap_off = (kh * g.w + kw) * g.c + ci;
      const bool khin = kc < g.k;
#pragma unroll
      for (int j = 0; j < BCH; ++j) {
        const int hi = b_hi0[j] + kh;
        const int wi = b_wi0[j] + kw;
        const bool ok = khin && (unsigned)hi < (unsigned)g.h && (unsigned)wi < (unsigned)g.w;
        rb[j] = bload16(rx, ok ? (uint32_t)(b_base[j] + tap_off) * ESZ : kOOB);
      }
    }
  };
  auto stash = [&](int buf, const i32x4 (&rb)[BCH]) __attribute__((always_inline)) {
    char* B = Bs + buf * TPX * kBKB;
#pragma unroll
    for (int j = 0; j < BCH; ++j) *reinterpret_cast<i32x4*>(B + lds_off((tid >> 3) + 32 * j, tid & 7)) = rb[j];
  };

  const int b_row0 = wpx * 32 + (lane & 15);
  const int co_w = co0 + 32 * wco + 4 * (lane >> 4);
  const OutRef o = out_ref(a.y, g.m, g.cout, ESZ == 2 ? 2 : (a.out_kind == OUT_I32 ? 4 : 1), a.e.res);
  QuadConsts qc[FCO];
  if ((g.cout & 3) == 0) {
#pragma unroll
    for (int i = 0; i < FCO; ++i) qc[i] = load_quad_consts_t<ESZ>(a.e, co_w + 16 * i, g.cout);
  } else {
#pragma unroll
    for (int i = 0; i < FCO; ++i) qc[i] = load_quad_consts<ESZ>(a.e, co_w + 16 * i, g.cout);
  }

  // K-tiles 0 and 1 of a pixel tile are fetched before it starts (for the
  // next tile: while the current one is stored)
  int pt = blockIdx.x;
  i32x4 r0[BCH], r1[BCH];
  if (pt < a.npx_tiles) {
    setup_rows(pt * TPX);
    fetch(0, r0);
    if (NKT > 1) fetch(1, r1);
  }
  for (; pt < a.npx_tiles; pt += gridDim.x) {
    const int px0 = pt * TPX;
    // every wave is done with both buffers of the previous tile
    __syncthreads();
    stash(0, r0);
    acc_t acc[FCO][FPX];
#pragma unroll
    for (int i = 0; i < FCO; ++i)
#pragma unroll
      for (int j = 0; j < FPX; ++j) acc[i][j] = acc_t{0, 0, 0, 0};
    // K-tile kt sits in buffer kt & 1; tile kt + 1 (registers r1) is written
    // into the other buffer after this tile's first K-step, then r1 is
    // re-issued for tile kt + 2
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      if (kt < nkt) {
        __syncthreads();
        const char* B = Bs + (kt & 1) * TPX * kBKB;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          if (2 * kt + s < KS) {
            const int c = 4 * s + (lane >> 4);
            i32x4 bf[FPX];
#pragma unroll
            for (int j = 0; j < FPX; ++j) bf[j] = *reinterpret_cast<const i32x4*>(B + lds_off(b_row0 + 16 * j, c));
            if (s == 0 && kt + 1 < nkt) {
              stash((kt + 1) & 1, r1);
              if (kt + 2 < nkt) fetch(kt + 2, r1);
            }
#pragma unroll
            for (int i = 0; i < FCO; ++i)
#pragma unroll
              for (int j = 0; j < FPX; ++j) acc[i][j] = Mfma<ESZ>::run(af[i][2 * kt + s], bf[j], acc[i][j]);
          }
        }
      }
    }
    // the next pixel tile's first K-tile is in flight during the stores
    const int pn = pt + gridDim.x;
    if (pn < a.npx_tiles) {
      setup_rows(pn * TPX);
      fetch(0, r0);
      if (NKT > 1) fetch(1, r1);
    }

    // ---- fused epilogue
    const int px_w = px0 + wpx * 32 + (lane & 15);
    if ((g.cout & 3) == 0) {
      with_epilogue<ESZ>(a.out_kind, a.e.act, [&](auto oc, auto ac) {
        constexpr int OUT = decltype(oc)::value, ACT = decltype(ac)::value;
#pragma unroll
        for (int i = 0; i < FCO; ++i)
#pragma unroll
          for (int j = 0; j < FPX; ++j) store_quad_t<ESZ, OUT, ACT>(acc[i][j], qc[i], co_w + 16 * i, px_w + 16 * j, o);
      });
    } else {
#pragma unroll
      for (int i = 0; i < FCO; ++i) {
        const int co = co_w + 16 * i;
        if (co >= g.cout) continue;
#pragma unroll
        for (int j = 0; j < FPX; ++j) {
          const int px = px_w + 16 * j;
          if (px < g.m) store_quad<ESZ>(acc[i][j], qc[i], co, px, g.cout, a.out_kind, a.e.act, a.y, a.e.res);
        }
      }
    }
  }
}

template <int ESZ, int LOADER>
hipError_t launch_ks(int ks, const WsArgs& args, dim3 grid, hipStream_t s) {
  switch (ks) {
    case 2: hipLaunchKernelGGL((igemm_ws_kernel<ESZ, LOADER, 2>), grid, dim3(256), 0, s, args); break;
    default: hipLaunchKernelGGL((igemm_ws_kernel<ESZ, LOADER, 4>), grid, dim3(256), 0, s, args); break;
  }
  return hipGetLastError();
}

template <int ESZ>
hipError_t launch_loader(int loader, int ks, const WsArgs& args, dim3 grid, hipStream_t s) {
  switch (loader) {
    case LOAD_TAP: return launch_ks<ESZ, LOAD_TAP>(ks, args, grid, s);
    case LOAD_1X1: return launch_ks<ESZ, LOAD_1X1>(ks, args, grid, s);
    default: return launch_ks<ESZ, LOAD_VEC>(ks, args, grid, s);
  }
}

}  // namespace

// K-steps of 64 bytes the weight registers hold (2 or 4), or 0 when the
// layer does not take the weight-stationary kernel.
int ws_ksteps(const Geometry& g, int esz, int loader) {
  if (loader == LOAD_GENERIC) return 0;
  const int steps = (g.k * esz + 63) / 64;
  return steps <= 2 ? 2 : steps <= 4 ? 4 : 0;
}

// Workgroups along the pixel tiles: two per CU (the weight registers allow
// two waves per SIMD), shared by the channel tiles.
int ws_grid_x(const conv_plan* p) {
  const int npx = (p->g.m + 63) / 64;
  const int nco = (p->g.cout + 63) / 64;
  const int slots = 2 * p->cus;
  const int per = std::max(1, slots / nco);
  return std::min(npx, per);
}

hipError_t launch_ws(const conv_plan* p, const void* x, const void* w, const Epi& e, void* y, hipStream_t s) {
  WsArgs args;
  args.x = static_cast<const char*>(x);
  args.w = static_cast<const char*>(w);
  args.y = y;
  args.e = e;
  args.g = p->g;
  args.out_kind = p->out_kind;
  args.x_bytes = (int)p->x_bytes;
  args.w_bytes = (int)p->w_bytes;
  args.rcp_c = 1.0f / (float)p->g.c;
  args.rcp_kw = 1.0f / (float)p->g.kw;
  args.x_shift = (p->g.ph * p->g.w + p->g.pw) * p->g.c * p->in_esz;
  args.npx_tiles = (p->g.m + 63) / 64;
  const dim3 grid(ws_grid_x(p), (p->g.cout + 63) / 64);
  const int ks = ws_ksteps(p->g, p->in_esz, p->loader);
  return p->in_esz == 2 ? launch_loader<2>(p->loader, ks, args, grid, s)
                        : launch_loader<1>(p->loader, ks, args, grid, s);
}

}  // namespace convnhwc
