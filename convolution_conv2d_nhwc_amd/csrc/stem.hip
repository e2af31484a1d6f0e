// stem.hip -- the first convolution of a bf16 network on an input whose
// pixels are padded to 8 channels (16 bytes): 3x3, stride 1, at most 8 real
// input channels (the 640x640 mosaic canvas: 3 colour channels, padded by
// the mosaic packer), fused bias + activation (+ residual) epilogue.
//
// The small-K kernel (smallk.hip) gathers every tap of every pixel from
// global memory with per-element address arithmetic; on the 640x640 stem
// that arithmetic, not the bytes, sets its time. With 16-byte pixels a
// workgroup instead copies its output patch's input window (6 x 66 pixels
// for 4 x 64 outputs) straight into LDS (`buffer_load ... lds`, one 16-byte
// pixel per lane, whole rows per instruction), and each MFMA B fragment is
// 16 lanes reading 16 consecutive window pixels at one tap: K = 9 taps x 8
// channel slots, in three K-steps of four taps (tap slots 10 to 12 and the
// channels past c_in are masked to zero, so whatever the pad channels hold
// never reaches a sum). Each lane loads its six A fragments (the weights of
// the workgroup's 32 output channels) once.
//
//   * workgroup: 4 waves, output patch of 4 rows x 64 columns; wave w owns
//     row w: 4 fragments of 16 pixels x 2 of 16 channels (v_mfma_f32_16x16x32_bf16,
//     A = weights, rows = channels; B = pixels, as in igemm.hip);
//   * two patches per workgroup, both windows copied at once (800
//     workgroups for the 640x640 stem: at the kernel's four waves per SIMD
//     all are resident in one round); the time left is the epilogue (Mish
//     on 32 outputs per lane per patch) and the 64-byte output pixels.
#include "igemm_common.h"

namespace convnhwc {

namespace {

constexpr int kSR = 4, kSC = 64;                 // output patch
constexpr int kWR = kSR + 2, kWC = kSC + 2;      // input window (3x3, stride 1)
constexpr int kWinPx = kWR * kWC;                // 396 pixels
constexpr int kWinGroups = (kWinPx + 63) / 64;   // 1 KiB copies: 7
constexpr int kStemTco = 32;                     // output channels per workgroup
#ifndef STEM_WG_PER_CU
#define STEM_WG_PER_CU 2
#endif

struct StemArgs {
  const char* x;
  const char* w;
  void* y;
  Epi e;
  Geometry g;
  int x_bytes;
  int w_bytes;
  int npr, npc;  // patches per image: rows, columns
  int npatch;    // n * npr * npc
  // MOS: the input is the four-tile mosaic of each canvas, tiles
  // [4 n][th][tw][c] (A top-left, B top-right, C bottom-left, D
  // bottom-right), read and rounded to bf16 here instead of a packed canvas
  int th, tw;
};

__device__ __forceinline__ void dma16_lds(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, (int)voff, 0, 0, 0);
}

// MOS 0: x is the canvas padded to 16-byte pixels, copied into LDS;
// MOS 1 / 2: x is the mosaic's fp32 / bf16 tiles, each window pixel gathered
// from its tile, rounded to bf16 (as the mosaic packer rounds) and written
// into LDS zero-padded to 16 bytes.
template <int MOS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MOS ? 3 : 4))) void stem_window_kernel(StemArgs a) {
  __shared__ __attribute__((aligned(1024))) char win[2][kWinGroups * 1024];

  const Geometry g = a.g;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int per_img = a.npr * a.npc;
  const int co0 = blockIdx.y * kStemTco;
  // patch p: image n, output rows r0 .., columns c0 ..
  auto origin = [&](int p, int& n, int& r0, int& c0) {
    n = p / per_img;
    const int rem = p - n * per_img;
    const int rb = rem / a.npc;
    r0 = rb * kSR;
    c0 = (rem - rb * a.npc) * kSC;
  };

  // Start the copy of patch p's window into win[buf]. MOS 0: group k (wave k
  // and wave k + 4) covers window pixels 64 k .. 64 k + 63, lane l pixel
  // 64 k + l (rows of kWC pixels), copied straight into LDS. MOS 1 / 2: this
  // thread's pixels tid and tid + 256 are gathered from their tiles into
  // `pre` (raw fp32 / bf16 bits; zero outside the image and past c_in), and
  // land() writes them into LDS.
  const __amdgpu_buffer_rsrc_t rx = rsrc(a.x, a.x_bytes);
  uint32_t pre[2][8];
  auto issue = [&](int p, int buf) {
    int n, r0, c0;
    origin(p, n, r0, c0);
    const int hi0 = r0 - g.ph, wi0 = c0 - g.pw;
    if constexpr (MOS == 0) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int k = wave + 4 * i;
        if (k < kWinGroups) {
          const int q = 64 * k + lane;
          const int hr = q / kWC, hc = q - hr * kWC;
          const int hi = hi0 + hr, wi = wi0 + hc;
          const bool ok = q < kWinPx && (unsigned)hi < (unsigned)g.h && (unsigned)wi < (unsigned)g.w;
          dma16_lds(rx, win[buf] + k * 1024, ok ? (uint32_t)(((n * g.h + hi) * g.w + wi) * 16) : kOOB);
        }
      }
    } else {
      constexpr int ESZ_IN = MOS == 1 ? 4 : 2;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int q = tid + 256 * i;
        const int hr = q / kWC, hc = q - hr * kWC;
        const int hi = hi0 + hr, wi = wi0 + hc;
        const bool ok = q < kWinPx && (unsigned)hi < (unsigned)g.h && (unsigned)wi < (unsigned)g.w;
        const int qy = hi >= a.th, qx = wi >= a.tw;
        const int src = (((4 * n + 2 * qy + qx) * a.th + hi - qy * a.th) * a.tw + wi - qx * a.tw) * g.c;
#pragma unroll
        for (int ci = 0; ci < 8; ++ci) {
          pre[i][ci] = 0;
          if (ci < g.c) {
            const uint32_t off = ok ? (uint32_t)(src + ci) * ESZ_IN : kOOB;
            if constexpr (MOS == 1)
              pre[i][ci] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rx, off, 0, 0);
            else
              pre[i][ci] = bload_elem<2>(rx, off);
          }
        }
      }
    }
  };
  // MOS 1 / 2: the gathered pixels, rounded to bf16 (as the mosaic packer
  // rounds), into win[buf], zero-padded to 16 bytes
  auto land = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = tid + 256 * i;
      if (q < kWinPx) {
        uint32_t h[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          h[k] = MOS == 1 ? bf16x2_bits(__builtin_bit_cast(float, pre[i][2 * k]), __builtin_bit_cast(float, pre[i][2 * k + 1]))
                          : pre[i][2 * k] | (pre[i][2 * k + 1] << 16);
        *reinterpret_cast<u32x4*>(win[buf] + q * 16) = u32x4{h[0], h[1], h[2], h[3]};
      }
    }
  };

  // Patches blockIdx.x, + gridDim.x, ... (the host makes the grid no larger
  // than the patch count); the next patch's window is copied while the
  // current one is computed.
  int p = blockIdx.x;
  if (p >= a.npatch) return;
  issue(p, 0);

  // A fragments: wa[ks][i] = channel row co0 + 16 i + (lane & 15), tap
  // 4 ks + (lane >> 4), its 8 channel slots (zero past c_in and past tap 8),
  // element by element from the OHWI weights (a tap's c_in values need not
  // be 4-byte aligned); the loop over slots stops at c_in (uniform)
  const int q = lane >> 4;
  i32x4 wa[3][2];
  {
    const __amdgpu_buffer_rsrc_t rw = rsrc(a.w, a.w_bytes);
#pragma unroll
    for (int ks = 0; ks < 3; ++ks)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int tap = 4 * ks + q;
        const int co = co0 + 16 * i + (lane & 15);
        const bool ok = tap < 9 && co < g.cout;
        const uint32_t base = (uint32_t)((co * 9 + tap) * g.c) * 2;
        uint32_t h[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int ci = 0; ci < 8; ++ci)
          if (ci < g.c) h[ci] = bload_elem<2>(rw, ok ? base + 2 * ci : kOOB);
        wa[ks][i] = i32x4{(int)(h[0] | (h[1] << 16)), (int)(h[2] | (h[3] << 16)), (int)(h[4] | (h[5] << 16)),
                          (int)(h[6] | (h[7] << 16))};
      }
  }
  // B masks: the channel slots c_in .. 7 of an input pixel read as zero
  // (tap slots past the ninth: all zero). The mosaic modes write those slots
  // as zeros into LDS, so only the tap mask remains.
  uint32_t bmask[4], bmask2[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    bmask[d] = MOS != 0 || 2 * d < g.c ? 0xffffu : 0u;
    bmask[d] |= MOS != 0 || 2 * d + 1 < g.c ? 0xffff0000u : 0u;
    bmask2[d] = 8 + q < 9 ? bmask[d] : 0u;
  }
  // the bias is the accumulators' starting value
  const QuadConsts qb0 = load_quad_consts_t<2>(a.e, co0 + 4 * q, g.cout);
  const QuadConsts qb1 = load_quad_consts_t<2>(a.e, co0 + 16 + 4 * q, g.cout);
  if constexpr (MOS != 0) land(0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // B: lane (q, p = lane & 15) of fragment j reads window pixel (wave + kh,
  // 16 j + p + kw) for its tap (taps past the ninth read tap 8's pixel and
  // are masked to zero)
  typedef f32x4 acc_t;
  const int pbase = (wave * kWC + (lane & 15)) * 16;
  const OutRef o = out_ref(a.y, g.m, g.cout, 2, a.e.res);
  for (int it = 0; p < a.npatch; p += gridDim.x, ++it) {
    const int buf = it & 1;
    const int pn = p + gridDim.x;
    const bool more = pn < a.npatch;  // uniform
    // win[buf ^ 1] was last read before the previous iteration's barrier
    if (more) issue(pn, buf ^ 1);
    int n, r0, c0;
    origin(p, n, r0, c0);
    acc_t acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const QuadConsts& qb = i ? qb1 : qb0;
        acc[i][j] = acc_t{qb.bsf[0], qb.bsf[1], qb.bsf[2], qb.bsf[3]};
      }
#pragma unroll
    for (int ks = 0; ks < 3; ++ks) {
      const int tap = min(4 * ks + q, 8);
      const int kh = tap / 3, kw = tap - 3 * (tap / 3);
      const int off = pbase + (kh * kWC + kw) * 16;
      const uint32_t* const mk = ks == 2 ? bmask2 : bmask;  // taps 0-7 always exist
      const bool masked = MOS == 0 || ks == 2;
      i32x4 bf[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const i32x4 r = *reinterpret_cast<const i32x4*>(win[buf] + off + j * 256);
#pragma unroll
        for (int d = 0; d < 4; ++d) bf[j][d] = masked ? (int)((uint32_t)r[d] & mk[d]) : r[d];
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = Mfma<2>::run(wa[ks][i], bf[j], acc[i][j]);
    }

    // epilogue: channels co0 + 16 i + 4 (lane >> 4) .. +3 of pixel (r0 +
    // wave, c0 + 16 j + (lane & 15)): act(acc) [+ residual], bf16, one 8-byte
    // store per quad (the bias is already in acc). Every quad is computed
    // before the next window is landed and before any store, so the window
    // copy has the MFMAs and the activations to complete. (Restaging the
    // tile through LDS so that every store is a 16-byte piece of a 1 KiB run
    // measured no faster.)
    const int r = r0 + wave;
    // quad (j, i) of this lane lies at byte offset base + soff(j, i) in y
    // (soff uniform); a quad outside y goes to an offset past every tensor
    const int base = (((n * g.ho + r) * g.wo + c0 + (lane & 15)) * g.cout + co0 + 4 * q) * 2;
    auto soff = [&](int j, int i) { return (16 * j * g.cout + 16 * i) * 2; };
    auto voff = [&](int j, int i) {
      const bool in = r < g.ho && c0 + 16 * j + (lane & 15) < g.wo && co0 + 16 * i + 4 * q < g.cout;
      return in ? (uint32_t)base : kOOB;
    };
    u32x2 d[4][2];
    with_epilogue<2>(OUT_BF16, a.e.act, [&](auto, auto ac) {
      constexpr int ACT = decltype(ac)::value;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          float f[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) f[e] = act_t<ACT>(acc[i][j][e]);
          if (o.has_res) {
            const u32x2 rv = __builtin_amdgcn_raw_buffer_load_b64(o.rr, voff(j, i), soff(j, i), 0);
#pragma unroll
            for (int e = 0; e < 4; ++e) f[e] += bf16_bits_to_f32((e & 1) ? (rv[e >> 1] >> 16) : (rv[e >> 1] & 0xffffu));
          }
          d[j][i] = u32x2{bf16x2_bits(f[0], f[1]), bf16x2_bits(f[2], f[3])};
        }
      }
    });
    if constexpr (MOS != 0) {
      if (more) land(buf ^ 1);
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the next window has landed
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 2; ++i) __builtin_amdgcn_raw_buffer_store_b64(d[j][i], o.r, voff(j, i), soff(j, i), 0);
    // the next window is visible to every wave, and win[buf] is free
    __syncthreads();
  }
  // no copy into LDS is left in flight when the workgroup ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

}  // namespace

bool stem_eligible(const conv_desc& d, const Geometry& g, int64_t x_stride) {
  return d.dtype == CONV_BF16 && d.out_dtype == CONV_BF16 && d.groups == 1 && g.kh == 3 && g.kw == 3 && g.sh == 1 &&
         g.sw == 1 && g.c <= 8 && x_stride == 8 && g.ph <= 1 && g.pw <= 1 && (g.cout & 3) == 0;
}

bool stem_mosaic_ok(const conv_plan* p, int64_t th, int64_t tw) {
  return p->path == PATH_STEM && th > 0 && tw > 0 && p->g.h == 2 * th && p->g.w == 2 * tw;
}

// Persistent grid: STEM_WG_PER_CU workgroups per CU for each 32-channel
// tile, at most one per patch.
int stem_grid(const conv_plan* p) {
  const int npatch = p->g.n * ((p->g.ho + kSR - 1) / kSR) * ((p->g.wo + kSC - 1) / kSC);
  const int nct = (p->g.cout + kStemTco - 1) / kStemTco;
  return std::max(1, std::min(npatch, STEM_WG_PER_CU * p->cus / nct));
}

hipError_t launch_stem(const conv_plan* p, const void* x, const void* w, const Epi& e, void* y, hipStream_t s) {
  StemArgs a;
  a.x = static_cast<const char*>(x);
  a.w = static_cast<const char*>(w);
  a.y = y;
  a.e = e;
  a.g = p->g;
  a.x_bytes = (int)p->x_bytes;
  a.w_bytes = (int)p->w_bytes;
  a.npr = (p->g.ho + kSR - 1) / kSR;
  a.npc = (p->g.wo + kSC - 1) / kSC;
  a.npatch = p->g.n * a.npr * a.npc;
  a.th = a.tw = 0;
  const dim3 grid(stem_grid(p), (p->g.cout + kStemTco - 1) / kStemTco);
  hipLaunchKernelGGL(stem_window_kernel<0>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_stem_mosaic(const conv_plan* p, const void* tiles, int tiles_f32, int th, int tw, const void* w,
                              const Epi& e, void* y, hipStream_t s) {
  StemArgs a;
  a.x = static_cast<const char*>(tiles);
  a.w = static_cast<const char*>(w);
  a.y = y;
  a.e = e;
  a.g = p->g;
  a.x_bytes = (int)((int64_t)4 * p->g.n * th * tw * p->g.c * (tiles_f32 ? 4 : 2));
  a.w_bytes = (int)p->w_bytes;
  a.npr = (p->g.ho + kSR - 1) / kSR;
  a.npc = (p->g.wo + kSC - 1) / kSC;
  a.npatch = p->g.n * a.npr * a.npc;
  a.th = th;
  a.tw = tw;
  const dim3 grid(stem_grid(p), (p->g.cout + kStemTco - 1) / kStemTco);
  if (tiles_f32)
    hipLaunchKernelGGL(stem_window_kernel<1>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(stem_window_kernel<2>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace convnhwc
