// halo.hip -- 3x3 bf16 convolution over 32 or 64 input channels (stride 1 or
// 2) with the weights held in registers and the input read once per output
// patch: the "halo" kernel. NHWC activations, OHWI weights, fused epilogue,
// and optionally a following 1x1 layer applied before anything is stored.
//
// Why: on these layers (the 320x320 and 640x640 3x3 layers of the YOLO
// stack) the implicit-GEMM kernel gathers every input pixel once per tap
// (nine times) and the weights once per 64-pixel tile, each through a
// register round trip into LDS, one K-tile at a time; per 128-byte K-tile a
// workgroup moves 16 KiB for 32 MFMAs and its time is that traffic and its
// latency. Here:
//   * A workgroup owns TCO (64 or 128) output channels; each wave keeps its
//     32 channels' weights for all nine taps as MFMA A fragments in
//     registers, loaded once (the weight-stationary schedule of the three
//     TSO compares -- tensor slicing and tiling for multicore NPUs,
//     dataflow discussion -- which pays once nothing else has to stream).
//   * Output patches of 4 x 16 pixels are walked with a grid stride. A
//     patch's input window (6 x 18 pixels at stride 1, 9 x 33 at stride 2) is
//     copied from global memory straight into LDS (`buffer_load ... lds`, 16
//     bytes per lane, no registers), one 128-byte LDS row per input pixel,
//     and the nine taps read their B fragments from it at shifted rows: each
//     input pixel crosses the memory path about 1.7 (stride 1) or 4.6
//     (stride 2) times per output instead of nine.
//   * The next patch's window is loaded into the second buffer while the
//     current one is computed; one barrier per patch.
//
// LDS layout of a window: row = hr * HC + pos for input row hr and column
// position pos; at stride 2 the even input columns come first (pos = hc / 2)
// and the odd ones after them (pos = HCE + hc / 2), so the 16 output columns
// of a fragment read 16 consecutive rows at every tap. Chunk c (16 bytes,
// channels 8c .. 8c + 7) of a row sits at position c ^ (pos & 7): the 16
// rows a fragment reads are conflict-free and the DMA lane order (lane l
// writes byte 16 l of its 1 KiB group) realises the swizzle by choosing
// which chunk each lane fetches.
//
// Waves: 2 per 32 output channels (NW = TCO / 16 waves): wave w owns
// channels 32 (w >> 1) .. +31 and patch rows 2 (w & 1), 2 (w & 1) + 1 (two
// 16-pixel fragments). MFMA v_mfma_f32_16x16x32_bf16 with the operand layout
// of igemm.hip (A = weights, rows = channels; B = pixels), so per output the
// products are summed in the same order as the implicit-GEMM kernel (tap by
// tap, 32 channels per step) and the results are bit-identical to it.
//
// FU (fused 1x1): the patch's TCO x 64 outputs, bias + activation + bf16
// rounding as a store would do, go into the current window buffer (free once
// every wave is past its MFMAs) as the B operand of the 1x1 layer (at most
// 64 output channels, weights in registers); only that layer's output is
// stored.
#include <cstring>

#include "igemm_common.h"

namespace convnhwc {

namespace {

constexpr int kPR = 4, kPC = 16;  // output patch: 4 rows x 16 columns
#ifndef HALO_XR
#define HALO_XR 1
#endif

template <int S>
struct Win {
  static constexpr int HR = (kPR - 1) * S + 3;  // input rows of a window
  static constexpr int HC = (kPC - 1) * S + 3;  // input columns
  static constexpr int HCE = (HC + 1) / 2;      // stride 2: even columns first
  static constexpr int ROWS = HR * HC;          // LDS rows
};

struct HaloArgs {
  const char* x;
  const char* w;
  void* y;
  Epi e;
  Geometry g;
  int x_bytes;
  int w_bytes;
  int npr, npc;  // patches per image: rows, columns
  int npatch;    // n * npr * npc
  int gp;        // workgroups per channel tile
  int xr;        // 1: each XCD walks its own contiguous range of patches (gp % 8 == 0)
  // FU
  const char* w2;
  int w2_bytes;
  int cout2;
  Epi e2;
};

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, (int)voff, 0, 0, 0);
}

__device__ __forceinline__ void store_packed(const u32x2& d, int co, int px, const OutRef& o) {
  const bool in = px < o.m && co < o.cout;
  __builtin_amdgcn_raw_buffer_store_b64(d, o.r, in ? (uint32_t)(px * o.cout + co) * 2u : kOOB, 0, 0);
}

// S: stride; KS: K-steps of 32 channels per tap (1: 32 channels, 2: 64);
// TCO: output channels per workgroup; FU: fused 1x1 layer.
template <int S, int KS, int TCO, int FU>
__global__ __launch_bounds__(TCO * 4) __attribute__((amdgpu_waves_per_eu(2))) void halo_kernel(HaloArgs a) {
  typedef Win<S> W;
  constexpr int NW = TCO / 16;                        // waves
  constexpr int GROUPS = (W::ROWS + 7) / 8;           // 1 KiB DMA groups per window
  constexpr int NDMA = (GROUPS + NW - 1) / NW;        // per wave
  constexpr int BUF = NDMA * NW * 1024;               // bytes per window buffer
  constexpr int CB = 4 * KS;                          // 16-byte chunks per input pixel
  static_assert(FU == 0 || BUF >= kPR * kPC * TCO * 2, "window buffer holds the fused tile");
  static_assert(BUF >= NW * 2048, "window buffer holds the weight staging");
  // FU with 128 intermediate channels: the 1x1 layer's weights (64 x 128
  // bf16) live in LDS instead of registers
  constexpr bool WB_LDS = FU && TCO == 128;
  __shared__ __attribute__((aligned(1024))) char smem[2 * BUF + (WB_LDS ? 64 * TCO * 2 : 0)];

  const Geometry g = a.g;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cg = wave >> 1;  // channel group of 32
  const int pg = wave & 1;   // patch rows 2 pg, 2 pg + 1
  const int ct = blockIdx.x / a.gp;
  const int q0 = blockIdx.x - ct * a.gp;
  const int co0 = ct * TCO;
  const int cbytes = g.c * 2;
  const __amdgpu_buffer_rsrc_t rx = rsrc(a.x, a.x_bytes);
  const __amdgpu_buffer_rsrc_t rw = rsrc(a.w, a.w_bytes);

  // ---- the window copy: DMA slot i of this lane is LDS row 8 (wave + NW i)
  // + lane / 8, input pixel (hr, hc) of the window, chunk cc; d_rel[i] is the
  // byte offset of that chunk from the window's corner pixel (-1: a padding
  // row or a chunk past the channels)
  auto slot = [&](int i, int& hr, int& hc, int& cc) {
    const int row = 8 * (wave + NW * i) + (lane >> 3);
    const int pos = row % W::HC;
    hr = row / W::HC;
    cc = (lane & 7) ^ (pos & 7);
    hc = S == 1 ? pos : (pos < W::HCE ? 2 * pos : 2 * (pos - W::HCE) + 1);
    return row < W::ROWS && cc < CB && cc * 16 < cbytes;
  };
  int d_rel[NDMA];
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    int hr, hc, cc;
    const bool ok = slot(i, hr, hc, cc);
    d_rel[i] = ok ? (hr * g.w + hc) * cbytes + cc * 16 : -1;
  }
  auto patch_origin = [&](int p, int& n, int& r0, int& c0) {
    const int per_img = a.npr * a.npc;
    n = p / per_img;
    const int rem = p - n * per_img;
    const int rb = rem / a.npc;
    r0 = rb * kPR;
    c0 = (rem - rb * a.npc) * kPC;
  };
  // issue the window of patch p into buffer `buf` (a patch past the last
  // writes zeros: every wave issues exactly NDMA copies per patch); returns
  // the patch's origin, which the patch's epilogue uses later
  struct Origin {
    int n, r0, c0;
  };
  auto load_window = [&](int p, int buf) -> Origin {
    int n, r0, c0;
    patch_origin(p < a.npatch ? p : 0, n, r0, c0);
    const int hi0 = r0 * S - g.ph, wi0 = c0 * S - g.pw;
    const int base = ((n * g.h + hi0) * g.w + wi0) * cbytes;
    const bool live = p < a.npatch;
    const bool inside = hi0 >= 0 && wi0 >= 0 && hi0 + W::HR <= g.h && wi0 + W::HC <= g.w;
    char* dst = smem + buf * BUF;
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
      bool ok = live && d_rel[i] >= 0;
      if (!inside) {  // a border patch: test the pixel (recomputed, saves registers)
        int hr, hc, cc;
        slot(i, hr, hc, cc);
        ok = ok && (unsigned)(hi0 + hr) < (unsigned)g.h && (unsigned)(wi0 + hc) < (unsigned)g.w;
      }
      dma16(rx, dst + (wave + NW * i) * 1024, ok ? (uint32_t)(base + d_rel[i]) : kOOB);
    }
    return Origin{n, r0, c0};
  };

  // Patches of this workgroup: p_begin, p_begin + step, ... below p_end.
  // Workgroups go to the 8 XCDs round-robin by id; with xr, XCD x = q0 % 8
  // owns the contiguous range [x per, (x+1) per) of patches (per = npatch /
  // 8 rounded up) and its gp / 8 workgroups walk it together, so the window
  // rows that vertically and horizontally neighbouring patches share are
  // fetched through one L2. Otherwise the workgroups stride over all patches.
  int p_begin = q0, p_end = a.npatch, step = a.gp;
  if (a.xr) {
    const int per = (a.npatch + 7) >> 3;
    const int x = q0 & 7;
    step = a.gp >> 3;
    p_begin = x * per + (q0 >> 3);
    p_end = min(a.npatch, (x + 1) * per);
  }
  int p = p_begin;
  Origin cur = load_window(p < p_end ? p : a.npatch, 0);

  // ---- this wave's weights: wa[tap][ks][i] = channel row co0 + 32 cg + 16 i
  // + (lane & 15), channels 32 ks + 8 (lane >> 4) .. +7 of tap `tap` (the
  // MFMA A layout). Read in that layout, 16 consecutive lanes would touch 16
  // rows 1152 bytes apart. Instead each load has 8 consecutive lanes read
  // 128 contiguous bytes of one row (8 rows per load), and the rows go
  // through a 2 KiB slice of the second window buffer (free until the first
  // patch starts) per wave: written in the swizzled row layout, read back as
  // fragments. A row is NB 128-byte blocks: one tap each for 64 channels,
  // two taps each for 32.
  i32x4 wa[9][KS][2];
  {
    constexpr int NB = KS == 2 ? 9 : 5;
    const int kb = g.k * 2;  // bytes per weight row
    char* const stage = smem + BUF + wave * 2048;
    i32x4 raw[NB][2][2];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int co = co0 + 32 * cg + 16 * i + 8 * h + (lane >> 3);
          const int cb = 128 * b + 16 * (lane & 7);
          raw[b][i][h] = bload16(rw, (co < g.cout && cb < kb) ? (uint32_t)(co * kb + cb) : kOOB);
        }
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
          *reinterpret_cast<i32x4*>(stage + lds_off(8 * h + (lane >> 3), lane & 7)) = raw[b][i][h];
#pragma unroll
        for (int u = 0; u < 2; ++u) {  // KS 2: K-step u of tap b; KS 1: tap 2 b + u
          const int t = KS == 2 ? b : 2 * b + u;
          if (t < 9)
            wa[t][KS == 2 ? u : 0][i] = *reinterpret_cast<const i32x4*>(stage + lds_off(lane & 15, 4 * u + (lane >> 4)));
        }
      }
  }
  // FU: the 1x1 layer's weights, wave w: its output channels 32 (w & 1) +
  // 16 i + (lane & 15), K-step s = intermediate channels 32 s + 8 (lane >> 4)
  constexpr int KS2 = FU && !WB_LDS ? TCO / 32 : 1;
  i32x4 wb[2][KS2];
  char* const WB = smem + 2 * BUF;  // WB_LDS: block kt2 (channels 64 kt2 ..) of row c2 at kt2 * 8 KiB + lds_off(c2, .)
  if constexpr (WB_LDS) {
    const __amdgpu_buffer_rsrc_t rw2 = rsrc(a.w2, a.w2_bytes);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int q = tid + 512 * j;  // 64 rows x 16 chunks
      const int row = q >> 4, c16 = q & 15;
      const i32x4 v = bload16(rw2, row < a.cout2 ? (uint32_t)(row * TCO * 2 + c16 * 16) : kOOB);
      *reinterpret_cast<i32x4*>(WB + (c16 >> 3) * 64 * kBKB + lds_off(row, c16 & 7)) = v;
    }
  } else if constexpr (FU) {
    const __amdgpu_buffer_rsrc_t rw2 = rsrc(a.w2, a.w2_bytes);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c2 = 32 * (wave & 1) + 16 * i + (lane & 15);
#pragma unroll
      for (int s = 0; s < KS2; ++s)
        wb[i][s] = bload16(rw2, c2 < a.cout2 ? (uint32_t)(c2 * TCO * 2 + 64 * s + 16 * (lane >> 4)) : kOOB);
    }
  }

  // B-fragment addresses: boff[kw][s] = LDS byte offset (within a window
  // buffer, patch row 2 pg, tap row 0) of this lane's chunk
  const int pc = lane & 15;
  int boff[3][KS];
#pragma unroll
  for (int kw = 0; kw < 3; ++kw) {
    const int pos = S == 1 ? pc + kw : ((kw & 1) ? W::HCE + pc : pc + kw / 2);
#pragma unroll
    for (int s = 0; s < KS; ++s)
      boff[kw][s] = (2 * pg * S * W::HC + pos) * 128 + (((4 * s + (lane >> 4)) ^ (pos & 7)) << 4);
  }

  // the epilogue constants of this wave's channels, loaded once
  QuadConsts qc1[2], qc2[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    qc1[i] = load_quad_consts_t<2>(a.e, co0 + 32 * cg + 16 * i + 4 * (lane >> 4), g.cout);
    if constexpr (FU) qc2[i] = load_quad_consts_t<2>(a.e2, 32 * (wave & 1) + 16 * i + 4 * (lane >> 4), a.cout2);
  }

  const int m = g.m;
  const OutRef o = out_ref(a.y, m, FU ? a.cout2 : g.cout, 2, FU ? nullptr : a.e.res);
  typedef f32x4 acc_t;
  // Each wave's copies of a window are complete before it passes the
  // barrier that starts the window's patch: for the first window here, for
  // the others just before the previous patch's stores (by then the copy
  // has had that patch's MFMAs to land, and the stores, issued after the
  // wait, are never waited for inside the loop).
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  int it = 0;
  for (; p < p_end; p += step, ++it) {
    const int buf = it & 1;
    // the barrier makes everyone's copies of window p visible and frees the
    // other buffer (lgkmcnt: the first time, every wave's weight fragments
    // are out of that buffer before anyone copies a window into it)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __syncthreads();
    const Origin nxt = load_window(p + step < p_end ? p + step : a.npatch, buf ^ 1);

    acc_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = acc_t{0, 0, 0, 0};
    const char* win = smem + buf * BUF;
    // 9 * KS steps (tap, K-step), each 2 B fragments and 4 MFMAs; the next
    // step's fragments are read before the current step's MFMAs issue, so
    // the LDS latency hides behind them
    constexpr int NSTEP = 9 * KS;
    auto read_b = [&](int st, i32x4 (&bf)[2]) {
      const int t = st / KS, s = st % KS, kh = t / 3, kw = t % 3;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bf[j] = *reinterpret_cast<const i32x4*>(win + boff[kw][s] + (j * S + kh) * W::HC * 128);
    };
    i32x4 bcur[2], bnext[2];
    read_b(0, bcur);
    StaticFor<0, NSTEP>::run([&](auto stc) {
      constexpr int st = decltype(stc)::value;
      if constexpr (st + 1 < NSTEP) read_b(st + 1, bnext);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = Mfma<2>::run(wa[st / KS][st % KS][i], bcur[j], acc[i][j]);
      if constexpr (st + 1 < NSTEP) {
        bcur[0] = bnext[0];
        bcur[1] = bnext[1];
      }
    });

    const int n = cur.n, r0 = cur.r0, c0 = cur.c0;
    cur = nxt;
    if constexpr (FU == 0) {
      with_epilogue<2>(OUT_BF16, a.e.act, [&](auto, auto ac) {
        constexpr int ACT = decltype(ac)::value;
        u32x2 d[2][2];
        int pxs[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int r = r0 + 2 * pg + j, c = c0 + pc;
          pxs[j] = (r < g.ho && c < g.wo) ? (n * g.ho + r) * g.wo + c : m;
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int co = co0 + 32 * cg + 16 * i + 4 * (lane >> 4);
#pragma unroll
          for (int j = 0; j < 2; ++j) d[i][j] = pack_quad_bf16<ACT>(acc[i][j], qc1[i], co, pxs[j], o);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the next window has landed
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) store_packed(d[i][j], co0 + 32 * cg + 16 * i + 4 * (lane >> 4), pxs[j], o);
      });
    } else {
      // the intermediate tile into the (now free) window buffer: pixel row
      // px = 16 (2 pg + j) + pc, 128-byte channel block col / 64
      __syncthreads();
      char* Y = smem + buf * BUF;
      with_epilogue<2>(OUT_BF16, a.e.act, [&](auto, auto ac) {
        constexpr int ACT = decltype(ac)::value;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int col = 32 * cg + 16 * i + 4 * (lane >> 4);
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int row = 16 * (2 * pg + j) + pc;
            float f[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) f[r] = act_t<ACT>(acc[i][j][r] + qc1[i].bsf[r]);
            *reinterpret_cast<u32x2*>(Y + (col >> 6) * 64 * kBKB + lds_off(row, (col & 63) >> 3) + (col & 4) * 2) =
                u32x2{bf16x2_bits(f[0], f[1]), bf16x2_bits(f[2], f[3])};
          }
        }
      });
      __syncthreads();
      // the 1x1 layer: 64 (>= cout2) channels x 64 pixels; wave w: channels
      // 32 (w & 1) .., pixels 64 / (NW / 2) per wave group
      constexpr int FP2 = 8 / NW;  // 16-pixel fragments per wave: 2 (NW 4) or 1 (NW 8)
      acc_t acc2[2][FP2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < FP2; ++j) acc2[i][j] = acc_t{0, 0, 0, 0};
      const int prow0 = 16 * FP2 * (wave >> 1) + pc;
#pragma unroll
      for (int kt2 = 0; kt2 < TCO / 64; ++kt2) {
        const char* B2 = Y + kt2 * 64 * kBKB;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int c = 4 * s + (lane >> 4);
          i32x4 bf[FP2];
#pragma unroll
          for (int j = 0; j < FP2; ++j) bf[j] = *reinterpret_cast<const i32x4*>(B2 + lds_off(prow0 + 16 * j, c));
          i32x4 af[2];
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            if constexpr (WB_LDS)
              af[i] = *reinterpret_cast<const i32x4*>(WB + kt2 * 64 * kBKB +
                                                      lds_off(32 * (wave & 1) + 16 * i + pc, c));
            else
              af[i] = wb[i][2 * kt2 + s];
          }
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < FP2; ++j) acc2[i][j] = Mfma<2>::run(af[i], bf[j], acc2[i][j]);
        }
      }
      with_epilogue<2>(OUT_BF16, a.e2.act, [&](auto, auto ac) {
        constexpr int ACT = decltype(ac)::value;
        u32x2 d[2][FP2];
        int pxs[FP2];
#pragma unroll
        for (int j = 0; j < FP2; ++j) {
          const int prow = prow0 + 16 * j;  // pixel of the patch: row prow / 16, column pc
          const int r = r0 + (prow >> 4), c = c0 + pc;
          pxs[j] = (r < g.ho && c < g.wo) ? (n * g.ho + r) * g.wo + c : m;
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int c2 = 32 * (wave & 1) + 16 * i + 4 * (lane >> 4);
#pragma unroll
          for (int j = 0; j < FP2; ++j) d[i][j] = pack_quad_bf16<ACT>(acc2[i][j], qc2[i], c2, pxs[j], o);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the next window has landed
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < FP2; ++j) store_packed(d[i][j], 32 * (wave & 1) + 16 * i + 4 * (lane >> 4), pxs[j], o);
      });
    }
  }
  // the copies issued for the patch after the last must land before the
  // workgroup's LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int S, int KS, int TCO, int FU>
hipError_t launch_cfg(const HaloArgs& args, int nwg, hipStream_t s) {
  hipLaunchKernelGGL((halo_kernel<S, KS, TCO, FU>), dim3(nwg), dim3(TCO * 4), 0, s, args);
  return hipGetLastError();
}

void fill_args(const conv_plan* p, const void* x, const void* w, const Epi& e, void* y, HaloArgs& a) {
  std::memset(&a, 0, sizeof(a));
  a.x = static_cast<const char*>(x);
  a.w = static_cast<const char*>(w);
  a.y = y;
  a.e = e;
  a.g = p->g;
  a.x_bytes = (int)p->x_bytes;
  a.w_bytes = (int)p->w_bytes;
  a.npr = (p->g.ho + kPR - 1) / kPR;
  a.npc = (p->g.wo + kPC - 1) / kPC;
  a.npatch = p->g.n * a.npr * a.npc;
}

// XCD ranges of patches need every XCD to hold the same number of a channel
// tile's workgroups.
void set_gp(HaloArgs& a, int gp) {
  a.gp = gp;
  a.xr = HALO_XR && gp % 8 == 0;
}

// Workgroups per channel tile: enough to give every CU its share (two
// workgroups of 4 waves, or one of 8, per CU), at most one per patch.
int halo_gp(const conv_plan* p, int tco, int npatch) {
  const int nct = (p->g.cout + tco - 1) / tco;
  const int per_cu = tco == 64 ? 2 : 1;
  return std::max(1, std::min(npatch, per_cu * p->cus / nct));
}

hipError_t dispatch(int s, int ks, int tco, int fu, const HaloArgs& a, int nwg, hipStream_t st) {
  if (fu) {
    if (tco == 64) {
      if (s == 1) return ks == 1 ? launch_cfg<1, 1, 64, 1>(a, nwg, st) : launch_cfg<1, 2, 64, 1>(a, nwg, st);
      return ks == 1 ? launch_cfg<2, 1, 64, 1>(a, nwg, st) : launch_cfg<2, 2, 64, 1>(a, nwg, st);
    }
    if (s == 1) return ks == 1 ? launch_cfg<1, 1, 128, 1>(a, nwg, st) : launch_cfg<1, 2, 128, 1>(a, nwg, st);
    return ks == 1 ? launch_cfg<2, 1, 128, 1>(a, nwg, st) : launch_cfg<2, 2, 128, 1>(a, nwg, st);
  }
  if (s == 1) return ks == 1 ? launch_cfg<1, 1, 64, 0>(a, nwg, st) : launch_cfg<1, 2, 64, 0>(a, nwg, st);
  return ks == 1 ? launch_cfg<2, 1, 64, 0>(a, nwg, st) : launch_cfg<2, 2, 64, 0>(a, nwg, st);
}

}  // namespace

bool halo_eligible(const conv_desc& d, const Geometry& g) {
  return d.dtype == CONV_BF16 && d.out_dtype == CONV_BF16 && d.groups == 1 && g.kh == 3 && g.kw == 3 &&
         g.sh == g.sw && (g.sh == 1 || g.sh == 2) && (g.c == 32 || g.c == 64) && g.ph <= 2 && g.pw <= 2 &&
         (g.cout & 3) == 0;
}

// The automatic choice, from timings on MI355X of the 640x640 stack's 3x3
// layers against the implicit-GEMM kernel: the halo kernel wins at stride 1
// (320x320x64 -> 64: 15 against 22 us) and over 32 input channels (640x640
// -> 320x320, 32 -> 64: 15 against 17 us); at stride 2 over 64 channels it
// ties or loses (the window is 4.6 input pixels per output there, the
// implicit GEMM's 64x64 tiles keep five workgroups per CU). Layers with
// fewer than 512 patch units are left to the implicit GEMM.
bool halo_preferred(const conv_desc& d, const Geometry& g) {
  if (!halo_eligible(d, g) || !(g.sh == 1 || g.c == 32)) return false;
  const long units = (long)g.n * ((g.ho + kPR - 1) / kPR) * ((g.wo + kPC - 1) / kPC) * ((g.cout + 63) / 64);
  return units >= 512;
}

// The fused launch over the halo kernel: every eligible first layer with 64
// or 128 channels except 64 channels at stride 2 over 64 input channels
// (that instance does not fit its registers).
bool halo_fusable(const conv_desc& d, const Geometry& g) {
  return halo_eligible(d, g) && (g.cout == 64 || g.cout == 128) && !(g.cout == 64 && g.sh == 2 && g.c == 64);
}

int halo_grid(const conv_plan* p, int tco) {
  const int npatch = p->g.n * ((p->g.ho + kPR - 1) / kPR) * ((p->g.wo + kPC - 1) / kPC);
  return halo_gp(p, tco, npatch) * ((p->g.cout + tco - 1) / tco);
}

hipError_t launch_halo(const conv_plan* p, const void* x, const void* w, const Epi& e, void* y, hipStream_t s) {
  HaloArgs a;
  fill_args(p, x, w, e, y, a);
  set_gp(a, halo_gp(p, 64, a.npatch));
  const int nwg = a.gp * ((p->g.cout + 63) / 64);
  return dispatch(p->g.sh, p->g.c / 32, 64, 0, a, nwg, s);
}

hipError_t launch_halo_fused(const conv_plan* p1, const conv_plan* p2, const void* x, const void* w1, const Epi& e1,
                             const void* w2, const Epi& e2, void* y, hipStream_t s) {
  HaloArgs a;
  fill_args(p1, x, w1, e1, y, a);
  const int tco = p1->g.cout;  // 64 or 128: the whole intermediate per workgroup
  set_gp(a, halo_gp(p1, tco, a.npatch));
  a.w2 = static_cast<const char*>(w2);
  a.w2_bytes = (int)p2->w_bytes;
  a.cout2 = p2->g.cout;
  a.e2 = e2;
  return dispatch(p1->g.sh, p1->g.c / 32, tco, 1, a, a.gp, s);
}

}  // namespace convnhwc
