// igemm.hip -- implicit-GEMM convolution on gfx950 MFMA (bf16 -> fp32 and
// int8 -> int32), NHWC activations, OHWI weights.
//
// The convolution is the GEMM  Y[px][co] = sum_k X'[px][k] * W[co][k]  with
// px = (n, ho, wo) over N*Ho*Wo output pixels, k = (kh, kw, ci) over
// KH*KW*Cin, and X'[px][k] = x[n, ho*sh - ph + kh, wo*sw - pw + kw, ci] (0
// outside the image). X' is never materialised: each K-tile of it is gathered
// from NHWC straight into LDS (the GPU analogue of the im2col + GEMM path of
// the nanoinfer README; for a 1x1 stride-1 unpadded layer X' is the input
// itself, which the LOAD_1X1 loader uses). OHWI weights make W K-contiguous
// like X', so both operands are read along K (the layout the nanoinfer README
// found the vendor int8 GEMM to need).
//
// Work decomposition. A workgroup (4 x wave64) owns a TCO x TPX output tile
// and keeps its fp32/int32 accumulators in registers for the whole K loop
// (output-stationary, one of the schedules the TSO paper compares). K is
// walked in tiles of 128 bytes per row (64 bf16 or 128 int8); each tile is
// 8 chunks of 16 bytes per row.
//
// Memory pipeline. All global reads are buffer loads: an out-of-range offset
// returns zero, so image borders, the K tail and ragged tiles need no
// branches (a lane that must read zero gets the offset 0x80000000). Each
// thread keeps D K-tiles of chunks in flight in registers; at every K-tile it
// writes the oldest one into one of two LDS buffers, passes one barrier,
// re-issues the freed registers for the tile D ahead, and runs the MFMAs of
// the tile just written. LDS rows are 128 bytes with chunk c of row r stored
// at position c ^ (r & 7), so both the 16-byte stores and the ds_read_b128 of
// 16 consecutive rows hit distinct banks.
//
// MFMA operand mapping (v_mfma_f32_16x16x32_bf16 / v_mfma_i32_16x16x64_i8):
// the weights are the "A" operand (rows = output channels) and the gathered
// activations the "B" operand (columns = pixels). Lane l supplies row/column
// (l % 16) and 16 bytes of K at byte offset 16*(l / 16); it receives D rows
// 4*(l/16) .. 4*(l/16)+3 of column l % 16, i.e. four consecutive output
// channels of one pixel, which the epilogue stores as one NHWC vector.
#include <algorithm>
#include <cstring>

#include "igemm_common.h"

namespace convnhwc {

const TileCfg kTiles[kNumTiles] = {
    {64, 64, 2, 2},    // 1: few pixels or short reductions
    {128, 128, 2, 2},  // 2: 128 channels and enough tiles to fill the CUs
    {64, 128, 2, 2},   // 3
    {128, 64, 2, 2},   // 4
};

namespace {

struct IgArgs {
  const char* x;
  const char* w;
  void* y;
  Epi e;
  Geometry g;
  int out_kind;
  int nco_tiles;
  int x_bytes;
  int w_bytes;
  float rcp_c;   // 1.0f / Cin
  float rcp_kw;  // 1.0f / KW
  int x_shift;   // LOAD_TAP: bytes the x descriptor starts before x
  int co_group;  // tile order: channel tiles per group (nco_tiles: channel tile fastest; 1: pixel tile fastest)
  int ksplit;    // K-splits (gridDim.y); > 1 writes raw partial sums to ws
  int kt_per;    // K-tiles per split
  void* ws;      // [ksplit][m][cout] fp32 / int32 partial sums
  int kp;        // bfp8 weights: K padded to a multiple of 16 (mantissa row length)
  int w_exp_off; // bfp8 weights: byte offset of the exponent bytes in w
  // FU: a following 1x1 layer (c_in = this layer's Cout = TCO) applied to
  // the tile before anything is stored; y is then that layer's output
  const char* w2;  // its weights [cout2][TCO] bf16
  int w2_bytes;
  int cout2;       // <= 64, a multiple of 4
  Epi e2;          // its bias and activation
  // LOAD_CAT: the input is the channel concat of x (c0b bytes per pixel) and
  // x2 (the other g.c * ESZ - c0b), each at half resolution when its up flag
  // is set
  const char* x2;
  int x2_bytes;
  int c0b;
  int up0, up1;
};

// bfp8 weights (WQ): eight consecutive mantissas of one block (two dwords)
// and the block's exponent byte E -> the 8 bf16 values m * 2^(E - 133). Each
// is exact: (float)m has at most 7 significant bits, the power-of-two
// scaling is exact (fp32 keeps denormals), and the top half of such a float
// is its bf16 value.
__device__ __forceinline__ i32x4 bfp8_to_bf16x8(const i32x4& q) {
  const int sh = (int)((uint32_t)q[2] & 0xffu) - 133;
  uint32_t out[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t wd = (uint32_t)q[p >> 1];
    const int s0 = 16 * (p & 1);
    const float f0 = __builtin_ldexpf((float)(int)(int8_t)(wd >> s0), sh);
    const float f1 = __builtin_ldexpf((float)(int)(int8_t)(wd >> (s0 + 8)), sh);
    out[p] = (__builtin_bit_cast(uint32_t, f0) >> 16) | (__builtin_bit_cast(uint32_t, f1) & 0xffff0000u);
  }
  return i32x4{(int)out[0], (int)out[1], (int)out[2], (int)out[3]};
}


// ---------------------------------------------------------------- kernel

// The waves-per-SIMD hint lets the register allocator keep the accumulators
// of the unrolled two-stage loop in place; with the default target it copies
// them between AGPR ranges on every iteration.
#ifndef IGEMM_WPE
#define IGEMM_WPE 2
#endif

template <int ESZ, int TCO, int TPX, int WCO, int WPX, int LOADER, int D, int WQ, int FU>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(IGEMM_WPE))) void igemm_kernel(IgArgs a) {
  constexpr int VE = 16 / ESZ;      // elements per 16-byte chunk
  constexpr int BKE = kBKB / ESZ;   // elements per K-tile row
  constexpr int FCO = TCO / WCO / 16;
  constexpr int FPX = TPX / WPX / 16;
  constexpr int ACH = TCO / 32;     // 16-byte A chunks per thread per tile
  constexpr int BCH = TPX / 32;     // 16-byte B chunks per thread per tile
  static_assert(FCO >= 1 && FPX >= 1 && WCO * WPX == 4, "bad tile");
  static_assert(LOADER != LOAD_GENERIC || D == 1, "generic loader is single-stage");
  static_assert(WQ == 0 || (ESZ == 2 && LOADER != LOAD_GENERIC), "bfp8 weights: bf16, 16-byte loaders");
  static_assert(FU == 0 || (ESZ == 2 && TPX == 64 && (TCO == 64 || TCO == 128) && WCO == 2 && WPX == 2 && WQ == 0),
                "fused 1x1: bf16, tiles 64x64 or 128x64");
  typedef typename Mfma<ESZ>::acc_t acc_t;

  __shared__ __attribute__((aligned(16))) char smem[2 * (TCO + TPX) * kBKB];
  char* const As = smem;
  char* const Bs = smem + 2 * TCO * kBKB;

  const Geometry g = a.g;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wco = wave / WPX;
  const int wpx = wave % WPX;
  const __amdgpu_buffer_rsrc_t rx = rsrc(a.x, a.x_bytes);
  const __amdgpu_buffer_rsrc_t rw = rsrc(a.w, a.w_bytes);
  const __amdgpu_buffer_rsrc_t rx2 = rsrc(LOADER == LOAD_CAT ? a.x2 : a.x, LOADER == LOAD_CAT ? a.x2_bytes : 0);

  // Tiles are handed to the 8 XCDs round-robin by workgroup id; remap so each
  // XCD (own L2) gets a contiguous run of tiles: XCD x = id % 8 takes the
  // q = nwg / 8 tiles (one more for x < nwg % 8) from x q + min(x, nwg % 8)
  // on. The run walks groups of co_group channel tiles, the channel tile
  // fastest within a group, then the pixel tile: an XCD's run touches about
  // co_group channel tiles and run / co_group pixel tiles, so the group size
  // trades weight rows against activation rows (co_group_for picks it).
  const int nwg = gridDim.x;
  const int xcd = blockIdx.x & 7;
  const int lin = xcd * (nwg >> 3) + min(xcd, nwg & 7) + (blockIdx.x >> 3);
  const int npx_tiles = nwg / a.nco_tiles;
  const int span = a.co_group * npx_tiles;
  const int grp = lin / span;
  const int first = grp * a.co_group;
  const int gsz = min(a.nco_tiles - first, a.co_group);
  const int rem = lin - grp * span;
  const int co0 = (first + rem % gsz) * TCO;
  const int px0 = (rem / gsz) * TPX;
  const int hw_o = g.ho * g.wo;

  // ---- per-thread loader state -------------------------------------
  // VEC / 1X1: chunk j of this thread is (row tid/8 + 32 j, column tid%8).
  // GENERIC:   chunk j of this thread is (row tid%T, column (tid/T)*CH + j).
  int b_base[BCH], b_hi0[BCH], b_wi0[BCH];
  for (int j = 0; j < BCH; ++j) {
    int row;
    if constexpr (LOADER == LOAD_GENERIC)
      row = tid % TPX;
    else
      row = (tid >> 3) + 32 * j;
    const int p = px0 + row;
    if (p < g.m) {
      const int n = p / hw_o;
      const int r = p - n * hw_o;
      const int ho = r / g.wo;
      const int wo = r - ho * g.wo;
      if constexpr (LOADER == LOAD_1X1) {
        b_base[j] = p * g.c;
        b_hi0[j] = 0;
        b_wi0[j] = 0;
      } else if constexpr (LOADER == LOAD_CAT) {
        // pixel index of (n, ho, wo) in each map (b_base: x, b_wi0: x2)
        const int h0 = g.h >> a.up0, w0 = g.w >> a.up0, h1 = g.h >> a.up1, w1 = g.w >> a.up1;
        b_base[j] = (n * h0 + (ho >> a.up0)) * w0 + (wo >> a.up0);
        b_wi0[j] = (n * h1 + (ho >> a.up1)) * w1 + (wo >> a.up1);
        b_hi0[j] = 0;
      } else {
        const int hi0 = ho * g.sh - g.ph;
        const int wi0 = wo * g.sw - g.pw;
        b_hi0[j] = hi0;
        b_wi0[j] = wi0;
        b_base[j] = ((n * g.h + hi0) * g.w + wi0) * g.c;
      }
    } else {
      b_base[j] = 0;
      b_hi0[j] = -0x40000000;  // every bounds test fails
      b_wi0[j] = 0;
    }
  }

  // LOAD_TAP / LOAD_1X1: per-thread byte offsets that stay fixed for the
  // whole K loop; the K position enters every load as a wave-uniform soffset.
  // The x descriptor of LOAD_TAP starts x_shift = (ph*W + pw)*Cin*ESZ bytes
  // before x, so that the offset of a pixel's top-left tap is never negative.
  // tmask[j] bit t says whether tap t of row j lies inside the image.
  uint32_t voff_a[ACH], voff_b[BCH], tmask[BCH];
  __amdgpu_buffer_rsrc_t rxt = rx;
  const int cbytes = g.c * ESZ;
  const int nkt_all = (g.k * ESZ + kBKB - 1) / kBKB;
  // K-tiles [kt0, kt0 + nkt) belong to this workgroup's split
  const int kt0 = blockIdx.y * a.kt_per;
  const int nkt = min(a.kt_per, nkt_all - kt0);
  int t_kh = 0, t_kw = 0, t_cb = 0;  // uniform tap state of the next fetch
  if constexpr (LOADER == LOAD_TAP) {
    const int kb0 = kt0 * kBKB;
    const int tap0 = kb0 / cbytes;
    t_cb = kb0 - tap0 * cbytes;
    t_kh = tap0 / g.kw;
    t_kw = tap0 - t_kh * g.kw;
  }
  uint32_t voff_b2[LOADER == LOAD_CAT ? BCH : 1];
  if constexpr (LOADER == LOAD_CAT) {
    const int c16 = (tid & 7) * 16;
    const int c1b = cbytes - a.c0b;
#pragma unroll
    for (int j = 0; j < ACH; ++j) {
      const int co = co0 + (tid >> 3) + 32 * j;
      voff_a[j] = co < g.cout ? (uint32_t)(co * g.k * ESZ + c16) : kOOB;
    }
#pragma unroll
    for (int j = 0; j < BCH; ++j) {
      voff_b[j] = b_hi0[j] == 0 ? (uint32_t)(b_base[j] * a.c0b + c16) : kOOB;
      voff_b2[j] = b_hi0[j] == 0 ? (uint32_t)(b_wi0[j] * c1b + c16) : kOOB;
    }
  }
  if constexpr (LOADER == LOAD_TAP || LOADER == LOAD_1X1) {
    const int c16 = (tid & 7) * 16;
#pragma unroll
    for (int j = 0; j < ACH; ++j) {
      const int co = co0 + (tid >> 3) + 32 * j;
      voff_a[j] = co < g.cout ? (uint32_t)(co * g.k * ESZ + c16) : kOOB;
    }
    if constexpr (LOADER == LOAD_TAP) {
      rxt = rsrc(a.x - a.x_shift, a.x_bytes + a.x_shift);
#pragma unroll
      for (int j = 0; j < BCH; ++j) {
        voff_b[j] = (uint32_t)(b_base[j] * ESZ + a.x_shift + c16);
        uint32_t m = 0;
        for (int kh = 0, tap = 0; kh < g.kh; ++kh)
          for (int kw = 0; kw < g.kw; ++kw, ++tap) {
            const int hi = b_hi0[j] + kh, wi = b_wi0[j] + kw;
            if ((unsigned)hi < (unsigned)g.h && (unsigned)wi < (unsigned)g.w) m |= 1u << tap;
          }
        tmask[j] = m;
      }
    } else {
#pragma unroll
      for (int j = 0; j < BCH; ++j) voff_b[j] = b_hi0[j] == 0 ? (uint32_t)(b_base[j] * ESZ + c16) : kOOB;
    }
  }

  // bfp8 weights: chunk j of this thread covers elements kt*64 + e8 .. +7 of
  // row co (one block); its 8 mantissa bytes and its block's exponent byte
  // sit at these offsets plus kt*64 and kt*4.
  uint32_t voff_am[ACH], voff_ae[ACH];
  if constexpr (WQ) {
    const int e8 = (tid & 7) * 8;
#pragma unroll
    for (int j = 0; j < ACH; ++j) {
      const int co = co0 + (tid >> 3) + 32 * j;
      voff_am[j] = co < g.cout ? (uint32_t)(co * a.kp + e8) : kOOB;
      voff_ae[j] = co < g.cout ? (uint32_t)(a.w_exp_off + co * (a.kp >> 4) + (e8 >> 4)) : kOOB;
    }
  }
  // The raw bfp8 bytes of K-tile kt: {mantissas 0-3, 4-7, exponent, 0}.
  auto fetch_aq = [&](int kt, i32x4 (&ra)[ACH]) {
    const bool kin = kt * 64 + (tid & 7) * 8 < g.k;
#pragma unroll
    for (int j = 0; j < ACH; ++j) {
      const u32x2 mm = __builtin_amdgcn_raw_buffer_load_b64(rw, kin ? voff_am[j] : kOOB, kin ? kt * 64 : 0, 0);
      const uint32_t ee = __builtin_amdgcn_raw_buffer_load_b8(rw, kin ? voff_ae[j] : kOOB, kin ? kt * 4 : 0, 0);
      ra[j] = i32x4{(int)mm[0], (int)mm[1], (int)ee, 0};
    }
  };

  // Issue the global loads of K-tile kt into one register stage (tiles are
  // fetched in increasing order).
  auto fetch = [&](int kt, i32x4 (&ra)[ACH], i32x4 (&rb)[BCH]) {
    const int kb = kt * BKE;
    if constexpr (LOADER == LOAD_GENERIC) {
      // A: weights, element-wise (K * ESZ need not be 16-byte aligned).
      {
        constexpr int G = 256 / TCO;
        constexpr int CH = 8 / G;
        const int row = tid % TCO, grp = tid / TCO;
        const int co = co0 + row;
        const int k_first = kb + grp * CH * VE;
        uint32_t v[CH][VE];
#pragma unroll
        for (int j = 0; j < CH; ++j)
#pragma unroll
          for (int e = 0; e < VE; ++e) {
            const int k = k_first + j * VE + e;
            const uint32_t off = (co < g.cout && k < g.k) ? (uint32_t)(co * g.k + k) * ESZ : kOOB;
            v[j][e] = bload_elem<ESZ>(rw, off);
          }
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          uint32_t wd[4] = {0, 0, 0, 0};
#pragma unroll
          for (int e = 0; e < VE; ++e) wd[e * ESZ / 4] |= v[j][e] << (8 * ((e * ESZ) & 3));
          ra[j] = i32x4{(int)wd[0], (int)wd[1], (int)wd[2], (int)wd[3]};
        }
      }
      // B: activations, element-wise gather; every load is issued before
      // any is used.
      {
        constexpr int G = 256 / TPX;
        constexpr int CH = 8 / G;
        const int grp = tid / TPX;
        const int k_first = kb + grp * CH * VE;
        int tap = k_first / g.c;
        int ci = k_first - tap * g.c;
        int kh = tap / g.kw;
        int kw = tap - kh * g.kw;
        uint32_t v[CH][VE];
#pragma unroll
        for (int j = 0; j < CH; ++j)
#pragma unroll
          for (int e = 0; e < VE; ++e) {
            const int hi = b_hi0[0] + kh;
            const int wi = b_wi0[0] + kw;
            const bool ok = kh < g.kh && (unsigned)hi < (unsigned)g.h && (unsigned)wi < (unsigned)g.w;
            const uint32_t off = ok ? (uint32_t)(b_base[0] + (kh * g.w + kw) * g.c + ci) * ESZ : kOOB;
            v[j][e] = bload_elem<ESZ>(rx, off);
            if (++ci == g.c) {
              ci = 0;
              if (++kw == g.kw) {
                kw = 0;
                ++kh;
              }
            }
          }
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          uint32_t wd[4] = {0, 0, 0, 0};
#pragma unroll
          for (int e = 0; e < VE; ++e) wd[e * ESZ / 4] |= v[j][e] << (8 * ((e * ESZ) & 3));
          rb[j] = i32x4{(int)wd[0], (int)wd[1], (int)wd[2], (int)wd[3]};
        }
      }
    } else if constexpr (LOADER == LOAD_TAP) {
      // Cin*ESZ % 128 == 0: the whole K-tile is one tap, one 128-byte block of
      // channels; the tap offset is the same for every lane.
      const bool live = kt < nkt_all;
      const int tap = t_kh * g.kw + t_kw;
      const int soff_b = (t_kh * g.w + t_kw) * cbytes + t_cb;
      const int soff_a = kt * kBKB;
      if constexpr (WQ)
        fetch_aq(kt, ra);
      else
#pragma unroll
        for (int j = 0; j < ACH; ++j) ra[j] = bload16s(rw, live ? voff_a[j] : kOOB, live ? soff_a : 0);
#pragma unroll
      for (int j = 0; j < BCH; ++j) {
        const bool ok = live && ((tmask[j] >> (tap & 31)) & 1u);
        rb[j] = bload16s(rxt, ok ? voff_b[j] : kOOB, live ? soff_b : 0);
      }
      t_cb += kBKB;
      if (t_cb == cbytes) {
        t_cb = 0;
        if (++t_kw == g.kw) {
          t_kw = 0;
          ++t_kh;
        }
      }
    } else if constexpr (LOADER == LOAD_CAT) {
      // K = Cin; K-tile kt lies in x (kt * 128 < c0b) or in x2, whole (both
      // parts are multiples of 128 bytes); tiles past K read zeros
      const int soff = kt * kBKB;
      const bool live = kt < nkt_all;
      const bool second = soff >= a.c0b;
      const int so = second ? soff - a.c0b : soff;
#pragma unroll
      for (int j = 0; j < ACH; ++j) ra[j] = bload16s(rw, live ? voff_a[j] : kOOB, live ? soff : 0);
      if (second) {
#pragma unroll
        for (int j = 0; j < BCH; ++j) rb[j] = bload16s(rx2, live ? voff_b2[j] : kOOB, live ? so : 0);
      } else {
#pragma unroll
        for (int j = 0; j < BCH; ++j) rb[j] = bload16s(rx, live ? voff_b[j] : kOOB, live ? so : 0);
      }
    } else if constexpr (LOADER == LOAD_1X1) {
      // K = Cin: chunk c of tile kt is valid while kt*128 + 16c < Cin*ESZ.
      const int soff = kt * kBKB;
      const bool cin_ok = (tid & 7) * 16 < cbytes - soff;
      if constexpr (WQ)
        fetch_aq(kt, ra);
      else
#pragma unroll
        for (int j = 0; j < ACH; ++j) ra[j] = bload16s(rw, cin_ok ? voff_a[j] : kOOB, cin_ok ? soff : 0);
#pragma unroll
      for (int j = 0; j < BCH; ++j) rb[j] = bload16s(rx, cin_ok ? voff_b[j] : kOOB, cin_ok ? soff : 0);
    } else {
      const int kc = kb + (tid & 7) * VE;  // first element of this thread's chunk
      const bool kin = kc < g.k;
      if constexpr (WQ) {
        fetch_aq(kt, ra);
      } else {
#pragma unroll
        for (int j = 0; j < ACH; ++j) {
          const int co = co0 + (tid >> 3) + 32 * j;
          ra[j] = bload16(rw, (co < g.cout && kin) ? (uint32_t)(co * g.k + kc) * ESZ : kOOB);
        }
      }
      {
        // this thread's chunk starts at element kc = (kh, kw, ci) of the
        // pixel's receptive field; Cin * ESZ % 16 == 0 keeps it in one tap
        int tap, ci, kh, kw;
        divmod_small(kc, g.c, a.rcp_c, tap, ci);
        divmod_small(tap, g.kw, a.rcp_kw, kh, kw);
        const int tap_off = (kh * g.w + kw) * g.c + ci;
        const bool khin = kh < g.kh;
#pragma unroll
        for (int j = 0; j < BCH; ++j) {
          const int hi = b_hi0[j] + kh;
          const int wi = b_wi0[j] + kw;
          const bool ok = khin && (unsigned)hi < (unsigned)g.h && (unsigned)wi < (unsigned)g.w;
          rb[j] = bload16(rx, ok ? (uint32_t)(b_base[j] + tap_off) * ESZ : kOOB);
        }
      }
    }
  };

  auto stash = [&](int buf, const i32x4 (&ra)[ACH], const i32x4 (&rb)[BCH]) {
    char* A = As + buf * TCO * kBKB;
    char* B = Bs + buf * TPX * kBKB;
    if constexpr (LOADER == LOAD_GENERIC) {
      {
        constexpr int G = 256 / TCO;
        constexpr int CH = 8 / G;
        const int row = tid % TCO, grp = tid / TCO;
#pragma unroll
        for (int j = 0; j < CH; ++j) *reinterpret_cast<i32x4*>(A + lds_off(row, grp * CH + j)) = ra[j];
      }
      {
        constexpr int G = 256 / TPX;
        constexpr int CH = 8 / G;
        const int row = tid % TPX, grp = tid / TPX;
#pragma unroll
        for (int j = 0; j < CH; ++j) *reinterpret_cast<i32x4*>(B + lds_off(row, grp * CH + j)) = rb[j];
      }
    } else {
      const int col = tid & 7;
#pragma unroll
      for (int j = 0; j < ACH; ++j)
        *reinterpret_cast<i32x4*>(A + lds_off((tid >> 3) + 32 * j, col)) = WQ ? bfp8_to_bf16x8(ra[j]) : ra[j];
#pragma unroll
      for (int j = 0; j < BCH; ++j) *reinterpret_cast<i32x4*>(B + lds_off((tid >> 3) + 32 * j, col)) = rb[j];
    }
  };

  acc_t acc[FCO][FPX];
#pragma unroll
  for (int i = 0; i < FCO; ++i)
#pragma unroll
    for (int j = 0; j < FPX; ++j) acc[i][j] = acc_t{0, 0, 0, 0};

  // FU: the second layer's weights as MFMA A fragments, loaded now: wave
  // (wave >> 1) owns its output channels 32 (wave >> 1) + 16 i + (lane & 15);
  // K-step s covers bytes 64 s .. 64 s + 63 of the TCO-channel reduction
  constexpr int KS2 = FU ? TCO / 32 : 1;
  i32x4 a2[2][KS2];
  if constexpr (FU) {
    const __amdgpu_buffer_rsrc_t rw2 = rsrc(a.w2, a.w2_bytes);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c2 = 32 * (wave >> 1) + 16 * i + (lane & 15);
#pragma unroll
      for (int s2 = 0; s2 < KS2; ++s2)
        a2[i][s2] = bload16(rw2, c2 < a.cout2 ? (uint32_t)(c2 * TCO * 2 + 64 * s2 + 16 * (lane >> 4)) : kOOB);
    }
  }

  // MFMA operand addresses within a stage: row (lane & 15) of each 16-row
  // fragment, chunk 4*s + (lane >> 4) of the tile.
  const int a_row0 = wco * (TCO / WCO) + (lane & 15);
  const int b_row0 = wpx * (TPX / WPX) + (lane & 15);

  // MFMAs of the tile in LDS buffer `buf`; when `more`, the next tile
  // (registers ra_n/rb_n) is written into buffer `nbuf` between the first and
  // the second K-step, so the LDS stores overlap the matrix work.
  auto compute = [&](int buf, const i32x4 (&ra_n)[ACH], const i32x4 (&rb_n)[BCH], int nbuf, bool more) {
    const char* A = As + buf * TCO * kBKB;
    const char* B = Bs + buf * TPX * kBKB;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int c = 4 * s + (lane >> 4);
      i32x4 af[FCO], bf[FPX];
#pragma unroll
      for (int i = 0; i < FCO; ++i)
        af[i] = *reinterpret_cast<const i32x4*>(A + lds_off(a_row0 + 16 * i, c));
#pragma unroll
      for (int j = 0; j < FPX; ++j)
        bf[j] = *reinterpret_cast<const i32x4*>(B + lds_off(b_row0 + 16 * j, c));
      if (s == 0 && more) stash(nbuf, ra_n, rb_n);
#pragma unroll
      for (int i = 0; i < FCO; ++i)
#pragma unroll
        for (int j = 0; j < FPX; ++j) acc[i][j] = Mfma<ESZ>::run(af[i], bf[j], acc[i][j]);
    }
  };

  // Pipeline. LDS buffer t%2 holds K-tile t while it is consumed; register
  // set r holds a tile in flight from global memory. Step t: one barrier
  // (tile t is visible, and buffer (t+1)%2 is no longer read by anyone),
  // then the MFMAs of tile t run while tile t+1 is copied from its register
  // set into the other buffer, then that register set is re-issued for tile
  // t+1+D. Loads for tiles at or beyond nkt are all out of range (zero, no
  // memory traffic), so fetches need no guard.
  i32x4 ra[D][ACH], rb[D][BCH];
  {
    i32x4 a0[ACH], b0[BCH];
    fetch(kt0, a0, b0);
#pragma unroll
    for (int d = 0; d < D; ++d) fetch(kt0 + 1 + d, ra[d], rb[d]);
    stash(0, a0, b0);
  }
  int t = 0;
  for (; t + D <= nkt; t += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      __syncthreads();
      compute((t + d) & 1, ra[d], rb[d], (t + d + 1) & 1, t + d + 1 < nkt);
      fetch(kt0 + t + d + 1 + D, ra[d], rb[d]);
    }
  }
#pragma unroll
  for (int d = 0; d < D; ++d) {
    if (t + d < nkt) {
      __syncthreads();
      compute((t + d) & 1, ra[d], rb[d], (t + d + 1) & 1, t + d + 1 < nkt);
    }
  }

  // ---- fused epilogue -------------------------------------------------
  const int co_w = co0 + wco * (TCO / WCO) + 4 * (lane >> 4);
  const int px_w = px0 + wpx * (TPX / WPX) + (lane & 15);
  if constexpr (FU) {
    // This layer's output tile, bias + activation + bf16 rounding as a store
    // would do, goes into LDS as the B operand of the 1x1 layer: pixel rows
    // of 128-byte channel blocks (block kt2 = channels 64 kt2 .. 64 kt2 + 63),
    // the swizzled layout of the K loop's tiles.
    __syncthreads();  // every wave is done with the K loop's buffers
    char* const Y = smem;
    with_epilogue<2>(OUT_BF16, a.e.act, [&](auto, auto ac) {
      constexpr int ACT = decltype(ac)::value;
#pragma unroll
      for (int i = 0; i < FCO; ++i) {
        const int col = wco * (TCO / WCO) + 4 * (lane >> 4) + 16 * i;  // channel within the tile
        const QuadConsts q = load_quad_consts_t<2>(a.e, co0 + col, g.cout);
#pragma unroll
        for (int j = 0; j < FPX; ++j) {
          const int row = wpx * (TPX / WPX) + (lane & 15) + 16 * j;
          float f[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) f[r] = act_t<ACT>(acc[i][j][r] + q.bsf[r]);
          *reinterpret_cast<u32x2*>(Y + (col >> 6) * TPX * kBKB + lds_off(row, (col & 63) >> 3) + (col & 4) * 2) =
              u32x2{bf16x2_bits(f[0], f[1]), bf16x2_bits(f[2], f[3])};
        }
      }
    });
    __syncthreads();
    // the 1x1 layer: 64 (<= cout2) channels x 64 pixels, 2 x 2 waves of 32 x 32
    acc_t acc2[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc2[i][j] = acc_t{0, 0, 0, 0};
    const int row2 = 32 * (wave & 1) + (lane & 15);
#pragma unroll
    for (int kt2 = 0; kt2 < TCO / 64; ++kt2) {
      const char* B2 = Y + kt2 * TPX * kBKB;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int c = 4 * s + (lane >> 4);
        i32x4 bf[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) bf[j] = *reinterpret_cast<const i32x4*>(B2 + lds_off(row2 + 16 * j, c));
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc2[i][j] = Mfma<2>::run(a2[i][2 * kt2 + s], bf[j], acc2[i][j]);
      }
    }
    const OutRef o2 = out_ref(a.y, g.m, a.cout2, 2, nullptr);
    const int c2w = 32 * (wave >> 1) + 4 * (lane >> 4);
    const int p2w = px0 + 32 * (wave & 1) + (lane & 15);
    with_epilogue<2>(OUT_BF16, a.e2.act, [&](auto oc, auto ac) {
      constexpr int OUT = decltype(oc)::value, ACT = decltype(ac)::value;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const QuadConsts q = load_quad_consts_t<2>(a.e2, c2w + 16 * i, a.cout2);
#pragma unroll
        for (int j = 0; j < 2; ++j) store_quad_t<2, OUT, ACT>(acc2[i][j], q, c2w + 16 * i, p2w + 16 * j, o2);
      }
    });
    return;
  }
  if (a.ksplit > 1) {
    // raw partial sums of this split; Cout % 4 == 0 on this path
    acc_t* ws = reinterpret_cast<acc_t*>(a.ws) + (size_t)blockIdx.y * g.m * (g.cout / 4);
#pragma unroll
    for (int i = 0; i < FCO; ++i) {
      const int co = co_w + 16 * i;
      if (co >= g.cout) continue;
#pragma unroll
      for (int j = 0; j < FPX; ++j) {
        const int px = px_w + 16 * j;
        if (px < g.m) ws[(size_t)px * (g.cout / 4) + co / 4] = acc[i][j];
      }
    }
    return;
  }
  if ((g.cout & 3) == 0) {
    const OutRef o = out_ref(a.y, g.m, g.cout, ESZ == 2 ? 2 : (a.out_kind == OUT_I32 ? 4 : 1), a.e.res);
    with_epilogue<ESZ>(a.out_kind, a.e.act, [&](auto oc, auto ac) {
      constexpr int OUT = decltype(oc)::value, ACT = decltype(ac)::value;
      StaticFor<0, FCO>::run([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        const int co = co_w + 16 * i;
        const QuadConsts q = load_quad_consts_t<ESZ>(a.e, co, g.cout);
        StaticFor<0, FPX>::run([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          store_quad_t<ESZ, OUT, ACT>(acc[i][j], q, co, px_w + 16 * j, o);
        });
      });
    });
    return;
  }
  // Cout not a multiple of 4: per-element stores
  StaticFor<0, FCO>::run([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    const int co = co_w + 16 * i;
    if (co >= g.cout) return;
    const QuadConsts q = load_quad_consts<ESZ>(a.e, co, g.cout);
    StaticFor<0, FPX>::run([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const int px = px_w + 16 * j;
      if (px < g.m) store_quad<ESZ>(acc[i][j], q, co, px, g.cout, a.out_kind, a.e.act, a.y, a.e.res);
    });
  });
}

// Register stages per loader: the element-wise gather issues up to 64 loads
// per thread per tile and stays single-staged.
#ifndef IGEMM_STAGES
#define IGEMM_STAGES 2
#endif
template <int LOADER, int TCO, int TPX>
constexpr int kStages = (LOADER == LOAD_GENERIC || TCO + TPX >= 512) ? 1 : IGEMM_STAGES;

template <int ESZ, int TCO, int TPX, int WCO, int WPX, int WQ>
hipError_t launch_tile(int loader, const IgArgs& args, dim3 nwg, hipStream_t s) {
  switch (loader) {
    case LOAD_GENERIC:
      // the element-wise gather maps at least one thread to each tile row
      if constexpr (TCO <= 256 && TPX <= 256 && WQ == 0)
        hipLaunchKernelGGL((igemm_kernel<ESZ, TCO, TPX, WCO, WPX, LOAD_GENERIC, kStages<LOAD_GENERIC, TCO, TPX>, 0, 0>),
                           dim3(nwg), dim3(256), 0, s, args);
      else
        return hipErrorInvalidValue;  // refused by conv_prepare
      break;
    case LOAD_VEC:
      hipLaunchKernelGGL((igemm_kernel<ESZ, TCO, TPX, WCO, WPX, LOAD_VEC, kStages<LOAD_VEC, TCO, TPX>, WQ, 0>), dim3(nwg),
                         dim3(256), 0, s, args);
      break;
    case LOAD_1X1:
      hipLaunchKernelGGL((igemm_kernel<ESZ, TCO, TPX, WCO, WPX, LOAD_1X1, kStages<LOAD_1X1, TCO, TPX>, WQ, 0>), dim3(nwg),
                         dim3(256), 0, s, args);
      break;
    default:
      hipLaunchKernelGGL((igemm_kernel<ESZ, TCO, TPX, WCO, WPX, LOAD_TAP, kStages<LOAD_TAP, TCO, TPX>, WQ, 0>), dim3(nwg),
                         dim3(256), 0, s, args);
      break;
  }
  return hipGetLastError();
}

template <int ESZ, int WQ>
hipError_t launch_esz(int tile, int loader, const IgArgs& args, dim3 nwg, hipStream_t s) {
  switch (tile) {
    case 0: return launch_tile<ESZ, 64, 64, 2, 2, WQ>(loader, args, nwg, s);
    case 1: return launch_tile<ESZ, 128, 128, 2, 2, WQ>(loader, args, nwg, s);
    case 2: return launch_tile<ESZ, 64, 128, 2, 2, WQ>(loader, args, nwg, s);
    default: return launch_tile<ESZ, 128, 64, 2, 2, WQ>(loader, args, nwg, s);
  }
}

template <int ESZ>
hipError_t launch_cat_esz(int tile, const IgArgs& args, dim3 nwg, hipStream_t s) {
  switch (tile) {
    case 0:
      hipLaunchKernelGGL((igemm_kernel<ESZ, 64, 64, 2, 2, LOAD_CAT, kStages<LOAD_CAT, 64, 64>, 0, 0>), nwg, dim3(256), 0,
                         s, args);
      break;
    case 1:
      hipLaunchKernelGGL((igemm_kernel<ESZ, 128, 128, 2, 2, LOAD_CAT, kStages<LOAD_CAT, 128, 128>, 0, 0>), nwg,
                         dim3(256), 0, s, args);
      break;
    case 2:
      hipLaunchKernelGGL((igemm_kernel<ESZ, 64, 128, 2, 2, LOAD_CAT, kStages<LOAD_CAT, 64, 128>, 0, 0>), nwg, dim3(256),
                         0, s, args);
      break;
    default:
      hipLaunchKernelGGL((igemm_kernel<ESZ, 128, 64, 2, 2, LOAD_CAT, kStages<LOAD_CAT, 128, 64>, 0, 0>), nwg, dim3(256),
                         0, s, args);
      break;
  }
  return hipGetLastError();
}

template <int TCO, int LOADER>
hipError_t launch_fused_tile(const IgArgs& args, dim3 nwg, hipStream_t s) {
  hipLaunchKernelGGL((igemm_kernel<2, TCO, 64, 2, 2, LOADER, kStages<LOADER, TCO, 64>, 0, 1>), dim3(nwg), dim3(256), 0,
                     s, args);
  return hipGetLastError();
}

}  // namespace

// Distinct channel tiles (*tc) and pixel tiles (*tp) of the run of tile
// indices [l0, l1) in the grouped order with group size g (see the kernel),
// counted group by group without visiting the tiles: consecutive indices
// inside a group cycle through its channel tiles, and the pixel tiles of a
// run that spans two groups are the union of a tail and a head.
static void run_tiles(long nco, long npx, long g, long l0, long l1, long* tc, long* tp) {
  const long span = g * npx;
  const long g0 = l0 / span, g1 = (l1 - 1) / span;
  long c = 0;
  for (long k = g0; k <= g1; ++k) {
    const long lo = std::max(l0, k * span) - k * span, hi = std::min(l1, (k + 1) * span) - k * span;
    c += std::min(std::min(nco - k * g, g), hi - lo);
  }
  *tc = c;
  if (g0 == g1) {
    const long gsz = std::min(nco - g0 * g, g);
    *tp = (l1 - 1 - g0 * span) / gsz - (l0 - g0 * span) / gsz + 1;
  } else if (g1 == g0 + 1) {
    const long a = (l0 - g0 * span) / std::min(nco - g0 * g, g);
    const long b = (l1 - 1 - g1 * span) / std::min(nco - g1 * g, g);
    *tp = std::min(npx, (b + 1) + (npx - a));
  } else {
    *tp = npx;
  }
}

// Channel tiles per group of the implicit-GEMM kernels' tile order. XCD x
// runs the workgroups [x q + min(x, r), ...) (q = nwg / 8, one more for
// x < r = nwg % 8): the group size is the one whose runs touch the fewest
// bytes in all, counting the weight rows of each channel tile (w_bytes /
// nco) and the input share of each pixel tile (x_bytes / npx) once per XCD
// that touches it. Allocation-free (it runs at every launch).
int co_group_for(const conv_plan* p, int nco, int npx) {
  const long nwg = (long)nco * npx;
  const long q = nwg / 8, r = nwg % 8;
  const double wt = (double)p->w_bytes / nco, xt = (double)p->x_bytes / npx;
  int best = p->w_bytes > p->x_bytes ? 1 : nco;
  double best_b = -1;
  for (int g = 1; g <= nco; ++g) {
    double b = 0;
    for (long x = 0; x < 8; ++x) {
      const long lin0 = x * q + std::min(x, r), lin1 = lin0 + q + (x < r);
      if (lin1 <= lin0) continue;
      long tc, tp;
      run_tiles(nco, npx, g, lin0, lin1, &tc, &tp);
      b += tc * wt + tp * xt;
    }
    if (best_b < 0 || b < best_b - 1e-9 * best_b) {
      best = g;
      best_b = b;
    }
  }
  return best;
}

int igemm_stages(int loader, int tile) {
  const TileCfg& t = kTiles[tile];
  return (loader == LOAD_GENERIC || t.tco + t.tpx >= 512) ? 1 : IGEMM_STAGES;
}

hipError_t launch_igemm(const conv_plan* p, const void* x, const void* w, const Epi& e, void* y,
                        hipStream_t s) {
  IgArgs args;
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
  const TileCfg& t = kTiles[p->tile];
  args.nco_tiles = (p->g.cout + t.tco - 1) / t.tco;
  const int npx = (p->g.m + t.tpx - 1) / t.tpx;
  args.co_group = co_group_for(p, args.nco_tiles, npx);
  args.ksplit = p->ksplit;
  args.kt_per = p->kt_per;
  args.ws = p->ws;
  args.kp = p->kp;
  args.w_exp_off = (int)p->w_exp_off;
  const dim3 grid(npx * args.nco_tiles, p->ksplit);
  hipError_t err = p->in_esz == 1 ? launch_esz<1, 0>(p->tile, p->loader, args, grid, s)
                   : p->wq        ? launch_esz<2, 1>(p->tile, p->loader, args, grid, s)
                                  : launch_esz<2, 0>(p->tile, p->loader, args, grid, s);
  if (err != hipSuccess || p->ksplit == 1) return err;
  return launch_splitk_reduce(p, e, y, s);
}

int cat_tile(const conv_plan* p) { return p->path == PATH_IGEMM ? p->tile : 0; }

hipError_t launch_igemm_cat(const conv_plan* p, const void* s0, int c0b, int up0, const void* s1, int up1,
                            const void* w, const Epi& e, void* y, hipStream_t s) {
  IgArgs args;
  std::memset(&args, 0, sizeof(args));
  const Geometry& g = p->g;
  const int c1b = g.c * p->in_esz - c0b;
  args.x = static_cast<const char*>(s0);
  args.x_bytes = (int)((int64_t)g.n * (g.h >> up0) * (g.w >> up0) * c0b);
  args.x2 = static_cast<const char*>(s1);
  args.x2_bytes = (int)((int64_t)g.n * (g.h >> up1) * (g.w >> up1) * c1b);
  args.c0b = c0b;
  args.up0 = up0;
  args.up1 = up1;
  args.w = static_cast<const char*>(w);
  args.y = y;
  args.e = e;
  args.g = g;
  args.out_kind = p->out_kind;
  args.w_bytes = (int)p->w_bytes;
  const int tile = cat_tile(p);
  const TileCfg& t = kTiles[tile];
  args.nco_tiles = (g.cout + t.tco - 1) / t.tco;
  const int npx = (g.m + t.tpx - 1) / t.tpx;
  args.co_group = co_group_for(p, args.nco_tiles, npx);
  args.ksplit = 1;
  args.kt_per = (g.k * p->in_esz + kBKB - 1) / kBKB;
  const dim3 grid(npx * args.nco_tiles, 1);
  return p->in_esz == 1 ? launch_cat_esz<1>(tile, args, grid, s) : launch_cat_esz<2>(tile, args, grid, s);
}

// p1's layer with p2's 1x1 layer applied to each output tile before any
// store (fused_1x1_ok has validated the pair): one workgroup per 64-pixel
// tile holding all of p1's output channels.
hipError_t launch_igemm_fused(const conv_plan* p1, const conv_plan* p2, const void* x, const void* w1, const Epi& e1,
                              const void* w2, const Epi& e2, void* y, hipStream_t s) {
  IgArgs args;
  std::memset(&args, 0, sizeof(args));
  args.x = static_cast<const char*>(x);
  args.w = static_cast<const char*>(w1);
  args.y = y;
  args.e = e1;
  args.g = p1->g;
  args.out_kind = OUT_BF16;
  args.x_bytes = (int)p1->x_bytes;
  args.w_bytes = (int)p1->w_bytes;
  args.rcp_c = 1.0f / (float)p1->g.c;
  args.rcp_kw = 1.0f / (float)p1->g.kw;
  args.x_shift = (p1->g.ph * p1->g.w + p1->g.pw) * p1->g.c * p1->in_esz;
  args.nco_tiles = 1;
  args.co_group = 1;
  args.ksplit = 1;
  args.kt_per = (p1->g.k * 2 + kBKB - 1) / kBKB;
  args.w2 = static_cast<const char*>(w2);
  args.w2_bytes = (int)p2->w_bytes;
  args.cout2 = p2->g.cout;
  args.e2 = e2;
  const dim3 grid((p1->g.m + 63) / 64, 1);
  const bool tap = p1->loader == LOAD_TAP;
  if (p1->g.cout == 64) return tap ? launch_fused_tile<64, LOAD_TAP>(args, grid, s) : launch_fused_tile<64, LOAD_VEC>(args, grid, s);
  return tap ? launch_fused_tile<128, LOAD_TAP>(args, grid, s) : launch_fused_tile<128, LOAD_VEC>(args, grid, s);
}

}  // namespace convnhwc
