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
// one 16-byte chunk per (row, 1/8 of the tile). The next tile's chunks are
// fetched into registers while the MFMAs consume the current LDS buffer
// (double-buffered LDS, one barrier per tile). LDS rows are padded to 144
// bytes so the 16 rows one ds_read_b128 touches fall on distinct banks.
//
// MFMA operand mapping (v_mfma_f32_16x16x32_bf16 / v_mfma_i32_16x16x64_i8):
// the weights are the "A" operand (rows = output channels) and the gathered
// activations the "B" operand (columns = pixels). Lane l supplies row/column
// (l % 16) and 16 bytes of K at byte offset 16*(l / 16); it receives D rows
// 4*(l/16) .. 4*(l/16)+3 of column l % 16, i.e. four consecutive output
// channels of one pixel, which the epilogue stores as one NHWC vector.
#include "device_common.h"
#include "plan.h"

namespace convnhwc {

const TileCfg kTiles[kNumTiles] = {
    {32, 256, 1, 4},   // 1: narrow layers (Cout <= 32)
    {64, 128, 2, 2},   // 2
    {64, 256, 1, 4},   // 3: Cout = 64, many pixels
    {128, 128, 2, 2},  // 4
    {128, 64, 2, 2},   // 5
    {64, 64, 2, 2},    // 6: few pixels
    {256, 128, 2, 2},  // 7
    {128, 256, 2, 2},  // 8
};

namespace {

constexpr int kBKB = 128;     // bytes of K per tile row
constexpr int kLdsRow = 144;  // padded LDS row stride (bytes)

struct IgArgs {
  const char* x;
  const char* w;
  void* y;
  Epi e;
  Geometry g;
  int out_kind;
  int nco_tiles;
};

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

__device__ __forceinline__ i32x4 zero4() { return i32x4{0, 0, 0, 0}; }

__device__ __forceinline__ i32x4 ld16(const char* p) {
  return *reinterpret_cast<const i32x4*>(p);
}

// Read one element of ESZ bytes as an unsigned integer.
template <int ESZ>
__device__ __forceinline__ uint32_t ld_elem(const char* p) {
  if constexpr (ESZ == 2)
    return *reinterpret_cast<const uint16_t*>(p);
  else
    return *reinterpret_cast<const uint8_t*>(p);
}

// Put element e (of 16/ESZ) into a 16-byte chunk held as four dwords.
template <int ESZ>
__device__ __forceinline__ void put_elem(uint32_t (&wds)[4], int e, uint32_t v) {
  constexpr int PER = 4 / ESZ;
  wds[e / PER] |= v << (8 * ESZ * (e % PER));
}

// ---------------------------------------------------------------- kernel

template <int ESZ, int TCO, int TPX, int WCO, int WPX, int LOADER>
__global__ __launch_bounds__(256) void igemm_kernel(IgArgs a) {
  constexpr int VE = 16 / ESZ;      // elements per 16-byte chunk
  constexpr int BKE = kBKB / ESZ;   // elements per K-tile row
  constexpr int FCO = TCO / WCO / 16;
  constexpr int FPX = TPX / WPX / 16;
  constexpr int ACH = TCO / 32;     // 16-byte A chunks per thread per tile
  constexpr int BCH = TPX / 32;     // 16-byte B chunks per thread per tile
  static_assert(FCO >= 1 && FPX >= 1 && WCO * WPX == 4, "bad tile");
  typedef typename Mfma<ESZ>::acc_t acc_t;

  __shared__ __attribute__((aligned(16))) char smem[2 * (TCO + TPX) * kLdsRow];
  char* const As = smem;
  char* const Bs = smem + 2 * TCO * kLdsRow;

  const Geometry g = a.g;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wco = wave / WPX;
  const int wpx = wave % WPX;

  // Tiles are handed to the 8 XCDs round-robin by workgroup id; remap so each
  // XCD (own L2) gets a contiguous run of tiles that share activation rows.
  int lin = blockIdx.x;
  const int nwg = gridDim.x;
  if ((nwg & 7) == 0) lin = (lin & 7) * (nwg >> 3) + (lin >> 3);
  const int co0 = (lin % a.nco_tiles) * TCO;
  const int px0 = (lin / a.nco_tiles) * TPX;
  const int hw_o = g.ho * g.wo;

  // ---- per-thread loader state -------------------------------------
  // VEC / 1X1: chunk j of this thread is (row tid/8 + 32 j, column tid%8).
  // GENERIC:   chunk j of this thread is (row tid%T, column (tid/T)*CH + j).
  int b_base[BCH], b_hi0[BCH], b_wi0[BCH];
  int kh_s = 0, kw_s = 0, ci_s = 0;  // VEC: decomposition of this thread's k
  {
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
    if constexpr (LOADER == LOAD_VEC) {
      const int k0 = (tid & 7) * VE;
      const int tap = k0 / g.c;
      ci_s = k0 - tap * g.c;
      kh_s = tap / g.kw;
      kw_s = tap - kh_s * g.kw;
    }
  }

  i32x4 ra[ACH], rb[BCH];

  // Fetch K-tile kt into registers (tiles are fetched in increasing order).
  auto fetch = [&](int kt) {
    const int kb = kt * BKE;
    if constexpr (LOADER == LOAD_GENERIC) {
      // A: weights, element-wise (K * ESZ need not be 16-byte aligned).
      {
        constexpr int G = 256 / TCO;
        constexpr int CH = 8 / G;
        const int row = tid % TCO, grp = tid / TCO;
        const int co = co0 + row;
        const int k_first = kb + grp * CH * VE;
        for (int j = 0; j < CH; ++j) {
          uint32_t wds[4] = {0, 0, 0, 0};
          for (int e = 0; e < VE; ++e) {
            const int k = k_first + j * VE + e;
            if (co < g.cout && k < g.k)
              put_elem<ESZ>(wds, e, ld_elem<ESZ>(a.w + ((size_t)co * g.k + k) * ESZ));
          }
          ra[j] = i32x4{(int)wds[0], (int)wds[1], (int)wds[2], (int)wds[3]};
        }
      }
      // B: activations, element-wise gather with bounds tests.
      {
        constexpr int G = 256 / TPX;
        constexpr int CH = 8 / G;
        const int grp = tid / TPX;
        const int k_first = kb + grp * CH * VE;
        int tap = k_first / g.c;
        int ci = k_first - tap * g.c;
        int kh = tap / g.kw;
        int kw = tap - kh * g.kw;
        for (int j = 0; j < CH; ++j) {
          uint32_t wds[4] = {0, 0, 0, 0};
          for (int e = 0; e < VE; ++e) {
            const int hi = b_hi0[0] + kh;
            const int wi = b_wi0[0] + kw;
            if (kh < g.kh && (unsigned)hi < (unsigned)g.h && (unsigned)wi < (unsigned)g.w)
              put_elem<ESZ>(wds, e,
                            ld_elem<ESZ>(a.x + (size_t)(b_base[0] + (kh * g.w + kw) * g.c + ci) * ESZ));
            if (++ci == g.c) {
              ci = 0;
              if (++kw == g.kw) {
                kw = 0;
                ++kh;
              }
            }
          }
          rb[j] = i32x4{(int)wds[0], (int)wds[1], (int)wds[2], (int)wds[3]};
        }
      }
    } else {
      const int kc = kb + (tid & 7) * VE;  // first element of this thread's chunk
      // A: weights [cout][K], K-contiguous, 16-byte chunks.
      for (int j = 0; j < ACH; ++j) {
        const int co = co0 + (tid >> 3) + 32 * j;
        ra[j] = (co < g.cout && kc < g.k) ? ld16(a.w + ((size_t)co * g.k + kc) * ESZ) : zero4();
      }
      if constexpr (LOADER == LOAD_1X1) {
        for (int j = 0; j < BCH; ++j)
          rb[j] = (b_hi0[j] == 0 && kc < g.k) ? ld16(a.x + (size_t)(b_base[j] + kc) * ESZ) : zero4();
      } else {
        const int tap_off = (kh_s * g.w + kw_s) * g.c + ci_s;
        const bool kin = kh_s < g.kh;
        for (int j = 0; j < BCH; ++j) {
          const int hi = b_hi0[j] + kh_s;
          const int wi = b_wi0[j] + kw_s;
          rb[j] = (kin && (unsigned)hi < (unsigned)g.h && (unsigned)wi < (unsigned)g.w)
                      ? ld16(a.x + (size_t)(b_base[j] + tap_off) * ESZ)
                      : zero4();
        }
        // advance this thread's k by one tile
        ci_s += BKE;
        while (ci_s >= g.c) {
          ci_s -= g.c;
          if (++kw_s == g.kw) {
            kw_s = 0;
            ++kh_s;
          }
        }
      }
    }
  };

  auto stash = [&](int buf) {
    char* A = As + buf * TCO * kLdsRow;
    char* B = Bs + buf * TPX * kLdsRow;
    if constexpr (LOADER == LOAD_GENERIC) {
      {
        constexpr int G = 256 / TCO;
        constexpr int CH = 8 / G;
        const int row = tid % TCO, grp = tid / TCO;
        for (int j = 0; j < CH; ++j)
          *reinterpret_cast<i32x4*>(A + row * kLdsRow + (grp * CH + j) * 16) = ra[j];
      }
      {
        constexpr int G = 256 / TPX;
        constexpr int CH = 8 / G;
        const int row = tid % TPX, grp = tid / TPX;
        for (int j = 0; j < CH; ++j)
          *reinterpret_cast<i32x4*>(B + row * kLdsRow + (grp * CH + j) * 16) = rb[j];
      }
    } else {
      const int col = (tid & 7) * 16;
      for (int j = 0; j < ACH; ++j)
        *reinterpret_cast<i32x4*>(A + ((tid >> 3) + 32 * j) * kLdsRow + col) = ra[j];
      for (int j = 0; j < BCH; ++j)
        *reinterpret_cast<i32x4*>(B + ((tid >> 3) + 32 * j) * kLdsRow + col) = rb[j];
    }
  };

  acc_t acc[FCO][FPX];
  for (int i = 0; i < FCO; ++i)
    for (int j = 0; j < FPX; ++j) acc[i][j] = acc_t{0, 0, 0, 0};

  const int lrow = lane & 15;
  const int lk = (lane >> 4) * 16;
  const int a_row0 = wco * (TCO / WCO) + lrow;
  const int b_row0 = wpx * (TPX / WPX) + lrow;

  const int nkt = (g.k + BKE - 1) / BKE;
  fetch(0);
  stash(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nkt;
    if (more) fetch(kt + 1);
    const char* A = As + cur * TCO * kLdsRow;
    const char* B = Bs + cur * TPX * kLdsRow;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      i32x4 af[FCO], bf[FPX];
#pragma unroll
      for (int i = 0; i < FCO; ++i) af[i] = ld16(A + (a_row0 + 16 * i) * kLdsRow + s * 64 + lk);
#pragma unroll
      for (int j = 0; j < FPX; ++j) bf[j] = ld16(B + (b_row0 + 16 * j) * kLdsRow + s * 64 + lk);
#pragma unroll
      for (int i = 0; i < FCO; ++i)
#pragma unroll
        for (int j = 0; j < FPX; ++j) acc[i][j] = Mfma<ESZ>::run(af[i], bf[j], acc[i][j]);
    }
    if (more) stash(cur ^ 1);
    __syncthreads();
  }

  // ---- fused epilogue -------------------------------------------------
  const int co_w = co0 + wco * (TCO / WCO) + 4 * (lane >> 4);
  const int px_w = px0 + wpx * (TPX / WPX) + (lane & 15);
  const bool vec4 = (g.cout & 3) == 0;
#pragma unroll
  for (int i = 0; i < FCO; ++i) {
    const int co = co_w + 16 * i;
    if (co >= g.cout) continue;
    // per-channel constants of the 4 channels this lane owns
    float bsf[4] = {0.f, 0.f, 0.f, 0.f};
    int bsi[4] = {0, 0, 0, 0};
    float scl[4] = {0.f, 0.f, 0.f, 0.f};
    for (int r = 0; r < 4; ++r) {
      if (co + r < g.cout) {
        if constexpr (ESZ == 2) {
          if (a.e.bias) bsf[r] = a.e.bias[co + r];
        } else {
          if (a.e.ibias) bsi[r] = a.e.ibias[co + r];
          if (a.e.scale) scl[r] = a.e.scale[co + r];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < FPX; ++j) {
      const int px = px_w + 16 * j;
      if (px >= g.m) continue;
      const size_t off = (size_t)px * g.cout + co;
      if constexpr (ESZ == 2) {
        uint32_t hbits[4];
        for (int r = 0; r < 4; ++r)
          hbits[r] = f32_to_bf16_bits(apply_act(acc[i][j][r] + bsf[r], a.e.act));
        uint16_t* yp = reinterpret_cast<uint16_t*>(a.y) + off;
        if (vec4) {
          uint2 v;
          v.x = hbits[0] | (hbits[1] << 16);
          v.y = hbits[2] | (hbits[3] << 16);
          *reinterpret_cast<uint2*>(yp) = v;
        } else {
          for (int r = 0; r < 4; ++r)
            if (co + r < g.cout) yp[r] = (uint16_t)hbits[r];
        }
      } else if (a.out_kind == OUT_I32) {
        int v[4];
        for (int r = 0; r < 4; ++r) {
          v[r] = acc[i][j][r] + bsi[r];
          if (a.e.act == ACT_RELU) v[r] = v[r] > 0 ? v[r] : 0;
        }
        int32_t* yp = reinterpret_cast<int32_t*>(a.y) + off;
        if (vec4) {
          *reinterpret_cast<i32x4*>(yp) = i32x4{v[0], v[1], v[2], v[3]};
        } else {
          for (int r = 0; r < 4; ++r)
            if (co + r < g.cout) yp[r] = v[r];
        }
      } else {
        uint32_t q[4];
        for (int r = 0; r < 4; ++r)
          q[r] = (uint32_t)(requant_i8(acc[i][j][r] + bsi[r], scl[r], a.e.act) & 0xff);
        int8_t* yp = reinterpret_cast<int8_t*>(a.y) + off;
        if (vec4) {
          *reinterpret_cast<uint32_t*>(yp) = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
        } else {
          for (int r = 0; r < 4; ++r)
            if (co + r < g.cout) yp[r] = (int8_t)q[r];
        }
      }
    }
  }
}

template <int ESZ, int TCO, int TPX, int WCO, int WPX>
hipError_t launch_tile(int loader, const IgArgs& args, int nwg, hipStream_t s) {
  switch (loader) {
    case LOAD_GENERIC:
      hipLaunchKernelGGL((igemm_kernel<ESZ, TCO, TPX, WCO, WPX, LOAD_GENERIC>), dim3(nwg), dim3(256), 0, s, args);
      break;
    case LOAD_VEC:
      hipLaunchKernelGGL((igemm_kernel<ESZ, TCO, TPX, WCO, WPX, LOAD_VEC>), dim3(nwg), dim3(256), 0, s, args);
      break;
    default:
      hipLaunchKernelGGL((igemm_kernel<ESZ, TCO, TPX, WCO, WPX, LOAD_1X1>), dim3(nwg), dim3(256), 0, s, args);
      break;
  }
  return hipGetLastError();
}

template <int ESZ>
hipError_t launch_esz(int tile, int loader, const IgArgs& args, int nwg, hipStream_t s) {
  switch (tile) {
    case 0: return launch_tile<ESZ, 32, 256, 1, 4>(loader, args, nwg, s);
    case 1: return launch_tile<ESZ, 64, 128, 2, 2>(loader, args, nwg, s);
    case 2: return launch_tile<ESZ, 64, 256, 1, 4>(loader, args, nwg, s);
    case 3: return launch_tile<ESZ, 128, 128, 2, 2>(loader, args, nwg, s);
    case 4: return launch_tile<ESZ, 128, 64, 2, 2>(loader, args, nwg, s);
    case 5: return launch_tile<ESZ, 64, 64, 2, 2>(loader, args, nwg, s);
    case 6: return launch_tile<ESZ, 256, 128, 2, 2>(loader, args, nwg, s);
    default: return launch_tile<ESZ, 128, 256, 2, 2>(loader, args, nwg, s);
  }
}

}  // namespace

hipError_t launch_igemm(const conv_plan* p, const void* x, const void* w, const Epi& e, void* y,
                        hipStream_t s) {
  IgArgs args;
  args.x = static_cast<const char*>(x);
  args.w = static_cast<const char*>(w);
  args.y = y;
  args.e = e;
  args.g = p->g;
  args.out_kind = p->out_kind;
  const TileCfg& t = kTiles[p->tile];
  args.nco_tiles = (p->g.cout + t.tco - 1) / t.tco;
  const int npx = (p->g.m + t.tpx - 1) / t.tpx;
  const int nwg = npx * args.nco_tiles;
  if (p->in_esz == 2) return launch_esz<2>(p->tile, p->loader, args, nwg, s);
  return launch_esz<1>(p->tile, p->loader, args, nwg, s);
}

}  // namespace convnhwc
