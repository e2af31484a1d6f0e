// patch3x3.hip -- dense 3x3 convolution (stride 1 or 2) on MFMA, with the
// input halo patch staged in LDS once and all nine taps read from it.
//
// An implicit GEMM fetches every input pixel once per tap that covers it
// (nine times for a 3x3 kernel). Here a workgroup owns a 2-D block of output
// pixels (BH rows x 16 columns of one image) and 64 output channels. For each
// block of CB bytes of input channels it copies the block's receptive field
// -- ((BH-1)*s+3) x (15*s+3) input pixels -- into LDS once; the B operand of
// the MFMA for tap (kh, kw) is then read straight out of that patch at pixel
// (row*s + kh, col*s + kw): the im2col rows exist only as LDS addresses.
// The weights of one (tap, channel block), 64 x CB bytes, stream through a
// double-buffered LDS slot, fetched two steps ahead into registers, stored
// while the MFMAs of the previous step run, one barrier per step (the
// same pipeline as the implicit-GEMM kernel).
//
// Layout in LDS: patch pixel pp holds CB bytes as 16-byte chunks; chunk j is
// stored at position j ^ swz(pp), swz(pp) = (pp >> (s-1)) & (CB/16 - 1), so
// that the 8 lanes of a ds_read_b128 (8 consecutive output columns, i.e.
// pixels pp, pp+s, pp+2s, ...) land on distinct positions. Weight rows use
// the implicit-GEMM swizzle (chunk ^ (row & 7)).
//
// Waves: the 4 waves split the BH output rows (BH/4 rows = 16-pixel MFMA
// fragments each) and all share the 64 channels (4 fragments).
#include <algorithm>

#include "device_common.h"
#include "mfma_epilogue.h"
#include "plan.h"

namespace convnhwc {
namespace {

constexpr uint32_t kOOB = 0x80000000u;

struct PatchArgs {
  const char* x;
  const char* w;
  void* y;
  Epi e;
  Geometry g;
  int out_kind;
  int x_bytes;
  int w_bytes;
  int nbh, nbw, nco;  // blocks along ho, wo, and 64-channel tiles
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}

__device__ __forceinline__ i32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
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

// ESZ: element size; S: stride; BH: output rows per block; CB: channel bytes
// per K-block (64 or 128).
template <int ESZ, int S, int BH, int CB>
__global__ __launch_bounds__(256) void patch3x3_kernel(PatchArgs a) {
  constexpr int BW = 16;
  constexpr int TCO = 64;
  constexpr int PH = (BH - 1) * S + 3;
  constexpr int PW = (BW - 1) * S + 3;
  constexpr int NPIX = PH * PW;
  constexpr int CPP = CB / 16;             // 16-byte chunks per patch pixel
  constexpr int KSTEPS = CB / 64;          // MFMA K-steps per (tap, block)
  constexpr int FPX = BH / 4;              // 16-pixel fragments (rows) per wave
  constexpr int FCO = TCO / 16;
  constexpr int PCH = (NPIX * CPP + 255) / 256;  // patch chunks per thread
  constexpr int WCH = TCO * CPP / 256;           // weight chunks per thread (>= 1)
  static_assert(WCH >= 1, "weight slot smaller than the workgroup");
  typedef typename Mfma<ESZ>::acc_t acc_t;

  __shared__ __attribute__((aligned(16))) char patch[NPIX * CB];
  __shared__ __attribute__((aligned(16))) char wslot[2][TCO * CB];

  const Geometry g = a.g;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const __amdgpu_buffer_rsrc_t rx = rsrc(a.x, a.x_bytes);
  const __amdgpu_buffer_rsrc_t rw = rsrc(a.w, a.w_bytes);

  // block coordinates (XCD-aware: each XCD takes a contiguous run)
  int lin = blockIdx.x;
  const int nwg = gridDim.x;
  if ((nwg & 7) == 0) lin = (lin & 7) * (nwg >> 3) + (lin >> 3);
  const int cot = lin % a.nco;
  int r = lin / a.nco;
  const int bw = r % a.nbw;
  r /= a.nbw;
  const int bh = r % a.nbh;
  const int n = r / a.nbh;
  const int co0 = cot * TCO;
  const int ho0 = bh * BH, wo0 = bw * BW;
  const int hi0 = ho0 * S - g.ph, wi0 = wo0 * S - g.pw;  // patch origin in the image

  const int cbytes = g.c * ESZ;
  const int nkb = cbytes / CB;          // channel blocks
  const int nsteps = nkb * 9;           // (block, tap) steps
  const int krow = g.k * ESZ;           // bytes of one OHWI weight row

  // ---- patch loader: thread chunk q = tid + 256 i -> (pixel, chunk) -------
  auto patch_fetch = [&](int kb, i32x4 (&pr)[PCH]) {
#pragma unroll
    for (int i = 0; i < PCH; ++i) {
      const int q = tid + 256 * i;
      const int pp = q / CPP, j = q % CPP;
      const int pr_ = pp / PW, pc = pp % PW;
      const int hi = hi0 + pr_, wi = wi0 + pc;
      const bool ok = q < NPIX * CPP && (unsigned)hi < (unsigned)g.h && (unsigned)wi < (unsigned)g.w;
      pr[i] = bload16(rx, ok ? (uint32_t)(((n * g.h + hi) * g.w + wi) * cbytes + kb * CB + j * 16) : kOOB);
    }
  };
  auto patch_store = [&](const i32x4 (&pr)[PCH]) {
#pragma unroll
    for (int i = 0; i < PCH; ++i) {
      const int q = tid + 256 * i;
      if (q < NPIX * CPP) {
        const int pp = q / CPP, j = q % CPP;
        const int swz = (pp >> (S - 1)) & (CPP - 1);
        *reinterpret_cast<i32x4*>(patch + pp * CB + ((j ^ swz) << 4)) = pr[i];
      }
    }
  };

  // ---- weight slot loader: step st = kb*9 + tap -----------------------------
  // chunk q = tid + 256 i -> (row co, chunk j) of the 64 x CB slot
  auto w_fetch = [&](int st, i32x4 (&wr)[WCH]) {
    const int kb = st / 9, tap = st - kb * 9;
    const bool live = st < nsteps;
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int q = tid + 256 * i;
      const int row = q / CPP, j = q % CPP;
      const int co = co0 + row;
      const bool ok = live && co < g.cout;
      wr[i] = bload16(rw, ok ? (uint32_t)(co * krow + tap * cbytes + kb * CB + j * 16) : kOOB);
    }
  };
  auto w_store = [&](int buf, const i32x4 (&wr)[WCH]) {
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int q = tid + 256 * i;
      const int row = q / CPP, j = q % CPP;
      *reinterpret_cast<i32x4*>(&wslot[buf][row * CB + ((j ^ (row & (CPP - 1))) << 4)]) = wr[i];
    }
  };

  acc_t acc[FCO][FPX];
#pragma unroll
  for (int i = 0; i < FCO; ++i)
#pragma unroll
    for (int j = 0; j < FPX; ++j) acc[i][j] = acc_t{0, 0, 0, 0};

  const int lr = lane & 15, kg = lane >> 4;

  // MFMA of one step: weights from wslot[buf], pixels from the patch at tap
  auto compute = [&](int buf, int tap) {
    const int kh = tap / 3, kw = tap - kh * 3;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const int c = 4 * s + kg;  // chunk of this lane's 16 K bytes
      i32x4 af[FCO], bf[FPX];
#pragma unroll
      for (int i = 0; i < FCO; ++i) {
        const int row = 16 * i + lr;
        af[i] = *reinterpret_cast<const i32x4*>(&wslot[buf][row * CB + ((c ^ (row & (CPP - 1))) << 4)]);
      }
#pragma unroll
      for (int f = 0; f < FPX; ++f) {
        const int orow = wave * FPX + f;  // output row within the block
        const int pp = (orow * S + kh) * PW + lr * S + kw;
        const int swz = (pp >> (S - 1)) & (CPP - 1);
        bf[f] = *reinterpret_cast<const i32x4*>(patch + pp * CB + ((c ^ swz) << 4));
      }
#pragma unroll
      for (int i = 0; i < FCO; ++i)
#pragma unroll
        for (int f = 0; f < FPX; ++f) acc[i][f] = Mfma<ESZ>::run(af[i], bf[f], acc[i][f]);
    }
  };

  // ---- pipeline over steps st = (channel block, tap) -------------------------
  i32x4 pr[PCH];
  i32x4 w0[WCH], w1[WCH];
  patch_fetch(0, pr);
  w_fetch(0, w0);
  w_fetch(1, w1);
  w_store(0, w0);
  patch_store(pr);
  if (nkb > 1) patch_fetch(1, pr);  // next block's patch stays in flight
  w_fetch(2, w0);
  for (int st = 0; st < nsteps; ++st) {
    const int tap = st % 9;
    if (tap == 0 && st > 0) {
      // new channel block: every wave is done with the old patch
      __syncthreads();
      patch_store(pr);
      const int kb = st / 9;
      if (kb + 1 < nkb) patch_fetch(kb + 1, pr);
    }
    __syncthreads();
    // weights of step st+1 go into the other slot while step st computes
    if (st & 1) {
      if (st + 1 < nsteps) w_store(0, w0);
      compute(1, tap);
      w_fetch(st + 3, w0);
    } else {
      if (st + 1 < nsteps) w_store(1, w1);
      compute(0, tap);
      w_fetch(st + 3, w1);
    }
  }

  // ---- fused epilogue --------------------------------------------------------
  // A quad outside the image is sent past the output (px = m: not stored).
  const int wo = wo0 + lr;
  if ((g.cout & 3) == 0) {
    const OutRef o = out_ref(a.y, g.m, g.cout, ESZ == 2 ? 2 : (a.out_kind == OUT_I32 ? 4 : 1), a.e.res);
    with_epilogue<ESZ>(a.out_kind, a.e.act, [&](auto oc, auto ac) {
      constexpr int OUT = decltype(oc)::value, ACT = decltype(ac)::value;
#pragma unroll
      for (int i = 0; i < FCO; ++i) {
        const int co = co0 + 16 * i + 4 * kg;
        const QuadConsts q = load_quad_consts_t<ESZ>(a.e, co, g.cout);
#pragma unroll
        for (int f = 0; f < FPX; ++f) {
          const int ho = ho0 + wave * FPX + f;
          const int px = (ho < g.ho && wo < g.wo) ? (n * g.ho + ho) * g.wo + wo : g.m;
          store_quad_t<ESZ, OUT, ACT>(acc[i][f], q, co, px, o);
        }
      }
    });
    return;
  }
#pragma unroll
  for (int i = 0; i < FCO; ++i) {
    const int co = co0 + 16 * i + 4 * kg;
    if (co >= g.cout) continue;
    const QuadConsts q = load_quad_consts<ESZ>(a.e, co, g.cout);
#pragma unroll
    for (int f = 0; f < FPX; ++f) {
      const int ho = ho0 + wave * FPX + f;
      if (ho < g.ho && wo < g.wo)
        store_quad<ESZ>(acc[i][f], q, co, (n * g.ho + ho) * g.wo + wo, g.cout, a.out_kind, a.e.act, a.y, a.e.res);
    }
  }
}

template <int ESZ, int S, int BH, int CB>
hipError_t launch_cfg(const PatchArgs& base, hipStream_t s) {
  PatchArgs a = base;
  a.nbh = (a.g.ho + BH - 1) / BH;
  a.nbw = (a.g.wo + 15) / 16;
  a.nco = (a.g.cout + 63) / 64;
  const long nwg = (long)a.g.n * a.nbh * a.nbw * a.nco;
  hipLaunchKernelGGL((patch3x3_kernel<ESZ, S, BH, CB>), dim3((unsigned)nwg), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

// Patch-path eligibility: 3x3, stride 1 or 2 (both axes), groups 1, channel
// bytes a multiple of 64, and every tensor offset within 32 bits.
bool patch_eligible(const Geometry& g, int esz, int groups) {
  if (groups != 1 || g.kh != 3 || g.kw != 3 || g.sh != g.sw || (g.sh != 1 && g.sh != 2)) return false;
  return (g.c * esz) % 64 == 0;
}

int patch_cb(const Geometry& g, int esz) { return (g.c * esz) % 128 == 0 && g.sh == 1 ? 128 : 64; }

hipError_t launch_patch(const conv_plan* p, const void* x, const void* w, const Epi& e, void* y, hipStream_t s) {
  PatchArgs a;
  a.x = static_cast<const char*>(x);
  a.w = static_cast<const char*>(w);
  a.y = y;
  a.e = e;
  a.g = p->g;
  a.out_kind = p->out_kind;
  a.x_bytes = (int)p->x_bytes;
  a.w_bytes = (int)p->w_bytes;
  const int cb = patch_cb(p->g, p->in_esz);
  if (p->in_esz == 2) {
    if (p->g.sh == 1) return cb == 128 ? launch_cfg<2, 1, 16, 128>(a, s) : launch_cfg<2, 1, 16, 64>(a, s);
    return launch_cfg<2, 2, 8, 64>(a, s);
  }
  if (p->g.sh == 1) return cb == 128 ? launch_cfg<1, 1, 16, 128>(a, s) : launch_cfg<1, 1, 16, 64>(a, s);
  return launch_cfg<1, 2, 8, 64>(a, s);
}

}  // namespace convnhwc
