// igemm_xl.hip -- implicit-GEMM convolution for large layers: 256- and
// 128-channel by 128- to 256-pixel workgroup tiles, a 128x112 to 128x128
// output block per wave (64x112 to 64x128 for 128-channel tiles), and a
// software pipeline that keeps the matrix cores fed from one wave per SIMD.
//
// The GEMM view, operand layout, buffer loads and LDS swizzle are those of
// igemm.hip; this kernel differs in how it spends LDS bandwidth and latency.
//
// LDS bandwidth. Every MFMA operand is read from LDS once per wave, so the
// bytes read per MFMA fall as the wave's output block grows: a 128x128 block
// reads (128 + 128) rows per K-step for 64 MFMAs, a quarter of what a 32x32
// block needs per MFMA.
//
// Loads. Operands go from global memory straight into LDS (buffer loads with
// the LDS as destination, 16 bytes per lane, no registers); each lane fetches
// the chunk that lands its 16 bytes at the XOR-swizzled position. Measured on
// MI355X these loads move about 61 bytes per clock per CU and do not overlap
// the MFMAs, so a K-tile costs about its MFMA cycles plus 17 clocks per KiB
// loaded; conv_api.cpp picks the tile shape from that model.
//
// Pipeline. Two LDS buffers, one barrier per K-tile, each K-tile split at the
// barrier into two halves that never wait on their own operands:
//   half 1: run the K-step-0 MFMAs of tile t (operands read during the
//           previous half 2) while reading the K-step-1 operands of tile t;
//   barrier (the loads of tile t+1 have landed; nobody reads tile t's
//           buffer any more);
//   half 2: issue the loads of tile t+2 into tile t's buffer; run the
//           K-step-1 MFMAs of tile t while reading the K-step-0 operands of
//           tile t+1.
//
// Only the tap and 1x1 loaders (Cin * elem_size a multiple of 128 bytes) are
// offered, and Cout must be a multiple of the channel tile, so every weight
// row of a tile exists and a K-tile never straddles two taps.
#include "igemm_common.h"

namespace convnhwc {

const TileCfg kXlTiles[kNumXlTiles] = {
    {256, 256, 2, 2},  // 128x128 per wave
    {256, 128, 2, 2},  // 128x64 per wave
    {128, 256, 2, 2},  // 64x128 per wave (Cout = 128)
    {256, 224, 2, 2},  // 128x112 per wave: fills a few more CUs than 256x256
    {128, 224, 2, 2},  // 64x112 per wave
    {256, 160, 2, 2},  // 128x80 per wave
};

namespace {


struct XlArgs {
  const char* x;
  const char* w;
  void* y;
  Epi e;
  Geometry g;
  int out_kind;
  int nco_tiles;
  int x_bytes;
  int w_bytes;
  int x_shift;     // LOAD_TAP: bytes the x descriptor starts before x
  int co_group;    // tile order: channel tiles per group, as in igemm.hip
  int ksplit;      // K-splits (gridDim.y); > 1 writes raw partial sums to ws
  int kt_per;      // K-tiles per split
  void* ws;        // [ksplit][m][cout] fp32 / int32 partial sums
};

// MFMA with the accumulator tied to one AGPR quad (the compiler's own MFMA
// selection gives the result a different AGPR quad than the input and copies
// it back every iteration, which costs more issue slots than the MFMAs).
// Operands A/B come straight from LDS reads; the accumulator is only ever
// touched by MFMAs of the same opcode between the two guards below, for which
// the hardware interlocks back-to-back dependent issue.
template <int ESZ>
struct MfmaAgpr;
template <>
struct MfmaAgpr<2> {
  static __device__ __forceinline__ void run(f32x4& c, const i32x4& a, const i32x4& b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b) : "memory");
  }
};
template <>
struct MfmaAgpr<1> {
  static __device__ __forceinline__ void run(i32x4& c, const i32x4& a, const i32x4& b) {
    asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b) : "memory");
  }
};

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at lds + 16 l (lds is wave-uniform); an out-of-range offset writes zeros.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, (int)voff, soff, 0,
                                           0);
}

// Wait until every vector-memory load of this wave, the direct-to-LDS ones
// included, has completed.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wait states between a VALU write of an accumulator and its first MFMA, and
// between its last MFMA and a VALU read of it. The guards are volatile, so
// they keep their order relative to the MFMAs: every accumulator gets its own
// guard plus the guards of all accumulators after it.
template <typename T>
__device__ __forceinline__ void agpr_guard(T& c) {
  asm volatile("s_nop 4" : "+a"(c));
}

template <int ESZ, int TCO, int TPX, int LOADER>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void igemm_xl_kernel(XlArgs a) {
  constexpr int FCO = TCO / 32;  // 16-row fragments per wave (2x2 waves)
  constexpr int FPX = TPX / 32;
  constexpr int ACH = TCO / 32;  // 16-byte chunks per thread per K-tile
  constexpr int BCH = TPX / 32;
  constexpr int NMF = FCO * FPX;  // MFMAs per K-step per wave
  static_assert(LOADER == LOAD_TAP || LOADER == LOAD_1X1, "vector loaders only");
  typedef typename Mfma<ESZ>::acc_t acc_t;

  __shared__ __attribute__((aligned(16))) char smem[2 * (TCO + TPX) * kBKB];
  char* const As = smem;
  char* const Bs = smem + 2 * TCO * kBKB;

  const Geometry g = a.g;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wco = wave >> 1;
  const int wpx = wave & 1;

  // XCD-aware tile order, as in igemm.hip.
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

  // ---- loader state: chunk j of this thread is (row tid/8 + 32 j, column tid%8)
  const int row0 = tid >> 3;
  // The direct-to-LDS load writes lane l's 16 bytes at position l of the
  // wave's 1 KiB LDS block (row l / 8, chunk l % 8); to land the swizzled
  // layout (chunk c of row r at c ^ (r & 7)) lane l fetches chunk
  // (l % 8) ^ (l / 8) of its row (row & 7 == l / 8 for every block).
  const int c16 = ((tid & 7) ^ ((tid >> 3) & 7)) * 16;
  const int cbytes = g.c * ESZ;
  const int kbytes = g.k * ESZ;
  const int nkt_all = kbytes / kBKB;
  const int kt0 = blockIdx.y * a.kt_per;
  const int nkt = min(a.kt_per, nkt_all - kt0);
  const __amdgpu_buffer_rsrc_t rw = rsrc(a.w, a.w_bytes);
  const __amdgpu_buffer_rsrc_t rx =
      LOADER == LOAD_TAP ? rsrc(a.x - a.x_shift, a.x_bytes + a.x_shift) : rsrc(a.x, a.x_bytes);
  // weight rows co0 + row0 + 32 j all exist (Cout % TCO == 0); row j is
  // 32 * kbytes further on, which enters the load as its scalar offset
  const uint32_t voff_a = (uint32_t)((co0 + row0) * kbytes + c16);
  const int astride = 32 * kbytes;
  uint32_t voff_b[BCH];
  uint32_t tmask[BCH];  // LOAD_TAP: bit t = tap t of the row lies in the image
#pragma unroll
  for (int j = 0; j < BCH; ++j) {
    const int p = px0 + row0 + 32 * j;
    voff_b[j] = kOOB;
    tmask[j] = 0;
    if (p < g.m) {
      const int n = p / hw_o;
      const int r = p - n * hw_o;
      const int ho = r / g.wo;
      const int wo = r - ho * g.wo;
      if constexpr (LOADER == LOAD_1X1) {
        voff_b[j] = (uint32_t)(p * cbytes + c16);
        tmask[j] = 1;
      } else {
        const int hi0 = ho * g.sh - g.ph;
        const int wi0 = wo * g.sw - g.pw;
        voff_b[j] = (uint32_t)(((n * g.h + hi0) * g.w + wi0) * cbytes + a.x_shift + c16);
        uint32_t m = 0;
        for (int kh = 0, tap = 0; kh < g.kh; ++kh)
          for (int kw = 0; kw < g.kw; ++kw, ++tap)
            if ((unsigned)(hi0 + kh) < (unsigned)g.h && (unsigned)(wi0 + kw) < (unsigned)g.w) m |= 1u << tap;
        tmask[j] = m;
      }
    }
  }
  // Uniform position (channel block, tap) of the next K-tile to fetch.
  // LOAD_TAP walks the K-tiles channel block by channel block, all taps of a
  // block in turn: the taps of one block re-read the same input rows shifted
  // by a pixel or a row, so those reads hit in L2 instead of coming back a
  // whole channel sweep later. K-tile kt is block kt / taps, tap kt % taps;
  // the weight bytes of (tap, block) are contiguous in every OHWI row.
  const int ntaps = g.kh * g.kw;
  int t_kh = 0, t_kw = 0, t_cb = 0;
  if constexpr (LOADER == LOAD_TAP) {
    const int cb0 = kt0 / ntaps;
    const int tap0 = kt0 - cb0 * ntaps;
    t_cb = cb0 * kBKB;
    t_kh = tap0 / g.kw;
    t_kw = tap0 - t_kh * g.kw;
  }

  // Global loads of K-tile kt, one 16-byte chunk at a time (tiles are
  // fetched in increasing order). fetch_begin takes the tile's uniform
  // offsets and advances the tap position; a tile past the reduction reads
  // zeros and costs no memory traffic.
  struct Fetch {
    bool live;
    int soff_a;  // K byte offset of the tile in a weight row
    int soff_b;  // tap offset + channel block (LOAD_TAP), kt * 128 (LOAD_1X1)
    int tap;
  };
  auto fetch_begin = [&](int kt) {
    Fetch f;
    f.live = kt < nkt_all;
    f.tap = 0;
    if constexpr (LOADER == LOAD_TAP) {
      f.tap = t_kh * g.kw + t_kw;
      f.soff_a = f.tap * cbytes + t_cb;
      f.soff_b = f.live ? (t_kh * g.w + t_kw) * cbytes + t_cb : 0;
      if (++t_kw == g.kw) {
        t_kw = 0;
        if (++t_kh == g.kh) {
          t_kh = 0;
          t_cb += kBKB;
        }
      }
    } else {
      f.soff_a = kt * kBKB;
      f.soff_b = f.live ? kt * kBKB : 0;
    }
    return f;
  };
  // Chunk c < ACH: weight rows row0 + 32 c; else pixel rows row0 + 32 (c - ACH).
  // One instruction per wave moves 8 rows (1 KiB) from global memory straight
  // into LDS buffer buf, bypassing registers.
  const int wave_blk = (tid >> 6) * 1024;  // this wave's 1 KiB block of each 32-row group
  auto dma_chunk = [&](const Fetch& f, int buf, auto cc) {
    constexpr int c = decltype(cc)::value;
    if constexpr (c < ACH) {
      dma16(rw, As + buf * TCO * kBKB + c * 4096 + wave_blk, f.live ? voff_a : kOOB,
            f.live ? f.soff_a + c * astride : 0);
    } else {
      constexpr int j = c - ACH;
      bool ok = f.live;
      if constexpr (LOADER == LOAD_TAP) ok = ok && ((tmask[j] >> (f.tap & 31)) & 1u);
      dma16(rx, Bs + buf * TPX * kBKB + j * 4096 + wave_blk, ok ? voff_b[j] : kOOB, f.soff_b);
    }
  };
  auto dma_all = [&](int kt, int buf) {
    const Fetch f = fetch_begin(kt);
    StaticFor<0, ACH + BCH>::run([&](auto cc) { dma_chunk(f, buf, cc); });
  };

  // MFMA operand r of K-step s (0 or 1) of the tile in LDS buffer buf
  // (r < FCO: weight fragment r, else pixel fragment r - FCO): row (lane & 15)
  // of the 16-row fragment, chunk 4 s + lane / 16.
  const int a_row0 = wco * (TCO / 2) + (lane & 15);
  const int b_row0 = wpx * (TPX / 2) + (lane & 15);
  auto read_frag = [&](int buf, int s, auto rc, i32x4 (&af)[FCO], i32x4 (&bf)[FPX]) {
    constexpr int r = decltype(rc)::value;
    const int c = 4 * s + (lane >> 4);
    if constexpr (r < FCO)
      af[r] = *reinterpret_cast<const i32x4*>(As + buf * TCO * kBKB + lds_off(a_row0 + 16 * r, c));
    else
      bf[r - FCO] = *reinterpret_cast<const i32x4*>(Bs + buf * TPX * kBKB + lds_off(b_row0 + 16 * (r - FCO), c));
  };
  auto read_all = [&](int buf, int s, i32x4 (&af)[FCO], i32x4 (&bf)[FPX]) {
    StaticFor<0, FCO + FPX>::run([&](auto rc) { read_frag(buf, s, rc, af, bf); });
  };

  acc_t acc[FCO][FPX];
#pragma unroll
  for (int i = 0; i < FCO; ++i)
#pragma unroll
    for (int j = 0; j < FPX; ++j) acc[i][j] = acc_t{0, 0, 0, 0};

  // The accumulators live in AGPRs and every MFMA updates its accumulator in
  // place (see MfmaAgpr). The hazard guards order the AGPR zero-fill before
  // the first MFMA and the last MFMA before the epilogue reads.
  StaticFor<0, FCO>::run([&](auto ic) {
    StaticFor<0, FPX>::run([&](auto jc) { agpr_guard(acc[decltype(ic)::value][decltype(jc)::value]); });
  });
  // MFMAs number B .. E-1 of a K-step, in (i, j) row-major order
  auto mfma_range = [&](auto bc, auto ec, const i32x4 (&af)[FCO], const i32x4 (&bf)[FPX]) {
    StaticFor<decltype(bc)::value, decltype(ec)::value>::run([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      MfmaAgpr<ESZ>::run(acc[k / FPX][k % FPX], af[k / FPX], bf[k % FPX]);
    });
  };
  auto mfmas = [&](const i32x4 (&af)[FCO], const i32x4 (&bf)[FPX]) {
    mfma_range(std::integral_constant<int, 0>{}, std::integral_constant<int, NMF>{}, af, bf);
  };

  // LDS buffer t % 2 holds K-tile t. Tile t+1's loads were issued one
  // K-tile earlier; each step waits for them at its barrier.
  i32x4 a0[FCO], b0[FPX], a1[FCO], b1[FPX];
  dma_all(kt0, 0);
  dma_all(kt0 + 1, 1);
  wait_vmem();
  __syncthreads();
  read_all(0, 0, a0, b0);

  // One K-tile. Half 1 spreads the K-step-1 operand reads over the
  // K-step-0 MFMAs. After the barrier (tile t+1 complete and visible, every
  // read of buffer t % 2 done), half 2 issues the loads of tile t+2 into
  // buffer t % 2 and spreads the K-step-0 operand reads of tile t+1 over the
  // K-step-1 MFMAs. The MFMA statements are ordered memory barriers for the
  // compiler, so the interleaving is issued as written.
  constexpr int CH = ACH + BCH;
  constexpr int NR = FCO + FPX;
  auto step = [&](int t) {
    const int buf = t & 1;
    StaticFor<0, NR>::run([&](auto rc) {
      constexpr int r = decltype(rc)::value;
      mfma_range(std::integral_constant<int, r * NMF / NR>{}, std::integral_constant<int, (r + 1) * NMF / NR>{}, a0,
                 b0);
      read_frag(buf, 1, rc, a1, b1);
    });
    wait_vmem();
    __syncthreads();
    const Fetch f = fetch_begin(kt0 + t + 2);
    StaticFor<0, NR>::run([&](auto rc) {
      constexpr int r = decltype(rc)::value;
      if constexpr (r < CH) dma_chunk(f, buf, rc);
      read_frag(buf ^ 1, 0, rc, a0, b0);
      mfma_range(std::integral_constant<int, r * NMF / NR>{}, std::integral_constant<int, (r + 1) * NMF / NR>{}, a1,
                 b1);
    });
  };
  // K-tiles 0 .. nkt-2 of this split: the next tile always exists
  int t = 0;
  for (; t + 1 < nkt; ++t) step(t);
  // last K-tile; the loads issued past it read nothing anybody uses
  read_all(t & 1, 1, a1, b1);
  mfmas(a0, b0);
  mfmas(a1, b1);
  wait_vmem();
  StaticFor<0, FCO>::run([&](auto ic) {
    StaticFor<0, FPX>::run([&](auto jc) { agpr_guard(acc[decltype(ic)::value][decltype(jc)::value]); });
  });

  // ---- fused epilogue -------------------------------------------------
  const int co_w = co0 + wco * (TCO / 2) + 4 * (lane >> 4);
  const int px_w = px0 + wpx * (TPX / 2) + (lane & 15);
  if (a.ksplit > 1) {
    acc_t* ws = reinterpret_cast<acc_t*>(a.ws) + (size_t)blockIdx.y * g.m * (g.cout / 4);
    StaticFor<0, FCO>::run([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int co = co_w + 16 * i;
      StaticFor<0, FPX>::run([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        const int px = px_w + 16 * j;
        if (px < g.m) ws[(size_t)px * (g.cout / 4) + co / 4] = acc[i][j];
      });
    });
    return;
  }
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
}

template <int ESZ, int TCO, int TPX>
hipError_t launch_cfg(int loader, const XlArgs& args, dim3 grid, hipStream_t s) {
  if (loader == LOAD_TAP)
    hipLaunchKernelGGL((igemm_xl_kernel<ESZ, TCO, TPX, LOAD_TAP>), grid, dim3(256), 0, s, args);
  else
    hipLaunchKernelGGL((igemm_xl_kernel<ESZ, TCO, TPX, LOAD_1X1>), grid, dim3(256), 0, s, args);
  return hipGetLastError();
}

template <int ESZ>
hipError_t launch_esz(int tile, int loader, const XlArgs& args, dim3 grid, hipStream_t s) {
  switch (tile) {
    case 0: return launch_cfg<ESZ, 256, 256>(loader, args, grid, s);
    case 1: return launch_cfg<ESZ, 256, 128>(loader, args, grid, s);
    case 2: return launch_cfg<ESZ, 128, 256>(loader, args, grid, s);
    case 3: return launch_cfg<ESZ, 256, 224>(loader, args, grid, s);
    case 4: return launch_cfg<ESZ, 128, 224>(loader, args, grid, s);
    default: return launch_cfg<ESZ, 256, 160>(loader, args, grid, s);
  }
}

}  // namespace

bool xl_eligible(const Geometry& g, int esz, int loader, int tile) {
  if (loader != LOAD_TAP && loader != LOAD_1X1) return false;
  if (tile < 0 || tile >= kNumXlTiles) return false;
  return g.cout % kXlTiles[tile].tco == 0 && (int64_t)g.k * esz % kBKB == 0;
}

hipError_t launch_xl(const conv_plan* p, const void* x, const void* w, const Epi& e, void* y, hipStream_t s) {
  XlArgs args;
  args.x = static_cast<const char*>(x);
  args.w = static_cast<const char*>(w);
  args.y = y;
  args.e = e;
  args.g = p->g;
  args.out_kind = p->out_kind;
  args.x_bytes = (int)p->x_bytes;
  args.w_bytes = (int)p->w_bytes;
  args.x_shift = (p->g.ph * p->g.w + p->g.pw) * p->g.c * p->in_esz;
  const TileCfg& t = kXlTiles[p->tile];
  args.nco_tiles = p->g.cout / t.tco;
  const int npx = (p->g.m + t.tpx - 1) / t.tpx;
  args.co_group = co_group_for(p, args.nco_tiles, npx);
  args.ksplit = p->ksplit;
  args.kt_per = p->kt_per;
  args.ws = p->ws;
  const dim3 grid(npx * args.nco_tiles, p->ksplit);
  hipError_t err = p->in_esz == 2 ? launch_esz<2>(p->tile, p->loader, args, grid, s)
                                  : launch_esz<1>(p->tile, p->loader, args, grid, s);
  if (err != hipSuccess || p->ksplit == 1) return err;
  return launch_splitk_reduce(p, e, y, s);
}

}  // namespace convnhwc
