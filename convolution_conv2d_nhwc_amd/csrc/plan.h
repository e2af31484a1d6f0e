// plan.h -- host-side plan and the launchers each kernel file exports to the
// C-ABI layer (conv_api.cpp). Internal: not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/conv_nhwc.h"

namespace convnhwc {

enum Path {
  PATH_IGEMM = 1,  // MFMA implicit GEMM (bf16 / int8), dense KxK and 1x1
  PATH_DW = 2,     // depthwise 3x3, VALU stencil
  PATH_F32 = 3,    // true-fp32 direct convolution, VALU
  PATH_SMALLK = 4, // MFMA, operands straight from global memory: short K, odd Cin
  PATH_XL = 6,     // MFMA, direct-to-LDS loads, software-pipelined
  PATH_WS = 7,     // MFMA, weights held in registers, short reductions
  PATH_HALO = 8,   // MFMA, 3x3 over 32/64 channels: weights in registers, input windows in LDS
  PATH_STEM = 9    // MFMA, 3x3 stride-1 first layer on 16-byte (8-channel) pixels, windows in LDS
};

// How the implicit-GEMM kernel gathers its activation operand.
enum Loader {
  LOAD_GENERIC = 0,  // element-wise gather: any channel count
  LOAD_VEC = 1,      // 16-byte channel vectors: c_in * elem_size % 16 == 0
  LOAD_1X1 = 2,      // 1x1, stride 1, pad 0: the input is the GEMM operand
  LOAD_TAP = 3,      // Cin * elem_size % 128 == 0 and KH*KW <= 32: every K-tile
                     // lies in one tap, so the tap offset is wave-uniform
  LOAD_CAT = 4       // 1x1 over the channel concat of two maps, each optionally
                     // upsampled x2 (conv_run_upcat): every K-tile lies in one map
};

// One tile configuration of the implicit-GEMM kernel: a workgroup of four
// wave64s computes tco output channels x tpx output pixels; the waves are
// arranged wco x wpx.
struct TileCfg {
  int tco, tpx, wco, wpx;
};

constexpr int kNumTiles = 4;
extern const TileCfg kTiles[kNumTiles];  // index = algo - 1

// Tile configurations of the large-layer kernel; desc.algo kAlgoXl + i forces
// configuration i.
constexpr int kNumXlTiles = 6;
constexpr int kAlgoXl = kNumTiles + 1;
// desc.algo kAlgoWs forces the weight-stationary kernel, kAlgoHalo the halo
// kernel.
constexpr int kAlgoWs = kAlgoXl + kNumXlTiles;
constexpr int kAlgoHalo = kAlgoWs + 1;
constexpr int kAlgoLast = kAlgoHalo;
extern const TileCfg kXlTiles[kNumXlTiles];

struct Geometry {
  int n, h, w, c;        // input
  int ho, wo, cout;      // output
  int kh, kw, sh, sw, ph, pw;
  int m;                 // n * ho * wo (GEMM pixels)
  int k;                 // kh * kw * c (GEMM reduction length)
};

}  // namespace convnhwc

struct conv_plan {
  conv_desc d;
  convnhwc::Geometry g;
  int path;
  int loader;   // PATH_IGEMM
  int tile;     // PATH_IGEMM: index into kTiles; PATH_XL: into kXlTiles; PATH_DW: forced rows per lane (0 = chosen)
  int out_kind; // convnhwc::OutKind
  int in_esz, out_esz;
  int64_t x_bytes, w_bytes, y_bytes, b_bytes;
  int ksplit;       // PATH_IGEMM / PATH_XL: K-splits (1 = none)
  int kt_per;       // K-tiles per split
  void* ws;         // split-K partial sums [ksplit][m][cout] (fp32/int32), device
  int64_t ws_bytes;
  int ws_device;    // device the workspace lives on
  int ws_owned;     // ws was allocated for this plan (conv_destroy frees it)
  int cus;          // compute units of the device current at prepare (256 without one)
  int wq;           // weights as bfp8 blocks (conv_desc.w_format == CONV_W_BFP8)
  int kp;           // wq: K padded to a multiple of 16
  int64_t w_exp_off;  // wq: byte offset of the exponents in the weight image
};

namespace convnhwc {

hipError_t launch_igemm(const conv_plan* p, const void* x, const void* w, const Epi& e, void* y,
                        hipStream_t s);
bool xl_eligible(const Geometry& g, int esz, int loader, int tile);
int igemm_stages(int loader, int tile);  // register stages of the implicit-GEMM kernel
int co_group_for(const conv_plan* p, int nco, int npx);  // tile order of the implicit-GEMM kernels
hipError_t launch_xl(const conv_plan* p, const void* x, const void* w, const Epi& e, void* y, hipStream_t s);
// p's 1x1 layer over the concat of s0 (c0b bytes per pixel, upsampled x2
// when up0) and s1 (the rest of the channels, upsampled when up1), unsplit,
// on p's implicit-GEMM tile when p has one, else the 64x64 tile.
hipError_t launch_igemm_cat(const conv_plan* p, const void* s0, int c0b, int up0, const void* s1, int up1,
                            const void* w, const Epi& e, void* y, hipStream_t s);
hipError_t launch_igemm_fused(const conv_plan* p1, const conv_plan* p2, const void* x, const void* w1, const Epi& e1,
                              const void* w2, const Epi& e2, void* y, hipStream_t s);
int ws_ksteps(const Geometry& g, int esz, int loader);  // 0: not for the weight-stationary kernel
int ws_grid_x(const conv_plan* p);
hipError_t launch_ws(const conv_plan* p, const void* x, const void* w, const Epi& e, void* y, hipStream_t s);
bool stem_eligible(const conv_desc& d, const Geometry& g, int64_t x_stride);
int stem_grid(const conv_plan* p);  // workgroups per 32 output channels
hipError_t launch_stem(const conv_plan* p, const void* x, const void* w, const Epi& e, void* y, hipStream_t s);
bool stem_mosaic_ok(const conv_plan* p, int64_t th, int64_t tw);  // the stem plan reads th x tw tiles
hipError_t launch_stem_mosaic(const conv_plan* p, const void* tiles, int tiles_f32, int th, int tw, const void* w,
                              const Epi& e, void* y, hipStream_t s);
bool halo_eligible(const conv_desc& d, const Geometry& g);
bool halo_preferred(const conv_desc& d, const Geometry& g);  // the automatic choice
bool halo_fusable(const conv_desc& d, const Geometry& g);    // the fused launch can use the halo kernel
int halo_grid(const conv_plan* p, int tco);  // workgroups of a launch with tco channels per workgroup
hipError_t launch_halo(const conv_plan* p, const void* x, const void* w, const Epi& e, void* y, hipStream_t s);
hipError_t launch_halo_fused(const conv_plan* p1, const conv_plan* p2, const void* x, const void* w1, const Epi& e1,
                             const void* w2, const Epi& e2, void* y, hipStream_t s);
hipError_t launch_smallk(const conv_plan* p, const void* x, const void* w, const Epi& e, void* y,
                         hipStream_t s);
void smallk_shape(const Geometry& g, int esz, int* fco, int* ks);
void dw_shape(const conv_plan* p, int* ve, int* pw, int* th);
int dw_prefetch_rows();  // input rows in flight per lane in the row-window kernels
hipError_t launch_dw(const conv_plan* p, const void* x, const void* w, const Epi& e, void* y,
                     hipStream_t s);
hipError_t launch_f32(const conv_plan* p, const void* x, const void* w, const Epi& e, void* y,
                      hipStream_t s);
int spp_chunks(int64_t n, int64_t h, int64_t w, int64_t c, int dtype);  // 0: map too large
hipError_t launch_spp(const void* x, int dtype, void* y, int64_t n, int64_t h, int64_t w, int64_t c, int64_t x_bytes,
                      hipStream_t s);
hipError_t launch_upcat(const void* s0, int64_t c0_bytes, int up0, const void* s1, int64_t c1_bytes, int up1, void* y,
                        int64_t n, int64_t ho, int64_t wo, hipStream_t s);
hipError_t launch_bfp8_pack(const void* w, int w_f32, int rows, int k, void* packed, hipStream_t s);
hipError_t launch_mosaic(const void* tiles, int in_f32, void* canvas, int out_f32, int m, int th,
                         int tw, int c, int c_pad, hipStream_t s);

}  // namespace convnhwc
