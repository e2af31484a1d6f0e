// conv_api.cpp -- the C ABI of the library (declared in include/conv_nhwc.h).
//
// conv_prepare validates a layer description and picks the kernel path and
// launch shape on the host alone; every unsupported case is a named error at
// preparation time rather than a wrong answer later (the nanoinfer README's
// load-time op/dtype validation after an int8-through-float* bug; the SiMa
// box-decode page's plan step that rejects unsupported profiles before any
// buffer is bound). conv_run checks pointers, alignment and aliasing, then
// only enqueues one kernel on the caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>

#include "device_common.h"
#include "plan.h"

using namespace convnhwc;

// The split-K workspace of conv_run_noalloc, one copy per device, held until
// the process ends. Host code never passes the name itself to a kernel or a
// copy: it stands for a host-side shadow, so only the per-device address from
// hipGetSymbolAddress is used.
static __device__ __align__(256) unsigned char scratch[CONV_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_last_hip_error[256] = "";

// Device address of `scratch` per device, looked up at the first
// conv_run_noalloc call on that device (with it current).
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

constexpr int64_t kMaxBytes = (int64_t)1 << 31;  // per tensor, see header
constexpr int32_t kMaxSmall = 1 << 16;           // kernel, stride, pad limit

int esz_of(int dt) {
  switch (dt) {
    case CONV_F32: return 4;
    case CONV_BF16: return 2;
    case CONV_I8: return 1;
    case CONV_I32: return 4;
    default: return 0;
  }
}

// Tile choice, fitted to a sweep of every tile on every layer of the YOLO
// workloads on MI355X (64x64 workgroup tiles keep 4-5 workgroups per CU and
// win on short reductions and small layers; 128-channel tiles win once the
// reduction is long and there are enough of them to fill 256 CUs twice).
int choose_tile(const Geometry& g, int esz) {
  const long kbytes = (long)g.k * esz;
  auto nwg = [&](int ti) {
    const TileCfg& t = kTiles[ti];
    return (long)((g.cout + t.tco - 1) / t.tco) * ((g.m + t.tpx - 1) / t.tpx);
  };
  // Measured on MI355X over every tile: 128x128 wins whenever it still gives
  // at least 384 workgroups (1.5 per CU); below that the 64x64 tile keeps
  // the CUs busy.
  (void)kbytes;
  const int t128x128 = 1, t64x64 = 0;
  if (g.cout >= 128 && nwg(t128x128) >= 384) return t128x128;
  return t64x64;
}

// The large-layer kernel for long reductions over 128-byte channel blocks.
// One workgroup fills a CU (its LDS), so a configuration's time is its number
// of rounds of 256 workgroups times one workgroup's time, modelled per K-tile
// as the MFMA cycles of a wave (32 per 16x16 fragment pair) plus the cycles
// the CU's load path needs for the tile's rows (about 17 per 1 KiB, measured
// on MI355X; the two do not overlap), plus the epilogue (about 70 cycles per
// output element of a lane). The cheapest configuration is taken when it keeps
// at least 160 workgroups busy and the reduction is at least 2 KiB per output
// for 256-channel tiles, 4 KiB for 128-channel tiles (below that the
// implicit-GEMM tiles measured faster).
int choose_xl(const Geometry& g, int esz, int loader) {
  const long kbytes = (long)g.k * esz;
  if (kbytes < 2048) return -1;
  const double nkt = (double)(kbytes / 128);
  int best = -1;
  double best_t = 0;
  for (int ti = 0; ti < kNumXlTiles; ++ti) {
    if (!xl_eligible(g, esz, loader, ti)) continue;
    const TileCfg& t = kXlTiles[ti];
    if (t.tco < 256 && kbytes < 4096) continue;
    const long nwg = (long)(g.cout / t.tco) * ((g.m + t.tpx - 1) / t.tpx);
    if (nwg < 160) continue;
    const double rounds = (double)((nwg + 255) / 256);
    const double per_kt = (t.tco / 32.0) * (t.tpx / 32.0) * 32.0 + (t.tco + t.tpx) / 8.0 * 17.0;
    const double wg = nkt * per_kt + 7000.0 + 70.0 * t.tco * t.tpx / 256.0;
    const double tt = rounds * wg;
    if (best < 0 || tt < best_t) {
      best = ti;
      best_t = tt;
    }
  }
  return best;
}

// Split the reduction when the output tiles alone would fill fewer than half
// of the 256 CUs (under 128 workgroups) and each split still has >= 8 K-tiles
// of 128 bytes: aim at ~448 workgroups, at most 8 splits (the 20x20x512 ->
// 1024 3x3 layer of the 640x640 stack, 112 tiles: 4 splits measured 0.7 us
// faster than 5, 6 to 8 slower). (Splitting layers
// of 128..255 tiles measured slower on MI355X: the partial sums' extra write
// and read outweigh the occupancy gained, e.g. 177 against 120 us for the
// 16x40x40x512 3x3 layer on the large-layer kernel.) The splits' raw partial sums go to a
// device workspace; a second kernel adds them in split order and applies the
// epilogue. Every split writes its whole [m][cout] slice before the second
// kernel reads it, so the workspace never needs clearing.
//   scratch == nullptr: the workspace is allocated here and owned by the plan
//     (CONV_E_NOMEM if that fails). With no HIP device at all the plan stays
//     unsplit: it can be described but not run.
//   scratch != nullptr: the workspace is `scratch` (scratch_bytes long) and
//     nothing is allocated; CONV_E_SCRATCH if the partials do not fit.
conv_status plan_split_k(conv_plan* p, void* scratch, int64_t scratch_bytes) {
  const Geometry& g = p->g;
  const TileCfg& t = p->path == PATH_XL ? kXlTiles[p->tile] : kTiles[p->tile];
  const int tco = t.tco, tpx = t.tpx, target = 448, min_per = 8;
  const long nwg = (long)((g.cout + tco - 1) / tco) * ((g.m + tpx - 1) / tpx);
  const int nkt = p->kt_per;
  if (nwg >= 128 || nkt < 16 || (g.cout & 3)) return CONV_OK;
  int s = (int)((target + nwg - 1) / nwg);
  s = s < 8 ? s : 8;
  s = s < nkt / min_per ? s : nkt / min_per;
  if (s < 2) return CONV_OK;
  const int per = (nkt + s - 1) / s;
  s = (nkt + per - 1) / per;
  if (s < 2) return CONV_OK;
  const int64_t bytes = (int64_t)s * g.m * g.cout * 4;
  void* ws = scratch;
  if (scratch) {
    if (bytes > scratch_bytes) return CONV_E_SCRATCH;
  } else {
    int dev = 0, ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev == 0 || hipGetDevice(&dev) != hipSuccess) {
      (void)hipGetLastError();  // no device: an unsplit plan that cannot run anyway
      return CONV_OK;
    }
    if (hipMalloc(&ws, bytes) != hipSuccess) {
      (void)hipGetLastError();
      return CONV_E_NOMEM;
    }
    p->ws_device = dev;
    p->ws_owned = 1;
  }
  p->ksplit = s;
  p->kt_per = per;
  p->ws = ws;
  p->ws_bytes = bytes;
  return CONV_OK;
}

bool ranges_overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  if (!a || !b || na <= 0 || nb <= 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

}  // namespace

namespace {

// Validate d and fill *p (memory the caller owns) with its plan. The split-K
// workspace comes from plan_split_k(p, scratch, scratch_bytes).
conv_status build_plan(const conv_desc* d, conv_plan* p, void* scratch, int64_t scratch_bytes) {
  if (d->n <= 0 || d->h <= 0 || d->w <= 0 || d->c_in <= 0 || d->c_out <= 0 || d->kh <= 0 ||
      d->kw <= 0 || d->stride_h <= 0 || d->stride_w <= 0 || d->pad_h < 0 || d->pad_w < 0 ||
      d->groups <= 0)
    return CONV_E_SHAPE;
  if (d->c_in % d->groups || d->c_out % d->groups) return CONV_E_SHAPE;
  if (d->kh > kMaxSmall || d->kw > kMaxSmall || d->stride_h > kMaxSmall || d->stride_w > kMaxSmall ||
      d->pad_h > kMaxSmall || d->pad_w > kMaxSmall)
    return CONV_E_UNSUPPORTED;
  if (d->h > kMaxBytes || d->w > kMaxBytes || d->c_in > kMaxBytes || d->c_out > kMaxBytes ||
      d->n > kMaxBytes)
    return CONV_E_UNSUPPORTED;
  const int64_t hp = d->h + 2 * (int64_t)d->pad_h - d->kh;
  const int64_t wp = d->w + 2 * (int64_t)d->pad_w - d->kw;
  if (hp < 0 || wp < 0) return CONV_E_SHAPE;
  const int64_t ho = hp / d->stride_h + 1, wo = wp / d->stride_w + 1;

  // dtype / output / activation combinations
  const int dt = d->dtype, ot = d->out_dtype;
  if (!(dt == CONV_F32 && ot == CONV_F32) && !(dt == CONV_BF16 && ot == CONV_BF16) &&
      !(dt == CONV_I8 && (ot == CONV_I8 || ot == CONV_I32)))
    return CONV_E_UNSUPPORTED;
  if (d->act < CONV_ACT_NONE || d->act > CONV_ACT_MISH) return CONV_E_UNSUPPORTED;
  if (ot == CONV_I32 && d->act != CONV_ACT_NONE && d->act != CONV_ACT_RELU) return CONV_E_UNSUPPORTED;

  const int in_esz = esz_of(dt), out_esz = esz_of(ot);
  const int64_t cg = d->c_in / d->groups;
  // elements from one input pixel to the next
  const int64_t xs = d->x_pixel_stride == 0 ? d->c_in : d->x_pixel_stride;
  if (xs < d->c_in) return CONV_E_SHAPE;
  const int64_t x_bytes = d->n * d->h * d->w * xs * in_esz;
  // bfp8 weights: int8 mantissas [c_out][Kp] and one exponent byte per 16
  const bool wq = d->w_format == CONV_W_BFP8;
  if (d->w_format != CONV_W_PLAIN && !wq) return CONV_E_UNSUPPORTED;
  const int64_t kp = ((int64_t)d->kh * d->kw * cg + 15) / 16 * 16;
  const int64_t w_bytes = wq ? d->c_out * kp + d->c_out * (kp / 16) : d->c_out * (int64_t)d->kh * d->kw * cg * in_esz;
  const int64_t y_bytes = d->n * ho * wo * d->c_out * out_esz;
  if (x_bytes >= kMaxBytes || w_bytes >= kMaxBytes || y_bytes >= kMaxBytes) return CONV_E_UNSUPPORTED;
  // The kernels split a reduction index into (tap, channel) with an fp32
  // reciprocal, exact below 2^24.
  if ((int64_t)d->kh * d->kw * cg * in_esz >= ((int64_t)1 << 24)) return CONV_E_UNSUPPORTED;

  int path;
  int loader = LOAD_GENERIC;
  if (d->groups == 1) {
    path = dt == CONV_F32 ? PATH_F32 : PATH_IGEMM;
    if (path == PATH_IGEMM) {
      const bool vec = (d->c_in * in_esz) % 16 == 0;
      const bool tap = (d->c_in * in_esz) % 128 == 0 && (int64_t)d->kh * d->kw <= 32 &&
                       (x_bytes + ((int64_t)d->pad_h * d->w + d->pad_w) * d->c_in * in_esz) < kMaxBytes;
      if (vec && d->kh == 1 && d->kw == 1 && d->stride_h == 1 && d->stride_w == 1 && d->pad_h == 0 &&
          d->pad_w == 0)
        loader = LOAD_1X1;
      else if (tap)
        loader = LOAD_TAP;
      else if (vec)
        loader = LOAD_VEC;
    }
  } else {
    if (!(d->groups == d->c_in && d->c_in == d->c_out)) return CONV_E_UNSUPPORTED;
    if (d->kh != 3 || d->kw != 3) return CONV_E_UNSUPPORTED;
    path = PATH_DW;
    loader = (d->c_in * in_esz) % 16 == 0 ? LOAD_VEC : LOAD_GENERIC;
  }
  if (path == PATH_DW) {
    // algo 1..4 forces 1, 2, 4 or 8 rows per lane of the row-window kernels
    const bool rows = d->stride_h == 1 && d->stride_w == 1 && d->c_in % 4 == 0;
    if (d->algo != 0 && (!rows || d->algo < 1 || d->algo > 4)) return CONV_E_UNSUPPORTED;
  } else if (d->algo != 0 && (path != PATH_IGEMM || d->algo < 1 || d->algo > kAlgoLast)) {
    return CONV_E_UNSUPPORTED;
  }
  const bool ws_ok = path == PATH_IGEMM && !wq && loader != LOAD_GENERIC &&
                     (int64_t)d->kh * d->kw * cg * in_esz <= 256;
  if (d->algo == kAlgoWs && !ws_ok) return CONV_E_UNSUPPORTED;

  // bfp8 weights are decoded by the implicit-GEMM kernel's 16-byte weight
  // loaders: dense bf16 layers with c_in * 2 % 16 == 0, implicit-GEMM tiles
  // only (the first, 3-channel convolution stays bf16, as on the pages).
  if (wq && !(dt == CONV_BF16 && path == PATH_IGEMM && loader != LOAD_GENERIC && d->algo < kAlgoXl))
    return CONV_E_UNSUPPORTED;

  // A short reduction over an odd channel count (the 3-channel and 1-channel
  // stems) goes to the LDS-free small-K kernel unless a tile is forced.
  if (path == PATH_IGEMM && loader == LOAD_GENERIC && d->algo == 0 &&
      (int64_t)d->kh * d->kw * cg * in_esz <= 128)
    path = PATH_SMALLK;

  std::memset(p, 0, sizeof(*p));
  p->d = *d;
  Geometry& g = p->g;
  g.n = (int)d->n;
  g.h = (int)d->h;
  g.w = (int)d->w;
  g.c = (int)d->c_in;
  g.ho = (int)ho;
  g.wo = (int)wo;
  g.cout = (int)d->c_out;
  g.kh = d->kh;
  g.kw = d->kw;
  g.sh = d->stride_h;
  g.sw = d->stride_w;
  g.ph = d->pad_h;
  g.pw = d->pad_w;
  g.m = (int)(d->n * ho * wo);
  g.k = (int)(d->kh * d->kw * cg);
  p->path = path;
  p->loader = loader;
  p->in_esz = in_esz;
  p->out_esz = out_esz;
  p->out_kind = ot == CONV_F32 ? OUT_F32 : ot == CONV_BF16 ? OUT_BF16 : ot == CONV_I8 ? OUT_I8 : OUT_I32;
  p->cus = 256;
  {
    int dev = 0, ndev = 0, cus = 0;
    if (hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0 && hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
      p->cus = cus;
    (void)hipGetLastError();
  }
  if (d->algo >= kAlgoXl && d->algo < kAlgoWs) {
    if (!xl_eligible(g, in_esz, loader, d->algo - kAlgoXl)) return CONV_E_UNSUPPORTED;
    path = PATH_XL;
  }
  if (d->algo == kAlgoHalo) {
    if (path != PATH_IGEMM || wq || !halo_eligible(*d, g)) return CONV_E_UNSUPPORTED;
    path = PATH_HALO;
  }
  if (path == PATH_IGEMM && d->algo == 0 && !wq) {
    const int xt = choose_xl(g, in_esz, loader);
    if (xt >= 0) {
      path = PATH_XL;
      p->tile = xt;
    }
  }
  // 16-byte (8-channel) input pixels: the window stem kernel, the only one
  // that takes a pixel stride (and the best one for such layers)
  if (xs == 8 && stem_eligible(*d, g, xs) && !wq && d->algo == 0 && (path == PATH_IGEMM || path == PATH_SMALLK))
    path = PATH_STEM;
  else if (xs != d->c_in)
    return CONV_E_UNSUPPORTED;
  // 3x3 bf16 layers over 32 or 64 channels where the halo kernel wins
  if (path == PATH_IGEMM && d->algo == 0 && !wq && halo_preferred(*d, g)) path = PATH_HALO;
  // A reduction of at most 256 bytes on the 64x64 tile goes to the
  // weight-stationary kernel.
  if (path == PATH_IGEMM && ws_ok && (d->algo == kAlgoWs || (d->algo == 0 && choose_tile(g, in_esz) == 0)))
    path = PATH_WS;
  p->path = path;
  p->tile = path == PATH_IGEMM ? (d->algo ? d->algo - 1 : choose_tile(g, in_esz))
            : path == PATH_XL && d->algo == 0 ? p->tile
            : path == PATH_XL  ? d->algo - kAlgoXl
            : path == PATH_DW && d->algo ? 1 << (d->algo - 1)
                               : 0;
  if (path == PATH_IGEMM && loader == LOAD_GENERIC && (kTiles[p->tile].tco > 256 || kTiles[p->tile].tpx > 256))
    return CONV_E_UNSUPPORTED;  // the element-wise gather needs a thread per tile row
  p->ksplit = 1;
  p->kt_per = (int)((g.k * (int64_t)in_esz + 127) / 128);
  p->x_bytes = x_bytes;
  p->w_bytes = w_bytes;
  p->wq = wq;
  p->kp = (int)kp;
  p->w_exp_off = wq ? d->c_out * kp : 0;
  p->y_bytes = y_bytes;
  p->b_bytes = dt == CONV_I8 ? (ot == CONV_I8 ? 8 * d->c_out : 4 * d->c_out) : 4 * d->c_out;
  if (path == PATH_IGEMM || path == PATH_XL) return plan_split_k(p, scratch, scratch_bytes);
  return CONV_OK;
}

}  // namespace

extern "C" {

conv_status conv_prepare(const conv_desc* d, conv_plan** out) {
  if (!d || !out) return CONV_E_NULL;
  *out = nullptr;
  conv_plan* p = new (std::nothrow) conv_plan;
  if (!p) return CONV_E_NOMEM;
  const conv_status st = build_plan(d, p, nullptr, 0);
  if (st != CONV_OK) {
    delete p;  // build_plan allocates nothing on a failing return
    return st;
  }
  *out = p;
  return CONV_OK;
}

namespace {

conv_status run_common(const conv_plan* p, const void* x, const void* w, const void* b, const void* r, void* y,
                       void* stream) {
  if (!p || !x || !w || !y) return CONV_E_NULL;
  const bool i8out = p->d.dtype == CONV_I8 && p->d.out_dtype == CONV_I8;
  if (i8out && !b) return CONV_E_NULL;
  if (((uintptr_t)x | (uintptr_t)w | (uintptr_t)y | (uintptr_t)r) & 15) return CONV_E_ALIGN;
  if ((uintptr_t)b & 3) return CONV_E_ALIGN;
  if (ranges_overlap(y, p->y_bytes, x, p->x_bytes) || ranges_overlap(y, p->y_bytes, w, p->w_bytes) ||
      ranges_overlap(y, p->y_bytes, b, p->b_bytes))
    return CONV_E_ALIAS;
  // the residual may be y itself (every output element reads its own
  // residual element before it is written), but not partly overlap it
  if (r && r != y && ranges_overlap(y, p->y_bytes, r, p->y_bytes)) return CONV_E_ALIAS;

  Epi e;
  e.act = p->d.act;
  e.bias = nullptr;
  e.ibias = nullptr;
  e.scale = nullptr;
  e.res = r;
  if (p->d.dtype == CONV_I8) {
    e.ibias = static_cast<const int32_t*>(b);
    e.scale = b ? reinterpret_cast<const float*>(static_cast<const int32_t*>(b) + p->d.c_out) : nullptr;
    if (!i8out) e.scale = nullptr;
  } else {
    e.bias = static_cast<const float*>(b);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err;
  switch (p->path) {
    case PATH_IGEMM: err = launch_igemm(p, x, w, e, y, s); break;
    case PATH_DW: err = launch_dw(p, x, w, e, y, s); break;
    case PATH_SMALLK: err = launch_smallk(p, x, w, e, y, s); break;
    case PATH_XL: err = launch_xl(p, x, w, e, y, s); break;
    case PATH_WS: err = launch_ws(p, x, w, e, y, s); break;
    case PATH_HALO: err = launch_halo(p, x, w, e, y, s); break;
    case PATH_STEM: err = launch_stem(p, x, w, e, y, s); break;
    default: err = launch_f32(p, x, w, e, y, s); break;
  }
  if (err != hipSuccess) {
    std::snprintf(g_last_hip_error, sizeof(g_last_hip_error), "%s", hipGetErrorString(err));
    return CONV_E_HIP;
  }
  return CONV_OK;
}

}  // namespace

conv_status conv_run(const conv_plan* p, const void* x, const void* w, const void* b, void* y, void* stream) {
  return run_common(p, x, w, b, nullptr, y, stream);
}

conv_status conv_run_residual(const conv_plan* p, const void* x, const void* w, const void* b, const void* r,
                              void* y, void* stream) {
  if (!p || !r) return CONV_E_NULL;
  if (p->out_kind == OUT_I32) return CONV_E_UNSUPPORTED;
  return run_common(p, x, w, b, r, y, stream);
}

conv_status conv_run_noalloc(const conv_desc* d, const void* x, const void* w, const void* b, const void* r,
                             void* y, void* stream) {
  if (!d) return CONV_E_NULL;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    std::snprintf(g_last_hip_error, sizeof(g_last_hip_error), "%s", hipGetErrorString(hipGetLastError()));
    return CONV_E_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return CONV_E_UNSUPPORTED;
  void* ws = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!ws) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ws = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!ws) {
      const hipError_t err = hipGetSymbolAddress(&ws, HIP_SYMBOL(scratch));
      if (err != hipSuccess || !ws) {
        std::snprintf(g_last_hip_error, sizeof(g_last_hip_error), "hipGetSymbolAddress(scratch): %s",
                      hipGetErrorString(err));
        (void)hipGetLastError();
        return CONV_E_HIP;
      }
      g_scratch_ptr[dev].store(ws, std::memory_order_release);
    }
  }
  conv_plan p;  // on this call's stack: no allocation
  const conv_status st = build_plan(d, &p, ws, CONV_NOALLOC_SCRATCH_BYTES);
  if (st != CONV_OK) return st;
  if (r && p.out_kind == OUT_I32) return CONV_E_UNSUPPORTED;
  return run_common(&p, x, w, b, r, y, stream);
}

namespace {

// A KxK bf16 layer on the implicit-GEMM kernel, unsplit, whose output tile
// can hold all its channels (64 or 128, one workgroup per 64 pixels),
// followed by a 1x1 s1 p0 bf16 layer on exactly that output with at most 64
// output channels.
bool fused_1x1_ok(const conv_plan* p1, const conv_plan* p2) {
  const conv_desc& a = p1->d;
  const conv_desc& b = p2->d;
  if (a.dtype != CONV_BF16 || a.out_dtype != CONV_BF16 || p1->wq || p1->ksplit != 1) return false;
  if (p1->path != PATH_IGEMM && p1->path != PATH_HALO) return false;
  if (p1->path == PATH_HALO && !halo_fusable(p1->d, p1->g)) return false;
  if (p1->loader != LOAD_TAP && p1->loader != LOAD_VEC) return false;
  if (p1->g.cout != 64 && p1->g.cout != 128) return false;
  if (b.dtype != CONV_BF16 || b.out_dtype != CONV_BF16 || b.groups != 1 || p2->wq) return false;
  if (b.kh != 1 || b.kw != 1 || b.stride_h != 1 || b.stride_w != 1 || b.pad_h != 0 || b.pad_w != 0) return false;
  if (b.n != a.n || b.h != p1->g.ho || b.w != p1->g.wo || b.c_in != p1->g.cout) return false;
  return p2->g.cout <= 64 && (p2->g.cout & 3) == 0;
}

}  // namespace

namespace {

// The fused launch runs on the halo kernel when the first layer does, or
// when its kernel was left to the library and the halo kernel can fuse it
// (it beats the implicit-GEMM fusion on every such pair measured); a first
// layer forced onto an implicit-GEMM tile keeps that kernel.
bool fused_on_halo(const conv_plan* p1) {
  return p1->path == PATH_HALO || (p1->d.algo == 0 && halo_fusable(p1->d, p1->g));
}

}  // namespace

conv_status conv_fuse_check(const conv_plan* p1, const conv_plan* p2) {
  if (!p1 || !p2) return CONV_E_NULL;
  return fused_1x1_ok(p1, p2) ? CONV_OK : CONV_E_UNSUPPORTED;
}

conv_status conv_describe_fused(const conv_plan* p1, const conv_plan* p2, char* buf, int32_t len) {
  if (!p1 || !p2 || !buf || len <= 0) return CONV_E_NULL;
  if (!fused_1x1_ok(p1, p2)) return CONV_E_UNSUPPORTED;
  static const char* kLoader[] = {"generic", "vec16", "1x1", "tap"};
  const int tco = p1->g.cout;
  if (fused_on_halo(p1)) {
    std::snprintf(buf, len,
                  "halo fused_1x1 co%d patch=4x16 stride=%d cin=%d then 1x1 %d->%d wgs=%d m=%d k=%d "
                  "kernel=halo_kernel<%d, %d, %d, 1>",
                  tco, p1->g.sh, p1->g.c, tco, p2->g.cout, halo_grid(p1, tco), p1->g.m, p1->g.k, p1->g.sh,
                  p1->g.c / 32, tco);
    return CONV_OK;
  }
  std::snprintf(buf, len,
                "igemm fused_1x1 loader=%s co%dxpx64 then 1x1 %d->%d wgs=%d m=%d k=%d "
                "kernel=igemm_kernel<2, %d, 64, 2, 2, %d, %d, 0, 1>",
                kLoader[p1->loader], tco, tco, p2->g.cout, (p1->g.m + 63) / 64, p1->g.m, p1->g.k, tco, p1->loader,
                (tco + 64 >= 512) ? 1 : 2);
  return CONV_OK;
}

conv_status conv_run_fused(const conv_plan* p1, const conv_plan* p2, const void* x, const void* w1, const void* b1,
                           const void* w2, const void* b2, void* y, void* stream) {
  if (!p1 || !p2 || !x || !w1 || !w2 || !y) return CONV_E_NULL;
  if (!fused_1x1_ok(p1, p2)) return CONV_E_UNSUPPORTED;
  if (((uintptr_t)x | (uintptr_t)w1 | (uintptr_t)w2 | (uintptr_t)y) & 15) return CONV_E_ALIGN;
  if (((uintptr_t)b1 | (uintptr_t)b2) & 3) return CONV_E_ALIGN;
  if (ranges_overlap(y, p2->y_bytes, x, p1->x_bytes) || ranges_overlap(y, p2->y_bytes, w1, p1->w_bytes) ||
      ranges_overlap(y, p2->y_bytes, w2, p2->w_bytes) || ranges_overlap(y, p2->y_bytes, b1, p1->b_bytes) ||
      ranges_overlap(y, p2->y_bytes, b2, p2->b_bytes))
    return CONV_E_ALIAS;
  Epi e1, e2;
  std::memset(&e1, 0, sizeof(e1));
  std::memset(&e2, 0, sizeof(e2));
  e1.bias = static_cast<const float*>(b1);
  e1.act = p1->d.act;
  e2.bias = static_cast<const float*>(b2);
  e2.act = p2->d.act;
  const hipError_t err = fused_on_halo(p1)
                             ? launch_halo_fused(p1, p2, x, w1, e1, w2, e2, y, static_cast<hipStream_t>(stream))
                             : launch_igemm_fused(p1, p2, x, w1, e1, w2, e2, y, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) {
    std::snprintf(g_last_hip_error, sizeof(g_last_hip_error), "%s", hipGetErrorString(err));
    return CONV_E_HIP;
  }
  return CONV_OK;
}

conv_status conv_run_mosaic(const conv_plan* p, const void* tiles, int32_t tiles_dtype, int32_t th, int32_t tw,
                            const void* w, const void* b, void* y, void* stream) {
  if (!p || !tiles || !w || !y) return CONV_E_NULL;
  if (tiles_dtype != CONV_F32 && tiles_dtype != CONV_BF16) return CONV_E_UNSUPPORTED;
  if (!stem_mosaic_ok(p, th, tw)) return CONV_E_UNSUPPORTED;
  const int esz = tiles_dtype == CONV_F32 ? 4 : 2;
  const int64_t t_bytes = (int64_t)4 * p->g.n * th * tw * p->g.c * esz;
  if (t_bytes >= kMaxBytes) return CONV_E_UNSUPPORTED;
  if (((uintptr_t)w | (uintptr_t)y) & 15) return CONV_E_ALIGN;
  if (((uintptr_t)tiles & (esz - 1)) || ((uintptr_t)b & 3)) return CONV_E_ALIGN;
  if (ranges_overlap(y, p->y_bytes, tiles, t_bytes) || ranges_overlap(y, p->y_bytes, w, p->w_bytes) ||
      ranges_overlap(y, p->y_bytes, b, p->b_bytes))
    return CONV_E_ALIAS;
  Epi e;
  std::memset(&e, 0, sizeof(e));
  e.act = p->d.act;
  e.bias = static_cast<const float*>(b);
  const hipError_t err =
      launch_stem_mosaic(p, tiles, tiles_dtype == CONV_F32, th, tw, w, e, y, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) {
    std::snprintf(g_last_hip_error, sizeof(g_last_hip_error), "%s", hipGetErrorString(err));
    return CONV_E_HIP;
  }
  return CONV_OK;
}

conv_status conv_run_upcat(const conv_plan* p, const void* s0, int32_t c0, int32_t up0, const void* s1, int32_t up1,
                           const void* w, const void* b, void* y, void* stream) {
  if (!p || !s0 || !s1 || !w || !y) return CONV_E_NULL;
  const conv_desc& d = p->d;
  if ((d.dtype != CONV_BF16 && d.dtype != CONV_I8) || d.groups != 1 || d.kh != 1 || d.kw != 1 || d.stride_h != 1 ||
      d.stride_w != 1 || d.pad_h != 0 || d.pad_w != 0 || p->wq)
    return CONV_E_UNSUPPORTED;
  if ((up0 != 0 && up0 != 1) || (up1 != 0 && up1 != 1)) return CONV_E_SHAPE;
  if ((up0 || up1) && ((p->g.h & 1) || (p->g.w & 1))) return CONV_E_SHAPE;
  if (c0 <= 0 || c0 >= p->g.c) return CONV_E_SHAPE;
  const int esz = p->in_esz;
  const int c0b = c0 * esz, c1b = (p->g.c - c0) * esz;
  if (c0b % 128 || c1b % 128) return CONV_E_UNSUPPORTED;  // each 128-byte K-tile inside one map
  const bool i8out = d.dtype == CONV_I8 && d.out_dtype == CONV_I8;
  if (i8out && !b) return CONV_E_NULL;
  if (((uintptr_t)s0 | (uintptr_t)s1 | (uintptr_t)w | (uintptr_t)y) & 15) return CONV_E_ALIGN;
  if ((uintptr_t)b & 3) return CONV_E_ALIGN;
  const int64_t s0_bytes = (int64_t)p->g.n * (p->g.h >> up0) * (p->g.w >> up0) * c0b;
  const int64_t s1_bytes = (int64_t)p->g.n * (p->g.h >> up1) * (p->g.w >> up1) * c1b;
  if (ranges_overlap(y, p->y_bytes, s0, s0_bytes) || ranges_overlap(y, p->y_bytes, s1, s1_bytes) ||
      ranges_overlap(y, p->y_bytes, w, p->w_bytes) || ranges_overlap(y, p->y_bytes, b, p->b_bytes))
    return CONV_E_ALIAS;
  Epi e;
  std::memset(&e, 0, sizeof(e));
  e.act = d.act;
  if (d.dtype == CONV_I8) {
    e.ibias = static_cast<const int32_t*>(b);
    e.scale = i8out && b ? reinterpret_cast<const float*>(static_cast<const int32_t*>(b) + d.c_out) : nullptr;
  } else {
    e.bias = static_cast<const float*>(b);
  }
  const hipError_t err = launch_igemm_cat(p, s0, c0b, up0, s1, up1, w, e, y, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) {
    std::snprintf(g_last_hip_error, sizeof(g_last_hip_error), "%s", hipGetErrorString(err));
    return CONV_E_HIP;
  }
  return CONV_OK;
}

conv_status conv_destroy(conv_plan* p) {
  if (p && p->ws && p->ws_owned) {
    int cur = 0;
    const bool have = hipGetDevice(&cur) == hipSuccess;
    if (have && cur != p->ws_device) (void)hipSetDevice(p->ws_device);
    (void)hipFree(p->ws);
    if (have && cur != p->ws_device) (void)hipSetDevice(cur);
  }
  delete p;
  return CONV_OK;
}

conv_status conv_out_shape(const conv_plan* p, int64_t nhwc[4]) {
  if (!p || !nhwc) return CONV_E_NULL;
  nhwc[0] = p->g.n;
  nhwc[1] = p->g.ho;
  nhwc[2] = p->g.wo;
  nhwc[3] = p->g.cout;
  return CONV_OK;
}

conv_status conv_describe(const conv_plan* p, char* buf, int32_t len) {
  if (!p || !buf || len <= 0) return CONV_E_NULL;
  static const char* kLoader[] = {"generic", "vec16", "1x1", "tap"};
  static const char* kDt[] = {"f32", "bf16", "i8", "i32"};
  if (p->path == PATH_IGEMM) {
    const TileCfg& t = kTiles[p->tile];
    const long nwg = (long)((p->g.cout + t.tco - 1) / t.tco) * ((p->g.m + t.tpx - 1) / t.tpx);
    std::snprintf(buf, len,
                  "igemm dtype=%s out=%s%s loader=%s tile=%d co%dxpx%d waves=%dx%d wgs=%ld m=%d k=%d "
                  "ksplit=%d kernel=igemm_kernel<%d, %d, %d, %d, %d, %d, %d, %d, 0>",
                  kDt[p->d.dtype], kDt[p->d.out_dtype], p->wq ? " w=bfp8" : "", kLoader[p->loader], p->tile + 1,
                  t.tco, t.tpx, t.wco, t.wpx, nwg, p->g.m, p->g.k, p->ksplit, p->in_esz, t.tco, t.tpx, t.wco, t.wpx,
                  p->loader, igemm_stages(p->loader, p->tile), p->wq);
  } else if (p->path == PATH_XL) {
    const TileCfg& t = kXlTiles[p->tile];
    const long nwg = (long)(p->g.cout / t.tco) * ((p->g.m + t.tpx - 1) / t.tpx);
    std::snprintf(buf, len,
                  "igemm_xl dtype=%s out=%s loader=%s tile=%d co%dxpx%d waves=2x2 wgs=%ld m=%d k=%d ksplit=%d "
                  "kernel=igemm_xl_kernel<%d, %d, %d, %d>",
                  kDt[p->d.dtype], kDt[p->d.out_dtype], kLoader[p->loader], kAlgoXl + p->tile, t.tco, t.tpx, nwg,
                  p->g.m, p->g.k, p->ksplit, p->in_esz, t.tco, t.tpx, p->loader);
  } else if (p->path == PATH_WS) {
    std::snprintf(buf, len,
                  "igemm_ws dtype=%s out=%s loader=%s tile=%d co64xpx64 waves=2x2 grid=%dx%d m=%d k=%d "
                  "kernel=igemm_ws_kernel<%d, %d, %d>",
                  kDt[p->d.dtype], kDt[p->d.out_dtype], kLoader[p->loader], kAlgoWs, ws_grid_x(p),
                  (p->g.cout + 63) / 64, p->g.m, p->g.k, p->in_esz, p->loader, ws_ksteps(p->g, p->in_esz, p->loader));
  } else if (p->path == PATH_HALO) {
    std::snprintf(buf, len,
                  "halo dtype=bf16 out=bf16 tile=%d co64 patch=4x16 stride=%d cin=%d wgs=%d m=%d k=%d "
                  "kernel=halo_kernel<%d, %d, 64, 0>",
                  kAlgoHalo, p->g.sh, p->g.c, halo_grid(p, 64), p->g.m, p->g.k, p->g.sh, p->g.c / 32);
  } else if (p->path == PATH_STEM) {
    std::snprintf(buf, len,
                  "stem_window dtype=bf16 out=bf16 cin=%d x_stride=%d patch=4x64 co32 wgs=%d m=%d k=%d "
                  "kernel=stem_window_kernel<0>",
                  p->g.c, (int)(p->x_bytes / ((int64_t)p->g.n * p->g.h * p->g.w * 2)), stem_grid(p), p->g.m, p->g.k);
  } else if (p->path == PATH_SMALLK) {
    int fco, ks;
    smallk_shape(p->g, p->in_esz, &fco, &ks);
    std::snprintf(buf, len, "smallk dtype=%s out=%s m=%d k=%d kernel=smallk_kernel<%d, %d, %d>", kDt[p->d.dtype],
                  kDt[p->d.out_dtype], p->g.m, p->g.k, p->in_esz, fco, ks);
  } else if (p->path == PATH_DW) {
    static const char* kT[] = {"", "signed char", "unsigned short", "", "float"};
    int ve, pw, th = 0;
    dw_shape(p, &ve, &pw, &th);
    // the kernels' last two template arguments: activation, and the int8
    // output kind (the int32 checkpoint or not; also 2 for float layers)
    const int act = p->out_kind == OUT_I32 && p->d.act != CONV_ACT_RELU ? CONV_ACT_NONE : p->d.act;
    const int ok = p->out_kind == OUT_I32 ? OUT_I32 : OUT_I8;
    const int pf = dw_prefetch_rows();
    if (th && p->in_esz == 1)
      std::snprintf(buf, len,
                    "dw3x3 dtype=%s out=%s stride=%dx%d rows dot4 kernel=dw3x3_i8_kernel<%d, %d, %d, %d, %d>",
                    kDt[p->d.dtype], kDt[p->d.out_dtype], p->g.sh, p->g.sw, pw, th, act, ok, pf);
    else if (th)
      std::snprintf(buf, len,
                    "dw3x3 dtype=%s out=%s stride=%dx%d rows kernel=dw3x3_rows_kernel<%s, %d, %d, %d, %d, %d, %d>",
                    kDt[p->d.dtype], kDt[p->d.out_dtype], p->g.sh, p->g.sw, kT[p->in_esz], ve, pw, th, act, ok, pf);
    else
      std::snprintf(buf, len, "dw3x3 dtype=%s out=%s loader=%s stride=%dx%d kernel=dw3x3_kernel<%s, %d, %d, %d, %d>",
                    kDt[p->d.dtype], kDt[p->d.out_dtype], kLoader[p->loader], p->g.sh, p->g.sw, kT[p->in_esz], ve,
                    pw, act, ok);
  } else {
    std::snprintf(buf, len, "direct_f32 m=%d k=%d kernel=conv_f32_kernel", p->g.m, p->g.k);
  }
  return CONV_OK;
}

int32_t conv_algo_count(void) { return kAlgoLast; }

conv_status conv_mosaic_pack(const void* tiles, int32_t in_dtype, void* canvas, int32_t out_dtype, int32_t m,
                             int32_t th, int32_t tw, int32_t c, int32_t c_pad, void* stream) {
  if (!tiles || !canvas) return CONV_E_NULL;
  if (m <= 0 || th <= 0 || tw <= 0 || c <= 0 || c_pad < c) return CONV_E_SHAPE;
  if ((in_dtype != CONV_F32 && in_dtype != CONV_BF16) || (out_dtype != CONV_F32 && out_dtype != CONV_BF16))
    return CONV_E_UNSUPPORTED;
  const int64_t in_bytes = 4LL * m * th * tw * c * esz_of(in_dtype);
  const int64_t out_bytes = 4LL * m * th * tw * c_pad * esz_of(out_dtype);
  if (in_bytes >= kMaxBytes || out_bytes >= kMaxBytes) return CONV_E_UNSUPPORTED;
  if (((uintptr_t)tiles | (uintptr_t)canvas) & 15) return CONV_E_ALIGN;
  if (ranges_overlap(tiles, in_bytes, canvas, out_bytes)) return CONV_E_ALIAS;
  hipError_t err = launch_mosaic(tiles, in_dtype == CONV_F32, canvas, out_dtype == CONV_F32, m, th, tw, c, c_pad,
                                 static_cast<hipStream_t>(stream));
  if (err != hipSuccess) {
    std::snprintf(g_last_hip_error, sizeof(g_last_hip_error), "%s", hipGetErrorString(err));
    return CONV_E_HIP;
  }
  return CONV_OK;
}

int64_t conv_bfp8_bytes(int64_t c_out, int64_t k) {
  if (c_out <= 0 || k <= 0) return 0;
  const int64_t kp = (k + 15) / 16 * 16;
  return c_out * kp + c_out * (kp / 16);
}

conv_status conv_pack_bfp8(const void* w, int32_t w_dtype, int64_t c_out, int64_t k, void* packed, void* stream) {
  if (!w || !packed) return CONV_E_NULL;
  if (c_out <= 0 || k <= 0) return CONV_E_SHAPE;
  if (w_dtype != CONV_F32 && w_dtype != CONV_BF16) return CONV_E_UNSUPPORTED;
  const int64_t in_bytes = c_out * k * esz_of(w_dtype);
  const int64_t out_bytes = conv_bfp8_bytes(c_out, k);
  if (in_bytes >= kMaxBytes || out_bytes >= kMaxBytes) return CONV_E_UNSUPPORTED;
  if ((uintptr_t)packed & 15 || (uintptr_t)w & (esz_of(w_dtype) - 1)) return CONV_E_ALIGN;
  if (ranges_overlap(w, in_bytes, packed, out_bytes)) return CONV_E_ALIAS;
  hipError_t err = launch_bfp8_pack(w, w_dtype == CONV_F32, (int)c_out, (int)k, packed, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) {
    std::snprintf(g_last_hip_error, sizeof(g_last_hip_error), "%s", hipGetErrorString(err));
    return CONV_E_HIP;
  }
  return CONV_OK;
}

conv_status conv_spp_maxpool(const void* x, int32_t dtype, void* y, int32_t n, int32_t h, int32_t w, int32_t c,
                             void* stream) {
  if (!x || !y) return CONV_E_NULL;
  if (n <= 0 || h <= 0 || w <= 0 || c <= 0) return CONV_E_SHAPE;
  if (dtype != CONV_F32 && dtype != CONV_BF16 && dtype != CONV_I8) return CONV_E_UNSUPPORTED;
  const int64_t x_bytes = (int64_t)n * h * w * c * esz_of(dtype);
  if (4 * x_bytes >= kMaxBytes || spp_chunks(n, h, w, c, dtype) == 0) return CONV_E_UNSUPPORTED;
  if (((uintptr_t)x | (uintptr_t)y) & 15) return CONV_E_ALIGN;
  if (ranges_overlap(x, x_bytes, y, 4 * x_bytes)) return CONV_E_ALIAS;
  hipError_t err = launch_spp(x, dtype, y, n, h, w, c, x_bytes, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) {
    std::snprintf(g_last_hip_error, sizeof(g_last_hip_error), "%s", hipGetErrorString(err));
    return CONV_E_HIP;
  }
  return CONV_OK;
}

conv_status conv_upsample_concat(const void* s0, int32_t c0, int32_t up0, const void* s1, int32_t c1, int32_t up1,
                                 int32_t dtype, void* y, int32_t n, int32_t ho, int32_t wo, void* stream) {
  if (!s0 || !s1 || !y) return CONV_E_NULL;
  if (n <= 0 || ho <= 0 || wo <= 0 || c0 <= 0 || c1 <= 0 || up0 < 0 || up0 > 1 || up1 < 0 || up1 > 1 ||
      ((up0 || up1) && (ho % 2 || wo % 2)))
    return CONV_E_SHAPE;
  if (dtype != CONV_F32 && dtype != CONV_BF16 && dtype != CONV_I8) return CONV_E_UNSUPPORTED;
  const int64_t e = esz_of(dtype), b0 = (int64_t)c0 * e, b1 = (int64_t)c1 * e;
  const int64_t s0_bytes = (int64_t)n * (ho >> up0) * (wo >> up0) * b0;
  const int64_t s1_bytes = (int64_t)n * (ho >> up1) * (wo >> up1) * b1;
  const int64_t y_bytes = (int64_t)n * ho * wo * (b0 + b1);
  if (b0 % 16 || b1 % 16 || y_bytes >= kMaxBytes || (int64_t)n * ho > 65535 || (int64_t)wo * (b0 + b1) / 16 >= (1 << 22))
    return CONV_E_UNSUPPORTED;
  if (((uintptr_t)s0 | (uintptr_t)s1 | (uintptr_t)y) & 15) return CONV_E_ALIGN;
  if (ranges_overlap(y, y_bytes, s0, s0_bytes) || ranges_overlap(y, y_bytes, s1, s1_bytes)) return CONV_E_ALIAS;
  hipError_t err = launch_upcat(s0, b0, up0, s1, b1, up1, y, n, ho, wo, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) {
    std::snprintf(g_last_hip_error, sizeof(g_last_hip_error), "%s", hipGetErrorString(err));
    return CONV_E_HIP;
  }
  return CONV_OK;
}

const char* conv_status_str(int32_t status) {
  static thread_local char buf[320];
  switch (status) {
    case CONV_OK: return "CONV_OK";
    case CONV_E_NULL: return "CONV_E_NULL: a required pointer is NULL";
    case CONV_E_SHAPE: return "CONV_E_SHAPE: invalid sizes or empty output";
    case CONV_E_UNSUPPORTED: return "CONV_E_UNSUPPORTED: layer kind, dtype, activation, algo or size not supported";
    case CONV_E_ALIGN: return "CONV_E_ALIGN: x, w, y need 16-byte and b 4-byte alignment";
    case CONV_E_ALIAS: return "CONV_E_ALIAS: output overlaps an input";
    case CONV_E_NOMEM: return "CONV_E_NOMEM: plan or split-K workspace allocation failed";
    case CONV_E_SCRATCH:
      return "CONV_E_SCRATCH: the layer's split-K partial sums exceed the static scratch of conv_run_noalloc "
             "(CONV_NOALLOC_SCRATCH_BYTES)";
    case CONV_E_HIP:
      std::snprintf(buf, sizeof(buf), "CONV_E_HIP: %s", g_last_hip_error);
      return buf;
    default: return "unknown conv_status";
  }
}

}  // extern "C"
