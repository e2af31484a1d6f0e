/*
 * conv_nhwc.h -- C ABI of the MI355X (gfx950) fused NHWC conv2d library.
 *
 * One layer of edge / YOLO-style CNN inference:
 *
 *   y = act( conv(x, w) + b )            (fp32, bf16)
 *   y = requant( conv(x, w) + b, s, act) (int8)
 *
 * where conv is the 2-D cross-correlation (no kernel flip) with zero
 * padding, as used by PyTorch and by the nanoinfer engine (nanoinfer README,
 * naive reference convolution and its PyTorch parity table). Supported
 * layer kinds (nanoinfer README, "what is still slow" and GPU section): dense
 * KxK, 1x1 pointwise, and 3x3 depthwise (groups == Cin == Cout).
 *
 * Layouts (all tensors plain, dense, row-major):
 *   x  NHWC  [n][h][w][c_in]                      dtype
 *   w  OHWI  [c_out][kh][kw][c_in/groups]          dtype  (K-contiguous)
 *   y  NHWC  [n][ho][wo][c_out]                    out_dtype
 *   ho = (h + 2*pad_h - kh) / stride_h + 1, wo likewise (floor division).
 *   pad_h applies to the top and the bottom edge, pad_w to the left and the
 *   right edge (the per-axis padding of the keyword-spotting stem, 10x4
 *   kernel with pad (5,1), nanoinfer README, "Asymmetric padding collapsed
 *   to one axis").
 *
 * Precisions:
 *   F32  in, F32 out  : true fp32 multiply-add, fp32 accumulate (no
 *                       reduced-precision matrix mode; nanoinfer README,
 *                       cuDNN default-math paragraph).
 *   BF16 in, BF16 out : fp32 accumulate (YOLOv4 on Tenstorrent Wormhole,
 *                       section 7: 16-bit accumulation lost accuracy, fp32
 *                       fixed it); one round-to-nearest-even bf16 store.
 *   I8   in, I8 out   : int32 accumulate; R = acc + bias (int32);
 *                       v = fl32(fl32(R) * scale[co]); m = act(v);
 *                       y = clamp(round_half_even(m), -127, 127)
 *                       (symmetric per-output-channel scales, nanoinfer
 *                       README, quantization section).
 *   I8   in, I32 out  : the int32 checkpoint R (act NONE or RELU only).
 *
 * Activations (YOLOv4 on Tenstorrent Wormhole, section 7 table):
 *   NONE, RELU = max(v,0), RELU6 = min(max(v,0),6),
 *   MISH = v * tanh(ln(1 + e^v))   (the real function, not HardMish).
 *
 * Ownership: every device buffer (x, w, b, y, mosaic tiles and canvas) is
 * owned by the caller. A plan owns host metadata and, for a layer whose
 * reduction is split across workgroups (few output tiles, long K; conv_describe
 * shows ksplit > 1), one device workspace for the partial sums, allocated by
 * conv_prepare on the device current at that call and freed by conv_destroy.
 * A plan is immutable after conv_prepare and may be used from any thread.
 * conv_run only enqueues work on the given stream: it allocates nothing,
 * never synchronises, copies nothing between host and device and caches
 * nothing between calls (x, w, b are read afresh every call), so it can be
 * captured into a HIP graph.
 *
 * Errors: every entry point returns a conv_status; a negative value names
 * the failure and nothing was enqueued. Faults inside an enqueued kernel
 * surface at the caller's next synchronisation, as for any HIP call.
 *
 * Size limit: each of x, w and y must be smaller than 2^31 bytes.
 */
#ifndef CONV_NHWC_H
#define CONV_NHWC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum conv_dtype {
  CONV_F32 = 0,
  CONV_BF16 = 1,
  CONV_I8 = 2,
  CONV_I32 = 3 /* output only: the int32 checkpoint of an int8 layer */
} conv_dtype;

typedef enum conv_act {
  CONV_ACT_NONE = 0,
  CONV_ACT_RELU = 1,
  CONV_ACT_RELU6 = 2,
  CONV_ACT_MISH = 3
} conv_act;

/* Storage of the weights (conv_desc.w_format). */
typedef enum conv_wformat {
  CONV_W_PLAIN = 0, /* OHWI in the layer's dtype */
  CONV_W_BFP8 = 1   /* bfp8 blocks of 16 along K (conv_pack_bfp8) */
} conv_wformat;

typedef enum conv_status {
  CONV_OK = 0,
  CONV_E_NULL = -1,        /* a required pointer is NULL */
  CONV_E_SHAPE = -2,       /* non-positive size, empty output, c_in or c_out not divisible by groups */
  CONV_E_UNSUPPORTED = -3, /* groups not in {1, c_in==c_out}, depthwise not 3x3, dtype/out/act combination, size limit
                              (a tensor of 2^31 bytes or more, a reduction kh*kw*c_in/groups of 2^24 bytes or more),
                              bad algo */
  CONV_E_ALIGN = -4,       /* x, w or y not 16-byte aligned, or b not 4-byte aligned */
  CONV_E_ALIAS = -5,       /* y overlaps x, w or b */
  CONV_E_NOMEM = -6,       /* allocation of the plan, or of its split-K workspace, failed */
  CONV_E_HIP = -7,         /* the HIP launch reported an error */
  CONV_E_SCRATCH = -8      /* conv_run_noalloc: the split-K partial sums need more than
                              CONV_NOALLOC_SCRATCH_BYTES */
} conv_status;

/* Description of one layer. All sizes in elements. */
typedef struct conv_desc {
  int64_t n, h, w, c_in, c_out;
  int32_t kh, kw;
  int32_t stride_h, stride_w;
  int32_t pad_h, pad_w;   /* each applied to both edges of its axis */
  int32_t groups;         /* 1, or c_in (== c_out) for depthwise */
  int32_t dtype;          /* conv_dtype of x and w: F32, BF16 or I8 */
  int32_t out_dtype;      /* F32 for F32; BF16 for BF16; I8 or I32 for I8 */
  int32_t act;            /* conv_act */
  int32_t algo;           /* 0 = the library chooses the kernel and tile.
                             k > 0 forces one kernel configuration of a
                             dense bf16/int8 layer (for tests and tuning):
                             1..4 the implicit-GEMM tiles, 5 up to
                             conv_algo_count() - 2 the large-layer
                             kernel's tiles, conv_algo_count() - 1 the
                             weight-stationary kernel (reductions of at
                             most 256 bytes per output),
                             conv_algo_count() the halo kernel (3x3 bf16
                             over 32 or 64 input channels, stride 1 or 2,
                             pad <= 2, c_out % 4 == 0); conv_describe
                             names the one chosen. For a depthwise layer
                             with stride 1 and
                             c_in % 4 == 0, k = 1..4 forces 1, 2, 4 or 8
                             output rows per lane of the row-window kernel.
                             A configuration that cannot run the layer gives
                             CONV_E_UNSUPPORTED. */
  int32_t w_format;       /* conv_wformat: how w is stored. CONV_W_PLAIN:
                             OHWI of dtype. CONV_W_BFP8: block floating
                             point as conv_pack_bfp8 writes it (BF16 layers
                             with groups == 1 and c_in * 2 a multiple of 16
                             only; others give CONV_E_UNSUPPORTED). */
  int32_t x_pixel_stride; /* elements from one input pixel to the next: 0
                             (or c_in) for dense NHWC. 8 with c_in <= 8 is
                             the channel-padded input of a bf16 3x3
                             stride-1 first layer (the mosaic packer's
                             c_pad = 8 canvas): channels c_in .. 7 of each
                             pixel are ignored, whatever they hold, and the
                             layer runs on the window stem kernel. Any
                             other value gives CONV_E_UNSUPPORTED (below
                             c_in: CONV_E_SHAPE). */
} conv_desc;

typedef struct conv_plan conv_plan;

/* Validate d and choose the kernel and its launch shape. On success *out
 * holds a new plan (free with conv_destroy); on failure *out is NULL and the
 * return value names the reason. Every unsupported layer is refused here,
 * before any buffer is bound, by a named code rather than a wrong result
 * later (nanoinfer README, the bug list: op/dtype pairs are validated at load
 * so that an unsupported pair is a named load failure; SiMa box-decode page,
 * the YOLO profile: preparation validates the profile and returns a plan that
 * states what execution needs). The only device call is the allocation of the
 * split-K workspace when the plan splits the reduction (conv_describe shows
 * ksplit > 1), on the device current at this call: if that allocation fails,
 * CONV_E_NOMEM. With no HIP device present at all the plan is made unsplit
 * (it can be inspected but not run). */
conv_status conv_prepare(const conv_desc* d, conv_plan** out);

/* Enqueue the layer on `stream` (a hipStream_t; NULL = the default stream).
 *   x : device pointer, NHWC of dtype, 16-byte aligned.
 *   w : device pointer, OHWI of dtype, 16-byte aligned (for w_format
 *       CONV_W_BFP8: the conv_pack_bfp8 image of those weights).
 *   b : F32/BF16 layers: device float[c_out] bias, or NULL for zero bias.
 *       I8 layers: device block of int32 bias[c_out] immediately followed by
 *       float scale[c_out] (one allocation, 4-byte aligned). The scales are
 *       required for I8 output; I32 output reads only the bias and accepts
 *       NULL (zero bias).
 *   y : device pointer, NHWC of out_dtype, 16-byte aligned; must not overlap
 *       x, w or b (a layer reads its input while it writes its output, the
 *       planner-aliasing bug of the nanoinfer README).
 * Calls on different streams may run concurrently with one plan, except for
 * a plan with a split-K workspace (ksplit > 1 in conv_describe): its calls
 * share that workspace and must be ordered (one stream, or events). Run it
 * with the device of conv_prepare current. */
conv_status conv_run(const conv_plan* p, const void* x, const void* w,
                     const void* b, void* y, void* stream);

/* conv_run with a residual added after the activation, written once (YOLOv4
 * on Tenstorrent Wormhole, section 9 "Four custom Tensix kernels", K2: the ResBlock tail
 * computes Mish and adds the skip tensor in one pass instead of storing and
 * reloading the activation):
 *   F32  : y = act(conv + b) + r                      (one fp32 add)
 *   BF16 : y = bf16_rne(act(conv + b) + r)            (sum in fp32, one rounding)
 *   I8   : y = clamp(round_half_even(act(v) + r), -127, 127)
 *          with v as for conv_run and r an int8 value in the output's units:
 *          the exact sum act(v) + r is rounded once (at a half-integer the
 *          even neighbour of the sum wins, e.g. act(v) = 2.5, r = 1 gives 4),
 *          so no intermediate rounding of the activation comes before the
 *          add, as in K2
 *   r : device NHWC [n][ho][wo][c_out] of out_dtype, 16-byte aligned. It may
 *       be y itself (in-place add) but must not otherwise overlap y.
 * The int32 checkpoint output (I8 -> I32) gives CONV_E_UNSUPPORTED. Other
 * arguments, errors and ordering rules as for conv_run. */
conv_status conv_run_residual(const conv_plan* p, const void* x, const void* w,
                              const void* b, const void* r, void* y, void* stream);

/* Block-floating-point weights (the pages' bfp8: weights stored in groups
 * of 16 that share one exponent; YOLOv4 on Tenstorrent Wormhole, the table
 * "Precision in the selected m640 graph" and the glossary; zerolat.eu
 * technology page, "Spend precision selectively"). The pages fix no more
 * than that; the library's format:
 *   * Kp = 16 * ceil(K / 16), K = kh * kw * c_in; each output channel's K
 *     weights, zero-padded to Kp, form Kp / 16 blocks of 16 consecutive
 *     values along K;
 *   * a value is m * 2^(E - 133): m a signed byte in [-127, 127], E the
 *     block's exponent byte. With A the block's largest magnitude,
 *     e = max(floor(log2 A), -126), m = round_half_even(w / 2^(e - 6)), and
 *     e is raised by one if a mantissa would round to 128; E = e + 127 (an
 *     all-zero block has E = 0);
 *   * layout: int8 mantissas [c_out][Kp], then uint8 exponents
 *     [c_out][Kp / 16]; conv_bfp8_bytes(c_out, k) bytes in all.
 * Every decoded value is exactly a bf16 value, so a layer with bfp8 weights
 * computes the bf16 convolution of the decoded weights (fp32 accumulation).
 *
 * conv_pack_bfp8 encodes device weights w (OHWI, c_out rows of k values,
 * dtype CONV_F32 or CONV_BF16, finite, magnitudes below 2^126) into
 * `packed` (device, 16-byte aligned, conv_bfp8_bytes(c_out, k) bytes, not
 * overlapping w), on `stream`. CONV_E_NULL, CONV_E_SHAPE (c_out or k <= 0),
 * CONV_E_UNSUPPORTED (dtype, or more than 2^31 bytes), CONV_E_ALIGN,
 * CONV_E_ALIAS, CONV_E_HIP. conv_bfp8_bytes returns 0 for sizes <= 0. */
int64_t conv_bfp8_bytes(int64_t c_out, int64_t k);
conv_status conv_pack_bfp8(const void* w, int32_t w_dtype, int64_t c_out, int64_t k, void* packed,
                           void* stream);

/* Bytes of the static device array behind conv_run_noalloc (16 MiB, one copy
 * on each device the library runs on, held until the process ends). */
#define CONV_NOALLOC_SCRATCH_BYTES (16 << 20)

/* conv_prepare + conv_run (r == NULL) or conv_run_residual (r != NULL) +
 * conv_destroy in one call that allocates nothing, for callers that cannot
 * allocate: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. The plan lives on this call's stack and a split reduction
 * keeps its partial sums in the library's static device array of
 * CONV_NOALLOC_SCRATCH_BYTES instead of a per-plan workspace; no hipMalloc,
 * hipFree or host heap allocation is made (the first call on a device looks
 * up that device's address of the array once). The kernels, the split and so
 * the results are the same as conv_prepare + conv_run with the same d.
 *   d : layer description as for conv_prepare (host pointer, read only).
 *   x, w, b, r, y, stream : as for conv_run / conv_run_residual.
 * Errors: those of conv_prepare and conv_run / conv_run_residual, except that
 * CONV_E_NOMEM cannot occur; CONV_E_SCRATCH when the split-K partial sums
 * (ksplit * m * c_out * 4 bytes, m = n * ho * wo) exceed
 * CONV_NOALLOC_SCRATCH_BYTES; CONV_E_UNSUPPORTED for a device index of 64 or
 * more; CONV_E_HIP if the array's address cannot be found.
 * Every call on one device shares that device's array and leaves its partial
 * sums there (nothing in it needs clearing: a split call writes every partial
 * it reads). Calls that split and overlap on one device (different streams,
 * host threads on one stream without ordering) race on the array: order them. */
conv_status conv_run_noalloc(const conv_desc* d, const void* x, const void* w, const void* b,
                             const void* r, void* y, void* stream);

/* Two layers in one launch: p1's layer, then p2's 1x1 layer applied to each
 * of p1's output tiles before anything is stored, so p1's output never goes
 * to memory and the stack has one node less (YOLOv4 on Tenstorrent Wormhole,
 * section 10, "Why reducing operation count matters": fewer graph operations
 * and no intermediate write and read). y = layer2(layer1(x)) with layer1's
 * output rounded to bf16 exactly as conv_run would store it; the result is
 * the same as conv_run(p1) into a tensor t, then conv_run(p2) on t.
 * Fusable pairs (conv_fuse_check): p1 bf16 -> bf16 on the implicit-GEMM
 * or the halo kernel with the tap or vec16 gather, its reduction not split,
 * 64 or 128 output channels; p2 bf16 -> bf16, 1x1,
 * stride 1, pad 0, groups 1, plain weights, on p1's output shape, at most 64
 * output channels, a multiple of 4. No residual.
 *   x, w1, b1 : as conv_run for p1; w2, b2 : as conv_run for p2;
 *   y : p2's output, 16-byte aligned, overlapping none of the inputs.
 * The launch runs on the halo kernel when p1 does or when p1's kernel was
 * left to the library and the halo kernel can fuse it (3x3 over 32 or 64
 * input channels, except 64 -> 64 channels at stride 2 over 64), else on
 * the implicit-GEMM kernel; conv_describe_fused names it.
 * CONV_E_NULL, CONV_E_UNSUPPORTED (not a fusable pair), CONV_E_ALIGN,
 * CONV_E_ALIAS, CONV_E_HIP. conv_fuse_check returns CONV_OK or
 * CONV_E_UNSUPPORTED (CONV_E_NULL for a NULL plan). */
conv_status conv_fuse_check(const conv_plan* p1, const conv_plan* p2);
/* conv_describe for a fusable pair: the fused launch's kernel and shape. */
conv_status conv_describe_fused(const conv_plan* p1, const conv_plan* p2, char* buf, int32_t len);
conv_status conv_run_fused(const conv_plan* p1, const conv_plan* p2, const void* x, const void* w1,
                           const void* b1, const void* w2, const void* b2, void* y, void* stream);

/* The first layer of a stack fed by the mosaic, with the mosaic packing
 * folded into the layer's input gather: the canvas never exists
 * (YOLOv4/Wormhole section 4, the m640 layout of four photos in one canvas,
 * and section 10, fewer operations and no intermediate write and read).
 * p : a plan prepared with x_pixel_stride = 8 (the window stem kernel) for
 *     the canvas: n = m canvases, h = 2 th, w = 2 tw, c_in = the tiles'
 *     channels (<= 8).
 * tiles : device [4 m][th][tw][c_in] of tiles_dtype (CONV_F32 or
 *     CONV_BF16), A top-left, B top-right, C bottom-left, D bottom-right of
 *     each canvas, as conv_mosaic_pack takes them; read and rounded to bf16
 *     (RNE) exactly as conv_mosaic_pack writes the canvas.
 * w, b, y : as conv_run. y = conv_run(p) on conv_mosaic_pack(tiles, bf16,
 * c_pad = 8), bit for bit.
 * CONV_E_NULL, CONV_E_UNSUPPORTED (not a window-stem plan, tiles that do not
 * make its canvas, tile dtype), CONV_E_ALIGN (tiles to their element, w and
 * y to 16 bytes, b to 4), CONV_E_ALIAS (y overlapping tiles, w or b),
 * CONV_E_HIP. */
conv_status conv_run_mosaic(const conv_plan* p, const void* tiles, int32_t tiles_dtype, int32_t th, int32_t tw,
                            const void* w, const void* b, void* y, void* stream);

/* Free a plan and the workspace conv_prepare allocated for it; all device
 * memory a plan holds is taken at preparation and given back here, none in
 * between (nanoinfer README, memory planner: no allocations in the forward
 * pass after load). NULL is a no-op. Always CONV_OK. */
conv_status conv_destroy(conv_plan* p);

/* Output shape {n, ho, wo, c_out} of a plan: ho = (h + 2*pad_h - kh) /
 * stride_h + 1 and wo likewise, the floor rule of PyTorch from which the
 * nanoinfer engine takes its shapes (nanoinfer README, the bug list:
 * asymmetric padding collapsed to one axis; the output shapes came from
 * PyTorch). CONV_E_NULL if p or nhwc is NULL. */
conv_status conv_out_shape(const conv_plan* p, int64_t nhwc[4]);

/* Human-readable description of the chosen kernel path and tile, written
 * into buf (NUL-terminated, truncated to len). */
conv_status conv_describe(const conv_plan* p, char* buf, int32_t len);

/* Number of forceable kernel configurations (valid algo values are
 * 1..conv_algo_count()). */
int32_t conv_algo_count(void);

/* Mosaic packing (YOLOv4 on Tenstorrent Wormhole, section 4, the m640 2x2
 * layout): four th x tw x c tiles per canvas, tile 4i+0 top-left, 4i+1
 * top-right, 4i+2 bottom-left, 4i+3 bottom-right of canvas i.
 *   tiles  : device [4*m][th][tw][c] of in_dtype (F32 or BF16)
 *   canvas : device [m][2*th][2*tw][c_pad] of out_dtype (F32 or BF16);
 *            channels c..c_pad-1 are written as zero. fp32 -> bf16 rounds to
 *            nearest even.
 * Both pointers 16-byte aligned, non-overlapping; c_pad >= c. */
conv_status conv_mosaic_pack(const void* tiles, int32_t in_dtype, void* canvas,
                             int32_t out_dtype, int32_t m, int32_t th,
                             int32_t tw, int32_t c, int32_t c_pad,
                             void* stream);

/* SPP max-pool block (YOLOv4 on Tenstorrent Wormhole, section 9 "Four custom
 * Tensix kernels", K3; section 3 for the block's role): for each pixel, the maximum over
 * the 13x13, 9x9 and 5x5 windows centred on it (stride 1, output the size of
 * the input, positions outside the map ignored, i.e. padding with -infinity),
 * concatenated with the map itself:
 *   y[n][h][w][j*c + ch], j = 0, 1, 2, 3 = max13, max9, max5, x.
 *   x : device [n][h][w][c] of dtype (F32, BF16 or I8)
 *   y : device [n][h][w][4c] of the same dtype; every value is an input value
 *       (bit-exact; of a -0 and a +0 in one window the +0 is returned).
 * Both 16-byte aligned and non-overlapping. c must be a multiple of 8 (BF16,
 * I8) or 4 (F32) and h*w at most 2048 (CONV_E_UNSUPPORTED otherwise); y must
 * be smaller than 2^31 bytes. Enqueues one kernel on `stream`. */
conv_status conv_spp_maxpool(const void* x, int32_t dtype, void* y, int32_t n,
                             int32_t h, int32_t w, int32_t c, void* stream);

/* Upsample x2 + concat (YOLOv4 on Tenstorrent Wormhole, section 9 "Four custom
 * Tensix kernels", K4): two maps joined along channels in the NHWC layout the next
 * convolution reads, each repeated 2x in rows and columns (nearest
 * neighbour) when its up flag is 1:
 *   y[n][i][j][k]      = s0[n][i >> up0][j >> up0][k]       k < c0
 *   y[n][i][j][c0 + k] = s1[n][i >> up1][j >> up1][k]       k < c1
 *   s0 : device [n][ho >> up0][wo >> up0][c0] of dtype (F32, BF16 or I8)
 *   s1 : device [n][ho >> up1][wo >> up1][c1] of dtype
 *   y  : device [n][ho][wo][c0 + c1] of dtype; a byte copy (bit-exact).
 * up flags 0 or 1; ho and wo even when either is 1 (CONV_E_SHAPE otherwise).
 * All three pointers 16-byte aligned; y must not overlap s0 or s1. c0 and c1
 * must be whole 16-byte chunks (multiples of 4 for F32, 8 for BF16, 16 for
 * I8), n*ho at most 65535, y smaller than 2^31 bytes (CONV_E_UNSUPPORTED
 * otherwise). Enqueues one kernel on `stream`. */
conv_status conv_upsample_concat(const void* s0, int32_t c0, int32_t up0,
                                 const void* s1, int32_t c1, int32_t up1,
                                 int32_t dtype, void* y, int32_t n, int32_t ho,
                                 int32_t wo, void* stream);

/* The YOLOv4 neck join read straight by the convolution that follows it
 * (YOLOv4 on Tenstorrent Wormhole, section 9 "Four custom Tensix kernels",
 * K4: the join is written in the next convolution's layout; here the
 * convolution reads the two maps itself and the joined map is never
 * written). p is a 1x1, stride-1, unpadded, dense layer (BF16 or I8, plain
 * weights) whose input is the channel concat of conv_upsample_concat:
 *   x[n][i][j][k]      = s0[n][i >> up0][j >> up0][k]       k < c0
 *   x[n][i][j][c0 + k] = s1[n][i >> up1][j >> up1][k]       k < c_in - c0
 *   s0 : device [n][h >> up0][w >> up0][c0] of p's dtype
 *   s1 : device [n][h >> up1][w >> up1][c_in - c0] of p's dtype
 *   w, b, y, stream : as for conv_run (y [n][h][w][c_out]).
 * up flags 0 or 1, h and w even when either is 1, 0 < c0 < c_in
 * (CONV_E_SHAPE otherwise); c0 and c_in - c0 whole 128-byte blocks (multiples
 * of 64 for BF16, 128 for I8; CONV_E_UNSUPPORTED otherwise, as for other
 * layers). s0, s1, w, y 16-byte aligned (b 4-byte); y must not overlap s0,
 * s1, w or b (CONV_E_ALIAS). Runs the implicit-GEMM kernel with p's tile (the
 * 64x64 tile when p chose another kernel), the reduction unsplit: the result
 * equals conv_upsample_concat + conv_run up to the order of the fp32 sums
 * (bit-equal when p runs that tile unsplit; int8 always). Enqueues one kernel
 * on `stream`. */
conv_status conv_run_upcat(const conv_plan* p, const void* s0, int32_t c0, int32_t up0, const void* s1,
                           int32_t up1, const void* w, const void* b, void* y, void* stream);

/* Name and meaning of a status code ("CONV_OK", "CONV_E_SHAPE: ..."), so a
 * refusal reads as a named failure rather than quiet garbage (nanoinfer
 * README, the bug list). For CONV_E_HIP the text of the last HIP error seen
 * by this thread is appended. The string is static or thread-local: valid
 * until the next call on the same thread. */
const char* conv_status_str(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* CONV_NHWC_H */
