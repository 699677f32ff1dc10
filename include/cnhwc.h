/*
 * cnhwc.h -- C ABI of the channels-last convolution forward library for AMD
 * MI355X (gfx950).
 *
 * The operations are the ones three MLX pull requests discuss for Metal; this
 * library computes the same things with its own HIP kernels:
 *
 *   [tiling page]   MLX PR "Bound winograd conv2d working set by tiling the
 *                   batch" -- sections Problem, Fix, Testing and the review
 *                   comments (M4 Pro / M5 Max verification).
 *   [explicit page] MLX PR "Use the explicit gemm for wide convs on neural
 *                   accelerators" -- intro tables, Verified, Notes, the ResNet-50
 *                   and memory follow-ups.
 *   [3D page]       MLX PR "Decompose small kernel-depth 3D convs into 2D convs"
 *                   -- sections Problem, Change, Results, Tests, Open questions.
 *
 * Operation.  Cross-correlation (no kernel flip), zero padding, groups = 1:
 *   y[n,(od,)oh,ow,o] = sum_{(kd,)kh,kw,c} x[n,(id,)ih,iw,c] * w[o,(kd,)kh,kw,c]
 *   with ih = oh*stride_h - pad_h + kh*dil_h (likewise w, d), x = 0 outside.
 *   Output extent per dim: floor((in + 2*pad - dil*(k-1) - 1)/stride) + 1.
 *
 * Layouts (all dense, row-major, element type = desc.dtype):
 *   x  [N,H,W,C]  (2D)   or [N,D,H,W,C]  (3D)     -- channels-last input
 *   w  [O,KH,KW,C](2D)   or [O,KD,KH,KW,C](3D)    -- output channel outermost
 *   y  [N,OH,OW,O](2D)   or [N,OD,OH,OW,O](3D)
 * Arithmetic: products accumulate in fp32 for every dtype; the output is rounded
 * once to the dtype, round-to-nearest-even.  Winograd keeps its transformed
 * tensors in fp32 whatever the input dtype.
 *
 * Ownership and threading.  The caller owns x, w, y, the workspace and the
 * stream; they must stay valid until the work queued on the stream completes.
 * The library allocates no device memory, keeps no global state, never
 * synchronises and reads no environment variable.  Every call is thread-safe.
 * (The one exception is cnhwc_conv2d_fwd_noalloc, which takes its workspace
 * from a fixed device array the library holds per GPU; see there.)
 * The forward calls only queue kernels on the given HIP stream (NULL = the
 * default stream); device faults therefore surface at the caller's next
 * synchronisation.
 *
 * Errors.  Every call returns a status.  The forward calls validate every
 * argument and the plan before queueing any work; on any error nothing is
 * queued and y is left untouched.  A forced algorithm that cannot run returns
 * CNHWC_ERR_NOT_APPLICABLE (or CNHWC_ERR_BUDGET for Winograd over budget); the
 * library never silently falls back to another algorithm -- only
 * CNHWC_ALGO_AUTO selects, deterministically.  (The tiling page's Problem
 * section is about the opposite behaviour: a failed command buffer whose error
 * was dropped left an all-zero output.)
 */
#ifndef CNHWC_H_
#define CNHWC_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CNHWC_ABI_VERSION 4

/* Fewest GEMM rows (tile_batch * tiles_per_image) a Winograd batch tile may
 * carry when the batch does not fit in one tile; below it AUTO falls back to
 * implicit GEMM.  The tiling page (Fix) falls back when tiles carry too few
 * GEMM rows to amortise their fixed cost but gives no number; this value is
 * our reading. */
#define CNHWC_MIN_TILE_ROWS 256

/* Byte cap of one unfold chunk (rows * K * element size).  The explicit page
 * (Notes) says the unfold is tiled against a buffer limit and reuses one
 * buffer; the limit here is a fixed constant, never live memory. */
#define CNHWC_UNFOLD_CAP_BYTES (256ull << 20)

/* AUTO takes unfold+GEMM for fp16/bf16 2D convs with C_out >= this value that
 * no earlier rule took (explicit page: the rule is on the output-channel count
 * and only for half precision).  On MI355X the measured sweep (C_out 128..4096,
 * M = 1024..65536, K = 1152..9216, fp16 and bf16) never shows unfold+GEMM
 * ahead of the implicit GEMM beyond noise, so the threshold is out of reach:
 * AUTO does not unfold wide convs (it still unfolds convs with C % 8 != 0, see
 * cnhwc_conv_select), and CNHWC_ALGO_UNFOLD_GEMM stays available when forced. */
#define CNHWC_UNFOLD_MIN_COUT (1 << 30)

typedef enum { CNHWC_F32 = 0, CNHWC_F16 = 1, CNHWC_BF16 = 2 } cnhwc_dtype_t;

typedef enum {
  CNHWC_ALGO_AUTO = 0,
  CNHWC_ALGO_WINOGRAD = 1,      /* 3x3 stride-1 dilation-1 2D only */
  CNHWC_ALGO_IMPLICIT_GEMM = 2, /* any 2D conv; scratch-free */
  CNHWC_ALGO_UNFOLD_GEMM = 3,   /* any 2D conv; unfold buffer in the workspace */
  CNHWC_ALGO_SMALL_KD = 4,      /* 3D as KD accumulated 2D convs (3D: IMPLICIT_GEMM = native) */
  CNHWC_ALGO_WINOGRAD_HALF = 5  /* fp16/bf16 Winograd F(4x4,3x3), 2D and 3D (see below) */
} cnhwc_algo_t;

typedef enum {
  CNHWC_OK = 0,
  CNHWC_ERR_INVALID_ARGUMENT = 1,  /* bad descriptor, null/misaligned pointer */
  CNHWC_ERR_UNSUPPORTED = 2,       /* valid conv outside what this library runs */
  CNHWC_ERR_NOT_APPLICABLE = 3,    /* the forced algorithm cannot run this conv */
  CNHWC_ERR_BUDGET = 4,            /* forced Winograd: not one element fits */
  CNHWC_ERR_WORKSPACE_TOO_SMALL = 5,
  CNHWC_ERR_PLAN_MISMATCH = 6,     /* plan != cnhwc_conv_select(desc, plan.opts) */
  CNHWC_ERR_HIP = 7,               /* a kernel launch reported an error */
  CNHWC_ERR_INTERNAL = 8
} cnhwc_status_t;

/* Convolution descriptor.  For nd == 2 set d = kd = 1, and index 0 of
 * stride/pad/dil to 1/0/1.  Index order of the triples: depth, height, width.
 * conv1d is nd == 2 with h = kh = 1 (x [N,1,L,C], w [O,1,K,C]): the 1D conv
 * goes through the 2D dispatch (explicit page, Whisper follow-up). */
typedef struct {
  int32_t nd;        /* 2 or 3 */
  int32_t dtype;     /* cnhwc_dtype_t: element type of x, w and y */
  int64_t n, d, h, w, c, o, kd, kh, kw;  /* each in [1, 2^31]; an empty batch (n = 0)
                                            is INVALID_ARGUMENT: there is no work to plan.
                                            d + 2*pad[0], h + 2*pad[1], w + 2*pad[2]
                                            and c above 2^30 are UNSUPPORTED (the
                                            gathers index in 32-bit integers). */
  int32_t stride[3];
  int32_t pad[3];
  int32_t dil[3];
  int32_t groups;    /* must be 1 */
} cnhwc_conv_desc_t;

/* Selection options.  The selection depends on these and the descriptor only,
 * never on free memory (tiling page, review; explicit page, closing review). */
typedef struct {
  uint64_t ws_limit_bytes;   /* W: the device working-set figure, or an injected
                                budget (tiling page, Testing).  Must be > 0.  The
                                Winograd budget is floor(3/4 W) - own bytes. */
  int32_t force_algo;        /* cnhwc_algo_t; AUTO = select */
  int32_t force_inner_algo;  /* SMALL_KD only: per-tap 2D algorithm; AUTO = select */
  int64_t force_tile_batch;  /* Winograd: 0 = budget rule; else min(value, budget tile) */
  int64_t force_unfold_rows; /* Unfold: 0 = the fixed byte cap; else rows per chunk */
  int32_t force_gemm_config; /* 0 = select; else a GEMM tile configuration id for the
                                implicit / unfold GEMM (fp16/bf16: 10..16; fp32: 1..4).
                                16 is the implicit GEMM of 3x3 stride-1 dilation-1
                                convs with C % 64 == 0 that stages each input patch
                                in LDS once per 64 channels (K ordered depth tap,
                                64-channel chunk, kh, kw).  An id that does not suit
                                the dtype or the shape is CNHWC_ERR_NOT_APPLICABLE. */
  int32_t force_split_k;     /* implicit / unfold GEMM: 0 = select, 1 = no K split,
                                s > 1 = s splits of whole K chunks (trailing empty
                                splits dropped).  NOT_APPLICABLE with the 256-row
                                tiles (14, 15, 16) or for more splits than K chunks.
                                Winograd ignores it. */
} cnhwc_select_opts_t;

/* A plan: a plain value, a pure function of (descriptor, options). */
typedef struct {
  int32_t algo;              /* resolved algorithm, never AUTO */
  int32_t inner_algo;        /* SMALL_KD: per-tap 2D algorithm; else == algo */
  int64_t out_d, out_h, out_w;
  int64_t tile_batch;        /* Winograd: batch elements per tile (3D: frames) */
  int64_t n_tiles;           /* Winograd: number of batch tiles */
  int64_t tiles_per_image;   /* Winograd: ceil(OH/6) * ceil(OW/6) */
  int64_t unfold_rows;       /* Unfold: output rows per chunk */
  int64_t n_chunks;          /* Unfold: number of chunks */
  uint64_t own_bytes;        /* Winograd: bytes of x + y + transformed filter */
  uint64_t budget_bytes;     /* Winograd: floor(3/4 W) - own, 0 if negative */
  uint64_t scratch_per_element; /* Winograd: V + M bytes of one batch element */
  uint64_t workspace_bytes;  /* bytes the forward call needs in `workspace` */
  int32_t kernel_config;     /* GEMM tile configuration id */
  int32_t split_k;           /* implicit / unfold GEMM: K splits (1 = none).  With
                                s > 1 the GEMM grid is too small to fill the device:
                                split i sums its share of K into an fp32 slice of
                                the workspace, and a second kernel adds the slices
                                in order 0..s-1, so the result is still a function
                                of the plan and the data only. */
  cnhwc_select_opts_t opts;  /* the options this plan was made from */
} cnhwc_plan_t;

/* Returns CNHWC_ABI_VERSION.  No page passage defines it: it versions this
 * header's structs and entry points for the caller's binding. */
int cnhwc_abi_version(void);

/* Human-readable name of a status (static storage; never NULL).  Every call
 * returns a status because of the failure the tiling page's Problem section
 * describes: a command-buffer error that was dropped left a silent all-zero
 * output.  This names the status; it implements no conv operation. */
const char* cnhwc_status_string(cnhwc_status_t s);

/* Algorithm selection and memory planning (host only, no device call).
 *
 * AUTO, 2D, in order (tiling page, Problem and Fix; explicit page, Notes):
 *  1. Winograd when KH = KW = 3, stride 1, dilation 1, C % 32 == 0,
 *     O % 32 == 0, C + O >= 256 and dtype == F32, and the budget rule admits
 *     it: tile = min(N, floor(budget / scratch_per_element)); fall back if
 *     tile < 1, or if tile < N and tile * tiles_per_image < CNHWC_MIN_TILE_ROWS.
 *  1b. WINOGRAD_HALF for F16/BF16 where its geometry holds (below),
 *     KD*C >= 384, KD*C*O >= 13*(11*C + 20*O) and
 *     N * OD * ceil(OH/4) * ceil(OW/4) >= 512 (KD = OD = 1 in 2D), under the
 *     same budget rule: the measured crossover against the implicit GEMM on
 *     MI355X (the tiling page runs its Winograd path for half precision too).
 *  2. Unfold + GEMM for F16/BF16 with O >= CNHWC_UNFOLD_MIN_COUT, or with
 *     C % 8 != 0: the implicit GEMM would then gather its A operand element by
 *     element for every column tile, while the unfold gathers once and the GEMM
 *     reads dense 16-byte rows (measured 1.3-1.9x faster on such convs above
 *     the ~20 us launch floor, e.g. the 3-channel stem; at the floor within a
 *     few microseconds either way).
 *  3. Implicit GEMM.
 * AUTO, 3D: first WINOGRAD_HALF under rule 1b (the depth taps summed in its
 *   GEMMs).  Then (3D page, Change): SMALL_KD when N == 1, KD <= 7, depth stride 1,
 *   dilation 1 in every dim, depth pad 0, C % 16 == 0 and O % 16 == 0 and the
 *   per-tap 2D algorithm (AUTO-selected on the [OD,H,W,C] frame conv, or
 *   forced by force_inner_algo) is Winograd; the decomposition exists to give
 *   the frames the 2D Winograd path.  Otherwise IMPLICIT_GEMM: the native 3D
 *   implicit GEMM, one GEMM with K = KD*KH*KW*C over the NDHWC gather (any
 *   batch, depth stride, padding and dilation; the page's fall-through for
 *   what the guard rejects, and the decomposition with its taps fused).
 * WINOGRAD_HALF (the half-precision Winograd path; tiling page, Problem: the
 *   three-stage Winograd structure; 3D page, Change: a 3D conv as a sum of
 *   per-frame 2D convs over its depth taps).  F(4x4,3x3): 6x6 input tiles at
 *   stride 4, 36 tile positions.  The transformed input and filter are stored
 *   as fp16 scaled by powers of two that the device picks from max|x| and
 *   max|w| over the whole tensors (so no transformed value can overflow fp16,
 *   and batch tiles keep the untiled bits); the 36 GEMMs accumulate in fp32
 *   on the fp16 matrix cores into fp32 results, and the output transform
 *   undoes the scales exactly.  3D: the depth taps are summed inside each
 *   GEMM (K = KD * Cs, tap kd reading the transformed frames kd * dilation
 *   further on), then one output transform; any batch (one element per
 *   batch tile), depth pad and depth dilation, depth stride 1.  Needs dtype
 *   F16 or BF16, KH = KW = 3, stride 1, dilation 1 and padding <= 1 in the
 *   image plane, and C >= 16; otherwise NOT_APPLICABLE.  (The fp16 rounding
 *   of a tile scales with the whole 6x6 tile: with padding 2 a corner window
 *   holds one real pixel of nine and its error reaches 1-3e-2 of its own
 *   sum |x||w|; below 16 channels the rounding errors do not average down.)  The batch is tiled by the budget rule with
 *   scratch_per_element = 36 * tiles * (frames * Cs * 2 + OD * O * 4) bytes
 *   (Cs = C rounded up to 32); force_tile_batch applies to 2D only.
 *   force_gemm_config may name 14 or 15 (the 256-row tiles); force_split_k is
 *   ignored.  AUTO takes it by rule 1b.  Error: |y - conv| stays below
 *   5e-3 of sum |x||w| on independent, identically distributed data (the fp16
 *   rounding of the transformed operands; about 1e-3 at C = 256); see the
 *   accuracy note below for data with sharp contrast.  An output whose whole
 *   tile only holds values below about 2^-24 of max|x| also loses relative
 *   precision (fp16 subnormals).
 * Accuracy of both Winograd forms: the transforms round a tile's values at
 *   the scale of the largest ones in it, so the error is bounded relative to
 *   the tile, |y - conv| <= tol * (largest sum|x||w| among the outputs of the
 *   same tile: 6x6 outputs for WINOGRAD, 4x4 for WINOGRAD_HALF), with tol
 *   2e-5 (F32) and 1e-2 (F16/BF16).  Without sharp contrast inside a tile
 *   that is the per-output bound.  An output whose own window is 100x dimmer
 *   than the brightest part of its tile exceeds the per-output bound
 *   (measured: 2.7e-5 of its own sum |x||w| for WINOGRAD, 1.5-1.7e-2 for
 *   WINOGRAD_HALF; 2.9e-4 and 0.14-0.20 at 1000x).  The implicit and unfold
 *   GEMMs meet the per-output bound at any contrast.  Selection depends on
 *   shapes only, so a caller with such data forces IMPLICIT_GEMM.
 *   Exact zeros: an output whose window meets no nonzero input pixel (any
 *   channel; padding counts as zero) under a nonzero filter tap (any channel)
 *   is exactly 0 on both forms, as on the GEMM paths: the input transform
 *   records which pixels of each tile are nonzero, the filter transform which
 *   taps of each filter are, and the output transform stores 0 for such
 *   outputs (3D: over every depth tap).  An output whose products vanish only
 *   because its pixels' and its taps' nonzero channels never coincide is not
 *   detected and keeps the tile-relative bound.
 * Forcing: WINOGRAD needs only 3x3/stride 1/dilation 1 (the channel gates are
 *   skipped); a forced tile size is capped by the budget tile (tiling page,
 *   Testing).  SMALL_KD needs N == 1, depth stride 1, depth dilation 1, depth
 *   pad 0.  For 3D, IMPLICIT_GEMM (the native path) and SMALL_KD can be
 *   forced, and WINOGRAD_HALF; WINOGRAD and UNFOLD_GEMM are NOT_APPLICABLE,
 *   and force_inner_algo with the native path or WINOGRAD_HALF is
 *   INVALID_ARGUMENT (force_inner_algo never names WINOGRAD_HALF: the
 *   per-frame convs of SMALL_KD accumulate, which its output transform does
 *   not).
 * Returns OK and fills *plan, or an error (plan untouched). */
cnhwc_status_t cnhwc_conv_select(const cnhwc_conv_desc_t* desc, const cnhwc_select_opts_t* opts,
                                 cnhwc_plan_t* plan);

/* The Winograd batch-tiling rule alone, as select applies it (tiling page,
 * Fix): budget = floor(3/4 * ws_limit) - own (0 if negative);
 * tile = min(n, floor(budget / scratch_per_element)); with force_tile > 0,
 * tile = min(force_tile, that).  *tile_batch = 0 means "does not fit";
 * *fallback = 1 when AUTO would fall back to implicit GEMM (tile < 1, or
 * tile < n with tile * rows_per_element < CNHWC_MIN_TILE_ROWS and no forced
 * tile).  Exposed so callers can evaluate the rule with other buffer sets. */
cnhwc_status_t cnhwc_winograd_tile_rule(uint64_t ws_limit, uint64_t own_bytes,
                                        uint64_t scratch_per_element, int64_t n,
                                        int64_t rows_per_element, int64_t force_tile,
                                        int64_t* tile_batch, uint64_t* budget_bytes,
                                        int32_t* fallback);

/* 2D forward: y = conv2d(x, w) with the given plan (from cnhwc_conv_select on
 * this desc; re-derived and compared, CNHWC_ERR_PLAN_MISMATCH otherwise).
 * x, w, y: device pointers, 16-byte aligned, layouts above, not overlapping y.
 * workspace: device pointer, 16-byte aligned, >= plan.workspace_bytes (may be
 * NULL when that is 0), not overlapping x, w or y; contents on entry are
 * ignored, on exit undefined.  x and w may overlap each other (both are only
 * read); any other overlap is CNHWC_ERR_INVALID_ARGUMENT.
 * hip_stream: a hipStream_t (NULL = default stream).
 * Winograd runs the batch in plan.n_tiles tiles of plan.tile_batch elements
 * (the last may be shorter) through one workspace; the result is bit-identical
 * for every tile size (tiling page, Testing).  Unfold runs plan.n_chunks row
 * chunks through one buffer (explicit page, Notes). */
cnhwc_status_t cnhwc_conv2d_fwd(const cnhwc_conv_desc_t* desc, const cnhwc_plan_t* plan,
                                const void* x, const void* w, void* y, void* workspace,
                                uint64_t workspace_bytes, void* hip_stream);

/* 3D forward (nd == 3), same conventions.  IMPLICIT_GEMM: one GEMM over the
 * NDHWC gather, rows (n, od, oh, ow), k = ((kd*KH + kh)*KW + kw)*C + c, the
 * weight rows [O][KD*KH*KW*C] as they are.  SMALL_KD (3D page, Change): for each
 * depth tap kd, the frames x[0, kd:kd+OD] (a pointer offset) and the weight
 * slice w[:, kd] (a strided view) form a 2D conv with batch OD, computed by the
 * plan's inner algorithm and accumulated in fp32 (in y itself for F32, in the
 * workspace otherwise); the last tap rounds into y once.  KD == 1 gives the
 * same bits as conv2d on the [D,H,W,C] frames.  WINOGRAD_HALF: per batch
 * element, the input transform of its D + 2*pad frames (pad frames zero), the
 * 36 GEMMs with the KD taps in K, and one output transform into y. */
cnhwc_status_t cnhwc_conv3d_fwd(const cnhwc_conv_desc_t* desc, const cnhwc_plan_t* plan,
                                const void* x, const void* w, void* y, void* workspace,
                                uint64_t workspace_bytes, void* hip_stream);

/* Kinds of the kernels a forward call launches (for the timed variants). */
typedef enum {
  CNHWC_KERNEL_END = 0,          /* the event after the last kernel */
  CNHWC_KERNEL_WINO_FILTER = 1,  /* Winograd filter transform (once per call, per 3D tap) */
  CNHWC_KERNEL_WINO_INPUT = 2,   /* Winograd input transform (per batch tile) */
  CNHWC_KERNEL_WINO_GEMM = 3,    /* the 64 tile-position GEMMs of one batch tile */
  CNHWC_KERNEL_WINO_OUTPUT = 4,  /* Winograd output transform (per batch tile) */
  CNHWC_KERNEL_IMPLICIT_GEMM = 5,
  CNHWC_KERNEL_UNFOLD = 6,       /* one unfold chunk */
  CNHWC_KERNEL_UNFOLD_GEMM = 7,  /* the dense GEMM of one unfold chunk */
  CNHWC_KERNEL_SPLITK_REDUCE = 8, /* sum of the K-split partial sums + epilogue */
  CNHWC_KERNEL_WINO_SCALE = 9     /* half-precision Winograd: the max |x|, max |w| pass */
} cnhwc_kernel_kind_t;

/* Number of kernels a forward call with this plan launches (3D: over all
 * taps), or -1 if the plan is invalid for the descriptor. */
int64_t cnhwc_launch_count(const cnhwc_conv_desc_t* desc, const cnhwc_plan_t* plan);

/* Timed variants, for measurement: identical work to cnhwc_conv2d_fwd /
 * cnhwc_conv3d_fwd, and in addition hipEventRecord(events[i], stream) right
 * before the i-th kernel launch and once after the last one, with kinds[i] =
 * its cnhwc_kernel_kind_t (CNHWC_KERNEL_END for the final event).  events:
 * n_events hipEvent_t handles created by the caller; n_events must be at least
 * cnhwc_launch_count() + 1 (CNHWC_ERR_INVALID_ARGUMENT otherwise, nothing
 * queued).  kinds may be NULL.  Elapsed time between events i and i+1 is the
 * duration of kernel i on the stream. */
cnhwc_status_t cnhwc_conv2d_fwd_timed(const cnhwc_conv_desc_t* desc, const cnhwc_plan_t* plan,
                                      const void* x, const void* w, void* y, void* workspace,
                                      uint64_t workspace_bytes, void* hip_stream,
                                      void* const* events, int32_t n_events, int32_t* kinds);
cnhwc_status_t cnhwc_conv3d_fwd_timed(const cnhwc_conv_desc_t* desc, const cnhwc_plan_t* plan,
                                      const void* x, const void* w, void* y, void* workspace,
                                      uint64_t workspace_bytes, void* hip_stream,
                                      void* const* events, int32_t n_events, int32_t* kinds);

/* Bytes of the device array that cnhwc_conv2d_fwd_noalloc takes its workspace
 * from (one array per GPU). */
#define CNHWC_NOALLOC_SCRATCH_BYTES (64ull << 20)

/* Allocation-free 2D forward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Identical work to cnhwc_conv2d_fwd, with the workspace taken
 * from a CNHWC_NOALLOC_SCRATCH_BYTES device array that the library holds, one
 * per GPU, until the process ends.  desc, plan, x, w and y follow
 * cnhwc_conv2d_fwd; hip_stream must belong to the current device
 * (CNHWC_ERR_INVALID_ARGUMENT otherwise).  A plan with workspace_bytes above
 * CNHWC_NOALLOC_SCRATCH_BYTES is CNHWC_ERR_WORKSPACE_TOO_SMALL and nothing is
 * queued: plan such convs with a smaller ws_limit_bytes, tile or unfold row
 * count.  The call allocates nothing (no hipMalloc or hipFree).  All calls on
 * one GPU share its array; every kernel writes the scratch it reads within
 * the same call, so nothing carries over between calls, but calls whose work
 * overlaps in time on one GPU (two streams or two threads) race on the array:
 * the caller serialises them.  The first call on a device looks the array's
 * address up (hipGetSymbolAddress); make it outside graph capture. */
cnhwc_status_t cnhwc_conv2d_fwd_noalloc(const cnhwc_conv_desc_t* desc, const cnhwc_plan_t* plan,
                                        const void* x, const void* w, void* y, void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* CNHWC_H_ */
