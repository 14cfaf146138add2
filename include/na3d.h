/*
 * na3d.h -- C ABI of the MI355X (gfx950) library for the forward pass of
 * 3-D neighborhood attention (NA3D).
 *
 * Operation (ROCm/aiter PR "Add 3D neighborhood flash attention (na3d_flash)",
 * Motivation and Technical Details):
 *   For every batch b, head n and query token (t,h,w) of a T x H x W grid,
 *     out[b,t,h,w,n,:] = sum_j softmax_j( q[b,t,h,w,n,:] . k[b,j,n,:] ) v[b,j,n,:]
 *   where j runs over the KT x KH x KW box of key tokens starting, per axis, at
 *     start(i, K, L) = clamp(i - K/2, 0, L - K)          (integer K/2)
 *   i.e. the box is centred on the query and shifted inward at a border so it
 *   always holds exactly KT*KH*KW keys.  Q is expected to be pre-multiplied
 *   by head_dim^-0.5 by the caller; the library applies no further scale.
 *   Scores, softmax and the weighted sum are accumulated in fp32; the softmax
 *   weights are rounded to bf16 before the weighted sum (flash-attention style);
 *   the output is rounded to bf16 (round to nearest even).
 *
 * Layout: q, k, v and out are contiguous bf16 tensors of shape
 *   (B, T, H, W, NH, HD), HD fastest (the public launcher's layout on the
 *   same page).  Element (b,t,h,w,n,d) is at
 *   ((((b*T + t)*H + h)*W + w)*NH + n)*HD + d.
 *
 * Ownership: every pointer is a DEVICE pointer owned by the caller.  The
 *   library allocates nothing, frees nothing and keeps no pointer after a
 *   call returns.  out must not overlap q, k or v; q, k and v may alias each
 *   other (they are only read).
 *
 * Asynchrony: na3d_fwd enqueues its kernel on `stream` (a hipStream_t; NULL
 *   means the default stream) and returns without synchronising.  A fault
 *   during execution is reported by the caller's next synchronising call.
 *   No entry point allocates, copies between host and device or
 *   synchronises, so every call may be captured in a HIP graph.
 *
 * Errors: every function returns 0 on success or a negative NA3D_ERR_* code.
 *   All argument checks run before any device call, so a rejected call has
 *   no effect on the device.  Nothing is printed and no exception crosses
 *   the ABI.
 *
 * Library state: the library keeps three process-wide caches, each a
 *   memo of a pure function of its key, so no result depends on what they
 *   hold and calls from several threads are safe (a mutex guards the first,
 *   atomics the others):
 *   - launch plans keyed by every size, box, requested configuration and
 *     K/V span of a call (at most 4096 entries; when full it is emptied and
 *     refilled); the planner is deterministic, so a cached plan is the plan
 *     the call would compute;
 *   - per device, whether it is gfx950;
 *   - per kernel instantiation and device, the largest dynamic-LDS limit
 *     already raised with hipFuncSetAttribute (so a later launch, also under
 *     graph capture, makes no other runtime call).
 *   None of them holds a caller's pointer or device memory.
 */
#ifndef NA3D_H_
#define NA3D_H_

#ifdef __cplusplus
extern "C" {
#endif

#define NA3D_OK 0
#define NA3D_ERR_NULL (-1)     /* a tensor pointer is NULL */
#define NA3D_ERR_SHAPE (-2)    /* a dimension is < 1, or the tensor is too large */
#define NA3D_ERR_WINDOW (-3)   /* a window extent is < 1 or exceeds its grid axis */
#define NA3D_ERR_HEAD_DIM (-4) /* HD is not one of 16, 32, 64, 128, 256 */
#define NA3D_ERR_ALIGN (-5)    /* a pointer is not 16-byte aligned */
#define NA3D_ERR_OVERLAP (-6)  /* an output overlaps an input it must not overlap */
#define NA3D_ERR_DEVICE (-7)   /* the current HIP device is not gfx950 */
#define NA3D_ERR_LAUNCH (-8)   /* the kernel launch was rejected by HIP */
#define NA3D_ERR_CONFIG (-9)   /* an explicit launch configuration cannot run the sizes */
#define NA3D_ERR_STRIDE (-10)  /* a stride set na3d_fwd_strided cannot take (see there) */
#define NA3D_ERR_BOX (-11)     /* a query box that is empty or reaches outside the grid */
#define NA3D_ERR_VALUE (-12)   /* a scalar argument out of range (RMSNorm eps) */

/*
 * Forward pass of 3-D neighborhood attention.
 *   q, k, v : device pointers, bf16, (B,T,H,W,NH,HD) contiguous, 16-B aligned
 *   out     : device pointer, bf16, same shape; fully overwritten
 *   B,T,H,W : batch and grid extents (>= 1)
 *   NH, HD  : heads and head dimension (HD in {16,32,64,128,256})
 *   KT,KH,KW: window extents, 1 <= K <= the matching grid extent (even
 *             extents are accepted and follow the same start formula)
 *   stream  : hipStream_t to enqueue on, or NULL for the default stream
 * Returns NA3D_OK or a negative NA3D_ERR_* code.
 */
int na3d_fwd(const void* q, const void* k, const void* v, void* out, int B,
             int T, int H, int W, int NH, int HD, int KT, int KH, int KW,
             void* stream);

/*
 * The argument checks of na3d_fwd alone, without touching any device
 * (NULL pointers, dimensions, window extents, head dimension, alignment,
 * overlap).  Returns NA3D_OK or the code na3d_fwd would return.
 */
int na3d_check_args(const void* q, const void* k, const void* v,
                    const void* out, int B, int T, int H, int W, int NH,
                    int HD, int KT, int KH, int KW);

/* Static, NUL-terminated description of a status code. */
const char* na3d_status_string(int status);

/*
 * Launch plan na3d_fwd would use for these sizes, without touching a device:
 * plan[0] = kernel family id (1 general, 2 rolling), plan[1] = query planes
 * per (middle) run of a workgroup, plan[2] = tile extent along H, plan[3] =
 * tile extent along W, plan[4] = workgroups, plan[5] = threads per
 * workgroup, plan[6] = dynamic LDS bytes, plan[7] = most K/V planes staged
 * by one workgroup, plan[8] = rolling instantiation index (0 for the general
 * family), plan[9] = workgroups along T per spatial tile (the rolling family
 * splits T into runs of query planes, the planes that share the first or the
 * last window in runs of their own, and a workgroup streams one or more
 * consecutive runs).
 * `plan` must hold 10 ints.  Returns NA3D_OK or an NA3D_ERR_* code for
 * invalid sizes.
 */
int na3d_plan(int B, int T, int H, int W, int NH, int HD, int KT, int KH,
              int KW, int* plan);

/*
 * na3d_fwd with an explicit launch configuration, for tuning sweeps and for
 * testing each kernel instantiation on its own.
 *   family : 0 = automatic (exactly na3d_fwd), 1 = general family (one query
 *            plane per workgroup, no limit on window size), 2 = rolling
 *            family (a run of query planes per workgroup)
 *   variant: rolling instantiation, 0 .. na3d_num_variants()-1 (ignored
 *            otherwise); each is compiled for one head dimension
 *   tile_t : query planes per middle run of a rolling workgroup,
 *            0 = automatic
 * Same pointer/layout/ownership/stream contract as na3d_fwd.  Returns
 * NA3D_ERR_CONFIG when the configuration cannot run these sizes (wrong head
 * dimension for the variant, window union or halo beyond its static limits,
 * or more concurrently active query planes than its slots).
 */
int na3d_fwd_config(const void* q, const void* k, const void* v, void* out,
                    int B, int T, int H, int W, int NH, int HD, int KT, int KH,
                    int KW, int family, int variant, int tile_t, void* stream);

/* na3d_plan for an explicit configuration (see na3d_fwd_config). */
int na3d_plan_config(int B, int T, int H, int W, int NH, int HD, int KT,
                     int KH, int KW, int family, int variant, int tile_t,
                     int* plan);

/*
 * na3d_fwd on strided tensors, so that q, k and v can be read in place as
 * views of a fused QKV projection output (the pages' launcher makes a
 * contiguous copy of v before its kernel, and that copy is inside their
 * measured time: same PR, Performance), or of a head-major buffer.
 *   strides: 20 element (not byte) strides, four groups of five, in the
 *            order q, k, v, out; each group gives the step between
 *            neighbouring elements along B, T, H, W and NH.  The HD axis is
 *            contiguous (stride 1) in every tensor.  Element (b,t,h,w,n,d)
 *            of tensor X is at X + b*sB + t*sT + h*sH + w*sW + n*sN + d.
 *            The array is read during the call only.
 * Contract (checked before any device call; NA3D_ERR_STRIDE otherwise):
 *   - every stride is >= 0 and a multiple of 8 (16-byte rows stay aligned);
 *   - k and v have the same H, W and NH strides (one staging offset serves
 *     both; their B and T strides may differ);
 *   - no two elements of out share an address (its strides, ordered by
 *     size, each step over the whole extent of the smaller ones).
 *   out must not overlap the address range of q, k or v (NA3D_ERR_OVERLAP);
 *   q, k and v may overlap each other freely (they are only read).
 * Everything else (pointers, sizes, alignment, ownership, stream, errors)
 * is as for na3d_fwd, which is this call with the contiguous strides
 *   sN = HD, sW = NH*HD, sH = W*NH*HD, sT = H*W*NH*HD, sB = T*H*W*NH*HD.
 */
int na3d_fwd_strided(const void* q, const void* k, const void* v, void* out,
                     int B, int T, int H, int W, int NH, int HD, int KT,
                     int KH, int KW, const long long* strides, void* stream);

/* The argument checks of na3d_fwd_strided alone, without touching a device. */
int na3d_check_args_strided(const void* q, const void* k, const void* v,
                            const void* out, int B, int T, int H, int W,
                            int NH, int HD, int KT, int KH, int KW,
                            const long long* strides);

/* na3d_fwd_config on strided tensors (contract of na3d_fwd_strided). */
int na3d_fwd_strided_config(const void* q, const void* k, const void* v,
                            void* out, int B, int T, int H, int W, int NH,
                            int HD, int KT, int KH, int KW,
                            const long long* strides, int family, int variant,
                            int tile_t, void* stream);

/*
 * Forward pass for the queries of a sub-box of the grid, with every window
 * placed in the whole grid: the pages' exact reference takes a W sub-slice of
 * q with the full k and v and global W coordinates for the window bounds
 * (aiter PR, Technical Details); this is the same in all three axes, and is what a
 * caller that splits one grid's queries (across launches or GPUs) needs.
 *   k, v    : the whole grid, (B, T, H, W, NH, HD)
 *   q, out  : the queries [t0, t0+Tq) x [h0, h0+Hq) x [w0, w0+Wq),
 *             (B, Tq, Hq, Wq, NH, HD); element (b, i, j, l, n, d) is the
 *             query at grid position (t0+i, h0+j, w0+l)
 *   box     : 6 ints {t0, h0, w0, Tq, Hq, Wq}; 0 <= t0, t0 + Tq <= T, Tq >= 1
 *             and likewise for H and W (NA3D_ERR_BOX otherwise)
 *   strides : as for na3d_fwd_strided (q and out with the box extents), or
 *             NULL for contiguous tensors of those shapes
 * out[b, i, j, l, n, :] equals what na3d_fwd writes at (b, t0+i, h0+j, w0+l,
 * n, :) for the whole grid.  Other arguments and the contract are those of
 * na3d_fwd_strided.
 */
int na3d_fwd_subgrid(const void* q, const void* k, const void* v, void* out,
                     int B, int T, int H, int W, int NH, int HD, int KT,
                     int KH, int KW, const int* box, const long long* strides,
                     void* stream);

/* The argument checks of na3d_fwd_subgrid alone, without touching a device. */
int na3d_check_args_subgrid(const void* q, const void* k, const void* v,
                            const void* out, int B, int T, int H, int W,
                            int NH, int HD, int KT, int KH, int KW,
                            const int* box, const long long* strides);

/* na3d_fwd_config for a query box (contract of na3d_fwd_subgrid). */
int na3d_fwd_subgrid_config(const void* q, const void* k, const void* v,
                            void* out, int B, int T, int H, int W, int NH,
                            int HD, int KT, int KH, int KW, const int* box,
                            const long long* strides, int family, int variant,
                            int tile_t, void* stream);

/*
 * One tile of a batch: q, k, v and out are contiguous bf16 (B, T, H, W, NH,
 * HD) device tensors of this tile, with the NH, HD and window of the batch.
 */
typedef struct na3d_tile {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  int B, T, H, W;
} na3d_tile;

/*
 * na3d_fwd on many independent grids at once: the video decoder runs NA3D on
 * every tile of a tile grid, and its edge tiles are narrow (xDiT PR 773 page
 * "LTX-2.5 optimization: integrate faster AITER NA3D flash attention for
 * diffusion decoder", Summary; xDiT PR 759 page, Changes item 1: each tile's
 * decode is independent of the others).  out of every tile is bitwise what
 * na3d_fwd_config writes for that tile alone with the launch's rolling
 * instantiation (see na3d_plan_batch), and within rounding of na3d_fwd.
 *   tiles : host array of n descriptors, read during the call only
 *   n     : >= 0 (0 returns NA3D_OK without touching the device)
 *   NH, HD, KT, KH, KW : shared by every tile, as for na3d_fwd (the window
 *           must fit each tile's grid)
 * Tiles that the rolling instantiation chosen for the largest tile can run
 * share kernel launches, up to 16 tiles each, in the given order; any other
 * tile is run by a launch of its own.  All launches are enqueued on
 * `stream` in order.  Each tile must pass na3d_fwd's checks, and no tile's
 * out may overlap any tensor of another tile (NA3D_ERR_OVERLAP); inputs may
 * be shared between tiles.  Errors are detected before any launch.
 */
int na3d_fwd_batch(const na3d_tile* tiles, int n, int NH, int HD, int KT,
                   int KH, int KW, void* stream);

/* The argument checks of na3d_fwd_batch alone, without touching a device. */
int na3d_check_args_batch(const na3d_tile* tiles, int n, int NH, int HD,
                          int KT, int KH, int KW);

/*
 * How na3d_fwd_batch would run a batch (only the tiles' sizes are read):
 * plan[0] = kernel launches, plan[1] = rolling instantiation of the shared
 * launches (-1 if none), plan[2] = tiles in shared launches, plan[3] =
 * workgroups of the first shared launch.  `plan` must hold 4 ints.
 */
int na3d_plan_batch(const na3d_tile* tiles, int n, int NH, int HD, int KT,
                    int KH, int KW, int* plan);

/*
 * RMSNorm over the last axis, bf16 in and out: the transformer block norms
 * of the xDiT PR "LTX-2.5 optimizations: add parallel VAE decoding and AITER
 * RMSNorm" (Changes, item 2; a drop-in for a norm that normalises in float32,
 * with or without an elementwise weight).  For every row r and column j,
 *   y[r, j] = x[r, j] * w[j] / sqrt( (1/dim) * sum_k x[r, k]^2 + eps )
 * with w = 1 when weight is NULL.  The sum of squares, the scale and both
 * products are taken in fp32; y is rounded to bf16 once (round to nearest
 * even).  Squares are summed in fp32, so a row whose sum of squares exceeds
 * the fp32 range (|x| beyond about 1.8e19 / sqrt(dim)) normalises to zero.
 *   x      : device pointer, bf16, (rows, dim) contiguous (row stride dim)
 *   weight : device pointer, bf16, (dim,), or NULL for a unit weight
 *   y      : device pointer, bf16, (rows, dim) contiguous; fully overwritten.
 *            y == x (in place) is allowed; any other overlap of y with x, and
 *            any overlap of y with weight, is NA3D_ERR_OVERLAP
 *   rows   : >= 0; with 0 rows nothing is read or written, the call returns
 *            NA3D_OK after the dim and eps checks, and the pointers may be NULL
 *   dim    : a multiple of 8 in [8, 8192] (NA3D_ERR_SHAPE otherwise)
 *   eps    : finite and >= 0 (NA3D_ERR_VALUE otherwise); with eps = 0 an
 *            all-zero row gives NaN, as the formula does
 *   stream : hipStream_t to enqueue on, or NULL for the default stream
 * x, weight and y must be 16-byte aligned (NA3D_ERR_ALIGN).  Ownership,
 * asynchrony and error reporting are as for na3d_fwd.
 */
int na3d_rms_norm(const void* x, const void* weight, void* y, int rows, int dim,
                  float eps, void* stream);

/* The argument checks of na3d_rms_norm alone, without touching a device. */
int na3d_check_args_rms_norm(const void* x, const void* weight, const void* y,
                             int rows, int dim, float eps);

/*
 * na3d_rms_norm with an explicit grid of `workgroups` workgroups of w waves,
 * w = 8 for dim <= 4096 and 4 above (each wave normalises rows wave,
 * wave + w*workgroups, ...), for tuning sweeps and for testing the multi-row
 * path; 0 = automatic, negative or above 2^24 = NA3D_ERR_CONFIG.
 */
int na3d_rms_norm_config(const void* x, const void* weight, void* y, int rows,
                         int dim, float eps, int workgroups, void* stream);

/* Number of rolling-family instantiations compiled into the library. */
int na3d_num_variants(void);

/*
 * The compile-time shape of rolling instantiation `variant` (for tuning and
 * tests that pick configurations through na3d_fwd_config):
 *   info: host array of 10 ints, written on success: [0] head dim, [1] QH
 *         and [2] QW, the query block on one plane (16 / (QH*QW) consecutive
 *         query planes per block, 1 or 2), [3] WH block rows and [4] WT
 *         query-plane phases per workgroup (WH*WT computing waves of 64
 *         lanes; some instantiations add waves that only stage K/V, which
 *         the thread count of na3d_plan_config includes), [5]
 *         query-plane slots per wave, [6] 16-key tiles per softmax group, [7]
 *         groups, [8] staged plane buffers (1 or 2), [9] waves per SIMD the
 *         register allocation is capped for (0 = no cap).
 * Returns NA3D_OK, NA3D_ERR_NULL (info is NULL) or NA3D_ERR_CONFIG (variant
 * outside 0 .. na3d_num_variants()-1).  No device calls.
 */
int na3d_variant_info(int variant, int* info);

/* Library ABI version (incremented on incompatible changes). */
int na3d_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NA3D_H_ */
