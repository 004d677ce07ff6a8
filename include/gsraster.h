/*
 * gsraster.h — C ABI of libgsraster.so, the MI355X (gfx950) differentiable
 * tile rasterizer of 3D Gaussian Splatting.
 *
 * The five stages follow the pipeline the gsplat guide (lmnt.cn/news/262699)
 * describes in §2.1 — transform each Gaussian by (R, t, scale, rotation),
 * project it to depth and screen space, then alpha-blend it differentiably —
 * with the blending backward callable on its own (gsplat guide §2.2).  The
 * pages sum per-Gaussian gradients with atomics (3DGS deployment guide
 * (hmyw.cn/news/140031) §2.1; Moore Threads MUSA article
 * (qwbw.cn/news/278220) §2.1); here every tile instance gets its own
 * gradient slot instead, added up in a fixed order, so the backward is
 * deterministic.  The primitive is a position, a covariance
 * built from scale and rotation (MUSA article §3.3), an opacity and SH colour
 * coefficients (deployment guide §1).  Formulas below the stage level are the
 * textbook EWA-splatting reading; the pages print none.
 *
 * Conventions shared by every entry point
 *   - Device pointers unless marked HOST.  Every buffer is owned by the
 *     caller; the library allocates nothing and keeps no state between calls
 *     (calls on different streams may run concurrently on distinct buffers),
 *     except for the scratch array of gs_bin_and_sort_noalloc, described
 *     there.
 *   - Per-Gaussian arrays are fp32/int32 structure-of-arrays planes with a
 *     leading dimension ld >= N: plane p of array X starts at X + p*ld.
 *       means [3][ld] (world x,y,z)   scales [3][ld] (activated, > 0)
 *       quats [4][ld] (w,x,y,z, any non-zero norm; normalised inside)
 *       opacities [ld] (activated, in [0,1])
 *       sh [K*3][ld], K = (sh_degree+1)^2, plane k*3+c = coefficient k of
 *       colour channel c, coefficients ordered (l, m=-l..l), real SH with the
 *       Condon-Shortley phase; colour = max(0, sh_offset + sum_k Y_k(d) c_k)
 *       with d the unit vector from the camera centre to the mean.
 *     (Opacity = sigmoid(logit), scale = exp(log-scale) and the quaternion's
 *     w-first order are those of the gsplat guide §3.3; the activations stay
 *     with the caller, so gradients are with respect to activated values.)
 *   - Between stages, projected Gaussians and their gradients travel as the
 *     same [p][ld] planes (gsplat guide §3.3 passes its Gaussians to the
 *     rasterizer as such arrays; §2.2 makes the backward callable on its
 *     own):
 *       means2d [2][ld] (u, v: pixel coordinates of the mean),
 *       conics [3][ld] (A, B, C of q = A dx^2 + 2B dx dy + C dy^2, the
 *       inverse of the dilated 2D covariance),
 *       chol [3][ld] (L11, L21, L22: the conic's lower Cholesky factor,
 *       conic = L L^T, L11 = sqrt(A), L21 = B / L11, L22 = 1 / sqrt(c) with
 *       c the dilated 2D covariance's yy entry),
 *       depths [ld] (camera z), radii [ld] (int32, 0 = culled),
 *       colors [3][ld] (SH colour), tiles_touched [ld] (uint32);
 *     and backwards dL_dmeans2d [2][ld], dL_dconics [3][ld] (A, B, C as
 *     independent scalars), dL_dopacities [ld], dL_dcolors [3][ld].
 *     The compositing calls evaluate q as the completed square
 *     (L11 dx + L21 dy)^2 + (L22 dy)^2, which is why they take chol beside
 *     conics: the expanded form cancels for needle-like splats (terms up to
 *     1e5 times q), and L22 cannot be rebuilt from the conic in fp32 without
 *     the same cancellation.  Internally each compositing call first stages
 *     every visible row into a 64-byte record (one cache line per tile
 *     instance) in the caller's workspace; the backward may reuse the
 *     forward's records ("staged").
 *   - Images are row-major [H][W] (colour [H][W][3]); pixel (px,py) has its
 *     centre at (px+0.5, py+0.5); tiles are 16x16, T = ceil(W/16)*ceil(H/16),
 *     tile id = ty*ceil(W/16) + tx.
 *   - stream is a hipStream_t (NULL = the default stream).  Every call is
 *     asynchronous on it except the binning calls that return M to the host
 *     (gs_bin_and_sort and its packed, batched and no-allocation forms),
 *     which read it back once.
 *   - Errors: invalid arguments are rejected on the host before anything is
 *     launched (GS_ERR_INVALID_ARGUMENT); a failed launch returns GS_ERR_HIP.
 *     gs_last_error() gives a thread-local message.  Per-Gaussian pointers
 *     may be NULL when N = 0; tile_ranges and ids must come from
 *     gs_bin_and_sort for the same Gaussians and image.  Non-finite or degenerate
 *     Gaussians are not errors: they are culled (radius 0, no tiles, zero
 *     gradients).  N = 0 and zero instances are valid (background image).
 */
#ifndef GSRASTER_H
#define GSRASTER_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define GS_API __attribute__((visibility("default")))
#else
#define GS_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GS_OK = 0,
  GS_ERR_INVALID_ARGUMENT = 1,
  GS_ERR_CAPACITY = 2,
  GS_ERR_HIP = 3
} gs_status;

/* Pinhole camera (HOST struct, passed by pointer).  R, t map world to camera
 * coordinates, t_cam = R x + t, with OpenCV axes (+x right, +y down, +z
 * forward) as in the world-to-camera view matrix and [fx, fy, cx, cy]
 * intrinsics of the gsplat guide §3.3. */
typedef struct {
  float R[9]; /* row-major */
  float t[3];
  float fx, fy, cx, cy;
  int32_t width, height;
  float near_plane, far_plane; /* Gaussians with depth outside (near, far) are culled */
} gs_camera;

/* Constants of the method (HOST struct).  gs_default_settings() returns
 * eps2d 0.3 (screen-space dilation added to the 2D covariance diagonal),
 * alpha_min 1/255 (pairs below are skipped), alpha_max 0.99 (alpha clamp),
 * T_min 1e-4 (a pixel stops before the Gaussian that would take its
 * transmittance below this), fov_clamp 1.3 (the EWA Jacobian is evaluated
 * with x/z, y/z clamped to 1.3 times the half field of view), sh_offset 0.5. */
typedef struct {
  float eps2d, alpha_min, alpha_max, T_min, fov_clamp, sh_offset;
} gs_settings;

GS_API gs_settings gs_default_settings(void);
GS_API const char* gs_status_string(gs_status s);
GS_API const char* gs_last_error(void);
GS_API int32_t gs_num_tiles(int32_t width, int32_t height);

/* Stage 1 — projection (gsplat guide §2.1, its first two steps: the 3D
 * transform, then depth and screen-space projection; covariance from scale
 * and rotation, MUSA article §3.3).  Per Gaussian: t = R mean + t; cull
 * outside (near, far) or non-finite; Sigma = R(q) S S^T R(q)^T; 2D covariance
 * J W Sigma W^T J^T plus eps2d on the diagonal, with J the pinhole Jacobian
 * (culled unless positive definite); conic = its inverse and its Cholesky
 * factor; radius = ceil(3 sqrt(lambda_max)); pixel mean; number of 16x16
 * tiles the square [u-r,u+r]x[v-r,v+r] touches; SH colour.
 * Outputs ([p][ld] planes, see the conventions above): means2d, conics,
 * chol, depths, radii, colors, tiles_touched.  Culled Gaussians get radius
 * 0, tiles 0 and zeros in the other planes.  The geometric outputs are
 * computed in IEEE fp32 in a fixed operation order without contraction, so
 * they are reproducible bit for bit. */
GS_API gs_status gs_project_fwd(int64_t N, int64_t ld, int32_t sh_degree,
                         const float* means, const float* scales, const float* quats,
                         const float* sh, const gs_camera* cam, const gs_settings* settings,
                         float* means2d, float* conics, float* chol, float* depths,
                         int32_t* radii, float* colors, uint32_t* tiles_touched, void* stream);

/* Workspace needed by gs_bin_and_sort for N Gaussians and up to `capacity`
 * tile instances on a width x height image. */
GS_API size_t gs_bin_and_sort_workspace_size(int64_t N, uint64_t capacity, int32_t width,
                                      int32_t height);

/* Stages 2-3 — binning and sort.  offsets = exclusive scan of tiles_touched
 * (Gaussian order); M = total.  *num_instances (HOST) receives M; this is the
 * one device-to-host read of a frame (page-locked host memory there saves a
 * staging copy).  If M > capacity the call returns
 * GS_ERR_CAPACITY with offsets valid and keys untouched: grow the buffers and
 * call again.  Otherwise every visible Gaussian i is duplicated once per
 * touched tile (row-major within its rect) at slot offsets[i] + k with key
 * (tile_id << 32) | bits(depth_i) and value i; the (key, value) pairs are
 * radix-sorted stably by key (equal keys keep ascending Gaussian index) into
 * keys [capacity] / ids [capacity]; tile_ranges [T][2] receives each tile's
 * [start, end) in the sorted list ((0,0) for empty tiles).  M must be below
 * 2^30.  workspace: device memory of at least
 * gs_bin_and_sort_workspace_size() bytes, 256-byte aligned. */
GS_API gs_status gs_bin_and_sort(int64_t N, int64_t ld, const float* means2d, const int32_t* radii,
                          const float* depths, const uint32_t* tiles_touched, int32_t width,
                          int32_t height, uint32_t* offsets, uint64_t capacity,
                          uint64_t* num_instances, uint64_t* keys, uint32_t* ids,
                          uint32_t* tile_ranges, void* workspace, size_t workspace_bytes,
                          void* stream);

/* gs_bin_and_sort without the read-back: the instance count stays on the
 * device, so the call never waits for the GPU and a whole frame can be
 * captured into a HIP graph.  counts (DEVICE uint64[2]) receives M and an
 * overflow flag: with M > capacity the flag is 1 and the list is left
 * empty (every tile range (0, 0), so the compositing yields the
 * background; the backward stays within its buffers but its gradients are
 * not meaningful); the caller reads counts when convenient, grows the
 * buffers and runs the frame again.  Otherwise as gs_bin_and_sort, with the same
 * workspace size.  The kernels are sized for capacity, not M. */
GS_API gs_status gs_bin_and_sort_device(int64_t N, int64_t ld, const float* means2d,
                                        const int32_t* radii, const float* depths,
                                        const uint32_t* tiles_touched, int32_t width,
                                        int32_t height, uint32_t* offsets, uint64_t capacity,
                                        uint64_t* counts, uint64_t* keys, uint32_t* ids,
                                        uint32_t* tile_ranges, void* workspace,
                                        size_t workspace_bytes, void* stream);

/* gs_bin_and_sort for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and results, with the sort's scratch in
 * a 64 MiB array inside the library instead of a workspace argument.  The
 * caller still passes every input and output.  Limit: the
 * gs_bin_and_sort_workspace_size() of (N, capacity, width, height) must be
 * at most 64 MiB (capacity up to about 4.4 million instances for a million
 * Gaussians at 1920x1080); larger requests return GS_ERR_INVALID_ARGUMENT
 * before anything runs.  The call allocates nothing: each device holds its
 * own copy of the array from the library's first use on it until the
 * process ends.  Every call on one device uses that device's array, so calls
 * that overlap on one device (other streams, other host threads) race; the
 * array keeps the last call's contents, and each call clears what must start
 * at zero itself.  Otherwise as gs_bin_and_sort, including the one
 * device-to-host read of M and the GS_ERR_CAPACITY protocol. */
GS_API gs_status gs_bin_and_sort_noalloc(int64_t N, int64_t ld, const float* means2d,
                                         const int32_t* radii, const float* depths,
                                         const uint32_t* tiles_touched, int32_t width,
                                         int32_t height, uint32_t* offsets, uint64_t capacity,
                                         uint64_t* num_instances, uint64_t* keys, uint32_t* ids,
                                         uint32_t* tile_ranges, void* stream);

/* Schedule of the compositing kernels (no step of the method: a launch
 * order).  For each of num_cams cameras, tile_order (DEVICE uint32
 * [num_cams * T]) receives that camera's tile indices 0 .. T-1 ordered by
 * decreasing list length in tile_ranges (lengths bucketed about 12% apart;
 * the order within a bucket is not fixed).  Passed to the gs_rasterize_*
 * calls, it makes their workgroups take the longest tiles first, so that a
 * few long lists do not run on their own at the end of the launch.  Their
 * results do not depend on it.  One workgroup per camera; it reads only
 * tile_ranges, so it can run in a captured graph. */
GS_API gs_status gs_tile_order(int32_t num_cams, int32_t width, int32_t height,
                               const uint32_t* tile_ranges, uint32_t* tile_order, void* stream);

/* Workspace of the compositing calls: the staged 64-byte record of each of
 * `rows` splat rows (rows = N for one camera, num_cams * ld for a batch),
 * 256-byte aligned. */
GS_API size_t gs_rasterize_workspace_size(int64_t rows);

/* Stage 4 — front-to-back alpha compositing per 16x16 tile (gsplat guide
 * §2.1, its third, differentiable blending step).  Reads the projection's
 * planes means2d, conics, chol, colors, radii and the caller's opacities
 * [ld] (activated, in [0,1]); stages the visible rows into workspace
 * (gs_rasterize_workspace_size(N) bytes), then per pixel, over its tile's
 * sorted list: q at (px+0.5-u, py+0.5-v) as the completed square of chol;
 * alpha = min(alpha_max, o exp(-q/2)); skip alpha < alpha_min; stop (without
 * blending) when T (1-alpha) < T_min; else C += colour alpha T, T *= 1-alpha.
 * Outputs: image [H][W][3] = C + T bg; final_T [H][W]; last_idx [H][W] =
 * number of the tile's list entries up to and including the last blended one
 * (0 if none); out_depth [H][W] = sum alpha T depth and out_alpha [H][W] =
 * 1 - T when non-NULL (out_depth needs depths [ld]; otherwise depths may be
 * NULL).  background: HOST float[3].
 * tile_order: NULL (a fixed XCD-aware order), or the schedule
 * gs_tile_order wrote for these tile_ranges; it decides which workgroup
 * takes which tile, never the outputs.  (With other contents, entries that
 * are no tile index are skipped and tiles left out keep their old outputs.)
 * The same argument of the other gs_rasterize_* calls means the same.
 * counters: NULL, or device uint64[4] that the call adds work counts to:
 * [0] pixel-splat pairs evaluated by the kernel, [1] pairs blended, [2] pairs
 * the plain per-pixel method evaluates (per pixel, its tile's entries up to
 * the one that stops it), [3] pairs the plain tile loop evaluates (256 x a
 * tile's entries up to the last of its pixels' stops).  Counting uses a
 * separate kernel variant. */
GS_API gs_status gs_rasterize_fwd(int64_t N, int64_t ld, int32_t width, int32_t height,
                                  const uint32_t* tile_ranges, const uint32_t* tile_order,
                                  const uint32_t* ids, const float* means2d,
                                  const float* conics, const float* chol,
                                  const float* opacities, const float* colors,
                                  const int32_t* radii, const float* depths,
                                  const float* background, const gs_settings* settings,
                                  float* image, float* final_T, uint32_t* last_idx,
                                  float* out_depth, float* out_alpha, void* workspace,
                                  size_t workspace_bytes, uint64_t* counters, void* stream);

/* gs_rasterize_fwd with the image loss gradient fused in: while each
 * pixel's colour is in registers, dL_dimage [H][W][3] receives the gradient
 * of the sum-reduced loss against target [H][W][3] (kind 0: L2, 2 (x - y);
 * kind 1: L1, sign(x - y) with sign(0) = 0), the same values
 * gs_image_loss_grad writes, and *loss (a device float; NULL to skip) the
 * loss value (its summation order across tiles is not fixed).  The image
 * is not read back.  dL_dimage must not alias image or target. */
GS_API gs_status gs_rasterize_fwd_loss(int64_t N, int64_t ld, int32_t width, int32_t height,
                                       const uint32_t* tile_ranges,
                                       const uint32_t* tile_order, const uint32_t* ids,
                                       const float* means2d, const float* conics,
                                       const float* chol, const float* opacities,
                                       const float* colors, const int32_t* radii,
                                       const float* depths, const float* background,
                                       const gs_settings* settings, int32_t kind,
                                       const float* target, float* image, float* final_T,
                                       uint32_t* last_idx, float* out_depth, float* out_alpha,
                                       float* dL_dimage, float* loss, void* workspace,
                                       size_t workspace_bytes, uint64_t* counters,
                                       void* stream);

/* Stage 5a — compositing backward (gsplat guide §2.2).  The same planes as
 * the forward, plus offsets and tiles_touched of the binning and the
 * forward's final_T and last_idx.  staged: 1 when workspace still holds
 * what gs_rasterize_fwd (or _fwd_loss) staged from these same planes
 * (nothing is staged again), 0 to stage here.  Walks each pixel's blended
 * list back to front from last_idx, recovering T by division and
 * accumulating the colour behind, and sums per Gaussian the gradients of
 * the loss with respect to u, v, the conic (A, B, C as scalars of
 * q = A dx^2 + 2B dx dy + C dy^2), opacity and colour, given dL_dimage
 * [H][W][3].  Each tile writes its sums for each of its Gaussians with a
 * plain store into that instance's slot of partials (offsets[i] + k for the
 * k-th tile, row-major, of Gaussian i's rect; partials [capacity][12] floats,
 * 64-byte aligned, capacity >= num_instances); a segmented reduction then
 * adds each Gaussian's slots, in slot order, into dL_dmeans2d [2][ld],
 * dL_dconics [3][ld], dL_dopacities [ld], dL_dcolors [3][ld].  There are no
 * atomics, so the result is bit-for-bit reproducible.  accumulate = 0
 * overwrites every plane (zeros for Gaussians without tiles); 1 adds to
 * every plane (Gaussians without tiles are left alone); 2 adds to the
 * gradients that are final after this stage (dL_dopacities and the
 * absolute sums) and overwrites the per-camera ones (dL_dmeans2d,
 * dL_dconics, dL_dcolors), which is how a loop over cameras sums them: the
 * projection backward of each camera then reads that camera's planes and
 * adds its own terms with its own accumulate.
 * Pairs whose alpha was clamped at alpha_max carry no opacity/conic/mean
 * gradient.  The opacity gradient comes from this stage only (opacity enters
 * only compositing).
 * dL_dmeans2d_abs: NULL, or [2][ld] receiving (or, with accumulate, adding)
 * the sums over pixels of |dL/du| and |dL/dv| of each pixel's own
 * contribution: the absolute-gradient statistic that densification
 * thresholds (gsplat guide §4.1 trains with it).  NULL skips that work.
 * counters: NULL, or device uint64[4]: [0] pairs evaluated, [1] pairs with a
 * gradient, [2] pairs the plain tile loop walks (256 x a tile's entries up
 * to its pixels' last blended one), [3] wavefront reductions. */
GS_API gs_status gs_rasterize_bwd(int64_t N, int64_t ld, int32_t width, int32_t height,
                                  const uint32_t* tile_ranges, const uint32_t* tile_order,
                                  const uint32_t* ids, const float* means2d,
                                  const float* conics, const float* chol,
                                  const float* opacities, const float* colors,
                                  const int32_t* radii, const uint32_t* offsets,
                                  const uint32_t* tiles_touched, uint64_t num_instances,
                                  const float* background, const gs_settings* settings,
                                  const float* final_T, const uint32_t* last_idx,
                                  const float* dL_dimage, void* workspace,
                                  size_t workspace_bytes, int32_t staged, float* partials,
                                  uint64_t partials_capacity, float* dL_dmeans2d,
                                  float* dL_dconics, float* dL_dopacities, float* dL_dcolors,
                                  float* dL_dmeans2d_abs, int32_t accumulate,
                                  uint64_t* counters, void* stream);

/* Stage 5b — projection backward: chain rule from dL_dmeans2d [2][ld],
 * dL_dconics [3][ld] and dL_dcolors [3][ld] to means [3][ld], scales [3][ld],
 * quats [4][ld] (through the normalisation) and sh [K*3][ld].  The geometry
 * is recomputed from the parameters in fp64; visibility comes from radii
 * (the forward's decisions are kept: the fov clamp and the colour clamp are
 * re-evaluated from the same fp32 inputs).  accumulate = 0 overwrites
 * (zeros for culled Gaussians); 1 adds, which sums cameras. */
GS_API gs_status gs_project_bwd(int64_t N, int64_t ld, int32_t sh_degree, const float* means,
                                const float* scales, const float* quats, const float* sh,
                                const gs_camera* cam, const gs_settings* settings,
                                const int32_t* radii, const float* dL_dmeans2d,
                                const float* dL_dconics, const float* dL_dcolors,
                                float* dL_dmeans, float* dL_dscales, float* dL_dquats,
                                float* dL_dsh, int32_t accumulate, void* stream);

/* Batched cameras: one launch per stage for num_cams cameras (1 .. 8) of one
 * image size, the Gaussians read once.  Row c * ld + i of the per-camera
 * outputs is Gaussian i seen by camera c: each per-camera plane set is a
 * block [c][P][ld] (radii, depths, tiles_touched [c][ld]), and tile c * T + t
 * is tile t of camera c, so a batch is one list of num_cams * ld rows over
 * num_cams * T tiles and its results per camera equal those of the
 * single-camera calls (keys carry the tile number c * T + t; ids the row
 * c * ld + i).
 *
 * gs_project_fwd_batched: gs_project_fwd for every camera of cams (HOST
 * array); outputs means2d [c][2][ld], conics [c][3][ld], chol [c][3][ld],
 * depths [c][ld], radii [c][ld], colors [c][3][ld], tiles_touched [c][ld].
 * Rows N .. ld-1 of each camera get radius 0 and no tiles, so the outputs
 * are valid input to gs_bin_and_sort_batched.  num_cams * ld < 2^31. */
GS_API gs_status gs_project_fwd_batched(int32_t num_cams, const gs_camera* cams, int64_t N,
                                        int64_t ld, int32_t sh_degree, const float* means,
                                        const float* scales, const float* quats,
                                        const float* sh, const gs_settings* settings,
                                        float* means2d, float* conics, float* chol,
                                        float* depths, int32_t* radii, float* colors,
                                        uint32_t* tiles_touched, void* stream);

/* gs_bin_and_sort_batched: gs_bin_and_sort over the num_cams * ld rows of a
 * batch (offsets [num_cams * ld]; tile_ranges [num_cams * T][2]).  The
 * sorted list holds camera 0's tiles first.  Capacity protocol and errors as
 * gs_bin_and_sort; workspace of gs_bin_and_sort_batched_workspace_size()
 * bytes (0 for an invalid num_cams). */
GS_API size_t gs_bin_and_sort_batched_workspace_size(int32_t num_cams, int64_t ld,
                                                     uint64_t capacity, int32_t width,
                                                     int32_t height);
GS_API gs_status gs_bin_and_sort_batched(int32_t num_cams, int64_t ld, const float* means2d,
                                         const int32_t* radii, const float* depths,
                                         const uint32_t* tiles_touched, int32_t width,
                                         int32_t height, uint32_t* offsets, uint64_t capacity,
                                         uint64_t* num_instances, uint64_t* keys, uint32_t* ids,
                                         uint32_t* tile_ranges, void* workspace,
                                         size_t workspace_bytes, void* stream);

/* gs_rasterize_fwd_batched: gs_rasterize_fwd for every camera of a batch
 * (planes [c][P][ld] as gs_project_fwd_batched wrote them, opacities [ld]
 * shared by the cameras; workspace of gs_rasterize_workspace_size(num_cams *
 * ld) bytes); image [c][H][W][3], final_T, last_idx, out_depth, out_alpha
 * [c][H][W] (depths [c][ld]).  last_idx counts entries of the tile's own
 * list, as in the single-camera call. */
GS_API gs_status gs_rasterize_fwd_batched(int32_t num_cams, int64_t ld, int32_t width,
                                          int32_t height, const uint32_t* tile_ranges,
                                          const uint32_t* tile_order, const uint32_t* ids,
                                          const float* means2d, const float* conics,
                                          const float* chol, const float* opacities,
                                          const float* colors, const int32_t* radii,
                                          const float* depths, const float* background,
                                          const gs_settings* settings, float* image,
                                          float* final_T, uint32_t* last_idx, float* out_depth,
                                          float* out_alpha, void* workspace,
                                          size_t workspace_bytes, uint64_t* counters,
                                          void* stream);

/* gs_rasterize_fwd_loss_batched: gs_rasterize_fwd_loss for every camera of
 * a batch (layouts as gs_rasterize_fwd_batched): target and dL_dimage are
 * [c][H][W][3], each camera's pixels against its own target, and *loss
 * (NULL to skip) the sum over all cameras' pixels.  The values equal
 * gs_rasterize_fwd_batched followed by gs_image_loss_grad over the batch's
 * images. */
GS_API gs_status gs_rasterize_fwd_loss_batched(int32_t num_cams, int64_t ld, int32_t width,
                                               int32_t height, const uint32_t* tile_ranges,
                                               const uint32_t* tile_order, const uint32_t* ids,
                                               const float* means2d, const float* conics,
                                               const float* chol, const float* opacities,
                                               const float* colors, const int32_t* radii,
                                               const float* depths, const float* background,
                                               const gs_settings* settings, int32_t kind,
                                               const float* target, float* image,
                                               float* final_T, uint32_t* last_idx,
                                               float* out_depth, float* out_alpha,
                                               float* dL_dimage, float* loss, void* workspace,
                                               size_t workspace_bytes, uint64_t* counters,
                                               void* stream);

/* gs_rasterize_bwd_batched: gs_rasterize_bwd for every camera of a batch
 * (final_T, last_idx [c][H][W], dL_dimage [c][H][W][3]); the 2D gradient
 * planes are per camera: dL_dmeans2d [c][2][ld], dL_dconics [c][3][ld],
 * dL_dopacities [c][ld], dL_dcolors [c][3][ld] (dL_dmeans2d_abs [c][2][ld]
 * or NULL).  gs_project_bwd_batched sums them over the cameras. */
GS_API gs_status gs_rasterize_bwd_batched(int32_t num_cams, int64_t ld, int32_t width,
                                          int32_t height, const uint32_t* tile_ranges,
                                          const uint32_t* tile_order, const uint32_t* ids,
                                          const float* means2d, const float* conics,
                                          const float* chol, const float* opacities,
                                          const float* colors, const int32_t* radii,
                                          const uint32_t* offsets, const uint32_t* tiles_touched,
                                          uint64_t num_instances, const float* background,
                                          const gs_settings* settings, const float* final_T,
                                          const uint32_t* last_idx, const float* dL_dimage,
                                          void* workspace, size_t workspace_bytes,
                                          int32_t staged, float* partials,
                                          uint64_t partials_capacity, float* dL_dmeans2d,
                                          float* dL_dconics, float* dL_dopacities,
                                          float* dL_dcolors, float* dL_dmeans2d_abs,
                                          int32_t accumulate, uint64_t* counters,
                                          void* stream);

/* gs_project_bwd_batched: gs_project_bwd summed over the cameras of a batch
 * (radii [c][ld], 2D gradient planes [c][P][ld]): each Gaussian's
 * parameters are read once and the cameras that see it add their chain-rule
 * terms in camera order, as num_cams single-camera calls with accumulate
 * would.  With dL_dopacities_cams [c][ld] and dL_dopacities [ld] (both or
 * neither), the per-camera opacity gradients are summed the same way, so a
 * batch's opacity gradient comes out beside the others.  accumulate = 0:
 * Gaussians no camera sees get zeros. */
GS_API gs_status gs_project_bwd_batched(int32_t num_cams, const gs_camera* cams, int64_t N,
                                        int64_t ld, int32_t sh_degree, const float* means,
                                        const float* scales, const float* quats,
                                        const float* sh, const gs_settings* settings,
                                        const int32_t* radii, const float* dL_dmeans2d,
                                        const float* dL_dconics, const float* dL_dcolors,
                                        const float* dL_dopacities_cams, float* dL_dmeans,
                                        float* dL_dscales, float* dL_dquats,
                                        float* dL_dopacities, float* dL_dsh,
                                        int32_t accumulate, void* stream);

/* Packed mode (the gsplat guide §4.1 trains with its packed and sparse
 * gradient switches on: only the Gaussians that reach the image take part
 * after the projection, and only they receive gradients).  The visible set
 * is the list of Gaussians with tiles_touched > 0, in ascending index order;
 * V is its length.  The three calls below replace gs_bin_and_sort,
 * gs_rasterize_bwd and gs_project_bwd of a frame; projection, compositing and
 * the loss are the same calls as in the dense path.
 *
 * gs_bin_and_sort_packed: gs_bin_and_sort, and in the same pass the visible
 * list vis_ids [N] (its first V entries are written).  counts (HOST
 * uint64[2]) receives M then V in the call's one device-to-host read.
 * Capacity handling and errors as gs_bin_and_sort (with GS_ERR_CAPACITY both
 * counts and vis_ids are valid). */
GS_API gs_status gs_bin_and_sort_packed(int64_t N, int64_t ld, const float* means2d,
                                        const int32_t* radii, const float* depths,
                                        const uint32_t* tiles_touched, int32_t width,
                                        int32_t height, uint32_t* offsets, uint64_t capacity,
                                        uint64_t* counts, uint64_t* keys, uint32_t* ids,
                                        uint32_t* tile_ranges, uint32_t* vis_ids,
                                        void* workspace, size_t workspace_bytes, void* stream);

/* gs_rasterize_bwd_packed: gs_rasterize_bwd with the segmented reduction run
 * over the visible list: row r of the 2D gradient planes (leading dimension
 * ldv >= num_visible: dL_dmeans2d [2][ldv], dL_dconics [3][ldv],
 * dL_dopacities [ldv], dL_dcolors [3][ldv], dL_dmeans2d_abs [2][ldv] or
 * NULL) receives the gradients of Gaussian vis_ids[r].  Nothing is written
 * for Gaussians off the list.  vis_ids / num_visible as
 * gs_bin_and_sort_packed returned them for the same frame (entries must be
 * < N). */
GS_API gs_status gs_rasterize_bwd_packed(int64_t N, int64_t ld, int32_t width, int32_t height,
                                         const uint32_t* tile_ranges,
                                         const uint32_t* tile_order, const uint32_t* ids,
                                         const float* means2d, const float* conics,
                                         const float* chol, const float* opacities,
                                         const float* colors, const int32_t* radii,
                                         const uint32_t* offsets, const uint32_t* tiles_touched,
                                         uint64_t num_instances, const uint32_t* vis_ids,
                                         int64_t num_visible, int64_t ldv,
                                         const float* background, const gs_settings* settings,
                                         const float* final_T, const uint32_t* last_idx,
                                         const float* dL_dimage, void* workspace,
                                         size_t workspace_bytes, int32_t staged,
                                         float* partials, uint64_t partials_capacity,
                                         float* dL_dmeans2d, float* dL_dconics,
                                         float* dL_dopacities, float* dL_dcolors,
                                         float* dL_dmeans2d_abs, int32_t accumulate,
                                         uint64_t* counters, void* stream);

/* gs_project_bwd_packed: gs_project_bwd for the num_visible Gaussians of
 * vis_ids only, in sparse form: the parameters are read at vis_ids[r]
 * (planes [p][ld] of the N Gaussians), the 2D gradients at row r of the
 * packed 2D planes, and the gradients go to column r of the packed output
 * planes (dL_dmeans [3][ldv], dL_dscales [3][ldv], dL_dquats [4][ldv],
 * dL_dsh [K*3][ldv], ldv >= num_visible; the packed opacity gradients are
 * those gs_rasterize_bwd_packed wrote).  Together with vis_ids they are the
 * gradient as (index, value) rows; Gaussians off the list have zero
 * gradient and nothing is written for them.  accumulate = 1 adds into the
 * packed rows (the same list only). */
GS_API gs_status gs_project_bwd_packed(int64_t num_visible, const uint32_t* vis_ids, int64_t N,
                                       int64_t ld, int64_t ldv, int32_t sh_degree,
                                       const float* means, const float* scales,
                                       const float* quats, const float* sh,
                                       const gs_camera* cam, const gs_settings* settings,
                                       const int32_t* radii, const float* dL_dmeans2d,
                                       const float* dL_dconics, const float* dL_dcolors,
                                       float* dL_dmeans, float* dL_dscales, float* dL_dquats,
                                       float* dL_dsh, int32_t accumulate, void* stream);

/* Loss gradient of a rendered image against a target, both [count] floats:
 * kind 0 = L2 (sum (x-y)^2, gradient 2(x-y)), kind 1 = L1 (sum |x-y|,
 * gradient sign(x-y), sign(0) = 0).  Writes dL_dimage [count]; if loss (a
 * device float) is non-NULL it is overwritten with the loss value.  Sum
 * reduction, as the L2 loss of the 1,024-Gaussian case and the L1 loss of the
 * clustered cases are defined. */
GS_API gs_status gs_image_loss_grad(int32_t kind, int64_t count, const float* image,
                             const float* target, float* dL_dimage, float* loss,
                             void* stream);

/* Image loss of a training step (the gsplat guide §4.1 trains on the mean
 * absolute error plus 0.2 times (1 - SSIM)).  For [H][W][3] images x =
 * image and y = target with n = 3 H W elements:
 *   loss = sum|x - y| / n + lambda (1 - sum ssim / n),
 * where ssim is the structural similarity index per pixel and channel:
 * windowed means and second moments under an 11 x 11 Gaussian window
 * (standard deviation 1.5, normalised to sum 1; zero outside the image),
 * s = (2 mx my + C1)(2 sxy + C2) / ((mx^2 + my^2 + C1)(sx^2 + sy^2 + C2)),
 * C1 = 0.01^2, C2 = 0.03^2.  Writes dL_dimage [H][W][3] (sign(0) = 0 in the
 * L1 term) and, if loss (a device float) is non-NULL, the loss value; the
 * value and the gradient are reproducible bit for bit.  workspace: device
 * memory of gs_l1_dssim_workspace_size() bytes, 256-byte aligned.
 * dL_dimage must not alias image or target. */
GS_API size_t gs_l1_dssim_workspace_size(int32_t width, int32_t height);
GS_API gs_status gs_l1_dssim_loss_grad(int32_t width, int32_t height, const float* image,
                                       const float* target, float lambda, float* dL_dimage,
                                       float* loss, void* workspace, size_t workspace_bytes,
                                       void* stream);

/* One Adam step per parameter group (the gsplat guide §4.2: a learning rate
 * per group, betas (0.9, 0.99), eps 1e-15; gs_default_adam_config() returns
 * those, with the page's rates means 1.6e-4, scales 5e-3, quats 1e-3,
 * opacities 5e-2, SH 2.5e-3). */
typedef struct {
  float lr_means, lr_scales, lr_quats, lr_opacities, lr_sh;
  float beta1, beta2, eps;
} gs_adam_config;

GS_API gs_adam_config gs_default_adam_config(void);

/* The step updates the stored parameters in place: means [3][ld],
 * log_scales [3][ld], quats [4][ld], logit_opacities [ld], sh [K*3][ld].
 * The gradients are those the backward returns, with respect to means,
 * activated scales, quats, activated opacities and SH; they are first
 * carried to the stored values through the activated ones the forward used
 * (scales [3][ld] = exp(log_scales), opacities [ld] = sigmoid(logits)):
 * d/dlog_s = d/ds * s, d/dlogit = d/do * o (1 - o).  Then, per element,
 * m = beta1 m + (1 - beta1) g, v = beta2 v + (1 - beta2) g^2,
 * p -= lr / (1 - beta1^step) * m / (sqrt(v) / sqrt(1 - beta2^step) + eps),
 * and scales / opacities are rewritten from the new stored values.
 * exp_avg and exp_avg_sq are the moments, [P][ld] each with P = 11 + 3K
 * planes in the order means, scales, quats, opacity, SH (zero before the
 * first step).  step counts from 1. */
GS_API gs_status gs_adam_step(int64_t N, int64_t ld, int32_t sh_degree, int64_t step,
                              const gs_adam_config* cfg, float* means, float* log_scales,
                              float* quats, float* logit_opacities, float* sh, float* scales,
                              float* opacities, const float* dL_dmeans, const float* dL_dscales,
                              const float* dL_dquats, const float* dL_dopacities,
                              const float* dL_dsh, float* exp_avg, float* exp_avg_sq,
                              void* stream);

/* The packed form: the gradients are the packed rows of
 * gs_project_bwd_packed ([p][ldv], row r for Gaussian vis_ids[r]); only the
 * listed Gaussians are updated, the others keep parameters and moments
 * (sparse Adam). */
GS_API gs_status gs_adam_step_packed(int64_t num_visible, const uint32_t* vis_ids, int64_t ldv,
                                     int64_t N, int64_t ld, int32_t sh_degree, int64_t step,
                                     const gs_adam_config* cfg, float* means, float* log_scales,
                                     float* quats, float* logit_opacities, float* sh,
                                     float* scales, float* opacities, const float* dL_dmeans,
                                     const float* dL_dscales, const float* dL_dquats,
                                     const float* dL_dopacities, const float* dL_dsh,
                                     float* exp_avg, float* exp_avg_sq, void* stream);

/* Densify and prune between training steps (the count-changing step of the
 * gsplat guide §4.1, which clones by the mean-gradient magnitude and prunes
 * Gaussians of opacity below 0.005).  Out of place: the N Gaussians in
 * (means ... sh, planes [P][ld]) become *num_out Gaussians in the output
 * planes ([P][ld_out], distinct memory):
 *   1. n_clone = floor(clone_fraction * N + 0.5) (in double) Gaussians are
 *      selected by the key (gx*gx + gy*gy) + gz*gz of dL_dmeans [3][ld],
 *      evaluated in fp32 in that order (NaN taken as +inf): the n_clone
 *      largest keys, equal keys by lower index;
 *   2. the candidates are the N originals in index order followed by exact
 *      copies of the selected ones in index order;
 *   3. candidates with opacity < min_opacity are dropped; the others keep
 *      their order.
 * clone_fraction in [0, 1]; ld_out >= N + n_clone; N + n_clone < 2^30.
 * *num_out (HOST) receives the new count: the call's one device-to-host
 * read.  workspace: at least gs_densify_prune_workspace_size() bytes,
 * 256-byte aligned. */
GS_API size_t gs_densify_prune_workspace_size(int64_t N, float clone_fraction);
GS_API gs_status gs_densify_prune(int64_t N, int64_t ld, int32_t sh_degree, const float* means,
                                  const float* scales, const float* quats,
                                  const float* opacities, const float* sh,
                                  const float* dL_dmeans, float clone_fraction,
                                  float min_opacity, int64_t ld_out, float* means_out,
                                  float* scales_out, float* quats_out, float* opacities_out,
                                  float* sh_out, int64_t* num_out, void* workspace,
                                  size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* GSRASTER_H */
