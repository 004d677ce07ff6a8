/*
 * oracle.h — C ABI of the CPU oracle for the tile-based 3D Gaussian Splatting
 * rasterizer.  TEST INFRASTRUCTURE ONLY: this library is the slow, plain
 * reference that the HIP path is checked against.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it; the product
 * path never does.
 *
 * Every array is host memory in the natural per-Gaussian layout ([N,3] means,
 * [N,3] scales, [N,4] quaternions w-first, [N] opacities, [N,K,3] SH with
 * K=(deg+1)^2).  Inputs are doubles; in mode ORC_MODE_F32KEY they must hold
 * fp32-representable values, which the geometric key path then computes in
 * IEEE fp32 (no contraction, correctly rounded div/sqrt) while colours,
 * compositing and gradients are computed in fp64.
 *
 * What is computed, stage by stage, follows the three-stage pipeline of the
 * gsplat guide (lmnt.cn/news/262699) §2.1 (3D transform of R,t,scale,rot ->
 * depth and screen projection -> differentiable alpha blending), the
 * covariance-from-scale-and-rotation step of the Moore Threads MUSA article
 * (qwbw.cn/news/278220) §3.3, the quaternion order and activations of the
 * gsplat guide §3.3, and the separately callable backward of the gsplat
 * guide §2.2.  Formulas below the stage level are the textbook EWA-splatting
 * reading; the pages print none.
 */
#ifndef GS_ORACLE_H
#define GS_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  double R[9];      /* world-to-camera rotation, row-major; OpenCV axes */
  double t[3];      /* world-to-camera translation */
  double fx, fy, cx, cy;
  int32_t width, height;
  double near_plane, far_plane;
} orc_camera;

typedef struct {
  float eps2d, alpha_min, alpha_max, T_min, fov_clamp, sh_offset;
} orc_settings;

enum { ORC_MODE_F32KEY = 0, ORC_MODE_F64 = 1 };
enum { ORC_LOSS_L2 = 0, ORC_LOSS_L1 = 1 };

/* Projection (steps 1-8).  Outputs (all [N,...]):
 *   means2d [N,2], conics [N,3] (A,B,C of q = A dx^2 + 2B dx dy + C dy^2),
 *   chol [N,3] (L11, L21, L22 with conic = L L^T, so that
 *   q = (L11 dx + L21 dy)^2 + (L22 dy)^2),
 *   cov2d [N,3] (a,b,c after the eps2d dilation), depths [N], radii [N],
 *   tiles [N] (tiles touched), rect [N,4] (x0,x1,y0,y1), colors [N,3],
 *   clamped [N,3] (1 where the colour's max(0,.) clamp was active).
 * Culled Gaussians get radius 0, tiles 0 and zeros everywhere else.
 * Optional outputs may be NULL.  Returns 0. */
int orc_project(int mode, int64_t N, int sh_degree,
                const double* means, const double* scales, const double* quats,
                const double* sh, const orc_camera* cam, const orc_settings* st,
                double* means2d, double* conics, double* chol, double* cov2d,
                double* depths, int32_t* radii, uint32_t* tiles, int32_t* rect,
                double* colors, uint8_t* clamped);

/* Binning + stable sort + tile ranges (steps 9-11) on the fp32 key path.
 * means2d [N,2] and depths [N] are fp32.  Writes offsets [N] (exclusive scan
 * of tiles touched); when M <= capacity also keys [M], ids [M] and
 * ranges [T,2] (T = ceil(W/16)*ceil(H/16); empty tiles -> (0,0)).
 * Returns M. */
int64_t orc_bin_f32(int64_t N, const float* means2d, const int32_t* radii,
                    const float* depths, int32_t width, int32_t height,
                    int64_t capacity, uint32_t* offsets, uint64_t* keys,
                    uint32_t* ids, uint32_t* ranges);

/* Same binning with every decision taken in fp64 (rect from fp64 means2d,
 * stable sort by (tile, fp64 depth)).  No keys are produced. Returns M. */
int64_t orc_bin_f64(int64_t N, const double* means2d, const int32_t* radii,
                    const double* depths, int32_t width, int32_t height,
                    int64_t capacity, uint32_t* ids, uint32_t* ranges);

/* Front-to-back compositing (step 12), fp64, with q evaluated from chol
 * [N,3] as the completed square.  image [H,W,3], final_T [H,W],
 * last [H,W] (number of the tile's list entries up to and including the
 * last blended one; 0 if none), depth/alpha/margin [H,W] optional (NULL).
 * margin = smallest relative distance of a threshold decision taken for the
 * pixel (alpha vs alpha_min, o*G vs alpha_max, T' vs T_min). */
int orc_composite(int32_t width, int32_t height, const uint32_t* ranges,
                  const uint32_t* ids, const double* means2d,
                  const double* chol, const double* opacities,
                  const double* colors, const double* depths,
                  const double* background, const orc_settings* st,
                  double* image, double* final_T, uint32_t* last,
                  double* out_depth, double* out_alpha, double* margin);

/* Compositing backward (step 13, first half), fp64, recomputing the forward
 * per pixel (q from chol) and keeping every layer's transmittance; the
 * derivatives of q with respect to u, v and the conic use conics.  Writes (overwrites)
 * g_means2d [N,2], g_conics [N,3], g_opacities [N], g_colors [N,3], and if
 * non-NULL abs_sum [N,9] = sum of |per-pixel contribution| for each of those
 * nine fields (u,v,A,B,C,o,r,g,b), a conditioning measure. */
int orc_composite_bwd(int32_t width, int32_t height, int64_t N,
                      const uint32_t* ranges, const uint32_t* ids,
                      const double* means2d, const double* chol, const double* conics,
                      const double* opacities, const double* colors,
                      const double* background, const orc_settings* st,
                      const double* dL_dimage, double* g_means2d,
                      double* g_conics, double* g_opacities, double* g_colors,
                      double* abs_sum);

/* Projection backward (step 13, second half), fp64 from the parameters.
 * Visibility is taken from radii (radius 0 -> zero gradients); every other
 * decision (fov clamp, colour clamp) is recomputed in fp64.  Overwrites
 * g_means [N,3], g_scales [N,3], g_quats [N,4], g_sh [N,K,3]. */
int orc_project_bwd(int64_t N, int sh_degree, const double* means,
                    const double* scales, const double* quats,
                    const double* sh, const orc_camera* cam,
                    const orc_settings* st, const int32_t* radii,
                    const double* g_means2d, const double* g_conics,
                    const double* g_colors, double* g_means, double* g_scales,
                    double* g_quats, double* g_sh);

/* Sensitivity bound of the projection backward to its 2D gradient inputs.
 * With the discrete decisions fixed by the parameters, orc_project_bwd is
 * linear in (g_means2d, g_conics, g_colors), so changing those inputs by
 * d with |d_k| <= s_k changes each output o by at most
 *   e_o = sum_k |d o / d g2_k| s_k,
 * and exactly that much for d_k = s_k sign(d o / d g2_k).  Writes e for
 * every output (zeros for culled Gaussians).  The parity tests use it to
 * bound what a projection backward inherits from 2D gradients known only to
 * within s (fp32 rounding, or the 2D tolerance end to end). */
int orc_project_bwd_bound(int64_t N, int sh_degree, const double* means,
                          const double* scales, const double* quats,
                          const double* sh, const orc_camera* cam,
                          const orc_settings* st, const int32_t* radii,
                          const double* s_means2d, const double* s_conics,
                          const double* s_colors, double* e_means, double* e_scales,
                          double* e_quats, double* e_sh);

/* Whole forward in fp64 (or with forward-mode dual numbers when any
 * direction pointer is non-NULL) followed by the loss against target
 * [H,W,3] (L2: sum (C-T)^2; L1: sum |C-T|).  Writes loss, its directional
 * derivative along the given direction (0 if no direction), and a 64-bit
 * signature of every discrete decision taken (visibility, tile lists,
 * skipped/blended pairs, stop points, clamps), so that finite differences
 * can detect steps that crossed a decision boundary; image_out [H,W,3]
 * (optional) receives the rendered image.  Returns M. */
int64_t orc_loss_jvp(int64_t N, int sh_degree, const double* means,
                     const double* scales, const double* quats,
                     const double* opacities, const double* sh,
                     const double* d_means, const double* d_scales,
                     const double* d_quats, const double* d_opacities,
                     const double* d_sh, const orc_camera* cam,
                     const orc_settings* st, const double* background,
                     int loss_kind, const double* target, double* loss,
                     double* dloss, uint64_t* signature, double* image_out);

/* Threads the oracle's parallel loops use from now on (n > 0), for timing
 * it in one-thread and all-core modes; returns the current setting. */
int orc_set_threads(int n);

/* Building blocks exposed for the pins. */
void orc_rotation(const double* quat, double* R);          /* R [3,3] of q/|q| */
void orc_cov3d(const double* quat, const double* scale, double* Sigma); /* [3,3] */
void orc_sh_basis(int sh_degree, const double* dir, double* Y);  /* K values */
void orc_sh_basis_grad(int sh_degree, const double* dir, double* dY); /* [K,3] */

#ifdef __cplusplus
}
#endif
#endif
