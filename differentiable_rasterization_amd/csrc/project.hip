// project.hip — stage 1 (projection) and its backward.
//
// Gaussian-parallel and HBM-bound: one lane per Gaussian, every parameter
// plane read once with coalesced 4-byte loads (the planes are structure-of-
// arrays with leading dimension ld), outputs written the same way.
//
// The geometric key path (camera transform, covariance, EWA Jacobian, 2D
// covariance, conic, radius, pixel mean, tile rect) follows the pipeline of
// the gsplat guide (lmnt.cn/news/262699) §2.1 and the scale/rotation
// covariance of the Moore Threads MUSA article (qwbw.cn/news/278220) §3.3.
// It is evaluated in IEEE fp32 in one fixed operation order with no
// contraction, with correctly rounded division and square root, so its
// outputs (and the tile keys derived from them) are reproducible bit for bit.
#include "gs_common.h"

namespace gs {

struct Geom {
  float u, v, depth, a, b, c, A, B, C;
  float L11, L21, L22;  // conic = L L^T, L lower triangular
  int32_t radius;
  int x0, x1, y0, y1;
  bool clampx, clampy;
};

// Rotation of the unit quaternion (w,x,y,z), row-major.
__device__ inline void quat_to_rot(float w, float x, float y, float z, float R[9]) {
  R[0] = 1.0f - 2.0f * (y * y + z * z);
  R[1] = 2.0f * (x * y - w * z);
  R[2] = 2.0f * (x * z + w * y);
  R[3] = 2.0f * (x * y + w * z);
  R[4] = 1.0f - 2.0f * (x * x + z * z);
  R[5] = 2.0f * (y * z - w * x);
  R[6] = 2.0f * (x * z - w * y);
  R[7] = 2.0f * (y * z + w * x);
  R[8] = 1.0f - 2.0f * (x * x + y * y);
}

__device__ inline float sel_min(float a, float b) { return (b < a) ? b : a; }
__device__ inline float sel_max(float a, float b) { return (a < b) ? b : a; }

// Returns false when the Gaussian is culled.  qn receives the unit
// quaternion and its norm, Sig the 3D covariance, Tm = J W (2x3).
__device__ inline bool project_geom(const float m[3], const float s[3], const float q[4],
                                    const Cam& cam, const Settings& st, Geom& g, float qn[5],
                                    float Rq[9], float Sig[6], float Tm[6], float tcam[3]) {
  for (int i = 0; i < 3; ++i)
    if (!__builtin_isfinite(m[i]) || !__builtin_isfinite(s[i])) return false;
  for (int i = 0; i < 4; ++i)
    if (!__builtin_isfinite(q[i])) return false;
  const float* W = cam.R;
  const float tx = ((W[0] * m[0] + W[1] * m[1]) + W[2] * m[2]) + cam.t[0];
  const float ty = ((W[3] * m[0] + W[4] * m[1]) + W[5] * m[2]) + cam.t[1];
  const float tz = ((W[6] * m[0] + W[7] * m[1]) + W[8] * m[2]) + cam.t[2];
  if (!(tz > cam.near_p && tz < cam.far_p)) return false;
  if (!__builtin_isfinite(tx) || !__builtin_isfinite(ty)) return false;
  tcam[0] = tx; tcam[1] = ty; tcam[2] = tz;

  const float n2 = ((q[0] * q[0] + q[1] * q[1]) + q[2] * q[2]) + q[3] * q[3];
  if (!(n2 > 0.0f) || !__builtin_isfinite(n2)) return false;
  const float nr = sqrtf(n2);
  qn[0] = q[0] / nr; qn[1] = q[1] / nr; qn[2] = q[2] / nr; qn[3] = q[3] / nr; qn[4] = nr;
  quat_to_rot(qn[0], qn[1], qn[2], qn[3], Rq);
  float M[9];
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 3; ++j) M[i * 3 + j] = Rq[i * 3 + j] * s[j];
  // Sigma = M M^T (upper triangle: 00 01 02 11 12 22)
  {
    int k = 0;
    for (int i = 0; i < 3; ++i)
      for (int j = i; j < 3; ++j)
        Sig[k++] = (M[i * 3 + 0] * M[j * 3 + 0] + M[i * 3 + 1] * M[j * 3 + 1]) +
                   M[i * 3 + 2] * M[j * 3 + 2];
  }
  const float S00 = Sig[0], S01 = Sig[1], S02 = Sig[2], S11 = Sig[3], S12 = Sig[4], S22 = Sig[5];
  const float Sf[9] = {S00, S01, S02, S01, S11, S12, S02, S12, S22};

  const float txz = tx / tz, tyz = ty / tz;
  const float tanx = (0.5f * (float)cam.W) / cam.fx;
  const float tany = (0.5f * (float)cam.H) / cam.fy;
  const float limx = st.fov_clamp * tanx;
  const float limy = st.fov_clamp * tany;
  const float cxz = sel_min(limx, sel_max(-limx, txz));
  const float cyz = sel_min(limy, sel_max(-limy, tyz));
  g.clampx = (txz > limx) || (txz < -limx);
  g.clampy = (tyz > limy) || (tyz < -limy);
  const float xc = cxz * tz, yc = cyz * tz;
  const float tz2 = tz * tz;
  const float J00 = cam.fx / tz;
  const float J02 = -((cam.fx * xc) / tz2);
  const float J11 = cam.fy / tz;
  const float J12 = -((cam.fy * yc) / tz2);
  for (int j = 0; j < 3; ++j) {
    Tm[0 * 3 + j] = J00 * W[0 * 3 + j] + J02 * W[2 * 3 + j];
    Tm[1 * 3 + j] = J11 * W[1 * 3 + j] + J12 * W[2 * 3 + j];
  }
  float U[6];
  for (int a = 0; a < 2; ++a)
    for (int j = 0; j < 3; ++j)
      U[a * 3 + j] = (Tm[a * 3 + 0] * Sf[0 * 3 + j] + Tm[a * 3 + 1] * Sf[1 * 3 + j]) +
                     Tm[a * 3 + 2] * Sf[2 * 3 + j];
  const float c00 = (U[0] * Tm[0] + U[1] * Tm[1]) + U[2] * Tm[2];
  const float c01 = (U[0] * Tm[3] + U[1] * Tm[4]) + U[2] * Tm[5];
  const float c11 = (U[3] * Tm[3] + U[4] * Tm[4]) + U[5] * Tm[5];
  const float a = c00 + st.eps2d;
  const float b = c01;
  const float c = c11 + st.eps2d;

  // conic = inverse of the (positive definite) dilated 2D covariance, and
  // its Cholesky factor, with which the quadratic form is the completed
  // square q = (L11 dx + L21 dy)^2 + (L22 dy)^2: no cancellation for
  // needle-like splats, where the expanded form loses about u (|A| dx^2 +
  // 2|B dx dy| + |C| dy^2) with those terms 1e4-1e5 times q
  const float det = a * c - b * b;
  if (!(det > 0.0f) || !__builtin_isfinite(det) || !(a > 0.0f)) return false;
  const float A = c / det;
  const float B = -(b / det);
  const float C = a / det;
  const float L11 = sqrtf(A);
  const float L21 = B / L11;
  const float L22 = 1.0f / sqrtf(c);

  const float mid = 0.5f * (a + c);
  const float disc = mid * mid - det;
  const float lam = mid + sqrtf(sel_max(disc, 0.0f));
  if (!__builtin_isfinite(lam)) return false;
  float rf = ceilf(3.0f * sqrtf(lam));
  if (rf > 16777216.0f) rf = 16777216.0f;
  const int32_t radius = (int32_t)rf;
  if (radius <= 0) return false;

  const float u = cam.fx * txz + cam.cx;
  const float v = cam.fy * tyz + cam.cy;
  if (!__builtin_isfinite(u) || !__builtin_isfinite(v)) return false;

  const int gx = grid_dim(cam.W), gy = grid_dim(cam.H);
  tile_rect(u, v, radius, gx, gy, g.x0, g.x1, g.y0, g.y1);
  if (g.x1 <= g.x0 || g.y1 <= g.y0) return false;

  g.u = u; g.v = v; g.depth = tz;
  g.a = a; g.b = b; g.c = c;
  g.A = A; g.B = B; g.C = C;
  g.L11 = L11; g.L21 = L21; g.L22 = L22;
  g.radius = radius;
  return true;
}

// Real spherical harmonics up to degree 3 at the unit direction (x,y,z),
// ordered (l, m=-l..l), Condon-Shortley phase.  Each constant is
// N_lm = sqrt((2l+1)/(4 pi) (l-|m|)!/(l+|m|)!) (times sqrt 2 for m != 0)
// times the integer factor of the Cartesian polynomial of P_l^|m|.
namespace shc {
constexpr double D0 = 0.28209479177387814;
constexpr double D1 = 0.4886025119029199;
constexpr double D2a = 1.0925484305920792;   // xy, yz, xz
constexpr double D2b = 0.31539156525252005;  // 3z^2 - 1
constexpr double D2c = 0.5462742152960396;   // x^2 - y^2
constexpr double D3a = 0.5900435899266435;   // y(3x^2-y^2), x(x^2-3y^2)
constexpr double D3b = 2.890611442640554;    // xyz
constexpr double D3c = 0.4570457994644658;   // y(5z^2-1), x(5z^2-1)
constexpr double D3d = 0.3731763325901154;   // z(5z^2-3)
constexpr double D3e = 1.445305721320277;    // z(x^2-y^2)
// the fp32 forward's constants: the same values rounded to fp32
constexpr float C0 = (float)D0, C1 = (float)D1, C2a = (float)D2a, C2b = (float)D2b,
                C2c = (float)D2c, C3a = (float)D3a, C3b = (float)D3b, C3c = (float)D3c,
                C3d = (float)D3d, C3e = (float)D3e;
}  // namespace shc

__device__ inline void sh_basis(int deg, float x, float y, float z, float Y[16]) {
  using namespace shc;
  Y[0] = C0;
  if (deg < 1) return;
  Y[1] = -C1 * y;
  Y[2] = C1 * z;
  Y[3] = -C1 * x;
  if (deg < 2) return;
  const float xx = x * x, yy = y * y, zz = z * z;
  Y[4] = C2a * (x * y);
  Y[5] = -C2a * (y * z);
  Y[6] = C2b * (3.0f * zz - 1.0f);
  Y[7] = -C2a * (x * z);
  Y[8] = C2c * (xx - yy);
  if (deg < 3) return;
  Y[9] = -C3a * (y * (3.0f * xx - yy));
  Y[10] = C3b * (x * y * z);
  Y[11] = -C3c * (y * (5.0f * zz - 1.0f));
  Y[12] = C3d * (z * (5.0f * zz - 3.0f));
  Y[13] = -C3c * (x * (5.0f * zz - 1.0f));
  Y[14] = C3e * (z * (xx - yy));
  Y[15] = -C3a * (x * (xx - 3.0f * yy));
}

// g[0..2] += w * grad Y_j(x,y,z) for the Cartesian polynomials above.
__device__ inline void sh_basis_grad_acc(int j, float w, float x, float y, float z, float g[3]) {
  using namespace shc;
  const float xx = x * x, yy = y * y, zz = z * z;
  float dx = 0.0f, dy = 0.0f, dz = 0.0f;
  switch (j) {
    case 1: dy = -C1; break;
    case 2: dz = C1; break;
    case 3: dx = -C1; break;
    case 4: dx = C2a * y; dy = C2a * x; break;
    case 5: dy = -C2a * z; dz = -C2a * y; break;
    case 6: dz = 6.0f * C2b * z; break;
    case 7: dx = -C2a * z; dz = -C2a * x; break;
    case 8: dx = 2.0f * C2c * x; dy = -2.0f * C2c * y; break;
    case 9: dx = -C3a * 6.0f * x * y; dy = -C3a * (3.0f * xx - 3.0f * yy); break;
    case 10: dx = C3b * y * z; dy = C3b * x * z; dz = C3b * x * y; break;
    case 11: dy = -C3c * (5.0f * zz - 1.0f); dz = -C3c * 10.0f * y * z; break;
    case 12: dz = C3d * (15.0f * zz - 3.0f); break;
    case 13: dx = -C3c * (5.0f * zz - 1.0f); dz = -C3c * 10.0f * x * z; break;
    case 14: dx = 2.0f * C3e * x * z; dy = -2.0f * C3e * y * z; dz = C3e * (xx - yy); break;
    case 15: dx = -C3a * (3.0f * xx - 3.0f * yy); dy = C3a * 6.0f * x * y; break;
    default: break;
  }
  g[0] = fmaf(w, dx, g[0]);
  g[1] = fmaf(w, dy, g[1]);
  g[2] = fmaf(w, dz, g[2]);
}

__device__ inline void camera_centre(const Cam& cam, float c[3]) {
  for (int j = 0; j < 3; ++j)
    c[j] = -(cam.R[0 * 3 + j] * cam.t[0] + cam.R[1 * 3 + j] * cam.t[1] +
             cam.R[2 * 3 + j] * cam.t[2]);
}

// Camera blockIdx.y of the batch writes its outputs to block c of each
// output ([c][plane][ld] planes).  Rows N .. rows-1 (the padding of a batch,
// rows = ld) get radius 0 and no tiles.
template <int DEG>
__global__ __launch_bounds__(256) void project_fwd_kernel(
    int64_t N, int64_t rows, int64_t ld, const float* __restrict__ means,
    const float* __restrict__ scales, const float* __restrict__ quats,
    const float* __restrict__ sh, CamBatch cams, Settings st, float* __restrict__ means2d,
    float* __restrict__ conics, float* __restrict__ chol, float* __restrict__ depths,
    int32_t* __restrict__ radii, float* __restrict__ colors, uint32_t* __restrict__ tiles) {
  constexpr int K = (DEG + 1) * (DEG + 1);
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows) return;
  const int64_t cb = (int64_t)blockIdx.y;
  means2d += cb * 2 * ld;
  conics += cb * 3 * ld;
  chol += cb * 3 * ld;
  depths += cb * ld;
  radii += cb * ld;
  colors += cb * 3 * ld;
  tiles += cb * ld;
  if (i >= N) {
    radii[i] = 0;
    tiles[i] = 0u;
    return;
  }
  const Cam cam = cams.c[blockIdx.y];
  // all loads first: every lane keeps its parameters and SH coefficients in
  // flight together (culled lanes share cache lines with visible ones, so
  // their SH lines are fetched anyway)
  const float m[3] = {means[i], means[ld + i], means[2 * ld + i]};
  const float s[3] = {scales[i], scales[ld + i], scales[2 * ld + i]};
  const float q[4] = {quats[i], quats[ld + i], quats[2 * ld + i], quats[3 * ld + i]};
  float shv[3 * K];
#pragma unroll
  for (int k = 0; k < 3 * K; ++k) shv[k] = sh[(int64_t)k * ld + i];

  Geom g;
  float qn[5], Rq[9], Sig[6], Tm[6], tc[3];
  const bool vis = project_geom(m, s, q, cam, st, g, qn, Rq, Sig, Tm, tc);
  float col[3] = {0.0f, 0.0f, 0.0f};
  if (vis) {
    float cc[3];
    camera_centre(cam, cc);
    const float dir[3] = {m[0] - cc[0], m[1] - cc[1], m[2] - cc[2]};
    const float L = sqrtf(dir[0] * dir[0] + dir[1] * dir[1] + dir[2] * dir[2]);
    const float d[3] = {dir[0] / L, dir[1] / L, dir[2] / L};
    float Y[16];
    sh_basis(DEG, d[0], d[1], d[2], Y);
    float raw[3] = {st.sh_offset, st.sh_offset, st.sh_offset};
#pragma unroll
    for (int j = 0; j < K; ++j)
#pragma unroll
      for (int ch = 0; ch < 3; ++ch) raw[ch] = fmaf(Y[j], shv[j * 3 + ch], raw[ch]);
#pragma unroll
    for (int ch = 0; ch < 3; ++ch) col[ch] = raw[ch] < 0.0f ? 0.0f : raw[ch];
  }
  // one store path for culled (zeros) and visible lanes
  means2d[i] = vis ? g.u : 0.0f;
  means2d[ld + i] = vis ? g.v : 0.0f;
  conics[i] = vis ? g.A : 0.0f;
  conics[ld + i] = vis ? g.B : 0.0f;
  conics[2 * ld + i] = vis ? g.C : 0.0f;
  chol[i] = vis ? g.L11 : 0.0f;
  chol[ld + i] = vis ? g.L21 : 0.0f;
  chol[2 * ld + i] = vis ? g.L22 : 0.0f;
  depths[i] = vis ? g.depth : 0.0f;
  radii[i] = vis ? g.radius : 0;
  tiles[i] = vis ? (uint32_t)(g.x1 - g.x0) * (uint32_t)(g.y1 - g.y0) : 0u;
#pragma unroll
  for (int ch = 0; ch < 3; ++ch) colors[(int64_t)ch * ld + i] = col[ch];
}

// Real SH basis and its gradient in fp64, for the backward (the same
// polynomials as the fp32 forward above, with the constants in fp64: the
// colour clamp is decided on this fp64 value, and fp32-rounded constants
// (relative error up to 3e-8) would decide it differently for a colour
// within ~1e-8 of zero).
__device__ inline void sh_basis64(int deg, double x, double y, double z, double Y[16]) {
  using namespace shc;
  Y[0] = D0;
  if (deg < 1) return;
  Y[1] = -D1 * y;
  Y[2] = D1 * z;
  Y[3] = -D1 * x;
  if (deg < 2) return;
  const double xx = x * x, yy = y * y, zz = z * z;
  Y[4] = D2a * (x * y);
  Y[5] = -D2a * (y * z);
  Y[6] = D2b * (3.0 * zz - 1.0);
  Y[7] = -D2a * (x * z);
  Y[8] = D2c * (xx - yy);
  if (deg < 3) return;
  Y[9] = -D3a * (y * (3.0 * xx - yy));
  Y[10] = D3b * (x * y * z);
  Y[11] = -D3c * (y * (5.0 * zz - 1.0));
  Y[12] = D3d * (z * (5.0 * zz - 3.0));
  Y[13] = -D3c * (x * (5.0 * zz - 1.0));
  Y[14] = D3e * (z * (xx - yy));
  Y[15] = -D3a * (x * (xx - 3.0 * yy));
}

__device__ inline void sh_basis_grad_acc64(int j, double w, double x, double y, double z,
                                           double g[3]) {
  using namespace shc;
  const double xx = x * x, yy = y * y, zz = z * z;
  double dx = 0.0, dy = 0.0, dz = 0.0;
  switch (j) {
    case 1: dy = -D1; break;
    case 2: dz = D1; break;
    case 3: dx = -D1; break;
    case 4: dx = D2a * y; dy = D2a * x; break;
    case 5: dy = -D2a * z; dz = -D2a * y; break;
    case 6: dz = 6.0 * D2b * z; break;
    case 7: dx = -D2a * z; dz = -D2a * x; break;
    case 8: dx = 2.0 * D2c * x; dy = -2.0 * D2c * y; break;
    case 9: dx = -D3a * 6.0 * x * y; dy = -D3a * (3.0 * xx - 3.0 * yy); break;
    case 10: dx = D3b * y * z; dy = D3b * x * z; dz = D3b * x * y; break;
    case 11: dy = -D3c * (5.0 * zz - 1.0); dz = -D3c * 10.0 * y * z; break;
    case 12: dz = D3d * (15.0 * zz - 3.0); break;
    case 13: dx = -D3c * (5.0 * zz - 1.0); dz = -D3c * 10.0 * x * z; break;
    case 14:
      dx = 2.0 * D3e * x * z; dy = -2.0 * D3e * y * z;
      dz = D3e * (xx - yy);
      break;
    case 15: dx = -D3a * (3.0 * xx - 3.0 * yy); dy = D3a * 6.0 * x * y; break;
    default: break;
  }
  g[0] = fma(w, dx, g[0]);
  g[1] = fma(w, dy, g[1]);
  g[2] = fma(w, dz, g[2]);
}

// Backward of the projection: the chain rule from the 2D gradient record to
// the mean, scale, quaternion and SH coefficients, evaluated in fp64 (inputs
// converted exactly, each output rounded once to fp32).  The geometry is
// recomputed in fp64 from the parameters; visibility is the forward's
// (radius > 0), the fov and colour clamps are re-decided in fp64.  fp64
// because the chain through a nearly singular 2D covariance (needle-like
// splats, condition numbers 1e4-1e5) loses about u times the condition
// number in fp32; the kernel moves ~300 bytes per Gaussian against a few
// hundred fp64 operations, so it stays memory-bound.

// The SH side of one camera: view direction d (and 1 / distance), the
// colour clamp decision in fp64, and the colour gradient gcol that passes it.
template <int DEG>
__device__ inline void sh_view(const Cam& cam, const float pm[3], const float* shv,
                               float sh_offset, const float gin[3], double d[3], double& iL,
                               float gcol[3]) {
  constexpr int K = (DEG + 1) * (DEG + 1);
  double cc[3];
  for (int j = 0; j < 3; ++j)
    cc[j] = -(((double)cam.R[j] * (double)cam.t[0] + (double)cam.R[3 + j] * (double)cam.t[1]) +
              (double)cam.R[6 + j] * (double)cam.t[2]);
  const double dir[3] = {(double)pm[0] - cc[0], (double)pm[1] - cc[1], (double)pm[2] - cc[2]};
  iL = 1.0 / sqrt(dir[0] * dir[0] + dir[1] * dir[1] + dir[2] * dir[2]);
  for (int j = 0; j < 3; ++j) d[j] = dir[j] * iL;
  double Y[16];
  sh_basis64(DEG, d[0], d[1], d[2], Y);
  double raw[3] = {(double)sh_offset, (double)sh_offset, (double)sh_offset};
#pragma unroll
  for (int j = 0; j < K; ++j)
#pragma unroll
    for (int ch = 0; ch < 3; ++ch) raw[ch] = fma(Y[j], (double)shv[j * 3 + ch], raw[ch]);
  for (int ch = 0; ch < 3; ++ch) gcol[ch] = raw[ch] < 0.0 ? 0.0f : gin[ch];
}

// SH coefficient gradients Y_j(d) gcol (fp32 products, handed to `sink` as
// (coefficient index, value)) and the view direction's share of the mean
// gradient, vterm.
template <int DEG, typename Sink>
__device__ inline void sh_grads(const double d[3], double iL, const float gcol[3],
                                const float* shv, Sink sink, double vterm[3]) {
  constexpr int K = (DEG + 1) * (DEG + 1);
  float Yf[16];
  sh_basis(DEG, (float)d[0], (float)d[1], (float)d[2], Yf);
  double gd[3] = {0.0, 0.0, 0.0};
#pragma unroll
  for (int j = 0; j < K; ++j) {
    double wj = 0.0;
#pragma unroll
    for (int ch = 0; ch < 3; ++ch) {
      sink(j * 3 + ch, Yf[j] * gcol[ch]);
      wj = fma((double)gcol[ch], (double)shv[j * 3 + ch], wj);
    }
    if (j > 0) sh_basis_grad_acc64(j, wj, d[0], d[1], d[2], gd);
  }
  const double dd = d[0] * gd[0] + d[1] * gd[1] + d[2] * gd[2];
  for (int e = 0; e < 3; ++e) vterm[e] = (gd[e] - d[e] * dd) * iL;
}

// The geometry chain of one camera in fp64: mean (with the view-direction
// term vterm added before rounding), scale and quaternion gradients.
// r0 = (dL/du, dL/dv, dL/dA, dL/dB), r1.x = dL/dC.
__device__ inline void geom_grads(const Cam& cam, const Settings& st, const float pm[3],
                                  const float ps[3], const float pq[4], float4 r0, float4 r1,
                                  const double vterm[3], float om[3], float os[3], float oq[4]) {
  const double m[3] = {pm[0], pm[1], pm[2]};
  const double s[3] = {ps[0], ps[1], ps[2]};
  const double q[4] = {pq[0], pq[1], pq[2], pq[3]};
  double W[9];
  for (int k = 0; k < 9; ++k) W[k] = cam.R[k];
  const double fx = cam.fx, fy = cam.fy;
  const double tx = ((W[0] * m[0] + W[1] * m[1]) + W[2] * m[2]) + (double)cam.t[0];
  const double ty = ((W[3] * m[0] + W[4] * m[1]) + W[5] * m[2]) + (double)cam.t[1];
  const double tz = ((W[6] * m[0] + W[7] * m[1]) + W[8] * m[2]) + (double)cam.t[2];

  // unit quaternion, rotation, M = R diag(s), Sigma = M M^T
  const double n2 = ((q[0] * q[0] + q[1] * q[1]) + q[2] * q[2]) + q[3] * q[3];
  // (fp64 reciprocals stand in for divisions: their rounding is far below
  // the fp32 outputs')
  const double nr = sqrt(n2), inr = 1.0 / nr;
  const double w = q[0] * inr, x = q[1] * inr, y = q[2] * inr, z = q[3] * inr;
  double Rq[9];
  Rq[0] = 1.0 - 2.0 * (y * y + z * z);
  Rq[1] = 2.0 * (x * y - w * z);
  Rq[2] = 2.0 * (x * z + w * y);
  Rq[3] = 2.0 * (x * y + w * z);
  Rq[4] = 1.0 - 2.0 * (x * x + z * z);
  Rq[5] = 2.0 * (y * z - w * x);
  Rq[6] = 2.0 * (x * z - w * y);
  Rq[7] = 2.0 * (y * z + w * x);
  Rq[8] = 1.0 - 2.0 * (x * x + y * y);
  double M[9];
  for (int r = 0; r < 3; ++r)
    for (int j = 0; j < 3; ++j) M[r * 3 + j] = Rq[r * 3 + j] * s[j];
  double Sf[9];
  for (int r = 0; r < 3; ++r)
    for (int j = r; j < 3; ++j) {
      const double v = (M[r * 3] * M[j * 3] + M[r * 3 + 1] * M[j * 3 + 1]) +
                       M[r * 3 + 2] * M[j * 3 + 2];
      Sf[r * 3 + j] = v;
      Sf[j * 3 + r] = v;
    }

  // EWA Jacobian with the fov clamp, T = J W, 2D covariance and conic
  const double itz = 1.0 / tz, itz2 = itz * itz, itz3 = itz2 * itz;
  const double txz = tx * itz, tyz = ty * itz;
  const double limx = (double)st.fov_clamp * ((0.5 * (double)cam.W) / fx);
  const double limy = (double)st.fov_clamp * ((0.5 * (double)cam.H) / fy);
  const bool clampx = (txz > limx) || (txz < -limx);
  const bool clampy = (tyz > limy) || (tyz < -limy);
  const double xc = (clampx ? (txz > 0.0 ? limx : -limx) : txz) * tz;
  const double yc = (clampy ? (tyz > 0.0 ? limy : -limy) : tyz) * tz;
  const double J00 = fx * itz, J02 = -(fx * xc * itz2);
  const double J11 = fy * itz, J12 = -(fy * yc * itz2);
  double Tm[6];
  for (int j = 0; j < 3; ++j) {
    Tm[j] = J00 * W[j] + J02 * W[6 + j];
    Tm[3 + j] = J11 * W[3 + j] + J12 * W[6 + j];
  }
  double ST0[3], ST1[3];
  for (int r = 0; r < 3; ++r) {
    ST0[r] = Sf[r * 3] * Tm[0] + Sf[r * 3 + 1] * Tm[1] + Sf[r * 3 + 2] * Tm[2];
    ST1[r] = Sf[r * 3] * Tm[3] + Sf[r * 3 + 1] * Tm[4] + Sf[r * 3 + 2] * Tm[5];
  }
  const double a = (Tm[0] * ST0[0] + Tm[1] * ST0[1] + Tm[2] * ST0[2]) + (double)st.eps2d;
  const double b = Tm[0] * ST1[0] + Tm[1] * ST1[1] + Tm[2] * ST1[2];
  const double c = (Tm[3] * ST1[0] + Tm[4] * ST1[1] + Tm[5] * ST1[2]) + (double)st.eps2d;
  const double idet = 1.0 / (a * c - b * b);
  const double A = c * idet, B = -(b * idet), C = a * idet;

  // conic = Sigma2D^-1: dL/dSigma2D = -conic G conic, G = [[gA, gB/2], [gB/2, gC]]
  const double gA = r0.z, gB = r0.w, gC = r1.x;
  const double ga = -(gA * A * A + gB * A * B + gC * B * B);
  const double gb = -(2.0 * gA * A * B + gB * (A * C + B * B) + 2.0 * gC * B * C);
  const double gc = -(gA * B * B + gB * B * C + gC * C * C);

  // Sigma2D = T Sigma T^T: dL/dSigma = T^T G2 T, dL/dT = 2 G2 T Sigma
  double gT0[3], gT1[3];
  for (int r = 0; r < 3; ++r) {
    gT0[r] = 2.0 * ga * ST0[r] + gb * ST1[r];
    gT1[r] = gb * ST0[r] + 2.0 * gc * ST1[r];
  }
  double gJ00 = 0.0, gJ02 = 0.0, gJ11 = 0.0, gJ12 = 0.0;
  for (int j = 0; j < 3; ++j) {
    gJ00 += gT0[j] * W[j];
    gJ02 += gT0[j] * W[6 + j];
    gJ11 += gT1[j] * W[3 + j];
    gJ12 += gT1[j] * W[6 + j];
  }
  double gt[3] = {0.0, 0.0, 0.0};
  gt[2] += gJ00 * (-fx * itz2) + gJ11 * (-fy * itz2);
  if (clampx) {
    gt[2] += gJ02 * (fx * (txz > 0.0 ? limx : -limx) * itz2);
  } else {
    gt[0] += gJ02 * (-fx * itz2);
    gt[2] += gJ02 * (2.0 * fx * tx * itz3);
  }
  if (clampy) {
    gt[2] += gJ12 * (fy * (tyz > 0.0 ? limy : -limy) * itz2);
  } else {
    gt[1] += gJ12 * (-fy * itz2);
    gt[2] += gJ12 * (2.0 * fy * ty * itz3);
  }
  const double gu = r0.x, gv = r0.y;
  gt[0] += gu * fx * itz;
  gt[2] += gu * (-fx * tx * itz2);
  gt[1] += gv * fy * itz;
  gt[2] += gv * (-fy * ty * itz2);
  double gm[3];
  for (int j = 0; j < 3; ++j) gm[j] = W[j] * gt[0] + W[3 + j] * gt[1] + W[6 + j] * gt[2];

  // Sigma = M M^T, M = R diag(s): dL/dM = (G + G^T) M with
  // G = dL/dSigma = ga T0^T T0 + gb T0^T T1 + gc T1^T T1 (formed row by row)
  double gs[3] = {0.0, 0.0, 0.0}, gR[9];
  for (int r = 0; r < 3; ++r) {
    double Gr[3];
    for (int j = 0; j < 3; ++j)
      Gr[j] = 2.0 * (ga * Tm[r] * Tm[j] + gc * Tm[3 + r] * Tm[3 + j]) +
              gb * (Tm[r] * Tm[3 + j] + Tm[3 + r] * Tm[j]);
    for (int k = 0; k < 3; ++k) {
      const double acc = (Gr[0] * M[k] + Gr[1] * M[3 + k]) + Gr[2] * M[6 + k];
      gs[k] += acc * Rq[r * 3 + k];
      gR[r * 3 + k] = acc * s[k];
    }
  }
  double gqn[4];
  gqn[0] = 2.0 * (-z * gR[1] + y * gR[2] + z * gR[3] - x * gR[5] - y * gR[6] + x * gR[7]);
  gqn[1] = 2.0 * (y * gR[1] + z * gR[2] + y * gR[3] - w * gR[5] + z * gR[6] + w * gR[7]) -
           4.0 * x * (gR[4] + gR[8]);
  gqn[2] = 2.0 * (x * gR[1] + w * gR[2] + x * gR[3] + z * gR[5] - w * gR[6] + z * gR[7]) -
           4.0 * y * (gR[0] + gR[8]);
  gqn[3] = 2.0 * (-w * gR[1] + x * gR[2] + w * gR[3] + y * gR[5] + x * gR[6] + y * gR[7]) -
           4.0 * z * (gR[0] + gR[4]);
  const double dot = w * gqn[0] + x * gqn[1] + y * gqn[2] + z * gqn[3];
  oq[0] = (float)((gqn[0] - w * dot) * inr);
  oq[1] = (float)((gqn[1] - x * dot) * inr);
  oq[2] = (float)((gqn[2] - y * dot) * inr);
  oq[3] = (float)((gqn[3] - z * dot) * inr);
  for (int k = 0; k < 3; ++k) os[k] = (float)gs[k];

  for (int k = 0; k < 3; ++k) om[k] = (float)(gm[k] + vterm[k]);
}

// Packed form (kPacked): row r handles Gaussian vis_ids[r]; its 2D
// gradients are row r of the 2D gradient planes and its gradients go to row
// r of the output planes (leading dimension ldo for both), so nothing is
// written for Gaussians off the list.  Otherwise row r is Gaussian r and
// ldo = ld.
template <int DEG, bool kPacked>
__global__ __launch_bounds__(256) void project_bwd_kernel(
    int64_t N, int64_t ld, const uint32_t* __restrict__ vis_ids, int64_t ldo,
    const float* __restrict__ means,
    const float* __restrict__ scales, const float* __restrict__ quats,
    const float* __restrict__ sh, Cam cam, Settings st,
    const int32_t* __restrict__ radii, const float* __restrict__ g_m2,
    const float* __restrict__ g_con, const float* __restrict__ g_col,
    float* __restrict__ o_means, float* __restrict__ o_scales, float* __restrict__ o_quats,
    float* __restrict__ o_sh, int accumulate) {
  constexpr int K = (DEG + 1) * (DEG + 1);
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= N) return;
  const int64_t i = kPacked ? (int64_t)vis_ids[r] : r;
  const bool vis = radii[i] > 0;
  // every load of a visible lane (parameters, its 2D gradients, all 3K SH
  // coefficients) is issued here, ahead of the fp64 chain, so that each lane
  // keeps its whole working set in flight (the kernel runs at two waves per
  // SIMD)
  float pm[3] = {0, 0, 0}, ps[3] = {0, 0, 0}, pq[4] = {1, 0, 0, 0}, shv[3 * K];
  float4 r0 = make_float4(0, 0, 0, 0), r1 = r0;
  float gin[3] = {0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int k = 0; k < 3 * K; ++k) shv[k] = 0.0f;
  if (vis) {
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      pm[k] = means[(int64_t)k * ld + i];
      ps[k] = scales[(int64_t)k * ld + i];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) pq[k] = quats[(int64_t)k * ld + i];
    r0 = make_float4(g_m2[r], g_m2[ldo + r], g_con[r], g_con[ldo + r]);
    r1.x = g_con[2 * ldo + r];
#pragma unroll
    for (int k = 0; k < 3; ++k) gin[k] = g_col[(int64_t)k * ldo + r];
#pragma unroll
    for (int k = 0; k < 3 * K; ++k) shv[k] = sh[(int64_t)k * ld + i];
  }
  // culled Gaussians get zeros (overwrite) or are left alone (accumulate);
  // both kinds of lanes store through the same instructions below, so a
  // cache line of a plane is written once
  const bool store = vis || !accumulate;

  // Phase 1, the SH side (done first so that the 3K SH registers are free
  // before the fp64 geometry chain).
  double d[3] = {0.0, 0.0, 1.0}, iL = 1.0, vterm[3] = {0.0, 0.0, 0.0};
  float gcol[3] = {0.0f, 0.0f, 0.0f};
  if (vis) sh_view<DEG>(cam, pm, shv, st.sh_offset, gin, d, iL, gcol);
  if (store)
    sh_grads<DEG>(
        d, iL, gcol, shv,
        [&](int k, float g) {
          const int64_t p = (int64_t)k * ldo + r;
          o_sh[p] = accumulate ? o_sh[p] + g : g;
        },
        vterm);

  // Phase 2, the geometry chain in fp64.
  float om[3] = {0.0f, 0.0f, 0.0f}, os[3] = {0.0f, 0.0f, 0.0f};
  float oq[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (vis) geom_grads(cam, st, pm, ps, pq, r0, r1, vterm, om, os, oq);
  if (store) {
    for (int k = 0; k < 3; ++k) {
      const int64_t p = (int64_t)k * ldo + r;
      o_means[p] = accumulate ? o_means[p] + om[k] : om[k];
      o_scales[p] = accumulate ? o_scales[p] + os[k] : os[k];
    }
    for (int k = 0; k < 4; ++k) {
      const int64_t p = (int64_t)k * ldo + r;
      o_quats[p] = accumulate ? o_quats[p] + oq[k] : oq[k];
    }
  }
}

// Batched form: Gaussian r seen by cameras 0 .. ncams-1 (radii [c][ld], 2D
// gradient planes [c][P][ld]); the outputs are the sums over the cameras, in
// camera order, with the same fp32 additions as ncams single-camera calls
// with accumulate (the first overwriting unless `accumulate`).  The sums
// stay in registers and are written once.  Two passes over the cameras keep
// the register set of each side apart: the SH side for every camera first
// (its view-direction terms parked in LDS, three doubles per camera and
// lane), then the geometry chain for every camera.  -0.0f starts a sum:
// adding it leaves every value's bits unchanged.  With o_opac, the
// per-camera opacity gradients g_op [c][ld] are summed the same way.
template <int DEG>
__global__ __launch_bounds__(256) void project_bwd_batched_kernel(
    int64_t N, int64_t ld, const float* __restrict__ means, const float* __restrict__ scales,
    const float* __restrict__ quats, const float* __restrict__ sh, CamBatch cams, int ncams,
    Settings st, const int32_t* __restrict__ radii, const float* __restrict__ g_m2,
    const float* __restrict__ g_con, const float* __restrict__ g_op,
    const float* __restrict__ g_col, float* __restrict__ o_means,
    float* __restrict__ o_scales, float* __restrict__ o_quats, float* __restrict__ o_opac,
    float* __restrict__ o_sh, int accumulate) {
  constexpr int K = (DEG + 1) * (DEG + 1);
  extern __shared__ double s_vterm[];  // [ncams][3][256]
  const int t = threadIdx.x;
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + t;
  if (r >= N) return;
  bool anyvis = false;
  for (int c = 0; c < ncams; ++c) anyvis |= radii[(int64_t)c * ld + r] > 0;
  if (accumulate && !anyvis) return;  // nothing to add
  float pm[3] = {0, 0, 0}, ps[3] = {0, 0, 0}, pq[4] = {1, 0, 0, 0}, shv[3 * K];
#pragma unroll
  for (int k = 0; k < 3 * K; ++k) shv[k] = 0.0f;
  if (anyvis) {
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      pm[k] = means[(int64_t)k * ld + r];
      ps[k] = scales[(int64_t)k * ld + r];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) pq[k] = quats[(int64_t)k * ld + r];
#pragma unroll
    for (int k = 0; k < 3 * K; ++k) shv[k] = sh[(int64_t)k * ld + r];
  }

  // pass 1: the SH side of every camera
  {
    float a_sh[3 * K];
#pragma unroll
    for (int k = 0; k < 3 * K; ++k) a_sh[k] = accumulate ? o_sh[(int64_t)k * ld + r] : -0.0f;
    for (int c = 0; c < ncams; ++c) {
      const bool vis = radii[(int64_t)c * ld + r] > 0;
      // a camera adds where it sees the Gaussian; the first one of an
      // overwriting call also stands for the zeros a culled lane writes
      const bool store = vis || (c == 0 && !accumulate);
      double d[3] = {0.0, 0.0, 1.0}, iL = 1.0, vterm[3] = {0.0, 0.0, 0.0};
      float gcol[3] = {0.0f, 0.0f, 0.0f};
      if (vis) {
        const float* gc = g_col + (int64_t)c * 3 * ld + r;
        const float gin[3] = {gc[0], gc[ld], gc[2 * ld]};
        sh_view<DEG>(cams.c[c], pm, shv, st.sh_offset, gin, d, iL, gcol);
      }
      if (store)
        sh_grads<DEG>(d, iL, gcol, shv, [&](int k, float g) { a_sh[k] += g; }, vterm);
      for (int e = 0; e < 3; ++e) s_vterm[(c * 3 + e) * 256 + t] = vterm[e];
    }
#pragma unroll
    for (int k = 0; k < 3 * K; ++k) o_sh[(int64_t)k * ld + r] = a_sh[k];
  }

  // pass 2: the geometry chain of every camera
  float a_m[3], a_s[3], a_q[4], a_o;
  for (int k = 0; k < 3; ++k) {
    a_m[k] = accumulate ? o_means[(int64_t)k * ld + r] : -0.0f;
    a_s[k] = accumulate ? o_scales[(int64_t)k * ld + r] : -0.0f;
  }
  for (int k = 0; k < 4; ++k) a_q[k] = accumulate ? o_quats[(int64_t)k * ld + r] : -0.0f;
  a_o = (o_opac && accumulate) ? o_opac[r] : -0.0f;
  for (int c = 0; c < ncams; ++c) {
    const bool vis = radii[(int64_t)c * ld + r] > 0;
    const bool store = vis || (c == 0 && !accumulate);
    float om[3] = {0.0f, 0.0f, 0.0f}, os[3] = {0.0f, 0.0f, 0.0f};
    float oq[4] = {0.0f, 0.0f, 0.0f, 0.0f}, oo = 0.0f;
    if (vis) {
      const float* gm = g_m2 + (int64_t)c * 2 * ld + r;
      const float* gn = g_con + (int64_t)c * 3 * ld + r;
      const float4 r0 = make_float4(gm[0], gm[ld], gn[0], gn[ld]);
      const float4 r1 = make_float4(gn[2 * ld], 0.0f, 0.0f, 0.0f);
      double vterm[3];
      for (int e = 0; e < 3; ++e) vterm[e] = s_vterm[(c * 3 + e) * 256 + t];
      if (o_opac) oo = g_op[(int64_t)c * ld + r];
      geom_grads(cams.c[c], st, pm, ps, pq, r0, r1, vterm, om, os, oq);
    }
    if (store) {
      for (int k = 0; k < 3; ++k) {
        a_m[k] += om[k];
        a_s[k] += os[k];
      }
      for (int k = 0; k < 4; ++k) a_q[k] += oq[k];
      a_o += oo;
    }
  }
  for (int k = 0; k < 3; ++k) {
    o_means[(int64_t)k * ld + r] = a_m[k];
    o_scales[(int64_t)k * ld + r] = a_s[k];
  }
  for (int k = 0; k < 4; ++k) o_quats[(int64_t)k * ld + r] = a_q[k];
  if (o_opac) o_opac[r] = a_o;
}

}  // namespace gs

// One camera (ncams = 1: rows 0 .. N-1 written) or a batch of ncams
// cameras (outputs [c][...], rows N .. ld-1 padded).
extern "C" hipError_t gs_launch_project_fwd(int64_t N, int64_t ld, int deg, const float* means,
                                            const float* scales, const float* quats,
                                            const float* sh, int ncams, const gs::Cam* cams,
                                            const gs::Settings& st, float* means2d,
                                            float* conics, float* chol, float* depths,
                                            int32_t* radii, float* colors, uint32_t* tiles,
                                            hipStream_t stream) {
  const int64_t rows = ncams > 1 ? ld : N;
  if (rows == 0) return hipSuccess;
  gs::CamBatch cb;
  for (int c = 0; c < ncams; ++c) cb.c[c] = cams[c];
  const dim3 grid((unsigned)((rows + 255) / 256), (unsigned)ncams);
#define GS_PFWD(D)                                                                        \
  hipLaunchKernelGGL(gs::project_fwd_kernel<D>, grid, dim3(256), 0, stream, N, rows, ld,    \
                     means, scales, quats, sh, cb, st, means2d, conics, chol, depths, radii, \
                     colors, tiles)
  switch (deg) {
    case 0: GS_PFWD(0); break;
    case 1: GS_PFWD(1); break;
    case 2: GS_PFWD(2); break;
    default: GS_PFWD(3); break;
  }
#undef GS_PFWD
  return hipGetLastError();
}

// vis_ids NULL: N Gaussians, 2D gradients and outputs with leading dimension
// ld.  Otherwise N rows of the packed list vis_ids, 2D gradients and outputs
// with leading dimension ldo.  ncams > 1: a batch of cameras (dense rows
// only, 2D gradients [c][P][ld]), summed into the outputs; o_opac (batch
// only, optional) receives the sum of the per-camera opacity gradients g.op.
extern "C" hipError_t gs_launch_project_bwd(int64_t N, int64_t ld, const uint32_t* vis_ids,
                                            int64_t ldo, int deg, const float* means,
                                            const float* scales, const float* quats,
                                            const float* sh, int ncams, const gs::Cam* cams,
                                            const gs::Settings& st, const int32_t* radii,
                                            const gs::Grad2D& g, float* o_means,
                                            float* o_scales, float* o_quats, float* o_opac,
                                            float* o_sh, int accumulate, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  gs::CamBatch cb;
  for (int c = 0; c < ncams; ++c) cb.c[c] = cams[c];
  const int64_t blocks = (N + 255) / 256;
  const size_t vterm_lds = sizeof(double) * 3 * 256 * (size_t)ncams;
#define GS_PBWD(D, PK)                                                                    \
  hipLaunchKernelGGL((gs::project_bwd_kernel<D, PK>), dim3((unsigned)blocks), dim3(256), 0,  \
                     stream, N, ld, vis_ids, PK ? ldo : ld, means, scales, quats, sh,       \
                     cams[0], st, radii, g.m2, g.con, g.col, o_means, o_scales, o_quats,    \
                     o_sh, accumulate)
#define GS_PBWD_B(D)                                                                       \
  hipLaunchKernelGGL(gs::project_bwd_batched_kernel<D>, dim3((unsigned)blocks), dim3(256),    \
                     vterm_lds, stream, N, ld, means, scales, quats, sh, cb, ncams, st,      \
                     radii, g.m2, g.con, g.op, g.col, o_means, o_scales, o_quats, o_opac,    \
                     o_sh, accumulate)
#define GS_PBWD2(D)                     \
  if (ncams > 1) GS_PBWD_B(D);          \
  else if (vis_ids) GS_PBWD(D, true);   \
  else GS_PBWD(D, false)
  switch (deg) {
    case 0: GS_PBWD2(0); break;
    case 1: GS_PBWD2(1); break;
    case 2: GS_PBWD2(2); break;
    default: GS_PBWD2(3); break;
  }
#undef GS_PBWD2
#undef GS_PBWD_B
#undef GS_PBWD
  return hipGetLastError();
}
