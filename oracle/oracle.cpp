/*
 * oracle.cpp — plain CPU oracle of the differentiable tile rasterizer of 3D
 * Gaussian Splatting.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the slow, obviously-correct reference
 * the HIP path is checked against; it shares no source with that path and
 * must only be loaded by the tests, the smoke check and the benchmark's CPU
 * baseline.  Build: g++ -O2 -ffp-contract=off -fopenmp (no fast-math): the
 * fp32 key path relies on IEEE single arithmetic with correctly rounded
 * division and square root and no fused multiply-add.
 *
 * Sources on the pages (none prints a formula; everything below the stage
 * level is the textbook EWA-splatting / 3DGS reading):
 *   - three stages: 3D transform (R, t, scale, rot) -> depth and screen
 *     projection -> differentiable alpha blending: gsplat guide
 *     (lmnt.cn/news/262699) §2.1;
 *   - covariance built from scaling and rotation: Moore Threads MUSA article
 *     (qwbw.cn/news/278220) §3.3;
 *   - primitive = position, covariance, opacity, SH colour: 3DGS deployment
 *     guide (hmyw.cn/news/140031) §1; MUSA article §2.1;
 *   - quaternion (w,x,y,z) with identity [1,0,0,0], opacity = sigmoid(logit),
 *     scale = exp(log-scale): gsplat guide §3.3 (the activations stay with
 *     the caller; this oracle takes activated values);
 *   - world-to-camera view and intrinsics [fx, fy, cx, cy]: gsplat guide §3.3;
 *   - background colour choice: 3DGS deployment guide §3 (white_background);
 *   - a separately callable backward that accumulates per-Gaussian
 *     gradients: gsplat guide §2.2; deployment guide §2.1; MUSA article §2.1.
 *
 * Parity unpinned by the pages: they print no worked example, so every pin of
 * this oracle is mathematical (closed forms, invariants, brute force, finite
 * differences, dual-number directional derivatives); see tests/.
 */
#include "oracle.h"

#include <omp.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <utility>
#include <vector>

namespace {

/* ------------------------------------------------------------------------ */
/* Forward-mode dual numbers (value, tangent) for exact directional          */
/* derivatives.                                                               */
/* ------------------------------------------------------------------------ */
struct Dual {
  double v, d;
  Dual() : v(0), d(0) {}
  Dual(double x) : v(x), d(0) {}
  Dual(double x, double dx) : v(x), d(dx) {}
};
inline Dual operator+(Dual a, Dual b) { return Dual(a.v + b.v, a.d + b.d); }
inline Dual operator-(Dual a, Dual b) { return Dual(a.v - b.v, a.d - b.d); }
inline Dual operator-(Dual a) { return Dual(-a.v, -a.d); }
inline Dual operator*(Dual a, Dual b) { return Dual(a.v * b.v, a.d * b.v + a.v * b.d); }
inline Dual operator/(Dual a, Dual b) {
  return Dual(a.v / b.v, (a.d * b.v - a.v * b.d) / (b.v * b.v));
}
inline bool operator<(Dual a, Dual b) { return a.v < b.v; }
inline bool operator>(Dual a, Dual b) { return a.v > b.v; }
inline bool operator<=(Dual a, Dual b) { return a.v <= b.v; }
inline bool operator>=(Dual a, Dual b) { return a.v >= b.v; }

inline double val(float x) { return x; }
inline double val(double x) { return x; }
inline double val(Dual x) { return x.v; }

inline float s_sqrt(float x) { return std::sqrt(x); }
inline double s_sqrt(double x) { return std::sqrt(x); }
inline Dual s_sqrt(Dual x) {
  double r = std::sqrt(x.v);
  return Dual(r, x.d / (2.0 * r));
}
inline double s_exp(double x) { return std::exp(x); }
inline Dual s_exp(Dual x) {
  double e = std::exp(x.v);
  return Dual(e, e * x.d);
}
inline bool s_finite(float x) { return std::isfinite(x); }
inline bool s_finite(double x) { return std::isfinite(x); }
inline bool s_finite(Dual x) { return std::isfinite(x.v); }
/* min/max return the selected operand, so the tangent follows the branch */
template <class T> inline T s_min(T a, T b) { return (b < a) ? b : a; }
template <class T> inline T s_max(T a, T b) { return (a < b) ? b : a; }

inline uint32_t f32_bits(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return u;
}

constexpr int kTile = 16;

inline int grid_x(int W) { return (W + kTile - 1) / kTile; }
inline int grid_y(int H) { return (H + kTile - 1) / kTile; }

/* Camera in scalar type T (fp32 key path uses the camera's fp32 values). */
template <class T> struct Cam {
  T R[9], t[3], fx, fy, cx, cy, near_p, far_p;
  int W, H;
};
template <class T> Cam<T> cam_as(const orc_camera& c) {
  Cam<T> o;
  for (int i = 0; i < 9; ++i) o.R[i] = T(c.R[i]);
  for (int i = 0; i < 3; ++i) o.t[i] = T(c.t[i]);
  o.fx = T(c.fx); o.fy = T(c.fy); o.cx = T(c.cx); o.cy = T(c.cy);
  o.near_p = T(c.near_plane); o.far_p = T(c.far_plane);
  o.W = c.width; o.H = c.height;
  return o;
}
template <> Cam<float> cam_as<float>(const orc_camera& c) {
  Cam<float> o;
  for (int i = 0; i < 9; ++i) o.R[i] = (float)c.R[i];
  for (int i = 0; i < 3; ++i) o.t[i] = (float)c.t[i];
  o.fx = (float)c.fx; o.fy = (float)c.fy; o.cx = (float)c.cx; o.cy = (float)c.cy;
  o.near_p = (float)c.near_plane; o.far_p = (float)c.far_plane;
  o.W = c.width; o.H = c.height;
  return o;
}

/* ------------------------------------------------------------------------ */
/* Rotation from a quaternion (w,x,y,z) and the 3D covariance               */
/* Sigma = R S S^T R^T (MUSA article §3.3: covariance from scaling and      */
/* rotation; gsplat guide §3.3 for w-first order).                          */
/* ------------------------------------------------------------------------ */
template <class T> void rotation_from_unit_quat(T w, T x, T y, T z, T R[9]) {
  const T one = T(1), two = T(2);
  R[0] = one - two * (y * y + z * z);
  R[1] = two * (x * y - w * z);
  R[2] = two * (x * z + w * y);
  R[3] = two * (x * y + w * z);
  R[4] = one - two * (x * x + z * z);
  R[5] = two * (y * z - w * x);
  R[6] = two * (x * z - w * y);
  R[7] = two * (y * z + w * x);
  R[8] = one - two * (x * x + y * y);
}

/* Sigma = M M^T with M = R diag(s); entries summed left to right. */
template <class T> void cov3d_from(const T R[9], const T s[3], T Sig[9]) {
  T M[9];
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 3; ++j) M[i * 3 + j] = R[i * 3 + j] * s[j];
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 3; ++j)
      Sig[i * 3 + j] = (M[i * 3 + 0] * M[j * 3 + 0] + M[i * 3 + 1] * M[j * 3 + 1]) +
                       M[i * 3 + 2] * M[j * 3 + 2];
}

/* ------------------------------------------------------------------------ */
/* Real spherical harmonics, degree <= 3, ordered (l, m = -l..l).           */
/* Y_l0 = N_l0 P_l(z); for m > 0: Y_lm = sqrt2 N_lm P_l^m(z) cos(m phi) and  */
/* Y_l,-m = sqrt2 N_lm P_l^m(z) sin(m phi), where P_l^m carries the Condon-  */
/* Shortley phase (-1)^m and N_lm = sqrt((2l+1)/(4 pi) (l-m)!/(l+m)!).       */
/* In Cartesian form on the unit sphere: sin^m(theta) cos(m phi) =           */
/* Re((x+iy)^m), sin^m(theta) sin(m phi) = Im((x+iy)^m), and               */
/* P_l^m(z) = (-1)^m (1-z^2)^(m/2) d^m P_l/dz^m.                            */
/* The pages name "SH coefficients" only (deployment guide §1; gauss-splat   */
/* distributed guide); this convention is the reading fixed here.           */
/* ------------------------------------------------------------------------ */
struct Legendre {
  /* coefficient c[l][m][k] of z^k in d^m P_l / dz^m, l,m <= 3 */
  double c[4][5][4];
  Legendre() {
    std::memset(c, 0, sizeof(c));
    double P[4][4] = {{0}};
    P[0][0] = 1.0;
    P[1][1] = 1.0;
    for (int n = 1; n < 3; ++n) { /* (n+1) P_{n+1} = (2n+1) z P_n - n P_{n-1} */
      for (int k = 0; k < 4; ++k) {
        double v = 0.0;
        if (k >= 1) v += (2.0 * n + 1.0) * P[n][k - 1];
        v -= n * P[n - 1][k];
        P[n + 1][k] = v / (n + 1.0);
      }
    }
    for (int l = 0; l < 4; ++l) {
      double cur[4];
      for (int k = 0; k < 4; ++k) cur[k] = P[l][k];
      for (int m = 0; m <= 4; ++m) {
        for (int k = 0; k < 4; ++k) c[l][m][k] = cur[k];
        double nxt[4] = {0, 0, 0, 0};
        for (int k = 1; k < 4; ++k) nxt[k - 1] = k * cur[k];
        for (int k = 0; k < 4; ++k) cur[k] = nxt[k];
      }
    }
  }
};
const Legendre& legendre() {
  static const Legendre L;
  return L;
}
double factorial(int n) {
  double f = 1.0;
  for (int i = 2; i <= n; ++i) f *= i;
  return f;
}
double sh_norm(int l, int m) { /* m >= 0 */
  const double pi = 3.14159265358979323846;
  return std::sqrt((2.0 * l + 1.0) / (4.0 * pi) * factorial(l - m) / factorial(l + m));
}
template <class T> T poly_z(int l, int m, T z) {
  const Legendre& L = legendre();
  T r = T(0);
  for (int k = 3; k >= 0; --k) r = r * z + T(L.c[l][m][k]);
  return r;
}
/* Re/Im of (x + i y)^m */
template <class T> void cpow(T x, T y, int m, T& re, T& im) {
  re = T(1);
  im = T(0);
  for (int i = 0; i < m; ++i) {
    T nr = re * x - im * y;
    T ni = re * y + im * x;
    re = nr;
    im = ni;
  }
}
/* Y[K] at unit direction (x,y,z) */
template <class T> void sh_basis(int deg, T x, T y, T z, T* Y) {
  const double sqrt2 = std::sqrt(2.0);
  int j = 0;
  for (int l = 0; l <= deg; ++l) {
    for (int m = -l; m <= l; ++m, ++j) {
      int am = m < 0 ? -m : m;
      double sign = (am % 2) ? -1.0 : 1.0; /* Condon-Shortley (-1)^m */
      T dz = poly_z(l, am, z);
      if (m == 0) {
        Y[j] = T(sh_norm(l, 0)) * dz;
      } else {
        T re, im;
        cpow(x, y, am, re, im);
        T ang = (m > 0) ? re : im;
        Y[j] = T(sqrt2 * sh_norm(l, am) * sign) * dz * ang;
      }
    }
  }
}
/* dY[K][3]: gradient of the Cartesian polynomial of each Y */
template <class T> void sh_basis_grad(int deg, T x, T y, T z, T* dY) {
  const double sqrt2 = std::sqrt(2.0);
  int j = 0;
  for (int l = 0; l <= deg; ++l) {
    for (int m = -l; m <= l; ++m, ++j) {
      int am = m < 0 ? -m : m;
      double sign = (am % 2) ? -1.0 : 1.0;
      T dz = poly_z(l, am, z);
      T dz1 = poly_z(l, am + 1, z);
      if (m == 0) {
        T c = T(sh_norm(l, 0));
        dY[j * 3 + 0] = T(0.0);
        dY[j * 3 + 1] = T(0.0);
        dY[j * 3 + 2] = c * dz1;
      } else {
        T c = T(sqrt2 * sh_norm(l, am) * sign);
        T re, im, re1, im1;
        cpow(x, y, am, re, im);
        cpow(x, y, am - 1, re1, im1);
        T ang, dang_dx, dang_dy;
        if (m > 0) { /* Re((x+iy)^m) */
          ang = re;
          dang_dx = T(am) * re1;
          dang_dy = T(-am) * im1;
        } else { /* Im((x+iy)^m) */
          ang = im;
          dang_dx = T(am) * im1;
          dang_dy = T(am) * re1;
        }
        dY[j * 3 + 0] = c * dz * dang_dx;
        dY[j * 3 + 1] = c * dz * dang_dy;
        dY[j * 3 + 2] = c * dz1 * ang;
      }
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Projection geometry (steps 1-7): camera transform, cull, covariance, EWA */
/* Jacobian, 2D covariance + dilation, conic, radius, pixel mean, tile rect. */
/* For T = float this is the fp32 key path: every expression is evaluated   */
/* in the order written, in IEEE single precision, without contraction.     */
/* ------------------------------------------------------------------------ */
template <class T> struct Geom {
  bool vis = false;
  T u = T(0), v = T(0), depth = T(0);
  T a = T(0), b = T(0), c = T(0);     /* dilated 2D covariance */
  T A = T(0), B = T(0), C = T(0);     /* conic */
  T L11 = T(0), L21 = T(0), L22 = T(0); /* conic = L L^T, L lower triangular */
  int32_t radius = 0;
  int32_t rect[4] = {0, 0, 0, 0};     /* x0, x1, y0, y1 (exclusive ends) */
  uint32_t ntiles = 0;
  bool clampx = false, clampy = false; /* fov clamp of the Jacobian active */
};

template <class T>
Geom<T> project_geom(const T mean[3], const T scale[3], const T quat[4],
                     const Cam<T>& cam, const orc_settings& st) {
  Geom<T> g;
  for (int i = 0; i < 3; ++i)
    if (!s_finite(mean[i]) || !s_finite(scale[i])) return g;
  for (int i = 0; i < 4; ++i)
    if (!s_finite(quat[i])) return g;

  /* 1. camera space t = R mu + t */
  const T* W = cam.R;
  T tx = ((W[0] * mean[0] + W[1] * mean[1]) + W[2] * mean[2]) + cam.t[0];
  T ty = ((W[3] * mean[0] + W[4] * mean[1]) + W[5] * mean[2]) + cam.t[1];
  T tz = ((W[6] * mean[0] + W[7] * mean[1]) + W[8] * mean[2]) + cam.t[2];
  if (!(tz > cam.near_p && tz < cam.far_p)) return g;
  if (!s_finite(tx) || !s_finite(ty)) return g;

  /* 2. unit quaternion, rotation, Sigma = M M^T */
  T n2 = ((quat[0] * quat[0] + quat[1] * quat[1]) + quat[2] * quat[2]) + quat[3] * quat[3];
  if (!(n2 > T(0)) || !s_finite(n2)) return g;
  T nr = s_sqrt(n2);
  T qw = quat[0] / nr, qx = quat[1] / nr, qy = quat[2] / nr, qz = quat[3] / nr;
  T Rq[9], Sig[9];
  rotation_from_unit_quat(qw, qx, qy, qz, Rq);
  cov3d_from(Rq, scale, Sig);

  /* 3. EWA Jacobian of the pinhole projection at t (x', y' clamped to
   *    fov_clamp times the half field of view), then Sigma2D = T Sigma T^T
   *    with T = J W. */
  T txz = tx / tz, tyz = ty / tz;
  T tanx = (T(0.5f) * T((float)cam.W)) / cam.fx;
  T tany = (T(0.5f) * T((float)cam.H)) / cam.fy;
  T limx = T(st.fov_clamp) * tanx;
  T limy = T(st.fov_clamp) * tany;
  T cxz = s_min(limx, s_max(-limx, txz));
  T cyz = s_min(limy, s_max(-limy, tyz));
  g.clampx = (txz > limx) || (txz < -limx);
  g.clampy = (tyz > limy) || (tyz < -limy);
  T xc = cxz * tz, yc = cyz * tz;
  T tz2 = tz * tz;
  T J00 = cam.fx / tz;
  T J02 = -((cam.fx * xc) / tz2);
  T J11 = cam.fy / tz;
  T J12 = -((cam.fy * yc) / tz2);
  T Tm[6];
  for (int j = 0; j < 3; ++j) {
    Tm[0 * 3 + j] = J00 * W[0 * 3 + j] + J02 * W[2 * 3 + j];
    Tm[1 * 3 + j] = J11 * W[1 * 3 + j] + J12 * W[2 * 3 + j];
  }
  T U[6];
  for (int a = 0; a < 2; ++a)
    for (int j = 0; j < 3; ++j)
      U[a * 3 + j] = (Tm[a * 3 + 0] * Sig[0 * 3 + j] + Tm[a * 3 + 1] * Sig[1 * 3 + j]) +
                     Tm[a * 3 + 2] * Sig[2 * 3 + j];
  T c00 = (U[0] * Tm[0] + U[1] * Tm[1]) + U[2] * Tm[2];
  T c01 = (U[0] * Tm[3] + U[1] * Tm[4]) + U[2] * Tm[5];
  T c11 = (U[3] * Tm[3] + U[4] * Tm[4]) + U[5] * Tm[5];
  T a = c00 + T(st.eps2d);
  T b = c01;
  T c = c11 + T(st.eps2d);

  /* 4. conic = inverse of the dilated 2D covariance (which must be positive
   *    definite), and its Cholesky factor L (conic = L L^T), with which the
   *    quadratic form is the completed square
   *      q = (L11 dx + L21 dy)^2 + (L22 dy)^2,
   *    L11 = sqrt(A), L21 = B / L11, L22 = 1 / sqrt(c). */
  T det = a * c - b * b;
  if (!(det > T(0)) || !s_finite(det) || !(a > T(0))) return g;
  T A = c / det;
  T B = -(b / det);
  T C = a / det;
  T L11 = s_sqrt(A);
  T L21 = B / L11;
  T L22 = T(1) / s_sqrt(c);

  /* 5. radius = ceil(3 sqrt(lambda_max)) */
  T mid = T(0.5f) * (a + c);
  T disc = mid * mid - det;
  T lam = mid + s_sqrt(s_max(disc, T(0)));
  if (!s_finite(lam)) return g;
  double rf = std::ceil(val(T(3.0f) * s_sqrt(lam)));
  if (rf > 16777216.0) rf = 16777216.0;
  int32_t radius = (int32_t)rf;
  if (radius <= 0) return g;

  /* 6. pixel mean (pixel (px,py) has its centre at (px+0.5, py+0.5)) */
  T u = cam.fx * txz + cam.cx;
  T v = cam.fy * tyz + cam.cy;
  if (!s_finite(u) || !s_finite(v)) return g;

  /* 7. tile rect of the square [u-r, u+r] x [v-r, v+r] */
  const int gx = grid_x(cam.W), gy = grid_y(cam.H);
  T rT = T((float)radius);
  double fx0 = std::floor(val((u - rT) / T(16.0f)));
  double fx1 = std::floor(val((u + rT) / T(16.0f))) + 1.0;
  double fy0 = std::floor(val((v - rT) / T(16.0f)));
  double fy1 = std::floor(val((v + rT) / T(16.0f))) + 1.0;
  auto clampi = [](double f, int hi) {
    return (int32_t)std::min(std::max(f, 0.0), (double)hi);
  };
  int32_t x0 = clampi(fx0, gx), x1 = clampi(fx1, gx);
  int32_t y0 = clampi(fy0, gy), y1 = clampi(fy1, gy);
  if (x1 <= x0 || y1 <= y0) return g;

  g.vis = true;
  g.u = u; g.v = v; g.depth = tz;
  g.a = a; g.b = b; g.c = c;
  g.A = A; g.B = B; g.C = C;
  g.L11 = L11; g.L21 = L21; g.L22 = L22;
  g.radius = radius;
  g.rect[0] = x0; g.rect[1] = x1; g.rect[2] = y0; g.rect[3] = y1;
  g.ntiles = (uint32_t)(x1 - x0) * (uint32_t)(y1 - y0);
  return g;
}

/* Step 8: view-dependent colour, clamped at zero. */
template <class T>
void sh_color(int deg, const T mean[3], const T* sh, const T campos[3],
              double sh_offset, T out[3], bool clamped[3]) {
  T dx = mean[0] - campos[0], dy = mean[1] - campos[1], dz = mean[2] - campos[2];
  T L = s_sqrt(dx * dx + dy * dy + dz * dz);
  T x = dx / L, y = dy / L, z = dz / L;
  int K = (deg + 1) * (deg + 1);
  T Y[16];
  sh_basis(deg, x, y, z, Y);
  for (int ch = 0; ch < 3; ++ch) {
    T s = T(sh_offset);
    for (int j = 0; j < K; ++j) s = s + Y[j] * sh[j * 3 + ch];
    clamped[ch] = s < T(0);
    out[ch] = clamped[ch] ? T(0) : s;
  }
}

template <class T> void camera_center(const Cam<T>& cam, T c[3]) {
  for (int j = 0; j < 3; ++j)
    c[j] = -(cam.R[0 * 3 + j] * cam.t[0] + cam.R[1 * 3 + j] * cam.t[1] + cam.R[2 * 3 + j] * cam.t[2]);
}

/* ------------------------------------------------------------------------ */
/* Steps 9-11: duplicate every visible Gaussian once per touched tile in    */
/* instance order (Gaussian index ascending, tiles row-major inside its      */
/* rect), stable-sort by (tile, depth), and extract per-tile ranges.         */
/* ------------------------------------------------------------------------ */
struct Inst {
  uint32_t tile;
  double depth;
  uint32_t id;
  uint64_t key; /* fp32 path only */
};

std::vector<Inst> build_instances(int64_t N, const std::vector<int32_t>& rects,
                                  const std::vector<uint8_t>& vis,
                                  const std::vector<double>& depth,
                                  const std::vector<uint32_t>& dbits, int gx) {
  std::vector<Inst> out;
  for (int64_t i = 0; i < N; ++i) {
    if (!vis[i]) continue;
    const int32_t* r = &rects[i * 4];
    for (int ty = r[2]; ty < r[3]; ++ty)
      for (int tx = r[0]; tx < r[1]; ++tx) {
        Inst in;
        in.tile = (uint32_t)(ty * gx + tx);
        in.depth = depth[i];
        in.id = (uint32_t)i;
        in.key = ((uint64_t)in.tile << 32) | (uint64_t)(dbits.empty() ? 0u : dbits[i]);
        out.push_back(in);
      }
  }
  std::stable_sort(out.begin(), out.end(), [](const Inst& a, const Inst& b) {
    if (a.tile != b.tile) return a.tile < b.tile;
    return a.depth < b.depth;
  });
  return out;
}

void fill_ranges(const std::vector<Inst>& inst, int T, uint32_t* ranges) {
  for (int t = 0; t < T; ++t) ranges[2 * t] = ranges[2 * t + 1] = 0;
  size_t M = inst.size();
  for (size_t m = 0; m < M; ++m) {
    uint32_t t = inst[m].tile;
    if (m == 0 || inst[m - 1].tile != t) ranges[2 * t] = (uint32_t)m;
    if (m + 1 == M || inst[m + 1].tile != t) ranges[2 * t + 1] = (uint32_t)(m + 1);
  }
}

/* ------------------------------------------------------------------------ */
/* Step 12: per-pixel front-to-back compositing.                            */
/* ------------------------------------------------------------------------ */
enum PairOutcome : uint8_t { SKIP_ALPHA = 2, STOP = 3, BLEND = 4, BLEND_CLAMPED = 5 };

struct Layer { /* one blended entry of a pixel (fp64 backward) */
  uint32_t pos; /* position in the sorted list */
  uint32_t id;
  double alpha, T, G, dx, dy;
  bool clamped;
};

inline uint64_t mix(uint64_t h, uint64_t x) {
  h ^= x + 0x9e3779b97f4a7c15ULL + (h << 6) + (h >> 2);
  return h;
}

template <class T> struct PixelOut {
  T color[3];
  T finalT, depth;
  uint32_t last;
  double margin;
  uint64_t sig;
};

inline double rel_dist(double x, double th) { return std::fabs(x - th) / std::fabs(th); }

/* Composite one pixel of tile [start, end). Optionally records the blended
 * layers (for the backward). */
template <class T>
PixelOut<T> composite_pixel(int px, int py, uint32_t start, uint32_t end,
                            const uint32_t* ids, const T* means2d, const T* chol,
                            const T* opac, const T* colors, const T* depths,
                            const double* bg, const orc_settings& st,
                            std::vector<Layer>* layers) {
  const double a_min = st.alpha_min, a_max = st.alpha_max, T_min = st.T_min;
  PixelOut<T> o;
  T Tr = T(1);
  T Cc[3] = {T(0), T(0), T(0)};
  T D = T(0);
  uint32_t last = 0;
  double margin = std::numeric_limits<double>::infinity();
  uint64_t sig = 1469598103934665603ULL;
  const double pcx = px + 0.5, pcy = py + 0.5;
  for (uint32_t j = start; j < end; ++j) {
    uint32_t i = ids[j];
    T dx = T(pcx) - means2d[2 * i + 0];
    T dy = T(pcy) - means2d[2 * i + 1];
    /* q = [dx dy] conic [dx dy]^T as the completed square (never negative) */
    T e1 = chol[3 * i + 0] * dx + chol[3 * i + 1] * dy;
    T e2 = chol[3 * i + 2] * dy;
    T q = e1 * e1 + e2 * e2;
    T G = s_exp(T(-0.5) * q);
    T oG = opac[i] * G;
    bool clamped = oG > T(a_max);
    T alpha = clamped ? T(a_max) : oG;
    margin = std::min(margin, rel_dist(val(oG), a_max));
    margin = std::min(margin, rel_dist(val(alpha), a_min));
    if (alpha < T(a_min)) {
      sig = mix(sig, (uint64_t)(j - start) * 8 + SKIP_ALPHA);
      continue;
    }
    T Tn = Tr * (T(1) - alpha);
    margin = std::min(margin, rel_dist(val(Tn), T_min));
    if (Tn < T(T_min)) {
      sig = mix(sig, (uint64_t)(j - start) * 8 + STOP);
      break;
    }
    for (int ch = 0; ch < 3; ++ch) Cc[ch] = Cc[ch] + colors[3 * i + ch] * alpha * Tr;
    D = D + depths[i] * alpha * Tr;
    if (layers)
      layers->push_back(Layer{j, i, val(alpha), val(Tr), val(G), val(dx), val(dy), clamped});
    Tr = Tn;
    last = j - start + 1;
    sig = mix(sig, (uint64_t)(j - start) * 8 + (clamped ? BLEND_CLAMPED : BLEND));
  }
  for (int ch = 0; ch < 3; ++ch) o.color[ch] = Cc[ch] + Tr * T(bg[ch]);
  o.finalT = Tr;
  o.depth = D;
  o.last = last;
  o.margin = margin;
  o.sig = sig;
  return o;
}

template <class T>
uint64_t composite_image(int W, int H, const uint32_t* ranges, const uint32_t* ids,
                         const T* means2d, const T* chol, const T* opac,
                         const T* colors, const T* depths, const double* bg,
                         const orc_settings& st, T* image, T* finalT, uint32_t* last,
                         T* out_depth, T* out_alpha, double* margin) {
  const int gx = grid_x(W), gy = grid_y(H), NT = gx * gy;
  std::vector<uint64_t> tile_sig(NT, 0);
#pragma omp parallel for schedule(dynamic, 4)
  for (int t = 0; t < NT; ++t) {
    int tx = t % gx, ty = t / gx;
    uint64_t h = 0;
    for (int py = ty * kTile; py < std::min(H, (ty + 1) * kTile); ++py)
      for (int px = tx * kTile; px < std::min(W, (tx + 1) * kTile); ++px) {
        PixelOut<T> o = composite_pixel<T>(px, py, ranges[2 * t], ranges[2 * t + 1], ids,
                                           means2d, chol, opac, colors, depths, bg, st,
                                           nullptr);
        size_t p = (size_t)py * W + px;
        if (image)
          for (int ch = 0; ch < 3; ++ch) image[3 * p + ch] = o.color[ch];
        if (finalT) finalT[p] = o.finalT;
        if (last) last[p] = o.last;
        if (out_depth) out_depth[p] = o.depth;
        if (out_alpha) out_alpha[p] = T(1) - o.finalT;
        if (margin) margin[p] = o.margin;
        h = mix(h, o.sig);
      }
    tile_sig[t] = h;
  }
  uint64_t sig = 0;
  for (int t = 0; t < NT; ++t) sig = mix(sig, tile_sig[t]);
  return sig;
}

/* ------------------------------------------------------------------------ */
/* Step 13a: compositing backward (fp64).  For the blended layers k=1..n of  */
/* a pixel, C = sum_k c_k a_k T_k + T_{n+1} bg, T_{k+1} = T_k (1 - a_k), so  */
/*   dC/dc_k = a_k T_k,  dC/da_k = c_k T_k - R_{k+1} / (1 - a_k),           */
/* with R_{k+1} = sum_{j>k} c_j a_j T_j + T_{n+1} bg.                        */
/* ------------------------------------------------------------------------ */
void composite_bwd_impl(int W, int H, int64_t N, const uint32_t* ranges,
                        const uint32_t* ids, const double* means2d, const double* chol,
                        const double* conics, const double* opac,
                        const double* colors, const double* bg,
                        const orc_settings& st, const double* dLdI,
                        double* g_m2, double* g_con, double* g_op, double* g_col,
                        double* abs_sum) {
  const int gx = grid_x(W), gy = grid_y(H), NT = gx * gy;
  int64_t Mtot = 0;
  for (int t = 0; t < NT; ++t) Mtot = std::max<int64_t>(Mtot, ranges[2 * t + 1]);
  /* per-instance partial sums: tile t's list positions are disjoint, so no
   * two threads write the same slot; reduced per Gaussian in list order. */
  std::vector<double> contrib((size_t)Mtot * 9, 0.0), contrib_abs;
  if (abs_sum) contrib_abs.assign((size_t)Mtot * 9, 0.0);
#pragma omp parallel for schedule(dynamic, 4)
  for (int t = 0; t < NT; ++t) {
    int tx = t % gx, ty = t / gx;
    uint32_t start = ranges[2 * t], end = ranges[2 * t + 1];
    std::vector<Layer> layers;
    for (int py = ty * kTile; py < std::min(H, (ty + 1) * kTile); ++py)
      for (int px = tx * kTile; px < std::min(W, (tx + 1) * kTile); ++px) {
        layers.clear();
        PixelOut<double> o = composite_pixel<double>(px, py, start, end, ids, means2d, chol,
                                                     opac, colors, colors /*unused*/, bg, st,
                                                     &layers);
        size_t p = (size_t)py * W + px;
        const double* g = &dLdI[3 * p];
        const size_t n = layers.size();
        double R[3];
        for (int ch = 0; ch < 3; ++ch) R[ch] = o.finalT * bg[ch];
        for (size_t kk = n; kk-- > 0;) {
          const Layer& Lk = layers[kk];
          const uint32_t i = Lk.id;
          double dL_da = 0.0;
          double gc[3];
          for (int ch = 0; ch < 3; ++ch) {
            double c = colors[3 * i + ch];
            double dC_da = c * Lk.T - R[ch] / (1.0 - Lk.alpha);
            dL_da += g[ch] * dC_da;
            gc[ch] = g[ch] * Lk.alpha * Lk.T;
            R[ch] += c * Lk.alpha * Lk.T;
          }
          double f[9] = {0, 0, 0, 0, 0, 0, gc[0], gc[1], gc[2]};
          if (!Lk.clamped) {
            double dL_dq = dL_da * (-0.5 * Lk.alpha);
            double A = conics[3 * i], B = conics[3 * i + 1], C = conics[3 * i + 2];
            double dx = Lk.dx, dy = Lk.dy;
            f[0] = dL_dq * (-2.0 * (A * dx + B * dy));  /* u: dq/du */
            f[1] = dL_dq * (-2.0 * (B * dx + C * dy));  /* v */
            f[2] = dL_dq * (dx * dx);                   /* A */
            f[3] = dL_dq * (2.0 * dx * dy);             /* B */
            f[4] = dL_dq * (dy * dy);                   /* C */
            f[5] = dL_da * Lk.G;                        /* opacity */
          }
          size_t slot = (size_t)Lk.pos * 9;
          for (int q = 0; q < 9; ++q) {
            contrib[slot + q] += f[q];
            if (abs_sum) contrib_abs[slot + q] += std::fabs(f[q]);
          }
        }
      }
  }
  std::fill(g_m2, g_m2 + 2 * N, 0.0);
  std::fill(g_con, g_con + 3 * N, 0.0);
  std::fill(g_op, g_op + N, 0.0);
  std::fill(g_col, g_col + 3 * N, 0.0);
  if (abs_sum) std::fill(abs_sum, abs_sum + 9 * N, 0.0);
  for (int64_t m = 0; m < Mtot; ++m) {
    uint32_t i = ids[m];
    const double* f = &contrib[(size_t)m * 9];
    g_m2[2 * i] += f[0];
    g_m2[2 * i + 1] += f[1];
    for (int q = 0; q < 3; ++q) g_con[3 * i + q] += f[2 + q];
    g_op[i] += f[5];
    for (int q = 0; q < 3; ++q) g_col[3 * i + q] += f[6 + q];
    if (abs_sum)
      for (int q = 0; q < 9; ++q) abs_sum[9 * (size_t)i + q] += contrib_abs[(size_t)m * 9 + q];
  }
}

/* ------------------------------------------------------------------------ */
/* Step 13b: projection backward, chain rule from (u, v), the conic and the  */
/* colour to mean, scale, quaternion and SH coefficients.  With every        */
/* discrete decision (visibility, fov clamp, colour clamp) fixed by the      */
/* parameters, it is linear in the 2D gradients it is given.                 */
/* ------------------------------------------------------------------------ */
template <class S>
void project_bwd_one(int deg, const S* mean, const S* scale, const S* quat, const S* sh,
                     const Cam<S>& cam, const orc_settings& st, const S* gm2, const S* gcon,
                     const S* gcol, S* g_mean, S* g_scale, S* g_quat, S* g_sh) {
  const int K = (deg + 1) * (deg + 1);
  const S* W = cam.R;
  S t[3];
  for (int r = 0; r < 3; ++r)
    t[r] = W[r * 3 + 0] * mean[0] + W[r * 3 + 1] * mean[1] + W[r * 3 + 2] * mean[2] + cam.t[r];
  const S tx = t[0], ty = t[1], tz = t[2];
  S n2 = quat[0] * quat[0] + quat[1] * quat[1] + quat[2] * quat[2] + quat[3] * quat[3];
  S nr = s_sqrt(n2);
  S qn[4] = {quat[0] / nr, quat[1] / nr, quat[2] / nr, quat[3] / nr};
  S Rq[9], Sig[9];
  rotation_from_unit_quat(qn[0], qn[1], qn[2], qn[3], Rq);
  cov3d_from(Rq, scale, Sig);

  const S fx = cam.fx, fy = cam.fy;
  const S limx = S((double)st.fov_clamp) * (S(0.5 * cam.W) / fx);
  const S limy = S((double)st.fov_clamp) * (S(0.5 * cam.H) / fy);
  const S txz = tx / tz, tyz = ty / tz;
  const bool clx = txz > limx || txz < -limx;
  const bool cly = tyz > limy || tyz < -limy;
  const S xc = clx ? (txz > S(0) ? limx : -limx) * tz : tx;
  const S yc = cly ? (tyz > S(0) ? limy : -limy) * tz : ty;
  const S J00 = fx / tz, J02 = -fx * xc / (tz * tz);
  const S J11 = fy / tz, J12 = -fy * yc / (tz * tz);
  S Tm[6];
  for (int j = 0; j < 3; ++j) {
    Tm[j] = J00 * W[j] + J02 * W[6 + j];
    Tm[3 + j] = J11 * W[3 + j] + J12 * W[6 + j];
  }
  S ST0[3], ST1[3]; /* Sigma T0^T, Sigma T1^T */
  for (int i = 0; i < 3; ++i) {
    ST0[i] = Sig[i * 3] * Tm[0] + Sig[i * 3 + 1] * Tm[1] + Sig[i * 3 + 2] * Tm[2];
    ST1[i] = Sig[i * 3] * Tm[3] + Sig[i * 3 + 1] * Tm[4] + Sig[i * 3 + 2] * Tm[5];
  }
  S a = Tm[0] * ST0[0] + Tm[1] * ST0[1] + Tm[2] * ST0[2] + S((double)st.eps2d);
  S b = Tm[3] * ST0[0] + Tm[4] * ST0[1] + Tm[5] * ST0[2];
  S c = Tm[3] * ST1[0] + Tm[4] * ST1[1] + Tm[5] * ST1[2] + S((double)st.eps2d);
  S det = a * c - b * b, det2 = det * det;

  /* conic (A,B,C) = (c, -b, a)/det -> (a, b, c) */
  const S gA = gcon[0], gB = gcon[1], gC = gcon[2];
  S ga = gA * (-c * c / det2) + gB * (b * c / det2) + gC * (1.0 / det - a * c / det2);
  S gb = gA * (2.0 * b * c / det2) + gB * (-1.0 / det - 2.0 * b * b / det2) +
              gC * (2.0 * a * b / det2);
  S gc = gA * (1.0 / det - a * c / det2) + gB * (a * b / det2) + gC * (-a * a / det2);

  /* Sigma2D entries: cov00 = T0 S T0^T, cov01 = T0 S T1^T, cov11 = T1 S T1^T */
  S gSig[9];
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 3; ++j)
      gSig[i * 3 + j] = ga * Tm[i] * Tm[j] + gb * Tm[i] * Tm[3 + j] + gc * Tm[3 + i] * Tm[3 + j];
  S gT0[3], gT1[3];
  for (int i = 0; i < 3; ++i) {
    gT0[i] = 2.0 * ga * ST0[i] + gb * ST1[i];
    gT1[i] = gb * ST0[i] + 2.0 * gc * ST1[i];
  }
  S gJ00 = S(0), gJ02 = S(0), gJ11 = S(0), gJ12 = S(0);
  for (int j = 0; j < 3; ++j) {
    gJ00 += gT0[j] * W[j];
    gJ02 += gT0[j] * W[6 + j];
    gJ11 += gT1[j] * W[3 + j];
    gJ12 += gT1[j] * W[6 + j];
  }
  S gt[3] = {S(0), S(0), S(0)};
  gt[2] += gJ00 * (-fx / (tz * tz)) + gJ11 * (-fy / (tz * tz));
  if (clx) {
    S cx_ = txz > S(0) ? limx : -limx;
    gt[2] += gJ02 * (fx * cx_ / (tz * tz));
  } else {
    gt[0] += gJ02 * (-fx / (tz * tz));
    gt[2] += gJ02 * (2.0 * fx * tx / (tz * tz * tz));
  }
  if (cly) {
    S cy_ = tyz > S(0) ? limy : -limy;
    gt[2] += gJ12 * (fy * cy_ / (tz * tz));
  } else {
    gt[1] += gJ12 * (-fy / (tz * tz));
    gt[2] += gJ12 * (2.0 * fy * ty / (tz * tz * tz));
  }
  /* pixel mean u = fx tx/tz + cx, v = fy ty/tz + cy */
  gt[0] += gm2[0] * fx / tz;
  gt[2] += gm2[0] * (-fx * tx / (tz * tz));
  gt[1] += gm2[1] * fy / tz;
  gt[2] += gm2[1] * (-fy * ty / (tz * tz));
  for (int j = 0; j < 3; ++j)
    g_mean[j] = W[j] * gt[0] + W[3 + j] * gt[1] + W[6 + j] * gt[2];

  /* Sigma = M M^T, M = R diag(s) */
  S M[9];
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 3; ++j) M[i * 3 + j] = Rq[i * 3 + j] * scale[j];
  S gM[9];
  for (int i = 0; i < 3; ++i)
    for (int k = 0; k < 3; ++k) {
      S s = S(0.0);
      for (int j = 0; j < 3; ++j) s += (gSig[i * 3 + j] + gSig[j * 3 + i]) * M[j * 3 + k];
      gM[i * 3 + k] = s;
    }
  S gR[9];
  for (int j = 0; j < 3; ++j) {
    S s = S(0.0);
    for (int i = 0; i < 3; ++i) {
      s += gM[i * 3 + j] * Rq[i * 3 + j];
      gR[i * 3 + j] = gM[i * 3 + j] * scale[j];
    }
    g_scale[j] = s;
  }
  const S w = qn[0], x = qn[1], y = qn[2], z = qn[3];
  S gq[4] = {S(0), S(0), S(0), S(0)};
  /* partial derivatives of each rotation entry wrt (w, x, y, z) */
  const S dR[9][4] = {
      {S(0), S(0), -4 * y, -4 * z},          {-2 * z, 2 * y, 2 * x, -2 * w},
      {2 * y, 2 * z, 2 * w, 2 * x},    {2 * z, 2 * y, 2 * x, 2 * w},
      {S(0), -4 * x, S(0), -4 * z},          {-2 * x, -2 * w, 2 * z, 2 * y},
      {-2 * y, 2 * z, -2 * w, 2 * x},  {2 * x, 2 * w, 2 * z, 2 * y},
      {S(0), -4 * x, -4 * y, S(0)}};
  for (int e = 0; e < 9; ++e)
    for (int k = 0; k < 4; ++k) gq[k] += gR[e] * dR[e][k];
  S dot = qn[0] * gq[0] + qn[1] * gq[1] + qn[2] * gq[2] + qn[3] * gq[3];
  for (int k = 0; k < 4; ++k) g_quat[k] = (gq[k] - qn[k] * dot) / nr;

  /* colour -> SH coefficients and view direction */
  S campos[3];
  camera_center(cam, campos);
  S dir[3] = {mean[0] - campos[0], mean[1] - campos[1], mean[2] - campos[2]};
  S L = s_sqrt(dir[0] * dir[0] + dir[1] * dir[1] + dir[2] * dir[2]);
  S d[3] = {dir[0] / L, dir[1] / L, dir[2] / L};
  S Y[16], dY[48];
  sh_basis(deg, d[0], d[1], d[2], Y);
  sh_basis_grad(deg, d[0], d[1], d[2], dY);
  S gd[3] = {S(0), S(0), S(0)};
  for (int ch = 0; ch < 3; ++ch) {
    S raw = S((double)st.sh_offset);
    for (int j = 0; j < K; ++j) raw += Y[j] * sh[j * 3 + ch];
    bool pass = !(raw < S(0.0));
    for (int j = 0; j < K; ++j) {
      g_sh[j * 3 + ch] = pass ? Y[j] * gcol[ch] : S(0.0);
      if (pass)
        for (int e = 0; e < 3; ++e) gd[e] += gcol[ch] * sh[j * 3 + ch] * dY[j * 3 + e];
    }
  }
  S dd = d[0] * gd[0] + d[1] * gd[1] + d[2] * gd[2];
  for (int e = 0; e < 3; ++e) g_mean[e] += (gd[e] - d[e] * dd) / L;
}

/* ------------------------------------------------------------------------ */
/* Full forward + loss in scalar T (double or Dual).                        */
/* ------------------------------------------------------------------------ */
template <class T>
int64_t full_loss(int64_t N, int deg, const std::vector<T>& means, const std::vector<T>& scales,
                  const std::vector<T>& quats, const std::vector<T>& opac,
                  const std::vector<T>& sh, const orc_camera& camd, const orc_settings& st,
                  const double* bg, int loss_kind, const double* target, T& loss,
                  uint64_t& sig, double* image_out) {
  const int K = (deg + 1) * (deg + 1);
  Cam<T> cam = cam_as<T>(camd);
  T campos[3];
  camera_center(cam, campos);
  std::vector<T> m2(2 * N), chol(3 * N), col(3 * N), dep(N);
  std::vector<int32_t> rects(4 * N);
  std::vector<uint8_t> vis(N);
  std::vector<double> depd(N);
  sig = 0;
  for (int64_t i = 0; i < N; ++i) {
    Geom<T> g = project_geom<T>(&means[3 * i], &scales[3 * i], &quats[4 * i], cam, st);
    vis[i] = g.vis;
    sig = mix(sig, g.vis ? (1 + g.rect[0] + 7 * g.rect[1] + 131 * g.rect[2] + 2711 * g.rect[3] +
                            (g.clampx ? 1u << 30 : 0) + (g.clampy ? 1u << 29 : 0))
                         : 0);
    for (int q = 0; q < 4; ++q) rects[4 * i + q] = g.rect[q];
    m2[2 * i] = g.u; m2[2 * i + 1] = g.v;
    chol[3 * i] = g.L11; chol[3 * i + 1] = g.L21; chol[3 * i + 2] = g.L22;
    dep[i] = g.depth;
    depd[i] = val(g.depth);
    if (g.vis) {
      bool cl[3];
      sh_color<T>(deg, &means[3 * i], &sh[(size_t)K * 3 * i], campos, st.sh_offset, &col[3 * i], cl);
      sig = mix(sig, (uint64_t)cl[0] + 2 * cl[1] + 4 * cl[2]);
    }
  }
  const int W = camd.width, H = camd.height;
  const int gx = grid_x(W), gy = grid_y(H), NT = gx * gy;
  std::vector<Inst> inst = build_instances(N, rects, vis, depd, std::vector<uint32_t>(), gx);
  std::vector<uint32_t> ids(inst.size()), ranges(2 * (size_t)NT);
  for (size_t m = 0; m < inst.size(); ++m) ids[m] = inst[m].id;
  fill_ranges(inst, NT, ranges.data());
  for (size_t m = 0; m < inst.size(); ++m) sig = mix(sig, inst[m].id);
  std::vector<T> img(3 * (size_t)W * H);
  uint64_t csig = composite_image<T>(W, H, ranges.data(), ids.data(), m2.data(), chol.data(),
                                     opac.data(), col.data(), dep.data(), bg, st, img.data(),
                                     nullptr, nullptr, nullptr, nullptr, nullptr);
  sig = mix(sig, csig);
  if (image_out)
    for (size_t p = 0; p < img.size(); ++p) image_out[p] = val(img[p]);
  T L = T(0);
  for (size_t p = 0; p < img.size(); ++p) {
    T r = img[p] - T(target[p]);
    if (loss_kind == ORC_LOSS_L2) {
      L = L + r * r;
    } else {
      L = L + ((r < T(0)) ? -r : r);
    }
  }
  loss = L;
  return (int64_t)inst.size();
}

/* Projection backward of every Gaussian (fp64).  Culled Gaussians (radius
 * 0) get zeros. */
template <class S>
void project_bwd_all(int64_t N, int deg, const double* means, const double* scales,
                     const double* quats, const double* sh, const orc_camera& camd,
                     const orc_settings& st, const int32_t* radii, const double* g_means2d,
                     const double* g_conics, const double* g_colors, double* g_means,
                     double* g_scales, double* g_quats, double* g_sh) {
  const int K = (deg + 1) * (deg + 1);
  Cam<S> cam = cam_as<S>(camd);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < N; ++i) {
    double* gm = &g_means[3 * i];
    double* gs = &g_scales[3 * i];
    double* gq = &g_quats[4 * i];
    double* gsh = &g_sh[(size_t)K * 3 * i];
    if (radii[i] <= 0) {
      std::fill(gm, gm + 3, 0.0);
      std::fill(gs, gs + 3, 0.0);
      std::fill(gq, gq + 4, 0.0);
      std::fill(gsh, gsh + 3 * K, 0.0);
      continue;
    }
    S m[3], sc[3], q[4], shv[48], gm2[2], gc[3], gcol[3], om[3], os[3], oq[4], osh[48];
    for (int k = 0; k < 3; ++k) { m[k] = S(means[3 * i + k]); sc[k] = S(scales[3 * i + k]); }
    for (int k = 0; k < 4; ++k) q[k] = S(quats[4 * i + k]);
    for (int k = 0; k < 3 * K; ++k) shv[k] = S(sh[(size_t)K * 3 * i + k]);
    for (int k = 0; k < 2; ++k) gm2[k] = S(g_means2d[2 * i + k]);
    for (int k = 0; k < 3; ++k) {
      gc[k] = S(g_conics[3 * i + k]);
      gcol[k] = S(g_colors[3 * i + k]);
    }
    project_bwd_one(deg, m, sc, q, shv, cam, st, gm2, gc, gcol, om, os, oq, osh);
    for (int k = 0; k < 3; ++k) { gm[k] = val(om[k]); gs[k] = val(os[k]); }
    for (int k = 0; k < 4; ++k) gq[k] = val(oq[k]);
    for (int k = 0; k < 3 * K; ++k) gsh[k] = val(osh[k]);
  }
}

}  // namespace

/* ======================================================================== */
/* C ABI                                                                    */
/* ======================================================================== */
extern "C" {

int orc_project(int mode, int64_t N, int deg, const double* means, const double* scales,
                const double* quats, const double* sh, const orc_camera* camd,
                const orc_settings* st, double* means2d, double* conics, double* chol,
                double* cov2d, double* depths, int32_t* radii, uint32_t* tiles,
                int32_t* rect, double* colors, uint8_t* clamped) {
  const int K = (deg + 1) * (deg + 1);
  Cam<double> camD = cam_as<double>(*camd);
  Cam<float> camF = cam_as<float>(*camd);
  double campos[3];
  camera_center(camD, campos);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < N; ++i) {
    bool vis;
    double u, v, dep, a, b, c, A, B, C, L11, L21, L22;
    int32_t rad, rc[4];
    uint32_t nt;
    if (mode == ORC_MODE_F32KEY) {
      float mf[3], sf[3], qf[4];
      for (int k = 0; k < 3; ++k) { mf[k] = (float)means[3 * i + k]; sf[k] = (float)scales[3 * i + k]; }
      for (int k = 0; k < 4; ++k) qf[k] = (float)quats[4 * i + k];
      Geom<float> g = project_geom<float>(mf, sf, qf, camF, *st);
      vis = g.vis; u = g.u; v = g.v; dep = g.depth; a = g.a; b = g.b; c = g.c;
      A = g.A; B = g.B; C = g.C; rad = g.radius; nt = g.ntiles;
      L11 = g.L11; L21 = g.L21; L22 = g.L22;
      for (int k = 0; k < 4; ++k) rc[k] = g.rect[k];
    } else {
      Geom<double> g = project_geom<double>(&means[3 * i], &scales[3 * i], &quats[4 * i], camD, *st);
      vis = g.vis; u = g.u; v = g.v; dep = g.depth; a = g.a; b = g.b; c = g.c;
      A = g.A; B = g.B; C = g.C; rad = g.radius; nt = g.ntiles;
      L11 = g.L11; L21 = g.L21; L22 = g.L22;
      for (int k = 0; k < 4; ++k) rc[k] = g.rect[k];
    }
    double col[3] = {0, 0, 0};
    bool cl[3] = {false, false, false};
    if (vis) {
      double md[3];
      if (mode == ORC_MODE_F32KEY)
        for (int k = 0; k < 3; ++k) md[k] = (double)(float)means[3 * i + k];
      else
        for (int k = 0; k < 3; ++k) md[k] = means[3 * i + k];
      sh_color<double>(deg, md, &sh[(size_t)K * 3 * i], campos, st->sh_offset, col, cl);
    }
    if (means2d) { means2d[2 * i] = u; means2d[2 * i + 1] = v; }
    if (conics) { conics[3 * i] = A; conics[3 * i + 1] = B; conics[3 * i + 2] = C; }
    if (chol) { chol[3 * i] = L11; chol[3 * i + 1] = L21; chol[3 * i + 2] = L22; }
    if (cov2d) { cov2d[3 * i] = a; cov2d[3 * i + 1] = b; cov2d[3 * i + 2] = c; }
    if (depths) depths[i] = dep;
    if (radii) radii[i] = rad;
    if (tiles) tiles[i] = nt;
    if (rect) for (int k = 0; k < 4; ++k) rect[4 * i + k] = rc[k];
    if (colors) for (int k = 0; k < 3; ++k) colors[3 * i + k] = col[k];
    if (clamped) for (int k = 0; k < 3; ++k) clamped[3 * i + k] = cl[k];
  }
  return 0;
}

int64_t orc_bin_f32(int64_t N, const float* means2d, const int32_t* radii, const float* depths,
                    int32_t W, int32_t H, int64_t capacity, uint32_t* offsets, uint64_t* keys,
                    uint32_t* ids, uint32_t* ranges) {
  const int gx = grid_x(W), gy = grid_y(H), NT = gx * gy;
  std::vector<int32_t> rects(4 * (size_t)N, 0);
  std::vector<uint8_t> vis(N, 0);
  std::vector<double> dep(N);
  std::vector<uint32_t> bits(N);
  uint64_t run = 0;
  for (int64_t i = 0; i < N; ++i) {
    if (offsets) offsets[i] = (uint32_t)run;
    dep[i] = depths[i];
    bits[i] = f32_bits(depths[i]);
    if (radii[i] <= 0) continue;
    /* same rect rule as the projection's step 7, in fp32 */
    float u = means2d[2 * i], v = means2d[2 * i + 1];
    float r = (float)radii[i];
    double fx0 = std::floor((u - r) / 16.0f), fx1 = std::floor((u + r) / 16.0f) + 1.0;
    double fy0 = std::floor((v - r) / 16.0f), fy1 = std::floor((v + r) / 16.0f) + 1.0;
    auto clampi = [](double f, int hi) { return (int32_t)std::min(std::max(f, 0.0), (double)hi); };
    int32_t* rc = &rects[4 * i];
    rc[0] = clampi(fx0, gx); rc[1] = clampi(fx1, gx);
    rc[2] = clampi(fy0, gy); rc[3] = clampi(fy1, gy);
    if (rc[1] <= rc[0] || rc[3] <= rc[2]) continue;
    vis[i] = 1;
    run += (uint64_t)(rc[1] - rc[0]) * (uint64_t)(rc[3] - rc[2]);
  }
  if ((int64_t)run > capacity) return (int64_t)run;
  std::vector<Inst> inst = build_instances(N, rects, vis, dep, bits, gx);
  for (size_t m = 0; m < inst.size(); ++m) {
    if (keys) keys[m] = inst[m].key;
    if (ids) ids[m] = inst[m].id;
  }
  if (ranges) fill_ranges(inst, NT, ranges);
  return (int64_t)inst.size();
}

int64_t orc_bin_f64(int64_t N, const double* means2d, const int32_t* radii, const double* depths,
                    int32_t W, int32_t H, int64_t capacity, uint32_t* ids, uint32_t* ranges) {
  const int gx = grid_x(W), gy = grid_y(H), NT = gx * gy;
  std::vector<int32_t> rects(4 * (size_t)N, 0);
  std::vector<uint8_t> vis(N, 0);
  std::vector<double> dep(depths, depths + N);
  uint64_t run = 0;
  for (int64_t i = 0; i < N; ++i) {
    if (radii[i] <= 0) continue;
    double u = means2d[2 * i], v = means2d[2 * i + 1], r = radii[i];
    auto clampi = [](double f, int hi) { return (int32_t)std::min(std::max(f, 0.0), (double)hi); };
    int32_t* rc = &rects[4 * i];
    rc[0] = clampi(std::floor((u - r) / 16.0), gx);
    rc[1] = clampi(std::floor((u + r) / 16.0) + 1.0, gx);
    rc[2] = clampi(std::floor((v - r) / 16.0), gy);
    rc[3] = clampi(std::floor((v + r) / 16.0) + 1.0, gy);
    if (rc[1] <= rc[0] || rc[3] <= rc[2]) continue;
    vis[i] = 1;
    run += (uint64_t)(rc[1] - rc[0]) * (uint64_t)(rc[3] - rc[2]);
  }
  if ((int64_t)run > capacity) return (int64_t)run;
  std::vector<Inst> inst = build_instances(N, rects, vis, dep, std::vector<uint32_t>(), gx);
  for (size_t m = 0; m < inst.size(); ++m)
    if (ids) ids[m] = inst[m].id;
  if (ranges) fill_ranges(inst, NT, ranges);
  return (int64_t)inst.size();
}

int orc_composite(int32_t W, int32_t H, const uint32_t* ranges, const uint32_t* ids,
                  const double* means2d, const double* chol, const double* opacities,
                  const double* colors, const double* depths, const double* bg,
                  const orc_settings* st, double* image, double* final_T, uint32_t* last,
                  double* out_depth, double* out_alpha, double* margin) {
  composite_image<double>(W, H, ranges, ids, means2d, chol, opacities, colors, depths, bg, *st,
                          image, final_T, last, out_depth, out_alpha, margin);
  return 0;
}

int orc_composite_bwd(int32_t W, int32_t H, int64_t N, const uint32_t* ranges,
                      const uint32_t* ids, const double* means2d, const double* chol,
                      const double* conics, const double* opacities, const double* colors,
                      const double* bg, const orc_settings* st, const double* dL_dimage,
                      double* g_means2d, double* g_conics, double* g_opacities,
                      double* g_colors, double* abs_sum) {
  composite_bwd_impl(W, H, N, ranges, ids, means2d, chol, conics, opacities, colors, bg, *st,
                     dL_dimage, g_means2d, g_conics, g_opacities, g_colors, abs_sum);
  return 0;
}

int orc_project_bwd(int64_t N, int deg, const double* means, const double* scales,
                    const double* quats, const double* sh, const orc_camera* camd,
                    const orc_settings* st, const int32_t* radii, const double* g_means2d,
                    const double* g_conics, const double* g_colors, double* g_means,
                    double* g_scales, double* g_quats, double* g_sh) {
  project_bwd_all<double>(N, deg, means, scales, quats, sh, *camd, *st, radii, g_means2d,
                          g_conics, g_colors, g_means, g_scales, g_quats, g_sh);
  return 0;
}

int orc_project_bwd_bound(int64_t N, int deg, const double* means, const double* scales,
                          const double* quats, const double* sh, const orc_camera* camd,
                          const orc_settings* st, const int32_t* radii,
                          const double* s_means2d, const double* s_conics,
                          const double* s_colors, double* e_means, double* e_scales,
                          double* e_quats, double* e_sh) {
  const int K = (deg + 1) * (deg + 1);
  Cam<double> cam = cam_as<double>(*camd);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < N; ++i) {
    double* em = &e_means[3 * i];
    double* es = &e_scales[3 * i];
    double* eq = &e_quats[4 * i];
    double* esh = &e_sh[(size_t)K * 3 * i];
    std::fill(em, em + 3, 0.0);
    std::fill(es, es + 3, 0.0);
    std::fill(eq, eq + 4, 0.0);
    std::fill(esh, esh + 3 * K, 0.0);
    if (radii[i] <= 0) continue;
    const double* mean = &means[3 * i];
    const double* scale = &scales[3 * i];
    const double* quat = &quats[4 * i];
    const double* shv = &sh[(size_t)K * 3 * i];
    /* column k of the Jacobian = the backward of the k-th unit 2D gradient
     * (u, v, A, B, C, r, g, b); each output's bound adds |column| * s_k */
    const double s_in[8] = {s_means2d[2 * i], s_means2d[2 * i + 1], s_conics[3 * i],
                            s_conics[3 * i + 1], s_conics[3 * i + 2], s_colors[3 * i],
                            s_colors[3 * i + 1], s_colors[3 * i + 2]};
    for (int k = 0; k < 8; ++k) {
      if (s_in[k] == 0.0) continue;
      double g2[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      g2[k] = 1.0;
      double om[3], os[3], oq[4], osh[48];
      project_bwd_one(deg, mean, scale, quat, shv, cam, *st, &g2[0], &g2[2], &g2[5], om, os,
                      oq, osh);
      for (int j = 0; j < 3; ++j) { em[j] += std::fabs(om[j]) * s_in[k]; es[j] += std::fabs(os[j]) * s_in[k]; }
      for (int j = 0; j < 4; ++j) eq[j] += std::fabs(oq[j]) * s_in[k];
      for (int j = 0; j < 3 * K; ++j) esh[j] += std::fabs(osh[j]) * s_in[k];
    }
  }
  return 0;
}

int64_t orc_loss_jvp(int64_t N, int deg, const double* means, const double* scales,
                     const double* quats, const double* opacities, const double* sh,
                     const double* d_means, const double* d_scales, const double* d_quats,
                     const double* d_opacities, const double* d_sh, const orc_camera* cam,
                     const orc_settings* st, const double* bg, int loss_kind,
                     const double* target, double* loss, double* dloss, uint64_t* signature,
                     double* image_out) {
  const int K = (deg + 1) * (deg + 1);
  bool dual = d_means || d_scales || d_quats || d_opacities || d_sh;
  uint64_t sig = 0;
  int64_t M;
  if (!dual) {
    std::vector<double> m(means, means + 3 * N), s(scales, scales + 3 * N),
        q(quats, quats + 4 * N), o(opacities, opacities + N), c(sh, sh + (size_t)K * 3 * N);
    double L;
    M = full_loss<double>(N, deg, m, s, q, o, c, *cam, *st, bg, loss_kind, target, L, sig,
                          image_out);
    *loss = L;
    if (dloss) *dloss = 0.0;
  } else {
    auto mk = [](const double* x, const double* dx, size_t n) {
      std::vector<Dual> v(n);
      for (size_t k = 0; k < n; ++k) v[k] = Dual(x[k], dx ? dx[k] : 0.0);
      return v;
    };
    std::vector<Dual> m = mk(means, d_means, 3 * N), s = mk(scales, d_scales, 3 * N),
                      q = mk(quats, d_quats, 4 * N), o = mk(opacities, d_opacities, N),
                      c = mk(sh, d_sh, (size_t)K * 3 * N);
    Dual L;
    M = full_loss<Dual>(N, deg, m, s, q, o, c, *cam, *st, bg, loss_kind, target, L, sig,
                        image_out);
    *loss = L.v;
    if (dloss) *dloss = L.d;
  }
  if (signature) *signature = sig;
  return M;
}

int orc_set_threads(int n) {
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
}

void orc_rotation(const double* quat, double* R) {
  double n = std::sqrt(quat[0] * quat[0] + quat[1] * quat[1] + quat[2] * quat[2] + quat[3] * quat[3]);
  rotation_from_unit_quat(quat[0] / n, quat[1] / n, quat[2] / n, quat[3] / n, R);
}

void orc_cov3d(const double* quat, const double* scale, double* Sigma) {
  double R[9];
  orc_rotation(quat, R);
  cov3d_from(R, scale, Sigma);
}

void orc_sh_basis(int deg, const double* dir, double* Y) { sh_basis(deg, dir[0], dir[1], dir[2], Y); }

void orc_sh_basis_grad(int deg, const double* dir, double* dY) {
  sh_basis_grad(deg, dir[0], dir[1], dir[2], dY);
}

}  // extern "C"
