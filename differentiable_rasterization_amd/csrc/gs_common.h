// gs_common.h — device-side helpers shared by the HIP kernels of libgsraster.
//
// Everything in this library is compiled with -ffp-contract=off: the
// projection's geometric outputs must be reproducible bit for bit in IEEE
// fp32, and the forward and backward compositing kernels must take identical
// alpha decisions, so every fused multiply-add below is written explicitly.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gsraster.h"

namespace gs {

constexpr int kTile = 16;
constexpr int kTilePixels = kTile * kTile;  // 256 = one workgroup per tile
constexpr float kLog2e = 1.4426950408889634f;
// sqrt(log2(e) / 2): factors of the conic scaled by it give the Gaussian as
// exp2(-(e1^2 + e2^2)).
constexpr float kSqrtHalfLog2e = 0.8493218002880191f;

// Camera and settings travel to the kernels by value.
struct Cam {
  float R[9];
  float t[3];
  float fx, fy, cx, cy;
  int32_t W, H;
  float near_p, far_p;
};

// Up to eight cameras of one batched launch (by value; blockIdx.y selects).
constexpr int kMaxCams = 8;
struct CamBatch {
  Cam c[kMaxCams];
};

struct Settings {
  float eps2d, alpha_min, alpha_max, T_min, fov_clamp, sh_offset;
};

__host__ inline Cam make_cam(const gs_camera& c) {
  Cam o;
  for (int i = 0; i < 9; ++i) o.R[i] = c.R[i];
  for (int i = 0; i < 3; ++i) o.t[i] = c.t[i];
  o.fx = c.fx; o.fy = c.fy; o.cx = c.cx; o.cy = c.cy;
  o.W = c.width; o.H = c.height;
  o.near_p = c.near_plane; o.far_p = c.far_plane;
  return o;
}

__host__ inline Settings make_settings(const gs_settings& s) {
  return Settings{s.eps2d, s.alpha_min, s.alpha_max, s.T_min, s.fov_clamp, s.sh_offset};
}

__host__ __device__ inline int grid_dim(int pixels) { return (pixels + kTile - 1) / kTile; }

// 2D gradient planes of the compositing backward (and the projection
// backward's input).  Field q of row r is at base + c*P*ld + q*ld + i with
// c = r / ld, i = r % ld: one camera (rows < ld), a batch of cameras (row
// c*ld + i, camera-major blocks of P planes), or packed rows (ld = the
// packed leading dimension).  abs may be NULL (no absolute-gradient sums).
struct Grad2D {
  float* m2;   // dL/du, dL/dv            [.][2][ld]
  float* con;  // dL/dA, dL/dB, dL/dC     [.][3][ld]
  float* op;   // dL/dopacity             [.][1][ld]
  float* col;  // dL/dcolour r, g, b      [.][3][ld]
  float* abs;  // sum |dL/du|, |dL/dv|    [.][2][ld]
  int64_t ld;
};

// Tile rect of the square [u-r, u+r] x [v-r, v+r]: tiles [x0,x1) x [y0,y1).
// Division by 16 is exact in fp32; the clamp happens before the integer
// conversion so that off-screen means stay in range.
__device__ inline void tile_rect(float u, float v, int32_t radius, int gx, int gy, int& x0,
                                 int& x1, int& y0, int& y1) {
  const float r = (float)radius;
  const float fx0 = floorf((u - r) / 16.0f);
  const float fx1 = floorf((u + r) / 16.0f) + 1.0f;
  const float fy0 = floorf((v - r) / 16.0f);
  const float fy1 = floorf((v + r) / 16.0f) + 1.0f;
  x0 = (int)fminf(fmaxf(fx0, 0.0f), (float)gx);
  x1 = (int)fminf(fmaxf(fx1, 0.0f), (float)gx);
  y0 = (int)fminf(fmaxf(fy0, 0.0f), (float)gy);
  y1 = (int)fminf(fmaxf(fy1, 0.0f), (float)gy);
}

// Sum of a wavefront's 64 lanes, left in lane 63: an inclusive scan inside
// each 16-lane row by DPP row shifts (out-of-row sources read 0), then the
// row totals folded in with the row_bcast:15 / row_bcast:31 broadcasts.
#define GS_DPP_ADD(v, ctrl, rmask)                                                         \
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(                              \
                                     0, __builtin_bit_cast(int, v), ctrl, rmask, 0xF, true))
__device__ inline float wave_sum_lane63(float v) {
  GS_DPP_ADD(v, 0x111, 0xF);  // row_shr:1
  GS_DPP_ADD(v, 0x112, 0xF);  // row_shr:2
  GS_DPP_ADD(v, 0x114, 0xF);  // row_shr:4
  GS_DPP_ADD(v, 0x118, 0xF);  // row_shr:8
  GS_DPP_ADD(v, 0x142, 0xA);  // row_bcast:15 into rows 1 and 3
  GS_DPP_ADD(v, 0x143, 0xC);  // row_bcast:31 into rows 2 and 3
  return v;
}
#undef GS_DPP_ADD

__device__ inline uint64_t ballot(bool p) { return __ballot(p); }

}  // namespace gs
