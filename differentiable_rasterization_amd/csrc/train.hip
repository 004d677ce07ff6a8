// train.hip — the two pieces of a training step around the rasterizer (the
// training loop of the gsplat guide (lmnt.cn/news/262699) §4.1 and its
// parameter groups of §4.2):
//   - the image loss mean|x - y| + lambda (1 - SSIM(x, y)) and its gradient,
//     with the structural similarity index over an 11 x 11 Gaussian window
//     (sigma 1.5, zero padding, C1 = 0.01^2, C2 = 0.03^2) per channel;
//   - one Adam step per parameter group on the stored parameters, through
//     the exp / sigmoid activations of scales and opacities.
//
// SSIM is a stencil: each 32 x 16 output tile stages its 42 x 26 halo in
// LDS, one channel at a time, and applies the separable window as a row
// pass (four outputs per lane from a 14-value register window) then a
// column pass (two outputs per lane).  Each XCD takes a contiguous band of
// tiles so that halos are shared through its L2.
// The gradient needs the window twice (statistics, then the adjoint on the
// derivative maps), hence two kernels with the derivative maps in between.
// Adam is one pass over the parameter planes, bound by HBM.
#include "gs_common.h"

#include <cmath>

namespace gs {

constexpr int kSsimR = 5;
constexpr int kSsimTaps = 2 * kSsimR + 1;
constexpr int kSsimTx = 32;  // output tile columns (one wave covers two rows)
constexpr int kSsimTy = 16;  // output tile rows
constexpr int kSsimHx = kSsimTx + 2 * kSsimR;
constexpr int kSsimHy = kSsimTy + 2 * kSsimR;
constexpr float kSsimC1 = 0.0001f;  // (0.01 * dynamic range 1)^2
constexpr float kSsimC2 = 0.0009f;  // (0.03 * dynamic range 1)^2

struct SsimWindow {
  float w[kSsimTaps];  // 1D factor, sums to 1
};

__device__ inline double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Sum over the workgroup in a fixed order (lanes by butterfly, then the
// four waves in index order).
__device__ inline double block_sum_f64(double v, double* s_w) {
  v = wave_sum_f64(v);
  if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = v;
  __syncthreads();
  const double r = (s_w[0] + s_w[1]) + (s_w[2] + s_w[3]);
  __syncthreads();
  return r;
}

constexpr int kSsimLd = 44;  // LDS row stride of a halo row (16-byte aligned rows)
constexpr int kSsimXcds = 8;

// Tile of a workgroup: each XCD (workgroups are dealt to the eight XCDs in
// turn) takes a contiguous run of tiles in row-major order, so neighbouring
// tiles share their halo rows through that XCD's L2.  -1 past the last tile.
__device__ inline int ssim_tile(int nb) {
  const int per = (nb + kSsimXcds - 1) / kSsimXcds;
  const int tile = (int)(blockIdx.x % kSsimXcds) * per + (int)(blockIdx.x / kSsimXcds);
  return tile < nb ? tile : -1;
}

// Row pass item: four adjacent outputs of one halo row from the 14 inputs
// they span (a sliding window in registers).
__device__ inline void load14(const float* row, float v[14]) {
  const float4 a = *(const float4*)(row);
  const float4 b = *(const float4*)(row + 4);
  const float4 c = *(const float4*)(row + 8);
  const float2 e = *(const float2*)(row + 12);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  v[8] = c.x; v[9] = c.y; v[10] = c.z; v[11] = c.w;
  v[12] = e.x; v[13] = e.y;
}

// Pass 1.  For every pixel and channel: the windowed means and second
// moments of x and y, the index s, and its partial derivatives with respect
// to mu_x, E[x^2] and E[xy], written to d as nine planes [map][channel][H][W].
// Per tile, the sums of s and |x - y| (fp64) go to partials[tile][2].  One
// channel is staged at a time, which keeps LDS near 26 KB per workgroup.
__global__ __launch_bounds__(256) void ssim_stats_kernel(int W, int H, int tiles_x, int nb,
                                                         const float* __restrict__ x,
                                                         const float* __restrict__ y,
                                                         SsimWindow win, float* __restrict__ d,
                                                         double* __restrict__ partials) {
  __shared__ __align__(16) float sx[kSsimHy][kSsimLd];
  __shared__ __align__(16) float sy[kSsimHy][kSsimLd];
  __shared__ float hb[5][kSsimHy][kSsimTx];
  __shared__ double s_w[4];
  const int tile = ssim_tile(nb);
  if (tile < 0) return;
  const int t = threadIdx.x;
  const int x0 = (tile % tiles_x) * kSsimTx, y0 = (tile / tiles_x) * kSsimTy;
  const int64_t plane = (int64_t)W * H;
  double acc_s = 0.0, acc_l1 = 0.0;
  const int ox = t & 31, oy0 = (t >> 5) * 2;  // column pass: two rows per thread
  // halo element k of this thread (rows of 42 as 64 lanes): its pixel's
  // offset, -1 outside the image (zero there); the next channel's values are
  // loaded into registers while the current channel is computed
  constexpr int kLd = (kSsimHy * 64 + 255) / 256;
  int64_t hpix[kLd];
#pragma unroll
  for (int k = 0; k < kLd; ++k) {
    const int idx = t + 256 * k, r = idx >> 6, px = idx & 63;
    const int gx = x0 - kSsimR + px, gy = y0 - kSsimR + r;
    hpix[k] = (idx < kSsimHy * 64 && px < kSsimHx && gx >= 0 && gx < W && gy >= 0 && gy < H)
                  ? ((int64_t)gy * W + gx) * 3 : -1;
  }
  float px_[kLd], py_[kLd];
#pragma unroll
  for (int k = 0; k < kLd; ++k) {
    px_[k] = hpix[k] >= 0 ? x[hpix[k]] : 0.0f;
    py_[k] = hpix[k] >= 0 ? y[hpix[k]] : 0.0f;
  }
  for (int c = 0; c < 3; ++c) {
    // channel c of the halo into LDS
#pragma unroll
    for (int k = 0; k < kLd; ++k) {
      const int idx = t + 256 * k, px = idx & 63;
      if (idx < kSsimHy * 64 && px < kSsimHx) {
        sx[idx >> 6][px] = px_[k];
        sy[idx >> 6][px] = py_[k];
      }
    }
    __syncthreads();
    if (c < 2) {
#pragma unroll
      for (int k = 0; k < kLd; ++k) {
        px_[k] = hpix[k] >= 0 ? x[hpix[k] + c + 1] : 0.0f;
        py_[k] = hpix[k] >= 0 ? y[hpix[k] + c + 1] : 0.0f;
      }
    }
    // row pass: 26 rows x 8 groups of four outputs
    if (t < kSsimHy * 8) {
      const int r = t >> 3, j0 = (t & 7) * 4;
      float xv[14], yv[14];
      load14(&sx[r][j0], xv);
      load14(&sy[r][j0], yv);
#pragma unroll
      for (int o = 0; o < 4; ++o) {
        float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f, a4 = 0.0f;
#pragma unroll
        for (int k = 0; k < kSsimTaps; ++k) {
          const float xk = xv[o + k], yk = yv[o + k];
          const float wx = win.w[k] * xk, wy = win.w[k] * yk;
          a0 += wx;
          a1 += wy;
          a2 = fmaf(wx, xk, a2);
          a3 = fmaf(wy, yk, a3);
          a4 = fmaf(wx, yk, a4);
        }
        hb[0][r][j0 + o] = a0;
        hb[1][r][j0 + o] = a1;
        hb[2][r][j0 + o] = a2;
        hb[3][r][j0 + o] = a3;
        hb[4][r][j0 + o] = a4;
      }
    }
    __syncthreads();
    // column pass: outputs (oy0, ox) and (oy0 + 1, ox) from 12 rows
    float st[5][2];
#pragma unroll
    for (int q = 0; q < 5; ++q) {
      float col[12];
#pragma unroll
      for (int k = 0; k < 12; ++k) col[k] = hb[q][oy0 + k][ox];
      float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
      for (int k = 0; k < kSsimTaps; ++k) {
        s0 = fmaf(win.w[k], col[k], s0);
        s1 = fmaf(win.w[k], col[k + 1], s1);
      }
      st[q][0] = s0;
      st[q][1] = s1;
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int gx = x0 + ox, gy = y0 + oy0 + p;
      if (gx < W && gy < H) {
        const float mx = st[0][p], my = st[1][p];
        const float vx = st[2][p] - mx * mx, vy = st[3][p] - my * my;
        const float cxy = st[4][p] - mx * my;
        const float A1 = 2.0f * mx * my + kSsimC1, A2 = 2.0f * cxy + kSsimC2;
        const float B1 = mx * mx + my * my + kSsimC1, B2 = vx + vy + kSsimC2;
        const float iB1 = __builtin_amdgcn_rcpf(B1), iB2 = __builtin_amdgcn_rcpf(B2);
        const float iB = iB1 * iB2;
        const float s = A1 * A2 * iB;
        const float dmu = 2.0f * my * (A2 - A1) * iB + 2.0f * mx * s * (iB2 - iB1);
        const float dxx = -s * iB2;
        const float dxy = 2.0f * A1 * iB;
        const int64_t o = (int64_t)gy * W + gx;
        d[(int64_t)c * plane + o] = dmu;
        d[(int64_t)(3 + c) * plane + o] = dxx;
        d[(int64_t)(6 + c) * plane + o] = dxy;
        acc_s += (double)s;
        acc_l1 += (double)fabsf(sx[oy0 + p + kSsimR][ox + kSsimR] -
                                sy[oy0 + p + kSsimR][ox + kSsimR]);
      }
    }
    __syncthreads();  // sx, sy and hb are rewritten for the next channel
  }
  const double ts = block_sum_f64(acc_s, s_w);
  const double tl = block_sum_f64(acc_l1, s_w);
  if (t == 0) {
    partials[2 * tile] = ts;
    partials[2 * tile + 1] = tl;
  }
}

// Pass 2.  The adjoint of the windowed sums: the same window over the three
// derivative maps (zero outside the image), combined per pixel and channel
// into dL/dx = sign(x - y) / n - (lambda / n) (w*d_mu + 2 x w*d_xx + y w*d_xy).
// One channel's three maps are staged at a time; the next channel's are
// loaded into registers while the current one is computed.
__global__ __launch_bounds__(256) void ssim_grad_kernel(int W, int H, int tiles_x, int nb,
                                                        const float* __restrict__ x,
                                                        const float* __restrict__ y,
                                                        SsimWindow win,
                                                        const float* __restrict__ d,
                                                        float inv_n, float lam_n,
                                                        float* __restrict__ g) {
  __shared__ __align__(16) float sd[3][kSsimHy][kSsimLd];
  __shared__ float hb[3][kSsimHy][kSsimTx];
  const int tile = ssim_tile(nb);
  if (tile < 0) return;
  const int t = threadIdx.x;
  const int x0 = (tile % tiles_x) * kSsimTx, y0 = (tile / tiles_x) * kSsimTy;
  const int64_t plane = (int64_t)W * H;
  const int ox = t & 31, oy0 = (t >> 5) * 2;
  // halo element k of this thread as in pass 1 (offset into a plane, -1
  // outside); the next channel's three maps are loaded while one is computed
  constexpr int kLd = (kSsimHy * 64 + 255) / 256;
  int hpix[kLd];
#pragma unroll
  for (int k = 0; k < kLd; ++k) {
    const int idx = t + 256 * k, r = idx >> 6, px = idx & 63;
    const int gx = x0 - kSsimR + px, gy = y0 - kSsimR + r;
    hpix[k] = (idx < kSsimHy * 64 && px < kSsimHx && gx >= 0 && gx < W && gy >= 0 && gy < H)
                  ? gy * W + gx : -1;
  }
  float pf[3][kLd];
#pragma unroll
  for (int m = 0; m < 3; ++m)
#pragma unroll
    for (int k = 0; k < kLd; ++k)
      pf[m][k] = hpix[k] >= 0 ? d[(int64_t)(3 * m) * plane + hpix[k]] : 0.0f;
  float gv[2][3];
  for (int c = 0; c < 3; ++c) {
#pragma unroll
    for (int k = 0; k < kLd; ++k) {
      const int idx = t + 256 * k, px = idx & 63;
      if (idx < kSsimHy * 64 && px < kSsimHx) {
#pragma unroll
        for (int m = 0; m < 3; ++m) sd[m][idx >> 6][px] = pf[m][k];
      }
    }
    __syncthreads();
    if (c < 2) {
#pragma unroll
      for (int m = 0; m < 3; ++m)
#pragma unroll
        for (int k = 0; k < kLd; ++k)
          pf[m][k] = hpix[k] >= 0 ? d[(int64_t)(3 * m + c + 1) * plane + hpix[k]] : 0.0f;
    }
    if (t < kSsimHy * 8) {
      const int r = t >> 3, j0 = (t & 7) * 4;
#pragma unroll
      for (int m = 0; m < 3; ++m) {
        float v[14];
        load14(&sd[m][r][j0], v);
#pragma unroll
        for (int o = 0; o < 4; ++o) {
          float b = 0.0f;
#pragma unroll
          for (int k = 0; k < kSsimTaps; ++k) b = fmaf(win.w[k], v[o + k], b);
          hb[m][r][j0 + o] = b;
        }
      }
    }
    __syncthreads();
    float bs[3][2];
#pragma unroll
    for (int m = 0; m < 3; ++m) {
      float col[12];
#pragma unroll
      for (int k = 0; k < 12; ++k) col[k] = hb[m][oy0 + k][ox];
      float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
      for (int k = 0; k < kSsimTaps; ++k) {
        s0 = fmaf(win.w[k], col[k], s0);
        s1 = fmaf(win.w[k], col[k + 1], s1);
      }
      bs[m][0] = s0;
      bs[m][1] = s1;
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int gx = x0 + ox, gy = y0 + oy0 + p;
      float r = 0.0f;
      if (gx < W && gy < H) {
        const int64_t o = ((int64_t)gy * W + gx) * 3 + c;
        const float xv = x[o], yv = y[o];
        const float diff = xv - yv;
        const float sg = diff > 0.0f ? 1.0f : (diff < 0.0f ? -1.0f : 0.0f);
        const float gs = bs[0][p] + 2.0f * xv * bs[1][p] + yv * bs[2][p];
        r = sg * inv_n - lam_n * gs;
      }
      gv[p][c] = r;
    }
    __syncthreads();  // sd and hb are rewritten for the next channel
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int gx = x0 + ox, gy = y0 + oy0 + p;
    if (gx < W && gy < H) {
      const int64_t o = ((int64_t)gy * W + gx) * 3;
      g[o] = gv[p][0];
      g[o + 1] = gv[p][1];
      g[o + 2] = gv[p][2];
    }
  }
}

// The loss value from the per-workgroup sums, added in a fixed order.
__global__ __launch_bounds__(256) void ssim_loss_kernel(const double* __restrict__ partials,
                                                        int64_t nb, double n, float lambda,
                                                        float* __restrict__ loss) {
  __shared__ double s_w[4];
  double s = 0.0, l1 = 0.0;
  for (int64_t b = threadIdx.x; b < nb; b += 256) {
    s += partials[2 * b];
    l1 += partials[2 * b + 1];
  }
  const double ts = block_sum_f64(s, s_w);
  const double tl = block_sum_f64(l1, s_w);
  if (threadIdx.x == 0) *loss = (float)(tl / n + (double)lambda * (1.0 - ts / n));
}

// ---------------------------------------------------------------------------
// Adam over the parameter planes.  Plane p (blockIdx.y) of the moments is
// plane p of the concatenation means (3), scales (3), quats (4), opacity
// (1), SH (3K); its group fixes the learning rate and the activation.
// ---------------------------------------------------------------------------
struct AdamArgs {
  float* raw[5];          // means, log-scales, quats, opacity logits, SH
  const float* grad[5];   // gradients with respect to the activated values
  float* scales;          // activated scales [3][ld], read then rewritten
  float* opacities;       // activated opacities [ld], read then rewritten
  float step_size[5];     // lr / (1 - beta1^step) per group
  float beta1, beta2, inv_sqrt_bc2, eps;
};

template <bool kPacked>
__global__ __launch_bounds__(256) void adam_kernel(int64_t rows, int64_t ld, int64_t ldg,
                                                   const uint32_t* __restrict__ vis_ids,
                                                   AdamArgs a, float* __restrict__ m,
                                                   float* __restrict__ v) {
  const int p = blockIdx.y;
  int grp, q;
  if (p < 3) {
    grp = 0; q = p;
  } else if (p < 6) {
    grp = 1; q = p - 3;
  } else if (p < 10) {
    grp = 2; q = p - 6;
  } else if (p == 10) {
    grp = 3; q = 0;
  } else {
    grp = 4; q = p - 11;
  }
  float* raw = a.raw[grp] + (int64_t)q * ld;
  const float* gp = a.grad[grp] + (int64_t)q * ldg;
  float* mp = m + (int64_t)p * ld;
  float* vp = v + (int64_t)p * ld;
  const float step_size = a.step_size[grp];
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < rows; r += stride) {
    const int64_t i = kPacked ? (int64_t)vis_ids[r] : r;
    float g = gp[r];
    // to the stored value: d/dlog_s = d/ds * s, d/dlogit = d/do * o (1 - o)
    if (grp == 1) g *= a.scales[(int64_t)q * ld + i];
    if (grp == 3) {
      const float o = a.opacities[i];
      g *= o * (1.0f - o);
    }
    const float mm = a.beta1 * mp[i] + (1.0f - a.beta1) * g;
    const float vv = a.beta2 * vp[i] + (1.0f - a.beta2) * (g * g);
    const float pn = raw[i] - step_size * mm / (sqrtf(vv) * a.inv_sqrt_bc2 + a.eps);
    mp[i] = mm;
    vp[i] = vv;
    raw[i] = pn;
    if (grp == 1) a.scales[(int64_t)q * ld + i] = expf(pn);
    if (grp == 3) a.opacities[i] = 1.0f / (1.0f + expf(-pn));
  }
}

static inline size_t talign(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace gs

extern "C" size_t gs_ssim_workspace_bytes(int32_t W, int32_t H) {
  const int64_t nb = (int64_t)((W + gs::kSsimTx - 1) / gs::kSsimTx) *
                     ((H + gs::kSsimTy - 1) / gs::kSsimTy);
  return gs::talign(sizeof(float) * 9 * (size_t)W * (size_t)H) +
         gs::talign(sizeof(double) * 2 * (size_t)(nb ? nb : 1));
}

extern "C" hipError_t gs_launch_l1_dssim(int32_t W, int32_t H, const float* img,
                                         const float* tgt, float lambda, float* g, float* loss,
                                         void* workspace, hipStream_t s) {
  using namespace gs;
  SsimWindow win;
  {
    // the Gaussian factor exp(-k^2 / (2 * 1.5^2)), normalised in double
    double wd[kSsimTaps], sum = 0.0;
    for (int k = 0; k < kSsimTaps; ++k) {
      const double u = (double)(k - kSsimR);
      wd[k] = std::exp(-u * u / (2.0 * 1.5 * 1.5));
      sum += wd[k];
    }
    for (int k = 0; k < kSsimTaps; ++k) win.w[k] = (float)(wd[k] / sum);
  }
  const int tiles_x = (W + kSsimTx - 1) / kSsimTx;
  const int nb = tiles_x * ((H + kSsimTy - 1) / kSsimTy);
  const int per = (nb + kSsimXcds - 1) / kSsimXcds;
  const dim3 grid((unsigned)(per * kSsimXcds));
  float* d = (float*)workspace;
  double* partials =
      (double*)((char*)workspace + talign(sizeof(float) * 9 * (size_t)W * (size_t)H));
  const double n = 3.0 * (double)W * (double)H;
  hipLaunchKernelGGL(ssim_stats_kernel, grid, dim3(256), 0, s, W, H, tiles_x, nb, img, tgt, win,
                     d, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ssim_grad_kernel, grid, dim3(256), 0, s, W, H, tiles_x, nb, img, tgt, win, d,
                     (float)(1.0 / n), (float)((double)lambda / n), g);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (loss) {
    hipLaunchKernelGGL(ssim_loss_kernel, dim3(1), dim3(256), 0, s, partials, nb, n, lambda, loss);
    e = hipGetLastError();
  }
  return e;
}

// vis_ids NULL: rows = N Gaussians, gradients [P][ld].  Otherwise rows =
// the list's length, gradients [P][ldg] in list order.
extern "C" hipError_t gs_launch_adam(int64_t rows, int64_t ld, int64_t ldg,
                                     const uint32_t* vis_ids, int deg, int64_t step,
                                     const gs_adam_config& cfg, float* const raw[5],
                                     const float* const grad[5], float* scales,
                                     float* opacities, float* m, float* v, hipStream_t s) {
  using namespace gs;
  if (rows == 0) return hipSuccess;
  AdamArgs a;
  const float lr[5] = {cfg.lr_means, cfg.lr_scales, cfg.lr_quats, cfg.lr_opacities, cfg.lr_sh};
  const double bc1 = 1.0 - std::pow((double)cfg.beta1, (double)step);
  const double bc2 = 1.0 - std::pow((double)cfg.beta2, (double)step);
  for (int k = 0; k < 5; ++k) {
    a.raw[k] = raw[k];
    a.grad[k] = grad[k];
    a.step_size[k] = (float)((double)lr[k] / bc1);
  }
  a.scales = scales;
  a.opacities = opacities;
  a.beta1 = cfg.beta1;
  a.beta2 = cfg.beta2;
  a.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(bc2));
  a.eps = cfg.eps;
  const int planes = 11 + 3 * (deg + 1) * (deg + 1);
  int64_t bx = (rows + 255) / 256;
  if (bx > 1024) bx = 1024;
  const dim3 grid((unsigned)bx, (unsigned)planes);
  if (vis_ids)
    hipLaunchKernelGGL(adam_kernel<true>, grid, dim3(256), 0, s, rows, ld, ldg, vis_ids, a, m, v);
  else
    hipLaunchKernelGGL(adam_kernel<false>, grid, dim3(256), 0, s, rows, ld, ldg, nullptr, a, m,
                       v);
  return hipGetLastError();
}
