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
// LDS and applies the separable window as a row pass then a column pass.
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

// Pass 1.  For every pixel and channel: the windowed means and second
// moments of x and y, the index s, and its partial derivatives with respect
// to mu_x, E[x^2] and E[xy], written to d as nine planes [map][channel][H][W].
// Per workgroup, the sums of s and |x - y| (fp64) go to partials[block][2].
__global__ __launch_bounds__(256) void ssim_stats_kernel(int W, int H,
                                                         const float* __restrict__ x,
                                                         const float* __restrict__ y,
                                                         SsimWindow win, float* __restrict__ d,
                                                         double* __restrict__ partials) {
  __shared__ float sx[3][kSsimHy][kSsimHx];
  __shared__ float sy[3][kSsimHy][kSsimHx];
  __shared__ float hb[5][kSsimHy][kSsimTx];
  __shared__ double s_w[4];
  const int t = threadIdx.x;
  const int x0 = blockIdx.x * kSsimTx, y0 = blockIdx.y * kSsimTy;
  // the halo, zero outside the image; a halo row is 42 pixels x 3 channels
  // contiguous in memory
  constexpr int kRow = kSsimHx * 3;
  for (int idx = t; idx < kSsimHy * kRow; idx += 256) {
    const int r = idx / kRow, col = idx - r * kRow;
    const int px = col / 3, c = col - px * 3;
    const int gx = x0 - kSsimR + px, gy = y0 - kSsimR + r;
    float vx = 0.0f, vy = 0.0f;
    if (gx >= 0 && gx < W && gy >= 0 && gy < H) {
      const int64_t o = ((int64_t)gy * W + gx) * 3 + c;
      vx = x[o];
      vy = y[o];
    }
    sx[c][r][px] = vx;
    sy[c][r][px] = vy;
  }
  __syncthreads();
  const int64_t plane = (int64_t)W * H;
  double acc_s = 0.0, acc_l1 = 0.0;
  for (int c = 0; c < 3; ++c) {
    // row pass: the five sums along x for every halo row
    for (int idx = t; idx < kSsimHy * kSsimTx; idx += 256) {
      const int r = idx >> 5, j = idx & 31;
      float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f, a4 = 0.0f;
#pragma unroll
      for (int k = 0; k < kSsimTaps; ++k) {
        const float xv = sx[c][r][j + k], yv = sy[c][r][j + k];
        const float wx = win.w[k] * xv, wy = win.w[k] * yv;
        a0 += wx;
        a1 += wy;
        a2 = fmaf(wx, xv, a2);
        a3 = fmaf(wy, yv, a3);
        a4 = fmaf(wx, yv, a4);
      }
      hb[0][r][j] = a0;
      hb[1][r][j] = a1;
      hb[2][r][j] = a2;
      hb[3][r][j] = a3;
      hb[4][r][j] = a4;
    }
    __syncthreads();
    // column pass and the pointwise index
    for (int idx = t; idx < kSsimTy * kSsimTx; idx += 256) {
      const int oy = idx >> 5, ox = idx & 31;
      float mx = 0.0f, my = 0.0f, exx = 0.0f, eyy = 0.0f, exy = 0.0f;
#pragma unroll
      for (int k = 0; k < kSsimTaps; ++k) {
        const float wk = win.w[k];
        mx = fmaf(wk, hb[0][oy + k][ox], mx);
        my = fmaf(wk, hb[1][oy + k][ox], my);
        exx = fmaf(wk, hb[2][oy + k][ox], exx);
        eyy = fmaf(wk, hb[3][oy + k][ox], eyy);
        exy = fmaf(wk, hb[4][oy + k][ox], exy);
      }
      const int gx = x0 + ox, gy = y0 + oy;
      if (gx < W && gy < H) {
        const float vx = exx - mx * mx, vy = eyy - my * my, cxy = exy - mx * my;
        const float A1 = 2.0f * mx * my + kSsimC1, A2 = 2.0f * cxy + kSsimC2;
        const float B1 = mx * mx + my * my + kSsimC1, B2 = vx + vy + kSsimC2;
        const float iB1 = 1.0f / B1, iB2 = 1.0f / B2;
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
        acc_l1 += (double)fabsf(sx[c][oy + kSsimR][ox + kSsimR] - sy[c][oy + kSsimR][ox + kSsimR]);
      }
    }
    __syncthreads();  // hb is rewritten for the next channel
  }
  const double ts = block_sum_f64(acc_s, s_w);
  const double tl = block_sum_f64(acc_l1, s_w);
  if (t == 0) {
    const int64_t b = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
    partials[2 * b] = ts;
    partials[2 * b + 1] = tl;
  }
}

// Pass 2.  The adjoint of the windowed sums: the same window over the three
// derivative maps (zero outside the image), combined per pixel and channel
// into dL/dx = sign(x - y) / n - (lambda / n) (w*d_mu + 2 x w*d_xx + y w*d_xy).
__global__ __launch_bounds__(256) void ssim_grad_kernel(int W, int H,
                                                        const float* __restrict__ x,
                                                        const float* __restrict__ y,
                                                        SsimWindow win,
                                                        const float* __restrict__ d,
                                                        float inv_n, float lam_n,
                                                        float* __restrict__ g) {
  __shared__ float sd[9][kSsimHy][kSsimHx];
  __shared__ float hb[3][kSsimHy][kSsimTx];
  const int t = threadIdx.x;
  const int x0 = blockIdx.x * kSsimTx, y0 = blockIdx.y * kSsimTy;
  const int64_t plane = (int64_t)W * H;
  constexpr int kHalo = kSsimHy * kSsimHx;
  for (int idx = t; idx < 9 * kHalo; idx += 256) {
    const int q = idx / kHalo, rem = idx - q * kHalo;
    const int r = rem / kSsimHx, px = rem - r * kSsimHx;
    const int gx = x0 - kSsimR + px, gy = y0 - kSsimR + r;
    float v = 0.0f;
    if (gx >= 0 && gx < W && gy >= 0 && gy < H) v = d[(int64_t)q * plane + (int64_t)gy * W + gx];
    sd[q][r][px] = v;
  }
  __syncthreads();
  float gv[2][3];
  for (int c = 0; c < 3; ++c) {
    for (int idx = t; idx < kSsimHy * kSsimTx; idx += 256) {
      const int r = idx >> 5, j = idx & 31;
      float b0 = 0.0f, b1 = 0.0f, b2 = 0.0f;
#pragma unroll
      for (int k = 0; k < kSsimTaps; ++k) {
        const float wk = win.w[k];
        b0 = fmaf(wk, sd[c][r][j + k], b0);
        b1 = fmaf(wk, sd[3 + c][r][j + k], b1);
        b2 = fmaf(wk, sd[6 + c][r][j + k], b2);
      }
      hb[0][r][j] = b0;
      hb[1][r][j] = b1;
      hb[2][r][j] = b2;
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int idx = t + 256 * p;
      const int oy = idx >> 5, ox = idx & 31;
      float c0 = 0.0f, c1 = 0.0f, c2 = 0.0f;
#pragma unroll
      for (int k = 0; k < kSsimTaps; ++k) {
        const float wk = win.w[k];
        c0 = fmaf(wk, hb[0][oy + k][ox], c0);
        c1 = fmaf(wk, hb[1][oy + k][ox], c1);
        c2 = fmaf(wk, hb[2][oy + k][ox], c2);
      }
      const int gx = x0 + ox, gy = y0 + oy;
      float r = 0.0f;
      if (gx < W && gy < H) {
        const int64_t o = ((int64_t)gy * W + gx) * 3 + c;
        const float xv = x[o], yv = y[o];
        const float diff = xv - yv;
        const float sg = diff > 0.0f ? 1.0f : (diff < 0.0f ? -1.0f : 0.0f);
        const float gs = c0 + 2.0f * xv * c1 + yv * c2;
        r = sg * inv_n - lam_n * gs;
      }
      gv[p][c] = r;
    }
    __syncthreads();
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int idx = t + 256 * p;
    const int gx = x0 + (idx & 31), gy = y0 + (idx >> 5);
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
  const dim3 grid((unsigned)((W + kSsimTx - 1) / kSsimTx), (unsigned)((H + kSsimTy - 1) / kSsimTy));
  const int64_t nb = (int64_t)grid.x * grid.y;
  float* d = (float*)workspace;
  double* partials =
      (double*)((char*)workspace + talign(sizeof(float) * 9 * (size_t)W * (size_t)H));
  const double n = 3.0 * (double)W * (double)H;
  hipLaunchKernelGGL(ssim_stats_kernel, grid, dim3(256), 0, s, W, H, img, tgt, win, d, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ssim_grad_kernel, grid, dim3(256), 0, s, W, H, img, tgt, win, d,
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
