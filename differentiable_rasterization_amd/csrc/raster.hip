// raster.hip — stage 4 (front-to-back compositing) and stage 5a (its
// backward), plus the image loss gradient.
//
// One 256-lane workgroup (four wave64) per 16x16 tile, one lane per pixel;
// a wave covers four pixel rows of the tile.  The tile's depth-sorted list
// is walked in batches of 256 splats that the workgroup first stages into
// LDS (one gather per lane), after which every lane reads the batch with
// broadcast LDS loads.  The work is bound by VALU issue (about a dozen
// operations per pixel-splat pair plus one transcendental), not by memory,
// so nothing here is shaped for MFMA.  The forward stops the whole tile as
// soon as every pixel has terminated.
//
// The backward walks the same lists back to front from each pixel's last
// blended entry.  Per splat each wave reduces its 64 pixels' nine gradient
// terms with DPP row shifts and row broadcasts (skipped with a ballot when
// no lane of the wave touched the splat); the four wave partials meet in LDS
// and one lane per splat issues at most nine fp32 atomics per tile, instead
// of one per pixel.
//
// Decisions (q < 0, alpha < alpha_min, alpha clamp, stop at T < T_min) are
// taken by the same inline code in both kernels, compiled without
// contraction, so the backward replays exactly the forward's choices.
#include "gs_common.h"

namespace gs {

// Splat staged in LDS: mean, conic pre-scaled so that exp2 of the quadratic
// form is the Gaussian (qa = -log2e/2 A, qb = -log2e B, qc = -log2e/2 C),
// opacity, colour, depth.
struct SplatLds {
  float u, v, qa, qb, qc, o, r, g, b, z;
};

__device__ inline void stage_splat(SplatLds& s, uint32_t id, int64_t ld,
                                   const float* __restrict__ means2d,
                                   const float* __restrict__ conics,
                                   const float* __restrict__ opac,
                                   const float* __restrict__ colors,
                                   const float* __restrict__ depths) {
  s.u = means2d[id];
  s.v = means2d[ld + id];
  s.qa = (-0.5f * kLog2e) * conics[id];
  s.qb = (-kLog2e) * conics[ld + id];
  s.qc = (-0.5f * kLog2e) * conics[2 * ld + id];
  s.o = opac[id];
  s.r = colors[id];
  s.g = colors[ld + id];
  s.b = colors[2 * ld + id];
  s.z = depths ? depths[id] : 0.0f;
}

// log2 of the Gaussian at pixel offset (dx, dy): -log2e * q / 2.
__device__ inline float splat_power2(const SplatLds& s, float dx, float dy) {
  return fmaf(s.qa * dx, dx, fmaf(s.qc * dy, dy, s.qb * (dx * dy)));
}

__global__ __launch_bounds__(256) void raster_fwd_kernel(
    int W, int H, int gx, const uint32_t* __restrict__ ranges, const uint32_t* __restrict__ ids,
    int64_t ld, const float* __restrict__ means2d, const float* __restrict__ conics,
    const float* __restrict__ opac, const float* __restrict__ colors,
    const float* __restrict__ depths, float bg0, float bg1, float bg2, Settings st,
    float* __restrict__ image, float* __restrict__ final_T, uint32_t* __restrict__ last_idx,
    float* __restrict__ out_depth, float* __restrict__ out_alpha) {
  __shared__ SplatLds s_sp[256];
  const int tile = blockIdx.x;
  const int tx = tile % gx, ty = tile / gx;
  const int tid = threadIdx.x;
  const int px = tx * kTile + (tid & 15), py = ty * kTile + (tid >> 4);
  const bool inside = px < W && py < H;
  const float fpx = (float)px + 0.5f, fpy = (float)py + 0.5f;
  const uint32_t start = ranges[2 * tile], end = ranges[2 * tile + 1];

  float T = 1.0f, C0 = 0.0f, C1 = 0.0f, C2 = 0.0f, D = 0.0f;
  uint32_t last = 0;
  bool done = !inside;
  for (uint32_t b = start; b < end; b += 256) {
    if (__syncthreads_count(done) == 256) break;
    const uint32_t j = b + (uint32_t)tid;
    if (j < end) stage_splat(s_sp[tid], ids[j], ld, means2d, conics, opac, colors, depths);
    __syncthreads();
    const int n = (int)((end - b) < 256u ? (end - b) : 256u);
    if (!done) {
      for (int k = 0; k < n; ++k) {
        const SplatLds& s = s_sp[k];
        const float dx = fpx - s.u, dy = fpy - s.v;
        const float p2 = splat_power2(s, dx, dy);
        if (p2 > 0.0f) continue;
        const float oG = s.o * __builtin_amdgcn_exp2f(p2);
        const float alpha = oG > st.alpha_max ? st.alpha_max : oG;
        if (alpha < st.alpha_min) continue;
        const float Tn = T * (1.0f - alpha);
        if (Tn < st.T_min) {
          done = true;
          break;
        }
        const float w = alpha * T;
        C0 = fmaf(s.r, w, C0);
        C1 = fmaf(s.g, w, C1);
        C2 = fmaf(s.b, w, C2);
        D = fmaf(s.z, w, D);
        T = Tn;
        last = b - start + (uint32_t)k + 1u;
      }
    }
  }
  if (!inside) return;
  const int64_t p = (int64_t)py * W + px;
  image[3 * p + 0] = fmaf(T, bg0, C0);
  image[3 * p + 1] = fmaf(T, bg1, C1);
  image[3 * p + 2] = fmaf(T, bg2, C2);
  final_T[p] = T;
  last_idx[p] = last;
  if (out_depth) out_depth[p] = D;
  if (out_alpha) out_alpha[p] = 1.0f - T;
}

// Gradient slots of one splat: u, v, A, B, C, opacity, r, g, b.
constexpr int kFields = 9;

__global__ __launch_bounds__(256) void raster_bwd_kernel(
    int W, int H, int gx, const uint32_t* __restrict__ ranges, const uint32_t* __restrict__ ids,
    int64_t ld, const float* __restrict__ means2d, const float* __restrict__ conics,
    const float* __restrict__ opac, const float* __restrict__ colors, float bg0, float bg1,
    float bg2, Settings st, const float* __restrict__ final_T,
    const uint32_t* __restrict__ last_idx, const float* __restrict__ dL_dimage,
    float* __restrict__ g_m2, float* __restrict__ g_con, float* __restrict__ g_op,
    float* __restrict__ g_col) {
  __shared__ SplatLds s_sp[256];
  __shared__ uint32_t s_id[256];
  __shared__ float s_part[4][kFields][256];
  __shared__ uint32_t s_maxlast;
  const int tile = blockIdx.x;
  const int tx = tile % gx, ty = tile / gx;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int px = tx * kTile + (tid & 15), py = ty * kTile + (tid >> 4);
  const bool inside = px < W && py < H;
  const float fpx = (float)px + 0.5f, fpy = (float)py + 0.5f;
  const uint32_t start = ranges[2 * tile], end = ranges[2 * tile + 1];

  float T = 1.0f, g0 = 0.0f, g1 = 0.0f, g2 = 0.0f;
  uint32_t last = 0;
  if (inside) {
    const int64_t p = (int64_t)py * W + px;
    T = final_T[p];
    last = last_idx[p];
    g0 = dL_dimage[3 * p + 0];
    g1 = dL_dimage[3 * p + 1];
    g2 = dL_dimage[3 * p + 2];
  }
  // colour accumulated behind the current splat, background included
  float R0 = T * bg0, R1 = T * bg1, R2 = T * bg2;
  if (tid == 0) s_maxlast = 0;
  __syncthreads();
  if (last) atomicMax(&s_maxlast, last);
  __syncthreads();
  const uint32_t stop = start + s_maxlast;  // nothing at or after this is blended
  if (stop > end) return;  // inconsistent inputs: leave gradients untouched

  for (uint32_t b_end = stop; b_end > start;) {
    const uint32_t b_begin = (b_end - start) > 256u ? b_end - 256u : start;
    const int n = (int)(b_end - b_begin);
    __syncthreads();
    if (tid < n) {
      const uint32_t id = ids[b_end - 1u - (uint32_t)tid];  // slot k = tid: back to front
      s_id[tid] = id;
      stage_splat(s_sp[tid], id, ld, means2d, conics, opac, colors, nullptr);
    }
    __syncthreads();
    for (int k = 0; k < n; ++k) {
      const SplatLds& s = s_sp[k];
      const uint32_t rel = b_end - 1u - (uint32_t)k - start;  // list position in the tile
      float f[kFields] = {0, 0, 0, 0, 0, 0, 0, 0, 0};
      bool hit = inside && rel < last;
      if (hit) {
        const float dx = fpx - s.u, dy = fpy - s.v;
        const float p2 = splat_power2(s, dx, dy);
        const float G = __builtin_amdgcn_exp2f(p2);
        const float oG = s.o * G;
        const bool clamped = oG > st.alpha_max;
        const float alpha = clamped ? st.alpha_max : oG;
        hit = !(p2 > 0.0f) && !(alpha < st.alpha_min);
        if (hit) {
          const float om = 1.0f - alpha;
          const float rom = 1.0f / om;
          T = T * rom;  // transmittance in front of this splat
          const float wgt = alpha * T;
          f[6] = g0 * wgt;
          f[7] = g1 * wgt;
          f[8] = g2 * wgt;
          // dC/dalpha = c T - R / (1 - alpha)
          float dLda = g0 * fmaf(s.r, T, -R0 * rom);
          dLda = fmaf(g1, fmaf(s.g, T, -R1 * rom), dLda);
          dLda = fmaf(g2, fmaf(s.b, T, -R2 * rom), dLda);
          R0 = fmaf(s.r, wgt, R0);
          R1 = fmaf(s.g, wgt, R1);
          R2 = fmaf(s.b, wgt, R2);
          if (!clamped) {
            // q = A dx^2 + 2B dx dy + C dy^2, alpha = o exp(-q/2)
            const float dLdq = -0.5f * alpha * dLda;
            const float A = s.qa * (-2.0f / kLog2e), B = s.qb * (-1.0f / kLog2e),
                        C = s.qc * (-2.0f / kLog2e);
            f[0] = dLdq * (-2.0f * fmaf(A, dx, B * dy));
            f[1] = dLdq * (-2.0f * fmaf(B, dx, C * dy));
            f[2] = dLdq * (dx * dx);
            f[3] = dLdq * (2.0f * dx * dy);
            f[4] = dLdq * (dy * dy);
            f[5] = dLda * G;
          }
        }
      }
      if (__ballot(hit) != 0ull) {
#pragma unroll
        for (int q = 0; q < kFields; ++q) {
          const float r = wave_sum_lane63(f[q]);
          if (lane == 63) s_part[wave][q][k] = r;
        }
      } else if (lane == 0) {
#pragma unroll
        for (int q = 0; q < kFields; ++q) s_part[wave][q][k] = 0.0f;
      }
    }
    __syncthreads();
    if (tid < n) {
      const uint32_t id = s_id[tid];
      float acc[kFields];
#pragma unroll
      for (int q = 0; q < kFields; ++q)
        acc[q] = (s_part[0][q][tid] + s_part[1][q][tid]) + (s_part[2][q][tid] + s_part[3][q][tid]);
      if (acc[0] != 0.0f) atomicAdd(&g_m2[id], acc[0]);
      if (acc[1] != 0.0f) atomicAdd(&g_m2[ld + id], acc[1]);
      if (acc[2] != 0.0f) atomicAdd(&g_con[id], acc[2]);
      if (acc[3] != 0.0f) atomicAdd(&g_con[ld + id], acc[3]);
      if (acc[4] != 0.0f) atomicAdd(&g_con[2 * ld + id], acc[4]);
      if (acc[5] != 0.0f) atomicAdd(&g_op[id], acc[5]);
      if (acc[6] != 0.0f) atomicAdd(&g_col[id], acc[6]);
      if (acc[7] != 0.0f) atomicAdd(&g_col[ld + id], acc[7]);
      if (acc[8] != 0.0f) atomicAdd(&g_col[2 * ld + id], acc[8]);
    }
    b_end = b_begin;
  }
}

__global__ void fill_f32_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.0f;
}

__global__ __launch_bounds__(256) void loss_grad_kernel(int kind, int64_t n,
                                                        const float* __restrict__ img,
                                                        const float* __restrict__ tgt,
                                                        float* __restrict__ g,
                                                        float* __restrict__ loss) {
  float acc = 0.0f;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const float r = img[i] - tgt[i];
    if (kind == 0) {
      g[i] = 2.0f * r;
      acc = fmaf(r, r, acc);
    } else {
      g[i] = r > 0.0f ? 1.0f : (r < 0.0f ? -1.0f : 0.0f);
      acc += fabsf(r);
    }
  }
  if (loss) {
    const float w = wave_sum_lane63(acc);
    if ((threadIdx.x & 63) == 63) atomicAdd(loss, w);
  }
}

static hipError_t zero_f32(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace gs

extern "C" hipError_t gs_launch_raster_fwd(int32_t W, int32_t H, const uint32_t* ranges,
                                           const uint32_t* ids, int64_t ld, const float* means2d,
                                           const float* conics, const float* opac,
                                           const float* colors, const float* depths,
                                           const float* bg, const gs::Settings& st, float* image,
                                           float* final_T, uint32_t* last_idx, float* out_depth,
                                           float* out_alpha, hipStream_t s) {
  const int gx = gs::grid_dim(W), gy = gs::grid_dim(H);
  hipLaunchKernelGGL(gs::raster_fwd_kernel, dim3((unsigned)(gx * gy)), dim3(256), 0, s, W, H, gx,
                     ranges, ids, ld, means2d, conics, opac, colors,
                     out_depth ? depths : nullptr, bg[0], bg[1], bg[2], st, image, final_T,
                     last_idx, out_depth, out_alpha);
  return hipGetLastError();
}

extern "C" hipError_t gs_launch_raster_bwd(int64_t N, int32_t W, int32_t H, const uint32_t* ranges,
                                           const uint32_t* ids, int64_t ld, const float* means2d,
                                           const float* conics, const float* opac,
                                           const float* colors, const float* bg,
                                           const gs::Settings& st, const float* final_T,
                                           const uint32_t* last_idx, const float* dL_dimage,
                                           float* g_m2, float* g_con, float* g_op, float* g_col,
                                           int accumulate, hipStream_t s) {
  hipError_t e;
  if (!accumulate) {
    for (int k = 0; k < 2; ++k)
      if ((e = gs::zero_f32(g_m2 + k * ld, N, s)) != hipSuccess) return e;
    for (int k = 0; k < 3; ++k)
      if ((e = gs::zero_f32(g_con + k * ld, N, s)) != hipSuccess) return e;
    if ((e = gs::zero_f32(g_op, N, s)) != hipSuccess) return e;
    for (int k = 0; k < 3; ++k)
      if ((e = gs::zero_f32(g_col + k * ld, N, s)) != hipSuccess) return e;
  }
  const int gx = gs::grid_dim(W), gy = gs::grid_dim(H);
  hipLaunchKernelGGL(gs::raster_bwd_kernel, dim3((unsigned)(gx * gy)), dim3(256), 0, s, W, H, gx,
                     ranges, ids, ld, means2d, conics, opac, colors, bg[0], bg[1], bg[2], st,
                     final_T, last_idx, dL_dimage, g_m2, g_con, g_op, g_col);
  return hipGetLastError();
}

extern "C" hipError_t gs_launch_loss_grad(int kind, int64_t n, const float* img, const float* tgt,
                                          float* g, float* loss, hipStream_t s) {
  hipError_t e;
  if (loss && (e = gs::zero_f32(loss, 1, s)) != hipSuccess) return e;
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(gs::loss_grad_kernel, dim3((unsigned)blocks), dim3(256), 0, s, kind, n, img,
                     tgt, g, loss);
  return hipGetLastError();
}
