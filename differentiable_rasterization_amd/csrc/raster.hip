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
// Each staged batch is compacted per wavefront: a splat enters a wave's list
// only if its alpha >= alpha_min footprint (a padded, conservative box) can
// reach one of that wave's four pixel rows, so waves skip splats that cannot
// touch them; the inner loops are branch-free.
//
// The backward walks the same lists back to front from each pixel's last
// blended entry.  Per splat each wave reduces its 64 pixels' nine gradient
// terms with two gfx950 lane-swap transpose steps and a DPP row scan
// (skipped with a ballot when no lane of the wave touched the splat); the
// wave partials meet in LDS and one lane per splat issues at most nine fp32
// atomics per tile, instead of one per pixel.
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
                                   const float* __restrict__ depths, float& A, float& B,
                                   float& C) {
  s.u = means2d[id];
  s.v = means2d[ld + id];
  A = conics[id];
  B = conics[ld + id];
  C = conics[2 * ld + id];
  s.qa = (-0.5f * kLog2e) * A;
  s.qb = (-kLog2e) * B;
  s.qc = (-0.5f * kLog2e) * C;
  s.o = opac[id];
  s.r = colors[id];
  s.g = colors[ld + id];
  s.b = colors[2 * ld + id];
  s.z = depths ? depths[id] : 0.0f;
}

// Which of the tile's four 4-row bands (one wavefront each) can hold a pixel
// centre where the splat reaches alpha_min.  alpha >= alpha_min needs
// q <= Q = 2 ln(o / alpha_min); the ellipse {q <= Q} lies inside
// |dx| <= sqrt(Q Sxx), |dy| <= sqrt(Q Syy) with S = conic^-1.  Q and the
// extents are padded (2% + constants) so that fp32 rounding of the pixel test
// can never reach alpha_min outside the box: a skipped pair is one the
// forward would have skipped too.  Ill-conditioned conics keep every band.
__device__ inline uint32_t band_mask(const SplatLds& s, float A, float B, float C,
                                     float alpha_min, int tx0, int ty0) {
  if (!(s.o >= alpha_min)) return 0u;  // alpha <= o everywhere
  const float tr = A + C;
  const float det = A * C - B * B;
  if (!(det > 1e-4f * tr * tr)) return 0xFu;
  const float Q = fmaf(2.0f * (__logf(s.o) - __logf(alpha_min)), 1.02f, 0.05f);
  const float ex = sqrtf(Q * (C / det)) + 0.02f;
  const float ey = sqrtf(Q * (A / det)) + 0.02f;
  const float x0 = (float)tx0 + 0.5f, x1 = (float)tx0 + 15.5f;
  if (!(s.u + ex >= x0 && s.u - ex <= x1)) return 0u;
  uint32_t m = 0u;
#pragma unroll
  for (int bnd = 0; bnd < 4; ++bnd) {
    const float y0 = (float)(ty0 + 4 * bnd) + 0.5f, y1 = y0 + 3.0f;
    if (s.v + ey >= y0 && s.v - ey <= y1) m |= 1u << bnd;
  }
  return m;
}

__device__ inline uint64_t lanemask_lt64() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Order-preserving compaction of the batch slots by band: s_list[b] receives
// the slots whose mask has bit b, in ascending slot order; s_cnt[b] their
// number.  Called by all 256 threads.
__device__ inline void compact_bands(uint32_t mask, uint8_t (*s_list)[256], uint32_t* s_cnt,
                                     uint32_t (*s_wc)[4]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t lt = lanemask_lt64();
  uint32_t pre[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint64_t bal = __ballot((mask >> b) & 1u);
    pre[b] = (uint32_t)__popcll(bal & lt);
    if (lane == 0) s_wc[b][wave] = (uint32_t)__popcll(bal);
  }
  __syncthreads();
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    if ((mask >> b) & 1u) {
      uint32_t off = pre[b];
      for (int w = 0; w < wave; ++w) off += s_wc[b][w];
      s_list[b][off] = (uint8_t)tid;
    }
  }
  if (tid < 4) s_cnt[tid] = s_wc[tid][0] + s_wc[tid][1] + s_wc[tid][2] + s_wc[tid][3];
  __syncthreads();
}

// log2 of the Gaussian at pixel offset (dx, dy): -log2e * q / 2.
__device__ inline float splat_power2(const SplatLds& s, float dx, float dy) {
  return fmaf(s.qa * dx, dx, fmaf(s.qc * dy, dy, s.qb * (dx * dy)));
}

// Work counters (optional diagnostics, one atomic per workgroup):
//   [0] pixel-splat pairs the kernel evaluated (after the band culling),
//   [1] pairs blended (alpha >= alpha_min before the pixel's stop),
//   [2] pairs the plain method evaluates: per pixel, its tile's entries up to
//       and including the one that stops it (all of them if none does),
//   [3] wavefront reductions executed (backward only).
__device__ inline void add_counters(uint64_t* cnt, uint64_t a, uint64_t b, uint64_t c,
                                    uint64_t d) {
  __shared__ uint64_t s_c[4];
  if (threadIdx.x < 4) s_c[threadIdx.x] = 0;
  __syncthreads();
  if (a) atomicAdd((unsigned long long*)&s_c[0], (unsigned long long)a);
  if (b) atomicAdd((unsigned long long*)&s_c[1], (unsigned long long)b);
  if (c) atomicAdd((unsigned long long*)&s_c[2], (unsigned long long)c);
  if (d) atomicAdd((unsigned long long*)&s_c[3], (unsigned long long)d);
  __syncthreads();
  if (threadIdx.x < 4 && s_c[threadIdx.x])
    atomicAdd((unsigned long long*)&cnt[threadIdx.x], (unsigned long long)s_c[threadIdx.x]);
}

template <bool kDepth, bool kStats>
__global__ __launch_bounds__(256) void raster_fwd_kernel(
    int W, int H, int gx, const uint32_t* __restrict__ ranges, const uint32_t* __restrict__ ids,
    int64_t ld, const float* __restrict__ means2d, const float* __restrict__ conics,
    const float* __restrict__ opac, const float* __restrict__ colors,
    const float* __restrict__ depths, float bg0, float bg1, float bg2, Settings st,
    float* __restrict__ image, float* __restrict__ final_T, uint32_t* __restrict__ last_idx,
    float* __restrict__ out_depth, float* __restrict__ out_alpha, uint64_t* __restrict__ cnt) {
  __shared__ SplatLds s_sp[256];
  __shared__ uint8_t s_list[4][256];
  __shared__ uint32_t s_cnt[4];
  __shared__ uint32_t s_wc[4][4];
  const int tile = blockIdx.x;
  const int tx = tile % gx, ty = tile / gx;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int px = tx * kTile + (tid & 15), py = ty * kTile + (tid >> 4);
  const bool inside = px < W && py < H;
  const float fpx = (float)px + 0.5f, fpy = (float)py + 0.5f;
  const uint32_t start = ranges[2 * tile], end = ranges[2 * tile + 1];
  const float amin = st.alpha_min, amax = st.alpha_max, Tmin = st.T_min;

  float T = 1.0f, C0 = 0.0f, C1 = 0.0f, C2 = 0.0f, D = 0.0f;
  uint32_t last = 0;
  bool done = !inside;
  uint32_t n_eval = 0, n_blend = 0, stop_at = 0;  // counters (kStats only)
  for (uint32_t b = start; b < end; b += 256) {
    if (__syncthreads_count(done) == 256) break;
    const uint32_t j = b + (uint32_t)tid;
    uint32_t mask = 0u;
    if (j < end) {
      float A, B, C;
      stage_splat(s_sp[tid], ids[j], ld, means2d, conics, opac, colors,
                  kDepth ? depths : nullptr, A, B, C);
      mask = band_mask(s_sp[tid], A, B, C, amin, tx * kTile, ty * kTile);
    }
    compact_bands(mask, s_list, s_cnt, s_wc);
    const int cnt = (int)s_cnt[wave];
    const uint32_t base = b - start + 1u;
    if (__ballot(!done) == 0ull) continue;
    for (int i = 0; i < cnt; ++i) {
      const int k = s_list[wave][i];
      const SplatLds& s = s_sp[k];
      const float dx = fpx - s.u, dy = fpy - s.v;
      const float p2 = splat_power2(s, dx, dy);
      const float oG = s.o * __builtin_amdgcn_exp2f(p2);
      const float alpha = oG > amax ? amax : oG;
      const bool ok = !done & !(p2 > 0.0f) & !(alpha < amin);
      const float Tn = T * (1.0f - alpha);
      const bool low = Tn < Tmin;
      const bool blend = ok & !low;
      if (kStats) {
        n_eval += 1u;
        n_blend += blend ? 1u : 0u;
        stop_at = (ok & low) ? base + (uint32_t)k : stop_at;
      }
      done = done | (ok & low);
      const float w = blend ? alpha * T : 0.0f;
      C0 = fmaf(s.r, w, C0);
      C1 = fmaf(s.g, w, C1);
      C2 = fmaf(s.b, w, C2);
      if (kDepth) D = fmaf(s.z, w, D);
      T = blend ? Tn : T;
      last = blend ? base + (uint32_t)k : last;
    }
  }
  if (kStats) {
    const uint32_t plain = inside ? (stop_at ? stop_at : end - start) : 0u;
    add_counters(cnt, inside ? n_eval : 0u, n_blend, plain, 0u);
  }
  if (!inside) return;
  const int64_t p = (int64_t)py * W + px;
  image[3 * p + 0] = fmaf(T, bg0, C0);
  image[3 * p + 1] = fmaf(T, bg1, C1);
  image[3 * p + 2] = fmaf(T, bg2, C2);
  final_T[p] = T;
  last_idx[p] = last;
  if (kDepth) out_depth[p] = D;
  if (out_alpha) out_alpha[p] = 1.0f - T;
}

// ---------------------------------------------------------------------------
// Wavefront reduction of nine fields: two transpose steps with the gfx950
// lane swaps (v_permlane32_swap exchanges the upper half of one register
// with the lower half of another, v_permlane16_swap the odd 16-lane rows of
// one with the even rows of another), so that after them every 16-lane row
// of a register carries one field; then an inclusive DPP row scan leaves each
// row's total in its lane 15.  About 30 instructions instead of six DPP
// steps per field.
// ---------------------------------------------------------------------------
__device__ inline float swap_add32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float swap_add16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
#define GS_ROW_ADD(v, ctrl)                                                                \
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(                              \
                                     0, __builtin_bit_cast(int, v), ctrl, 0xF, 0xF, true))
__device__ inline float row_total_lane15(float v) {
  GS_ROW_ADD(v, 0x111);  // row_shr:1
  GS_ROW_ADD(v, 0x112);  // row_shr:2
  GS_ROW_ADD(v, 0x114);  // row_shr:4
  GS_ROW_ADD(v, 0x118);  // row_shr:8
  return v;
}
#undef GS_ROW_ADD

// Sums f[0..8] over the wavefront and stores field q at dst[q * stride].
__device__ inline void reduce9_store(const float f[9], float* dst, int stride) {
  const float s01 = swap_add32(f[0], f[1]);
  const float s23 = swap_add32(f[2], f[3]);
  const float s45 = swap_add32(f[4], f[5]);
  const float s67 = swap_add32(f[6], f[7]);
  const float s8 = swap_add32(f[8], 0.0f);
  // rows of t0: fields 0, 2, 1, 3; of t1: 4, 6, 5, 7; of t2: 8, -, -, -
  float t0 = swap_add16(s01, s23);
  float t1 = swap_add16(s45, s67);
  float t2 = swap_add16(s8, 0.0f);
  t0 = row_total_lane15(t0);
  t1 = row_total_lane15(t1);
  t2 = row_total_lane15(t2);
  const int lane = threadIdx.x & 63;
  if ((lane & 15) == 15) {
    const int row = lane >> 4;
    const int q = (row == 1) ? 2 : (row == 2 ? 1 : row);
    dst[q * stride] = t0;
    dst[(4 + q) * stride] = t1;
    if (row == 0) dst[8 * stride] = t2;
  }
}

// Gradient slots of one splat, in moment form: m dx, m dy, m dx^2, m dx dy,
// m dy^2 with m = dL/dq, then dL/do and the three colour gradients.  The
// mean and conic gradients follow after the reduction:
//   dL/du = -2 (A Sx + B Sy), dL/dv = -2 (B Sx + C Sy),
//   dL/dA = Sxx, dL/dB = 2 Sxy, dL/dC = Syy.
constexpr int kFields = 9;

template <bool kStats>
__global__ __launch_bounds__(256) void raster_bwd_kernel(
    int W, int H, int gx, const uint32_t* __restrict__ ranges, const uint32_t* __restrict__ ids,
    int64_t ld, const float* __restrict__ means2d, const float* __restrict__ conics,
    const float* __restrict__ opac, const float* __restrict__ colors, float bg0, float bg1,
    float bg2, Settings st, const float* __restrict__ final_T,
    const uint32_t* __restrict__ last_idx, const float* __restrict__ dL_dimage,
    float* __restrict__ g_m2, float* __restrict__ g_con, float* __restrict__ g_op,
    float* __restrict__ g_col, uint64_t* __restrict__ cnt) {
  __shared__ SplatLds s_sp[256];
  __shared__ uint32_t s_id[256];
  __shared__ uint8_t s_mask[256];
  __shared__ uint8_t s_list[4][256];
  __shared__ uint32_t s_cnt[4];
  __shared__ uint32_t s_wc[4][4];
  __shared__ float s_part[4][kFields][256];
  __shared__ uint32_t s_maxlast;
  const int tile = blockIdx.x;
  const int tx = tile % gx, ty = tile / gx;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int px = tx * kTile + (tid & 15), py = ty * kTile + (tid >> 4);
  const bool inside = px < W && py < H;
  const float fpx = (float)px + 0.5f, fpy = (float)py + 0.5f;
  const uint32_t start = ranges[2 * tile], end = ranges[2 * tile + 1];
  const float amin = st.alpha_min, amax = st.alpha_max;

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
  uint32_t n_eval = 0, n_hit = 0, n_red = 0;  // counters (kStats only)

  for (uint32_t b_end = stop; b_end > start;) {
    const uint32_t b_begin = (b_end - start) > 256u ? b_end - 256u : start;
    const int n = (int)(b_end - b_begin);
    __syncthreads();
    uint32_t mask = 0u;
    if (tid < n) {
      const uint32_t id = ids[b_end - 1u - (uint32_t)tid];  // slot k = tid: back to front
      float A, B, C;
      s_id[tid] = id;
      stage_splat(s_sp[tid], id, ld, means2d, conics, opac, colors, nullptr, A, B, C);
      mask = band_mask(s_sp[tid], A, B, C, amin, tx * kTile, ty * kTile);
      s_mask[tid] = (uint8_t)mask;
    }
    compact_bands(mask, s_list, s_cnt, s_wc);
    const int cnt = (int)s_cnt[wave];
    const uint32_t relbase = b_end - 1u - start;
    for (int i = 0; i < cnt; ++i) {
      const int k = s_list[wave][i];
      const SplatLds& s = s_sp[k];
      const uint32_t rel = relbase - (uint32_t)k;  // list position in the tile
      const float dx = fpx - s.u, dy = fpy - s.v;
      const float p2 = splat_power2(s, dx, dy);
      const float G = __builtin_amdgcn_exp2f(p2);
      const float oG = s.o * G;
      const bool clamped = oG > amax;
      const float alpha = clamped ? amax : oG;
      const bool hit = (rel < last) & !(p2 > 0.0f) & !(alpha < amin);
      const float rom = __builtin_amdgcn_rcpf(1.0f - alpha);
      T = hit ? T * rom : T;  // transmittance in front of this splat
      const float wgt = hit ? alpha * T : 0.0f;
      float f[kFields];
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
      const bool geo = hit & !clamped;
      // q = A dx^2 + 2B dx dy + C dy^2, alpha = o exp(-q/2): dL/dq = -alpha/2 dL/dalpha
      const float m = geo ? (-0.5f * alpha) * dLda : 0.0f;
      f[5] = geo ? dLda * G : 0.0f;
      const float mx = m * dx, my = m * dy;
      f[0] = mx;
      f[1] = my;
      f[2] = mx * dx;
      f[3] = mx * dy;
      f[4] = my * dy;
      float* dst = &s_part[wave][0][k];
      if (kStats) {
        n_eval += inside ? 1u : 0u;
        n_hit += hit ? 1u : 0u;
      }
      if (__ballot(hit) != 0ull) {
        if (kStats) n_red += (lane == 0) ? 1u : 0u;
        reduce9_store(f, dst, 256);
      } else if (lane == 0) {
#pragma unroll
        for (int q = 0; q < kFields; ++q) dst[q * 256] = 0.0f;
      }
    }
    __syncthreads();
    if (tid < n) {
      const uint32_t id = s_id[tid];
      const uint32_t msk = s_mask[tid];
      float acc[kFields];
#pragma unroll
      for (int q = 0; q < kFields; ++q) acc[q] = 0.0f;
      for (int w = 0; w < 4; ++w)
        if ((msk >> w) & 1u)
#pragma unroll
          for (int q = 0; q < kFields; ++q) acc[q] += s_part[w][q][tid];
      const SplatLds& s = s_sp[tid];
      const float A = s.qa * (-2.0f / kLog2e), B = s.qb * (-1.0f / kLog2e),
                  C = s.qc * (-2.0f / kLog2e);
      const float gu = -2.0f * fmaf(A, acc[0], B * acc[1]);
      const float gv = -2.0f * fmaf(B, acc[0], C * acc[1]);
      const float gA = acc[2], gB = 2.0f * acc[3], gC = acc[4];
      if (gu != 0.0f) atomicAdd(&g_m2[id], gu);
      if (gv != 0.0f) atomicAdd(&g_m2[ld + id], gv);
      if (gA != 0.0f) atomicAdd(&g_con[id], gA);
      if (gB != 0.0f) atomicAdd(&g_con[ld + id], gB);
      if (gC != 0.0f) atomicAdd(&g_con[2 * ld + id], gC);
      if (acc[5] != 0.0f) atomicAdd(&g_op[id], acc[5]);
      if (acc[6] != 0.0f) atomicAdd(&g_col[id], acc[6]);
      if (acc[7] != 0.0f) atomicAdd(&g_col[ld + id], acc[7]);
      if (acc[8] != 0.0f) atomicAdd(&g_col[2 * ld + id], acc[8]);
    }
    b_end = b_begin;
  }
  if (kStats) add_counters(cnt, n_eval, n_hit, 0u, n_red);
}

// Zero the first n entries of nine gradient planes in one launch.
struct ZeroPlanes {
  float* p[9];
};
__global__ void zero_planes_kernel(ZeroPlanes z, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
#pragma unroll
    for (int k = 0; k < 9; ++k) z.p[k][i] = 0.0f;
}

__global__ void zero_f32_kernel(float* __restrict__ p) { *p = 0.0f; }

// dL/dimage and (optionally) the summed loss: per-lane partial sums, a DPP
// row reduction, a cross-wave sum in LDS, then one atomic per workgroup.
__global__ __launch_bounds__(256) void loss_grad_kernel(int kind, int64_t n,
                                                        const float* __restrict__ img,
                                                        const float* __restrict__ tgt,
                                                        float* __restrict__ g,
                                                        float* __restrict__ loss) {
  __shared__ float s_w[16];
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
  if (!loss) return;
  acc = row_total_lane15(acc);
  const int lane = threadIdx.x & 63;
  if ((lane & 15) == 15) s_w[threadIdx.x >> 4] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.0f;
    for (int k = 0; k < 16; ++k) t += s_w[k];
    atomicAdd(loss, t);
  }
}

}  // namespace gs

extern "C" hipError_t gs_launch_raster_fwd(int32_t W, int32_t H, const uint32_t* ranges,
                                           const uint32_t* ids, int64_t ld, const float* means2d,
                                           const float* conics, const float* opac,
                                           const float* colors, const float* depths,
                                           const float* bg, const gs::Settings& st, float* image,
                                           float* final_T, uint32_t* last_idx, float* out_depth,
                                           float* out_alpha, uint64_t* counters, hipStream_t s) {
  const int gx = gs::grid_dim(W), gy = gs::grid_dim(H);
  const dim3 grid((unsigned)(gx * gy)), block(256);
  if (counters) {
    if (out_depth)
      hipLaunchKernelGGL((gs::raster_fwd_kernel<true, true>), grid, block, 0, s, W, H, gx, ranges,
                         ids, ld, means2d, conics, opac, colors, depths, bg[0], bg[1], bg[2], st,
                         image, final_T, last_idx, out_depth, out_alpha, counters);
    else
      hipLaunchKernelGGL((gs::raster_fwd_kernel<false, true>), grid, block, 0, s, W, H, gx, ranges,
                         ids, ld, means2d, conics, opac, colors, nullptr, bg[0], bg[1], bg[2], st,
                         image, final_T, last_idx, nullptr, out_alpha, counters);
  } else {
    if (out_depth)
      hipLaunchKernelGGL((gs::raster_fwd_kernel<true, false>), grid, block, 0, s, W, H, gx, ranges,
                         ids, ld, means2d, conics, opac, colors, depths, bg[0], bg[1], bg[2], st,
                         image, final_T, last_idx, out_depth, out_alpha, nullptr);
    else
      hipLaunchKernelGGL((gs::raster_fwd_kernel<false, false>), grid, block, 0, s, W, H, gx,
                         ranges, ids, ld, means2d, conics, opac, colors, nullptr, bg[0], bg[1],
                         bg[2], st, image, final_T, last_idx, nullptr, out_alpha, nullptr);
  }
  return hipGetLastError();
}

extern "C" hipError_t gs_launch_raster_bwd(int64_t N, int32_t W, int32_t H, const uint32_t* ranges,
                                           const uint32_t* ids, int64_t ld, const float* means2d,
                                           const float* conics, const float* opac,
                                           const float* colors, const float* bg,
                                           const gs::Settings& st, const float* final_T,
                                           const uint32_t* last_idx, const float* dL_dimage,
                                           float* g_m2, float* g_con, float* g_op, float* g_col,
                                           int accumulate, uint64_t* counters, hipStream_t s) {
  if (N > 0) {
    // the 2D gradients are per call; the opacity gradient is a parameter
    // gradient and keeps its contents when accumulating
    gs::ZeroPlanes z = {{g_m2, g_m2 + ld, g_con, g_con + ld, g_con + 2 * ld, g_col, g_col + ld,
                         g_col + 2 * ld, accumulate ? g_col : g_op}};
    int64_t blocks = (N + 255) / 256;
    if (blocks > 2048) blocks = 2048;
    hipLaunchKernelGGL(gs::zero_planes_kernel, dim3((unsigned)blocks), dim3(256), 0, s, z, N);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int gx = gs::grid_dim(W), gy = gs::grid_dim(H);
  const dim3 grid((unsigned)(gx * gy)), block(256);
  if (counters)
    hipLaunchKernelGGL(gs::raster_bwd_kernel<true>, grid, block, 0, s, W, H, gx, ranges, ids, ld,
                       means2d, conics, opac, colors, bg[0], bg[1], bg[2], st, final_T, last_idx,
                       dL_dimage, g_m2, g_con, g_op, g_col, counters);
  else
    hipLaunchKernelGGL(gs::raster_bwd_kernel<false>, grid, block, 0, s, W, H, gx, ranges, ids, ld,
                       means2d, conics, opac, colors, bg[0], bg[1], bg[2], st, final_T, last_idx,
                       dL_dimage, g_m2, g_con, g_op, g_col, nullptr);
  return hipGetLastError();
}

extern "C" hipError_t gs_launch_loss_grad(int kind, int64_t n, const float* img, const float* tgt,
                                          float* g, float* loss, hipStream_t s) {
  if (loss) {
    hipLaunchKernelGGL(gs::zero_f32_kernel, dim3(1), dim3(1), 0, s, loss);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(gs::loss_grad_kernel, dim3((unsigned)blocks), dim3(256), 0, s, kind, n, img,
                     tgt, g, loss);
  return hipGetLastError();
}
