// raster.hip — stage 4 (front-to-back compositing) and stage 5a (its
// backward), plus the image loss gradient.
//
// One 256-lane workgroup (four wave64) per 16x16 tile, one lane per pixel;
// a wave covers one 8x8 quadrant of the tile.  The tile's depth-sorted list
// is walked in batches of 256 splats that the workgroup first stages into
// LDS (one gather per lane), after which every lane reads the batch with
// LDS loads.  The work is bound by VALU issue (about a dozen operations per
// pixel-splat pair plus one or two transcendentals), not by memory, so
// nothing here is shaped for MFMA.  The forward stops the whole tile as soon
// as every pixel has terminated.  With a schedule (tile_order_kernel, below)
// workgroups take the tiles with the longest lists first.
//
// Each staged batch is compacted: a splat enters a list only if its
// alpha >= alpha_min footprint (a padded, conservative box) can reach the
// list's pixels, so lanes skip splats that cannot touch them; the inner
// loops are branch-free.  The backward keeps one list per wave (its 8x8
// quadrant); the forward one per 4x4 block, each 16-lane row of a wave
// walking its own block's list.
//
// The backward walks the same lists back to front from each pixel's last
// blended entry.  Per splat each wave reduces its 64 pixels' nine gradient
// terms with two gfx950 lane-swap transpose steps, an 8-lane merge and DPP
// half-row totals (skipped with a ballot when no lane of the wave touched
// the splat); the wave partials meet in LDS and the tile stores its sums for
// the splat, with a plain 48-byte store, into the instance's own slot (the
// Gaussian's offset plus the tile's index in its rect; slots are packed 48
// bytes apart, so no line carries unused bytes).  A second kernel adds each
// Gaussian's slots in a fixed order.  No global atomics: device-scope float
// atomics go to memory on this part, and a fixed order makes gradients
// reproducible.
//
// The calls take the projection's planes; pack_splats_kernel first stages
// each visible row into a 64-byte record in the caller's workspace, so that
// staging a tile instance costs one cache line.
//
// Decisions (alpha < alpha_min, alpha clamp, stop at T < T_min) are
// taken by the same inline code in both kernels, compiled without
// contraction, so the backward replays exactly the forward's choices.
#include "gs_common.h"

namespace gs {

// Splat staged in LDS: mean, the conic's Cholesky factor scaled by
// sqrt(log2(e)/2) (l11, l21, l22: the Gaussian is exp2(-(e1^2 + e2^2)) with
// e1 = l11 dx + l21 dy, e2 = l22 dy), opacity, colour, and z: the depth in
// the forward, 1/opacity in the backward.
struct SplatLds {
  float u, v, l11, l21, l22, o, r, g, b, z;
};

// A splat record (its first three 16-byte quarters, plus the depth when the
// forward outputs depth) held in registers between its global load and its
// staging into LDS; the forward fetches the next batch's records this way.
struct RecordRegs {
  float4 a, b, c;
  float z;
  __device__ inline void load(const float4* __restrict__ splats, const float* __restrict__ depths,
                              uint32_t id, bool with_depth) {
    const float4* r = splats + 4 * (size_t)id;
    a = r[0];
    b = r[1];
    c = r[2];
    z = with_depth ? depths[id] : 0.0f;
  }
  __device__ inline void stage(SplatLds& s, int32_t& radius, float& ex, float& ey) const {
    s.u = a.x; s.v = a.y; s.l11 = a.z; s.l21 = a.w;
    s.l22 = b.x; s.o = b.y; s.r = b.z; s.g = b.w;
    s.b = c.x; s.z = z;
    radius = __float_as_int(c.y);
    ex = c.z;
    ey = c.w;
  }
};

// Padded half-extents of the footprint where alpha = o exp(-q/2) can reach
// alpha_min: q <= Q = 2 ln(o / alpha_min), whose ellipse lies inside
// |dx| <= sqrt(Q a), |dy| <= sqrt(Q c) for the 2D covariance (a, b, c) =
// conic^-1.  From the conic's Cholesky factor L (conic = L L^T) without
// cancellation: c = 1 / L22^2, a = (1 + (L21 / L22)^2) / L11^2, and
// det = 1 / (L11 L22)^2.  Q and the extents are padded (2% + constants) so
// that the compositing kernels' fp32 pixel test can never reach alpha_min
// outside the box; nearly singular covariances (det <= 1e-4 (a + c)^2,
// condition numbers above ~1e4) are left unbounded.  Negative: the Gaussian
// never reaches alpha_min (o < alpha_min).
__device__ inline void footprint(float L11, float L21, float L22, float o, float alpha_min,
                                 float& ex, float& ey) {
  if (!(o >= alpha_min)) {
    ex = ey = -1.0f;
    return;
  }
  const float t = L21 / L22;
  const float c = 1.0f / (L22 * L22);
  const float a = fmaf(t, t, 1.0f) / (L11 * L11);
  const float det = 1.0f / ((L11 * L22) * (L11 * L22));
  const float tr = a + c;
  if (!(det > 1e-4f * tr * tr)) {
    ex = ey = __builtin_inff();
    return;
  }
  const float Q = fmaf(2.0f * (__logf(o) - __logf(alpha_min)), 1.02f, 0.05f);
  ex = sqrtf(Q * a) + 0.02f;
  ey = sqrtf(Q * c) + 0.02f;
}

// Stages row r of the projection's planes into record r of rec when its
// radius is > 0 (rows of other Gaussians are never referenced by a tile
// list).  Row r is Gaussian i = r % ld seen by camera c = r / ld (one camera:
// r < ld); plane p of camera c starts at c * P * ld + p * ld, opacities are
// per Gaussian.  Record: u, v, k L11, k L21, k L22 (k = sqrt(log2(e) / 2), so
// that the Gaussian is exp2(-(e1^2 + e2^2))), opacity, colour, radius,
// footprint extents, conic.
__global__ __launch_bounds__(256) void pack_splats_kernel(
    int64_t rows, int64_t ld, const float* __restrict__ means2d, const float* __restrict__ conics,
    const float* __restrict__ chol, const float* __restrict__ opac,
    const float* __restrict__ colors, const int32_t* __restrict__ radii, float alpha_min,
    float4* __restrict__ rec) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  const int32_t rad = radii[r];
  if (rad <= 0) return;
  const int64_t c = r / ld, i = r - c * ld;
  const float* m2 = means2d + c * 2 * ld + i;
  const float* cn = conics + c * 3 * ld + i;
  const float* ch = chol + c * 3 * ld + i;
  const float* co = colors + c * 3 * ld + i;
  const float L11 = ch[0], L21 = ch[ld], L22 = ch[2 * ld];
  const float o = opac[i];
  float ex, ey;
  footprint(L11, L21, L22, o, alpha_min, ex, ey);
  float4* out = rec + 4 * r;
  out[0] = make_float4(m2[0], m2[ld], kSqrtHalfLog2e * L11, kSqrtHalfLog2e * L21);
  out[1] = make_float4(kSqrtHalfLog2e * L22, o, co[0], co[ld]);
  out[2] = make_float4(co[2 * ld], __int_as_float(rad), ex, ey);
  out[3] = make_float4(cn[0], cn[ld], cn[2 * ld], 0.0f);
}

// Workgroup -> tile mapping aware of the eight XCDs (each with its own L2):
// workgroup b runs on XCD b % 8, so each XCD is handed whole 2x2 groups of
// tiles (group x, x + 8, x + 16, ... for XCD x).  A splat that overlaps
// neighbouring tiles of a group is then fetched into one L2, while groups
// stay interleaved over the image for load balance.  Workgroups past the
// tile grid return at once.
constexpr int kXcds = 8, kGroupW = 2, kGroupH = 2, kGroup = kGroupW * kGroupH;

__host__ __device__ inline int tile_groups(int gx, int gy) {
  return ((gx + kGroupW - 1) / kGroupW) * ((gy + kGroupH - 1) / kGroupH);
}
__host__ inline unsigned tile_grid_blocks(int gx, int gy) {
  const int ng = tile_groups(gx, gy);
  return (unsigned)(((ng + kXcds - 1) / kXcds) * kXcds * kGroup);
}
__device__ inline bool block_tile(int b, int gx, int gy, int& tx, int& ty) {
  const int xcd = b % kXcds, l = b / kXcds;
  const int group = (l / kGroup) * kXcds + xcd, within = l % kGroup;
  const int ggx = (gx + kGroupW - 1) / kGroupW;
  tx = (group % ggx) * kGroupW + within % kGroupW;
  ty = (group / ggx) * kGroupH + within / kGroupW;
  return tx < gx && ty < gy;
}

// Tile of this workgroup: with a schedule (tile_order_kernel), workgroup b
// of camera c takes tile order[c * T + b], so that the longest lists start
// first; without one, the XCD-aware mapping above.  Workgroups past the last
// tile, and entries that are no tile index, return at once.
__device__ inline bool schedule_tile(const uint32_t* __restrict__ order, int gx, int gy, int& tx,
                                     int& ty) {
  if (!order) return block_tile((int)blockIdx.x, gx, gy, tx, ty);
  const int nt = gx * gy;
  if ((int)blockIdx.x >= nt) return false;
  const uint32_t t = order[(int64_t)blockIdx.y * nt + blockIdx.x];
  if (t >= (uint32_t)nt) return false;
  tx = (int)t % gx;
  ty = (int)t / gx;
  return true;
}

// Schedule bucket of a tile with n list entries: n itself below 8, else
// eight buckets per power of two (about 12% apart), so 256 buckets cover
// any 32-bit length.
__device__ inline uint32_t length_bucket(uint32_t n) {
  if (n < 8u) return n;
  const uint32_t e = 31u - (uint32_t)__clz((int)n);  // 3 .. 31
  return (e - 2u) * 8u + ((n >> (e - 3u)) & 7u);
}

// Pixel of lane `tid` within its tile: wave w covers quadrant (w & 1, w >> 1),
// lane l its pixel (l & 7, l >> 3).
__device__ inline int quad_px(int tid) { return ((tid >> 6) & 1) * 8 + (tid & 7); }
__device__ inline int quad_py(int tid) { return (tid >> 7) * 8 + ((tid >> 3) & 7); }

// Which of the tile's four 8x8 quadrants (one wavefront each) can hold a
// pixel centre where the splat reaches alpha_min, from the record's padded
// footprint half-extents (a skipped pair is one the forward skips too).
__device__ inline uint32_t quad_mask(const SplatLds& s, float ex, float ey, int tx0, int ty0) {
  if (!(ex >= 0.0f)) return 0u;  // opacity below alpha_min
  const float xa = (float)tx0 + 0.5f, ya = (float)ty0 + 0.5f;
  // columns 0-7 and 8-15, rows 0-7 and 8-15 (pixel centres)
  const bool c0 = s.u + ex >= xa && s.u - ex <= xa + 7.0f;
  const bool c1 = s.u + ex >= xa + 8.0f && s.u - ex <= xa + 15.0f;
  const bool r0 = s.v + ey >= ya && s.v - ey <= ya + 7.0f;
  const bool r1 = s.v + ey >= ya + 8.0f && s.v - ey <= ya + 15.0f;
  return (uint32_t)(c0 & r0) | ((uint32_t)(c1 & r0) << 1) | ((uint32_t)(c0 & r1) << 2) |
         ((uint32_t)(c1 & r1) << 3);
}

// The forward's pixel layout: wave w covers quadrant (w & 1, w >> 1) as in
// the backward, but each 16-lane row r of it a 4x4 block of that quadrant,
// at (r & 1, r >> 1) in 4-pixel steps; lane j of the row takes pixel
// (j & 3, j >> 2) of the block.  Block index wave * 4 + r.
__device__ inline int sub_px(int tid) {
  return ((tid >> 6) & 1) * 8 + ((tid >> 4) & 1) * 4 + (tid & 3);
}
__device__ inline int sub_py(int tid) {
  return (tid >> 7) * 8 + ((tid >> 5) & 1) * 4 + ((tid >> 2) & 3);
}

// Which of the tile's sixteen 4x4 blocks (numbered as above) can hold a
// pixel centre where the splat reaches alpha_min, from the record's padded
// footprint half-extents.
__device__ inline uint32_t sub_mask(const SplatLds& s, float ex, float ey, int tx0, int ty0) {
  if (!(ex >= 0.0f)) return 0u;  // opacity below alpha_min
  const float xa = (float)tx0 + 0.5f, ya = (float)ty0 + 0.5f;
  uint32_t cx = 0u, cy = 0u;  // 4-pixel column and row bands the box reaches
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float x0 = xa + (float)(4 * i), y0 = ya + (float)(4 * i);
    cx |= (uint32_t)(s.u + ex >= x0 && s.u - ex <= x0 + 3.0f) << i;
    cy |= (uint32_t)(s.v + ey >= y0 && s.v - ey <= y0 + 3.0f) << i;
  }
  uint32_t m = 0u;
#pragma unroll
  for (int b = 0; b < 16; ++b) {
    const int w = b >> 2, r = b & 3;
    const int bx = (w & 1) * 2 + (r & 1), by = (w >> 1) * 2 + (r >> 1);
    m |= ((cx >> bx) & (cy >> by) & 1u) << b;
  }
  return m;
}

__device__ inline uint64_t lanemask_lt64() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Order-preserving compaction of the batch slots by quadrant: s_list[b] receives
// the slots whose mask has bit b, in ascending slot order; s_cnt[b] their
// number.  Called by all 256 threads.  s_wc[b][w] first holds wave w's
// count for band b, then (NB * 4 lanes, one pass) the count of the waves
// before it.
template <int NB, int LD>
__device__ inline void compact_bands(uint32_t mask, uint8_t (*s_list)[LD], uint32_t* s_cnt,
                                     uint32_t (*s_wc)[4]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t lt = lanemask_lt64();
  uint32_t pre[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const uint64_t bal = __ballot((mask >> b) & 1u);
    pre[b] = (uint32_t)__popcll(bal & lt);
    if (lane == 0) s_wc[b][wave] = (uint32_t)__popcll(bal);
  }
  __syncthreads();
  uint32_t c4 = 0, ex = 0;
  if (tid < NB * 4) {
    const int b = tid >> 2, w = tid & 3;
    const uint32_t c0 = s_wc[b][0], c1 = s_wc[b][1], c2 = s_wc[b][2], c3 = s_wc[b][3];
    ex = (w > 0 ? c0 : 0u) + (w > 1 ? c1 : 0u) + (w > 2 ? c2 : 0u);
    c4 = c0 + c1 + c2 + c3;
  }
  __syncthreads();
  if (tid < NB * 4) {
    s_wc[tid >> 2][tid & 3] = ex;
    if ((tid & 3) == 0) s_cnt[tid >> 2] = c4;
  }
  __syncthreads();
#pragma unroll
  for (int b = 0; b < NB; ++b)
    if ((mask >> b) & 1u) s_list[b][pre[b] + s_wc[b][wave]] = (uint8_t)tid;
  __syncthreads();
}

// log2 of the Gaussian at pixel offset (dx, dy): -log2e * q / 2, from the
// completed square (never positive).
__device__ inline float splat_power2(const SplatLds& s, float dx, float dy, float& e1,
                                     float& e2) {
  e1 = fmaf(s.l11, dx, s.l21 * dy);
  e2 = s.l22 * dy;
  return -fmaf(e1, e1, e2 * e2);
}
__device__ inline float splat_power2(const SplatLds& s, float dx, float dy) {
  float e1, e2;
  return splat_power2(s, dx, dy, e1, e2);
}

// Work counters (optional diagnostics, one atomic per workgroup):
//   [0] pixel-splat pairs the kernel evaluated (after the quadrant culling),
//   [1] pairs blended (alpha >= alpha_min before the pixel's stop),
//   [2] forward: pairs the plain per-pixel method evaluates (per pixel, its
//       tile's entries up to and including the one that stops it, all of
//       them if none does); backward: pairs the plain tile loop walks
//       (256 x the tile's entries up to its pixels' last blended one),
//   [3] forward: pairs the plain tile loop evaluates (256 x the tile's
//       entries up to the last of its pixels' stops); backward: wavefront
//       reductions executed.
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

// Inclusive DPP row scan: each 16-lane row's total lands in its lane 15.
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

__global__ void zero_f32_kernel(float* __restrict__ p) { *p = 0.0f; }

// Per-element loss gradient (kind 0: L2, 2 (x - y); kind 1: L1, sign(x - y)),
// adding the element's loss to acc.
__device__ inline float loss_term(int kind, float r, float& acc) {
  if (kind == 0) {
    acc = fmaf(r, r, acc);
    return 2.0f * r;
  }
  acc += fabsf(r);
  return r > 0.0f ? 1.0f : (r < 0.0f ? -1.0f : 0.0f);
}

template <bool kDepth, bool kStats>
__global__ __launch_bounds__(256) void raster_fwd_kernel(
    int W, int H, int gx, const uint32_t* __restrict__ ranges, const uint32_t* __restrict__ ids,
    const float4* __restrict__ splats, const float* __restrict__ depths, float bg0, float bg1,
    float bg2, Settings st, float* __restrict__ image, float* __restrict__ final_T,
    uint32_t* __restrict__ last_idx, float* __restrict__ out_depth,
    float* __restrict__ out_alpha, uint64_t* __restrict__ cnt, int loss_kind,
    const float* __restrict__ target, float* __restrict__ dl, float* __restrict__ loss,
    const uint32_t* __restrict__ order) {
  __shared__ SplatLds s_sp[256];
  // rows padded to 260 bytes: the four rows a wave reads at once sit in
  // different LDS banks
  __shared__ uint8_t s_list[16][260];
  __shared__ uint32_t s_cnt[16];
  __shared__ uint32_t s_wc[16][4];
  int tx, ty;
  const int gy = grid_dim(H);
  if (!schedule_tile(order, gx, gy, tx, ty)) return;
  // camera blockIdx.y of a batch: its tiles follow the earlier cameras'
  // (gx * gy each) and its pixels their images
  const int tile = (int)blockIdx.y * gx * gy + ty * gx + tx;
  const int tid = threadIdx.x;
  const int sb = tid >> 4;  // this lane's 4x4 block: each row of the wave walks its own list
  const int px = tx * kTile + sub_px(tid), py = ty * kTile + sub_py(tid);
  const bool inside = px < W && py < H;
  const float fpx = (float)px + 0.5f, fpy = (float)py + 0.5f;
  const uint32_t start = ranges[2 * tile], end = ranges[2 * tile + 1];
  const float amin = st.alpha_min, amax = st.alpha_max, Tmin = st.T_min;

  float T = 1.0f, C0 = 0.0f, C1 = 0.0f, C2 = 0.0f, D = 0.0f;
  uint32_t last = 0;
  bool done = !inside;
  uint32_t n_eval = 0, n_blend = 0, stop_at = 0;  // counters (kStats only)
  // Each lane's record for the next batch is fetched from global memory
  // while the current batch is composited (its index before the batch's
  // compaction, the record itself after it), so a long list does not wait
  // for two dependent global loads per batch.
  RecordRegs rec;
  if (start + (uint32_t)tid < end) rec.load(splats, depths, ids[start + tid], kDepth);
  for (uint32_t b = start; b < end; b += 256) {
    if (__syncthreads_count(done) == 256) break;
    const uint32_t j = b + (uint32_t)tid;
    uint32_t mask = 0u;
    if (j < end) {
      float ex, ey;
      int32_t rad;
      rec.stage(s_sp[tid], rad, ex, ey);
      mask = sub_mask(s_sp[tid], ex, ey, tx * kTile, ty * kTile);
    }
    const uint32_t jn = j + 256u;
    uint32_t next_id = jn < end ? ids[jn] : 0u;
    // zero lists: past the end of its block's list a row reads slot 0
    for (int q = tid; q < 16 * 260 / 4; q += 256) reinterpret_cast<uint32_t*>(&s_list[0][0])[q] = 0u;
    compact_bands<16, 260>(mask, s_list, s_cnt, s_wc);
    // (an empty asm that takes the index: its first use stays here, after
    // the compaction, so the wait for the index load is not hoisted above it)
    asm volatile("" : "+v"(next_id));
    if (jn < end) rec.load(splats, depths, next_id, kDepth);
    // each row walks its block's list; the wave runs for the longest of its
    // four (wave-uniform trip count, on scalar registers)
    const int my_cnt = (int)s_cnt[sb];
    const int c01 = max(__builtin_amdgcn_readlane(my_cnt, 0), __builtin_amdgcn_readlane(my_cnt, 16));
    const int c23 = max(__builtin_amdgcn_readlane(my_cnt, 32), __builtin_amdgcn_readlane(my_cnt, 48));
    const int cnt = max(c01, c23);
    const uint32_t base = b - start + 1u;
    if (__ballot(!done) == 0ull) continue;
    for (int i = 0; i < cnt; ++i) {
      // past the end of this row's list the lane reads slot 0 (the lists'
      // zeroed tail), a record of this batch, and ignores it (a stale slot
      // could hold a non-finite record, and 0 * NaN would reach the sums)
      const bool act = i < my_cnt;
      const int k = (int)s_list[sb][i];
      const SplatLds& s = s_sp[k];
      const float dx = fpx - s.u, dy = fpy - s.v;
      const float p2 = splat_power2(s, dx, dy);
      const float oG = s.o * __builtin_amdgcn_exp2f(p2);
      // the backward's choice (oG > amax ? amax : oG) for every finite oG; a
      // non-finite oG belongs to a lane that ignores it
      const float alpha = fminf(oG, amax);
      const bool ok = act & !done & !(alpha < amin);
      const float Tn = T * (1.0f - alpha);
      // stop (ok and T would fall below T_min) or blend (ok otherwise): one
      // compare, the other mask by exclusive or
      const bool stop = ok & (Tn < Tmin);
      const bool blend = ok ^ stop;
      if (kStats) {
        n_eval += act ? 1u : 0u;
        n_blend += blend ? 1u : 0u;
        stop_at = stop ? base + (uint32_t)k : stop_at;
      }
      done = done | stop;
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
    __shared__ uint32_t s_tmax;
    if (threadIdx.x == 0) s_tmax = 0u;
    __syncthreads();
    if (plain) atomicMax(&s_tmax, plain);
    __syncthreads();
    const uint64_t tile_plain = threadIdx.x == 0 ? 256ull * s_tmax : 0ull;
    add_counters(cnt, inside ? n_eval : 0u, n_blend, plain, tile_plain);
  }
  const int64_t p = ((int64_t)blockIdx.y * H + py) * W + px;
  const float c0 = fmaf(T, bg0, C0), c1 = fmaf(T, bg1, C1), c2 = fmaf(T, bg2, C2);
  float lacc = 0.0f;
  if (inside) {
    image[3 * p + 0] = c0;
    image[3 * p + 1] = c1;
    image[3 * p + 2] = c2;
    final_T[p] = T;
    last_idx[p] = last;
    if (kDepth) out_depth[p] = D;
    if (out_alpha) out_alpha[p] = 1.0f - T;
    // the image loss gradient while the colour is in registers
    if (loss_kind >= 0) {
      dl[3 * p + 0] = loss_term(loss_kind, c0 - target[3 * p + 0], lacc);
      dl[3 * p + 1] = loss_term(loss_kind, c1 - target[3 * p + 1], lacc);
      dl[3 * p + 2] = loss_term(loss_kind, c2 - target[3 * p + 2], lacc);
    }
  }
  if (loss_kind >= 0 && loss) {  // uniform: every lane of the workgroup arrives
    __shared__ float s_l[16];
    lacc = row_total_lane15(lacc);
    if ((tid & 15) == 15) s_l[tid >> 4] = lacc;
    __syncthreads();
    if (tid == 0) {
      float t = 0.0f;
      for (int k = 0; k < 16; ++k) t += s_l[k];
      atomicAdd(loss, t);
    }
  }
}

// ---------------------------------------------------------------------------
// Wavefront reduction of nine fields: two transpose steps with the gfx950
// lane swaps (v_permlane32_swap exchanges the upper half of one register
// with the lower half of another, v_permlane16_swap the odd 16-lane rows of
// one with the even rows of another), so that after them every 16-lane row
// of a register carries one field; a third step at 8-lane granularity (two
// selects and an add from the lanes 8 apart in the row) puts fields 0-3 and
// 4-7 in the two halves of each row of one register; then three DPP adds
// (half-row mirror, two quad permutations) leave each 8-lane half's total in
// all of its lanes.  About 27 instructions instead of six DPP steps per
// field.
// ---------------------------------------------------------------------------
// DPP lane permutations within 16-lane rows (no lane reads outside its row).
constexpr int kRowRor8 = 0x128;       // row_ror:8: lane i reads lane (i + 8) mod 16
constexpr int kRowHalfMirror = 0x141;  // row_half_mirror: lane i reads 7 - i in its half
constexpr int kQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]
template <int kCtrl>
__device__ inline float dpp_f32(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, true));
}
// The total of each 8-lane half-row, in all eight of its lanes: lane i plus
// lane 7 - i, then the pairs and the halves of each quad.
__device__ inline float half_row_total(float v) {
  v += dpp_f32<kRowHalfMirror>(v);
  v += dpp_f32<kQuadSwap2>(v);
  v += dpp_f32<kQuadSwap1>(v);
  return v;
}

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

// Sums f[0..8] (and f[9], f[10] when kAbs) over the wavefront and adds field
// q to dst[q * stride] (LDS, atomically).  Callers give each pair of
// wavefronts its own slots: from a zero start, two float additions give the
// same bits in either order, so the result does not depend on which
// wavefront of the pair came first.
template <bool kAbs>
__device__ inline void reduce_add(const float* f, float* dst, int stride) {
  const float s01 = swap_add32(f[0], f[1]);
  const float s23 = swap_add32(f[2], f[3]);
  const float s45 = swap_add32(f[4], f[5]);
  const float s67 = swap_add32(f[6], f[7]);
  // without absgrad field 8 is paired with itself (its sums then fill both
  // halves and every row; only row 0's total is used)
  const float s89 = swap_add32(f[8], kAbs ? f[9] : f[8]);
  const float sA = kAbs ? swap_add32(f[10], f[10]) : s89;
  // rows of t0: fields 0, 2, 1, 3; of t1: 4, 6, 5, 7; of t2: 8, 10, 9, -
  const float t0 = swap_add16(s01, s23);
  const float t1 = swap_add16(s45, s67);
  float t2 = swap_add16(s89, sA);
  // the low half of each row keeps t0's partial sums (lane i plus lane i + 8),
  // the high half t1's (lane i plus lane i - 8)
  const bool hi = (threadIdx.x & 8) != 0;
  float m = (hi ? t1 : t0) + dpp_f32<kRowRor8>(hi ? t0 : t1);
  m = half_row_total(m);
  t2 += dpp_f32<kRowRor8>(t2);
  t2 = half_row_total(t2);  // the row's total, in every lane of the row
  const int lane = threadIdx.x & 63;
  if ((lane & 7) == 7) {
    const int row = lane >> 4;
    const int q = ((row == 1) ? 2 : (row == 2 ? 1 : row)) + (hi ? 4 : 0);
    atomicAdd(&dst[q * stride], m);
    if (hi) {
      if (row == 0) atomicAdd(&dst[8 * stride], t2);
      if (kAbs && row == 1) atomicAdd(&dst[10 * stride], t2);
      if (kAbs && row == 2) atomicAdd(&dst[9 * stride], t2);
    }
  }
}

// Gradient slots of one splat, in moment form: w dx, w dy, w dx^2, w dx dy,
// w dy^2 with w = -2 dL/dq = alpha dL/dalpha, then w itself and the three
// colour gradients.  The mean, conic and opacity gradients follow after the
// reduction (S the sums of the w moments, Sw the sum of w):
//   dL/du = A Sx + B Sy, dL/dv = B Sx + C Sy,
//   dL/dA = -Sxx / 2, dL/dB = -Sxy, dL/dC = -Syy / 2, dL/do = Sw / o.
// With absgrad, two more: the per-pixel |dL/du| and |dL/dv| summed over the
// pixels (the absolute-gradient statistic of densification).
constexpr int kFields = 9;
constexpr int kFieldsAbs = 11;
// |dL/du| = |w (A dx + B dy)| and A dx + B dy = l11 e1 / k^2 with the
// record's factors scaled by k = sqrt(log2(e) / 2): 1 / k^2 = 2 ln 2
constexpr float kAbsScale = 1.3862943611198906f;

// Slot of Gaussian `id`'s instance for tile (tx, ty): its offset plus the
// tile's row-major index inside the Gaussian's rect.
__device__ inline uint64_t instance_slot(float u, float v, int32_t radius, uint32_t offset, int tx,
                                         int ty, int gx, int gy) {
  int x0, x1, y0, y1;
  tile_rect(u, v, radius, gx, gy, x0, x1, y0, y1);
  const int w = (x1 > x0) ? x1 - x0 : 1;
  return (uint64_t)offset + (uint64_t)((ty - y0) * w + (tx - x0));
}

template <bool kStats, bool kAbs>
__global__ __launch_bounds__(256) void raster_bwd_kernel(
    int W, int H, int gx, const uint32_t* __restrict__ ranges, const uint32_t* __restrict__ ids,
    const float4* __restrict__ splats, const uint32_t* __restrict__ offsets, float bg0,
    float bg1, float bg2, Settings st, const float* __restrict__ final_T,
    const uint32_t* __restrict__ last_idx, const float* __restrict__ dL_dimage,
    float4* __restrict__ partials, uint64_t capacity, uint64_t* __restrict__ cnt,
    const uint32_t* __restrict__ order) {
  // one LDS block with the staged splats at offset 0, so that the inner
  // loop's three reads of a splat share one address (read2 immediates reach
  // only 2 KB past it)
  struct Lds {
    SplatLds sp[256];
    float acc[2][kAbs ? kFieldsAbs : kFields][256];  // one set per pair of wavefronts
    uint8_t list[4][256];
    uint32_t cnt[4];
    uint32_t wc[4][4];
    uint32_t wlast[4];  // per wavefront: the largest last index of its pixels
  };
  __shared__ Lds lds;
  SplatLds* s_sp = lds.sp;
  auto& s_acc = lds.acc;
  auto& s_list = lds.list;
  uint32_t* s_cnt = lds.cnt;
  auto& s_wc = lds.wc;
  uint32_t* s_wlast = lds.wlast;
  int tx, ty;
  const int gy = grid_dim(H);
  if (!schedule_tile(order, gx, gy, tx, ty)) return;
  // camera blockIdx.y of a batch (tiles and images after the earlier ones')
  const int tile = (int)blockIdx.y * gx * gy + ty * gx + tx;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int px = tx * kTile + quad_px(tid), py = ty * kTile + quad_py(tid);
  const bool inside = px < W && py < H;
  const float fpx = (float)px + 0.5f, fpy = (float)py + 0.5f;
  const uint32_t start = ranges[2 * tile], end = ranges[2 * tile + 1];
  const float amin = st.alpha_min, amax = st.alpha_max;

  float T = 1.0f, g0 = 0.0f, g1 = 0.0f, g2 = 0.0f;
  uint32_t last = 0;
  if (inside) {
    const int64_t p = ((int64_t)blockIdx.y * H + py) * W + px;
    T = final_T[p];
    last = last_idx[p];
    g0 = dL_dimage[3 * p + 0];
    g1 = dL_dimage[3 * p + 1];
    g2 = dL_dimage[3 * p + 2];
  }
  // S = sum_c dL/dC_c R_c, with R the colour accumulated behind the current
  // splat, background included
  float S = T * fmaf(g0, bg0, fmaf(g1, bg1, g2 * bg2));
  if (tid < 4) s_wlast[tid] = 0;
  __syncthreads();
  if (last) atomicMax(&s_wlast[wave], last);
  __syncthreads();
  const uint32_t maxlast = max(max(s_wlast[0], s_wlast[1]), max(s_wlast[2], s_wlast[3]));
  // nothing at or after `stop` is blended; last indices beyond the tile's
  // list (inputs that do not belong together) give the tile zero gradients
  const uint32_t stop = (maxlast > end - start) ? start : start + maxlast;
  uint32_t n_eval = 0, n_hit = 0, n_red = 0;  // counters (kStats only)

  // entries no pixel of the tile blends: their instance slots get zeros
  for (uint32_t j = stop + (uint32_t)tid; j < end; j += 256u) {
    const uint32_t id = ids[j];
    const float4 a = splats[4 * (size_t)id], c = splats[4 * (size_t)id + 2];
    const uint64_t slot =
        instance_slot(a.x, a.y, __float_as_int(c.y), offsets[id], tx, ty, gx, gy);
    if (slot < capacity) {
      const float4 z = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      partials[3 * slot + 0] = z;
      partials[3 * slot + 1] = z;
      partials[3 * slot + 2] = z;
    }
  }

  for (uint32_t b_end = stop; b_end > start;) {
    const uint32_t b_begin = (b_end - start) > 256u ? b_end - 256u : start;
    const int n = (int)(b_end - b_begin);
    __syncthreads();
    uint32_t mask = 0u, my_off = 0u;
    int32_t my_rad = 0;
    float cA = 0.0f, cB = 0.0f, cC = 0.0f;  // raw conic of the splat this thread stages
    if (tid < n) {
      const uint32_t my_id = ids[b_end - 1u - (uint32_t)tid];  // slot k = tid: back to front
      my_off = offsets[my_id];
      RecordRegs rec;
      rec.load(splats, nullptr, my_id, false);
      float ex, ey;
      rec.stage(s_sp[tid], my_rad, ex, ey);
      // the backward keeps 1/o in the depth slot (o >= alpha_min > 0 for
      // any splat that blends)
      const float o = rec.b.y;
      s_sp[tid].z = o > 0.0f ? 1.0f / o : 0.0f;
      const float4 d = splats[4 * (size_t)my_id + 3];
      cA = d.x; cB = d.y; cC = d.z;
      mask = quad_mask(s_sp[tid], ex, ey, tx * kTile, ty * kTile);
      // a wavefront whose pixels all stopped in front of this entry (list
      // position rel) skips it
      const uint32_t rel = b_end - 1u - start - (uint32_t)tid;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (rel >= s_wlast[q]) mask &= ~(1u << q);
    }
    constexpr int kF = kAbs ? kFieldsAbs : kFields;
#pragma unroll
    for (int q = 0; q < kF; ++q) {
      s_acc[0][q][tid] = 0.0f;
      s_acc[1][q][tid] = 0.0f;
    }
    compact_bands<4, 256>(mask, s_list, s_cnt, s_wc);
    const int cnt_w = __builtin_amdgcn_readfirstlane((int)s_cnt[wave]);
    // batch slot k holds list position rel = b_end - 1 - start - k; the pixel
    // blended it only if rel < last, i.e. k > kthr
    const int kthr = (int)(b_end - 1u - start) - (int)last;
    // one list entry: slot k's splat s, evaluated for this lane's pixel
    auto eval = [&](const SplatLds& s, int k) {
      const float dx = fpx - s.u, dy = fpy - s.v;
      float e1, e2;
      const float p2 = splat_power2(s, dx, dy, e1, e2);
      const float G = __builtin_amdgcn_exp2f(p2);
      const float oG = s.o * G;
      const bool clamped = oG > amax;
      // the forward's alpha for every finite oG (a non-finite one belongs to
      // no evaluated list entry: its footprint mask is empty)
      const float alpha = fminf(oG, amax);
      const bool hit = (k > kthr) & !(alpha < amin);
      // a lane that does not blend this splat takes alpha 0: its T is
      // multiplied by 1/(1 - 0) = 1 exactly and its weight is 0
      const float ah = hit ? alpha : 0.0f;
      const float rom = __builtin_amdgcn_rcpf(1.0f - ah);
      T = T * rom;  // transmittance in front of this splat
      const float wgt = ah * T;
      float f[kF];
      f[6] = g0 * wgt;
      f[7] = g1 * wgt;
      f[8] = g2 * wgt;
      // dC_c/dalpha = c_c T - R_c / (1 - alpha), so with gc = sum_c dL/dC_c c_c:
      // dL/dalpha = gc T - S / (1 - alpha), and S grows by gc wgt
      const float gc = fmaf(g0, s.r, fmaf(g1, s.g, g2 * s.b));
      const float dLda = fmaf(gc, T, -S * rom);
      S = fmaf(gc, wgt, S);
      const bool geo = hit & !clamped;
      // q = A dx^2 + 2B dx dy + C dy^2, alpha = o exp(-q/2): dL/dq = -alpha/2
      // dL/dalpha = -w/2; dL/do = G dL/dalpha = w / o, summed as w and
      // divided by o once per splat
      const float m = geo ? alpha * dLda : 0.0f;
      f[5] = m;
      const float mx = m * dx, my = m * dy;
      f[0] = mx;
      f[1] = my;
      f[2] = mx * dx;
      f[3] = mx * dy;
      f[4] = my * dy;
      if (kAbs) {
        f[9] = fabsf(m * s.l11 * e1) * kAbsScale;
        f[10] = fabsf(m * fmaf(s.l21, e1, s.l22 * e2)) * kAbsScale;
      }
      if (kStats) {
        n_eval += inside ? 1u : 0u;
        n_hit += hit ? 1u : 0u;
      }
      if (__ballot(hit) != 0ull) {
        if (kStats) n_red += (lane == 0) ? 1u : 0u;
        reduce_add<kAbs>(f, &s_acc[wave >> 1][0][k], 256);
      }
    };
    // Software pipeline over the wave's list: each splat record is read
    // from LDS two entries ahead of its use, into three rotating register
    // sets, so that a use never waits on the LDS additions of the entry just
    // before it; the list (at most 256 one-byte slots) is held in one
    // register, four slots per lane, and read with lane reads.  Reads past
    // the end repeat the last entry.
    if (cnt_w > 0) {
      const uint32_t lw = reinterpret_cast<const uint32_t*>(s_list[wave])[lane];
      const int lastp = cnt_w - 1;
      auto slot_at = [&](int i) {
        i = min(i, lastp);
        const uint32_t w = (uint32_t)__builtin_amdgcn_readlane((int)lw, i >> 2);
        return (int)((w >> (8 * (i & 3))) & 0xffu);
      };
      int k0 = slot_at(0), k1 = slot_at(1), k2;
      SplatLds s0 = s_sp[k0], s1 = s_sp[k1], s2;
      int i = 0;
      // whole trips of three entries ...
      for (; i + 2 <= lastp; i += 3) {
        k2 = slot_at(i + 2);
        s2 = s_sp[k2];
        eval(s0, k0);
        k0 = slot_at(i + 3);
        s0 = s_sp[k0];
        eval(s1, k1);
        k1 = slot_at(i + 4);
        s1 = s_sp[k1];
        eval(s2, k2);
      }
      // ... then the one or two entries left, if any
      if (i <= lastp) eval(s0, k0);
      if (i + 1 <= lastp) eval(s1, k1);
    }
    __syncthreads();
    if (tid < n) {
      float acc[kF];
#pragma unroll
      for (int q = 0; q < kF; ++q) acc[q] = s_acc[0][q][tid] + s_acc[1][q][tid];
      // moments -> gradients of u, v and the conic
      const float gu = fmaf(cA, acc[0], cB * acc[1]);
      const float gv = fmaf(cB, acc[0], cC * acc[1]);
      const uint64_t slot =
          instance_slot(s_sp[tid].u, s_sp[tid].v, my_rad, my_off, tx, ty, gx, gy);
      if (slot < capacity) {
        partials[3 * slot + 0] = make_float4(gu, gv, -0.5f * acc[2], -acc[3]);
        partials[3 * slot + 1] =
            make_float4(-0.5f * acc[4], acc[5] * s_sp[tid].z, acc[6], acc[7]);
        partials[3 * slot + 2] =
            make_float4(acc[8], kAbs ? acc[kF - 2] : 0.0f, kAbs ? acc[kF - 1] : 0.0f, 0.0f);
      }
    }
    b_end = b_begin;
  }
  if (kStats)
    add_counters(cnt, n_eval, n_hit, threadIdx.x == 0 ? 256ull * (stop - start) : 0ull, n_red);
}

// Sum each visible Gaussian's instance slots [offsets[i], offsets[i] +
// tiles[i]) of partials into its 2D gradient record, in slot order, so the
// result does not depend on scheduling.  A lane sums a Gaussian touching at
// most kSmallSeg tiles on its own; larger ones are summed by the whole
// workgroup with a fixed-shape tree.
constexpr uint32_t kSmallSeg = 32;

__device__ inline void add_rec(float a[kFieldsAbs], const float4* __restrict__ p) {
  const float4 x = p[0], y = p[1], z = p[2];
  a[0] += x.x; a[1] += x.y; a[2] += x.z; a[3] += x.w;
  a[4] += y.x; a[5] += y.y; a[6] += y.z; a[7] += y.w;
  a[8] += z.x; a[9] += z.y; a[10] += z.z;
}

// Writes row r's eleven sums to the 2D gradient planes.  mode 0 overwrites
// every plane, 1 adds to every plane, 2 adds to the per-Gaussian results
// that are final after this stage (opacity, absolute sums) and overwrites
// the per-camera ones the projection backward reads (mean, conic, colour).
// has: the row has tiles; without, the added planes are left alone.
__device__ inline void store_grads(const Grad2D& g, int64_t r, const float a[kFieldsAbs],
                                   int mode, bool has) {
  const int64_t c = r / g.ld, i = r - c * g.ld;
  auto put = [&](float* base, int P, int q, float v, bool add) {
    float* p = base + c * P * g.ld + q * g.ld + i;
    if (add) {
      if (has) *p = *p + v;
    } else {
      *p = v;
    }
  };
  const bool add_cam = mode == 1, add_fin = mode != 0;
  put(g.m2, 2, 0, a[0], add_cam);
  put(g.m2, 2, 1, a[1], add_cam);
  put(g.con, 3, 0, a[2], add_cam);
  put(g.con, 3, 1, a[3], add_cam);
  put(g.con, 3, 2, a[4], add_cam);
  put(g.op, 1, 0, a[5], add_fin);
  put(g.col, 3, 0, a[6], add_cam);
  put(g.col, 3, 1, a[7], add_cam);
  put(g.col, 3, 2, a[8], add_cam);
  if (g.abs) {
    put(g.abs, 2, 0, a[9], add_fin);
    put(g.abs, 2, 1, a[10], add_fin);
  }
}

// Row r of the 2D gradient planes sums the slots of Gaussian row r, or of
// Gaussian vis_ids[r] in the packed form (kPacked), where the rows follow
// that list.  Rows without tiles get zeros in the overwritten planes (mode,
// see store_grads).
// Slots past `capacity` (a binning that overflowed its buffers and left an
// empty list) are never read: such a Gaussian gets zeros.
template <bool kPacked>
__global__ __launch_bounds__(256) void reduce_partials_kernel(
    int64_t N, const uint32_t* __restrict__ vis_ids, const uint32_t* __restrict__ offsets,
    const uint32_t* __restrict__ tiles, const float4* __restrict__ partials, uint64_t capacity,
    Grad2D g, int mode) {
  __shared__ uint32_t s_big[256];
  __shared__ uint32_t s_nbig;
  __shared__ float s_red[kFieldsAbs][256];
  const int t = threadIdx.x;
  const int64_t r = (int64_t)blockIdx.x * 256 + t;
  if (t == 0) s_nbig = 0;
  __syncthreads();
  if (r < N) {
    const int64_t i = kPacked ? (int64_t)vis_ids[r] : r;
    const uint32_t cnt = tiles[i];
    const bool fits = cnt == 0 || (uint64_t)offsets[i] + cnt <= capacity;
    if (cnt > kSmallSeg && fits) {
      s_big[atomicAdd(&s_nbig, 1u)] = (uint32_t)t;
    } else if (cnt > 0 || mode != 1) {
      float a[kFieldsAbs] = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
      const uint64_t base = offsets[i];
      if (fits) {
        // four slots' loads in flight before their (in-order) additions
        uint32_t k = 0;
        for (; k + 4 <= cnt; k += 4) {
          const float4* p = partials + 3 * (base + k);
          float4 x[4][3];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            x[j][0] = p[3 * j];
            x[j][1] = p[3 * j + 1];
            x[j][2] = p[3 * j + 2];
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            a[0] += x[j][0].x; a[1] += x[j][0].y; a[2] += x[j][0].z; a[3] += x[j][0].w;
            a[4] += x[j][1].x; a[5] += x[j][1].y; a[6] += x[j][1].z; a[7] += x[j][1].w;
            a[8] += x[j][2].x; a[9] += x[j][2].y; a[10] += x[j][2].z;
          }
        }
        for (; k < cnt; ++k) add_rec(a, partials + 3 * (base + k));
      }
      store_grads(g, r, a, mode, cnt > 0);
    }
  }
  __syncthreads();
  const uint32_t nbig = s_nbig;
  for (uint32_t b = 0; b < nbig; ++b) {
    const int64_t gr = (int64_t)blockIdx.x * 256 + s_big[b];
    const int64_t gi = kPacked ? (int64_t)vis_ids[gr] : gr;
    const uint32_t cnt = tiles[gi];
    const uint64_t base = offsets[gi];
    float a[kFieldsAbs] = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    for (uint32_t k = (uint32_t)t; k < cnt; k += 256u) add_rec(a, partials + 3 * (base + k));
#pragma unroll
    for (int q = 0; q < kFieldsAbs; ++q) s_red[q][t] = a[q];
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
      if (t < h)
#pragma unroll
        for (int q = 0; q < kFieldsAbs; ++q) s_red[q][t] += s_red[q][t + h];
      __syncthreads();
    }
    if (t == 0) {
      float sum[kFieldsAbs];
#pragma unroll
      for (int q = 0; q < kFieldsAbs; ++q) sum[q] = s_red[q][0];
      store_grads(g, gr, sum, mode, true);
    }
    __syncthreads();
  }
}


// dL/dimage and (optionally) the summed loss: per-lane partial sums, a DPP
// row reduction, a cross-wave sum in LDS, then one atomic per workgroup.
// float4 accesses when the three arrays are 16-byte aligned; the tail (and
// unaligned arrays) go element by element.

__global__ __launch_bounds__(256) void loss_grad_kernel(int kind, int64_t n, int64_t n4,
                                                        const float* __restrict__ img,
                                                        const float* __restrict__ tgt,
                                                        float* __restrict__ g,
                                                        float* __restrict__ loss) {
  __shared__ float s_w[16];
  float acc = 0.0f;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const float4* img4 = (const float4*)img;
  const float4* tgt4 = (const float4*)tgt;
  float4* g4 = (float4*)g;
  for (int64_t i = t0; i < n4; i += stride) {
    const float4 x = img4[i], y = tgt4[i];
    float4 o;
    o.x = loss_term(kind, x.x - y.x, acc);
    o.y = loss_term(kind, x.y - y.y, acc);
    o.z = loss_term(kind, x.z - y.z, acc);
    o.w = loss_term(kind, x.w - y.w, acc);
    g4[i] = o;
  }
  for (int64_t i = 4 * n4 + t0; i < n; i += stride) g[i] = loss_term(kind, img[i] - tgt[i], acc);
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

// Workgroup c orders camera c's T tiles by decreasing list length (bucketed
// by length_bucket; within a bucket the order is whatever the LDS counters
// give).  The compositing kernels' results do not depend on it: it only
// decides which tiles start first, so that the longest lists do not start
// last and leave the GPU to a few workgroups at the end.  Each lane takes
// kOrderItems tiles per round with all their range loads in flight; the
// buckets of up to kOrderKeep tiles stay in LDS for the second pass.
constexpr int kOrderThreads = 1024, kOrderItems = 8, kOrderKeep = 32768;

__global__ __launch_bounds__(kOrderThreads) void tile_order_kernel(
    const uint32_t* __restrict__ ranges, int T, uint32_t* __restrict__ order) {
  __shared__ uint32_t h[256];
  __shared__ uint8_t kept[kOrderKeep];
  const int tid = threadIdx.x;
  const uint32_t* rr = ranges + 2 * (int64_t)blockIdx.y * T;
  uint32_t* out = order + (int64_t)blockIdx.y * T;
  const bool keep = T <= kOrderKeep;
  if (tid < 256) h[tid] = 0u;
  __syncthreads();
  for (int t0 = 0; t0 < T; t0 += kOrderThreads * kOrderItems) {
    uint32_t r0[kOrderItems], r1[kOrderItems];
#pragma unroll
    for (int j = 0; j < kOrderItems; ++j) {
      const int t = t0 + j * kOrderThreads + tid;
      r0[j] = t < T ? rr[2 * t] : 0u;
      r1[j] = t < T ? rr[2 * t + 1] : 0u;
    }
#pragma unroll
    for (int j = 0; j < kOrderItems; ++j) {
      const int t = t0 + j * kOrderThreads + tid;
      const uint32_t b = 255u - length_bucket(r1[j] - r0[j]);
      if (t < T) {
        if (keep) kept[t] = (uint8_t)b;
        atomicAdd(&h[b], 1u);
      }
    }
  }
  __syncthreads();
  if (tid < 64) {  // exclusive scan of the 256 counts, four per lane
    uint32_t c[4], run = 0;
    for (int j = 0; j < 4; ++j) { c[j] = h[4 * tid + j]; run += c[j]; }
    uint32_t incl = run;
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t o = __shfl_up(incl, d);
      if (tid >= d) incl += o;
    }
    uint32_t base = incl - run;
    for (int j = 0; j < 4; ++j) { h[4 * tid + j] = base; base += c[j]; }
  }
  __syncthreads();
  for (int t0 = 0; t0 < T; t0 += kOrderThreads) {
    const int t = t0 + tid;
    if (t < T) {
      const uint32_t b =
          keep ? (uint32_t)kept[t] : 255u - length_bucket(rr[2 * t + 1] - rr[2 * t]);
      out[atomicAdd(&h[b], 1u)] = (uint32_t)t;
    }
  }
}

}  // namespace gs

extern "C" hipError_t gs_launch_tile_order(int32_t W, int32_t H, int ncams,
                                           const uint32_t* ranges, uint32_t* order,
                                           hipStream_t s) {
  const int T = gs::grid_dim(W) * gs::grid_dim(H);
  if (T == 0 || ncams == 0) return hipSuccess;
  hipLaunchKernelGGL(gs::tile_order_kernel, dim3(1, (unsigned)ncams), dim3(1024), 0, s, ranges,
                     T, order);
  return hipGetLastError();
}

// Stages the records of rows [0, rows) (a batch: rows = ncams * ld) into rec.
extern "C" hipError_t gs_launch_pack_splats(int64_t rows, int64_t ld, const float* means2d,
                                            const float* conics, const float* chol,
                                            const float* opac, const float* colors,
                                            const int32_t* radii, float alpha_min, float* rec,
                                            hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(gs::pack_splats_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0,
                     s, rows, ld, means2d, conics, chol, opac, colors, radii, alpha_min,
                     (float4*)rec);
  return hipGetLastError();
}

// ncams images of W x H (a batch: ranges over ncams * T tiles, outputs
// [c][H][W]), from the staged records.  loss_kind >= 0: also dL/dimage
// against target (and the loss value into *loss when non-NULL).
extern "C" hipError_t gs_launch_raster_fwd(int32_t W, int32_t H, int ncams,
                                           const uint32_t* ranges, const uint32_t* order,
                                           const uint32_t* ids,
                                           const float* splats, const float* depths,
                                           const float* bg, const gs::Settings& st, float* image,
                                           float* final_T, uint32_t* last_idx, float* out_depth,
                                           float* out_alpha, uint64_t* counters, int loss_kind,
                                           const float* target, float* dl, float* loss,
                                           hipStream_t s) {
  const int gx = gs::grid_dim(W), gy = gs::grid_dim(H);
  const dim3 grid(gs::tile_grid_blocks(gx, gy), (unsigned)ncams), block(256);
  const float4* sp = (const float4*)splats;
  if (loss_kind >= 0 && loss) {
    hipLaunchKernelGGL(gs::zero_f32_kernel, dim3(1), dim3(1), 0, s, loss);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
#define GS_RFWD(DEPTH, STATS)                                                                  \
  hipLaunchKernelGGL((gs::raster_fwd_kernel<DEPTH, STATS>), grid, block, 0, s, W, H, gx, ranges, \
                     ids, sp, DEPTH ? depths : nullptr, bg[0], bg[1], bg[2], st, image,        \
                     final_T, last_idx, DEPTH ? out_depth : nullptr, out_alpha,               \
                     STATS ? counters : nullptr, loss_kind, target, dl, loss, order)
  if (counters) {
    if (out_depth) GS_RFWD(true, true); else GS_RFWD(false, true);
  } else {
    if (out_depth) GS_RFWD(true, false); else GS_RFWD(false, false);
  }
#undef GS_RFWD
  return hipGetLastError();
}

// ncams > 1: a batch (N = ncams * ld rows, ranges over ncams * T tiles,
// images [c][H][W]).  The 2D gradients go to the planes of g (rows as
// Grad2D describes; packed rows follow vis_ids).
extern "C" hipError_t gs_launch_raster_bwd(int64_t N, int32_t W, int32_t H, int ncams,
                                           const uint32_t* ranges, const uint32_t* order,
                                           const uint32_t* ids, const float* splats,
                                           const uint32_t* offsets, const uint32_t* tiles,
                                           const float* bg, const gs::Settings& st,
                                           const float* final_T, const uint32_t* last_idx,
                                           const float* dL_dimage, float* partials,
                                           uint64_t capacity, const gs::Grad2D& g,
                                           int accumulate, const uint32_t* vis_ids,
                                           int64_t num_visible, uint64_t* counters,
                                           hipStream_t s) {
  const int gx = gs::grid_dim(W), gy = gs::grid_dim(H);
  const dim3 grid(gs::tile_grid_blocks(gx, gy), (unsigned)ncams), block(256);
  const float4* sp = (const float4*)splats;
  float4* part = (float4*)partials;
  const bool absgrad = g.abs != nullptr;
#define GS_RBWD(STATS, ABS)                                                                 \
  hipLaunchKernelGGL((gs::raster_bwd_kernel<STATS, ABS>), grid, block, 0, s, W, H, gx, ranges, \
                     ids, sp, offsets, bg[0], bg[1], bg[2], st, final_T, last_idx,          \
                     dL_dimage, part, capacity, counters, order)
  if (counters) {
    if (absgrad) GS_RBWD(true, true); else GS_RBWD(true, false);
  } else {
    if (absgrad) GS_RBWD(false, true); else GS_RBWD(false, false);
  }
#undef GS_RBWD
  hipError_t e = hipGetLastError();
  // dense rows: one per Gaussian; packed rows: one per entry of vis_ids
  const int64_t rows = vis_ids ? num_visible : N;
  if (e != hipSuccess || rows == 0) return e;
  const dim3 rgrid((unsigned)((rows + 255) / 256));
  if (vis_ids)
    hipLaunchKernelGGL(gs::reduce_partials_kernel<true>, rgrid, dim3(256), 0, s, rows, vis_ids,
                       offsets, tiles, part, capacity, g, accumulate);
  else
    hipLaunchKernelGGL(gs::reduce_partials_kernel<false>, rgrid, dim3(256), 0, s, rows, nullptr,
                       offsets, tiles, part, capacity, g, accumulate);
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
  const bool al = (((uintptr_t)img | (uintptr_t)tgt | (uintptr_t)g) & 15u) == 0;
  const int64_t n4 = al ? n / 4 : 0;
  int64_t blocks = ((al ? n4 : n) + 255) / 256;
  if (blocks < 1) blocks = 1;  // fewer than four elements: the tail loop alone
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(gs::loss_grad_kernel, dim3((unsigned)blocks), dim3(256), 0, s, kind, n, n4,
                     img, tgt, g, loss);
  return hipGetLastError();
}
