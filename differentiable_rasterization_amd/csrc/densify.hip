// densify.hip — the count-changing step between training iterations, on the
// device: clone the Gaussians whose mean gradient is largest and drop the
// faint ones (the densify / prune of the gsplat guide (lmnt.cn/news/262699)
// §4.1, which clones by a gradient threshold and prunes below opacity
// 0.005).
//
// Everything here is data movement, bound by HBM: a selection key per
// Gaussian, a stable radix sort of the keys (descending, ties by lower
// index), two scans and one gather of every parameter plane into the output
// planes.  Selection decisions use the key's fp32 bits, computed in one
// fixed order, so that they are reproducible.
#include "gs_common.h"

#include <cmath>

extern "C" size_t gs_pairsort_workspace_bytes(uint64_t n, int bits);
extern "C" hipError_t gs_pairsort(uint64_t* keys, uint32_t* vals, uint64_t n, int bits,
                                  void* workspace, hipStream_t s);
extern "C" size_t gs_scan_workspace_bytes(int64_t n);
extern "C" hipError_t gs_scan_u32(const uint32_t* in, int64_t n, uint32_t* out, uint64_t* total,
                                  void* workspace, hipStream_t s);

namespace gs {

static inline size_t dalign(size_t x) { return (x + 255) & ~(size_t)255; }

// Selection key: the squared fp32 norm of the mean gradient, (gx gx + gy gy)
// + gz gz, with NaN taken as +inf.  Sorting ~bits ascending orders these
// non-negative keys descending; the stable sort keeps ascending index among
// equal keys.  Also clears the selection flags.
__global__ __launch_bounds__(256) void densify_key_kernel(int64_t N, int64_t ld,
                                                          const float* __restrict__ g,
                                                          uint64_t* __restrict__ keys,
                                                          uint32_t* __restrict__ vals,
                                                          uint32_t* __restrict__ sel) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N) return;
  const float gx = g[i], gy = g[ld + i], gz = g[2 * ld + i];
  float k = (gx * gx + gy * gy) + gz * gz;
  if (__builtin_isnan(k)) k = __builtin_inff();
  keys[i] = (uint64_t)(~__float_as_uint(k));
  vals[i] = (uint32_t)i;
  sel[i] = 0u;
}

__global__ __launch_bounds__(256) void densify_mark_kernel(int64_t n_clone,
                                                           const uint32_t* __restrict__ vals,
                                                           uint32_t* __restrict__ sel) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r < n_clone) sel[vals[r]] = 1u;
}

// Source of output candidate j: j itself for the originals, then the
// selected Gaussians in index order.  keep[j] = opacity of the source >=
// min_opacity.
__global__ __launch_bounds__(256) void densify_keep_kernel(
    int64_t N, int64_t n_clone, const uint32_t* __restrict__ sel,
    const uint32_t* __restrict__ crank, const float* __restrict__ opac, float min_opacity,
    uint32_t* __restrict__ clone_src, uint32_t* __restrict__ keep) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j < N) {
    keep[j] = opac[j] >= min_opacity ? 1u : 0u;
    if (sel[j]) {
      const uint32_t r = crank[j];
      clone_src[r] = (uint32_t)j;
      keep[N + r] = keep[j];
    }
  }
  (void)n_clone;
}

// Base pointers of every parameter plane, passed by value.
constexpr int kMaxPlanes = 64;
struct Planes {
  const float* in[kMaxPlanes];
  float* out[kMaxPlanes];
  int n;
};

// Gather every parameter plane: output dest[j] of each kept candidate j.
__global__ __launch_bounds__(256) void densify_copy_kernel(int64_t N, int64_t n_cand,
                                                           const uint32_t* __restrict__ clone_src,
                                                           const uint32_t* __restrict__ keep,
                                                           const uint32_t* __restrict__ dest,
                                                           Planes pl) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n_cand || !keep[j]) return;
  const int64_t src = j < N ? j : (int64_t)clone_src[j - N];
  const int64_t d = dest[j];
  for (int a = 0; a < pl.n; ++a) pl.out[a][d] = pl.in[a][src];
}

struct DensifyWs {
  uint64_t* keys;
  uint32_t* vals;
  uint32_t* sel;
  uint32_t* crank;
  uint32_t* clone_src;
  uint32_t* keep;
  uint32_t* dest;
  uint64_t* totals;  // [2]
  void* sort_ws;
  void* scan_ws;
  size_t bytes;
};

static DensifyWs carve_densify(void* base, int64_t N, int64_t n_clone) {
  DensifyWs w;
  char* p = (char*)base;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* r = p ? p + off : nullptr;
    off += dalign(bytes);
    return r;
  };
  const size_t n = (size_t)(N ? N : 1), nc = (size_t)(N + n_clone ? N + n_clone : 1);
  w.keys = (uint64_t*)take(sizeof(uint64_t) * n);
  w.vals = (uint32_t*)take(sizeof(uint32_t) * n);
  w.sel = (uint32_t*)take(sizeof(uint32_t) * n);
  w.crank = (uint32_t*)take(sizeof(uint32_t) * n);
  w.clone_src = (uint32_t*)take(sizeof(uint32_t) * (size_t)(n_clone ? n_clone : 1));
  w.keep = (uint32_t*)take(sizeof(uint32_t) * nc);
  w.dest = (uint32_t*)take(sizeof(uint32_t) * nc);
  w.totals = (uint64_t*)take(sizeof(uint64_t) * 2);
  w.sort_ws = take(gs_pairsort_workspace_bytes((uint64_t)N, 32));
  w.scan_ws = take(gs_scan_workspace_bytes(N + n_clone));
  w.bytes = off;
  return w;
}

}  // namespace gs

extern "C" int64_t gs_densify_clone_count(int64_t N, float clone_fraction) {
  return (int64_t)std::floor((double)clone_fraction * (double)N + 0.5);
}

extern "C" size_t gs_densify_workspace_bytes(int64_t N, float clone_fraction) {
  return gs::carve_densify(nullptr, N, gs_densify_clone_count(N, clone_fraction)).bytes;
}

// Runs the whole step; *num_out (host) receives the new count (one
// synchronising read).  in_planes / out_planes: nplanes (<= 64) plane base
// pointers, host arrays.
extern "C" hipError_t gs_launch_densify(int64_t N, int nplanes, const float* const* in_planes,
                                        int64_t ld, const float* dL_dmeans,
                                        const float* opacities, float clone_fraction,
                                        float min_opacity, float* const* out_planes,
                                        int64_t* num_out, void* workspace, hipStream_t s) {
  using namespace gs;
  const int64_t n_clone = gs_densify_clone_count(N, clone_fraction);
  DensifyWs w = carve_densify(workspace, N, n_clone);
  hipError_t e;
  if (N == 0) {
    *num_out = 0;
    return hipSuccess;
  }
  Planes pl;
  pl.n = nplanes;
  for (int a = 0; a < kMaxPlanes; ++a) {
    pl.in[a] = a < nplanes ? in_planes[a] : nullptr;
    pl.out[a] = a < nplanes ? out_planes[a] : nullptr;
  }
  const unsigned b1 = (unsigned)((N + 255) / 256);
  hipLaunchKernelGGL(densify_key_kernel, dim3(b1), dim3(256), 0, s, N, ld, dL_dmeans, w.keys,
                     w.vals, w.sel);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (n_clone > 0) {
    if ((e = gs_pairsort(w.keys, w.vals, (uint64_t)N, 32, w.sort_ws, s)) != hipSuccess) return e;
    hipLaunchKernelGGL(densify_mark_kernel, dim3((unsigned)((n_clone + 255) / 256)), dim3(256), 0,
                       s, n_clone, w.vals, w.sel);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = gs_scan_u32(w.sel, N, w.crank, w.totals, w.scan_ws, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(densify_keep_kernel, dim3(b1), dim3(256), 0, s, N, n_clone, w.sel, w.crank,
                     opacities, min_opacity, w.clone_src, w.keep);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t nc = N + n_clone;
  if ((e = gs_scan_u32(w.keep, nc, w.dest, w.totals + 1, w.scan_ws, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(densify_copy_kernel, dim3((unsigned)((nc + 255) / 256)), dim3(256), 0, s, N,
                     nc, w.clone_src, w.keep, w.dest, pl);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  uint64_t tot = 0;
  if ((e = hipMemcpyAsync(&tot, w.totals + 1, sizeof(uint64_t), hipMemcpyDeviceToHost, s)) !=
      hipSuccess)
    return e;
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return e;
  *num_out = (int64_t)tot;
  return hipSuccess;
}
