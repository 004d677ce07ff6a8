// api.hip — host side of the C ABI declared in include/gsraster.h: argument
// validation, status codes and kernel launches.  Holds no state between
// calls except a thread-local error message.
#include <stdio.h>
#include <string.h>

#include <cmath>

#include <mutex>

#include "gs_common.h"

// The scratch of gs_bin_and_sort_noalloc (see noalloc_scratch below).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

extern "C" {
hipError_t gs_launch_project_fwd(int64_t N, int64_t ld, int deg, const float* means,
                                 const float* scales, const float* quats, const float* sh,
                                 int ncams, const gs::Cam* cams, const gs::Settings& st,
                                 float* means2d, float* conics, float* chol, float* depths,
                                 int32_t* radii, float* colors, uint32_t* tiles,
                                 hipStream_t stream);
hipError_t gs_launch_project_bwd(int64_t N, int64_t ld, const uint32_t* vis_ids, int64_t ldo,
                                 int deg, const float* means, const float* scales,
                                 const float* quats, const float* sh, int ncams,
                                 const gs::Cam* cams, const gs::Settings& st,
                                 const int32_t* radii, const gs::Grad2D& g, float* o_means,
                                 float* o_scales, float* o_quats, float* o_opac, float* o_sh,
                                 int accumulate, hipStream_t stream);
size_t gs_binsort_workspace_bytes(int64_t N, uint64_t capacity, int32_t T);
hipError_t gs_launch_bin_front(int64_t N, int64_t ld, const float* means2d,
                               const int32_t* radii, const float* depths, const uint32_t* tiles,
                               uint32_t* offsets, uint32_t* vis_ids, int32_t W, int32_t H,
                               int ncams, uint64_t* keys, uint32_t* ids, uint32_t* ranges,
                               void* workspace, uint64_t capacity, uint64_t* totals_host,
                               int* dbits, uint64_t* dev_counts, hipStream_t s);
hipError_t gs_launch_bin_back(int64_t N, int32_t W, int32_t H, int ncams, uint64_t M, int dbits,
                              bool device_count, uint64_t* keys, uint32_t* ids, uint32_t* ranges,
                              void* workspace, uint64_t capacity, hipStream_t s);
hipError_t gs_launch_tile_order(int32_t W, int32_t H, int ncams, const uint32_t* ranges,
                                uint32_t* order, hipStream_t s);
hipError_t gs_launch_pack_splats(int64_t rows, int64_t ld, const float* means2d,
                                 const float* conics, const float* chol, const float* opac,
                                 const float* colors, const int32_t* radii, float alpha_min,
                                 float* rec, hipStream_t s);
hipError_t gs_launch_raster_fwd(int32_t W, int32_t H, int ncams, const uint32_t* ranges,
                                const uint32_t* order, const uint32_t* ids, const float* splats,
                                const float* depths,
                                const float* bg, const gs::Settings& st, float* image,
                                float* final_T, uint32_t* last_idx, float* out_depth,
                                float* out_alpha, uint64_t* counters, int loss_kind,
                                const float* target, float* dl, float* loss, hipStream_t s);
hipError_t gs_launch_raster_bwd(int64_t N, int32_t W, int32_t H, int ncams,
                                const uint32_t* ranges, const uint32_t* order,
                                const uint32_t* ids, const float* splats, const uint32_t* offsets,
                                const uint32_t* tiles, const float* bg, const gs::Settings& st,
                                const float* final_T, const uint32_t* last_idx,
                                const float* dL_dimage, float* partials, uint64_t capacity,
                                const gs::Grad2D& g, int accumulate, const uint32_t* vis_ids,
                                int64_t num_visible, uint64_t* counters, hipStream_t s);
hipError_t gs_launch_loss_grad(int kind, int64_t n, const float* img, const float* tgt, float* g,
                               float* loss, hipStream_t s);
size_t gs_ssim_workspace_bytes(int32_t W, int32_t H);
hipError_t gs_launch_l1_dssim(int32_t W, int32_t H, const float* img, const float* tgt,
                              float lambda, float* g, float* loss, void* workspace,
                              hipStream_t s);
hipError_t gs_launch_adam(int64_t rows, int64_t ld, int64_t ldg, const uint32_t* vis_ids, int deg,
                          int64_t step, const gs_adam_config& cfg, float* const raw[5],
                          const float* const grad[5], float* scales, float* opacities,
                          float* m, float* v, hipStream_t s);
int64_t gs_densify_clone_count(int64_t N, float clone_fraction);
size_t gs_densify_workspace_bytes(int64_t N, float clone_fraction);
hipError_t gs_launch_densify(int64_t N, int nplanes, const float* const* in_planes, int64_t ld,
                             const float* dL_dmeans, const float* opacities, float clone_fraction,
                             float min_opacity, float* const* out_planes, int64_t* num_out,
                             void* workspace, hipStream_t s);
}

namespace {

thread_local char g_err[512] = "";

gs_status fail(gs_status s, const char* fmt, const char* what) {
  snprintf(g_err, sizeof(g_err), fmt, what);
  return s;
}

gs_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) {
    g_err[0] = 0;
    return GS_OK;
  }
  snprintf(g_err, sizeof(g_err), "%s: %s", where, hipGetErrorString(e));
  return GS_ERR_HIP;
}

#define GS_REQUIRE(cond, msg)                                        \
  do {                                                               \
    if (!(cond)) return fail(GS_ERR_INVALID_ARGUMENT, "%s", msg);    \
  } while (0)

gs_status check_sizes(int64_t N, int64_t ld) {
  GS_REQUIRE(N >= 0, "N must be >= 0");
  GS_REQUIRE(ld >= N, "ld must be >= N");
  GS_REQUIRE(N < (int64_t)1 << 31, "N must be < 2^31");
  GS_REQUIRE(ld <= ((int64_t)1 << 40), "ld too large");
  return GS_OK;
}

gs_status check_image(int32_t W, int32_t H) {
  GS_REQUIRE(W > 0 && H > 0, "width and height must be > 0");
  GS_REQUIRE((int64_t)W * H < ((int64_t)1 << 31), "image too large");
  return GS_OK;
}

gs_status check_camera(const gs_camera* cam) {
  GS_REQUIRE(cam != nullptr, "camera is NULL");
  gs_status s = check_image(cam->width, cam->height);
  if (s != GS_OK) return s;
  GS_REQUIRE(cam->fx > 0.0f && cam->fy > 0.0f, "fx and fy must be > 0");
  GS_REQUIRE(cam->near_plane > 0.0f && cam->far_plane > cam->near_plane,
             "need 0 < near_plane < far_plane");
  return GS_OK;
}

gs_status check_settings(const gs_settings* st) {
  GS_REQUIRE(st != nullptr, "settings is NULL");
  GS_REQUIRE(st->eps2d >= 0.0f, "eps2d must be >= 0");
  GS_REQUIRE(st->alpha_min > 0.0f && st->alpha_max < 1.0f && st->alpha_min <= st->alpha_max,
             "need 0 < alpha_min <= alpha_max < 1");
  GS_REQUIRE(st->T_min > 0.0f && st->T_min < 1.0f, "need 0 < T_min < 1");
  GS_REQUIRE(st->fov_clamp > 0.0f, "fov_clamp must be > 0");
  return GS_OK;
}

bool aligned64(const void* p) { return ((uintptr_t)p & 63u) == 0; }

#define GS_CHECK(expr)               \
  do {                               \
    gs_status _s = (expr);           \
    if (_s != GS_OK) return _s;      \
  } while (0)

gs_status check_bin_args(int64_t N, int64_t ld, const float* means2d, const int32_t* radii,
                         const float* depths, const uint32_t* tiles_touched, int32_t width,
                         int32_t height, uint32_t* offsets, uint64_t capacity,
                         uint64_t* num_instances, uint64_t* keys, uint32_t* ids,
                         uint32_t* tile_ranges) {
  GS_CHECK(check_sizes(N, ld));
  GS_CHECK(check_image(width, height));
  GS_REQUIRE(num_instances != nullptr, "num_instances is NULL");
  GS_REQUIRE(tile_ranges != nullptr, "tile_ranges is NULL");
  GS_REQUIRE(capacity < ((uint64_t)1 << 30), "capacity must be < 2^30");
  if (N > 0)
    GS_REQUIRE(means2d && radii && depths && tiles_touched && offsets, "NULL array pointer");
  if (capacity > 0) GS_REQUIRE(keys && ids, "keys/ids are NULL");
  return GS_OK;
}

// Scan and duplicate while M is read back, then sort and extract the
// ranges, with the sort's scratch in `workspace` (at least
// gs_binsort_workspace_bytes).
gs_status bin_and_sort_impl(int64_t N, int64_t ld, const float* means2d, const int32_t* radii,
                            const float* depths, const uint32_t* tiles_touched, int32_t width,
                            int32_t height, uint32_t* offsets, uint64_t capacity,
                            uint64_t* num_instances, uint64_t* keys, uint32_t* ids,
                            uint32_t* tile_ranges, void* workspace, hipStream_t s,
                            const char* name) {
  int dbits = 32;
  gs_status st = hip_status(gs_launch_bin_front(N, ld, means2d, radii, depths, tiles_touched,
                                                offsets, nullptr, width, height, 1, keys, ids,
                                                tile_ranges, workspace, capacity, num_instances,
                                                &dbits, nullptr, s),
                            name);
  if (st != GS_OK) return st;
  const uint64_t M = *num_instances;
  if (M >= ((uint64_t)1 << 30))
    return fail(GS_ERR_INVALID_ARGUMENT, "%s", "tile instance count must be < 2^30");
  if (M > capacity) {
    snprintf(g_err, sizeof(g_err), "%s: %llu instances exceed capacity %llu", name,
             (unsigned long long)M, (unsigned long long)capacity);
    return GS_ERR_CAPACITY;
  }
  return hip_status(gs_launch_bin_back(N, width, height, 1, M, dbits, false, keys, ids,
                                       tile_ranges, workspace, capacity, s),
                    name);
}

gs_status check_batch(int32_t num_cams, int64_t ld) {
  GS_REQUIRE(num_cams >= 1 && num_cams <= gs::kMaxCams, "num_cams must be in [1, 8]");
  GS_REQUIRE((int64_t)num_cams * ld < ((int64_t)1 << 31), "num_cams * ld must be < 2^31");
  return GS_OK;
}

size_t staging_bytes(int64_t rows) { return (size_t)(rows > 0 ? rows : 1) * 64; }

// Arguments shared by the compositing calls: `rows` splat rows are staged
// (N for one camera, ncams * ld for a batch).
gs_status check_raster_common(int ncams, int64_t rows, int64_t N, int64_t ld, int32_t width,
                              int32_t height,
                              const uint32_t* tile_ranges, const uint32_t* ids,
                              const float* means2d, const float* conics, const float* chol,
                              const float* opacities, const float* colors, const int32_t* radii,
                              const float* background, const gs_settings* settings,
                              const float* final_T, const uint32_t* last_idx, void* workspace,
                              size_t workspace_bytes) {
  GS_CHECK(check_sizes(N, ld));
  if (ncams > 1) GS_CHECK(check_batch(ncams, ld));
  GS_CHECK(check_image(width, height));
  GS_CHECK(check_settings(settings));
  GS_REQUIRE((int64_t)ncams * width * height < ((int64_t)1 << 31), "images too large");
  GS_REQUIRE(background != nullptr, "background is NULL");
  GS_REQUIRE(tile_ranges && final_T && last_idx, "NULL range, T or last-index pointer");
  if (rows > 0) {
    GS_REQUIRE(ids && means2d && conics && chol && opacities && colors && radii,
               "NULL plane or id pointer");
    GS_REQUIRE(workspace != nullptr, "workspace is NULL");
    GS_REQUIRE(((uintptr_t)workspace & 255u) == 0, "workspace must be 256-byte aligned");
    GS_REQUIRE(workspace_bytes >= staging_bytes(rows),
               "workspace smaller than gs_rasterize_workspace_size()");
  }
  return GS_OK;
}

gs_status check_fwd(int ncams, int64_t rows, int64_t N, int64_t ld, int32_t width,
                    int32_t height,
                    const uint32_t* tile_ranges, const uint32_t* ids, const float* means2d,
                    const float* conics, const float* chol, const float* opacities,
                    const float* colors, const int32_t* radii, const float* depths,
                    const float* background, const gs_settings* settings, float* image,
                    float* final_T, uint32_t* last_idx, float* out_depth, void* workspace,
                    size_t workspace_bytes) {
  GS_CHECK(check_raster_common(ncams, rows, N, ld, width, height, tile_ranges, ids, means2d,
                               conics, chol, opacities, colors, radii, background, settings,
                               final_T, last_idx, workspace, workspace_bytes));
  GS_REQUIRE(image != nullptr, "image is NULL");
  if (out_depth) GS_REQUIRE(depths != nullptr, "out_depth needs depths");
  return GS_OK;
}

gs_status check_loss(int32_t kind, const float* target, const float* image,
                     const float* dL_dimage) {
  GS_REQUIRE(kind == 0 || kind == 1, "kind must be 0 (L2) or 1 (L1)");
  GS_REQUIRE(target && dL_dimage, "NULL target or gradient pointer");
  GS_REQUIRE(dL_dimage != image && dL_dimage != target, "dL_dimage must not alias the images");
  return GS_OK;
}

// out_rows: rows of the 2D gradient planes written (N for one camera,
// ncams * ld for a batch, the visible count for packed rows).
gs_status check_bwd(int ncams, int64_t rows, int64_t N, int64_t ld, int64_t out_rows,
                    int32_t width, int32_t height, const uint32_t* tile_ranges, const uint32_t* ids,
                    const float* means2d, const float* conics, const float* chol,
                    const float* opacities, const float* colors, const int32_t* radii,
                    const uint32_t* offsets, const uint32_t* tiles_touched,
                    uint64_t num_instances, const float* background,
                    const gs_settings* settings, const float* final_T, const uint32_t* last_idx,
                    const float* dL_dimage, void* workspace, size_t workspace_bytes,
                    int32_t staged, float* partials, uint64_t partials_capacity,
                    float* dL_dmeans2d, float* dL_dconics, float* dL_dopacities,
                    float* dL_dcolors, int32_t accumulate) {
  GS_CHECK(check_raster_common(ncams, rows, N, ld, width, height, tile_ranges, ids, means2d,
                               conics, chol, opacities, colors, radii, background, settings,
                               final_T, last_idx, workspace, workspace_bytes));
  GS_REQUIRE(dL_dimage != nullptr, "dL_dimage is NULL");
  GS_REQUIRE(staged == 0 || staged == 1, "staged must be 0 or 1");
  GS_REQUIRE(accumulate >= 0 && accumulate <= 2, "accumulate must be 0, 1 or 2");
  GS_REQUIRE(num_instances <= partials_capacity, "partials smaller than num_instances");
  if (rows > 0) GS_REQUIRE(offsets && tiles_touched, "NULL offset or tile-count pointer");
  if (out_rows > 0)
    GS_REQUIRE(dL_dmeans2d && dL_dconics && dL_dopacities && dL_dcolors,
               "NULL gradient plane pointer");
  if (num_instances > 0) {
    GS_REQUIRE(partials != nullptr, "partials is NULL");
    GS_REQUIRE(aligned64(partials), "partials must be 64-byte aligned");
  }
  return GS_OK;
}

// Scratch of gs_bin_and_sort_noalloc: a file-scope device array, so that the
// call never allocates.  Each device holds its own copy at its own address;
// the host-side name is only a stand-in, so the address is looked up once
// per device with hipGetSymbolAddress and kept.  Calls on one device share
// the array (overlapping calls there race).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

gs_status noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "gs_bin_and_sort_noalloc(hipGetDevice)");
  GS_REQUIRE(dev >= 0 && dev < kMaxDevices, "device index out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol,
                        "gs_bin_and_sort_noalloc(hipGetSymbolAddress)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GS_OK;
}

}  // namespace

extern "C" {

gs_settings gs_default_settings(void) {
  gs_settings s;
  s.eps2d = 0.3f;
  s.alpha_min = 1.0f / 255.0f;
  s.alpha_max = 0.99f;
  s.T_min = 1e-4f;
  s.fov_clamp = 1.3f;
  s.sh_offset = 0.5f;
  return s;
}

const char* gs_status_string(gs_status s) {
  switch (s) {
    case GS_OK: return "GS_OK";
    case GS_ERR_INVALID_ARGUMENT: return "GS_ERR_INVALID_ARGUMENT";
    case GS_ERR_CAPACITY: return "GS_ERR_CAPACITY";
    case GS_ERR_HIP: return "GS_ERR_HIP";
  }
  return "GS_ERR_UNKNOWN";
}

const char* gs_last_error(void) { return g_err; }

int32_t gs_num_tiles(int32_t width, int32_t height) {
  if (width <= 0 || height <= 0) return 0;
  return gs::grid_dim(width) * gs::grid_dim(height);
}

gs_status gs_project_fwd(int64_t N, int64_t ld, int32_t sh_degree, const float* means,
                         const float* scales, const float* quats, const float* sh,
                         const gs_camera* cam, const gs_settings* settings, float* means2d,
                         float* conics, float* chol, float* depths, int32_t* radii,
                         float* colors, uint32_t* tiles_touched, void* stream) {
  GS_CHECK(check_sizes(N, ld));
  GS_REQUIRE(sh_degree >= 0 && sh_degree <= 3, "sh_degree must be in [0, 3]");
  GS_CHECK(check_camera(cam));
  GS_CHECK(check_settings(settings));
  if (N > 0)
    GS_REQUIRE(means && scales && quats && sh && means2d && conics && chol && depths && radii &&
                   colors && tiles_touched,
               "NULL array pointer");
  const gs::Cam c = gs::make_cam(*cam);
  return hip_status(gs_launch_project_fwd(N, ld, sh_degree, means, scales, quats, sh, 1, &c,
                                          gs::make_settings(*settings), means2d, conics, chol,
                                          depths, radii, colors, tiles_touched,
                                          (hipStream_t)stream),
                    "gs_project_fwd");
}

size_t gs_bin_and_sort_workspace_size(int64_t N, uint64_t capacity, int32_t width,
                                      int32_t height) {
  if (N < 0 || width <= 0 || height <= 0) return 0;
  return gs_binsort_workspace_bytes(N, capacity, gs_num_tiles(width, height));
}

gs_status gs_bin_and_sort(int64_t N, int64_t ld, const float* means2d, const int32_t* radii,
                          const float* depths, const uint32_t* tiles_touched, int32_t width,
                          int32_t height, uint32_t* offsets, uint64_t capacity,
                          uint64_t* num_instances, uint64_t* keys, uint32_t* ids,
                          uint32_t* tile_ranges, void* workspace, size_t workspace_bytes,
                          void* stream) {
  GS_CHECK(check_bin_args(N, ld, means2d, radii, depths, tiles_touched, width, height, offsets,
                          capacity, num_instances, keys, ids, tile_ranges));
  GS_REQUIRE(workspace != nullptr, "workspace is NULL");
  GS_REQUIRE(((uintptr_t)workspace & 255u) == 0, "workspace must be 256-byte aligned");
  GS_REQUIRE(workspace_bytes >= gs_binsort_workspace_bytes(N, capacity, gs_num_tiles(width, height)),
             "workspace smaller than gs_bin_and_sort_workspace_size()");
  return bin_and_sort_impl(N, ld, means2d, radii, depths, tiles_touched, width, height, offsets,
                           capacity, num_instances, keys, ids, tile_ranges, workspace,
                           (hipStream_t)stream, "gs_bin_and_sort");
}

gs_status gs_bin_and_sort_noalloc(int64_t N, int64_t ld, const float* means2d,
                                  const int32_t* radii, const float* depths,
                                  const uint32_t* tiles_touched, int32_t width, int32_t height,
                                  uint32_t* offsets, uint64_t capacity, uint64_t* num_instances,
                                  uint64_t* keys, uint32_t* ids, uint32_t* tile_ranges,
                                  void* stream) {
  GS_CHECK(check_bin_args(N, ld, means2d, radii, depths, tiles_touched, width, height, offsets,
                          capacity, num_instances, keys, ids, tile_ranges));
  const size_t need = gs_binsort_workspace_bytes(N, capacity, gs_num_tiles(width, height));
  if (need > kNoAllocScratchBytes) {
    snprintf(g_err, sizeof(g_err),
             "gs_bin_and_sort_noalloc: N = %lld, capacity = %llu and a %dx%d image need %zu "
             "bytes of scratch, more than its %zu",
             (long long)N, (unsigned long long)capacity, (int)width, (int)height, need,
             kNoAllocScratchBytes);
    return GS_ERR_INVALID_ARGUMENT;
  }
  void* ws = nullptr;
  GS_CHECK(noalloc_scratch(&ws));
  return bin_and_sort_impl(N, ld, means2d, radii, depths, tiles_touched, width, height, offsets,
                           capacity, num_instances, keys, ids, tile_ranges, ws,
                           (hipStream_t)stream, "gs_bin_and_sort_noalloc");
}

gs_status gs_bin_and_sort_device(int64_t N, int64_t ld, const float* means2d,
                                 const int32_t* radii, const float* depths,
                                 const uint32_t* tiles_touched, int32_t width, int32_t height,
                                 uint32_t* offsets, uint64_t capacity, uint64_t* counts,
                                 uint64_t* keys, uint32_t* ids, uint32_t* tile_ranges,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  GS_CHECK(check_sizes(N, ld));
  GS_CHECK(check_image(width, height));
  GS_REQUIRE(counts != nullptr, "counts is NULL");
  GS_REQUIRE(tile_ranges != nullptr, "tile_ranges is NULL");
  GS_REQUIRE(workspace != nullptr, "workspace is NULL");
  GS_REQUIRE(((uintptr_t)workspace & 255u) == 0, "workspace must be 256-byte aligned");
  GS_REQUIRE(capacity < ((uint64_t)1 << 30), "capacity must be < 2^30");
  if (N > 0)
    GS_REQUIRE(means2d && radii && depths && tiles_touched && offsets, "NULL array pointer");
  if (capacity > 0) GS_REQUIRE(keys && ids, "keys/ids are NULL");
  const int32_t T = gs_num_tiles(width, height);
  GS_REQUIRE(workspace_bytes >= gs_binsort_workspace_bytes(N, capacity, T),
             "workspace smaller than gs_bin_and_sort_workspace_size()");
  hipStream_t s = (hipStream_t)stream;
  gs_status st = hip_status(gs_launch_bin_front(N, ld, means2d, radii, depths, tiles_touched,
                                                offsets, nullptr, width, height, 1, keys, ids,
                                                tile_ranges, workspace, capacity, nullptr,
                                                nullptr, counts, s),
                            "gs_bin_and_sort_device(scan)");
  if (st != GS_OK) return st;
  return hip_status(gs_launch_bin_back(N, width, height, 1, 0, 32, true, keys, ids, tile_ranges,
                                       workspace, capacity, s),
                    "gs_bin_and_sort_device");
}

gs_status gs_tile_order(int32_t num_cams, int32_t width, int32_t height,
                        const uint32_t* tile_ranges, uint32_t* tile_order, void* stream) {
  GS_REQUIRE(num_cams >= 1 && num_cams <= gs::kMaxCams, "num_cams must be in [1, 8]");
  GS_CHECK(check_image(width, height));
  GS_REQUIRE(tile_ranges && tile_order, "NULL range or order pointer");
  GS_REQUIRE((const void*)tile_ranges != (const void*)tile_order,
             "tile_order must not alias tile_ranges");
  return hip_status(gs_launch_tile_order(width, height, num_cams, tile_ranges, tile_order,
                                         (hipStream_t)stream),
                    "gs_tile_order");
}

size_t gs_rasterize_workspace_size(int64_t rows) {
  if (rows < 0) return 0;
  return (size_t)(rows > 0 ? rows : 1) * 64;
}

gs_status gs_rasterize_fwd(int64_t N, int64_t ld, int32_t width, int32_t height,
                           const uint32_t* tile_ranges, const uint32_t* tile_order,
                           const uint32_t* ids, const float* means2d, const float* conics,
                           const float* chol, const float* opacities, const float* colors,
                           const int32_t* radii, const float* depths, const float* background,
                           const gs_settings* settings, float* image, float* final_T,
                           uint32_t* last_idx, float* out_depth, float* out_alpha,
                           void* workspace, size_t workspace_bytes, uint64_t* counters,
                           void* stream) {
  GS_CHECK(check_fwd(1, N, N, ld, width, height, tile_ranges, ids, means2d, conics, chol,
                     opacities, colors, radii, depths, background, settings, image, final_T,
                     last_idx, out_depth, workspace, workspace_bytes));
  hipStream_t s = (hipStream_t)stream;
  GS_CHECK(hip_status(gs_launch_pack_splats(N, ld, means2d, conics, chol, opacities, colors,
                                            radii, settings->alpha_min, (float*)workspace, s),
                      "gs_rasterize_fwd(stage)"));
  return hip_status(gs_launch_raster_fwd(width, height, 1, tile_ranges, tile_order, ids,
                                         (const float*)workspace, depths, background,
                                         gs::make_settings(*settings), image, final_T, last_idx,
                                         out_depth, out_alpha, counters, -1, nullptr, nullptr,
                                         nullptr, s),
                    "gs_rasterize_fwd");
}

gs_status gs_rasterize_fwd_loss(int64_t N, int64_t ld, int32_t width, int32_t height,
                                const uint32_t* tile_ranges, const uint32_t* tile_order,
                                const uint32_t* ids, const float* means2d, const float* conics,
                                const float* chol, const float* opacities, const float* colors,
                                const int32_t* radii, const float* depths,
                                const float* background, const gs_settings* settings,
                                int32_t kind, const float* target, float* image, float* final_T,
                                uint32_t* last_idx, float* out_depth, float* out_alpha,
                                float* dL_dimage, float* loss, void* workspace,
                                size_t workspace_bytes, uint64_t* counters, void* stream) {
  GS_CHECK(check_fwd(1, N, N, ld, width, height, tile_ranges, ids, means2d, conics, chol,
                     opacities, colors, radii, depths, background, settings, image, final_T,
                     last_idx, out_depth, workspace, workspace_bytes));
  GS_CHECK(check_loss(kind, target, image, dL_dimage));
  hipStream_t s = (hipStream_t)stream;
  GS_CHECK(hip_status(gs_launch_pack_splats(N, ld, means2d, conics, chol, opacities, colors,
                                            radii, settings->alpha_min, (float*)workspace, s),
                      "gs_rasterize_fwd_loss(stage)"));
  return hip_status(gs_launch_raster_fwd(width, height, 1, tile_ranges, tile_order, ids,
                                         (const float*)workspace, depths, background,
                                         gs::make_settings(*settings), image, final_T, last_idx,
                                         out_depth, out_alpha, counters, kind, target, dL_dimage,
                                         loss, s),
                    "gs_rasterize_fwd_loss");
}

gs_status gs_rasterize_bwd(int64_t N, int64_t ld, int32_t width, int32_t height,
                           const uint32_t* tile_ranges, const uint32_t* tile_order,
                           const uint32_t* ids, const float* means2d, const float* conics,
                           const float* chol, const float* opacities, const float* colors,
                           const int32_t* radii, const uint32_t* offsets,
                           const uint32_t* tiles_touched, uint64_t num_instances,
                           const float* background, const gs_settings* settings,
                           const float* final_T, const uint32_t* last_idx,
                           const float* dL_dimage, void* workspace, size_t workspace_bytes,
                           int32_t staged, float* partials, uint64_t partials_capacity,
                           float* dL_dmeans2d, float* dL_dconics, float* dL_dopacities,
                           float* dL_dcolors, float* dL_dmeans2d_abs, int32_t accumulate,
                           uint64_t* counters, void* stream) {
  GS_CHECK(check_bwd(1, N, N, ld, N, width, height, tile_ranges, ids, means2d, conics, chol,
                     opacities, colors, radii, offsets, tiles_touched, num_instances, background,
                     settings, final_T, last_idx, dL_dimage, workspace, workspace_bytes, staged,
                     partials, partials_capacity, dL_dmeans2d, dL_dconics, dL_dopacities,
                     dL_dcolors, accumulate));
  hipStream_t s = (hipStream_t)stream;
  if (!staged)
    GS_CHECK(hip_status(gs_launch_pack_splats(N, ld, means2d, conics, chol, opacities, colors,
                                              radii, settings->alpha_min, (float*)workspace, s),
                        "gs_rasterize_bwd(stage)"));
  const gs::Grad2D g{dL_dmeans2d, dL_dconics, dL_dopacities, dL_dcolors, dL_dmeans2d_abs, ld};
  return hip_status(gs_launch_raster_bwd(N, width, height, 1, tile_ranges, tile_order, ids,
                                         (const float*)workspace, offsets, tiles_touched,
                                         background, gs::make_settings(*settings), final_T,
                                         last_idx, dL_dimage, partials, num_instances, g,
                                         accumulate, nullptr, 0, counters, s),
                    "gs_rasterize_bwd");
}

gs_status gs_project_bwd(int64_t N, int64_t ld, int32_t sh_degree, const float* means,
                         const float* scales, const float* quats, const float* sh,
                         const gs_camera* cam, const gs_settings* settings,
                         const int32_t* radii, const float* dL_dmeans2d,
                         const float* dL_dconics, const float* dL_dcolors, float* dL_dmeans,
                         float* dL_dscales, float* dL_dquats, float* dL_dsh,
                         int32_t accumulate, void* stream) {
  GS_CHECK(check_sizes(N, ld));
  GS_REQUIRE(sh_degree >= 0 && sh_degree <= 3, "sh_degree must be in [0, 3]");
  GS_CHECK(check_camera(cam));
  GS_CHECK(check_settings(settings));
  GS_REQUIRE(accumulate == 0 || accumulate == 1, "accumulate must be 0 or 1");
  if (N > 0)
    GS_REQUIRE(means && scales && quats && sh && radii && dL_dmeans2d && dL_dconics &&
                   dL_dcolors && dL_dmeans && dL_dscales && dL_dquats && dL_dsh,
               "NULL array pointer");
  const gs::Cam c = gs::make_cam(*cam);
  const gs::Grad2D g{(float*)dL_dmeans2d, (float*)dL_dconics, nullptr, (float*)dL_dcolors,
                     nullptr, ld};
  return hip_status(gs_launch_project_bwd(N, ld, nullptr, ld, sh_degree, means, scales, quats, sh,
                                          1, &c, gs::make_settings(*settings), radii, g,
                                          dL_dmeans, dL_dscales, dL_dquats, nullptr, dL_dsh,
                                          accumulate, (hipStream_t)stream),
                    "gs_project_bwd");
}

gs_status gs_bin_and_sort_packed(int64_t N, int64_t ld, const float* means2d,
                                 const int32_t* radii, const float* depths,
                                 const uint32_t* tiles_touched, int32_t width, int32_t height,
                                 uint32_t* offsets, uint64_t capacity, uint64_t* counts,
                                 uint64_t* keys, uint32_t* ids, uint32_t* tile_ranges,
                                 uint32_t* vis_ids, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  GS_CHECK(check_sizes(N, ld));
  GS_CHECK(check_image(width, height));
  GS_REQUIRE(counts != nullptr, "counts is NULL");
  GS_REQUIRE(tile_ranges != nullptr, "tile_ranges is NULL");
  GS_REQUIRE(workspace != nullptr, "workspace is NULL");
  GS_REQUIRE(((uintptr_t)workspace & 255u) == 0, "workspace must be 256-byte aligned");
  GS_REQUIRE(capacity < ((uint64_t)1 << 30), "capacity must be < 2^30");
  if (N > 0)
    GS_REQUIRE(means2d && radii && depths && tiles_touched && offsets && vis_ids,
               "NULL array pointer");
  if (capacity > 0) GS_REQUIRE(keys && ids, "keys/ids are NULL");
  const int32_t T = gs_num_tiles(width, height);
  GS_REQUIRE(workspace_bytes >= gs_binsort_workspace_bytes(N, capacity, T),
             "workspace smaller than gs_bin_and_sort_workspace_size()");
  hipStream_t s = (hipStream_t)stream;
  int dbits = 32;
  gs_status st = hip_status(gs_launch_bin_front(N, ld, means2d, radii, depths, tiles_touched,
                                                offsets, vis_ids, width, height, 1, keys, ids,
                                                tile_ranges, workspace, capacity, counts, &dbits,
                                                nullptr, s),
                            "gs_bin_and_sort_packed(scan)");
  if (st != GS_OK) return st;
  const uint64_t M = counts[0];
  if (M >= ((uint64_t)1 << 30))
    return fail(GS_ERR_INVALID_ARGUMENT, "%s", "tile instance count must be < 2^30");
  if (M > capacity) {
    snprintf(g_err, sizeof(g_err), "gs_bin_and_sort_packed: %llu instances exceed capacity %llu",
             (unsigned long long)M, (unsigned long long)capacity);
    return GS_ERR_CAPACITY;
  }
  return hip_status(gs_launch_bin_back(N, width, height, 1, M, dbits, false, keys, ids,
                                       tile_ranges, workspace, capacity, s),
                    "gs_bin_and_sort_packed");
}

gs_status gs_rasterize_bwd_packed(int64_t N, int64_t ld, int32_t width, int32_t height,
                                  const uint32_t* tile_ranges, const uint32_t* tile_order,
                                  const uint32_t* ids, const float* means2d,
                                  const float* conics, const float* chol,
                                  const float* opacities, const float* colors,
                                  const int32_t* radii, const uint32_t* offsets,
                                  const uint32_t* tiles_touched, uint64_t num_instances,
                                  const uint32_t* vis_ids, int64_t num_visible, int64_t ldv,
                                  const float* background, const gs_settings* settings,
                                  const float* final_T, const uint32_t* last_idx,
                                  const float* dL_dimage, void* workspace,
                                  size_t workspace_bytes, int32_t staged, float* partials,
                                  uint64_t partials_capacity, float* dL_dmeans2d,
                                  float* dL_dconics, float* dL_dopacities, float* dL_dcolors,
                                  float* dL_dmeans2d_abs, int32_t accumulate,
                                  uint64_t* counters, void* stream) {
  GS_REQUIRE(num_visible >= 0 && num_visible <= N, "num_visible must be in [0, N]");
  GS_REQUIRE(ldv >= num_visible && ldv <= ((int64_t)1 << 40), "ldv must be >= num_visible");
  GS_CHECK(check_bwd(1, N, N, ld, num_visible, width, height, tile_ranges, ids, means2d, conics,
                     chol, opacities, colors, radii, offsets, tiles_touched, num_instances,
                     background, settings, final_T, last_idx, dL_dimage, workspace,
                     workspace_bytes, staged, partials, partials_capacity, dL_dmeans2d,
                     dL_dconics, dL_dopacities, dL_dcolors, accumulate));
  if (num_visible > 0) GS_REQUIRE(vis_ids != nullptr, "vis_ids is NULL");
  hipStream_t s = (hipStream_t)stream;
  if (!staged)
    GS_CHECK(hip_status(gs_launch_pack_splats(N, ld, means2d, conics, chol, opacities, colors,
                                              radii, settings->alpha_min, (float*)workspace, s),
                        "gs_rasterize_bwd_packed(stage)"));
  // an empty list still needs a non-NULL pointer to select the packed rows
  static const uint32_t kNoIds = 0;
  const gs::Grad2D g{dL_dmeans2d, dL_dconics, dL_dopacities, dL_dcolors, dL_dmeans2d_abs,
                     ldv > 0 ? ldv : 1};
  return hip_status(gs_launch_raster_bwd(N, width, height, 1, tile_ranges, tile_order, ids,
                                         (const float*)workspace, offsets, tiles_touched,
                                         background, gs::make_settings(*settings), final_T,
                                         last_idx, dL_dimage, partials, num_instances, g,
                                         accumulate, vis_ids ? vis_ids : &kNoIds, num_visible,
                                         counters, s),
                    "gs_rasterize_bwd_packed");
}

gs_status gs_project_bwd_packed(int64_t num_visible, const uint32_t* vis_ids, int64_t N,
                                int64_t ld, int64_t ldv, int32_t sh_degree, const float* means,
                                const float* scales, const float* quats, const float* sh,
                                const gs_camera* cam, const gs_settings* settings,
                                const int32_t* radii, const float* dL_dmeans2d,
                                const float* dL_dconics, const float* dL_dcolors,
                                float* dL_dmeans, float* dL_dscales, float* dL_dquats,
                                float* dL_dsh, int32_t accumulate, void* stream) {
  GS_CHECK(check_sizes(N, ld));
  GS_REQUIRE(num_visible >= 0 && num_visible <= N, "num_visible must be in [0, N]");
  GS_REQUIRE(ldv >= num_visible, "ldv must be >= num_visible");
  GS_REQUIRE(ldv <= ((int64_t)1 << 40), "ldv too large");
  GS_REQUIRE(sh_degree >= 0 && sh_degree <= 3, "sh_degree must be in [0, 3]");
  GS_CHECK(check_camera(cam));
  GS_CHECK(check_settings(settings));
  GS_REQUIRE(accumulate == 0 || accumulate == 1, "accumulate must be 0 or 1");
  if (num_visible == 0) return GS_OK;
  GS_REQUIRE(vis_ids && means && scales && quats && sh && radii && dL_dmeans2d && dL_dconics &&
                 dL_dcolors && dL_dmeans && dL_dscales && dL_dquats && dL_dsh,
             "NULL array pointer");
  const gs::Cam c = gs::make_cam(*cam);
  const gs::Grad2D g{(float*)dL_dmeans2d, (float*)dL_dconics, nullptr, (float*)dL_dcolors,
                     nullptr, ldv};
  return hip_status(gs_launch_project_bwd(num_visible, ld, vis_ids, ldv, sh_degree, means, scales,
                                          quats, sh, 1, &c, gs::make_settings(*settings), radii,
                                          g, dL_dmeans, dL_dscales, dL_dquats, nullptr, dL_dsh,
                                          accumulate, (hipStream_t)stream),
                    "gs_project_bwd_packed");
}

gs_status gs_project_fwd_batched(int32_t num_cams, const gs_camera* cams, int64_t N, int64_t ld,
                                 int32_t sh_degree, const float* means, const float* scales,
                                 const float* quats, const float* sh,
                                 const gs_settings* settings, float* means2d, float* conics,
                                 float* chol, float* depths, int32_t* radii, float* colors,
                                 uint32_t* tiles_touched, void* stream) {
  GS_CHECK(check_sizes(N, ld));
  GS_CHECK(check_batch(num_cams, ld));
  GS_REQUIRE(sh_degree >= 0 && sh_degree <= 3, "sh_degree must be in [0, 3]");
  GS_REQUIRE(cams != nullptr, "cams is NULL");
  GS_CHECK(check_settings(settings));
  gs::Cam cb[gs::kMaxCams];
  for (int c = 0; c < num_cams; ++c) {
    GS_CHECK(check_camera(&cams[c]));
    GS_REQUIRE(cams[c].width == cams[0].width && cams[c].height == cams[0].height,
               "the cameras of a batch must share one image size");
    cb[c] = gs::make_cam(cams[c]);
  }
  if (ld > 0)
    GS_REQUIRE(means2d && conics && chol && depths && radii && colors && tiles_touched,
               "NULL output pointer");
  if (N > 0) GS_REQUIRE(means && scales && quats && sh, "NULL parameter pointer");
  return hip_status(gs_launch_project_fwd(N, ld, sh_degree, means, scales, quats, sh, num_cams,
                                          cb, gs::make_settings(*settings), means2d, conics,
                                          chol, depths, radii, colors, tiles_touched,
                                          (hipStream_t)stream),
                    "gs_project_fwd_batched");
}

size_t gs_bin_and_sort_batched_workspace_size(int32_t num_cams, int64_t ld, uint64_t capacity,
                                              int32_t width, int32_t height) {
  if (num_cams < 1 || num_cams > gs::kMaxCams || ld < 0) return 0;
  return gs_binsort_workspace_bytes((int64_t)num_cams * ld, capacity,
                                    num_cams * gs_num_tiles(width, height));
}

gs_status gs_bin_and_sort_batched(int32_t num_cams, int64_t ld, const float* means2d,
                                  const int32_t* radii, const float* depths,
                                  const uint32_t* tiles_touched, int32_t width, int32_t height,
                                  uint32_t* offsets, uint64_t capacity, uint64_t* num_instances,
                                  uint64_t* keys, uint32_t* ids, uint32_t* tile_ranges,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  GS_CHECK(check_sizes(0, ld));
  GS_CHECK(check_batch(num_cams, ld));
  GS_CHECK(check_image(width, height));
  GS_REQUIRE(num_instances != nullptr, "num_instances is NULL");
  GS_REQUIRE(tile_ranges != nullptr, "tile_ranges is NULL");
  GS_REQUIRE(workspace != nullptr, "workspace is NULL");
  GS_REQUIRE(((uintptr_t)workspace & 255u) == 0, "workspace must be 256-byte aligned");
  GS_REQUIRE(capacity < ((uint64_t)1 << 30), "capacity must be < 2^30");
  const int64_t rows = (int64_t)num_cams * ld;
  const int64_t T = (int64_t)num_cams * gs_num_tiles(width, height);
  GS_REQUIRE(T < ((int64_t)1 << 31), "too many tiles");
  if (rows > 0)
    GS_REQUIRE(means2d && radii && depths && tiles_touched && offsets, "NULL array pointer");
  if (capacity > 0) GS_REQUIRE(keys && ids, "keys/ids are NULL");
  GS_REQUIRE(workspace_bytes >= gs_binsort_workspace_bytes(rows, capacity, (int32_t)T),
             "workspace smaller than gs_bin_and_sort_batched_workspace_size()");
  hipStream_t s = (hipStream_t)stream;
  int dbits = 32;
  gs_status st = hip_status(gs_launch_bin_front(rows, ld, means2d, radii, depths, tiles_touched,
                                                offsets, nullptr, width, height, num_cams, keys,
                                                ids, tile_ranges, workspace, capacity,
                                                num_instances, &dbits, nullptr, s),
                            "gs_bin_and_sort_batched(scan)");
  if (st != GS_OK) return st;
  const uint64_t M = *num_instances;
  if (M >= ((uint64_t)1 << 30))
    return fail(GS_ERR_INVALID_ARGUMENT, "%s", "tile instance count must be < 2^30");
  if (M > capacity) {
    snprintf(g_err, sizeof(g_err), "gs_bin_and_sort_batched: %llu instances exceed capacity %llu",
             (unsigned long long)M, (unsigned long long)capacity);
    return GS_ERR_CAPACITY;
  }
  return hip_status(gs_launch_bin_back(rows, width, height, num_cams, M, dbits, false, keys, ids,
                                       tile_ranges, workspace, capacity, s),
                    "gs_bin_and_sort_batched");
}

gs_status gs_rasterize_fwd_batched(int32_t num_cams, int64_t ld, int32_t width, int32_t height,
                                   const uint32_t* tile_ranges, const uint32_t* tile_order,
                                   const uint32_t* ids, const float* means2d,
                                   const float* conics, const float* chol,
                                   const float* opacities, const float* colors,
                                   const int32_t* radii, const float* depths,
                                   const float* background, const gs_settings* settings,
                                   float* image, float* final_T, uint32_t* last_idx,
                                   float* out_depth, float* out_alpha, void* workspace,
                                   size_t workspace_bytes, uint64_t* counters, void* stream) {
  GS_CHECK(check_batch(num_cams, ld));
  GS_CHECK(check_fwd(num_cams, (int64_t)num_cams * ld, ld, ld, width, height, tile_ranges, ids,
                     means2d, conics, chol, opacities, colors, radii, depths, background,
                     settings, image, final_T, last_idx, out_depth, workspace,
                     workspace_bytes));
  hipStream_t s = (hipStream_t)stream;
  GS_CHECK(hip_status(gs_launch_pack_splats((int64_t)num_cams * ld, ld, means2d, conics, chol,
                                            opacities, colors, radii, settings->alpha_min,
                                            (float*)workspace, s),
                      "gs_rasterize_fwd_batched(stage)"));
  return hip_status(gs_launch_raster_fwd(width, height, num_cams, tile_ranges, tile_order, ids,
                                         (const float*)workspace, depths, background,
                                         gs::make_settings(*settings), image, final_T, last_idx,
                                         out_depth, out_alpha, counters, -1, nullptr, nullptr,
                                         nullptr, s),
                    "gs_rasterize_fwd_batched");
}

gs_status gs_rasterize_fwd_loss_batched(int32_t num_cams, int64_t ld, int32_t width,
                                        int32_t height, const uint32_t* tile_ranges,
                                        const uint32_t* tile_order, const uint32_t* ids,
                                        const float* means2d, const float* conics,
                                        const float* chol, const float* opacities,
                                        const float* colors, const int32_t* radii,
                                        const float* depths, const float* background,
                                        const gs_settings* settings, int32_t kind,
                                        const float* target, float* image, float* final_T,
                                        uint32_t* last_idx, float* out_depth, float* out_alpha,
                                        float* dL_dimage, float* loss, void* workspace,
                                        size_t workspace_bytes, uint64_t* counters,
                                        void* stream) {
  GS_CHECK(check_batch(num_cams, ld));
  GS_CHECK(check_fwd(num_cams, (int64_t)num_cams * ld, ld, ld, width, height, tile_ranges, ids,
                     means2d, conics, chol, opacities, colors, radii, depths, background,
                     settings, image, final_T, last_idx, out_depth, workspace,
                     workspace_bytes));
  GS_CHECK(check_loss(kind, target, image, dL_dimage));
  hipStream_t s = (hipStream_t)stream;
  GS_CHECK(hip_status(gs_launch_pack_splats((int64_t)num_cams * ld, ld, means2d, conics, chol,
                                            opacities, colors, radii, settings->alpha_min,
                                            (float*)workspace, s),
                      "gs_rasterize_fwd_loss_batched(stage)"));
  return hip_status(gs_launch_raster_fwd(width, height, num_cams, tile_ranges, tile_order, ids,
                                         (const float*)workspace, depths, background,
                                         gs::make_settings(*settings), image, final_T, last_idx,
                                         out_depth, out_alpha, counters, kind, target, dL_dimage,
                                         loss, s),
                    "gs_rasterize_fwd_loss_batched");
}

gs_status gs_rasterize_bwd_batched(int32_t num_cams, int64_t ld, int32_t width, int32_t height,
                                   const uint32_t* tile_ranges, const uint32_t* tile_order,
                                   const uint32_t* ids, const float* means2d,
                                   const float* conics, const float* chol,
                                   const float* opacities, const float* colors,
                                   const int32_t* radii, const uint32_t* offsets,
                                   const uint32_t* tiles_touched, uint64_t num_instances,
                                   const float* background, const gs_settings* settings,
                                   const float* final_T, const uint32_t* last_idx,
                                   const float* dL_dimage, void* workspace,
                                   size_t workspace_bytes, int32_t staged, float* partials,
                                   uint64_t partials_capacity, float* dL_dmeans2d,
                                   float* dL_dconics, float* dL_dopacities, float* dL_dcolors,
                                   float* dL_dmeans2d_abs, int32_t accumulate,
                                   uint64_t* counters, void* stream) {
  GS_CHECK(check_batch(num_cams, ld));
  const int64_t rows = (int64_t)num_cams * ld;
  GS_CHECK(check_bwd(num_cams, rows, ld, ld, rows, width, height, tile_ranges, ids,
                     means2d, conics, chol, opacities, colors, radii, offsets, tiles_touched,
                     num_instances, background, settings, final_T, last_idx, dL_dimage,
                     workspace, workspace_bytes, staged, partials, partials_capacity,
                     dL_dmeans2d, dL_dconics, dL_dopacities, dL_dcolors, accumulate));
  hipStream_t s = (hipStream_t)stream;
  if (!staged)
    GS_CHECK(hip_status(gs_launch_pack_splats(rows, ld, means2d, conics, chol, opacities, colors,
                                              radii, settings->alpha_min, (float*)workspace, s),
                        "gs_rasterize_bwd_batched(stage)"));
  const gs::Grad2D g{dL_dmeans2d, dL_dconics, dL_dopacities, dL_dcolors, dL_dmeans2d_abs,
                     ld > 0 ? ld : 1};
  return hip_status(gs_launch_raster_bwd(rows, width, height, num_cams, tile_ranges, tile_order,
                                         ids, (const float*)workspace, offsets, tiles_touched,
                                         background, gs::make_settings(*settings), final_T,
                                         last_idx, dL_dimage, partials, num_instances, g,
                                         accumulate, nullptr, 0, counters, s),
                    "gs_rasterize_bwd_batched");
}

gs_status gs_project_bwd_batched(int32_t num_cams, const gs_camera* cams, int64_t N, int64_t ld,
                                 int32_t sh_degree, const float* means, const float* scales,
                                 const float* quats, const float* sh, const gs_settings* settings,
                                 const int32_t* radii, const float* dL_dmeans2d,
                                 const float* dL_dconics, const float* dL_dcolors,
                                 const float* dL_dopacities_cams, float* dL_dmeans,
                                 float* dL_dscales, float* dL_dquats, float* dL_dopacities,
                                 float* dL_dsh, int32_t accumulate, void* stream) {
  GS_CHECK(check_sizes(N, ld));
  GS_CHECK(check_batch(num_cams, ld));
  GS_REQUIRE(sh_degree >= 0 && sh_degree <= 3, "sh_degree must be in [0, 3]");
  GS_REQUIRE(cams != nullptr, "cams is NULL");
  GS_CHECK(check_settings(settings));
  GS_REQUIRE(accumulate == 0 || accumulate == 1, "accumulate must be 0 or 1");
  GS_REQUIRE((dL_dopacities_cams == nullptr) == (dL_dopacities == nullptr),
             "dL_dopacities_cams and dL_dopacities go together");
  gs::Cam cb[gs::kMaxCams];
  for (int c = 0; c < num_cams; ++c) {
    GS_CHECK(check_camera(&cams[c]));
    cb[c] = gs::make_cam(cams[c]);
  }
  if (N > 0)
    GS_REQUIRE(means && scales && quats && sh && radii && dL_dmeans2d && dL_dconics &&
                   dL_dcolors && dL_dmeans && dL_dscales && dL_dquats && dL_dsh,
               "NULL array pointer");
  const gs::Grad2D g{(float*)dL_dmeans2d, (float*)dL_dconics, (float*)dL_dopacities_cams,
                     (float*)dL_dcolors, nullptr, ld};
  return hip_status(gs_launch_project_bwd(N, ld, nullptr, ld, sh_degree, means, scales, quats, sh,
                                          num_cams, cb, gs::make_settings(*settings), radii, g,
                                          dL_dmeans, dL_dscales, dL_dquats, dL_dopacities,
                                          dL_dsh, accumulate, (hipStream_t)stream),
                    "gs_project_bwd_batched");
}

size_t gs_l1_dssim_workspace_size(int32_t width, int32_t height) {
  if (width <= 0 || height <= 0) return 0;
  return gs_ssim_workspace_bytes(width, height);
}

gs_status gs_l1_dssim_loss_grad(int32_t width, int32_t height, const float* image,
                                const float* target, float lambda, float* dL_dimage,
                                float* loss, void* workspace, size_t workspace_bytes,
                                void* stream) {
  GS_CHECK(check_image(width, height));
  GS_REQUIRE(std::isfinite(lambda) && lambda >= 0.0f, "lambda must be finite and >= 0");
  GS_REQUIRE(image && target && dL_dimage, "NULL image pointer");
  GS_REQUIRE(dL_dimage != image && dL_dimage != target, "dL_dimage must not alias the images");
  GS_REQUIRE(workspace != nullptr, "workspace is NULL");
  GS_REQUIRE(((uintptr_t)workspace & 255u) == 0, "workspace must be 256-byte aligned");
  GS_REQUIRE(workspace_bytes >= gs_ssim_workspace_bytes(width, height),
             "workspace smaller than gs_l1_dssim_workspace_size()");
  return hip_status(gs_launch_l1_dssim(width, height, image, target, lambda, dL_dimage, loss,
                                       workspace, (hipStream_t)stream),
                    "gs_l1_dssim_loss_grad");
}

gs_adam_config gs_default_adam_config(void) {
  gs_adam_config c;
  c.lr_means = 1.6e-4f;
  c.lr_scales = 5e-3f;
  c.lr_quats = 1e-3f;
  c.lr_opacities = 5e-2f;
  c.lr_sh = 2.5e-3f;
  c.beta1 = 0.9f;
  c.beta2 = 0.99f;
  c.eps = 1e-15f;
  return c;
}

namespace {

gs_status check_adam(int64_t step, const gs_adam_config* cfg, int32_t sh_degree) {
  GS_REQUIRE(cfg != nullptr, "cfg is NULL");
  GS_REQUIRE(step >= 1, "step must be >= 1");
  GS_REQUIRE(sh_degree >= 0 && sh_degree <= 3, "sh_degree must be in [0, 3]");
  const float lr[5] = {cfg->lr_means, cfg->lr_scales, cfg->lr_quats, cfg->lr_opacities,
                       cfg->lr_sh};
  for (float x : lr) GS_REQUIRE(std::isfinite(x) && x >= 0.0f, "learning rates must be >= 0");
  GS_REQUIRE(cfg->beta1 >= 0.0f && cfg->beta1 < 1.0f, "beta1 must be in [0, 1)");
  GS_REQUIRE(cfg->beta2 >= 0.0f && cfg->beta2 < 1.0f, "beta2 must be in [0, 1)");
  GS_REQUIRE(std::isfinite(cfg->eps) && cfg->eps >= 0.0f, "eps must be >= 0");
  return GS_OK;
}

}  // namespace

gs_status gs_adam_step(int64_t N, int64_t ld, int32_t sh_degree, int64_t step,
                       const gs_adam_config* cfg, float* means, float* log_scales, float* quats,
                       float* logit_opacities, float* sh, float* scales, float* opacities,
                       const float* dL_dmeans, const float* dL_dscales, const float* dL_dquats,
                       const float* dL_dopacities, const float* dL_dsh, float* exp_avg,
                       float* exp_avg_sq, void* stream) {
  GS_CHECK(check_sizes(N, ld));
  GS_CHECK(check_adam(step, cfg, sh_degree));
  if (N == 0) return GS_OK;
  GS_REQUIRE(means && log_scales && quats && logit_opacities && sh && scales && opacities,
             "NULL parameter pointer");
  GS_REQUIRE(dL_dmeans && dL_dscales && dL_dquats && dL_dopacities && dL_dsh,
             "NULL gradient pointer");
  GS_REQUIRE(exp_avg && exp_avg_sq, "NULL moment pointer");
  float* raw[5] = {means, log_scales, quats, logit_opacities, sh};
  const float* grad[5] = {dL_dmeans, dL_dscales, dL_dquats, dL_dopacities, dL_dsh};
  return hip_status(gs_launch_adam(N, ld, ld, nullptr, sh_degree, step, *cfg, raw, grad, scales,
                                   opacities, exp_avg, exp_avg_sq, (hipStream_t)stream),
                    "gs_adam_step");
}

gs_status gs_adam_step_packed(int64_t num_visible, const uint32_t* vis_ids, int64_t ldv,
                              int64_t N, int64_t ld, int32_t sh_degree, int64_t step,
                              const gs_adam_config* cfg, float* means, float* log_scales,
                              float* quats, float* logit_opacities, float* sh, float* scales,
                              float* opacities, const float* dL_dmeans, const float* dL_dscales,
                              const float* dL_dquats, const float* dL_dopacities,
                              const float* dL_dsh, float* exp_avg, float* exp_avg_sq,
                              void* stream) {
  GS_CHECK(check_sizes(N, ld));
  GS_CHECK(check_adam(step, cfg, sh_degree));
  GS_REQUIRE(num_visible >= 0 && num_visible <= N, "num_visible must be in [0, N]");
  GS_REQUIRE(ldv >= num_visible && ldv <= ((int64_t)1 << 40), "ldv must be >= num_visible");
  if (num_visible == 0) return GS_OK;
  GS_REQUIRE(vis_ids != nullptr, "vis_ids is NULL");
  GS_REQUIRE(means && log_scales && quats && logit_opacities && sh && scales && opacities,
             "NULL parameter pointer");
  GS_REQUIRE(dL_dmeans && dL_dscales && dL_dquats && dL_dopacities && dL_dsh,
             "NULL gradient pointer");
  GS_REQUIRE(exp_avg && exp_avg_sq, "NULL moment pointer");
  float* raw[5] = {means, log_scales, quats, logit_opacities, sh};
  const float* grad[5] = {dL_dmeans, dL_dscales, dL_dquats, dL_dopacities, dL_dsh};
  return hip_status(gs_launch_adam(num_visible, ld, ldv, vis_ids, sh_degree, step, *cfg, raw,
                                   grad, scales, opacities, exp_avg, exp_avg_sq,
                                   (hipStream_t)stream),
                    "gs_adam_step_packed");
}

gs_status gs_image_loss_grad(int32_t kind, int64_t count, const float* image,
                             const float* target, float* dL_dimage, float* loss,
                             void* stream) {
  GS_REQUIRE(kind == 0 || kind == 1, "kind must be 0 (L2) or 1 (L1)");
  GS_REQUIRE(count >= 0, "count must be >= 0");
  if (count > 0) GS_REQUIRE(image && target && dL_dimage, "NULL array pointer");
  return hip_status(gs_launch_loss_grad(kind, count, image, target, dL_dimage, loss,
                                        (hipStream_t)stream),
                    "gs_image_loss_grad");
}

size_t gs_densify_prune_workspace_size(int64_t N, float clone_fraction) {
  if (N < 0 || !(clone_fraction >= 0.0f && clone_fraction <= 1.0f)) return 0;
  return gs_densify_workspace_bytes(N, clone_fraction);
}

gs_status gs_densify_prune(int64_t N, int64_t ld, int32_t sh_degree, const float* means,
                           const float* scales, const float* quats, const float* opacities,
                           const float* sh, const float* dL_dmeans, float clone_fraction,
                           float min_opacity, int64_t ld_out, float* means_out,
                           float* scales_out, float* quats_out, float* opacities_out,
                           float* sh_out, int64_t* num_out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  GS_CHECK(check_sizes(N, ld));
  GS_REQUIRE(sh_degree >= 0 && sh_degree <= 3, "sh_degree must be in [0, 3]");
  GS_REQUIRE(clone_fraction >= 0.0f && clone_fraction <= 1.0f,
             "clone_fraction must be in [0, 1]");
  GS_REQUIRE(min_opacity == min_opacity, "min_opacity is NaN");
  GS_REQUIRE(num_out != nullptr, "num_out is NULL");
  const int64_t n_clone = gs_densify_clone_count(N, clone_fraction);
  GS_REQUIRE(N + n_clone < ((int64_t)1 << 30), "N plus clones must be < 2^30");
  GS_REQUIRE(ld_out >= N + n_clone, "ld_out must hold N plus the clones");
  if (N > 0) {
    GS_REQUIRE(means && scales && quats && opacities && sh && dL_dmeans && means_out &&
                   scales_out && quats_out && opacities_out && sh_out,
               "NULL array pointer");
    GS_REQUIRE(workspace != nullptr, "workspace is NULL");
    GS_REQUIRE(((uintptr_t)workspace & 255u) == 0, "workspace must be 256-byte aligned");
    GS_REQUIRE(workspace_bytes >= gs_densify_workspace_bytes(N, clone_fraction),
               "workspace smaller than gs_densify_prune_workspace_size()");
  }
  const int K = (sh_degree + 1) * (sh_degree + 1);
  const float* in[64];
  float* out[64];
  int n = 0;
  auto add = [&](const float* a, float* b, int planes) {
    for (int k = 0; k < planes; ++k, ++n) {
      in[n] = a ? a + (int64_t)k * ld : nullptr;
      out[n] = b ? b + (int64_t)k * ld_out : nullptr;
    }
  };
  add(means, means_out, 3);
  add(scales, scales_out, 3);
  add(quats, quats_out, 4);
  add(opacities, opacities_out, 1);
  add(sh, sh_out, 3 * K);
  return hip_status(gs_launch_densify(N, n, in, ld, dL_dmeans, opacities, clone_fraction,
                                      min_opacity, out, num_out, workspace,
                                      (hipStream_t)stream),
                    "gs_densify_prune");
}

}  // extern "C"
