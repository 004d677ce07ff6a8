// binsort.hip — stages 2-3: scan of tiles touched, key duplication, onesweep
// LSD radix sort of the (tile_id << 32 | depth bits, Gaussian id) pairs, and
// per-tile ranges.
//
// All of it is data movement, bound by HBM bandwidth (or by latency at small
// instance counts):
//   - the scan is reduce-then-scan over 2048-element blocks;
//   - duplication is balanced by output slot: a workgroup owns 256 Gaussians
//     and writes all of their instances with consecutive, coalesced stores,
//     so one Gaussian touching thousands of tiles does not serialise a lane;
//   - the sort is a onesweep LSD radix sort with 9-bit digits: one pass
//     computes every digit's global histogram, then each digit pass reads and
//     writes the keys once.  A workgroup takes its partition from an atomic
//     ticket (so it only ever waits on partitions already running), ranks
//     its 4096 keys stably with wave64 ballots into LDS histograms, publishes
//     per-digit counts and resolves its global offsets by decoupled
//     look-back, then scatters through LDS so that global writes come out
//     in digit runs.  Only the low 32 + ceil(log2 T) key bits are sorted.
#include "gs_common.h"

namespace gs {

// ---------------------------------------------------------------------------
// Fill
// ---------------------------------------------------------------------------
__global__ void fill_u32_kernel(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// Zero up to four u32 segments in one launch.
struct Segs {
  uint32_t* p[4];
  int64_t n[4];
};
__global__ void zero_segs_kernel(Segs sg) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int k = 0; k < 4; ++k)
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < sg.n[k]; i += stride)
      sg.p[k][i] = 0u;
}

static hipError_t fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Block-wide scans (256 threads = 4 wave64)
// ---------------------------------------------------------------------------
__device__ inline uint64_t wave_incl_scan_u64(uint64_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

// Exclusive scan of one value per thread of an NW-wave workgroup; returns
// the block total.
template <int NW = 4>
__device__ inline uint64_t block_excl_scan_u64(uint64_t x, uint64_t& excl) {
  __shared__ uint64_t s_w[NW];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t inc = wave_incl_scan_u64(x);
  if (lane == 63) s_w[w] = inc;
  __syncthreads();
  uint64_t off = 0, tot = 0;
  for (int k = 0; k < NW; ++k) {
    if (k < w) off += s_w[k];
    tot += s_w[k];
  }
  excl = off + inc - x;
  __syncthreads();
  return tot;
}

// ---------------------------------------------------------------------------
// Stage 2: exclusive scan of tiles_touched -> offsets, total M.  The packed
// form (kVis) carries a second running sum in the same pass, the count of
// Gaussians with tiles_touched > 0, and writes their indices in ascending
// order to vis_ids; its per-block sums follow the first set at sums + nb.
// ---------------------------------------------------------------------------
constexpr int kScanItems = 8;
constexpr int kScanBlock = 256 * kScanItems;

template <bool kVis>
__global__ __launch_bounds__(256) void scan_reduce_kernel(const uint32_t* __restrict__ in,
                                                          int64_t N,
                                                          uint64_t* __restrict__ block_sums) {
  const int64_t base = (int64_t)blockIdx.x * kScanBlock;
  uint64_t s = 0, c = 0;
  for (int k = 0; k < kScanItems; ++k) {
    const int64_t i = base + (int64_t)k * 256 + threadIdx.x;
    if (i < N) {
      const uint32_t x = in[i];
      s += x;
      c += x > 0u ? 1u : 0u;
    }
  }
  uint64_t excl;
  const uint64_t tot = block_excl_scan_u64(s, excl);
  if (threadIdx.x == 0) block_sums[blockIdx.x] = tot;
  if (kVis) {
    const uint64_t ctot = block_excl_scan_u64(c, excl);
    if (threadIdx.x == 0) block_sums[gridDim.x + blockIdx.x] = ctot;
  }
}

// One workgroup per set of nb block sums (blockIdx.x selects the set):
// exclusive scan in place, the set's total to total[blockIdx.x].
__global__ __launch_bounds__(256) void scan_partials_kernel(uint64_t* __restrict__ sums,
                                                            int64_t nb,
                                                            uint64_t* __restrict__ total) {
  sums += (int64_t)blockIdx.x * nb;
  uint64_t carry = 0;
  for (int64_t b = 0; b < nb; b += 256) {
    const int64_t i = b + threadIdx.x;
    const uint64_t x = i < nb ? sums[i] : 0;
    uint64_t excl;
    const uint64_t tot = block_excl_scan_u64(x, excl);
    if (i < nb) sums[i] = carry + excl;
    carry += tot;
  }
  if (threadIdx.x == 0) total[blockIdx.x] = carry;
}

template <bool kVis>
__global__ __launch_bounds__(256) void scan_down_kernel(const uint32_t* __restrict__ in, int64_t N,
                                                        const uint64_t* __restrict__ sums,
                                                        uint32_t* __restrict__ out,
                                                        uint32_t* __restrict__ vis_ids) {
  const int64_t base = (int64_t)blockIdx.x * kScanBlock + (int64_t)threadIdx.x * kScanItems;
  uint32_t v[kScanItems];
  uint64_t s = 0, c = 0;
  for (int k = 0; k < kScanItems; ++k) {
    const int64_t i = base + k;
    v[k] = i < N ? in[i] : 0u;
    s += v[k];
    c += v[k] > 0u ? 1u : 0u;
  }
  uint64_t excl;
  block_excl_scan_u64(s, excl);
  uint64_t run = sums[blockIdx.x] + excl;
  for (int k = 0; k < kScanItems; ++k) {
    const int64_t i = base + k;
    if (i < N) out[i] = (uint32_t)run;
    run += v[k];
  }
  if (kVis) {
    block_excl_scan_u64(c, excl);
    uint64_t vrun = sums[gridDim.x + blockIdx.x] + excl;
    for (int k = 0; k < kScanItems; ++k)
      if (v[k] > 0u) vis_ids[vrun++] = (uint32_t)(base + k);
  }
}

// ---------------------------------------------------------------------------
// Stage 3a: duplicate each visible Gaussian once per touched tile
// ---------------------------------------------------------------------------
// A batch of cameras is one list of C * ld rows: row c * ld + i is Gaussian
// i seen by camera c, whose means2d are [c][2][ld] and whose tiles are
// numbered from c * T (batched = true).
__global__ __launch_bounds__(256) void duplicate_kernel(
    int64_t N, const float* __restrict__ means2d, int64_t ld, const int32_t* __restrict__ radii,
    const float* __restrict__ depths, const uint32_t* __restrict__ tiles_touched,
    const uint32_t* __restrict__ offsets, int gx, int gy, bool batched,
    const uint32_t* __restrict__ meff, uint64_t* __restrict__ keys, uint32_t* __restrict__ ids) {
  if (*meff == 0u) return;  // no instances, or more than the buffers hold
  __shared__ uint32_t s_off[257];
  __shared__ int32_t s_x0[256], s_w[256], s_y0[256];
  __shared__ uint32_t s_db[256], s_tb[256];
  const int t = threadIdx.x;
  const int64_t g0 = (int64_t)blockIdx.x * 256;
  const int64_t i = g0 + t;
  const int64_t nloc = (N - g0) < 256 ? (N - g0) : 256;
  if (i < N) {
    const uint32_t off = offsets[i];
    const uint32_t cnt = tiles_touched[i];
    s_off[t] = off;
    int x0 = 0, x1 = 0, y0 = 0, y1 = 0;
    const int64_t c = batched ? i / ld : 0;
    if (cnt > 0)
      tile_rect(means2d[i + c * ld], means2d[i + c * ld + ld], radii[i], gx, gy, x0, x1, y0, y1);
    s_x0[t] = x0;
    s_w[t] = (x1 > x0) ? (x1 - x0) : 1;
    s_y0[t] = y0;
    s_db[t] = __float_as_uint(depths[i]);
    s_tb[t] = (uint32_t)c * (uint32_t)gx * (uint32_t)gy;
    if (i == N - 1 || t == 255) s_off[t + 1] = off + cnt;
  }
  __syncthreads();
  const uint32_t begin = s_off[0], end = s_off[nloc];
  for (uint32_t slot = begin + t; slot < end; slot += 256) {
    // last j with s_off[j] <= slot (zero-count Gaussians share offsets)
    int lo = 0, hi = (int)nloc;  // invariant: s_off[lo] <= slot < s_off[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_off[mid] <= slot) lo = mid; else hi = mid;
    }
    const uint32_t k = slot - s_off[lo];
    const uint32_t w = (uint32_t)s_w[lo];
    const uint32_t ty = (uint32_t)s_y0[lo] + k / w;
    const uint32_t tx = (uint32_t)s_x0[lo] + k % w;
    const uint32_t tile = s_tb[lo] + ty * (uint32_t)gx + tx;
    keys[slot] = ((uint64_t)tile << 32) | (uint64_t)s_db[lo];
    ids[slot] = (uint32_t)(g0 + lo);
  }
}

// ---------------------------------------------------------------------------
// Stage 3b: onesweep radix sort
// ---------------------------------------------------------------------------
constexpr int kRadixBits = 9;  // 45 key bits at 1080p: 5 passes
constexpr int kRadix = 1 << kRadixBits;
constexpr int kSortItems = 8;
// 512-lane workgroups (a lane per digit) of 4096 keys: ~66 KB of LDS, so a
// partition finds room on a CU beside other kernels' workgroups
constexpr int kSortWaves = 8;
constexpr int kSortThreads = 64 * kSortWaves;
constexpr int kPart = kSortThreads * kSortItems;  // keys per partition
static_assert(kRadix <= kSortThreads, "a sort lane per digit");
static_assert(kRadix % 64 == 0, "digits in whole wavefronts");
constexpr int kMaxPasses = 8;
constexpr uint32_t kFlagAgg = 1u << 30;
constexpr uint32_t kFlagPrefix = 2u << 30;
constexpr uint32_t kCountMask = (1u << 30) - 1u;
constexpr int kLookback = 8;  // partitions examined per look-back step

// Global histogram of every pass's digit (one LDS histogram per pass).
__global__ __launch_bounds__(256) void sort_histogram_kernel(const uint64_t* __restrict__ keys,
                                                             const uint32_t* __restrict__ meff,
                                                             int passes,
                                                             uint32_t* __restrict__ hist) {
  const uint32_t M = *meff;
  __shared__ uint32_t s_h[kMaxPasses][kRadix];
  for (int k = threadIdx.x; k < kMaxPasses * kRadix; k += 256) (&s_h[0][0])[k] = 0;
  __syncthreads();
  for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < M; i += gridDim.x * 256u) {
    const uint64_t key = keys[i];
    for (int p = 0; p < passes; ++p)
      atomicAdd(&s_h[p][(key >> (p * kRadixBits)) & (kRadix - 1)], 1u);
  }
  __syncthreads();
  for (int k = threadIdx.x; k < passes * kRadix; k += 256) {
    const uint32_t v = (&s_h[0][0])[k];
    if (v) atomicAdd(&hist[k], v);
  }
}

// hist[p][d] -> exclusive offsets, one workgroup per pass, a lane per digit.
__global__ __launch_bounds__(kRadix) void sort_hist_scan_kernel(uint32_t* __restrict__ hist) {
  uint32_t* h = hist + blockIdx.x * kRadix;
  const uint64_t x = h[threadIdx.x];
  uint64_t excl;
  block_excl_scan_u64<kRadix / 64>(x, excl);
  h[threadIdx.x] = (uint32_t)excl;
}

__device__ inline uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

__global__ __launch_bounds__(kSortThreads) void sort_pass_kernel(
    const uint64_t* __restrict__ kin, const uint32_t* __restrict__ vin,
    uint64_t* __restrict__ kout, uint32_t* __restrict__ vout, const uint32_t* __restrict__ meff,
    int shift, const uint32_t* __restrict__ digit_offsets, uint32_t* __restrict__ status,
    uint32_t* __restrict__ ticket) {
  const uint32_t M = *meff;
  __shared__ uint64_t s_keys[kPart];
  __shared__ uint32_t s_vals[kPart];
  __shared__ uint32_t s_wh[kSortWaves][kRadix];  // per-wave digit counts, later wave offsets
  __shared__ uint32_t s_start[kRadix];  // block-local exclusive digit start
  __shared__ uint32_t s_gbase[kRadix];  // global base minus local start
  __shared__ uint32_t s_part;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) s_part = atomicAdd(ticket, 1u);
  for (int k = tid; k < kSortWaves * kRadix; k += kSortThreads) (&s_wh[0][0])[k] = 0;
  __syncthreads();
  const uint32_t part = s_part;
  // a grid sized for the buffers' capacity: workgroups past the last
  // partition leave (nothing waits on a later partition)
  if ((uint64_t)part * (uint64_t)kPart >= (uint64_t)M) return;
  const uint32_t base = part * (uint32_t)kPart;
  const uint32_t nvalid = (M - base) < (uint32_t)kPart ? (M - base) : (uint32_t)kPart;

  uint64_t k[kSortItems];
  uint32_t v[kSortItems];
  uint32_t rank[kSortItems];
  const uint32_t wbase = base + (uint32_t)wave * 64u * kSortItems;
#pragma unroll
  for (int it = 0; it < kSortItems; ++it) {
    const uint32_t idx = wbase + (uint32_t)it * 64u + (uint32_t)lane;
    const bool valid = idx < M;
    k[it] = valid ? kin[idx] : ~0ull;  // padding ranks last in digit 255
    v[it] = valid ? vin[idx] : 0u;
  }
  const uint64_t lt = lanemask_lt();
#pragma unroll
  for (int it = 0; it < kSortItems; ++it) {
    const uint32_t d = (uint32_t)(k[it] >> shift) & (kRadix - 1);
    uint64_t match = ~0ull;
#pragma unroll
    for (int b = 0; b < kRadixBits; ++b) {
      const uint64_t bal = __ballot((d >> b) & 1u);
      match &= ((d >> b) & 1u) ? bal : ~bal;
    }
    const uint32_t before = s_wh[wave][d];
    rank[it] = before + (uint32_t)__popcll(match & lt);
    const int leader = __ffsll((long long)match) - 1;
    __builtin_amdgcn_wave_barrier();
    if (lane == leader) s_wh[wave][d] = before + (uint32_t)__popcll(match);
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();

  // per digit (thread = digit, the first 256 lanes): wave offsets, block
  // count, block-local start
  const bool dl = tid < kRadix;
  const uint32_t d = dl ? (uint32_t)tid : 0u;
  uint32_t cnt = 0;
  if (dl) {
    for (int w = 0; w < kSortWaves; ++w) {
      const uint32_t c = s_wh[w][d];
      s_wh[w][d] = cnt;
      cnt += c;
    }
  }
  uint64_t excl64;
  block_excl_scan_u64<kSortWaves>(cnt, excl64);
  if (dl) s_start[d] = (uint32_t)excl64;
  const uint32_t pad = (uint32_t)kPart - nvalid;  // padding keys sit in digit 255
  const uint32_t mine = (d == kRadix - 1) ? cnt - pad : cnt;

  // decoupled look-back over earlier partitions, one lane per digit
  uint32_t* st = status + (size_t)part * kRadix;
  uint32_t prefix = 0;
  if (!dl) {
    // lanes past the digits take no part
  } else if (part == 0) {
    __hip_atomic_store(&st[d], kFlagPrefix | mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    __hip_atomic_store(&st[d], kFlagAgg | mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // look back kLookback partitions per step (all loads in flight at once):
    // add aggregates up to the nearest inclusive prefix; resume at the first
    // partition that has published nothing yet.  Partition 0 always
    // publishes a prefix, so the walk ends there at the latest.
    int64_t p = (int64_t)part - 1;
    while (p >= 0) {
      uint32_t sv[kLookback];
#pragma unroll
      for (int j = 0; j < kLookback; ++j)
        sv[j] = (p - j >= 0) ? __hip_atomic_load(&status[(size_t)(p - j) * kRadix + d],
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                             : kFlagPrefix;
      int j = 0;
      bool done = false;
      for (; j < kLookback; ++j) {
        const uint32_t flag = sv[j] & ~kCountMask;
        if (flag == 0u) break;
        prefix += sv[j] & kCountMask;
        if (flag == kFlagPrefix) {
          done = true;
          break;
        }
      }
      if (done) break;
      p -= j;
      if (j < kLookback) __builtin_amdgcn_s_sleep(1);
    }
    __hip_atomic_store(&st[d], kFlagPrefix | (prefix + mine), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  if (dl) s_gbase[d] = digit_offsets[d] + prefix - s_start[d];
  __syncthreads();

  // scatter into LDS in local sorted order
#pragma unroll
  for (int it = 0; it < kSortItems; ++it) {
    const uint32_t idx = wbase + (uint32_t)it * 64u + (uint32_t)lane;
    if (idx < M) {
      const uint32_t dd = (uint32_t)(k[it] >> shift) & (kRadix - 1);
      const uint32_t pos = s_start[dd] + s_wh[wave][dd] + rank[it];
      s_keys[pos] = k[it];
      s_vals[pos] = v[it];
    }
  }
  __syncthreads();
  // write out in local order: consecutive lanes hit consecutive slots of a digit run
  for (uint32_t j = (uint32_t)tid; j < nvalid; j += (uint32_t)kSortThreads) {
    const uint64_t key = s_keys[j];
    const uint32_t dd = (uint32_t)(key >> shift) & (kRadix - 1);
    const uint32_t out = s_gbase[dd] + j;
    kout[out] = key;
    vout[out] = s_vals[j];
  }
}

// ---------------------------------------------------------------------------
// Stage 3c: per-tile [start, end) ranges of the sorted keys
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void ranges_kernel(const uint64_t* __restrict__ keys,
                                                     const uint32_t* __restrict__ meff, uint32_t T,
                                                     uint32_t* __restrict__ ranges) {
  const uint32_t M = *meff;
  const uint32_t m = blockIdx.x * 256u + threadIdx.x;
  if (m >= M) return;
  const uint32_t tile = (uint32_t)(keys[m] >> 32);
  if (tile >= T) return;
  if (m == 0 || (uint32_t)(keys[m - 1] >> 32) != tile) ranges[2 * tile] = m;
  if (m == M - 1 || (uint32_t)(keys[m + 1] >> 32) != tile) ranges[2 * tile + 1] = m + 1;
}

// The instance count the binning kernels use: M when it fits the buffers,
// else 0 (an empty list).  counts (device, optional) receives M and the
// overflow flag.
__global__ void bin_count_kernel(const uint64_t* __restrict__ total, uint64_t capacity,
                                 uint32_t* __restrict__ meff, uint64_t* __restrict__ counts) {
  const uint64_t M = *total;
  const bool over = M > capacity;
  *meff = over ? 0u : (uint32_t)M;
  if (counts) {
    counts[0] = M;
    counts[1] = over ? 1ull : 0ull;
  }
}

// ---------------------------------------------------------------------------
// Workspace layout
// ---------------------------------------------------------------------------
struct SortPlan {
  int passes;
  uint32_t parts;
};

static inline int ceil_log2(uint32_t x) {
  int b = 0;
  while ((1ull << b) < x) ++b;
  return b;
}

static inline SortPlan sort_plan(uint64_t M, int32_t T) {
  const int bits = 32 + ceil_log2((uint32_t)T);
  SortPlan p;
  p.passes = (bits + kRadixBits - 1) / kRadixBits;
  p.parts = (uint32_t)((M + kPart - 1) / kPart);
  return p;
}

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Workspace {
  uint64_t* keys_alt;
  uint32_t* ids_alt;
  uint64_t* scan_sums;
  uint64_t* total;
  uint32_t* meff;    // [1] instance count used by the binning kernels
  uint32_t* hist;    // [passes][256]
  uint32_t* ticket;  // [passes]
  uint32_t* status;  // [passes][parts][256]
  size_t bytes;
};

static Workspace carve(void* base, int64_t N, uint64_t capacity, int32_t T) {
  const SortPlan sp = sort_plan(capacity, T);
  const int64_t nb = (N + kScanBlock - 1) / kScanBlock;
  Workspace w;
  char* p = (char*)base;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* r = p ? p + off : nullptr;
    off += align256(bytes);
    return r;
  };
  w.keys_alt = (uint64_t*)take(sizeof(uint64_t) * (capacity ? capacity : 1));
  w.ids_alt = (uint32_t*)take(sizeof(uint32_t) * (capacity ? capacity : 1));
  w.scan_sums = (uint64_t*)take(sizeof(uint64_t) * 2 * (nb ? nb : 1));
  w.total = (uint64_t*)take(sizeof(uint64_t) * 2);
  w.meff = (uint32_t*)take(sizeof(uint32_t));
  w.hist = (uint32_t*)take(sizeof(uint32_t) * kMaxPasses * kRadix);
  w.ticket = (uint32_t*)take(sizeof(uint32_t) * kMaxPasses);
  w.status = (uint32_t*)take(sizeof(uint32_t) * (size_t)sp.passes * (sp.parts ? sp.parts : 1) * kRadix);
  w.bytes = off;
  return w;
}

}  // namespace gs

extern "C" size_t gs_binsort_workspace_bytes(int64_t N, uint64_t capacity, int32_t T) {
  return gs::carve(nullptr, N, capacity, T).bytes;
}

// Scan; writes offsets and M to totals_host[0] (one synchronising read).
// With vis_ids non-NULL also the ascending indices of the Gaussians with
// tiles, and their count V to totals_host[1], in the same read.
extern "C" hipError_t gs_launch_scan(int64_t N, const uint32_t* tiles, uint32_t* offsets,
                                     uint32_t* vis_ids, void* workspace, uint64_t capacity,
                                     int32_t T, uint64_t* totals_host, hipStream_t s) {
  using namespace gs;
  Workspace w = carve(workspace, N, capacity, T);
  hipError_t e;
  const bool vis = vis_ids != nullptr;
  if (N == 0) {
    if (totals_host) {
      totals_host[0] = 0;
      if (vis) totals_host[1] = 0;
      return hipSuccess;
    }
    // the device count must still read 0
    hipLaunchKernelGGL(scan_partials_kernel, dim3(1), dim3(256), 0, s, w.scan_sums, (int64_t)0,
                       w.total);
    return hipGetLastError();
  }
  const int64_t nb = (N + kScanBlock - 1) / kScanBlock;
  if (vis)
    hipLaunchKernelGGL(scan_reduce_kernel<true>, dim3((unsigned)nb), dim3(256), 0, s, tiles, N,
                       w.scan_sums);
  else
    hipLaunchKernelGGL(scan_reduce_kernel<false>, dim3((unsigned)nb), dim3(256), 0, s, tiles, N,
                       w.scan_sums);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(scan_partials_kernel, dim3(vis ? 2 : 1), dim3(256), 0, s, w.scan_sums, nb,
                     w.total);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (vis)
    hipLaunchKernelGGL(scan_down_kernel<true>, dim3((unsigned)nb), dim3(256), 0, s, tiles, N,
                       w.scan_sums, offsets, vis_ids);
  else
    hipLaunchKernelGGL(scan_down_kernel<false>, dim3((unsigned)nb), dim3(256), 0, s, tiles, N,
                       w.scan_sums, offsets, nullptr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (!totals_host) return hipSuccess;  // the count stays on the device
  // straight into the caller's host words: page-locked memory there makes
  // this a direct transfer instead of a staged one
  if ((e = hipMemcpyAsync(totals_host, w.total, sizeof(uint64_t) * (vis ? 2 : 1),
                          hipMemcpyDeviceToHost, s)) != hipSuccess)
    return e;
  return hipStreamSynchronize(s);
}

// Duplicate, sort and extract ranges for M instances (M <= capacity).
// ncams > 1: a batch; N = ncams * ld rows, T = ncams tiles per camera.
// M: the instance count read back by the caller, or, with device_count,
// unknown on the host: the kernels then take it from the scan on the device,
// grids are sized for `capacity`, and counts (device, optional) receives M
// and an overflow flag (M > capacity leaves an empty list).
extern "C" hipError_t gs_launch_dup_sort_ranges(int64_t N, int64_t ld, const float* means2d,
                                                const int32_t* radii, const float* depths,
                                                const uint32_t* tiles, const uint32_t* offsets,
                                                int32_t W, int32_t H, int ncams, uint64_t M,
                                                bool device_count, uint64_t* counts,
                                                uint64_t* keys, uint32_t* ids, uint32_t* ranges,
                                                void* workspace, uint64_t capacity, hipStream_t s) {
  using namespace gs;
  const int gx = grid_dim(W), gy = grid_dim(H);
  const int32_t T = gx * gy * ncams;
  Workspace w = carve(workspace, N, capacity, T);
  hipError_t e;
  if (!device_count && M == 0) return fill_u32(ranges, 2 * (int64_t)T, 0u, s);
  // grids for M, or for the largest count the buffers hold
  const uint64_t Mg = device_count ? capacity : M;
  const SortPlan sp = sort_plan(Mg, T);
  {
    Segs sg = {{ranges, w.hist, w.ticket, w.status},
               {2 * (int64_t)T, (int64_t)kMaxPasses * kRadix, kMaxPasses,
                (int64_t)sp.passes * sp.parts * kRadix}};
    int64_t big = sg.n[0] > sg.n[3] ? sg.n[0] : sg.n[3];
    int64_t blocks = (big + 255) / 256;
    if (blocks > 2048) blocks = 2048;
    hipLaunchKernelGGL(zero_segs_kernel, dim3((unsigned)blocks), dim3(256), 0, s, sg);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(bin_count_kernel, dim3(1), dim3(1), 0, s, w.total, capacity, w.meff,
                     device_count ? counts : nullptr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (Mg == 0) return hipSuccess;
  // land the final pass in (keys, ids): start from the alternate buffer when
  // the pass count is odd
  uint64_t* ka = (sp.passes & 1) ? w.keys_alt : keys;
  uint32_t* ia = (sp.passes & 1) ? w.ids_alt : ids;
  uint64_t* kb = (sp.passes & 1) ? keys : w.keys_alt;
  uint32_t* ib = (sp.passes & 1) ? ids : w.ids_alt;
  const int64_t nblk = (N + 255) / 256;
  hipLaunchKernelGGL(duplicate_kernel, dim3((unsigned)nblk), dim3(256), 0, s, N, means2d, ld, radii,
                     depths, tiles, offsets, gx, gy, ncams > 1, w.meff, ka, ia);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  unsigned hblocks = (unsigned)((Mg + 256 * 16 - 1) / (256 * 16));
  if (hblocks > 1024) hblocks = 1024;
  hipLaunchKernelGGL(sort_histogram_kernel, dim3(hblocks), dim3(256), 0, s, ka, w.meff, sp.passes,
                     w.hist);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(sort_hist_scan_kernel, dim3(sp.passes), dim3(kRadix), 0, s, w.hist);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  for (int p = 0; p < sp.passes; ++p) {
    hipLaunchKernelGGL(sort_pass_kernel, dim3(sp.parts), dim3(kSortThreads), 0, s, ka, ia, kb, ib,
                       w.meff, p * kRadixBits, w.hist + p * kRadix,
                       w.status + (size_t)p * sp.parts * kRadix, w.ticket + p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    uint64_t* tk = ka; ka = kb; kb = tk;
    uint32_t* ti = ia; ia = ib; ib = ti;
  }
  const unsigned rblocks = (unsigned)((Mg + 255) / 256);
  hipLaunchKernelGGL(ranges_kernel, dim3(rblocks), dim3(256), 0, s, keys, w.meff, (uint32_t)T,
                     ranges);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Internal helpers for other stages (hidden, not part of the C ABI): a stable
// sort of (key, value) pairs by the low `bits` bits of the keys, and an
// exclusive scan of u32 values whose total stays on the device.
// ---------------------------------------------------------------------------
namespace gs {
struct PairSortWs {
  uint64_t* keys_alt;
  uint32_t* vals_alt;
  uint32_t* meff;
  uint32_t* hist;
  uint32_t* ticket;
  uint32_t* status;
  int passes;
  uint32_t parts;
  size_t bytes;
};

static PairSortWs carve_pairsort(void* base, uint64_t n, int bits) {
  PairSortWs w;
  w.passes = (bits + kRadixBits - 1) / kRadixBits;
  w.parts = (uint32_t)((n + kPart - 1) / kPart);
  char* p = (char*)base;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* r = p ? p + off : nullptr;
    off += align256(bytes);
    return r;
  };
  w.keys_alt = (uint64_t*)take(sizeof(uint64_t) * (n ? n : 1));
  w.vals_alt = (uint32_t*)take(sizeof(uint32_t) * (n ? n : 1));
  w.meff = (uint32_t*)take(sizeof(uint32_t));
  w.hist = (uint32_t*)take(sizeof(uint32_t) * kMaxPasses * kRadix);
  w.ticket = (uint32_t*)take(sizeof(uint32_t) * kMaxPasses);
  w.status = (uint32_t*)take(sizeof(uint32_t) * (size_t)w.passes * (w.parts ? w.parts : 1) * kRadix);
  w.bytes = off;
  return w;
}
}  // namespace gs

extern "C" size_t gs_pairsort_workspace_bytes(uint64_t n, int bits) {
  return gs::carve_pairsort(nullptr, n, bits).bytes;
}

// Sorts (keys, vals)[0, n) stably by the low `bits` bits of the keys; the
// result lands back in keys / vals.  n < 2^30, bits in [1, 64].
extern "C" hipError_t gs_pairsort(uint64_t* keys, uint32_t* vals, uint64_t n, int bits,
                                  void* workspace, hipStream_t s) {
  using namespace gs;
  if (n == 0) return hipSuccess;
  PairSortWs w = carve_pairsort(workspace, n, bits);
  hipError_t e;
  {
    Segs sg = {{w.hist, w.ticket, w.status, w.status},
               {(int64_t)kMaxPasses * kRadix, kMaxPasses,
                (int64_t)w.passes * w.parts * kRadix, 0}};
    int64_t blocks = (sg.n[2] + 255) / 256;
    if (blocks > 2048) blocks = 2048;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(zero_segs_kernel, dim3((unsigned)blocks), dim3(256), 0, s, sg);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // an odd pass count starts from a copy in the alternate buffers so that
  // the last pass writes keys / vals
  uint64_t* ka = keys;
  uint32_t* ia = vals;
  uint64_t* kb = w.keys_alt;
  uint32_t* ib = w.vals_alt;
  if (w.passes & 1) {
    if ((e = hipMemcpyAsync(w.keys_alt, keys, n * sizeof(uint64_t), hipMemcpyDeviceToDevice, s)) !=
        hipSuccess)
      return e;
    if ((e = hipMemcpyAsync(w.vals_alt, vals, n * sizeof(uint32_t), hipMemcpyDeviceToDevice, s)) !=
        hipSuccess)
      return e;
    ka = w.keys_alt; ia = w.vals_alt; kb = keys; ib = vals;
  }
  if ((e = fill_u32(w.meff, 1, (uint32_t)n, s)) != hipSuccess) return e;
  unsigned hblocks = (unsigned)((n + 256 * 16 - 1) / (256 * 16));
  if (hblocks > 1024) hblocks = 1024;
  hipLaunchKernelGGL(sort_histogram_kernel, dim3(hblocks), dim3(256), 0, s, ka, w.meff, w.passes,
                     w.hist);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(sort_hist_scan_kernel, dim3(w.passes), dim3(kRadix), 0, s, w.hist);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  for (int p = 0; p < w.passes; ++p) {
    hipLaunchKernelGGL(sort_pass_kernel, dim3(w.parts), dim3(kSortThreads), 0, s, ka, ia, kb, ib,
                       w.meff, p * kRadixBits, w.hist + p * kRadix,
                       w.status + (size_t)p * w.parts * kRadix, w.ticket + p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    uint64_t* tk = ka; ka = kb; kb = tk;
    uint32_t* ti = ia; ia = ib; ib = ti;
  }
  return hipSuccess;
}

extern "C" size_t gs_scan_workspace_bytes(int64_t n) {
  const int64_t nb = (n + gs::kScanBlock - 1) / gs::kScanBlock;
  return gs::align256(sizeof(uint64_t) * (size_t)(nb ? nb : 1));
}

// out[i] = in[0] + ... + in[i-1]; *total (device) = the whole sum.
extern "C" hipError_t gs_scan_u32(const uint32_t* in, int64_t n, uint32_t* out, uint64_t* total,
                                  void* workspace, hipStream_t s) {
  using namespace gs;
  hipError_t e;
  if (n == 0) {
    hipLaunchKernelGGL(scan_partials_kernel, dim3(1), dim3(256), 0, s, (uint64_t*)workspace,
                       (int64_t)0, total);
    return hipGetLastError();
  }
  uint64_t* sums = (uint64_t*)workspace;
  const int64_t nb = (n + kScanBlock - 1) / kScanBlock;
  hipLaunchKernelGGL(scan_reduce_kernel<false>, dim3((unsigned)nb), dim3(256), 0, s, in, n, sums);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(scan_partials_kernel, dim3(1), dim3(256), 0, s, sums, nb, total);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(scan_down_kernel<false>, dim3((unsigned)nb), dim3(256), 0, s, in, n, sums,
                     out, nullptr);
  return hipGetLastError();
}
