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
//   - the sort is a onesweep LSD radix sort with 10-bit digits: one kernel
//     histograms the first digit, and each digit pass, which reads and
//     writes the keys once, also totals the next digit.  A workgroup takes
//     its partition from an atomic ticket (so it only ever waits on
//     partitions already running), ranks its 7168 keys stably with wave64
//     ballots into LDS histograms, publishes per-digit counts and resolves
//     its global offsets by a two-level look-back (within a group of 16
//     partitions, then over groups), then scatters through LDS so that
//     global writes come out in digit runs.
//     Only the bits that vary within the frame are sorted: the scan also
//     finds the smallest and largest depth bits of the rows with tiles, and
//     the passes sort (tile, depth bits - smallest) in ceil(log2 T) +
//     bits(largest - smallest) bits; with the depths of a typical frame
//     spanning ~2^26 fp32 codes that is four passes at 1080p.  Where that
//     key, the row index and every pass's digit fit one 64-bit word, the
//     keys travel as such words and the last pass writes keys and ids.
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
// sort shapes the duplication needs (see the sort below)
constexpr int kDigitBits = 10;         // bits of a sort pass's digit
constexpr int kDigits = 1 << kDigitBits;  // radix of a sort pass
constexpr int kPartKeys = 7168;        // keys per sort partition
constexpr int kGroupPartitions = 16;   // partitions per look-back group
constexpr int kDbitsShift = 58;
constexpr uint64_t kCountBits = (1ull << kDbitsShift) - 1ull;
constexpr int kScanBlock = 256 * kScanItems;

// Passes of a sort over `bits` key bits (at least one).
__host__ __device__ inline int sort_pass_count(int bits) {
  return bits > 0 ? (bits + kDigitBits - 1) / kDigitBits : 1;
}

// How the sort runs, decided from the key map on the device (the duplication
// and the first digit's histogram run before the host has read the count
// back) and again on the host from the read-back depth bits, with the same
// result: the pass count for the key's bits, and whether the keys travel as
// key-id words (see pass_digit).  pass_dbits >= 0 plans for that many depth
// bits instead of the map's; idbits < 0 never uses words.
struct SortMode {
  int passes;
  bool words;
};
__host__ __device__ inline SortMode sort_mode(int dbits, int tbits, int idbits) {
  SortMode m;
  m.passes = sort_pass_count(dbits + tbits);
  m.words = idbits >= 0 && idbits + kDigitBits * m.passes <= 64;
  return m;
}

// Smallest and largest u32 over a 256-lane workgroup (valid in every lane).
__device__ inline void block_minmax_u32(uint32_t& lo, uint32_t& hi) {
  __shared__ uint32_t s_lo[4], s_hi[4];
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, o, 64));
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, o, 64));
  }
  if ((threadIdx.x & 63) == 0) {
    s_lo[threadIdx.x >> 6] = lo;
    s_hi[threadIdx.x >> 6] = hi;
  }
  __syncthreads();
  lo = min(min(s_lo[0], s_lo[1]), min(s_lo[2], s_lo[3]));
  hi = max(max(s_hi[0], s_hi[1]), max(s_hi[2], s_hi[3]));
  __syncthreads();
}

// Per block: the sum of tiles (and with kVis the count of rows with tiles),
// and, with depths and minmax, the smallest and largest depth bits of the
// rows with tiles (their keys' low words) at minmax[2 * block].
template <bool kVis>
__global__ __launch_bounds__(256) void scan_reduce_kernel(const uint32_t* __restrict__ in,
                                                          const float* __restrict__ depths,
                                                          int64_t N,
                                                          uint64_t* __restrict__ block_sums,
                                                          uint32_t* __restrict__ minmax) {
  const int64_t base = (int64_t)blockIdx.x * kScanBlock;
  uint64_t s = 0, c = 0;
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  for (int k = 0; k < kScanItems; ++k) {
    const int64_t i = base + (int64_t)k * 256 + threadIdx.x;
    if (i < N) {
      const uint32_t x = in[i];
      s += x;
      c += x > 0u ? 1u : 0u;
      if (x > 0u && depths) {
        const uint32_t db = __float_as_uint(depths[i]);
        lo = min(lo, db);
        hi = max(hi, db);
      }
    }
  }
  uint64_t excl;
  const uint64_t tot = block_excl_scan_u64(s, excl);
  if (threadIdx.x == 0) block_sums[blockIdx.x] = tot;
  if (kVis) {
    const uint64_t ctot = block_excl_scan_u64(c, excl);
    if (threadIdx.x == 0) block_sums[gridDim.x + blockIdx.x] = ctot;
  }
  if (!minmax) return;
  block_minmax_u32(lo, hi);
  if (threadIdx.x == 0) {
    minmax[2 * blockIdx.x] = lo;
    minmax[2 * blockIdx.x + 1] = hi;
  }
}

// One workgroup per set of nb block sums (blockIdx.x selects the set):
// exclusive scan in place, the set's total to total[blockIdx.x].  With
// minmax, the first also folds the blocks' depth-bit ranges into the sort's
// key map (keymap[0] = smallest depth bits, keymap[1] = bits the range
// needs) and puts that bit count above the total, in total[0] bits 58-63,
// so that the host reads it with M.  (M < 2^54: fewer than 2^31 rows, each
// touching fewer than 2^23 tiles.)
//
// With meff, the first also writes the instance count the binning kernels
// use: M when it fits `capacity`, else 0 (an empty list); counts (optional)
// receives M and the overflow flag.
__global__ __launch_bounds__(256) void scan_partials_kernel(uint64_t* __restrict__ sums,
                                                            int64_t nb,
                                                            const uint32_t* __restrict__ minmax,
                                                            uint64_t* __restrict__ total,
                                                            uint32_t* __restrict__ keymap,
                                                            uint64_t capacity,
                                                            uint32_t* __restrict__ meff,
                                                            uint64_t* __restrict__ counts) {
  sums += (int64_t)blockIdx.x * nb;
  uint64_t carry = 0;
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  for (int64_t b = 0; b < nb; b += 256) {
    const int64_t i = b + threadIdx.x;
    const uint64_t x = i < nb ? sums[i] : 0;
    if (i < nb && blockIdx.x == 0 && minmax) {
      lo = min(lo, minmax[2 * i]);
      hi = max(hi, minmax[2 * i + 1]);
    }
    uint64_t excl;
    const uint64_t tot = block_excl_scan_u64(x, excl);
    if (i < nb) sums[i] = carry + excl;
    carry += tot;
  }
  if (blockIdx.x == 0 && minmax) block_minmax_u32(lo, hi);
  if (threadIdx.x == 0) {
    uint64_t word = carry;
    if (blockIdx.x == 0 && minmax) {
      const uint32_t span = lo <= hi ? hi - lo : 0u;
      const uint32_t dbits = span ? 32u - (uint32_t)__clz((int)span) : 0u;
      keymap[0] = lo <= hi ? lo : 0u;
      keymap[1] = dbits;
      word |= (uint64_t)dbits << kDbitsShift;
    }
    if (blockIdx.x == 0 && meff) {
      const bool over = carry > capacity;
      *meff = over ? 0u : (uint32_t)carry;
      if (counts) {
        counts[0] = carry;
        counts[1] = over ? 1ull : 0ull;
      }
    }
    total[blockIdx.x] = word;
  }
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

// The down-sweep of the binning's scan without a separate pass over the
// block sums: block b adds up the sums of the blocks before it itself (at
// most a few hundred values), and the last block also forms the totals, the
// key map and the instance count the binning kernels use (as
// scan_partials_kernel does).
template <bool kVis>
__global__ __launch_bounds__(256) void scan_down_bin_kernel(
    const uint32_t* __restrict__ in, int64_t N, const uint64_t* __restrict__ block_sums,
    const uint32_t* __restrict__ minmax, uint32_t* __restrict__ out,
    uint32_t* __restrict__ vis_ids, uint64_t* __restrict__ total, uint32_t* __restrict__ keymap,
    uint64_t capacity, uint32_t* __restrict__ meff, uint64_t* __restrict__ counts) {
  const int64_t nb = gridDim.x, b = blockIdx.x;
  uint64_t ps = 0, pc = 0;
  for (int64_t j = threadIdx.x; j < b; j += 256) {
    ps += block_sums[j];
    if (kVis) pc += block_sums[nb + j];
  }
  uint64_t excl;
  const uint64_t sbase = block_excl_scan_u64(ps, excl);
  const uint64_t cbase = kVis ? block_excl_scan_u64(pc, excl) : 0;

  const int64_t base = b * kScanBlock + (int64_t)threadIdx.x * kScanItems;
  uint32_t v[kScanItems];
  uint64_t s = 0, c = 0;
  for (int k = 0; k < kScanItems; ++k) {
    const int64_t i = base + k;
    v[k] = i < N ? in[i] : 0u;
    s += v[k];
    c += v[k] > 0u ? 1u : 0u;
  }
  const uint64_t stot = block_excl_scan_u64(s, excl);
  uint64_t run = sbase + excl;
  for (int k = 0; k < kScanItems; ++k) {
    const int64_t i = base + k;
    if (i < N) out[i] = (uint32_t)run;
    run += v[k];
  }
  uint64_t ctot = 0;
  if (kVis) {
    ctot = block_excl_scan_u64(c, excl);
    uint64_t vrun = cbase + excl;
    for (int k = 0; k < kScanItems; ++k)
      if (v[k] > 0u) vis_ids[vrun++] = (uint32_t)(base + k);
  }
  if (b != nb - 1) return;
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  for (int64_t j = threadIdx.x; j < nb; j += 256) {
    lo = min(lo, minmax[2 * j]);
    hi = max(hi, minmax[2 * j + 1]);
  }
  block_minmax_u32(lo, hi);
  if (threadIdx.x == 0) {
    const uint64_t M = sbase + stot;
    const uint32_t span = lo <= hi ? hi - lo : 0u;
    const uint32_t dbits = span ? 32u - (uint32_t)__clz((int)span) : 0u;
    keymap[0] = lo <= hi ? lo : 0u;
    keymap[1] = dbits;
    total[0] = M | ((uint64_t)dbits << kDbitsShift);
    if (kVis) total[1] = cbase + ctot;
    const bool over = M > capacity;
    *meff = over ? 0u : (uint32_t)M;
    if (counts) {
      counts[0] = M;
      counts[1] = over ? 1ull : 0ull;
    }
  }
}

// ---------------------------------------------------------------------------
// Stage 3a: duplicate each visible Gaussian once per touched tile
// ---------------------------------------------------------------------------
// A batch of cameras is one list of C * ld rows: row c * ld + i is Gaussian
// i seen by camera c, whose means2d are [c][2][ld] and whose tiles are
// numbered from c * T (batched = true).
// What the sort and the ranges need zeroed before they run: the ranges, the
// digit totals and the partition tickets, and for each of `passes` passes
// (laid out for `parts` partitions and `groups` groups) the statuses of the
// partitions and groups the instance count actually uses.
struct SortZero {
  uint32_t* ranges;
  int64_t nranges;
  uint32_t* small;
  int64_t nsmall;
  uint32_t* pstat;
  uint32_t* gstat;
  uint32_t parts, groups;
  int passes;
};
__device__ inline void zero_span(uint32_t* p, int64_t n, int64_t first, int64_t stride) {
  for (int64_t i = first; i < n; i += stride) p[i] = 0u;
}

// Every block first takes its share of the zeroing (the grid may be larger
// than the rows need), then duplicates its 256 rows.
__global__ __launch_bounds__(256) void duplicate_kernel(
    int64_t N, const float* __restrict__ means2d, int64_t ld, const int32_t* __restrict__ radii,
    const float* __restrict__ depths, const uint32_t* __restrict__ tiles_touched,
    const uint32_t* __restrict__ offsets, int gx, int gy, bool batched,
    const uint32_t* __restrict__ meff, SortZero z, const uint32_t* __restrict__ keymap,
    int tbits, int idbits, int pass_dbits, uint64_t* __restrict__ keys,
    uint32_t* __restrict__ ids, uint64_t* __restrict__ keys_alt,
    uint32_t* __restrict__ ids_alt) {
  const uint32_t Meff = *meff;
  {
    const int64_t first = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * 256;
    zero_span(z.ranges, z.nranges, first, stride);
    zero_span(z.small, z.nsmall, first, stride);
    const uint32_t parts = (uint32_t)(((uint64_t)Meff + kPartKeys - 1) / kPartKeys);
    const uint32_t groups = (parts + kGroupPartitions - 1) / kGroupPartitions;
    for (int p = 0; p < z.passes; ++p) {
      zero_span(z.pstat + (size_t)p * z.parts * kDigits, (int64_t)parts * kDigits, first, stride);
      zero_span(z.gstat + (size_t)p * z.groups * kDigits, (int64_t)groups * kDigits, first,
                stride);
    }
  }
  if (Meff == 0u || (int64_t)blockIdx.x * 256 >= N) return;  // no instances, or too many
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
  const SortMode mode = sort_mode(pass_dbits >= 0 ? pass_dbits : (int)keymap[1], tbits, idbits);
  // the buffers the first pass reads: an odd pass count starts from the
  // alternate ones, so that the last pass writes (keys, ids)
  uint64_t* __restrict__ kdst = (mode.passes & 1) ? keys_alt : keys;
  uint32_t* __restrict__ idst = (mode.passes & 1) ? ids_alt : ids;
  const uint32_t dmin = keymap[0];
  const int dbits = (int)keymap[1];
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
    if (mode.words) {
      // the sort's own key (tile above the depth bits less the frame's
      // smallest) with the row index below it, in one word
      const uint64_t mk = ((uint64_t)tile << dbits) | (uint64_t)(s_db[lo] - dmin);
      kdst[slot] = (mk << idbits) | (uint64_t)(g0 + lo);
    } else {
      kdst[slot] = ((uint64_t)tile << 32) | (uint64_t)s_db[lo];
      idst[slot] = (uint32_t)(g0 + lo);
    }
  }
}

// ---------------------------------------------------------------------------
// Stage 3b: onesweep radix sort
// ---------------------------------------------------------------------------
// 10-bit digits: a frame's keys need only the bits that vary (see KeyMap),
// about 39 at 1080p, so four passes.
constexpr int kRadixBits = kDigitBits;
constexpr int kRadix = 1 << kRadixBits;
constexpr int kSortItems = 7;
// 1024-lane workgroups of 7168 keys, one digit per lane in the per-digit
// phase; ~66 KB of LDS (see sort_pass_kernel).  Large partitions keep the
// number of partitions, and with it the look-back, short; at 1080p 7168
// keys give about 200 partitions, one per CU, and the four passes of a
// frame's 1.47M keys take 100 us against 104.5 us with 8192 (180
// partitions, 76 CUs idle) and 100 us with 6144 (longer look-back).
// (512-lane partitions of 3584 or 4096 keys, two digits per lane and 38-43
// KB of LDS: binning a 1080p frame takes 0.155 or 0.172 instead of 0.138 ms
// one frame at a time, with no gain with frames in flight.)
constexpr int kSortWaves = 16;
constexpr int kSortThreads = 64 * kSortWaves;
constexpr int kPart = kSortThreads * kSortItems;  // keys per partition
constexpr int kDL = kRadix / kSortThreads;       // digits per lane: tid, tid + threads, ...
static_assert(kDL * kSortThreads == kRadix, "whole digits per sort lane");
static_assert(kPart <= 65535, "per-wave counts and local starts fit 16 bits");
constexpr int kMaxPasses = 8;
constexpr uint32_t kFlagAgg = 1u << 30;
constexpr uint32_t kFlagPrefix = 2u << 30;
constexpr uint32_t kCountMask = (1u << 30) - 1u;
// Look-back in two levels: partitions form groups of kGroupParts; a
// partition sums the aggregates of the earlier partitions of its group and
// takes the group-level prefix, which the group's last partition finds by a
// look-back over group statuses, kGroupLookback at a time.
constexpr int kGroupParts = 16;
constexpr int kGroupLookback = 8;
static_assert(kDigits == kRadix && kPartKeys == kPart && kGroupPartitions == kGroupParts,
              "the duplication zeroes what the sort uses");
// Most blocks of the first digit's histogram (its grid is sized before the
// count is known; 128 blocks of 8192-key strides took 0.145 ms of binning
// at 1080p one frame at a time, 256 blocks 0.147).
constexpr int kHistBlocks = 128;

// The key a pass takes its digit from: the tile id above the depth bits
// minus the frame's smallest depth bits, in dbits bits.  Within a frame this
// is monotone and one-to-one in the stored key (every depth lies in
// [dmin, dmin + 2^dbits)), so sorting by it orders the stored keys; dbits =
// 32, dmin = 0 (a NULL key map in the kernels) is the stored key itself.
// The all-ones padding key stays all ones (last in every digit).
struct KeyMap {
  uint32_t dmin;
  int dbits;
};
__device__ inline KeyMap load_keymap(const uint32_t* keymap) {
  return keymap ? KeyMap{keymap[0], (int)keymap[1]} : KeyMap{0u, 32};
}
__device__ inline uint64_t sort_key(uint64_t k, KeyMap m) {
  if (k == ~0ull) return ~0ull;
  return ((k >> 32) << m.dbits) | (uint64_t)((uint32_t)k - m.dmin);
}
__device__ inline uint32_t sort_digit(uint64_t k, KeyMap m, int shift) {
  return (uint32_t)(sort_key(k, m) >> shift) & (uint32_t)(kRadix - 1);
}
// Key-id words: (sort key << idbits) | row index, written by the
// duplication when both fit 64 bits with every pass's digit inside the word
// (idbits + kRadixBits * passes <= 64, so the all-ones padding word is in the
// last digit of every pass).  A pass then moves one 8-byte word per instance
// instead of a key and an id, and the last pass writes the stored key and the
// id back out.  The words are whole keys of a stable sort by the sort key:
// equal sort keys come from different rows and leave the duplication in row
// order, which the row index in the low bits keeps.
template <bool kIdInKey>
__device__ inline uint32_t pass_digit(uint64_t k, KeyMap m, int shift) {
  if constexpr (kIdInKey) return (uint32_t)(k >> shift) & (uint32_t)(kRadix - 1);
  else return sort_digit(k, m, shift);
}
__device__ inline uint64_t unpack_key(uint64_t w, KeyMap m, int idbits) {
  const uint64_t mk = w >> idbits;
  const uint64_t dmask = (1ull << m.dbits) - 1ull;  // dbits <= 32
  return ((mk >> m.dbits) << 32) | (uint64_t)((uint32_t)(mk & dmask) + m.dmin);
}

// Digit totals of the first pass: each block histograms a contiguous share
// of the keys in LDS and adds it to sum[] (agent-scope atomics, at most
// kRadix per block).  Each pass turns its digit's totals into offsets itself
// (sort_pass_kernel) and totals the next pass's digit.
constexpr int kHistThreads = 1024;
constexpr int kHistItems = 8;

// The keys are in `keys`, or in `keys_alt` for an odd pass count, as key-id
// words or not (sort_mode, from the key map unless pass_dbits >= 0; a NULL
// key map sorts the keys' own bits).
__global__ __launch_bounds__(kHistThreads) void sort_first_hist_kernel(
    const uint64_t* __restrict__ keys, const uint64_t* __restrict__ keys_alt,
    const uint32_t* __restrict__ meff, const uint32_t* __restrict__ keymap, int tbits,
    int idbits, int pass_dbits, uint32_t* __restrict__ sum) {
  static_assert(kHistThreads == kRadix, "a lane per digit");
  const uint32_t M = *meff;
  const KeyMap km = load_keymap(keymap);
  const SortMode mode = sort_mode(pass_dbits >= 0 ? pass_dbits : km.dbits, tbits, idbits);
  const uint64_t* __restrict__ kin = (mode.passes & 1) ? keys_alt : keys;
  __shared__ uint32_t s_h[kRadix];
  const int tid = threadIdx.x;
  s_h[tid] = 0u;
  __syncthreads();
  const uint32_t share = (uint32_t)(((uint64_t)M + gridDim.x - 1) / gridDim.x);
  const uint32_t lo = blockIdx.x * share;
  const uint32_t hi = (uint64_t)lo + share < (uint64_t)M ? lo + share : M;
  for (uint32_t b = lo; b < hi; b += kHistThreads * kHistItems) {
    uint64_t k[kHistItems];
#pragma unroll
    for (int it = 0; it < kHistItems; ++it) {
      const uint32_t i = b + (uint32_t)(it * kHistThreads + tid);
      k[it] = i < hi ? kin[i] : ~0ull;
    }
#pragma unroll
    for (int it = 0; it < kHistItems; ++it)
      if (b + (uint32_t)(it * kHistThreads + tid) < hi)
        atomicAdd(&s_h[mode.words ? pass_digit<true>(k[it], km, idbits)
                                  : pass_digit<false>(k[it], km, 0)],
                  1u);
  }
  __syncthreads();
  if (s_h[tid]) atomicAdd(&sum[tid], s_h[tid]);
}

__device__ inline uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

#define GS_LD(p) __hip_atomic_load((p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
#define GS_ST(p, v) __hip_atomic_store((p), (v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)

// One digit pass.  pstat[part][digit] holds a partition's flagged digit
// count; gstat[group][digit] a group's flagged aggregate, then its
// inclusive prefix.  Every wait is on a partition with a smaller ticket
// (one that started earlier), so the passes cannot deadlock.
// kIdInKey: the keys are key-id words (vin unused; vout NULL except in the
// last pass, which writes the stored keys and the ids).
template <bool kIdInKey>
__global__ __launch_bounds__(kSortThreads) void sort_pass_kernel(
    const uint64_t* __restrict__ kin, const uint32_t* __restrict__ vin,
    uint64_t* __restrict__ kout, uint32_t* __restrict__ vout, const uint32_t* __restrict__ meff,
    int shift, int idbits, const uint32_t* __restrict__ keymap,
    const uint32_t* __restrict__ digit_totals,
    uint32_t* __restrict__ pstat, uint32_t* __restrict__ gstat, uint32_t* __restrict__ ticket,
    uint32_t* __restrict__ next_sum) {
  const uint32_t M = *meff;
  const KeyMap km = load_keymap(keymap);
  const bool has_next = next_sum != nullptr;  // the next pass's digit is totalled here
  // One buffer in three roles, one after another: the per-wave digit counts
  // (then offsets) while ranking, the keys in local sorted order, then the
  // values.
  __shared__ uint64_t s_buf[kPart];
  static_assert(sizeof(uint16_t) * kSortWaves * kRadix <= sizeof(uint64_t) * kPart,
                "the digit counts fit the key buffer");
  uint16_t(*s_wh)[kRadix] = reinterpret_cast<uint16_t(*)[kRadix]>(s_buf);
  uint32_t* s_vals = reinterpret_cast<uint32_t*>(s_buf);
  __shared__ uint16_t s_start[kRadix];  // block-local exclusive digit start
  __shared__ uint32_t s_gbase[kRadix];  // global base minus local start
  __shared__ uint32_t s_next[kRadix];   // histogram of the next pass's digit
  __shared__ uint32_t s_part;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) s_part = atomicAdd(ticket, 1u);
  // this pass's digit totals (complete: the kernel before added them), turned
  // into offsets beside the partition's own counts below
  uint32_t dtot[kDL];
#pragma unroll
  for (int h = 0; h < kDL; ++h) dtot[h] = digit_totals[tid + h * kSortThreads];
  for (int k = tid; k < kSortWaves * kRadix / 2; k += kSortThreads)
    reinterpret_cast<uint32_t*>(&s_wh[0][0])[k] = 0u;
#pragma unroll
  for (int h = 0; h < kDL; ++h) s_next[tid + h * kSortThreads] = 0u;
  __syncthreads();
  const uint32_t part = s_part;
  const uint32_t parts = (uint32_t)(((uint64_t)M + kPart - 1) / kPart);
  // a grid sized for the buffers' capacity: workgroups past the last
  // partition leave (nothing waits on a later partition)
  if (part >= parts) return;
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
    k[it] = valid ? kin[idx] : ~0ull;  // padding ranks last in the last digit
    if constexpr (!kIdInKey) v[it] = valid ? vin[idx] : 0u;
  }
  // stable rank within the wave: keys in (item, lane) order
  const uint64_t lt = lanemask_lt();
#pragma unroll
  for (int it = 0; it < kSortItems; ++it) {
    const uint32_t d = pass_digit<kIdInKey>(k[it], km, shift);
    // the lanes whose digit equals this lane's: per bit, the ballot where
    // the lane's bit is set, its complement where it is clear, i.e. the
    // complement of (ballot xor m) with m the bit spread over a word, on the
    // two halves of the mask
    uint32_t mlo = ~0u, mhi = ~0u;
#pragma unroll
    for (int b = 0; b < kRadixBits; ++b) {
      const uint32_t m = (uint32_t)((int32_t)(d << (31 - b)) >> 31);
      const uint64_t bal = __ballot(m != 0u);
      mlo &= ~((uint32_t)bal ^ m);
      mhi &= ~((uint32_t)(bal >> 32) ^ m);
    }
    const uint64_t match = ((uint64_t)mhi << 32) | mlo;
    const uint32_t before = s_wh[wave][d];
    rank[it] = before + (uint32_t)__popcll(match & lt);
    const int leader = __ffsll((long long)match) - 1;
    __builtin_amdgcn_wave_barrier();
    if (lane == leader) s_wh[wave][d] = (uint16_t)(before + (uint32_t)__popcll(match));
    __builtin_amdgcn_wave_barrier();
    if (has_next && wbase + (uint32_t)it * 64u + (uint32_t)lane < M)
      atomicAdd(&s_next[pass_digit<kIdInKey>(k[it], km, shift + kRadixBits)], 1u);
  }
  __syncthreads();
  // this partition's share of the next pass's digit totals
  if (has_next) {
#pragma unroll
    for (int h = 0; h < kDL; ++h) {
      const uint32_t c = s_next[tid + h * kSortThreads];
      if (c) atomicAdd(&next_sum[tid + h * kSortThreads], c);
    }
  }

  // lane tid takes digits tid + h * threads: wave offsets, block count,
  // block-local start
  uint32_t cnt[kDL], start[kDL], mine[kDL];
#pragma unroll
  for (int h = 0; h < kDL; ++h) {
    const int d = tid + h * kSortThreads;
    uint32_t c = 0;
    for (int w = 0; w < kSortWaves; ++w) {
      const uint32_t x = s_wh[w][d];
      s_wh[w][d] = (uint16_t)c;
      c += x;
    }
    cnt[h] = c;
  }
  // publish this partition's digit counts (padding keys, all in the last
  // digit, left out) as soon as they are known
  const uint32_t pad = (uint32_t)kPart - nvalid;
#pragma unroll
  for (int h = 0; h < kDL; ++h) {
    const int d = tid + h * kSortThreads;
    mine[h] = (d == kRadix - 1) ? cnt[h] - pad : cnt[h];
    GS_ST(&pstat[(size_t)part * kRadix + d], kFlagAgg | mine[h]);
  }
  {
    uint64_t carry = 0;
#pragma unroll
    for (int h = 0; h < kDL; ++h) {
      uint64_t ex;
      const uint64_t t = block_excl_scan_u64<kSortWaves>(cnt[h], ex);
      start[h] = (uint32_t)(carry + ex);
      carry += t;
    }
  }
  uint32_t doff[kDL];  // where each of the lane's digits starts in the output
  {
    uint64_t carry = 0;
#pragma unroll
    for (int h = 0; h < kDL; ++h) {
      uint64_t ex;
      const uint64_t t = block_excl_scan_u64<kSortWaves>(dtot[h], ex);
      doff[h] = (uint32_t)(carry + ex);
      carry += t;
    }
  }
#pragma unroll
  for (int h = 0; h < kDL; ++h) s_start[tid + h * kSortThreads] = (uint16_t)start[h];
  __syncthreads();
  // each key's position in local sorted order (the counts' buffer is free
  // after this)
#pragma unroll
  for (int it = 0; it < kSortItems; ++it) {
    const uint32_t dd = pass_digit<kIdInKey>(k[it], km, shift);
    rank[it] += (uint32_t)s_start[dd] + (uint32_t)s_wh[wave][dd];
  }

  // look-back, level 1: the earlier partitions of this group (each
  // published its counts above without waiting)
  const uint32_t g = part / kGroupParts, r = part % kGroupParts;
  const bool glast = r == kGroupParts - 1 || part == parts - 1;
  // while the other partitions' counts travel: the keys into LDS in local
  // sorted order (the buffer held the per-wave counts, which every wave has
  // read once all have passed the barrier)
  __syncthreads();
#pragma unroll
  for (int it = 0; it < kSortItems; ++it)
    if (wbase + (uint32_t)it * 64u + (uint32_t)lane < M) s_buf[rank[it]] = k[it];
  uint32_t sin[kDL];
#pragma unroll
  for (int h = 0; h < kDL; ++h) sin[h] = 0;
  if (r > 0) {
    const uint32_t need = (1u << r) - 1u;
    uint32_t have[kDL];  // bit q: partition g * kGroupParts + q added
#pragma unroll
    for (int h = 0; h < kDL; ++h) have[h] = 0;
    for (;;) {
      uint32_t sv[kDL][kGroupParts - 1];
#pragma unroll
      for (int h = 0; h < kDL; ++h)
#pragma unroll
        for (int q = 0; q < kGroupParts - 1; ++q)
          sv[h][q] = ((uint32_t)q < r && !((have[h] >> q) & 1u))
                         ? GS_LD(&pstat[(size_t)(g * kGroupParts + q) * kRadix + tid +
                                        h * kSortThreads])
                         : 0u;
      bool all = true;
#pragma unroll
      for (int h = 0; h < kDL; ++h) {
#pragma unroll
        for (int q = 0; q < kGroupParts - 1; ++q)
          if (sv[h][q] & ~kCountMask) {
            sin[h] += sv[h][q] & kCountMask;
            have[h] |= 1u << q;
          }
        all &= have[h] == need;
      }
      if (all) break;
      __builtin_amdgcn_s_sleep(1);
    }
  }
  // level 2: the prefix of the earlier groups
  uint32_t gp[kDL];
#pragma unroll
  for (int h = 0; h < kDL; ++h) gp[h] = 0;
  if (glast) {
#pragma unroll
    for (int h = 0; h < kDL; ++h)
      GS_ST(&gstat[(size_t)g * kRadix + tid + h * kSortThreads],
            (g == 0 ? kFlagPrefix : kFlagAgg) | (sin[h] + mine[h]));
    if (g > 0) {
      // add group aggregates back to the nearest inclusive prefix; group 0
      // always publishes one, so each walk ends there at the latest
      int64_t q[kDL];
      bool done[kDL];
#pragma unroll
      for (int h = 0; h < kDL; ++h) {
        q[h] = (int64_t)g - 1;
        done[h] = false;
      }
      for (;;) {
        uint32_t sv[kDL][kGroupLookback];
#pragma unroll
        for (int h = 0; h < kDL; ++h)
#pragma unroll
          for (int j = 0; j < kGroupLookback; ++j)
            sv[h][j] = (!done[h] && q[h] - j >= 0)
                           ? GS_LD(&gstat[(size_t)(q[h] - j) * kRadix + tid + h * kSortThreads])
                           : kFlagPrefix;
        bool all = true, stalled = false;
#pragma unroll
        for (int h = 0; h < kDL; ++h) {
          if (done[h]) continue;
          int j = 0;
          for (; j < kGroupLookback; ++j) {
            const uint32_t flag = sv[h][j] & ~kCountMask;
            if (flag == 0u) break;
            gp[h] += sv[h][j] & kCountMask;
            if (flag == kFlagPrefix) {
              done[h] = true;
              break;
            }
          }
          if (!done[h]) {
            q[h] -= j;
            all = false;
            stalled |= j < kGroupLookback;
          }
        }
        if (all) break;
        if (stalled) __builtin_amdgcn_s_sleep(1);
      }
#pragma unroll
      for (int h = 0; h < kDL; ++h)
        GS_ST(&gstat[(size_t)g * kRadix + tid + h * kSortThreads],
              kFlagPrefix | (gp[h] + sin[h] + mine[h]));
    }
  } else if (g > 0) {
    // the previous group's inclusive prefix (its last partition has a
    // smaller ticket)
#pragma unroll
    for (int h = 0; h < kDL; ++h) {
      uint32_t x;
      while (((x = GS_LD(&gstat[(size_t)(g - 1) * kRadix + tid + h * kSortThreads])) &
              ~kCountMask) != kFlagPrefix)
        __builtin_amdgcn_s_sleep(1);
      gp[h] = x & kCountMask;
    }
  }
#pragma unroll
  for (int h = 0; h < kDL; ++h) {
    const int d = tid + h * kSortThreads;
    s_gbase[d] = doff[h] + gp[h] + sin[h] - start[h];
  }
  __syncthreads();

  // keys (then values) out of LDS in local sorted order; written out in
  // that order, consecutive lanes hit consecutive slots of a digit run (the
  // barrier after the offsets also covers the keys' LDS writes above)
  if constexpr (kIdInKey) {
    const uint64_t idmask = (1ull << idbits) - 1ull;  // idbits < 64
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
      const uint32_t j = (uint32_t)tid + (uint32_t)i * kSortThreads;
      if (j < nvalid) {
        const uint64_t word = s_buf[j];
        const uint32_t out = s_gbase[pass_digit<true>(word, km, shift)] + j;
        if (vout) {
          kout[out] = unpack_key(word, km, idbits);
          vout[out] = (uint32_t)(word & idmask);
        } else {
          kout[out] = word;
        }
      }
    }
  } else {
    uint32_t outj[kSortItems];
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
      const uint32_t j = (uint32_t)tid + (uint32_t)i * kSortThreads;
      if (j < nvalid) {
        const uint64_t key = s_buf[j];
        const uint32_t out = s_gbase[sort_digit(key, km, shift)] + j;
        kout[out] = key;
        outj[i] = out;
      }
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < kSortItems; ++it)
      if (wbase + (uint32_t)it * 64u + (uint32_t)lane < M) s_vals[rank[it]] = v[it];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
      const uint32_t j = (uint32_t)tid + (uint32_t)i * kSortThreads;
      if (j < nvalid) vout[outj[i]] = s_vals[j];
    }
  }
}
#undef GS_LD
#undef GS_ST

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

// ---------------------------------------------------------------------------
// Workspace layout
// ---------------------------------------------------------------------------
struct SortPlan {
  int passes;
  uint32_t parts;
  uint32_t groups;
  int hblocks;  // blocks of the first digit's histogram
};

static inline int ceil_log2(uint32_t x) {
  int b = 0;
  while ((1ull << b) < x) ++b;
  return b;
}
static inline int ceil_log2_u64(uint64_t x) {
  int b = 0;
  while (b < 64 && (1ull << b) < x) ++b;
  return b;
}

// dbits: the depth bits the frame's key map keeps (32 when unknown on the
// host).
static inline SortPlan sort_plan(uint64_t M, int32_t T, int dbits = 32) {
  SortPlan p;
  p.passes = sort_pass_count(dbits + ceil_log2((uint32_t)T));
  p.parts = (uint32_t)((M + kPart - 1) / kPart);
  p.groups = (p.parts + kGroupParts - 1) / kGroupParts;
  const uint64_t hb = (M + kHistThreads * kHistItems - 1) / (kHistThreads * kHistItems);
  p.hblocks = hb < 1 ? 1 : (hb > (uint64_t)kHistBlocks ? kHistBlocks : (int)hb);
  return p;
}

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Workspace {
  uint64_t* keys_alt;
  uint32_t* ids_alt;
  uint64_t* scan_sums;
  uint64_t* total;
  uint32_t* meff;    // [1] instance count used by the binning kernels
  uint32_t* minmax;  // [nb][2] per scan block: smallest, largest depth bits
  uint32_t* keymap;  // [2] the sort's key map: smallest depth bits, bits kept
  uint32_t* dsum;     // [kMaxPasses][kRadix] digit totals (zeroed per call)
  uint32_t* ticket;   // [kMaxPasses] partition tickets (zeroed per call)
  uint32_t* pstat;    // [passes][parts][kRadix] partition statuses
  uint32_t* gstat;    // [passes][groups][kRadix] group statuses
  size_t bytes;       // (passes, parts, groups as planned for 32 depth bits)
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
  w.minmax = (uint32_t*)take(sizeof(uint32_t) * 2 * (nb ? nb : 1));
  w.keymap = (uint32_t*)take(sizeof(uint32_t) * 2);
  w.dsum = (uint32_t*)take(sizeof(uint32_t) * kMaxPasses * kRadix);
  w.ticket = (uint32_t*)take(sizeof(uint32_t) * kMaxPasses);
  w.pstat = (uint32_t*)take(sizeof(uint32_t) * (size_t)sp.passes * (sp.parts ? sp.parts : 1) * kRadix);
  w.gstat = (uint32_t*)take(sizeof(uint32_t) * (size_t)sp.passes * (sp.groups ? sp.groups : 1) * kRadix);
  w.bytes = off;
  return w;
}

// The passes, ping-ponging between (ka, ia) and (kb, ib); an even pass
// count ends in (ka, ia).  The first digit's totals are in dsum (from
// sort_first_hist_kernel); ticket and the later digits' totals must be zero.
// Statuses are laid out for lay.parts partitions and lay.groups groups per
// pass.  idbits >= 0: ka holds key-id words (pass_digit); the passes move
// only the words, and the last writes the stored keys and the ids.
static hipError_t launch_sort_passes(const SortPlan& sp, const SortPlan& lay,
                                     const uint32_t* meff, const uint32_t* keymap,
                                     uint32_t* dsum, uint32_t* ticket, uint32_t* pstat,
                                     uint32_t* gstat, uint64_t* ka, uint32_t* ia, uint64_t* kb,
                                     uint32_t* ib, int idbits, hipStream_t s) {
  hipError_t e;
  const bool words = idbits >= 0;
  const int s0 = words ? idbits : 0;
  for (int p = 0; p < sp.passes; ++p) {
    const bool next = p + 1 < sp.passes;
    if (words)
      hipLaunchKernelGGL(sort_pass_kernel<true>, dim3(sp.parts), dim3(kSortThreads), 0, s,
                         (const uint64_t*)ka, (const uint32_t*)nullptr, kb,
                         next ? (uint32_t*)nullptr : ib, meff, s0 + p * kRadixBits, idbits,
                         keymap, (const uint32_t*)(dsum + p * kRadix),
                         pstat + (size_t)p * lay.parts * kRadix,
                         gstat + (size_t)p * lay.groups * kRadix, ticket + p,
                         next ? dsum + (p + 1) * kRadix : nullptr);
    else
      hipLaunchKernelGGL(sort_pass_kernel<false>, dim3(sp.parts), dim3(kSortThreads), 0, s,
                         (const uint64_t*)ka, (const uint32_t*)ia, kb, ib, meff, p * kRadixBits,
                         0, keymap, (const uint32_t*)(dsum + p * kRadix),
                         pstat + (size_t)p * lay.parts * kRadix,
                         gstat + (size_t)p * lay.groups * kRadix, ticket + p,
                         next ? dsum + (p + 1) * kRadix : nullptr);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    uint64_t* tk = ka; ka = kb; kb = tk;
    uint32_t* ti = ia; ia = ib; ib = ti;
  }
  return hipSuccess;
}

}  // namespace gs

extern "C" size_t gs_binsort_workspace_bytes(int64_t N, uint64_t capacity, int32_t T) {
  return gs::carve(nullptr, N, capacity, T).bytes;
}

namespace gs {
// One event per device and host thread marks the count's copy to the host
// (a thread's calls wait on their own copies only); it is created on the
// device of stream s, which need not be the current one.
static hipError_t count_copy_event(hipStream_t s, hipEvent_t* ev) {
  static thread_local hipEvent_t evs[64] = {};
  int cur = 0;
  hipDevice_t dev = 0;
  hipError_t e;
  if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
  if (!s) dev = cur;  // the null stream: the current device's
  else if ((e = hipStreamGetDevice(s, &dev)) != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!evs[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    e = hipEventCreateWithFlags(&evs[dev], hipEventDisableTiming);
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
  }
  *ev = evs[dev];
  return hipSuccess;
}
}  // namespace gs

// First half of binning: scan, duplication and the first digit's histogram.
// Writes offsets and, with totals_host, M to totals_host[0] (read back) and
// the depth bits the sort's key map keeps to *dbits; with vis_ids non-NULL
// also the ascending indices of the Gaussians with tiles and their count V
// (totals_host[1], same read).  The host waits only for that read, which is
// queued before the duplication, so the duplication and the histogram run
// while the count travels.  totals_host NULL: the count and the key map stay
// on the device (dbits is not written), dev_counts (device, optional)
// receives M and the overflow flag, and the passes are planned for 32 depth
// bits.  The kernels take M from the device, 0 when it exceeds `capacity`.
// ncams > 1: a batch; N = ncams * ld rows, T = ncams tiles per camera.
extern "C" hipError_t gs_launch_bin_front(int64_t N, int64_t ld, const float* means2d,
                                          const int32_t* radii, const float* depths,
                                          const uint32_t* tiles, uint32_t* offsets,
                                          uint32_t* vis_ids, int32_t W, int32_t H, int ncams,
                                          uint64_t* keys, uint32_t* ids, uint32_t* ranges,
                                          void* workspace, uint64_t capacity,
                                          uint64_t* totals_host, int* dbits,
                                          uint64_t* dev_counts, hipStream_t s) {
  using namespace gs;
  const int gx = grid_dim(W), gy = grid_dim(H);
  const int32_t T = gx * gy * ncams;
  Workspace w = carve(workspace, N, capacity, T);
  hipError_t e;
  const bool vis = vis_ids != nullptr;
  if (N == 0) {
    if (totals_host) {
      totals_host[0] = 0;
      if (vis) totals_host[1] = 0;
      *dbits = 0;
      return hipSuccess;
    }
    // the device count must still read 0 (and the key map be defined)
    hipLaunchKernelGGL(scan_partials_kernel, dim3(1), dim3(256), 0, s, w.scan_sums, (int64_t)0,
                       w.minmax, w.total, w.keymap, capacity, w.meff, dev_counts);
    return hipGetLastError();
  }
  const int64_t nb = (N + kScanBlock - 1) / kScanBlock;
  if (vis)
    hipLaunchKernelGGL(scan_reduce_kernel<true>, dim3((unsigned)nb), dim3(256), 0, s, tiles,
                       depths, N, w.scan_sums, w.minmax);
  else
    hipLaunchKernelGGL(scan_reduce_kernel<false>, dim3((unsigned)nb), dim3(256), 0, s, tiles,
                       depths, N, w.scan_sums, w.minmax);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  uint64_t* dcounts = totals_host ? nullptr : dev_counts;
  if (vis)
    hipLaunchKernelGGL(scan_down_bin_kernel<true>, dim3((unsigned)nb), dim3(256), 0, s, tiles, N,
                       (const uint64_t*)w.scan_sums, (const uint32_t*)w.minmax, offsets, vis_ids,
                       w.total, w.keymap, capacity, w.meff, dcounts);
  else
    hipLaunchKernelGGL(scan_down_bin_kernel<false>, dim3((unsigned)nb), dim3(256), 0, s, tiles,
                       N, (const uint64_t*)w.scan_sums, (const uint32_t*)w.minmax, offsets,
                       (uint32_t*)nullptr, w.total, w.keymap, capacity, w.meff, dcounts);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipEvent_t ev = nullptr;
  if (totals_host) {
    // straight into the caller's host words: page-locked memory there makes
    // this a direct transfer instead of a staged one
    if ((e = count_copy_event(s, &ev)) != hipSuccess) return e;
    if ((e = hipMemcpyAsync(totals_host, w.total, sizeof(uint64_t) * (vis ? 2 : 1),
                            hipMemcpyDeviceToHost, s)) != hipSuccess)
      return e;
    if ((e = hipEventRecord(ev, s)) != hipSuccess) return e;
  }
  if (capacity > 0) {
    // statuses laid out for the capacity and 32 depth bits (the most passes)
    const SortPlan lay = sort_plan(capacity, T);
    // ticket follows dsum: one span from the digit totals to the tickets
    const SortZero z = {ranges, 2 * (int64_t)T, w.dsum,
                        (int64_t)(w.ticket + kMaxPasses - w.dsum), w.pstat, w.gstat,
                        lay.parts, lay.groups, lay.passes};
    const int tbits = ceil_log2((uint32_t)T);
    // key-id words only when the host knows the pass count (see sort_mode)
    const int idbits = totals_host ? ceil_log2_u64((uint64_t)N) : -1;
    const int pass_dbits = totals_host ? -1 : 32;
    // enough blocks for the rows and for a few zeroing strides
    int64_t nblk = (N + 255) / 256;
    const int64_t zblk = (2 * (int64_t)T + (int64_t)lay.parts * kRadix + 4095) / 4096;
    if (nblk < zblk) nblk = zblk;
    hipLaunchKernelGGL(duplicate_kernel, dim3((unsigned)nblk), dim3(256), 0, s, N, means2d, ld,
                       radii, depths, tiles, (const uint32_t*)offsets, gx, gy, ncams > 1,
                       (const uint32_t*)w.meff, z, (const uint32_t*)w.keymap, tbits, idbits,
                       pass_dbits, keys, ids, w.keys_alt, w.ids_alt);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // the first digit's offsets, over a grid for the capacity (each block
    // takes its share of the device count)
    const uint64_t hb = (capacity + kHistThreads * kHistItems - 1) / (kHistThreads * kHistItems);
    const unsigned hblocks = hb > (uint64_t)kHistBlocks ? (unsigned)kHistBlocks : (unsigned)hb;
    hipLaunchKernelGGL(sort_first_hist_kernel, dim3(hblocks), dim3(kHistThreads), 0, s,
                       (const uint64_t*)keys, (const uint64_t*)w.keys_alt,
                       (const uint32_t*)w.meff, (const uint32_t*)w.keymap, tbits, idbits,
                       pass_dbits, w.dsum);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (!totals_host) return hipSuccess;  // the count stays on the device
  if ((e = hipEventSynchronize(ev)) != hipSuccess) return e;
  *dbits = (int)(totals_host[0] >> kDbitsShift);
  totals_host[0] &= kCountBits;
  return hipSuccess;
}

// Second half: the sort passes and the per-tile ranges for M instances
// (M <= capacity), after gs_launch_bin_front with the same arguments.  M,
// dbits: as read back by the first half, or, with device_count, unknown on
// the host: the kernels then take M from the device, grids are sized for
// `capacity` and the passes cover 32 depth bits.
extern "C" hipError_t gs_launch_bin_back(int64_t N, int32_t W, int32_t H, int ncams, uint64_t M,
                                         int dbits, bool device_count, uint64_t* keys,
                                         uint32_t* ids, uint32_t* ranges, void* workspace,
                                         uint64_t capacity, hipStream_t s) {
  using namespace gs;
  const int gx = grid_dim(W), gy = grid_dim(H);
  const int32_t T = gx * gy * ncams;
  Workspace w = carve(workspace, N, capacity, T);
  hipError_t e;
  // grids for M, or for the largest count the buffers hold
  const uint64_t Mg = device_count ? capacity : M;
  if (Mg == 0) return fill_u32(ranges, 2 * (int64_t)T, 0u, s);
  const SortPlan sp = sort_plan(Mg, T, device_count ? 32 : dbits);
  const SortPlan lay = sort_plan(capacity, T);
  // the same choice the first half made on the device
  const SortMode mode = sort_mode(device_count ? 32 : dbits, ceil_log2((uint32_t)T),
                                  device_count ? -1 : ceil_log2_u64((uint64_t)N));
  if (mode.passes != sp.passes) return hipErrorInvalidValue;
  uint64_t* ka = (sp.passes & 1) ? w.keys_alt : keys;
  uint32_t* ia = (sp.passes & 1) ? w.ids_alt : ids;
  uint64_t* kb = (sp.passes & 1) ? keys : w.keys_alt;
  uint32_t* ib = (sp.passes & 1) ? ids : w.ids_alt;
  if ((e = launch_sort_passes(sp, lay, w.meff, (const uint32_t*)w.keymap, w.dsum,
                               w.ticket, w.pstat, w.gstat, ka, ia, kb, ib,
                               mode.words ? ceil_log2_u64((uint64_t)N) : -1, s)) != hipSuccess)
    return e;
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
  uint32_t* dsum;
  uint32_t* ticket;
  uint32_t* pstat;
  uint32_t* gstat;
  SortPlan sp;
  size_t bytes;
};

static PairSortWs carve_pairsort(void* base, uint64_t n, int bits) {
  PairSortWs w;
  w.sp = sort_plan(n, 1, bits);
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
  w.dsum = (uint32_t*)take(sizeof(uint32_t) * kMaxPasses * kRadix);
  w.ticket = (uint32_t*)take(sizeof(uint32_t) * kMaxPasses);
  w.pstat = (uint32_t*)take(sizeof(uint32_t) * (size_t)w.sp.passes * (w.sp.parts ? w.sp.parts : 1) *
                            kRadix);
  w.gstat = (uint32_t*)take(sizeof(uint32_t) * (size_t)w.sp.passes * (w.sp.groups ? w.sp.groups : 1) *
                            kRadix);
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
    Segs sg = {{w.dsum, w.pstat, w.gstat, w.gstat},
               {(int64_t)(w.ticket + kMaxPasses - w.dsum),
                (int64_t)w.sp.passes * w.sp.parts * kRadix,
                (int64_t)w.sp.passes * w.sp.groups * kRadix, 0}};
    int64_t blocks = (sg.n[1] + 255) / 256;
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
  if (w.sp.passes & 1) {
    if ((e = hipMemcpyAsync(w.keys_alt, keys, n * sizeof(uint64_t), hipMemcpyDeviceToDevice, s)) !=
        hipSuccess)
      return e;
    if ((e = hipMemcpyAsync(w.vals_alt, vals, n * sizeof(uint32_t), hipMemcpyDeviceToDevice, s)) !=
        hipSuccess)
      return e;
    ka = w.keys_alt; ia = w.vals_alt; kb = keys; ib = vals;
  }
  if ((e = fill_u32(w.meff, 1, (uint32_t)n, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(sort_first_hist_kernel, dim3((unsigned)w.sp.hblocks), dim3(kHistThreads), 0,
                     s, (const uint64_t*)ka, (const uint64_t*)ka, (const uint32_t*)w.meff,
                     (const uint32_t*)nullptr, 0, -1, bits, w.dsum);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return launch_sort_passes(w.sp, w.sp, w.meff, nullptr, w.dsum, w.ticket, w.pstat,
                            w.gstat, ka, ia, kb, ib, -1, s);
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
                       (int64_t)0, (const uint32_t*)nullptr, total, (uint32_t*)nullptr,
                       (uint64_t)0, (uint32_t*)nullptr, (uint64_t*)nullptr);
    return hipGetLastError();
  }
  uint64_t* sums = (uint64_t*)workspace;
  const int64_t nb = (n + kScanBlock - 1) / kScanBlock;
  hipLaunchKernelGGL(scan_reduce_kernel<false>, dim3((unsigned)nb), dim3(256), 0, s, in,
                     (const float*)nullptr, n, sums, (uint32_t*)nullptr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(scan_partials_kernel, dim3(1), dim3(256), 0, s, sums, nb,
                     (const uint32_t*)nullptr, total, (uint32_t*)nullptr, (uint64_t)0,
                     (uint32_t*)nullptr, (uint64_t*)nullptr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(scan_down_kernel<false>, dim3((unsigned)nb), dim3(256), 0, s, in, n, sums,
                     out, nullptr);
  return hipGetLastError();
}
