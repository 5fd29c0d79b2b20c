// gs_bin.hip -- duplication of Gaussians into (tile | depth) keys, for gfx950.
//
// "Better Gaussian Splatting in Julia" (lshu.cn) s3.2 (assign_to_tiles) and
// "Implementing Better Gaussian Splatting in Julia" (pwwt.cn) s4.3 (16x16 tiles): each
// visible Gaussian is listed once in every tile its support rectangle covers.  The
// 32-bit index wrap section of "Training 10M Gaussians in 8 GB: Spirula Studio's VRAM
// efficiency" (mhpq.cn) is why every count and offset here is 64-bit; its visibility
// bitmap section is the model for the wavefront-ballot compaction below.
//
// Pairs are written in the order (tile & 255, depth, id): the visible Gaussians are
// compacted (ballot + popcount per wavefront, in id order) and radix-sorted once by the
// bit pattern of their fp32 depth (a stable sort, so equal depths stay in id order).
// Their tiles are then expanded in that order, and the expansion itself performs the
// first digit pass of the tile sort: a counting pass gives every partition of 1024 pairs
// its count per value of the tile's low byte, a column scan turns those into offsets, and
// the scattering pass writes each pair at its place.  The keys leave ordered by their low
// 40 bits, so the pair sort is left with the tile bits above the low byte: one digit pass
// at 1080p instead of six over unsorted keys.
//
// Two phases around the one host read of the pair count: the depth phase (compaction,
// depth sort, records gathered into depth order) reads the visible count on the device,
// so it can be queued before the host has the pair count; the emission phase, whose grids
// depend on the pair count, follows.
//
// Kernels:
//   k_count_blocks   per 1024 Gaussians: pair count and visible count
//   k_scan_blocks    one workgroup: exclusive scan of per-block sums, and the total
//   k_compact        visible Gaussians' (depth bits, id), in id order
//   (radix sort of the compacted depths, gs_sort.hip)
//   k_count_sorted   per 1024 depth-sorted Gaussians: pair count; gathers their tile
//                    records (kept runs, rectangle, count) into depth order
//   k_offsets        per depth-sorted Gaussian: its first pair; per partition: its first
//                    Gaussian
//   k_emit_count     per chunk of 2 partitions: counts of the tile's low byte, per
//                    partition as prefixes inside the chunk, and the chunk's totals
//   k_group_scan,    exclusive scan of the chunk totals over chunks, per digit, in two
//   k_digit_scan     levels (groups of chunks, then the groups); the digits' totals
//   k_emit_scatter   per partition: regenerate the pairs, rank them stably by digit in
//                    LDS, write one contiguous run per digit
#include "gs_device.h"
#include "gs_tiles.h"

namespace gs {

hipError_t radix_sort_u32(int64_t P, const uint64_t* dcount, uint32_t* keys, uint32_t* vals, uint32_t* keys_tmp,
                          uint32_t* vals_tmp, int lo, int hi, void* ws, hipStream_t s, bool copy_back, bool ws_zeroed);
size_t radix_zero_bytes(int64_t P, int lo, int hi);
const int32_t* radix_result_in_tmp(const void* ws);
hipError_t launch_fill_u32(void* p, int64_t count, uint32_t v, hipStream_t s);
size_t radix_workspace_bytes(int64_t P, int lo, int hi);

constexpr int kBinBlock = 256;
constexpr int kBinPer = 4;                      // Gaussians per thread
constexpr int kBinChunk = kBinBlock * kBinPer;  // Gaussians per workgroup
constexpr int kEmitPer = 4;                       // pairs per lane in the emission passes
constexpr int kEmitPart = kBinBlock * kEmitPer;  // pairs per emission partition
constexpr int kDigits = 256;                      // values of the tile's low byte
constexpr int kCountParts = 2;                    // partitions per counting workgroup
constexpr int kDigitCopies = 16;                  // copies of the tile-digit counts (spreads the atomics)
// Bit of a depth-ordered pair count (sn) marking a Gaussian whose rectangle has neither
// packed runs nor rows in the projection's row table.  The emission passes come in two
// variants: the common one expands packed runs and table rows with integer work only; the
// other also derives rows from the render record (float64), and runs for the partitions
// (counting chunks) that hold such a Gaussian.  Keeping the float64 path out of the common
// variant keeps its registers, and so its occupancy, low.
constexpr uint32_t kLargeRect = 0x80000000u;
constexpr int kLargeGrid = 64;  // workgroups of the large variants (persistent over their lists)


__global__ __launch_bounds__(kBinBlock) void k_count_blocks(int64_t n, const uint32_t* __restrict__ n_tiles,
                                                            const uint2* __restrict__ rows,
                                                            uint64_t* __restrict__ pair_sums,
                                                            uint64_t* __restrict__ vis_sums,
                                                            uint64_t* __restrict__ ovf_sums) {
  __shared__ uint64_t s_p[kBinBlock / kWave], s_v[kBinBlock / kWave];
  // the projection's overflow flags for this block's Gaussians: one per 64 (the last entry
  // of each wavefront region of the row table), read by the first kBinChunk / 64 lanes
  constexpr int kRegions = kBinChunk / kWave;
  constexpr int kRegionRows = GS_ROWS_PER_BLOCK / (GS_ROW_BLOCK / kWave);
  uint64_t ovf = 0;
  {
    const int64_t r = (int64_t)blockIdx.x * kRegions + threadIdx.x;
    if (threadIdx.x < kRegions && r * kWave < n) ovf = rows[r * kRegionRows + kRegionRows - 1].x;
  }
  if (threadIdx.x < kWave) {
    ovf = wave_sum(ovf);
    if (threadIdx.x == 0) ovf_sums[blockIdx.x] = ovf;
  }
  const int64_t base = (int64_t)blockIdx.x * kBinChunk;
  uint64_t acc = 0, vis = 0;
#pragma unroll
  for (int j = 0; j < kBinPer; ++j) {
    const int64_t i = base + j * kBinBlock + threadIdx.x;
    const uint32_t c = i < n ? n_tiles[i] : 0u;
    acc += c;
    vis += (uint64_t)__popcll(__ballot(c > 0)) * (__lane_id() == 0 ? 1u : 0u);
  }
  acc = wave_sum(acc);
  if (__lane_id() == 0) {
    s_p[threadIdx.x / kWave] = acc;
    s_v[threadIdx.x / kWave] = vis;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t t = 0, u = 0;
#pragma unroll
    for (int w = 0; w < kBinBlock / kWave; ++w) { t += s_p[w]; u += s_v[w]; }
    pair_sums[blockIdx.x] = t;
    vis_sums[blockIdx.x] = u;
  }
}

// Exclusive scans of nb block sums in place, of NA arrays side by side, by one workgroup of
// NT threads; array a's total goes to total[a].  Rounds of NT * kScanPer sums: thread t
// takes kScanPer consecutive ones of every array (loads all in flight), sums them, the
// workgroup scans the threads' sums, and each thread writes its run's prefixes.
constexpr int kScanPer = 8;
template <int NT, int NA>
__device__ __forceinline__ void scan_sums(int64_t nb, uint64_t* const (&sums)[NA], uint64_t* __restrict__ total) {
  __shared__ uint64_t s_w[NA][NT / kWave];
  __shared__ uint64_t s_carry[NA];
  if (threadIdx.x < NA) s_carry[threadIdx.x] = 0;
  __syncthreads();
  const int lane = __lane_id(), wave = threadIdx.x / kWave;
  for (int64_t off = 0; off < nb; off += (int64_t)NT * kScanPer) {
    const int64_t i0 = off + (int64_t)threadIdx.x * kScanPer;
    uint64_t x[NA][kScanPer], t[NA], inc[NA];
#pragma unroll
    for (int a = 0; a < NA; ++a) {
      t[a] = 0;
#pragma unroll
      for (int k = 0; k < kScanPer; ++k) {
        x[a][k] = i0 + k < nb ? sums[a][i0 + k] : 0;
        t[a] += x[a][k];
      }
    }
#pragma unroll
    for (int a = 0; a < NA; ++a) {
      inc[a] = wave_inclusive_scan(t[a]);
      if (lane == kWave - 1) s_w[a][wave] = inc[a];
    }
    __syncthreads();
    uint64_t pre[NA];
#pragma unroll
    for (int a = 0; a < NA; ++a) {
      pre[a] = s_carry[a] + inc[a] - t[a];
      for (int w = 0; w < wave; ++w) pre[a] += s_w[a][w];
#pragma unroll
      for (int k = 0; k < kScanPer; ++k) {
        if (i0 + k < nb) sums[a][i0 + k] = pre[a];
        pre[a] += x[a][k];
      }
    }
    __syncthreads();
    if (threadIdx.x == NT - 1)
#pragma unroll
      for (int a = 0; a < NA; ++a) s_carry[a] = pre[a];
    __syncthreads();
  }
  if (threadIdx.x < NA) total[threadIdx.x] = s_carry[threadIdx.x];
}

__global__ __launch_bounds__(1024) void k_scan_blocks(int64_t nb, uint64_t* __restrict__ sums,
                                                      uint64_t* __restrict__ total) {
  uint64_t* const arrays[1] = {sums};
  scan_sums<1024, 1>(nb, arrays, total);
}

// The count phase's scans (pair sums, visible sums, overflow flags) side by side in one
// launch: totals[0..2] = P, V, overflowing wavefront regions; then the host's report word
// totals[3] = P with bit kReportLarge set when a rectangle takes the float64 path
// (kReportTooLarge when P does not fit below that bit).
constexpr uint64_t kReportLarge = 1ull << 62;
constexpr uint64_t kReportTooLarge = ~0ull >> 1;
__global__ __launch_bounds__(1024) void k_scan_blocks3(int64_t nb, uint64_t* __restrict__ a, uint64_t* __restrict__ b,
                                                       uint64_t* __restrict__ c, uint64_t* __restrict__ totals) {
  uint64_t* const arrays[3] = {a, b, c};
  scan_sums<1024, 3>(nb, arrays, totals);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint64_t P = totals[0];
    totals[3] = P < kReportLarge ? P | (totals[2] ? kReportLarge : 0ull) : kReportTooLarge;
  }
}

// Visible Gaussians' (depth bits, id) in id order.  Round r of a workgroup covers ids
// base + 256 r + [0, 256); a wavefront finds its visible lanes with one ballot.
__global__ __launch_bounds__(kBinBlock) void k_compact(int64_t n, const uint32_t* __restrict__ n_tiles,
                                                       const float* __restrict__ depth,
                                                       const uint64_t* __restrict__ vis_off,
                                                       uint32_t* __restrict__ dkeys, uint32_t* __restrict__ dvals,
                                                       uint64_t* __restrict__ dcopies,
                                                       uint32_t* __restrict__ sort_ws, int64_t sort_words) {
  __shared__ uint32_t s_w[kBinPer][kBinBlock / kWave];
  const int64_t base = (int64_t)blockIdx.x * kBinChunk;
  const int tid = threadIdx.x, lane = __lane_id(), wave = tid / kWave;
  // the depth sort's counters and look-back words start cleared (spread over the grid)
  for (int64_t i = (int64_t)blockIdx.x * kBinBlock + tid; i < sort_words; i += (int64_t)gridDim.x * kBinBlock)
    sort_ws[i] = 0;
  if (dcopies)  // cleared here (spread over the grid), added to by k_emit_count
    for (int i = (int)blockIdx.x * kBinBlock + tid; i < kDigitCopies * GS_TILE_DIGIT_COUNTS;
         i += (int)gridDim.x * kBinBlock)
      dcopies[i] = 0;
  bool vis[kBinPer];
  uint32_t below[kBinPer];
#pragma unroll
  for (int r = 0; r < kBinPer; ++r) {
    const int64_t i = base + r * kBinBlock + tid;
    vis[r] = i < n && n_tiles[i] > 0;
    const uint64_t m = __ballot(vis[r]);
    below[r] = (uint32_t)__popcll(m & lanemask_lt());
    if (lane == 0) s_w[r][wave] = (uint32_t)__popcll(m);
  }
  __syncthreads();
  uint64_t pre = vis_off[blockIdx.x];
#pragma unroll
  for (int r = 0; r < kBinPer; ++r) {
    uint64_t off = pre;
    uint32_t round_total = 0;
#pragma unroll
    for (int w = 0; w < kBinBlock / kWave; ++w) {
      if (w < wave) off += s_w[r][w];
      round_total += s_w[r][w];
    }
    if (vis[r]) {
      const int64_t i = base + r * kBinBlock + tid;
      dkeys[off + below[r]] = __float_as_uint(depth[i]);
      dvals[off + below[r]] = (uint32_t)i;
    }
    pre += round_total;
  }
}

// Per 1024 depth-sorted Gaussians: their pair count; also gathers their tile records
// into depth order for the emission (the one random-access pass over the Gaussians), with
// words 6 and 7 (the count, and zero) replaced by the Gaussian's id and depth bits, and
// the count in sn, with kLargeRect set for a rectangle whose rows the projection could not
// keep in its row table.  The depth sort leaves its result in (dk0, dv0) or (dk1, dv1), as
// *in_tmp says.
__global__ __launch_bounds__(kBinBlock) void k_count_sorted(const uint64_t* __restrict__ vcount,
                                                            const int32_t* __restrict__ in_tmp,
                                                            const uint32_t* __restrict__ dk0,
                                                            const uint32_t* __restrict__ dv0,
                                                            const uint32_t* __restrict__ dk1,
                                                            const uint32_t* __restrict__ dv1,
                                                            const uint4* __restrict__ runs,
                                                            uint4* __restrict__ sruns, uint32_t* __restrict__ sn,
                                                            uint64_t* __restrict__ sums) {
  __shared__ uint64_t s_p[kBinBlock / kWave];
  const int64_t v = (int64_t)*vcount;  // visible Gaussians (the grid covers all of them)
  const bool tmp = *in_tmp != 0;
  const uint32_t* dbits = tmp ? dk1 : dk0;
  const uint32_t* order = tmp ? dv1 : dv0;
  const int64_t base = (int64_t)blockIdx.x * kBinChunk;
  // every gather in flight before any is used
  uint32_t id[kBinPer], db[kBinPer];
  uint4 a[kBinPer], b[kBinPer];
#pragma unroll
  for (int j = 0; j < kBinPer; ++j) {
    const int64_t i = base + j * kBinBlock + threadIdx.x;
    id[j] = i < v ? order[i] : 0u;
    db[j] = i < v ? dbits[i] : 0u;
  }
#pragma unroll
  for (int j = 0; j < kBinPer; ++j) {
    const int64_t i = base + j * kBinBlock + threadIdx.x;
    a[j] = b[j] = make_uint4(0u, 0u, 0u, 0u);
    if (i < v) {
      a[j] = runs[2 * (size_t)id[j]];
      b[j] = runs[2 * (size_t)id[j] + 1];
    }
  }
  uint64_t acc = 0;
#pragma unroll
  for (int j = 0; j < kBinPer; ++j) {
    const int64_t i = base + j * kBinBlock + threadIdx.x;
    if (i < v) {
      sruns[2 * i] = a[j];
      sruns[2 * i + 1] = make_uint4(b[j].x, b[j].y, id[j], db[j]);
      sn[i] = b[j].z | (a[j].x == kNoSpans ? kLargeRect : 0u);
      acc += b[j].z;
    }
  }
  acc = wave_sum(acc);
  if (__lane_id() == 0) s_p[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t t = 0;
#pragma unroll
    for (int w = 0; w < kBinBlock / kWave; ++w) t += s_p[w];
    sums[blockIdx.x] = t;
  }
}

// Per-Gaussian pair offsets in depth order and the first Gaussian of every emission
// partition: goff[i] = pairs of the depth-sorted Gaussians before i (i in [0, v]);
// gstart[b] = the Gaussian holding pair b * kEmitPart.  Every visible Gaussian has at
// least one pair, so each partition start falls inside exactly one Gaussian's range.
// A Gaussian marked kLargeRect flags the partitions and counting chunks its pairs fall
// in (pflag, cflag, cleared beforehand) and appends each one, once, to the lists that
// the large variants of the emission passes walk: plist / clist, with their lengths in
// lcount[0] / lcount[1] (the lists' order does not matter).
__global__ __launch_bounds__(kBinBlock) void k_offsets(const uint64_t* __restrict__ vcount,
                                                       const uint32_t* __restrict__ sn,
                                                       const uint64_t* __restrict__ block_off,
                                                       uint64_t* __restrict__ goff, uint32_t* __restrict__ gstart,
                                                       uint32_t* __restrict__ pflag, uint32_t* __restrict__ cflag,
                                                       uint32_t* __restrict__ plist, uint32_t* __restrict__ clist,
                                                       uint32_t* __restrict__ lcount) {
  __shared__ uint64_t s_w[kBinBlock / kWave];
  const int64_t v = (int64_t)*vcount;
  const int64_t base = (int64_t)blockIdx.x * kBinChunk;
  const int tid = threadIdx.x, lane = __lane_id(), wave = tid / kWave;
  uint32_t cnt[kBinPer];
  uint32_t large = 0;  // bit j: position j holds a large rectangle
  uint64_t tsum = 0;
#pragma unroll
  for (int j = 0; j < kBinPer; ++j) {  // each thread owns kBinPer consecutive positions
    const int64_t i = base + (int64_t)tid * kBinPer + j;
    const uint32_t c = i < v ? sn[i] : 0u;
    cnt[j] = c & ~kLargeRect;
    large |= (c & kLargeRect) ? 1u << j : 0u;
    tsum += cnt[j];
  }
  const uint64_t inc = wave_inclusive_scan(tsum);
  if (lane == kWave - 1) s_w[wave] = inc;
  __syncthreads();
  uint64_t pre = block_off[blockIdx.x] + inc - tsum;
  for (int w = 0; w < wave; ++w) pre += s_w[w];
#pragma unroll
  for (int j = 0; j < kBinPer; ++j) {
    const int64_t i = base + (int64_t)tid * kBinPer + j;
    if (i >= v) break;
    goff[i] = pre;
    for (uint64_t pb = (pre + kEmitPart - 1) / kEmitPart; pb * kEmitPart < pre + cnt[j]; ++pb)
      gstart[pb] = (uint32_t)i;
    if (pflag && ((large >> j) & 1u)) {
      for (uint64_t pb = pre / kEmitPart; pb * kEmitPart < pre + cnt[j]; ++pb) {
        if (atomicExch(&pflag[pb], 1u) == 0u) plist[atomicAdd(&lcount[0], 1u)] = (uint32_t)pb;
        const uint64_t cb = pb / kCountParts;
        if (atomicExch(&cflag[cb], 1u) == 0u) clist[atomicAdd(&lcount[1], 1u)] = (uint32_t)cb;
      }
    }
    pre += cnt[j];
    if (i == v - 1) goff[v] = pre;
  }
}

// The pairs of emission partition b, [b C, min(P, (b + 1) C)) in depth order, as the
// counting and the scattering kernels both generate them: lane t takes kEmitPer
// consecutive pairs, finds the Gaussian of its first one by binary search over the
// partition's staged offsets, then walks the Gaussians' tile rectangles (rows outer).
struct EmitPart {
  int64_t base;  // first pair of the partition
  int n;         // pairs in the partition
  uint32_t g0;   // its first Gaussian (depth-sorted position)
  int ng;        // its Gaussians: g0 .. g0 + ng - 1
};

// Gaussians of a partition whose tile records the scattering pass stages in LDS (the
// partitions of the 1M-Gaussian 1080p orbit scenes hold 104 on average, 209 at most); the
// records of any further ones are read from memory.
constexpr int kStagedRecs = 224;

// Stages s_rel[i] = goff[g0 + i] - base for i in [0, ng] (the last one is the end of the
// partition's last Gaussian) and, with s_runs, the tile records of its first kStagedRecs
// Gaussians (two uint4 each).  Call from every thread; the caller synchronises.
__device__ __forceinline__ EmitPart stage_partition(int64_t b, int64_t nparts, int64_t v, int64_t P,
                                                    const uint64_t* __restrict__ goff,
                                                    const uint32_t* __restrict__ gstart, int32_t* s_rel,
                                                    const uint4* __restrict__ sruns, uint4* s_runs) {
  EmitPart e;
  e.base = b * kEmitPart;
  e.n = (int)min((int64_t)kEmitPart, P - e.base);
  e.g0 = gstart[b];
  const uint32_t g1 = b + 1 < nparts ? gstart[b + 1] : (uint32_t)(v - 1);
  e.ng = (int)(g1 - e.g0) + 1;
  // the first round of both loops issues its loads together
  const int t = threadIdx.x, nrel = e.ng + 1, nrun = s_runs ? 2 * min(e.ng, kStagedRecs) : 0;
  const uint64_t rel = t < nrel ? goff[e.g0 + t] : 0;
  const uint4 run = t < nrun ? sruns[2 * (size_t)e.g0 + t] : make_uint4(0u, 0u, 0u, 0u);
  if (t < nrel) s_rel[t] = (int32_t)((int64_t)rel - e.base);
  if (t < nrun) s_runs[t] = run;
  for (int i = t + kBinBlock; i < nrel; i += kBinBlock) s_rel[i] = (int32_t)((int64_t)goff[e.g0 + i] - e.base);
  for (int i = t + kBinBlock; i < nrun; i += kBinBlock) s_runs[i] = sruns[2 * (size_t)e.g0 + i];
  return e;
}

// Kept columns [c0, c1] of a row-table entry (first kept column | count << 16).
__device__ __forceinline__ void table_row(const uint2 t, int& c0, int& c1) {
  c0 = (int)(t.x & 0xFFFFu);
  c1 = c0 + (int)(t.x >> 16) - 1;
}

// Last row k of a rectangle's `rows` table entries whose earlier rows hold at most `pair`
// kept tiles (entry k's .y); when pair is below the rectangle's total, row k holds it.
__device__ __forceinline__ int table_find(const uint2* __restrict__ t, int rows, uint32_t pair) {
  int a = 0, b = rows - 1;  // t[0].y = 0 <= pair
  while (a < b) {
    const int m = (a + b + 1) >> 1;
    if (t[m].y <= pair) a = m; else b = m - 1;
  }
  return a;
}

// Generates this lane's pairs; emit(k, tile, id, dbits) receives the pair's slot in the
// lane's run (0 .. kEmitPer - 1), its tile, its Gaussian's id and the bit pattern of that
// Gaussian's depth.  sruns holds the depth-sorted Gaussians' tile records (words 6 and 7:
// id and depth bits), s_runs the partition's first kStagedRecs of them.  A Gaussian's pairs
// are the tiles its ellipse test keeps, rows outer and columns inner: read from the runs
// the projection stored, or, for a rectangle too large for the record, computed row by row
// from its render record (rec, by id).  Every loop stays inside the rectangle.
template <bool kLarge, typename F>
__device__ __forceinline__ void lane_pairs(const EmitPart& e, const int32_t* s_rel, const uint4* __restrict__ sruns,
                                           const uint4* s_runs, const uint2* __restrict__ table,
                                           const float4* __restrict__ rec, int tiles_x, F&& emit) {
  const int p0 = (int)threadIdx.x * kEmitPer;
  if (p0 >= e.n) return;
  int lo = 0, hi = e.ng;  // invariant: s_rel[lo] <= p0 < s_rel[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_rel[mid] <= p0) lo = mid; else hi = mid;
  }
  ushort4 r;  // tile rectangle x0, x1, y0, y1
  uint4 sp;   // packed kept runs
  TileEllipse te;  // the ellipse of a rectangle without packed runs
  int ty = 0, c0 = 0, c1 = -1;  // current row and its kept columns [c0, c1]
  uint32_t dbits = 0, id = 0;
  auto row = [&]() {
    if (spans_packed(sp)) {
      packed_row(sp, ty - (int)r.z, (int)r.x, c0, c1);
    } else if (sp.x == kTableSpans) {
      table_row(table[sp.y + (uint32_t)(ty - (int)r.z)], c0, c1);
    } else if (kLarge) {
      tile_row_span(te, ty, (int)r.x, (int)r.y, c0, c1);
    } else {  // never: such a Gaussian's partitions run in the float64 variant
      c0 = (int)r.x;
      c1 = c0 - 1;
    }
  };
  auto skip_empty = [&]() {
    while (c1 < c0 && ty < (int)r.w) {
      ++ty;
      row();
    }
  };
  auto start = [&](int li) {  // the first kept tile of the partition's Gaussian li
    const uint4* src = li < kStagedRecs ? s_runs + 2 * li : sruns + 2 * ((size_t)e.g0 + (uint32_t)li);
    sp = src[0];
    const uint4 b = src[1];
    r = make_ushort4((uint16_t)(b.x & 0xFFFFu), (uint16_t)(b.x >> 16), (uint16_t)(b.y & 0xFFFFu), (uint16_t)(b.y >> 16));
    id = b.z;
    dbits = b.w;
    if (kLarge && !spans_packed(sp))
      te = tile_ellipse_rec(rec[3 * (size_t)id], rec[3 * (size_t)id + 1], rec[3 * (size_t)id + 2]);
    ty = (int)r.z;
    row();
    skip_empty();
  };
  start(lo);
  int local = p0 - s_rel[lo];  // pairs of this Gaussian before the lane's first
  if (sp.x == kTableSpans) {
    // the row holding pair `local`: the last row whose earlier rows hold at most `local`
    // pairs (such a row is never empty)
    const int k = table_find(table + sp.y, (int)r.w - (int)r.z + 1, (uint32_t)local);
    ty = (int)r.z + k;
    local -= (int)table[sp.y + (uint32_t)k].y;
    row();
  }
  while (local > c1 - c0 && ty < (int)r.w) {
    local -= c1 >= c0 ? c1 - c0 + 1 : 0;
    ++ty;
    row();
  }
  int col = min(c0 + local, c1);
  int next = s_rel[lo + 1];
  const int run = min(kEmitPer, e.n - p0);
  for (int k = 0; k < run; ++k) {
    while (p0 + k >= next) {  // on to the next Gaussian
      ++lo;
      start(lo);
      col = c0;
      next = s_rel[lo + 1];
    }
    emit(k, (uint32_t)ty * (uint32_t)tiles_x + (uint32_t)col, id, dbits);
    if (++col > c1 && ty < (int)r.w) {
      ++ty;
      row();
      skip_empty();
      col = c0;
    }
  }
}

// Adds the pairs [sa, sb) of a Gaussian's kept tiles that lie on one row, tile ids
// t0 .. t0 + (sb - sa) - 1 (consecutive), to the counts of the partitions they fall in: the
// tile's low byte through a difference array per partition (a circular run of digits adds
// 1 at its start and -1 past its end; whole turns of 256 add to every digit), the higher
// tile digits directly.
__device__ __forceinline__ void count_row_segment(int64_t sa, int64_t sb, uint32_t t0, int64_t chunk_first_part,
                                                  int hp, int32_t (*s_diff)[kDigits + 1], uint32_t* s_uni,
                                                  uint32_t* s_hi) {
  while (sa < sb) {
    const int64_t q = sa / kEmitPart;  // partition
    const int64_t end = min(sb, (q + 1) * kEmitPart);
    const uint32_t L = (uint32_t)(end - sa);
    const int qi = (int)(q - chunk_first_part);
    if (L >> 8) atomicAdd(&s_uni[qi], L >> 8);
    const uint32_t rem = L & (kDigits - 1);
    if (rem) {
      const uint32_t a = t0 & (kDigits - 1), b = a + rem;
      atomicAdd(&s_diff[qi][a], 1);
      if (b <= (uint32_t)kDigits) {
        atomicAdd(&s_diff[qi][b], -1);
      } else {
        atomicAdd(&s_diff[qi][0], 1);
        atomicAdd(&s_diff[qi][b - kDigits], -1);
      }
    }
    const uint32_t t1 = t0 + L - 1;
    for (int p = 0; p < hp; ++p) {
      const int sh = 8 + 8 * p;
      for (uint32_t h = t0 >> sh; h <= t1 >> sh; ++h) {
        const uint32_t lo = max(t0, h << sh), hi = min(t1, ((h + 1) << sh) - 1u);
        atomicAdd(&s_hi[p * kDigits + (h & (kDigits - 1))], hi - lo + 1);
      }
    }
    t0 += L;
    sa = end;
  }
}

// Counting pass: per partition, how many of its pairs have each value of the tile's low
// byte.  A workgroup takes kCountParts consecutive partitions (a chunk) and writes, per
// partition, the counts of the chunk's earlier partitions (cnt_pre[b][d]) and, per chunk,
// its totals (csum[c][d]); both are contiguous rows.  The pairs are not generated one by
// one: each lane takes whole Gaussians of the chunk and walks their kept tile rows (the
// same records and order the scattering pass expands), adding each row's run of
// consecutive tile ids at once.  With hp > 0 it also counts the tile-id digits above the
// low byte (bits [8 + 8q, 16 + 8q), q < hp) for the pair sort, into copy (chunk mod
// kDigitCopies) of them in dcopies.
template <bool kLarge>
__device__ __forceinline__ void emit_count_chunk(int64_t chunk, int64_t v, int64_t P, int64_t nparts,
                                                 const uint4* __restrict__ sruns, const uint2* __restrict__ table,
                                                 const float4* __restrict__ rec,
                                                 const uint64_t* __restrict__ goff,
                                                 const uint32_t* __restrict__ gstart, int tiles_x,
                                                 uint32_t* __restrict__ cnt_pre, uint64_t* __restrict__ csum, int hp,
                                                 uint64_t* __restrict__ dcopies) {
  __shared__ int32_t s_diff[kCountParts][kDigits + 1];
  __shared__ uint32_t s_uni[kCountParts];
  __shared__ uint32_t s_hi[GS_TILE_DIGIT_COUNTS];  // the chunk's counts of the higher digits
  __shared__ uint32_t s_w[kCountParts][kBinBlock / kWave];
  const int tid = threadIdx.x, lane = __lane_id(), wave = tid / kWave;
  const int64_t b0 = chunk * kCountParts;
  const int nq = (int)min((int64_t)kCountParts, nparts - b0);
  for (int i = tid; i < kCountParts * (kDigits + 1); i += kBinBlock) (&s_diff[0][0])[i] = 0;
  if (tid < kCountParts) s_uni[tid] = 0;
  for (int i = tid; i < hp * kDigits; i += kBinBlock) s_hi[i] = 0;
  __syncthreads();
  // the chunk's pairs [r0, r1) and the Gaussians holding them
  const int64_t r0 = b0 * kEmitPart, r1 = min((b0 + nq) * kEmitPart, P);
  const int64_t g_first = gstart[b0];
  const int64_t g_last = b0 + nq < nparts ? (int64_t)gstart[b0 + nq] : v - 1;
  for (int64_t g = g_first + tid; g <= g_last; g += kBinBlock) {
    const int64_t G0 = (int64_t)goff[g], G1 = (int64_t)goff[g + 1];
    const int64_t lo = max(G0, r0), hi = min(G1, r1);  // this Gaussian's pairs in the chunk
    if (lo >= hi) continue;
    const uint4 sp = sruns[2 * g], rb = sruns[2 * g + 1];
    const int tx0 = (int)(rb.x & 0xFFFFu), tx1 = (int)(rb.x >> 16);
    const int ty0 = (int)(rb.y & 0xFFFFu), ty1 = (int)(rb.y >> 16);
    const bool packed = spans_packed(sp), tabled = sp.x == kTableSpans;
    TileEllipse te;
    if (kLarge && !packed && !tabled)
      te = tile_ellipse_rec(rec[3 * (size_t)rb.z], rec[3 * (size_t)rb.z + 1], rec[3 * (size_t)rb.z + 2]);
    int64_t off = G0;
    int ty = ty0;
    if (tabled && lo > G0) {  // start at the row holding the chunk's first pair of this Gaussian
      const int k = table_find(table + sp.y, ty1 - ty0 + 1, (uint32_t)(lo - G0));
      ty = ty0 + k;
      off = G0 + table[sp.y + (uint32_t)k].y;
    }
    for (; ty <= ty1 && off < hi; ++ty) {
      int c0, c1;
      if (packed)
        packed_row(sp, ty - ty0, tx0, c0, c1);
      else if (tabled)
        table_row(table[sp.y + (uint32_t)(ty - ty0)], c0, c1);
      else if (kLarge)
        tile_row_span(te, ty, tx0, tx1, c0, c1);
      else  // never: such a Gaussian's chunks run in the float64 variant
        c1 = (c0 = tx0) - 1;
      if (c1 < c0) continue;
      const int64_t len = c1 - c0 + 1;
      const int64_t sa = max(off, lo), sb = min(off + len, hi);
      if (sa < sb)
        count_row_segment(sa, sb, (uint32_t)ty * (uint32_t)tiles_x + (uint32_t)c0 + (uint32_t)(sa - off), b0, hp,
                          s_diff, s_uni, s_hi);
      off += len;
    }
  }
  __syncthreads();
  // counts per partition: the inclusive scan of its difference array over digits
  uint32_t cnt[kCountParts];
#pragma unroll
  for (int q = 0; q < kCountParts; ++q) {
    const uint32_t x = (uint32_t)s_diff[q][tid];
    const uint32_t inc = wave_inclusive_scan(x);
    if (lane == kWave - 1) s_w[q][wave] = inc;
    cnt[q] = inc;
  }
  __syncthreads();
  uint32_t running = 0;  // digit tid's count in the chunk's earlier partitions
#pragma unroll
  for (int q = 0; q < kCountParts; ++q) {
    if (q >= nq) break;
    uint32_t c = cnt[q] + s_uni[q];
    for (int w = 0; w < wave; ++w) c += s_w[q][w];
    cnt_pre[(b0 + q) * kDigits + tid] = running;
    running += c;
  }
  csum[chunk * kDigits + tid] = running;
  uint64_t* dc = dcopies + (chunk % kDigitCopies) * GS_TILE_DIGIT_COUNTS;
  for (int i = tid; i < hp * kDigits; i += kBinBlock)
    if (s_hi[i]) atomicAdd(reinterpret_cast<unsigned long long*>(dc + i), (unsigned long long)s_hi[i]);
}

// The common variant: one workgroup per chunk; a chunk in the large list is left to
// k_emit_count_large.
__global__ __launch_bounds__(kBinBlock) void k_emit_count(const uint64_t* __restrict__ vcount, int64_t P,
                                                          int64_t nparts, const uint4* __restrict__ sruns,
                                                          const uint2* __restrict__ table,
                                                          const uint32_t* __restrict__ cflag,
                                                          const uint64_t* __restrict__ goff,
                                                          const uint32_t* __restrict__ gstart, int tiles_x,
                                                          uint32_t* __restrict__ cnt_pre, uint64_t* __restrict__ csum,
                                                          int hp, uint64_t* __restrict__ dcopies) {
  if (cflag && cflag[blockIdx.x]) return;  // left to k_emit_count_large
  emit_count_chunk<false>(blockIdx.x, (int64_t)*vcount, P, nparts, sruns, table, nullptr, goff, gstart, tiles_x,
                          cnt_pre, csum, hp, dcopies);
}

// The chunks of the large list (lcount[1] of them), taken in turn by a small grid.
__global__ __launch_bounds__(kBinBlock) void k_emit_count_large(
    const uint64_t* __restrict__ vcount, int64_t P, int64_t nparts, const uint4* __restrict__ sruns,
    const uint2* __restrict__ table, const float4* __restrict__ rec, const uint32_t* __restrict__ clist,
    const uint32_t* __restrict__ lcount,
    const uint64_t* __restrict__ goff, const uint32_t* __restrict__ gstart, int tiles_x,
    uint32_t* __restrict__ cnt_pre, uint64_t* __restrict__ csum, int hp, uint64_t* __restrict__ dcopies) {
  const uint32_t n = lcount[1];
  const int64_t v = (int64_t)*vcount;
  for (uint32_t it = blockIdx.x; it < n; it += gridDim.x) {
    emit_count_chunk<true>(clist[it], v, P, nparts, sruns, table, rec, goff, gstart, tiles_x, cnt_pre, csum, hp,
                           dcopies);
    __syncthreads();  // the next chunk reuses the shared arrays
  }
}

// The chunk totals' exclusive scan over chunks, per digit, in two levels so that every
// read of csum is a whole row (all 256 digits of one chunk, contiguous):
//   k_group_scan  per group of kScanGroup chunks: the scan inside the group (csum in place)
//                 and the group's total per digit (gsum[g][d])
//   k_digit_scan  per digit: exclusive scan of the group totals (gsum in place) and the
//                 digit's total; with digit_counts non-NULL, workgroup d also sums the
//                 copies of the higher tile-digit counts [0][d] and [1][d] into it
// A chunk's count of digit d in all earlier chunks is then csum[c][d] + gsum[c / kScanGroup][d].
constexpr int kScanGroup = 32;

__global__ __launch_bounds__(kBinBlock) void k_group_scan(int64_t nchunks, uint64_t* __restrict__ csum,
                                                          uint64_t* __restrict__ gsum) {
  const int d = threadIdx.x;
  const int64_t c0 = (int64_t)blockIdx.x * kScanGroup;
  const int n = (int)min((int64_t)kScanGroup, nchunks - c0);
  uint64_t x[kScanGroup];
#pragma unroll
  for (int i = 0; i < kScanGroup; ++i) x[i] = i < n ? csum[(c0 + i) * kDigits + d] : 0;  // all loads in flight
  uint64_t run = 0;
#pragma unroll
  for (int i = 0; i < kScanGroup; ++i) {
    if (i < n) csum[(c0 + i) * kDigits + d] = run;
    run += x[i];
  }
  gsum[blockIdx.x * kDigits + d] = run;
}

__global__ __launch_bounds__(kBinBlock) void k_digit_scan(int64_t ngroups, uint64_t* __restrict__ gsum,
                                                          uint64_t* __restrict__ totals,
                                                          const uint64_t* __restrict__ dcopies,
                                                          uint64_t* __restrict__ digit_counts) {
  if (digit_counts && threadIdx.x < GS_TILE_DIGIT_COUNTS / kDigits) {
    const int i = (int)threadIdx.x * kDigits + (int)blockIdx.x;
    uint64_t t = 0;
#pragma unroll
    for (int c = 0; c < kDigitCopies; ++c) t += dcopies[c * GS_TILE_DIGIT_COUNTS + i];
    digit_counts[i] = t;
  }
  __shared__ uint64_t s_w[kBinBlock / kWave];
  __shared__ uint64_t s_carry;
  const int tid = threadIdx.x, lane = __lane_id(), wave = tid / kWave;
  const int d = blockIdx.x;
  if (tid == 0) s_carry = 0;
  __syncthreads();
  for (int64_t off = 0; off < ngroups; off += kBinBlock) {
    const int64_t g = off + tid;
    const uint64_t x = g < ngroups ? gsum[g * kDigits + d] : 0;
    const uint64_t inc = wave_inclusive_scan(x);
    if (lane == kWave - 1) s_w[wave] = inc;
    __syncthreads();
    uint64_t pre = s_carry + inc - x;
    for (int w = 0; w < wave; ++w) pre += s_w[w];
    if (g < ngroups) gsum[g * kDigits + d] = pre;
    __syncthreads();
    if (tid == kBinBlock - 1) s_carry = pre + x;
    __syncthreads();
  }
  if (tid == 0) totals[d] = s_carry;
}

// Logical partition of workgroup i when the dispatcher deals workgroups to the 8 XCDs
// in turn (i on XCD i mod 8): XCD x takes one contiguous range of partitions, so the
// short digit runs that neighbouring partitions write next to each other meet in the same
// L2 and leave it as whole lines.  A bijection of [0, n).
__device__ __forceinline__ int64_t xcd_contiguous(int64_t i, int64_t n) {
  constexpr int64_t kXcds = 8;
  const int64_t x = i % kXcds, q = n / kXcds, r = n % kXcds;
  return x * q + (x < r ? x : r) + i / kXcds;
}

// Scattering pass: writes the partition's pairs, keys[p] = tile << 32 | depth bits and
// vals[p] = Gaussian id, at their place in the order (tile & 255, depth, id).  The pairs
// are generated as in the counting pass, moved through LDS into wavefront-striped order,
// ranked stably by digit (wavefront ballots match equal digits), regrouped by digit in
// LDS and written as one contiguous run per digit; a run starts at the digit's global
// base plus the digit's count in earlier partitions.
template <bool kLarge>
__device__ __forceinline__ void emit_scatter_part(int64_t b, int64_t v, int64_t P, int64_t nparts,
                                                  const uint4* __restrict__ sruns, const uint2* __restrict__ table,
                                                  const float4* __restrict__ rec,
                                                  const uint64_t* __restrict__ goff,
                                                  const uint32_t* __restrict__ gstart, int tiles_x,
                                                  const uint32_t* __restrict__ cnt_pre,
                                                  const uint64_t* __restrict__ cpre, const uint64_t* __restrict__ gpre,
                                                  const uint64_t* __restrict__ totals, uint64_t* __restrict__ keys,
                                                  uint32_t* __restrict__ vals) {
  constexpr int kPad = kEmitPart + kEmitPart / kEmitPer;  // one pad slot per lane run
  __shared__ int32_t s_rel[kEmitPart + 2];
  __shared__ uint64_t s_keys[kPad];
  __shared__ uint32_t s_vals[kPad];
  // the staged tile records serve the generation only, the digit arrays the ranking and
  // what follows it, so they share their LDS
  union Digits {
    uint4 runs[2 * kStagedRecs];
    struct {
      uint32_t wh[kBinBlock / kWave][kDigits];  // per-wave digit counters, then offsets
      uint32_t lbase[kDigits];                   // partition-local digit starts
      uint64_t gbase[kDigits];                   // global digit starts for this partition
    } d;
  };
  static_assert(sizeof(uint4) * 2 * kStagedRecs <= sizeof(Digits), "staged records fit the digit arrays");
  __shared__ Digits s_u;
  uint32_t (*s_wh)[kDigits] = s_u.d.wh;
  uint32_t* s_lbase = s_u.d.lbase;
  uint64_t* s_gbase = s_u.d.gbase;
  __shared__ uint64_t s_w[kBinBlock / kWave];
  __shared__ uint64_t s_gw[kBinBlock / kWave];
  const int tid = threadIdx.x, lane = __lane_id(), wave = tid / kWave;
  // digit tid's total and its count in earlier partitions: loaded now, used once the pairs
  // are ranked (the global start of this partition's run of the digit)
  const uint64_t gtot = totals[tid];
  const int64_t chunk = b / kCountParts;
  const uint64_t gpart = gpre[(chunk / kScanGroup) * kDigits + tid] + cpre[chunk * kDigits + tid] +
                         cnt_pre[b * kDigits + tid];
  const EmitPart e = stage_partition(b, nparts, v, P, goff, gstart, s_rel, sruns, s_u.runs);
  __syncthreads();
  // generate: lane-consecutive, one pad slot per lane so that a wavefront's 8-byte
  // stores spread over the LDS banks
  lane_pairs<kLarge>(e, s_rel, sruns, s_u.runs, table, rec, tiles_x,
                     [&](int k, uint32_t tile, uint32_t id, uint32_t dbits) {
                       const int slot = tid * (kEmitPer + 1) + k;
                       s_keys[slot] = ((uint64_t)tile << 32) | (uint64_t)dbits;
                       s_vals[slot] = id;
                     });
  __syncthreads();
  // the staged records are read: each wavefront clears its own row of digit counters
  // (its LDS operations stay in order, so the ranking's atomics below come after)
  for (int i = lane; i < kDigits; i += kWave) s_wh[wave][i] = 0;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  // wavefront-striped: wave w owns pairs [w * kWavePart, (w + 1) * kWavePart) of the partition
  constexpr int kWavePart = kEmitPer * kWave;
  uint64_t key[kEmitPer];
  uint32_t val[kEmitPer], rank[kEmitPer];
#pragma unroll
  for (int j = 0; j < kEmitPer; ++j) {
    const int p = wave * kWavePart + j * kWave + lane;
    const int slot = p + p / kEmitPer;
    key[j] = p < e.n ? s_keys[slot] : ~0ull;
    val[j] = p < e.n ? s_vals[slot] : 0u;
  }
  // stable ranking as in the onesweep passes: the lowest lane of each group of equal digits
  // advances the wavefront's counter with a returning LDS atomic (in issue order), and a
  // shuffle hands the group its base
  uint32_t prev[kEmitPer];
  int lead[kEmitPer];
#pragma unroll
  for (int j = 0; j < kEmitPer; ++j) {
    const int p = wave * kWavePart + j * kWave + lane;
    const bool valid = p < e.n;
    const uint32_t d = (uint32_t)(key[j] >> 32) & (kDigits - 1);
    const uint64_t m = match_digit(d, 8, __ballot(valid));
    const uint64_t lower = m & lanemask_lt();
    rank[j] = (uint32_t)__popcll(lower);
    lead[j] = valid ? (int)__builtin_ctzll(m) : lane;
    prev[j] = 0;
    if (valid && lower == 0) prev[j] = atomicAdd(&s_wh[wave][d], (uint32_t)__popcll(m));
  }
#pragma unroll
  for (int j = 0; j < kEmitPer; ++j) rank[j] += (uint32_t)__shfl((int)prev[j], lead[j], kWave);
  __syncthreads();
  {  // thread d owns digit d: per-wave offsets, the partition-local digit starts, and the
     // global start of the partition's run of d (the digit's base over all digits before it,
     // plus its count in earlier partitions)
    const int d = tid;
    uint32_t tot = 0;
#pragma unroll
    for (int w = 0; w < kBinBlock / kWave; ++w) {
      const uint32_t c = s_wh[w][d];
      s_wh[w][d] = tot;
      tot += c;
    }
    const uint64_t inc = wave_inclusive_scan((uint64_t)tot);
    const uint64_t ginc = wave_inclusive_scan(gtot);
    if (lane == kWave - 1) {
      s_w[wave] = inc;
      s_gw[wave] = ginc;
    }
    __syncthreads();
    uint64_t pre = inc - tot, gpre = ginc - gtot;
    for (int w = 0; w < wave; ++w) {
      pre += s_w[w];
      gpre += s_gw[w];
    }
    s_lbase[d] = (uint32_t)pre;
    s_gbase[d] = gpre + gpart;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kEmitPer; ++j) {  // regroup by digit (stable)
    const int p = wave * kWavePart + j * kWave + lane;
    if (p < e.n) {
      const uint32_t d = (uint32_t)(key[j] >> 32) & (kDigits - 1);
      const uint32_t pos = s_lbase[d] + s_wh[wave][d] + rank[j];
      s_keys[pos] = key[j];
      s_vals[pos] = val[j];
    }
  }
  __syncthreads();
  for (int i = tid; i < e.n; i += kBinBlock) {
    const uint64_t k = s_keys[i];
    const uint32_t d = (uint32_t)(k >> 32) & (kDigits - 1);
    const uint64_t g = s_gbase[d] + (uint64_t)(i - (int)s_lbase[d]);
    if (g < (uint64_t)P) {  // always, given the counting pass's counts
      keys[g] = k;
      vals[g] = s_vals[i];
    }
  }
}

// The common variant: one workgroup per partition (XCD-contiguous); a partition in the
// large list is left to k_emit_scatter_large.
__global__ __launch_bounds__(kBinBlock) void k_emit_scatter(
    const uint64_t* __restrict__ vcount, int64_t P, int64_t nparts, const uint4* __restrict__ sruns,
    const uint2* __restrict__ table, const uint32_t* __restrict__ pflag, const uint64_t* __restrict__ goff,
    const uint32_t* __restrict__ gstart,
    int tiles_x, const uint32_t* __restrict__ cnt_pre, const uint64_t* __restrict__ cpre,
    const uint64_t* __restrict__ gpre, const uint64_t* __restrict__ totals, uint64_t* __restrict__ keys,
    uint32_t* __restrict__ vals) {
  const int64_t b = xcd_contiguous(blockIdx.x, nparts);
  if (pflag && pflag[b]) return;  // left to k_emit_scatter_large
  emit_scatter_part<false>(b, (int64_t)*vcount, P, nparts, sruns, table, nullptr, goff, gstart, tiles_x, cnt_pre,
                           cpre, gpre, totals, keys, vals);
}

// The partitions of the large list (lcount[0] of them), taken in turn by a small grid.
__global__ __launch_bounds__(kBinBlock) void k_emit_scatter_large(
    const uint64_t* __restrict__ vcount, int64_t P, int64_t nparts, const uint4* __restrict__ sruns,
    const uint2* __restrict__ table, const float4* __restrict__ rec, const uint32_t* __restrict__ plist,
    const uint32_t* __restrict__ lcount,
    const uint64_t* __restrict__ goff, const uint32_t* __restrict__ gstart, int tiles_x,
    const uint32_t* __restrict__ cnt_pre, const uint64_t* __restrict__ cpre, const uint64_t* __restrict__ gpre,
    const uint64_t* __restrict__ totals, uint64_t* __restrict__ keys, uint32_t* __restrict__ vals) {
  const uint32_t n = lcount[0];
  const int64_t v = (int64_t)*vcount;
  for (uint32_t it = blockIdx.x; it < n; it += gridDim.x) {
    emit_scatter_part<true>(plist[it], v, P, nparts, sruns, table, rec, goff, gstart, tiles_x, cnt_pre, cpre, gpre,
                            totals, keys, vals);
    __syncthreads();  // the next partition reuses the shared arrays
  }
}

// Workspace layout (bytes).  The arrays sized by the pair count come last, so the count
// phase (which runs before P is known) and the emission phase agree on every offset.
struct BinLayout {
  size_t pair_sums, vis_sums, ovf_sums, sorted_sums, totals, dcopies, dk0, dv0, dk1, dv1, sort, goff, sruns, sn, dtotals, gstart,
      cnt_pre, csum, gsum, flags, plist, clist, total;
  int64_t nb, nparts, nchunks, ngroups;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static BinLayout bin_layout(int64_t n, int64_t P) {
  BinLayout l;
  l.nb = (n + kBinChunk - 1) / kBinChunk;
  l.nparts = (P + kEmitPart - 1) / kEmitPart;
  l.nchunks = (l.nparts + kCountParts - 1) / kCountParts;
  const size_t sums = align256(sizeof(uint64_t) * (size_t)(l.nb + 1));
  const size_t ids = align256(sizeof(uint32_t) * (size_t)(n > 0 ? n : 1));
  l.pair_sums = 0;
  l.vis_sums = l.pair_sums + sums;
  l.ovf_sums = l.vis_sums + sums;
  l.sorted_sums = l.ovf_sums + sums;
  l.totals = l.sorted_sums + sums;
  l.dcopies = l.totals + 256;
  l.dk0 = l.dcopies + sizeof(uint64_t) * kDigitCopies * GS_TILE_DIGIT_COUNTS;
  l.dv0 = l.dk0 + ids;
  l.dk1 = l.dv0 + ids;
  l.dv1 = l.dk1 + ids;
  l.sort = l.dv1 + ids;
  l.goff = l.sort + align256(radix_workspace_bytes(n, 0, 32));
  l.sruns = l.goff + align256(sizeof(uint64_t) * (size_t)(n + 1));
  l.sn = l.sruns + align256(2 * sizeof(uint4) * (size_t)(n > 0 ? n : 1));
  l.dtotals = l.sn + align256(sizeof(uint32_t) * (size_t)(n > 0 ? n : 1));
  l.gstart = l.dtotals + sizeof(uint64_t) * kDigits;
  l.cnt_pre = l.gstart + align256(sizeof(uint32_t) * (size_t)(l.nparts + 1));
  l.csum = l.cnt_pre + align256(sizeof(uint32_t) * kDigits * (size_t)l.nparts);
  l.ngroups = (l.nchunks + kScanGroup - 1) / kScanGroup;
  l.gsum = l.csum + align256(sizeof(uint64_t) * kDigits * (size_t)l.nchunks);
  // partition flags [nparts], chunk flags [nchunks] and the two list lengths, contiguous
  // (one clearing launch); then the lists of large partitions and chunks
  l.flags = l.gsum + align256(sizeof(uint64_t) * kDigits * (size_t)(l.ngroups > 0 ? l.ngroups : 1));
  l.plist = l.flags + align256(sizeof(uint32_t) * (size_t)(l.nparts + l.nchunks + 2));
  l.clist = l.plist + align256(sizeof(uint32_t) * (size_t)(l.nparts > 0 ? l.nparts : 1));
  l.total = l.clist + sizeof(uint32_t) * (size_t)(l.nchunks > 0 ? l.nchunks : 1);
  return l;
}

size_t bin_workspace_bytes(int64_t n, int64_t P) { return bin_layout(n, P).total; }

// Phase 1: per-block sums, their scans, P and the visible count V (device, totals[0..1]),
// and the report word for the host (totals[3]: P, and whether the float64 path is needed).
hipError_t launch_bin_count(int64_t n, const uint32_t* n_tiles, const uint32_t* rows, void* ws, hipStream_t s) {
  const BinLayout l = bin_layout(n, 0);
  char* w = static_cast<char*>(ws);
  uint64_t* ps = reinterpret_cast<uint64_t*>(w + l.pair_sums);
  uint64_t* vs = reinterpret_cast<uint64_t*>(w + l.vis_sums);
  uint64_t* os = reinterpret_cast<uint64_t*>(w + l.ovf_sums);
  uint64_t* totals = reinterpret_cast<uint64_t*>(w + l.totals);
  if (l.nb > 0)
    k_count_blocks<<<(unsigned)l.nb, kBinBlock, 0, s>>>(n, n_tiles, reinterpret_cast<const uint2*>(rows), ps, vs, os);
  k_scan_blocks3<<<1, 1024, 0, s>>>(l.nb, ps, vs, os, totals);
  return hipGetLastError();
}

// Decodes the report word: the pair count, and whether a rectangle takes the float64 path;
// false when the count does not fit below the flag bit.
bool bin_report(uint64_t report, int64_t* P, bool* large) {
  if (report == kReportTooLarge) return false;
  *large = (report & kReportLarge) != 0;
  *P = (int64_t)(report & ~kReportLarge);
  return true;
}

// Exclusive scan of nb per-workgroup sums in place by one workgroup; the total to *total.
hipError_t launch_scan_sums(int64_t nb, uint64_t* sums, uint64_t* total, hipStream_t s) {
  k_scan_blocks<<<1, 1024, 0, s>>>(nb, sums, total);
  return hipGetLastError();
}

// The report word the host reads (totals[3]).
uint64_t* bin_report_ptr(int64_t n, void* ws) {
  return reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + bin_layout(n, 0).totals) + 3;
}

// Depth phase, queued right after the count: compact the visible Gaussians, sort them by
// depth and gather their tile records into depth order, with per-block pair sums and
// their scan.  The visible count V is read on the device (totals[1]); every grid is sized
// for all n Gaussians, so no host value is needed.
hipError_t launch_bin_depth(int64_t n, const gs_projected& proj, uint64_t* digit_counts, void* ws, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const BinLayout l = bin_layout(n, 0);
  char* w = static_cast<char*>(ws);
  uint32_t* dk0 = reinterpret_cast<uint32_t*>(w + l.dk0);
  uint32_t* dv0 = reinterpret_cast<uint32_t*>(w + l.dv0);
  uint32_t* dk1 = reinterpret_cast<uint32_t*>(w + l.dk1);
  uint32_t* dv1 = reinterpret_cast<uint32_t*>(w + l.dv1);
  uint64_t* ss = reinterpret_cast<uint64_t*>(w + l.sorted_sums);
  uint64_t* totals = reinterpret_cast<uint64_t*>(w + l.totals);
  uint4* sruns = reinterpret_cast<uint4*>(w + l.sruns);
  uint32_t* sn = reinterpret_cast<uint32_t*>(w + l.sn);
  k_compact<<<(unsigned)l.nb, kBinBlock, 0, s>>>(n, proj.n_tiles, proj.depth,
                                                 reinterpret_cast<const uint64_t*>(w + l.vis_sums), dk0, dv0,
                                                 digit_counts ? reinterpret_cast<uint64_t*>(w + l.dcopies) : nullptr,
                                                 reinterpret_cast<uint32_t*>(w + l.sort),
                                                 (int64_t)(radix_zero_bytes(n, 0, 32) / 4));
  // the sorted depths stay where the last pass wrote them: k_count_sorted picks the buffer
  hipError_t e = radix_sort_u32(n, totals + 1, dk0, dv0, dk1, dv1, 0, 32, w + l.sort, s, false, true);
  if (e != hipSuccess) return e;
  k_count_sorted<<<(unsigned)l.nb, kBinBlock, 0, s>>>(totals + 1, radix_result_in_tmp(w + l.sort), dk0, dv0, dk1,
                                                      dv1, reinterpret_cast<const uint4*>(proj.runs), sruns, sn, ss);
  k_scan_blocks<<<1, 1024, 0, s>>>(l.nb, ss, totals + 4);
  return hipGetLastError();
}

// Emission phase (the host has read P, and the workspace holds the P-sized arrays): pair
// offsets and partition starts, then the two emission passes over partitions of
// kEmitPart pairs.
hipError_t launch_bin_emit(int64_t n, int64_t P, bool large, const gs_projected& proj, int tiles_x, int tile_bits,
                           uint64_t* digit_counts, void* ws, uint64_t* keys, uint32_t* vals, hipStream_t s) {
  if (n == 0 || P == 0)
    return digit_counts ? launch_fill_u32(digit_counts, 2 * GS_TILE_DIGIT_COUNTS, 0u, s) : hipSuccess;
  const BinLayout l = bin_layout(n, P);
  char* w = static_cast<char*>(ws);
  uint64_t* ss = reinterpret_cast<uint64_t*>(w + l.sorted_sums);
  const uint64_t* vcount = reinterpret_cast<uint64_t*>(w + l.totals) + 1;
  uint64_t* goff = reinterpret_cast<uint64_t*>(w + l.goff);
  uint64_t* dtotals = reinterpret_cast<uint64_t*>(w + l.dtotals);
  uint32_t* gstart = reinterpret_cast<uint32_t*>(w + l.gstart);
  uint4* sruns = reinterpret_cast<uint4*>(w + l.sruns);
  uint32_t* sn = reinterpret_cast<uint32_t*>(w + l.sn);
  uint32_t* cnt_pre = reinterpret_cast<uint32_t*>(w + l.cnt_pre);
  uint64_t* csum = reinterpret_cast<uint64_t*>(w + l.csum);
  uint64_t* gsum = reinterpret_cast<uint64_t*>(w + l.gsum);
  // the lists of the float64 variants, only when a rectangle needs them (large): its flags
  // are cleared first; otherwise the flags stay unread and those variants are not launched
  uint32_t* pflag = large ? reinterpret_cast<uint32_t*>(w + l.flags) : nullptr;
  uint32_t* cflag = large ? pflag + l.nparts : nullptr;
  uint32_t* lcount = large ? cflag + l.nchunks : nullptr;
  uint32_t* plist = reinterpret_cast<uint32_t*>(w + l.plist);
  uint32_t* clist = reinterpret_cast<uint32_t*>(w + l.clist);
  if (large) {
    const hipError_t e = launch_fill_u32(pflag, l.nparts + l.nchunks + 2, 0u, s);
    if (e != hipSuccess) return e;
  }
  k_offsets<<<(unsigned)l.nb, kBinBlock, 0, s>>>(vcount, sn, ss, goff, gstart, pflag, cflag, plist, clist, lcount);
  // digit passes of the pair sort above the low byte (tile ids have at most 24 bits)
  const int hp = digit_counts ? (tile_bits > 8 ? (tile_bits - 1) / 8 : 0) : 0;
  uint64_t* dcopies = reinterpret_cast<uint64_t*>(w + l.dcopies);
  const float4* rec = reinterpret_cast<const float4*>(proj.rec);
  // a chunk / partition holding a Gaussian with a large rectangle runs in the large
  // variant (small persistent grids over the lists k_offsets built), every other one in
  // the common variant
  const uint2* table = reinterpret_cast<const uint2*>(proj.rows);
  k_emit_count<<<(unsigned)l.nchunks, kBinBlock, 0, s>>>(vcount, P, l.nparts, sruns, table, cflag, goff, gstart,
                                                         tiles_x, cnt_pre, csum, hp, dcopies);
  if (large)
    k_emit_count_large<<<(unsigned)min(l.nchunks, (int64_t)kLargeGrid), kBinBlock, 0, s>>>(
        vcount, P, l.nparts, sruns, table, rec, clist, lcount, goff, gstart, tiles_x, cnt_pre, csum, hp, dcopies);
  k_group_scan<<<(unsigned)l.ngroups, kBinBlock, 0, s>>>(l.nchunks, csum, gsum);
  k_digit_scan<<<kDigits, kBinBlock, 0, s>>>(l.ngroups, gsum, dtotals, dcopies, digit_counts);
  k_emit_scatter<<<(unsigned)l.nparts, kBinBlock, 0, s>>>(vcount, P, l.nparts, sruns, table, pflag, goff, gstart,
                                                          tiles_x, cnt_pre, csum, gsum, dtotals, keys, vals);
  if (large)
    k_emit_scatter_large<<<(unsigned)min(l.nparts, (int64_t)kLargeGrid), kBinBlock, 0, s>>>(
        vcount, P, l.nparts, sruns, table, rec, plist, lcount, goff, gstart, tiles_x, cnt_pre, csum, gsum, dtotals,
        keys, vals);
  return hipGetLastError();
}

}  // namespace gs
