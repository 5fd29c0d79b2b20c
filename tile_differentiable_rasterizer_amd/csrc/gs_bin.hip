// gs_bin.hip -- duplication of Gaussians into (tile | depth) keys, for gfx950.
//
// "Better Gaussian Splatting in Julia" (lshu.cn) s3.2 (assign_to_tiles) and
// "Implementing Better Gaussian Splatting in Julia" (pwwt.cn) s4.3 (16x16 tiles): each
// visible Gaussian is listed once in every tile its support rectangle covers.  The
// 32-bit index wrap section of "Training 10M Gaussians in 8 GB: Spirula Studio's VRAM
// efficiency" (mhpq.cn) is why every count and offset here is 64-bit; its visibility
// bitmap section is the model for the wavefront-ballot compaction below.
//
// Pairs are written in depth order (ties by Gaussian id): the visible Gaussians are
// compacted (ballot + popcount per wavefront, in id order), radix-sorted once by the bit
// pattern of their fp32 depth (a stable sort, so equal depths stay in id order), and then
// expanded into their tiles.  Every tile's pairs are therefore already in (depth, id)
// order, and the pair sort only has to order the tile bits stably: 2 digit passes over
// the pairs instead of 6.
//
// Kernels:
//   k_count_blocks   per 1024 Gaussians: pair count and visible count
//   k_scan_blocks    one workgroup: exclusive scan of per-block sums, and the total
//   k_compact        visible Gaussians' (depth bits, id), in id order
//   (radix sort of the compacted depths, gs_sort.hip)
//   k_count_sorted   per 1024 depth-sorted Gaussians: pair count
//   k_emit           per 1024 depth-sorted Gaussians: in-LDS exclusive scan of n_tiles,
//                    then every lane writes consecutive output pairs (its Gaussian found by
//                    binary search over the scanned offsets), so the 12 B/pair stores are
//                    fully coalesced and a Gaussian covering many tiles is spread over
//                    many lanes.
#include "gs_device.h"

namespace gs {

hipError_t radix_sort_u32(int64_t P, uint32_t* keys, uint32_t* vals, uint32_t* keys_tmp, uint32_t* vals_tmp, int lo,
                          int hi, void* ws, hipStream_t s);
size_t radix_workspace_bytes(int64_t P, int lo, int hi);

constexpr int kBinBlock = 256;
constexpr int kBinPer = 4;                      // Gaussians per thread
constexpr int kBinChunk = kBinBlock * kBinPer;  // Gaussians per workgroup

__global__ __launch_bounds__(kBinBlock) void k_count_blocks(int64_t n, const uint32_t* __restrict__ n_tiles,
                                                            uint64_t* __restrict__ pair_sums,
                                                            uint64_t* __restrict__ vis_sums) {
  __shared__ uint64_t s_p[kBinBlock / kWave], s_v[kBinBlock / kWave];
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

// Exclusive scan of nb block sums in place; total written to *total.
__global__ __launch_bounds__(1024) void k_scan_blocks(int64_t nb, uint64_t* __restrict__ sums,
                                                      uint64_t* __restrict__ total) {
  __shared__ uint64_t s_w[16];
  __shared__ uint64_t s_carry;
  if (threadIdx.x == 0) s_carry = 0;
  __syncthreads();
  const int lane = __lane_id(), wave = threadIdx.x / kWave;
  for (int64_t off = 0; off < nb; off += 1024) {
    const int64_t i = off + threadIdx.x;
    const uint64_t x = i < nb ? sums[i] : 0;
    const uint64_t inc = wave_inclusive_scan(x);
    if (lane == kWave - 1) s_w[wave] = inc;
    __syncthreads();
    uint64_t wpre = 0;
    for (int w = 0; w < wave; ++w) wpre += s_w[w];
    const uint64_t carry = s_carry;
    if (i < nb) sums[i] = carry + wpre + inc - x;
    __syncthreads();
    if (threadIdx.x == 1023) s_carry = carry + wpre + inc;
    __syncthreads();
  }
  if (threadIdx.x == 0) *total = s_carry;
}

// Visible Gaussians' (depth bits, id) in id order.  Round r of a workgroup covers ids
// base + 256 r + [0, 256); a wavefront finds its visible lanes with one ballot.
__global__ __launch_bounds__(kBinBlock) void k_compact(int64_t n, const uint32_t* __restrict__ n_tiles,
                                                       const float* __restrict__ depth,
                                                       const uint64_t* __restrict__ vis_off,
                                                       uint32_t* __restrict__ dkeys, uint32_t* __restrict__ dvals) {
  __shared__ uint32_t s_w[kBinPer][kBinBlock / kWave];
  const int64_t base = (int64_t)blockIdx.x * kBinChunk;
  const int tid = threadIdx.x, lane = __lane_id(), wave = tid / kWave;
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

__global__ __launch_bounds__(kBinBlock) void k_count_sorted(int64_t v, const uint32_t* __restrict__ order,
                                                            const uint32_t* __restrict__ n_tiles,
                                                            uint64_t* __restrict__ sums) {
  __shared__ uint64_t s_p[kBinBlock / kWave];
  const int64_t base = (int64_t)blockIdx.x * kBinChunk;
  uint64_t acc = 0;
#pragma unroll
  for (int j = 0; j < kBinPer; ++j) {
    const int64_t i = base + j * kBinBlock + threadIdx.x;
    if (i < v) acc += n_tiles[order[i]];
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

// Expand the depth-sorted Gaussians order[0, v) into their tiles (rows outer, columns
// inner): keys[p] = tile << 32 | depth bits, vals[p] = Gaussian id.
__global__ __launch_bounds__(kBinBlock) void k_emit(int64_t v, const uint32_t* __restrict__ order,
                                                    const uint32_t* __restrict__ n_tiles,
                                                    const ushort4* __restrict__ rect,
                                                    const float* __restrict__ depth,
                                                    const uint64_t* __restrict__ block_off, int tiles_x,
                                                    uint64_t* __restrict__ keys, uint32_t* __restrict__ vals) {
  __shared__ uint64_t s_off[kBinChunk + 1];  // exclusive offsets relative to the block
  __shared__ uint32_t s_id[kBinChunk];
  __shared__ ushort4 s_rect[kBinChunk];      // the block's Gaussians, gathered once
  __shared__ uint32_t s_depth[kBinChunk];
  __shared__ uint64_t s_w[kBinBlock / kWave];
  const int64_t base = (int64_t)blockIdx.x * kBinChunk;
  const int tid = threadIdx.x, lane = __lane_id(), wave = tid / kWave;
  // each thread owns kBinPer consecutive sorted positions
  uint32_t cnt[kBinPer];
  uint64_t tsum = 0;
#pragma unroll
  for (int j = 0; j < kBinPer; ++j) {
    const int64_t i = base + (int64_t)tid * kBinPer + j;
    const uint32_t g = i < v ? order[i] : 0u;
    s_id[tid * kBinPer + j] = g;
    cnt[j] = i < v ? n_tiles[g] : 0u;
    if (i < v) {
      s_rect[tid * kBinPer + j] = rect[g];
      s_depth[tid * kBinPer + j] = __float_as_uint(depth[g]);
    }
    tsum += cnt[j];
  }
  const uint64_t inc = wave_inclusive_scan(tsum);
  if (lane == kWave - 1) s_w[wave] = inc;
  __syncthreads();
  uint64_t pre = inc - tsum;
  for (int w = 0; w < wave; ++w) pre += s_w[w];
#pragma unroll
  for (int j = 0; j < kBinPer; ++j) {
    s_off[tid * kBinPer + j] = pre;
    pre += cnt[j];
  }
  if (tid == kBinBlock - 1) s_off[kBinChunk] = pre;  // block total
  __syncthreads();
  const uint64_t total = s_off[kBinChunk];
  const uint64_t out0 = block_off[blockIdx.x];
  const int ng = (int)min((int64_t)kBinChunk, v - base);
  // each lane writes kEmitRun consecutive pairs: one binary search for the first, then walk
  // the Gaussians' tiles row by row; a wavefront's stores cover 64 * kEmitRun consecutive pairs
  constexpr int kEmitRun = 8;
  for (uint64_t chunk = 0; chunk < total; chunk += (uint64_t)kBinBlock * kEmitRun) {
    const uint64_t p0 = chunk + (uint64_t)tid * kEmitRun;
    if (p0 >= total) continue;
    int lo = 0, hi = ng;  // invariant: s_off[lo] <= p0 < s_off[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_off[mid] <= p0) lo = mid; else hi = mid;
    }
    uint32_t local = (uint32_t)(p0 - s_off[lo]);
    ushort4 r = s_rect[lo];
    uint32_t w = (uint32_t)r.y - (uint32_t)r.x + 1u;
    uint32_t row = local / w, col = local - row * w;
    uint64_t next = s_off[lo + 1];
    const int run = (int)min((uint64_t)kEmitRun, total - p0);
    for (int i = 0; i < run; ++i) {
      const uint64_t p = p0 + (uint64_t)i;
      while (p >= next) {  // on to the next Gaussian (every visible one has n_tiles > 0)
        ++lo;
        r = s_rect[lo];
        w = (uint32_t)r.y - (uint32_t)r.x + 1u;
        row = 0;
        col = 0;
        next = s_off[lo + 1];
      }
      const uint64_t tile = (uint64_t)((uint32_t)r.z + row) * (uint64_t)tiles_x + ((uint32_t)r.x + col);
      keys[out0 + p] = (tile << 32) | (uint64_t)s_depth[lo];
      vals[out0 + p] = s_id[lo];
      if (++col == w) {
        col = 0;
        ++row;
      }
    }
  }
}

// Workspace layout (bytes).
struct BinLayout {
  size_t pair_sums, vis_sums, sorted_sums, totals, dk0, dv0, dk1, dv1, sort, total;
  int64_t nb;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static BinLayout bin_layout(int64_t n) {
  BinLayout l;
  l.nb = (n + kBinChunk - 1) / kBinChunk;
  const size_t sums = align256(sizeof(uint64_t) * (size_t)(l.nb + 1));
  const size_t ids = align256(sizeof(uint32_t) * (size_t)(n > 0 ? n : 1));
  l.pair_sums = 0;
  l.vis_sums = l.pair_sums + sums;
  l.sorted_sums = l.vis_sums + sums;
  l.totals = l.sorted_sums + sums;
  l.dk0 = l.totals + 256;
  l.dv0 = l.dk0 + ids;
  l.dk1 = l.dv0 + ids;
  l.dv1 = l.dk1 + ids;
  l.sort = l.dv1 + ids;
  l.total = l.sort + align256(radix_workspace_bytes(n, 0, 32));
  return l;
}

size_t bin_workspace_bytes(int64_t n) { return bin_layout(n).total; }

// Phase 1: per-block sums, their scans, P and the visible count V (device, totals[0..1]).
hipError_t launch_bin_count(int64_t n, const uint32_t* n_tiles, void* ws, hipStream_t s) {
  const BinLayout l = bin_layout(n);
  char* w = static_cast<char*>(ws);
  uint64_t* ps = reinterpret_cast<uint64_t*>(w + l.pair_sums);
  uint64_t* vs = reinterpret_cast<uint64_t*>(w + l.vis_sums);
  uint64_t* totals = reinterpret_cast<uint64_t*>(w + l.totals);
  if (l.nb > 0) k_count_blocks<<<(unsigned)l.nb, kBinBlock, 0, s>>>(n, n_tiles, ps, vs);
  k_scan_blocks<<<1, 1024, 0, s>>>(l.nb, ps, totals);
  k_scan_blocks<<<1, 1024, 0, s>>>(l.nb, vs, totals + 1);
  return hipGetLastError();
}

uint64_t* bin_totals_ptr(int64_t n, void* ws) {
  return reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + bin_layout(n).totals);
}

// Phase 2 (after the host read P and V): compact, depth-sort, emit.
hipError_t launch_bin_emit(int64_t n, int64_t v, const gs_projected& proj, int tiles_x, void* ws, uint64_t* keys,
                           uint32_t* vals, hipStream_t s) {
  if (v == 0) return hipSuccess;
  const BinLayout l = bin_layout(n);
  char* w = static_cast<char*>(ws);
  uint32_t* dk0 = reinterpret_cast<uint32_t*>(w + l.dk0);
  uint32_t* dv0 = reinterpret_cast<uint32_t*>(w + l.dv0);
  uint32_t* dk1 = reinterpret_cast<uint32_t*>(w + l.dk1);
  uint32_t* dv1 = reinterpret_cast<uint32_t*>(w + l.dv1);
  uint64_t* ss = reinterpret_cast<uint64_t*>(w + l.sorted_sums);
  uint64_t* totals = reinterpret_cast<uint64_t*>(w + l.totals);
  k_compact<<<(unsigned)l.nb, kBinBlock, 0, s>>>(n, proj.n_tiles, proj.depth,
                                                 reinterpret_cast<const uint64_t*>(w + l.vis_sums), dk0, dv0);
  hipError_t e = radix_sort_u32(v, dk0, dv0, dk1, dv1, 0, 32, w + l.sort, s);
  if (e != hipSuccess) return e;
  const int64_t nbv = (v + kBinChunk - 1) / kBinChunk;
  k_count_sorted<<<(unsigned)nbv, kBinBlock, 0, s>>>(v, dv0, proj.n_tiles, ss);
  k_scan_blocks<<<1, 1024, 0, s>>>(nbv, ss, totals + 2);
  k_emit<<<(unsigned)nbv, kBinBlock, 0, s>>>(v, dv0, proj.n_tiles, reinterpret_cast<const ushort4*>(proj.rect),
                                             proj.depth, ss, tiles_x, keys, vals);
  return hipGetLastError();
}

}  // namespace gs
