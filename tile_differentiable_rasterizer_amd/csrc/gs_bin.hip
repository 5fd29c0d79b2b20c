// gs_bin.hip -- duplication of Gaussians into (tile | depth) keys, for gfx950.
//
// "Better Gaussian Splatting in Julia" (lshu.cn) s3.2 (assign_to_tiles) and
// "Implementing Better Gaussian Splatting in Julia" (pwwt.cn) s4.3 (16x16 tiles): each
// visible Gaussian is listed once in every tile its support rectangle covers.  The
// 32-bit index wrap section of "Training 10M Gaussians in 8 GB: Spirula Studio's VRAM
// efficiency" (mhpq.cn) is why every count and offset here is 64-bit.
//
// Three kernels:
//   k_count_blocks   per 1024 Gaussians: the sum of n_tiles (wavefront reductions)
//   k_scan_blocks    one workgroup: exclusive scan of those sums and the total P
//   k_emit           per 1024 Gaussians: in-LDS exclusive scan of n_tiles, then every
//                    lane writes consecutive output pairs (found by binary search over
//                    the scanned offsets), so the 12 B/pair stores are fully coalesced
//                    and a Gaussian covering many tiles is spread over many lanes.
#include "gs_device.h"

namespace gs {

constexpr int kBinBlock = 256;
constexpr int kBinPer = 4;                       // Gaussians per thread
constexpr int kBinChunk = kBinBlock * kBinPer;   // Gaussians per workgroup

__global__ __launch_bounds__(kBinBlock) void k_count_blocks(int64_t n, const uint32_t* __restrict__ n_tiles,
                                                            uint64_t* __restrict__ block_sums) {
  __shared__ uint64_t s_w[kBinBlock / kWave];
  const int64_t base = (int64_t)blockIdx.x * kBinChunk;
  uint64_t acc = 0;
#pragma unroll
  for (int j = 0; j < kBinPer; ++j) {
    const int64_t i = base + j * kBinBlock + threadIdx.x;
    if (i < n) acc += n_tiles[i];
  }
  acc = wave_sum(acc);
  if (__lane_id() == 0) s_w[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t t = 0;
#pragma unroll
    for (int w = 0; w < kBinBlock / kWave; ++w) t += s_w[w];
    block_sums[blockIdx.x] = t;
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

__global__ __launch_bounds__(kBinBlock) void k_emit(int64_t n, const uint32_t* __restrict__ n_tiles,
                                                    const ushort4* __restrict__ rect,
                                                    const float* __restrict__ depth,
                                                    const uint64_t* __restrict__ block_off, int tiles_x,
                                                    uint64_t* __restrict__ keys, uint32_t* __restrict__ vals) {
  __shared__ uint64_t s_off[kBinChunk + 1];  // exclusive offsets relative to the block
  __shared__ uint64_t s_w[kBinBlock / kWave];
  const int64_t base = (int64_t)blockIdx.x * kBinChunk;
  const int tid = threadIdx.x, lane = __lane_id(), wave = tid / kWave;
  // each thread owns kBinPer consecutive Gaussians
  uint32_t cnt[kBinPer];
  uint64_t tsum = 0;
#pragma unroll
  for (int j = 0; j < kBinPer; ++j) {
    const int64_t i = base + (int64_t)tid * kBinPer + j;
    cnt[j] = i < n ? n_tiles[i] : 0u;
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
  const int ng = (int)min((int64_t)kBinChunk, n - base);
  for (uint64_t p = tid; p < total; p += kBinBlock) {
    // last Gaussian g with s_off[g] <= p (n_tiles[g] > 0 guaranteed by p < s_off[g+1])
    int lo = 0, hi = ng;  // invariant: s_off[lo] <= p < s_off[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_off[mid] <= p) lo = mid; else hi = mid;
    }
    const int64_t g = base + lo;
    const uint32_t local = (uint32_t)(p - s_off[lo]);
    const ushort4 r = rect[g];
    const uint32_t w = (uint32_t)r.y - (uint32_t)r.x + 1u;
    const uint32_t row = local / w;
    const uint32_t tx = (uint32_t)r.x + (local - row * w);
    const uint32_t ty = (uint32_t)r.z + row;
    const uint64_t tile = (uint64_t)ty * (uint64_t)tiles_x + tx;
    keys[out0 + p] = (tile << 32) | (uint64_t)__float_as_uint(depth[g]);
    vals[out0 + p] = (uint32_t)g;
  }
}

size_t bin_workspace_bytes(int64_t n) {
  const int64_t nb = (n + kBinChunk - 1) / kBinChunk;
  return (size_t)(nb + 2) * sizeof(uint64_t);
}

// Phase 1: block sums, their scan and P (device).  ws: [nb] block offsets, then total.
hipError_t launch_bin_count(int64_t n, const uint32_t* n_tiles, void* ws, hipStream_t s) {
  const int64_t nb = (n + kBinChunk - 1) / kBinChunk;
  uint64_t* sums = static_cast<uint64_t*>(ws);
  uint64_t* total = sums + nb;
  if (nb > 0) {
    k_count_blocks<<<(unsigned)nb, kBinBlock, 0, s>>>(n, n_tiles, sums);
  }
  k_scan_blocks<<<1, 1024, 0, s>>>(nb, sums, total);
  return hipGetLastError();
}

uint64_t* bin_total_ptr(int64_t n, void* ws) {
  const int64_t nb = (n + kBinChunk - 1) / kBinChunk;
  return static_cast<uint64_t*>(ws) + nb;
}

// Phase 2: write the pairs.
hipError_t launch_bin_emit(int64_t n, const gs_projected& proj, int tiles_x, const void* ws,
                           uint64_t* keys, uint32_t* vals, hipStream_t s) {
  const int64_t nb = (n + kBinChunk - 1) / kBinChunk;
  if (nb == 0) return hipSuccess;
  k_emit<<<(unsigned)nb, kBinBlock, 0, s>>>(n, proj.n_tiles, reinterpret_cast<const ushort4*>(proj.rect),
                                           proj.depth, static_cast<const uint64_t*>(ws), tiles_x, keys,
                                           vals);
  return hipGetLastError();
}

}  // namespace gs
