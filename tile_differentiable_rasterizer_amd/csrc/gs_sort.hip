// gs_sort.hip -- stable LSD radix sort of (tile | depth) keys with single-pass
// ("onesweep") digit passes, and per-tile range extraction, for gfx950.
//
// "Better Gaussian Splatting in Julia" (lshu.cn) s3.2 (sort_by_depth!) and
// "Implementing Better Gaussian Splatting in Julia" (pwwt.cn) s3.3: each tile's list is
// ordered by the depth of the Gaussian centres.  Sorting the 64-bit key tile << 32 |
// bits(depth) orders by tile, then depth (positive floats order like their bit patterns);
// the sort is stable, so pairs emitted in Gaussian-id order keep id order among equal keys.
//
// Structure (the decoupled look-back scheme of Merrill & Garland, and the single-pass radix
// sort of Adinets & Merrill, re-designed for 64-wide wavefronts):
//   k_sort_hist   one read of the keys: histograms of every 8-bit digit at once (skipped
//                 when the caller has the digit counts, as the binning does for its pairs)
//   k_sort_plan   exclusive scan of each histogram (global digit bases); marks digits that
//                 are constant over all keys (those passes are skipped unless the caller
//                 needs every pass) and assigns the ping-pong buffers on the device, so no
//                 host round trip is needed.  Not launched when the counts are given and
//                 every pass is kept: the passes then scan the counts themselves
//   k_onesweep    per pass: each 1024-lane workgroup takes a 4096-key partition by atomic
//                 ticket, ranks its keys stably (wavefront ballots match equal digits;
//                 per-wave digit counters in LDS, advanced with pipelined LDS atomics),
//                 publishes per-digit counts and resolves its global offsets by looking
//                 back over earlier partitions' published counts (several earlier
//                 partitions per round trip), reorders the partition in LDS by digit and
//                 writes each digit's run contiguously; the last pass of a pair sort also
//                 records each tile's first and last positions (atomic maxima at the two
//                 ends of each run of equal tiles in the partition)
//   k_sort_copy   moves the result back to keys/vals after an odd number of passes, for
//                 callers that need it there
//   k_ranges      [first, last + 1) of every tile from the sorted keys, where no pass ran
//                 or where a pair sort's result is moved back to keys/vals on the way
//   k_tile_order  decodes the recorded starts, and orders the tiles by decreasing list
//                 length
#include "gs_device.h"

namespace gs {

// Records the kernel timer's event for a digit pass of a 64-bit key sort when the timer is
// armed for those passes (defined with the timer, in the API).
void mark_sort_pass(hipStream_t s);

constexpr int kHistThreads = 1024;                  // histogram workgroup: 16 wavefronts
constexpr int kSortKPT = 4;                         // keys per thread of the histogram
constexpr int kSortPart = kHistThreads * kSortKPT;  // keys per histogram round
// Onesweep partition and workgroup sizes, by key width: with more lanes each holds fewer
// keys, and the ranking (a chain of dependent ballots per key) has more wavefronts per
// SIMD to interleave.
constexpr int kOnesweepPart32 = 4096, kOnesweepPart64 = 4096;
constexpr int kOnesweepThreads32 = 1024, kOnesweepThreads64 = 1024;
template <typename K>
struct Onesweep {
  static constexpr int threads = sizeof(K) == 8 ? kOnesweepThreads64 : kOnesweepThreads32;
  static constexpr int part = sizeof(K) == 8 ? kOnesweepPart64 : kOnesweepPart32;
  static constexpr int kpt = part / threads;
};
constexpr int kMinPart = kOnesweepPart32 < kOnesweepPart64 ? kOnesweepPart32 : kOnesweepPart64;
constexpr int kRadix = 256;
constexpr int kMaxPasses = 8;
constexpr int kHistCopies = 16;                   // global histogram copies (spreads the atomics)

// Workspace layout (bytes from the workspace start).
struct SortLayout {
  size_t hist, base, plan, tickets, status, total;
  int64_t parts;
};

SortLayout sort_layout(int64_t n_pairs, int passes) {
  SortLayout l;
  l.parts = (n_pairs + kMinPart - 1) / kMinPart;  // enough status rows for either key width
  l.hist = 0;
  l.base = l.hist + sizeof(uint64_t) * kHistCopies * kMaxPasses * kRadix;
  l.plan = l.base + sizeof(uint64_t) * kMaxPasses * kRadix;
  l.tickets = l.plan + 256;
  l.status = l.tickets + 256;
  l.total = l.status + sizeof(uint64_t) * (size_t)passes * (size_t)l.parts * kRadix;
  return l;
}

// The key count of a sort: *dcount when the count lives on the device (then Pmax, which
// sizes the grids and the workspace, bounds it), else Pmax itself.
__device__ __forceinline__ int64_t sort_count(int64_t Pmax, const uint64_t* dcount) {
  if (!dcount) return Pmax;
  const uint64_t c = *dcount;
  return c < (uint64_t)Pmax ? (int64_t)c : Pmax;
}

__global__ void k_fill_u32(uint32_t* __restrict__ p, int64_t count, uint32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

hipError_t launch_fill_u32(void* p, int64_t count, uint32_t v, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  const int64_t want = (count + 255) / 256;
  const unsigned blocks = (unsigned)(want < 4096 ? want : 4096);
  k_fill_u32<<<blocks, 256, 0, s>>>(static_cast<uint32_t*>(p), count, v);
  return hipGetLastError();
}

// plan[p] = -1 (skip), 0 (keys -> tmp) or 1 (tmp -> keys); plan[kMaxPasses] = buffer
// holding the result (0 = keys, 1 = tmp).  With keep_all no pass is skipped (a pass over a
// constant digit moves the keys unchanged), so the result's buffer follows from the pass
// count alone and the host knows it.  Global digit bases: base[p][d] = exclusive scan of
// pass p's histogram, the sum of `copies` copies kMaxPasses * kRadix words apart (pass p's
// counts at p * kRadix in each).  Run by one workgroup of kRadix threads.
__device__ __forceinline__ void sort_plan(const uint64_t* __restrict__ hist, int copies, uint64_t* __restrict__ base,
                                          int32_t* __restrict__ plan, int passes, uint64_t P, int keep_all) {
  __shared__ uint64_t s_w[kRadix / kWave];
  const int tid = threadIdx.x, lane = __lane_id(), wave = tid / kWave;
  int cur = 0;
  for (int p = 0; p < passes; ++p) {
    uint64_t h = 0;
    if (copies == kHistCopies) {
#pragma unroll
      for (int c = 0; c < kHistCopies; ++c) h += hist[c * kMaxPasses * kRadix + p * kRadix + tid];
    } else {
      for (int c = 0; c < copies; ++c) h += hist[c * kMaxPasses * kRadix + p * kRadix + tid];
    }
    const uint64_t inc = wave_inclusive_scan(h);
    if (lane == kWave - 1) s_w[wave] = inc;
    __syncthreads();
    uint64_t pre = inc - h;
    for (int w = 0; w < wave; ++w) pre += s_w[w];
    base[p * kRadix + tid] = pre;
    const bool trivial = __syncthreads_or(h == P) != 0 && !keep_all;
    if (tid == 0) plan[p] = trivial ? -1 : cur;
    if (!trivial) cur ^= 1;
  }
  if (tid == 0) plan[kMaxPasses] = cur;
}

template <typename K>
__global__ __launch_bounds__(kHistThreads) void k_sort_hist(const K* __restrict__ keys, int64_t Pmax,
                                                          const uint64_t* __restrict__ dcount, int lo, int passes,
                                                          uint64_t* __restrict__ hist) {
  const int64_t P = sort_count(Pmax, dcount);
  // one LDS histogram per wavefront (atomics from different wavefronts never collide),
  // passes * kRadix words each: the launch sizes the LDS by the pass count
  extern __shared__ uint32_t s_hist[];
  const int wave = threadIdx.x / kWave;
  uint32_t* s_hw = s_hist + wave * passes * kRadix;
  for (int i = threadIdx.x; i < (kHistThreads / kWave) * passes * kRadix; i += kHistThreads) s_hist[i] = 0;
  __syncthreads();
  for (int64_t b = (int64_t)blockIdx.x * kSortPart; b < P; b += (int64_t)gridDim.x * kSortPart) {
    K k[kSortKPT];  // all loads in flight before the first atomic
#pragma unroll
    for (int j = 0; j < kSortKPT; ++j) {
      const int64_t i = b + j * kHistThreads + threadIdx.x;
      k[j] = i < P ? keys[i] : (K)0;
    }
#pragma unroll
    for (int j = 0; j < kSortKPT; ++j) {
      if (b + j * kHistThreads + threadIdx.x >= P) break;
      const uint64_t kk = (uint64_t)k[j] >> lo;
      for (int p = 0; p < passes; ++p) atomicAdd(&s_hw[p * kRadix + ((kk >> (8 * p)) & 0xFF)], 1u);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < passes * kRadix; i += kHistThreads) {
    uint32_t c = 0;
#pragma unroll
    for (int w = 0; w < kHistThreads / kWave; ++w) c += s_hist[w * passes * kRadix + i];
    // workgroup b adds into copy b % kHistCopies, so no address sees more than
    // 1/kHistCopies of the workgroups' atomics
    if (c)
      atomicAdd(reinterpret_cast<unsigned long long*>(&hist[(blockIdx.x % kHistCopies) * kMaxPasses * kRadix + i]),
                (unsigned long long)c);
  }
}

__global__ __launch_bounds__(kRadix) void k_sort_plan(const uint64_t* __restrict__ hist, int copies,
                                                      uint64_t* __restrict__ base, int32_t* __restrict__ plan,
                                                      int passes, int64_t Pmax, const uint64_t* __restrict__ dcount,
                                                      int keep_all) {
  sort_plan(hist, copies, base, plan, passes, (uint64_t)sort_count(Pmax, dcount), keep_all);
}


// At most 64 VGPRs (8 waves per SIMD), so that two 1024-lane workgroups share a CU (their
// LDS fits); with more registers only one would run.
template <typename K>
__global__ __launch_bounds__(Onesweep<K>::threads, 8) void k_onesweep(
    K* __restrict__ k0, uint32_t* __restrict__ v0, K* __restrict__ k1, uint32_t* __restrict__ v1,
    int64_t Pmax, const uint64_t* __restrict__ dcount, int pass, int shift, int bits,
    const int32_t* __restrict__ plan, int mode_arg, const uint64_t* __restrict__ dbase,
    const uint64_t* __restrict__ counts, int copies, int32_t* __restrict__ result_word,
    uint64_t* __restrict__ status, uint32_t* __restrict__ tickets, int64_t* __restrict__ tile_ranges,
    int64_t num_tiles, int write_keys) {
  // the buffers this pass reads and writes: given by the host when it knows them (no pass
  // skipped), else from the plan, which also marks passes to skip.  With write_keys = 0
  // (the last pass of a sort whose caller needs the ids only) the keys are not written.
  const int mode = mode_arg >= 0 ? mode_arg : plan[pass];
  if (mode < 0) return;  // digit constant over all keys: nothing to do
  const K* kin = mode ? k1 : k0;
  const uint32_t* vin = mode ? v1 : v0;
  K* kout = mode ? k0 : k1;
  uint32_t* vout = mode ? v0 : v1;
  const uint32_t dmask = (1u << bits) - 1u;
  constexpr int kNT = Onesweep<K>::threads, kKPT = Onesweep<K>::kpt, kPart = Onesweep<K>::part;
  constexpr int kWaves = kNT / kWave;
  static_assert(kNT >= kRadix && kPart % kNT == 0, "one thread per digit, whole keys per lane");

  __shared__ K s_keys[kPart];
  __shared__ uint32_t s_vals[kPart];
  __shared__ uint32_t s_wh[kWaves][kRadix];  // per-wave digit counters, then offsets
  __shared__ uint32_t s_lbase[kRadix];       // partition-local digit starts
  __shared__ uint64_t s_gbase[kRadix];       // global digit starts for this partition
  __shared__ uint32_t s_w[kRadix / kWave];
  __shared__ uint64_t s_cw[kRadix / kWave];
  __shared__ uint32_t s_part;

  const int tid = threadIdx.x, lane = __lane_id(), wave = tid / kWave;
  const bool owner = tid < kRadix;         // thread d < kRadix owns digit d
  const int nd = 1 << bits;                // digits of this pass: the status words' stride
  const bool live = owner && tid < nd;     // a digit keys can have
  const int64_t P = sort_count(Pmax, dcount);
  if (tid == 0) s_part = atomicAdd(tickets + pass, 1u);
  for (int i = tid; i < kWaves * kRadix; i += kNT) (&s_wh[0][0])[i] = 0;
  // with the digit counts given (the sum of `copies` copies, kMaxPasses * kRadix words
  // apart), the digit bases are their exclusive scan, computed with the partition's own
  // digit scan below; the loads are issued now and complete behind the ranking
  uint64_t cnt = 0;
  if (counts && live) {
    if (copies == kHistCopies) {
#pragma unroll
      for (int c = 0; c < kHistCopies; ++c) cnt += counts[c * kMaxPasses * kRadix + tid];
    } else {
      for (int c = 0; c < copies; ++c) cnt += counts[c * kMaxPasses * kRadix + tid];
    }
  }
  // without a plan, the last pass records which buffer holds the result
  if (result_word && blockIdx.x == 0 && tid == 0) *result_word = mode ? 0 : 1;
  __syncthreads();
  const int64_t part = s_part;
  const int64_t base = part * kPart;
  // a grid sized for Pmax keys: tickets past the last partition of P keys have no work
  // (tickets go out in order, so every partition below them is taken)
  if (base >= P) return;
  // start the look-back now: the predecessor's word for this thread's digit is usually
  // final by the time this partition has ranked its keys
  uint64_t early = live && part > 0 ? status_load(status + (part - 1) * nd + tid) : 0;
  uint64_t my_dbase = owner && !counts ? dbase[tid] : 0;  // this thread's digit's global base

  // wave-striped: wave w owns keys [w * 64 kKPT, (w + 1) * 64 kKPT) of the partition, in order
  K key[kKPT];
  uint32_t val[kKPT];
  uint32_t rank[kKPT];
#pragma unroll
  for (int j = 0; j < kKPT; ++j) {
    const int64_t idx = base + wave * (kKPT * kWave) + j * kWave + lane;
    key[j] = idx < P ? kin[idx] : (K)~(K)0;
    val[j] = idx < P ? vin[idx] : 0u;
  }
  // rank stably: lanes holding equal digits are matched by ballots; the lowest of them adds
  // the group's size to the wavefront's counter for that digit and gets the count before
  // it.  LDS atomics of one wavefront run in issue order, so the kKPT rounds pipeline
  // without waiting on each other, and a shuffle then hands each lane its group's base.
  uint32_t prev[kKPT];
  int lead[kKPT];
#pragma unroll
  for (int j = 0; j < kKPT; ++j) {
    const int64_t idx = base + wave * (kKPT * kWave) + j * kWave + lane;
    const bool valid = idx < P;
    const uint32_t d = (uint32_t)(key[j] >> shift) & dmask;
    const uint64_t m = match_digit(d, bits, __ballot(valid));
    const uint64_t lower = m & lanemask_lt();
    rank[j] = (uint32_t)__popcll(lower);
    lead[j] = valid ? (int)__builtin_ctzll(m) : lane;
    prev[j] = 0;
    if (valid && lower == 0) prev[j] = atomicAdd(&s_wh[wave][d], (uint32_t)__popcll(m));
  }
#pragma unroll
  for (int j = 0; j < kKPT; ++j) rank[j] += (uint32_t)__shfl((int)prev[j], lead[j], kWave);
  __syncthreads();

  // digit owners: wave offsets, publish the partition's count, partition-local exclusive
  // scan over digits
  const int d = tid;
  uint64_t* my_status = status + part * nd + d;
  uint32_t tot = 0, inc = 0;
  if (owner) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t c = s_wh[w][d];
      s_wh[w][d] = tot;
      tot += c;
    }
    if (live) status_store(my_status, (part == 0 ? kFlagPre : kFlagAgg) | (uint64_t)tot);
    inc = wave_inclusive_scan(tot);
    if (lane == kWave - 1) s_w[wave] = inc;
    if (counts) {
      const uint64_t cinc = wave_inclusive_scan(cnt);
      if (lane == kWave - 1) s_cw[wave] = cinc;
      my_dbase = cinc - cnt;
    }
  }
  __syncthreads();
  if (owner) {
    uint32_t pre = inc - tot;
    for (int w = 0; w < wave; ++w) pre += s_w[w];
    s_lbase[d] = pre;
    if (counts)
      for (int w = 0; w < wave; ++w) my_dbase += s_cw[w];
  }
  __syncthreads();
  // reorder the partition by digit in LDS (stable)
#pragma unroll
  for (int j = 0; j < kKPT; ++j) {
    const int64_t idx = base + wave * (kKPT * kWave) + j * kWave + lane;
    if (idx < P) {
      const uint32_t dd = (uint32_t)(key[j] >> shift) & dmask;
      const uint32_t pos = s_lbase[dd] + s_wh[wave][dd] + rank[j];
      s_keys[pos] = key[j];
      s_vals[pos] = val[j];
    }
  }
  // look back over earlier partitions for this digit's global offset
  if (owner) {
    uint64_t excl = 0;
    if (live && part > 0) {
      excl = lookback_exclusive(status + d, nd, part, early);
      status_store(my_status, kFlagPre | (excl + tot));
    }
    s_gbase[d] = my_dbase + excl;
  }
  __syncthreads();
  // write each digit's run contiguously
  const int nvalid = (int)min((int64_t)kPart, P - base);
  for (int i = tid; i < nvalid; i += kNT) {
    const K k = s_keys[i];
    const uint32_t dd = (uint32_t)(k >> shift) & dmask;
    const uint64_t g = s_gbase[dd] + (uint64_t)(i - (int)s_lbase[dd]);
    if (g < (uint64_t)P) {  // always, given exact digit counts; caller-supplied ones are not trusted
      if (write_keys) kout[g] = k;
      vout[g] = s_vals[i];
      if constexpr (sizeof(K) == 8) {
        // the last pass of a pair sort: the partition is in final order here, so a tile's
        // first and last pairs anywhere in the output start and end runs of its tile in
        // some partition.  The largest run end is the tile's end; the smallest run start
        // is recorded as the largest complement, so that cleared words (0) stay below
        // every position and an empty tile keeps 0.
        if (tile_ranges) {
          const uint64_t t = (uint64_t)k >> 32;
          if (t < (uint64_t)num_tiles) {
            if (i == 0 || ((uint64_t)s_keys[i - 1] >> 32) != t)
              atomicMax(reinterpret_cast<unsigned long long*>(tile_ranges + 2 * t), ~(unsigned long long)g);
            if (i + 1 == nvalid || ((uint64_t)s_keys[i + 1] >> 32) != t)
              atomicMax(reinterpret_cast<unsigned long long*>(tile_ranges + 2 * t + 1), (unsigned long long)(g + 1));
          }
        }
      }
    }
  }
}

template <typename K>
__global__ void k_sort_copy(const int32_t* __restrict__ plan, const K* __restrict__ k1,
                            const uint32_t* __restrict__ v1, K* __restrict__ k0, uint32_t* __restrict__ v0,
                            int64_t Pmax, const uint64_t* __restrict__ dcount) {
  if (plan[kMaxPasses] == 0) return;
  const int64_t P = sort_count(Pmax, dcount);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < P; i += (int64_t)gridDim.x * blockDim.x) {
    k0[i] = k1[i];
    v0[i] = v1[i];
  }
}

// Four consecutive keys per thread; a tile's first and last positions are where its id
// differs from the neighbour's.  The sorted pairs are read from (src, vsrc); with kdst
// non-NULL they are also moved to (kdst, vdst) on the way.
__global__ void k_ranges(const uint64_t* __restrict__ src, const uint32_t* __restrict__ vsrc,
                         uint64_t* __restrict__ kdst, uint32_t* __restrict__ vdst, int64_t P, int64_t num_tiles,
                         int64_t* __restrict__ ranges) {
  const int64_t i0 = 4 * ((int64_t)blockIdx.x * blockDim.x + threadIdx.x);
  if (i0 >= P) return;
  // 16-byte accesses when every buffer allows them (i0 is a multiple of 4)
  const bool vec16 = ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(vsrc) |
                       reinterpret_cast<uintptr_t>(kdst) | reinterpret_cast<uintptr_t>(vdst)) & 15) == 0;
  uint64_t k[6];  // keys i0 - 1 .. i0 + 4 (~0 outside [0, P))
  k[0] = i0 > 0 ? src[i0 - 1] : ~0ull;
  if (vec16 && i0 + 4 <= P) {
    const ulonglong2 a = reinterpret_cast<const ulonglong2*>(src + i0)[0];
    const ulonglong2 c = reinterpret_cast<const ulonglong2*>(src + i0)[1];
    k[1] = a.x; k[2] = a.y; k[3] = c.x; k[4] = c.y;
    k[5] = i0 + 4 < P ? src[i0 + 4] : ~0ull;
  } else {
#pragma unroll
    for (int j = 0; j < 5; ++j) k[j + 1] = i0 + j < P ? src[i0 + j] : ~0ull;
  }
  if (kdst) {
    if (vec16 && i0 + 4 <= P) {  // 16-byte moves
      reinterpret_cast<ulonglong2*>(kdst + i0)[0] = make_ulonglong2(k[1], k[2]);
      reinterpret_cast<ulonglong2*>(kdst + i0)[1] = make_ulonglong2(k[3], k[4]);
      reinterpret_cast<uint4*>(vdst + i0)[0] = reinterpret_cast<const uint4*>(vsrc + i0)[0];
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (i0 + j < P) {
          kdst[i0 + j] = k[j + 1];
          vdst[i0 + j] = vsrc[i0 + j];
        }
      }
    }
  }
#pragma unroll
  for (int j = 1; j <= 4; ++j) {
    const int64_t i = i0 + j - 1;
    const uint64_t t = k[j] >> 32;
    if (i >= P || t >= (uint64_t)num_tiles) continue;
    if ((k[j - 1] >> 32) != t) ranges[2 * t] = i;
    if ((k[j + 1] >> 32) != t) ranges[2 * t + 1] = i + 1;
  }
}

// tile_order: tile ids by decreasing list length (counting sort over 128 buckets, four per
// octave; order inside a bucket is arbitrary).  The compositing kernels take tiles in this
// order so that the longest lists start first.
__device__ __forceinline__ int length_bucket(int64_t len) {
  if (len < 4) return len > 0 ? (int)len : 0;
  const int lg = 63 - __clzll((unsigned long long)len);
  return min(127, 4 * lg + (int)((len >> (lg - 2)) & 3));
}

// With decode_starts the starts hold the bitwise complement of each tile's first position
// (0 for an empty tile), as the last sort pass wrote them: they are decoded in place.  With
// order NULL only that is done.
__global__ __launch_bounds__(1024) void k_tile_order(int64_t* __restrict__ ranges, int64_t num_tiles,
                                                    int decode_starts, int32_t* __restrict__ order) {
  constexpr int kPer = 8;  // tiles per thread per round, their loads all in flight together
  __shared__ uint32_t s_cnt[128];
  __shared__ uint32_t s_cur[128];
  __shared__ uint32_t s_w[2];
  const int tid = threadIdx.x, lane = __lane_id(), wave = tid / kWave;
  if (tid < 128) s_cnt[tid] = 0;
  __syncthreads();
  // a single round (num_tiles <= 8192, 1080p and below) keeps its buckets in registers
  int bk[kPer];
  for (int64_t t0 = 0; t0 < num_tiles; t0 += 1024 * kPer) {
    int64_t a[kPer], b[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int64_t t = t0 + j * 1024 + tid;
      a[j] = t < num_tiles ? ranges[2 * t] : 0;
      b[j] = t < num_tiles ? ranges[2 * t + 1] : 0;
    }
    if (decode_starts) {
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int64_t t = t0 + j * 1024 + tid;
        a[j] = a[j] ? ~a[j] : 0;
        if (t < num_tiles) ranges[2 * t] = a[j];
      }
    }
    if (!order) continue;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      bk[j] = length_bucket(b[j] - a[j]);
      if (t0 + j * 1024 + tid < num_tiles) atomicAdd(&s_cnt[bk[j]], 1u);
    }
  }
  if (!order) return;
  __syncthreads();
  // exclusive scan in decreasing bucket order: lane j of the first two wavefronts takes
  // bucket 127 - j
  uint32_t c = 0, inc = 0;
  if (tid < 128) {
    c = s_cnt[127 - tid];
    inc = wave_inclusive_scan(c);
    if (lane == kWave - 1) s_w[wave] = inc;
  }
  __syncthreads();
  if (tid < 128) s_cur[127 - tid] = inc - c + (wave == 1 ? s_w[0] : 0u);
  __syncthreads();
  const bool cached = num_tiles <= 1024 * kPer;
  for (int64_t t0 = 0; t0 < num_tiles; t0 += 1024 * kPer) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int64_t t = t0 + j * 1024 + tid;
      if (t >= num_tiles) break;
      const int bucket = cached ? bk[j] : length_bucket(ranges[2 * t + 1] - ranges[2 * t]);
      order[atomicAdd(&s_cur[bucket], 1u)] = (int32_t)t;
    }
  }
}

int sort_significant_bits(int64_t num_tiles) {
  int tb = 0;
  while (tb < 32 && ((int64_t)1 << tb) < num_tiles) ++tb;
  return 32 + tb;
}

static int radix_passes(int lo, int hi) { return hi > lo ? (hi - lo + 7) / 8 : 0; }

size_t radix_workspace_bytes(int64_t P, int lo, int hi) { return sort_layout(P, radix_passes(lo, hi)).total; }

// Stable LSD sort of (keys, vals) by key bits [lo, hi).  The result ends in keys/vals, or
// with copy_back = false in the buffer that plan[kMaxPasses] names (0 keys, 1 tmp).  With
// dcount non-NULL the key count is read on the device from *dcount, and P (which sizes
// the grids and the workspace) only bounds it, so the sort can be queued before the host
// knows the count.  With tile_ranges non-NULL (64-bit keys with the tile in the high word,
// and keep_all, so that the last pass runs) the last pass also writes into cleared ranges
// each tile's end and the complement of its start.
template <typename K>
static hipError_t radix_sort(int64_t P, const uint64_t* dcount, K* keys, uint32_t* vals, K* keys_tmp,
                             uint32_t* vals_tmp, int lo, int hi, void* ws, hipStream_t s, bool copy_back = true,
                             bool keep_all = false, const uint64_t* digit_counts = nullptr,
                             bool ws_zeroed = false, int64_t* tile_ranges = nullptr, int64_t num_tiles = 0,
                             bool ids_only = false) {
  const int passes = radix_passes(lo, hi);
  char* w = static_cast<char*>(ws);
  if (P <= 1 || passes == 0)  // nothing moves: the result is in keys/vals, as the word says
    return copy_back ? hipSuccess
                     : launch_fill_u32(w + sort_layout(0, 0).plan + sizeof(int32_t) * kMaxPasses, 1, 0u, s);
  const SortLayout l = sort_layout(P, passes);
  uint64_t* hist = reinterpret_cast<uint64_t*>(w + l.hist);
  uint64_t* dbase = reinterpret_cast<uint64_t*>(w + l.base);
  int32_t* plan = reinterpret_cast<int32_t*>(w + l.plan);
  uint32_t* tickets = reinterpret_cast<uint32_t*>(w + l.tickets);
  uint64_t* status = reinterpret_cast<uint64_t*>(w + l.status);
  // each pass's status words: one per partition and digit of that pass, packed
  int pbits[kMaxPasses];
  size_t poff[kMaxPasses], nstatus = 0;
  for (int p = 0; p < passes; ++p) {
    pbits[p] = hi - lo - 8 * p < 8 ? hi - lo - 8 * p : 8;
    poff[p] = nstatus;
    nstatus += (size_t)l.parts << pbits[p];
  }
  // with the digit counts given and every pass kept, the buffers are known without the
  // plan and the passes compute the digit bases from the counts; the last pass writes the
  // result's buffer word.  (Scanning the histogram's 16 copies in every workgroup instead
  // of once in the plan measured slower: 15.9 -> 18.8 us per 32-bit pass at 1M keys.)
  const bool planless = digit_counts && keep_all && !copy_back;
  // zero what this sort reads before writing: histograms (unless counts are given), plan,
  // tickets and the status words in use (no memset: capture-safe)
  // (ws_zeroed: the caller's previous kernel cleared radix_zero_bytes of the workspace)
  const size_t zfrom = digit_counts ? l.plan : l.hist;
  hipError_t e = hipSuccess;
  if (!ws_zeroed)
    e = launch_fill_u32(w + zfrom, (int64_t)((l.status + sizeof(uint64_t) * nstatus - zfrom) / 4), 0u, s);
  if (e != hipSuccess) return e;
  if (!digit_counts) {
    const int64_t want = (P + kSortPart - 1) / kSortPart;
    const unsigned blocks = (unsigned)(want < 2048 ? (want > 0 ? want : 1) : 2048);
    k_sort_hist<K><<<blocks, kHistThreads, sizeof(uint32_t) * (kHistThreads / kWave) * passes * kRadix, s>>>(
        keys, P, dcount, lo, passes, hist);
  }
  // counts the caller already has ([pass][digit], one copy) replace the counting read
  if (!planless)
    k_sort_plan<<<1, kRadix, 0, s>>>(digit_counts ? digit_counts : hist, digit_counts ? 1 : kHistCopies, dbase, plan,
                                     passes, P, dcount, keep_all ? 1 : 0);
  for (int p = 0; p < passes; ++p) {
    if constexpr (sizeof(K) == 8) mark_sort_pass(s);  // the kernel timer's events, when armed for it
    k_onesweep<K><<<(unsigned)((P + Onesweep<K>::part - 1) / Onesweep<K>::part), Onesweep<K>::threads, 0, s>>>(
        keys, vals, keys_tmp, vals_tmp, P, dcount, p, lo + 8 * p, pbits[p], plan, planless ? p % 2 : -1,
        dbase + p * kRadix, planless ? digit_counts + p * kRadix : nullptr, 1,
        planless && p == passes - 1 ? plan + kMaxPasses : nullptr, status + poff[p], tickets,
        p == passes - 1 ? tile_ranges : nullptr, num_tiles, ids_only && p == passes - 1 ? 0 : 1);
    if constexpr (sizeof(K) == 8) mark_sort_pass(s);
  }
  if (copy_back) {
    const int64_t want = (P + 255) / 256;
    const unsigned blocks = (unsigned)(want < 8192 ? want : 8192);
    k_sort_copy<K><<<blocks, 256, 0, s>>>(plan, keys_tmp, vals_tmp, keys, vals, P, dcount);
  }
  return hipGetLastError();
}

hipError_t radix_sort_u32(int64_t P, const uint64_t* dcount, uint32_t* keys, uint32_t* vals, uint32_t* keys_tmp,
                          uint32_t* vals_tmp, int lo, int hi, void* ws, hipStream_t s, bool copy_back, bool ws_zeroed) {
  return radix_sort<uint32_t>(P, dcount, keys, vals, keys_tmp, vals_tmp, lo, hi, ws, s, copy_back, false, nullptr,
                              ws_zeroed);
}

// The part of a sort workspace that a sort of P keys over bits [lo, hi) reads before it
// writes, and so needs cleared: [*off, *off + *len) bytes.  Histograms (only when the sort
// counts the digits itself), plan, tickets and the status words in use.
void radix_zero_span(int64_t P, int lo, int hi, bool counts_given, size_t* off, size_t* len) {
  const int passes = radix_passes(lo, hi);
  const SortLayout l = sort_layout(P, passes);
  size_t nstatus = 0;
  for (int p = 0; p < passes; ++p) nstatus += (size_t)l.parts << (hi - lo - 8 * p < 8 ? hi - lo - 8 * p : 8);
  *off = counts_given ? l.plan : l.hist;
  *len = l.status + sizeof(uint64_t) * nstatus - *off;
}
size_t radix_zero_bytes(int64_t P, int lo, int hi) {
  size_t off, len;
  radix_zero_span(P, lo, hi, false, &off, &len);
  return off + len;
}

// Two regions of 32-bit words set to zero in one launch.
__global__ void k_zero2(uint32_t* __restrict__ a, int64_t na, uint32_t* __restrict__ b, int64_t nb) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < na + nb; i += (int64_t)gridDim.x * blockDim.x) {
    if (i < na)
      a[i] = 0u;
    else
      b[i - na] = 0u;
  }
}

// Device word that a sort run with copy_back = false sets to 1 when its result is in the
// _tmp buffers (0: in keys/vals).  Its place in the workspace does not depend on the count.
const int32_t* radix_result_in_tmp(const void* ws) {
  return reinterpret_cast<const int32_t*>(static_cast<const char*>(ws) + sort_layout(0, 0).plan) + kMaxPasses;
}

size_t sort_workspace_bytes(int64_t n_pairs, int64_t num_tiles, int sorted_low_bits) {
  return radix_workspace_bytes(n_pairs, sorted_low_bits, sort_significant_bits(num_tiles));
}

// The pair sort.  No digit pass is skipped, so an odd pass count leaves the result in
// keys_tmp/vals_tmp: with result_in_tmp [host] non-NULL it stays there and the call
// reports where it is; with NULL, k_ranges moves it back to keys/vals.
hipError_t launch_sort(int64_t P, int64_t num_tiles, uint64_t* keys, uint32_t* vals, uint64_t* keys_tmp,
                       uint32_t* vals_tmp, int64_t* ranges, int32_t* order, int sorted_low_bits,
                       const uint64_t* digit_counts, int32_t* result_in_tmp, void* ws, hipStream_t s,
                       bool ids_only) {
  const int hi = sort_significant_bits(num_tiles);
  const int passes = P > 1 ? radix_passes(sorted_low_bits, hi) : 0;
  const bool in_tmp = passes % 2 == 1;
  hipError_t e = hipSuccess;
  if (passes > 0) {  // the ranges and the sort's counters and look-back words, cleared together
    size_t off, len;
    radix_zero_span(P, sorted_low_bits, hi, digit_counts != nullptr, &off, &len);
    const int64_t words = 4 * num_tiles + (int64_t)(len / 4);
    const unsigned blocks = (unsigned)min((words + 255) / 256, (int64_t)4096);
    k_zero2<<<blocks, 256, 0, s>>>(reinterpret_cast<uint32_t*>(ranges), 4 * num_tiles,
                                   reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + off), (int64_t)(len / 4));
    e = radix_sort<uint64_t>(P, nullptr, keys, vals, keys_tmp, vals_tmp, sorted_low_bits, hi, ws, s, false, true,
                             digit_counts, true, ranges, num_tiles, ids_only);
  } else {
    e = launch_fill_u32(ranges, 4 * num_tiles, 0u, s);
  }
  if (e != hipSuccess) return e;
  // the last pass wrote every tile's first and last positions; k_ranges finds them from
  // the sorted keys where nothing was sorted, or where it also moves the result back
  const bool move = in_tmp && !result_in_tmp;
  const bool recorded = passes > 0 && !move;
  if (P > 0 && !recorded)
    k_ranges<<<(unsigned)((P + 1023) / 1024), 256, 0, s>>>(in_tmp ? keys_tmp : keys, vals_tmp, move ? keys : nullptr,
                                                           move ? vals : nullptr, P, num_tiles, ranges);
  if (order || recorded) k_tile_order<<<1, 1024, 0, s>>>(ranges, num_tiles, recorded ? 1 : 0, order);
  if (result_in_tmp) *result_in_tmp = in_tmp ? 1 : 0;
  return hipGetLastError();
}

}  // namespace gs

namespace gs {

// Measurement only (gs_measure_scatter_io): lane i reads key i, id i and destination i,
// four per lane in 1024-element workgroups as a digit pass reads its partition, and
// writes the id (plus the key's low word, so that the key's load is used) to
// out[dest[i]].  Given the elements in the order a pass writes them, its time bounds what
// a pass with that read and write pattern can take.  Destinations outside [0, n) are
// skipped.
__global__ __launch_bounds__(256) void k_scatter_io(int64_t n, const uint64_t* __restrict__ keys,
                                                     const uint32_t* __restrict__ vals,
                                                     const uint32_t* __restrict__ dest, uint32_t* __restrict__ out) {
  const int64_t base = (int64_t)blockIdx.x * 1024;
  uint64_t k[4];
  uint32_t v[4], d[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t i = base + j * 256 + threadIdx.x;
    k[j] = i < n ? keys[i] : 0ull;
    v[j] = i < n ? vals[i] : 0u;
    d[j] = i < n ? dest[i] : ~0u;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if ((int64_t)d[j] < n) out[d[j]] = v[j] + (uint32_t)k[j];
}

hipError_t launch_scatter_io(int64_t n, const uint64_t* keys, const uint32_t* vals, const uint32_t* dest,
                             uint32_t* out, hipStream_t s) {
  k_scatter_io<<<(unsigned)((n + 1023) / 1024), 256, 0, s>>>(n, keys, vals, dest, out);
  return hipGetLastError();
}

}  // namespace gs
