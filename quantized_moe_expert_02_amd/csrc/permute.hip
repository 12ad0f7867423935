// Token-to-expert grouping: a stable counting sort of the (token, slot) pairs.
//
// The grouped expert GEMM walks a compact list of the tiles the routed
// segments actually hold, not a grid sized by the longest segment (gitee
// "dgpp" README, "Execution and performance", engine.expert_tile_list).  The
// segments are built here deterministically: counts come from per-chunk
// histograms (LDS integer atomics, order-free), offsets from a scan, and each
// pair's rank in its segment from a scan over chunks plus an in-order rank
// within the chunk, so the permutation is the same on every run.
#include "moe_launch.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void hist_kernel(const int* __restrict__ ids, int P, int E,
                                                   int* __restrict__ hist) {
  __shared__ int cnt[kMaxExperts];
  const int b = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += 256) cnt[e] = 0;
  __syncthreads();
  const int p0 = b * kPermChunk, p1 = min(P, p0 + kPermChunk);
  for (int p = p0 + threadIdx.x; p < p1; p += 256) {
    const int e = ids[p];
    if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);  // out-of-range ids are dropped
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) hist[(size_t)b * E + e] = cnt[e];
}

// Block-wide exclusive scan of one int per thread (1024 threads).
__device__ int block_exclusive_scan(int v, int* tmp, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  if (wave == 0) {  // exclusive scan of the (at most 16) wavefront totals by lane shuffles
    const int nw = (int)(blockDim.x >> 6);
    const int s = (lane < nw) ? tmp[lane] : 0;
    int y = s;
    for (int d = 1; d < 16; d <<= 1) {
      const int z = __shfl_up(y, d, 64);
      if (lane >= d) y += z;
    }
    if (lane < nw) tmp[lane] = y - s;
    if (lane == nw - 1) tmp[16] = y;
  }
  __syncthreads();
  const int r = tmp[wave] + x - v;
  total = tmp[16];
  __syncthreads();
  return r;
}

// One block of 1024 threads, thread e owns expert e (E <= 1024).
__global__ __launch_bounds__(1024) void scan_kernel(int NB, int E, int* __restrict__ hist,
                                                    int* __restrict__ counts,
                                                    int* __restrict__ offsets,
                                                    int* __restrict__ act, int* __restrict__ n_act,
                                                    int tile_m, int2* __restrict__ tiles,
                                                    int* __restrict__ n_tiles, int max_tiles,
                                                    int from_offsets) {
  __shared__ int tmp[17];
  const int e = threadIdx.x;
  int c = 0;
  if (from_offsets) {
    if (e < E) c = offsets[e + 1] - offsets[e];
  } else if (e < E) {
    // hist[b][e] becomes the rank of chunk b's first pair within expert e.
    // The loads of a batch (one per chunk, coalesced across the experts of a
    // wavefront) are issued before its stores, which may alias them, so a
    // batch costs one memory round trip: the 80 chunks of 8192 x 10 pairs
    // take one.
    constexpr int kB = 96;
    for (int b0 = 0; b0 < NB; b0 += kB) {
      int h[kB];
#pragma unroll
      for (int j = 0; j < kB; ++j) h[j] = (b0 + j < NB) ? hist[(size_t)(b0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        if (b0 + j < NB) {
          hist[(size_t)(b0 + j) * E + e] = c;
          c += h[j];
        }
      }
    }
    counts[e] = c;
  }
  int total;
  const int off = block_exclusive_scan(e < E ? c : 0, tmp, total);
  if (!from_offsets) {
    if (e < E) offsets[e] = off;  // the scatter adds it to the chunk ranks
    if (e == 0) offsets[E] = total;
  }
  // active experts in increasing id order
  int nact;
  const int ai = block_exclusive_scan((e < E && c > 0) ? 1 : 0, tmp, nact);
  if (e < E && c > 0) act[ai] = e;
  if (e == 0) *n_act = nact;
  if (tiles != nullptr) {
    const int nt_e = (e < E) ? (c + tile_m - 1) / tile_m : 0;
    int ntot;
    const int t0 = block_exclusive_scan(nt_e, tmp, ntot);
    const int base = (e < E) ? (from_offsets ? offsets[e] : off) : 0;
    for (int i = 0; i < nt_e; ++i)
      if (t0 + i < max_tiles) tiles[t0 + i] = make_int2(e, base + i * tile_m);
    if (e == 0) *n_tiles = ntot < max_tiles ? ntot : max_tiles;
  }
}

// One workgroup per chunk, four wavefronts of 256 consecutive pairs each:
// the wavefronts count their segments' experts, each expert's count is turned
// into the segment's first position (chunk base, then the earlier segments
// in order), and every wavefront ranks its pairs 64 at a time in order.
constexpr int kScatterWaves = 4;
constexpr int kScatterSeg = kPermChunk / kScatterWaves;

__global__ __launch_bounds__(kWave * kScatterWaves) void scatter_kernel(
    const int* __restrict__ ids, int P, int E, const int* __restrict__ rank0,
    const int* __restrict__ offsets, int* __restrict__ perm_to_pair, int* __restrict__ pair_to_perm) {
  __shared__ int cnt[kScatterWaves][kMaxExperts];
  const int b = blockIdx.x, lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  for (int i = threadIdx.x; i < kScatterWaves * kMaxExperts; i += kWave * kScatterWaves)
    (&cnt[0][0])[i] = 0;
  __syncthreads();
  const int p0 = b * kPermChunk + wave * kScatterSeg, p1 = min(P, p0 + kScatterSeg);
  constexpr int kIt = kScatterSeg / kWave;
  int my[kIt];
#pragma unroll
  for (int i = 0; i < kIt; ++i) {
    const int p = p0 + kWave * i + lane;
    const int e = (p < p1) ? ids[p] : -1;
    my[i] = ((unsigned)e < (unsigned)E) ? e : -1;
    if (my[i] >= 0) atomicAdd(&cnt[wave][my[i]], 1);
  }
  __syncthreads();
  // first position of each segment's pairs of expert e
  for (int e = threadIdx.x; e < E; e += kWave * kScatterWaves) {
    int pos = offsets[e] + rank0[(size_t)b * E + e];
#pragma unroll
    for (int w = 0; w < kScatterWaves; ++w) {
      const int n = cnt[w][e];
      cnt[w][e] = pos;
      pos += n;
    }
  }
  __syncthreads();
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int* const c = cnt[wave];
#pragma unroll
  for (int i = 0; i < kIt; ++i) {
    const int p = p0 + kWave * i + lane;
    const int e = my[i];
    const bool valid = e >= 0;
    // lanes holding the same expert id
    uint64_t same = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const uint64_t m = __ballot(valid && ((e >> bit) & 1));
      same &= ((e >> bit) & 1) ? m : ~m;
    }
    const int rank = __popcll(same & lt);
    const int pos = valid ? c[e] + rank : 0;
    __builtin_amdgcn_wave_barrier();  // every lane has read its counter
    if (valid) {
      perm_to_pair[pos] = p;
      pair_to_perm[p] = pos;
      // the last lane of each group advances the counter
      if ((same >> lane) == 1ull) c[e] = pos + 1;
    } else if (p < p1) {
      pair_to_perm[p] = -1;  // a dropped pair (expert id out of range)
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");  // the counters, before the next reads
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace

hipError_t launch_permute(const int* ids, int T, int k, int E, int* counts, int* offsets,
                          int* perm_to_pair, int* pair_to_perm, int* hist, int* act, int* n_act,
                          int tile_m, int* tiles, int* n_tiles, int max_tiles, hipStream_t s) {
  const PermPlan pp = perm_plan(T, k);
  hipError_t e = launch(hist_kernel, dim3(pp.NB), dim3(256), 0, s, ids, pp.P, E, hist);
  if (e != hipSuccess) return e;
  e = launch(scan_kernel, dim3(1), dim3(1024), 0, s, pp.NB, E, hist, counts, offsets, act, n_act,
             tile_m, reinterpret_cast<int2*>(tiles), n_tiles, max_tiles, 0);
  if (e != hipSuccess) return e;
  return launch(scatter_kernel, dim3(pp.NB), dim3(kWave * kScatterWaves), 0, s, ids, pp.P, E, hist,
                offsets, perm_to_pair, pair_to_perm);
}

hipError_t launch_groups_from_offsets(const int* offsets, int E, int* act, int* n_act, int tile_m,
                                      int* tiles, int* n_tiles, int max_tiles, hipStream_t s) {
  return launch(scan_kernel, dim3(1), dim3(1024), 0, s, 0, E, nullptr, nullptr,
                const_cast<int*>(offsets), act, n_act, tile_m, reinterpret_cast<int2*>(tiles),
                n_tiles, max_tiles, 1);
}

}  // namespace moe
