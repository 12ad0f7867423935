// Decode lowering (T <= 8 rows) of the whole layer.
//
// Decode is a weight-streaming problem (forum thread "DGPP: a GB10-optimized
// C++/CUDA inference engine", the "Lossless bf12" post: decode kernels read
// the weights at the memory's line rate).  On gfx950 a dependent kernel in the
// same stream starts about 1.5 us after its predecessor ends, while a
// cross-workgroup hand-off inside a kernel needs an agent-scope release
// (an L2 write-back) and costs far more; so the layer runs as five short
// launches with no intra-kernel hand-off:
//
//   1. router partial sums over (128-row slice x 32 experts) blocks; extra
//      blocks compute the shared expert's gate/up + SwiGLU (it does not
//      depend on routing);
//   2. one block per token: sum the slices, select the top-k by rank counting,
//      certify it against the exact logits (recomputing near ties), weights;
//   3. each active routed expert's gate/up + SwiGLU, its weights streamed once
//      for all of its tokens (blocks are laid out per routed pair slot; the
//      block of an expert's first pair derives the expert's (token, slot)
//      pairs from the <= 256 routed ids, the others exit); extra blocks run
//      the shared expert's down projection;
//   4. each active expert's down projection;
//   5. combine: per-expert partials in fp32, in slot order, then the shared
//      expert, rounded once to bf16.
//
// Rows of h and y are indexed by pair (t*k + j), so no permutation is needed.
#include "gemv_core.cuh"
#include "topk_core.cuh"

namespace moe {
namespace {

constexpr int kRH = 128;  // router rows per slice
constexpr int kTmax = 8;  // decode rows
constexpr int kPmax = kTmax * kMaxTopK;
constexpr int kRSBatch = 16;

struct RouterSmem {
  float xs[kTmax][kRH];
  double red[8][kTmax][kRouterCols];
  float reda[8][kTmax][kRouterCols];
};

template <int SFMT>
__global__ __launch_bounds__(256) void decode_router_kernel(DecodeArgs a) {
  __shared__ union {
    RouterSmem r;
    GemvSmem<GemvShape<kOpGateUp>::WN, GemvShape<kOpGateUp>::WK, 2> g;
  } sm;
  const int nrb = a.RS * a.CS;
  if ((int)blockIdx.x >= nrb) {  // shared expert gate/up + SwiGLU
    if constexpr (SFMT != 0) {
      GemvIO io{a.x, a.hs, nullptr, a.k, kInShared, a.T};
      gemv_tile<SFMT, kOpGateUp, 1, 4>(a.sg, a.su, io, GemvRows{0, 0, a.T, nullptr, nullptr},
                                       blockIdx.x - nrb, sm.g);
    }
    return;
  }
  const int T = a.T, H = a.H, E = a.E;
  const int cs = blockIdx.x / a.RS, rs = blockIdx.x % a.RS;
  const int col = threadIdx.x & 31, rg = threadIdx.x >> 5;
  const int e = cs * kRouterCols + col;
  const int h0 = rs * kRH, nh = min(kRH, H - h0);

  // router weights first (HBM), then the activations (L2) they multiply
  float wv[kRH / 8];
#pragma unroll
  for (int j = 0; j < kRH / 8; ++j) {
    const int h = rg + 8 * j;
    wv[j] = (e < E && h < nh) ? a.wr[(size_t)(h0 + h) * E + e] : 0.f;
  }
  for (int i = threadIdx.x; i < kTmax * kRH; i += 256) {
    const int t = i / kRH, h = i % kRH;
    sm.r.xs[t][h] = (t < T && h < nh) ? bf16_to_f32(a.x[(size_t)t * H + h0 + h]) : 0.f;
  }
  __syncthreads();
  double acc[kTmax];
  float aa[kTmax];
#pragma unroll
  for (int t = 0; t < kTmax; ++t) {
    acc[t] = 0.0;
    aa[t] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < kRH / 8; ++j) {
    const int h = rg + 8 * j;
    const double wd = wv[j];
    const float wa = fabsf(wv[j]);
#pragma unroll
    for (int t = 0; t < kTmax; ++t) {
      if (t < T) {  // bf16 * fp32 is exact in float64
        acc[t] = fma(static_cast<double>(sm.r.xs[t][h]), wd, acc[t]);
        aa[t] = fmaf(fabsf(sm.r.xs[t][h]), wa, aa[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kTmax; ++t) {
    sm.r.red[rg][t][col] = acc[t];
    sm.r.reda[rg][t][col] = aa[t];
  }
  __syncthreads();
  if (rg < T && e < E) {  // thread (t = rg, col) folds the 8 row groups
    const int t = rg;
    double s = 0.0;
    float av = 0.f;
    for (int g = 0; g < 8; ++g) {
      s += sm.r.red[g][t][col];
      av += sm.r.reda[g][t][col];
    }
    a.part[((size_t)rs * T + t) * E + e] = static_cast<float>(s);
    a.apart[((size_t)rs * T + t) * E + e] = av;
  }
}

__global__ __launch_bounds__(kTopkThreads) void decode_topk_kernel(DecodeArgs a) {
  __shared__ BlockTopkSmem sm;
  __shared__ float amax_w[kTopkThreads / kWave];
  const int t = blockIdx.x, T = a.T, E = a.E;
  float amax = 0.f;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    double l = 0.0;
    float av = 0.f;
    for (int r0 = 0; r0 < a.RS; r0 += kRSBatch) {
      float pv[kRSBatch], qv[kRSBatch];
#pragma unroll
      for (int j = 0; j < kRSBatch; ++j) {  // unconditional loads: one round trip per batch
        const int r = min(r0 + j, a.RS - 1);
        pv[j] = a.part[((size_t)r * T + t) * E + e];
        qv[j] = a.apart[((size_t)r * T + t) * E + e];
      }
#pragma unroll
      for (int j = 0; j < kRSBatch; ++j) {
        if (r0 + j < a.RS) {
          l += static_cast<double>(pv[j]);
          av += qv[j];
        }
      }
    }
    if (a.bias != nullptr) {
      const float b = a.bias[e];
      l += static_cast<double>(b);
      av += fabsf(b);
    }
    sm.v[e] = l;
    if (a.logits_out != nullptr) a.logits_out[(size_t)t * E + e] = static_cast<float>(l);
    amax = fmaxf(amax, av);
  }
  amax = wave_max_f(amax);
  if ((threadIdx.x & (kWave - 1)) == 0) amax_w[threadIdx.x / kWave] = amax;
  __syncthreads();
  float am = 0.f;
  for (int i = 0; i < (int)(blockDim.x / kWave); ++i) am = fmaxf(am, amax_w[i]);
  BlockTopkArgs ta;
  ta.E = E;
  ta.k = a.k;
  ta.renorm = a.renorm;
  // fast-logit error < 2^-23 * sum|x||w| (covers the fp32 slice roundings)
  ta.bound = static_cast<double>(am) * 0x1p-23;
  ta.certify = true;
  ta.xrow = a.x + (size_t)t * a.H;
  ta.wr = a.wr;
  ta.bias = a.bias;
  ta.H = a.H;
  ta.ids = a.ids + (size_t)t * a.k;
  ta.w = a.w + (size_t)t * a.k;
  block_topk(sm, ta);
}

// Expert group of pair slot q: the expert e = ids[q] and all (token, slot)
// pairs routed to it, in pair order.  Only the first pair of each expert
// proceeds (returns false for the others), so every active expert is
// processed exactly once.  Block-wide, two barriers.
struct GroupSmem {
  int pairs[kPmax];
  int toks[kPmax];
  int wcnt[4];
  int wdup[4];
};

__device__ inline bool derive_group(const DecodeArgs& a, int q, GroupSmem& g, int& e_out, int& n_out) {
  const int P = a.T * a.k;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int e = a.ids[q];
  const int j = threadIdx.x;  // P <= 256 = blockDim
  const int my = (j < P) ? a.ids[j] : -1;
  const bool m = (j < P) && my == e;
  const uint64_t bal = __ballot(m);
  const uint64_t dup = __ballot(m && j < q);
  if (lane == 0) {
    g.wcnt[wave] = __popcll(bal);
    g.wdup[wave] = dup != 0ull;
  }
  __syncthreads();
  if (g.wdup[0] | g.wdup[1] | g.wdup[2] | g.wdup[3]) return false;
  if ((unsigned)e >= (unsigned)a.E) return false;
  int base = 0;
  for (int w = 0; w < wave; ++w) base += g.wcnt[w];
  if (m) {
    const int pos = base + __popcll(bal & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
    g.pairs[pos] = j;
    g.toks[pos] = j / a.k;
  }
  e_out = e;
  n_out = g.wcnt[0] + g.wcnt[1] + g.wcnt[2] + g.wcnt[3];
  __syncthreads();
  return true;
}

template <int RFMT, int SFMT>
__global__ __launch_bounds__(256) void decode_gateup_kernel(DecodeArgs a) {
  __shared__ union {
    GemvSmem<1, 4, 2> g;
    GemvSmem<4, 1, 1> d;
  } sm;
  __shared__ GroupSmem grp;
  const int ntiles = a.I / gemv_rows_per_block<kOpGateUp>();
  const int nrouted = a.T * a.k * ntiles;
  if ((int)blockIdx.x < nrouted) {
    const int q = blockIdx.x / ntiles, tile = blockIdx.x % ntiles;
    int e, n;
    if (!derive_group(a, q, grp, e, n)) return;
    GemvIO io{a.x, a.h, nullptr, a.k, kInList, a.T};
    gemv_tile<RFMT, kOpGateUp, 1, 4>(a.gate, a.up, io, GemvRows{e, 0, n, grp.toks, grp.pairs}, tile,
                                     sm.g);
  } else if constexpr (SFMT != 0) {  // shared expert down projection
    GemvIO io{a.hs, a.ys, nullptr, a.k, kInShared, a.T};
    gemv_tile<SFMT, kOpDown, 4, 1>(a.sd, a.sd, io, GemvRows{0, 0, a.T, nullptr, nullptr},
                                   blockIdx.x - nrouted, sm.d);
  }
}

template <int RFMT>
__global__ __launch_bounds__(256) void decode_down_kernel(DecodeArgs a) {
  __shared__ GemvSmem<4, 1, 1> sm;
  __shared__ GroupSmem grp;
  constexpr int RPB = gemv_rows_per_block<kOpDown>();
  const int ntiles = (a.H + RPB - 1) / RPB;
  const int q = blockIdx.x / ntiles, tile = blockIdx.x % ntiles;
  int e, n;
  if (!derive_group(a, q, grp, e, n)) return;
  GemvIO io{a.h, a.y, nullptr, a.k, kInList, a.T * a.k};
  gemv_tile<RFMT, kOpDown, 4, 1>(a.down, a.down, io, GemvRows{e, 0, n, grp.pairs, grp.pairs}, tile,
                                 sm);
}

// out[t] = bf16( sum_j w[t,j] * y[t*k+j] + y_shared[t] ), four columns per thread.
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  const int t = blockIdx.y;
  const int n = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (n >= a.H) return;
  f32x4 yv[kMaxTopK];
  float wv[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j < a.k) {
      wv[j] = a.w[t * a.k + j];
      yv[j] = *reinterpret_cast<const f32x4*>(a.y + (size_t)(t * a.k + j) * a.H + n);
    }
  }
  f32x4 ys = (a.ys != nullptr) ? *reinterpret_cast<const f32x4*>(a.ys + (size_t)t * a.H + n)
                               : f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j < a.k) {
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = fmaf(wv[j], yv[j][q], acc[q]);
    }
  }
  acc = acc + ys;
  *reinterpret_cast<uint2*>(a.out + (size_t)t * a.H + n) =
      make_uint2(f32_to_bf16(acc[0]) | (uint32_t(f32_to_bf16(acc[1])) << 16),
                 f32_to_bf16(acc[2]) | (uint32_t(f32_to_bf16(acc[3])) << 16));
}

template <int RFMT, int SFMT>
hipError_t launch5(const DecodeArgs& a, hipStream_t s) {
  const int nrb = a.RS * a.CS;
  const int nsg = (SFMT != 0) ? a.I_shared / gemv_rows_per_block<kOpGateUp>() : 0;
  hipError_t err = launch(decode_router_kernel<SFMT>, dim3(nrb + nsg), dim3(256), 0, s, a);
  if (err != hipSuccess) return err;
  err = launch(decode_topk_kernel, dim3(a.T), dim3(kTopkThreads), 0, s, a);
  if (err != hipSuccess) return err;
  constexpr int RPD = gemv_rows_per_block<kOpDown>();
  const int ngu = a.T * a.k * (a.I / gemv_rows_per_block<kOpGateUp>());
  const int nsd = (SFMT != 0) ? (a.H + RPD - 1) / RPD : 0;
  err = launch(decode_gateup_kernel<RFMT, SFMT>, dim3(ngu + nsd), dim3(256), 0, s, a);
  if (err != hipSuccess) return err;
  const int nd = a.T * a.k * ((a.H + RPD - 1) / RPD);
  err = launch(decode_down_kernel<RFMT>, dim3(nd), dim3(256), 0, s, a);
  if (err != hipSuccess) return err;
  return launch(decode_combine_kernel, dim3((a.H / 4 + 255) / 256, a.T), dim3(256), 0, s, a);
}

template <int RFMT>
hipError_t launch_r(int sfmt, const DecodeArgs& a, hipStream_t s) {
  switch (sfmt) {
    case 0: return launch5<RFMT, 0>(a, s);
    case FMT_NVFP4: return launch5<RFMT, FMT_NVFP4>(a, s);
    case FMT_MXFP4: return launch5<RFMT, FMT_MXFP4>(a, s);
    case FMT_FP8: return launch5<RFMT, FMT_FP8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

DecodePlan decode_plan(int T, int H, int E) {
  DecodePlan p;
  p.RS = (H + kRH - 1) / kRH;
  p.CS = (E + kRouterCols - 1) / kRouterCols;
  p.down_tiles = (H + gemv_rows_per_block<kOpDown>() - 1) / gemv_rows_per_block<kOpDown>();
  (void)T;
  return p;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  const int sfmt = a.has_shared ? a.sg.fmt : 0;
  switch (a.gate.fmt) {
    case FMT_NVFP4: return launch_r<FMT_NVFP4>(sfmt, a, s);
    case FMT_MXFP4: return launch_r<FMT_MXFP4>(sfmt, a, s);
    case FMT_FP8: return launch_r<FMT_FP8>(sfmt, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
