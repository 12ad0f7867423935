// Router logits and certified top-k for gfx950.
//
// The pages keep the router outside the quantized path (one served model
// keeps its router BF16: "DGPP" README mirror, supported-models notes on
// DeepSeek-V4-Flash) and print no router function.  The layer here uses a
// softmax router over fp32 router weights, top-k with ties to the lower
// expert id, outputs in descending logit order.
//
// Exactness of the selection.  Routing is decided on the exact logit rounded
// once to float64.  The fast path sums exact float64 products per slice of
// router rows, rounds each slice sum to fp32 and adds the slices in float64;
// its error is below 2^-23 * sum_h |x_h||w_he| (+|b_e|).  The top-k kernel
// accepts the fast order when every adjacent gap among the top k+1 exceeds
// twice that bound; otherwise it recomputes the contested logits with a
// compensated (double-float64) sum and decides on those.  Large batches
// compute the fast logits on the matrix cores instead (router_gemm.hip),
// with a bound of their own; the top-k below serves both.
#include "moe_launch.h"
#include "topk_core.cuh"

namespace moe {

RouterPlan router_plan(int T, int H, int E) {
  RouterPlan p;
  // Up to kRouterSlicedRows tokens: 128-row slices, so that the (slice x 32
  // experts x 8 tokens) blocks fill the chip; the top-k adds the slices.
  // Larger batches (which take this router only when H is too large for the
  // matrix-core one): one slice, each block summing the whole contraction.
  p.RH = (T <= kRouterSlicedRows) ? 128 : H;
  p.RS = (H + p.RH - 1) / p.RH;
  p.CS = (E + kRouterCols - 1) / kRouterCols;
  return p;
}

namespace {

constexpr int kXStage = 256;

__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const float* __restrict__ wr, int T,
                                                            int H, int E, int RH,
                                                            float* __restrict__ part,
                                                            float* __restrict__ amax) {
  const int rs = blockIdx.x, cs = blockIdx.y, tg = blockIdx.z;
  const int col = threadIdx.x & 31, rg = threadIdx.x >> 5;  // 8 row groups
  const int e = cs * kRouterCols + col;
  const int t0 = tg * kRouterTokens;
  const int nt = min(kRouterTokens, T - t0);
  const int h0 = rs * RH, h1 = min(H, h0 + RH);
  const int CS = gridDim.y;

  __shared__ float xs[kRouterTokens][kXStage];
  __shared__ double red[8][kRouterTokens][kRouterCols];
  __shared__ float reda[8][kRouterTokens][kRouterCols];

  double acc[kRouterTokens];
  float aa[kRouterTokens];
#pragma unroll
  for (int t = 0; t < kRouterTokens; ++t) {
    acc[t] = 0.0;
    aa[t] = 0.f;
  }
  for (int hc = h0; hc < h1; hc += kXStage) {
    const int n = min(kXStage, h1 - hc);
    __syncthreads();
    for (int i = threadIdx.x; i < kRouterTokens * kXStage; i += 256) {
      const int t = i / kXStage, h = i % kXStage;
      xs[t][h] = (t < nt && h < n) ? bf16_to_f32(x[(size_t)(t0 + t) * H + hc + h]) : 0.f;
    }
    __syncthreads();
    if (e < E) {
      for (int h = rg; h < n; h += 8) {
        const float w = wr[(size_t)(hc + h) * E + e];
        const double wd = w;
        const float wa = fabsf(w);
#pragma unroll
        for (int t = 0; t < kRouterTokens; ++t) {
          // bf16 * fp32 is exact in float64; one rounding per addition.
          acc[t] = fma(static_cast<double>(xs[t][h]), wd, acc[t]);
          aa[t] = fmaf(fabsf(xs[t][h]), wa, aa[t]);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kRouterTokens; ++t) {
    red[rg][t][col] = acc[t];
    reda[rg][t][col] = aa[t];
  }
  __syncthreads();
  if (rg == 0) {
    for (int t = 0; t < nt; ++t) {
      double sum = 0.0;
      float a = 0.f;
      for (int g = 0; g < 8; ++g) {
        sum += red[g][t][col];
        a += reda[g][t][col];
      }
      if (e < E) part[((size_t)rs * T + t0 + t) * E + e] = static_cast<float>(sum);
      // per-token maximum over this block's columns (lanes 0..31 of wave 0)
      for (int m = 16; m >= 1; m >>= 1) a = fmaxf(a, __shfl_xor(a, m, 32));
      if (col == 0) amax[((size_t)rs * CS + cs) * T + t0 + t] = a;
    }
  }
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a) {
  __shared__ BlockTopkSmem sm;
  __shared__ float amax_w[kTopkThreads / kWave];
  __shared__ float bias_w[kTopkThreads / kWave];
  const int t = blockIdx.x, E = a.E;
  if (a.mode == 0) {
    for (int e = threadIdx.x; e < E; e += blockDim.x)
      sm.v[e] = static_cast<double>(a.part[(size_t)t * E + e]);
  } else {
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
      double l = 0.0;
      for (int r = 0; r < a.RS; ++r) l += static_cast<double>(a.part[((size_t)r * a.T + t) * E + e]);
      if (a.bias != nullptr) l += static_cast<double>(a.bias[e]);
      sm.v[e] = l;
      if (a.logits_out != nullptr) a.logits_out[(size_t)t * E + e] = static_cast<float>(l);
    }
  }
  // Error bound of the fast logits (mode 1): the router kernel's per-block
  // factors (amax) times its scale; see TopkArgs.  Each slice's fp32
  // rounding errs by at most 2^-24 of that slice's sum of |x||w|, so the
  // bound adds, over slices, the maximum over column blocks.
  float m = 0.f;
  if (a.mode == 1) {
    for (int r = threadIdx.x; r < a.RS; r += blockDim.x) {
      float mr = 0.f;
      for (int c = 0; c < a.CS; ++c) mr = fmaxf(mr, a.amax[((size_t)r * a.CS + c) * a.T + t]);
      m += mr;
    }
  }
  m = wave_sum_f(m);
  float mb = 0.f;
  if (a.mode == 1 && a.bias != nullptr)
    for (int e = threadIdx.x; e < E; e += blockDim.x) mb = fmaxf(mb, fabsf(a.bias[e]));
  mb = wave_max_f(mb);
  if ((threadIdx.x & (kWave - 1)) == 0) {
    amax_w[threadIdx.x / kWave] = m;
    bias_w[threadIdx.x / kWave] = mb;
  }
  __syncthreads();
  float am = 0.f, bm = 0.f;
  for (int i = 0; i < (int)(blockDim.x / kWave); ++i) {
    am += amax_w[i];
    bm = fmaxf(bm, bias_w[i]);
  }
  am += bm;
  // The sum over slices of the max over column blocks bounds every expert
  // of the token; max |bias| is added as a safe over-estimate of the float64
  // bias addition.
  BlockTopkArgs ta;
  ta.E = E;
  ta.k = a.k;
  ta.renorm = a.renorm;
  ta.bound = (a.mode == 1) ? static_cast<double>(am) * a.bound_scale + a.bound_abs : 0.0;
  ta.certify = a.mode == 1;
  ta.xrow = a.x ? a.x + (size_t)t * a.H : nullptr;
  ta.wr = a.wr;
  ta.bias = a.bias;
  ta.H = a.H;
  ta.ids = a.ids + (size_t)t * a.k;
  ta.w = a.w + (size_t)t * a.k;
  block_topk(sm, ta);
}

// Large batches: one wavefront per token, kWaveTopkTokens tokens per block.
// Only wave-level synchronisation is used, so a wave past the last token can
// leave early.
constexpr int kWaveTopkTokens = 4;

// NP: logits per lane, a power of two >= ceil(E / 64).  LDS (sized at launch
// by topk_wave_lds): per wavefront 64 * NP float64 logits, then the
// wavefronts' scratch; every slot a loop below can touch is inside it.
template <int NP>
__global__ __launch_bounds__(kWave * kWaveTopkTokens) void topk_wave_kernel(TopkArgs a) {
  extern __shared__ __align__(16) unsigned char topk_lds[];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  double* const vals = reinterpret_cast<double*>(topk_lds);
  WaveTopkScratch* const scratch = reinterpret_cast<WaveTopkScratch*>(
      topk_lds + sizeof(double) * kWaveTopkTokens * kWave * NP);
  const int t = blockIdx.x * kWaveTopkTokens + wave;
  if (t >= a.T) return;
  const int E = a.E;
  double* v = vals + (size_t)wave * kWave * NP;
  float m = 0.f;
  // All of a lane's loads (logits, offsets, bounds) are issued before any of
  // the stores below, which the compiler must otherwise assume may alias
  // them (one memory round trip per value).
  float pv[NP], bv[NP];
  const bool has_bias = a.mode != 0 && a.bias != nullptr;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int e = lane + kWave * i;
    const bool on = e < E;
    pv[i] = on ? a.part[(size_t)t * E + e] : 0.f;
    bv[i] = (on && has_bias) ? a.bias[e] : 0.f;
  }
  float am = 0.f;
  if (a.mode != 0) {
    for (int c = lane; c < a.CS; c += kWave) am = fmaxf(am, a.amax[(size_t)c * a.T + t]);
  }
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int e = lane + kWave * i;
    if (e >= E) continue;
    double l = static_cast<double>(pv[i]);
    if (has_bias) {  // mode 1: one slice plus the expert offset
      l += static_cast<double>(bv[i]);
      m = fmaxf(m, fabsf(bv[i]));
    }
    v[e] = l;
    if (a.mode != 0 && a.logits_out != nullptr) a.logits_out[(size_t)t * E + e] = static_cast<float>(l);
  }
  m = fmaxf(m, am);
  m = wave_max_f(m);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  TopkToken tk;
  tk.vals = v;
  tk.E = E;
  tk.k = a.k;
  tk.renorm = a.renorm;
  tk.bound = (a.mode == 1) ? static_cast<double>(m) * a.bound_scale + a.bound_abs : 0.0;
  tk.certify = a.mode == 1;
  tk.xrow = a.x ? a.x + (size_t)t * a.H : nullptr;
  tk.wr = a.wrt;
  tk.wr_sh = 1;
  tk.wr_se = (size_t)a.H;
  tk.bias = a.bias;
  tk.H = a.H;
  tk.ids = a.ids + (size_t)t * a.k;
  tk.w = a.w + (size_t)t * a.k;
  tk.recomputed = a.recomputed ? a.recomputed + t : nullptr;
  tk.sc = scratch + wave;
  wave_topk(tk);
}

// Token-table routing: one wavefront per token; lane j < k takes table entry
// j of the token's row; weights are the softmax (float64) of the logits at
// the selected experts (renormalised over them, or the full softmax
// gathered).  A token id outside [0, V) gives ids -1 and weights 0; an entry
// outside [0, E) gets weight 0 and no part in the normalisation.
constexpr int kTableTokens = 4;

__global__ __launch_bounds__(kWave * kTableTokens) void table_route_kernel(
    const int* __restrict__ tok, const int* __restrict__ table, int V, int T, int k, int E,
    const float* __restrict__ logits, int renorm, int* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * kTableTokens + (int)(threadIdx.x / kWave);
  if (t >= T) return;  // a whole wavefront leaves together
  const int v = tok[t];
  const bool tok_ok = (unsigned)v < (unsigned)V;
  int e = -1;
  if (lane < k && tok_ok) e = table[(size_t)v * k + lane];
  const bool ok = (unsigned)e < (unsigned)E;
  const float* lrow = logits + (size_t)t * E;
  const double l = ok ? static_cast<double>(lrow[e]) : 0.0;
  double m;
  double denom = 0.0;
  if (renorm) {
    m = ok ? l : -INFINITY;
    for (int s = 32; s >= 1; s >>= 1) m = fmax(m, __shfl_xor(m, s, kWave));
    double z = ok ? exp(l - m) : 0.0;
    denom = z;
    for (int s = 32; s >= 1; s >>= 1) denom += __shfl_xor(denom, s, kWave);
  } else {
    m = -INFINITY;
    for (int i = lane; i < E; i += kWave) m = fmax(m, static_cast<double>(lrow[i]));
    for (int s = 32; s >= 1; s >>= 1) m = fmax(m, __shfl_xor(m, s, kWave));
    for (int i = lane; i < E; i += kWave) denom += exp(static_cast<double>(lrow[i]) - m);
    for (int s = 32; s >= 1; s >>= 1) denom += __shfl_xor(denom, s, kWave);
  }
  if (lane < k) {
    ids[(size_t)t * k + lane] = tok_ok ? e : -1;
    const double wj = (ok && denom > 0.0) ? exp(l - m) / denom : 0.0;
    w[(size_t)t * k + lane] = static_cast<float>(wj);
  }
}

}  // namespace

hipError_t launch_table_route(const int* tok, const int* table, int V, int T, int k, int E,
                              const float* logits, int renorm, int* ids, float* w,
                              hipStream_t s) {
  if (k > kWave) return hipErrorInvalidValue;
  return launch(table_route_kernel, dim3((T + kTableTokens - 1) / kTableTokens),
                dim3(kWave * kTableTokens), 0, s, tok, table, V, T, k, E, logits, renorm, ids, w);
}

hipError_t launch_router_logits(const uint16_t* x, const float* wr, int T, int H, int E,
                                const RouterPlan& rp, float* part, float* amax, hipStream_t s) {
  dim3 grid(rp.RS, rp.CS, (T + kRouterTokens - 1) / kRouterTokens);
  return launch(router_logits_kernel, grid, dim3(256), 0, s, x, wr, T, H, E, rp.RH, part, amax);
}

template <int NP>
hipError_t launch_topk_wave(const TopkArgs& a, hipStream_t s) {
  const size_t lds = kWaveTopkTokens * (sizeof(double) * kWave * NP + sizeof(WaveTopkScratch));
  return launch(topk_wave_kernel<NP>, dim3((a.T + kWaveTopkTokens - 1) / kWaveTopkTokens),
                dim3(kWave * kWaveTopkTokens), lds, s, a);
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.wave) {
    if (a.mode == 1 && (a.RS != 1 || a.wrt == nullptr)) return hipErrorInvalidValue;
    if (a.E < 1 || a.E > kMaxExperts) return hipErrorInvalidValue;
    const int nper = (a.E + kWave - 1) / kWave;
    if (nper <= 1) return launch_topk_wave<1>(a, s);
    if (nper <= 2) return launch_topk_wave<2>(a, s);
    if (nper <= 4) return launch_topk_wave<4>(a, s);
    if (nper <= 8) return launch_topk_wave<8>(a, s);
    return launch_topk_wave<kMaxPerLane>(a, s);
  }
  return launch(topk_kernel, dim3(a.T), dim3(kTopkThreads), 0, s, a);
}

}  // namespace moe
