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
// compensated (double-float64) sum and decides on those.
#include <climits>

#include "moe_launch.h"

namespace moe {

RouterPlan router_plan(int T, int H, int E) {
  RouterPlan p;
  // Decode sizes: many slices so that a few hundred workgroups stream the
  // router weights once.  Prefill: one slice (the partial is the full sum).
  p.RH = (T <= kRouterTokens) ? 128 : H;
  if (p.RH > H) p.RH = H;
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

// Selection key: class 2 = a number (incl. +-inf), 1 = NaN, 0 = not eligible.
__device__ __forceinline__ bool better(int ca, double va, int ia, int cb, double vb, int ib) {
  if (ca != cb) return ca > cb;
  if (ca == 2 && va != vb) return va > vb;
  return ia < ib;
}

__device__ __forceinline__ void two_sum(double a, double b, double& s, double& err) {
  s = a + b;
  const double bp = s - a;
  const double ap = s - bp;
  err = (a - ap) + (b - bp);
}

// Compensated float64 logit of expert e for one token (whole wave).
__device__ double dd_logit(const uint16_t* __restrict__ xrow, const float* __restrict__ wr, int H,
                           int E, int e, const float* bias) {
  const int lane = __lane_id();
  double s = 0.0, c = 0.0;
  for (int h = lane; h < H; h += kWave) {
    const double p = static_cast<double>(bf16_to_f32(xrow[h])) *
                     static_cast<double>(wr[(size_t)h * E + e]);
    double err;
    two_sum(s, p, s, err);
    c += err;
  }
  // Pairwise combine; both lanes of a pair compute the same values, so every
  // lane ends with the same result.
  for (int m = 1; m < kWave; m <<= 1) {
    const double os = __shfl_xor(s, m, kWave);
    const double oc = __shfl_xor(c, m, kWave);
    double err;
    two_sum(s, os, s, err);
    c = (c + oc) + err;
  }
  if (bias != nullptr) {
    double err;
    two_sum(s, static_cast<double>(bias[e]), s, err);
    c += err;
  }
  return s + c;
}

constexpr int kEPL = kMaxExperts / kWave;  // logits per lane

__global__ __launch_bounds__(256) void topk_kernel(TopkArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  (void)wave;
  if (t >= a.T) return;  // no block-level barrier below: waves are independent
  const int E = a.E, k = a.k;

  double v[kEPL];
  uint32_t nanmask = 0;
#pragma unroll
  for (int i = 0; i < kEPL; ++i) {
    const int e = lane + kWave * i;
    double val = 0.0;
    if (e < E) {
      if (a.mode == 0) {
        val = static_cast<double>(a.part[(size_t)t * E + e]);
      } else {
        for (int r = 0; r < a.RS; ++r) val += static_cast<double>(a.part[((size_t)r * a.T + t) * E + e]);
        if (a.bias != nullptr) val += static_cast<double>(a.bias[e]);
        if (a.logits_out != nullptr) a.logits_out[(size_t)t * E + e] = static_cast<float>(val);
      }
      if (val != val) nanmask |= 1u << i;
    }
    v[i] = val;
  }

  // Error bound of the fast logits (mode 1).
  double bound = 0.0;
  if (a.mode == 1) {
    float sum = 0.f;
    for (int r = 0; r < a.RS; ++r) {
      float m = 0.f;
      for (int c = lane; c < a.CS; c += kWave) m = fmaxf(m, a.amax[((size_t)r * a.CS + c) * a.T + t]);
      sum += wave_max_f(m);
    }
    float bm = 0.f;
    if (a.bias != nullptr)
      for (int e = lane; e < E; e += kWave) bm = fmaxf(bm, fabsf(a.bias[e]));
    sum += wave_max_f(bm);
    bound = static_cast<double>(sum) * 0x1p-23;
  }

  uint32_t excluded = 0;  // lanes' experts not eligible (after a recompute)
  // Lane r keeps the r-th selected (value, id, class).
  double top_v = 0.0;
  int top_i = 0, top_c = 0;
  auto select = [&](int rounds) -> int {
    uint32_t sel = 0;
    int got = 0;
    for (int r = 0; r < rounds; ++r) {
      int bc = 0, bi = INT_MAX;
      double bv = 0.0;
#pragma unroll
      for (int i = 0; i < kEPL; ++i) {
        const int e = lane + kWave * i;
        if (e < E && !((sel >> i) & 1u) && !((excluded >> i) & 1u)) {
          const int c = ((nanmask >> i) & 1u) ? 1 : 2;
          if (better(c, v[i], e, bc, bv, bi)) {
            bc = c;
            bv = v[i];
            bi = e;
          }
        }
      }
      for (int m = 32; m >= 1; m >>= 1) {
        const int oc = __shfl_xor(bc, m, kWave);
        const double ov = __shfl_xor(bv, m, kWave);
        const int oi = __shfl_xor(bi, m, kWave);
        if (better(oc, ov, oi, bc, bv, bi)) {
          bc = oc;
          bv = ov;
          bi = oi;
        }
      }
      if (bc == 0) break;
      if ((bi & (kWave - 1)) == lane) sel |= 1u << (bi / kWave);
      if (lane == r) {
        top_v = bv;
        top_i = bi;
        top_c = bc;
      }
      ++got;
    }
    return got;
  };

  const int K1 = (k + 1 <= E) ? k + 1 : k;
  const int got = select(a.mode == 1 ? K1 : k);

  if (a.mode == 1) {
    // Lane r < got-1 checks the gap between the r-th and (r+1)-th values.
    const double next_v = __shfl_down(top_v, 1, kWave);
    const bool fin_r = (lane >= got) || (top_c == 2 && (top_v - top_v == 0.0));
    const bool finite = __all(fin_r);
    const bool gap_ok = (lane + 1 >= got) || (top_v - next_v > 2.0 * bound);
    const bool ok = (got == K1) && finite && __all(gap_ok);
    if (a.recomputed != nullptr && lane == 0) a.recomputed[t] = ok ? 0 : 1;
    if (!ok) {
      // Every exact top-k member has a fast logit >= (k-th fast value) - 2*bound.
      const double thr = __shfl(top_v, k - 1, kWave) - 2.0 * bound;
      const uint16_t* xrow = a.x + (size_t)t * a.H;
      for (int i = 0; i < kEPL; ++i) {
        const int e = lane + kWave * i;
        const bool cand = (e < E) && (!finite || (!((nanmask >> i) & 1u) && v[i] >= thr));
        if (e < E && !cand) excluded |= 1u << i;
        uint64_t mask = __ballot(cand);
        while (mask) {
          const int l = __builtin_ctzll(mask);
          mask &= mask - 1;
          const double val = dd_logit(xrow, a.wr, a.H, E, l + kWave * i, a.bias);
          if (lane == l) {
            v[i] = val;
            if (val != val) nanmask |= 1u << i;
            else nanmask &= ~(1u << i);
          }
        }
      }
      select(k);
    }
  }

  // Weights: softmax over the k selected (renormalised) or over all E.
  const double v0 = __shfl(top_v, 0, kWave);
  double z = 0.0;
  if (lane < k) z = exp(top_v - v0);
  double denom;
  if (a.renorm) {
    denom = z;
    for (int m = 32; m >= 1; m >>= 1) denom += __shfl_xor(denom, m, kWave);
  } else {
    double part = 0.0;
#pragma unroll
    for (int i = 0; i < kEPL; ++i) {
      const int e = lane + kWave * i;
      if (e < E) part += exp(v[i] - v0);
    }
    denom = part;
    for (int m = 32; m >= 1; m >>= 1) denom += __shfl_xor(denom, m, kWave);
  }
  if (lane < k) {
    a.ids[(size_t)t * k + lane] = top_i;
    a.w[(size_t)t * k + lane] = static_cast<float>(z / denom);
  }
}

}  // namespace

hipError_t launch_router_logits(const uint16_t* x, const float* wr, int T, int H, int E,
                                const RouterPlan& rp, float* part, float* amax, hipStream_t s) {
  dim3 grid(rp.RS, rp.CS, (T + kRouterTokens - 1) / kRouterTokens);
  return launch(router_logits_kernel, grid, dim3(256), 0, s, x, wr, T, H, E, rp.RH, part, amax);
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  dim3 grid((a.T + 3) / 4);
  return launch(topk_kernel, grid, dim3(256), 0, s, a);
}

}  // namespace moe
