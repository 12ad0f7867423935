// Per-token top-k selection (one wavefront per token) and small-batch
// grouping (one wavefront), shared by the standalone and fused kernels.
//
// Selection order: larger logit first, then lower expert id; NaN after every
// number.  Routing is decided on the exact logit rounded once to float64: the
// caller's fast logits come with a rigorous error bound, and when the bound
// cannot separate two adjacent entries of the top k+1, the contested logits
// are recomputed with a compensated float64 sum (products of a bf16 input and
// an fp32 router weight are exact in float64).
#pragma once
#include <climits>

#include "moe_device.cuh"

namespace moe {

// Selection key: class 2 = a number (incl. +-inf), 1 = NaN, 0 = not eligible.
__device__ __forceinline__ bool key_better(int ca, double va, int ia, int cb, double vb, int ib) {
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

// Compensated float64 logit of expert e for one token (whole wave; every lane
// returns the same value).  Router weight (h, e) is w[h*sh + e*se]: sh = E,
// se = 1 for the [H][E] layout, sh = 1, se = H for a transposed [E][H] copy.
// Each lane takes 8 consecutive h per step, and the loads of up to 4 steps
// are issued before any of them is summed, so one call waits about one
// memory round trip rather than one per step.  Needs H % 8 == 0 and, for
// sh == 1, 16-byte aligned rows of w.
__device__ __forceinline__ void dd_add(double& s, double& c, double p) {
  double err;
  two_sum(s, p, s, err);
  c += err;
}

__device__ inline double dd_logit(const uint16_t* __restrict__ xrow, const float* __restrict__ w,
                                  size_t sh, size_t se, int H, int e, const float* bias) {
  constexpr int D = 4;
  const int lane = __lane_id();
  double s = 0.0, c = 0.0;
  const float* we = w + (size_t)e * se;
  for (int hb = 0; hb < H; hb += 8 * kWave * D) {
    u32x4 xv[D];
    f32x4 w0[D], w1[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int h = hb + 8 * (lane + kWave * d);
      const bool on = h < H;
      const int hh = on ? h : 0;
      xv[d] = *reinterpret_cast<const u32x4*>(xrow + hh);
      if (sh == 1) {
        w0[d] = *reinterpret_cast<const f32x4*>(we + hh);
        w1[d] = *reinterpret_cast<const f32x4*>(we + hh + 4);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          w0[d][j] = we[(size_t)(hh + j) * sh];
          w1[d][j] = we[(size_t)(hh + 4 + j) * sh];
        }
      }
      if (!on) xv[d] = u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (hb + 8 * (lane + kWave * d) >= H) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float xl = __uint_as_float(xv[d][j] << 16);
        const float xh = __uint_as_float(xv[d][j] & 0xffff0000u);
        const float wl = (j < 2) ? w0[d][2 * j] : w1[d][2 * j - 4];
        const float wh = (j < 2) ? w0[d][2 * j + 1] : w1[d][2 * j - 3];
        dd_add(s, c, static_cast<double>(xl) * static_cast<double>(wl));
        dd_add(s, c, static_cast<double>(xh) * static_cast<double>(wh));
      }
    }
  }
  // Pairwise combine: both lanes of a pair compute identical values.
  for (int m = 1; m < kWave; m <<= 1) {
    const double os = __shfl_xor(s, m, kWave);
    const double oc = __shfl_xor(c, m, kWave);
    double err;
    two_sum(s, os, s, err);
    c = (c + oc) + err;
  }
  if (bias != nullptr) dd_add(s, c, static_cast<double>(bias[e]));
  // An infinite or NaN term makes the running sum s the IEEE result of the
  // exact sum (finite bf16 x fp32 terms cannot overflow float64), while the
  // compensation has turned NaN: return s alone then.
  return (s - s == 0.0) ? s + c : s;
}

// dd_logit for up to four experts of one token at once, with contiguous
// expert rows (w + e * se, K stride 1).  Each expert's sum takes the same
// terms in the same order as dd_logit (identical results); the x loads are
// shared and the four rows' loads are in flight together, so a batch costs
// about one memory round trip.  e[q] < 0: slot unused (out[q] = 0).
__device__ inline void dd_logits4(const uint16_t* __restrict__ xrow, const float* __restrict__ w,
                                  size_t se, int H, const int (&e)[4], const float* bias,
                                  double (&out)[4]) {
  constexpr int D = 2;  // with dd_logit's D = 4 the per-lane term order is the same
  const int lane = __lane_id();
  double s[4], c[4];
  const float* we[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    s[q] = 0.0;
    c[q] = 0.0;
    we[q] = w + (size_t)(e[q] >= 0 ? e[q] : 0) * se;
  }
  for (int hb = 0; hb < H; hb += 8 * kWave * D) {
    u32x4 xv[D];
    f32x4 w0[4][D], w1[4][D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int h = hb + 8 * (lane + kWave * d);
      const int hh = h < H ? h : 0;
      xv[d] = *reinterpret_cast<const u32x4*>(xrow + hh);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        w0[q][d] = *reinterpret_cast<const f32x4*>(we[q] + hh);
        w1[q][d] = *reinterpret_cast<const f32x4*>(we[q] + hh + 4);
      }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (hb + 8 * (lane + kWave * d) >= H) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float xl = __uint_as_float(xv[d][j] << 16);
        const float xh = __uint_as_float(xv[d][j] & 0xffff0000u);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (e[q] < 0) continue;
          const float wl = (j < 2) ? w0[q][d][2 * j] : w1[q][d][2 * j - 4];
          const float wh = (j < 2) ? w0[q][d][2 * j + 1] : w1[q][d][2 * j - 3];
          dd_add(s[q], c[q], static_cast<double>(xl) * static_cast<double>(wl));
          dd_add(s[q], c[q], static_cast<double>(xh) * static_cast<double>(wh));
        }
      }
    }
  }
  for (int m = 1; m < kWave; m <<= 1) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const double os = __shfl_xor(s[q], m, kWave);
      const double oc = __shfl_xor(c[q], m, kWave);
      double err;
      two_sum(s[q], os, s[q], err);
      c[q] = (c[q] + oc) + err;
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (e[q] < 0) {
      out[q] = 0.0;
      continue;
    }
    if (bias != nullptr) dd_add(s[q], c[q], static_cast<double>(bias[e[q]]));
    out[q] = (s[q] - s[q] == 0.0) ? s[q] + c[q] : s[q];
  }
}

struct TopkToken {
  double* vals;        // LDS, [E] logits of this token (may be overwritten)
  int E, k, renorm;
  double bound;        // error bound of vals (ignored when !certify)
  bool certify;
  const uint16_t* xrow;  // for the recompute (certify only)
  const float* wr;       // router weights, element (h, e) at wr[h*wr_sh + e*wr_se]
  size_t wr_sh, wr_se;
  const float* bias;
  int H;
  int* ids;            // [k] out
  float* w;            // [k] out
  int* recomputed;     // out flag or nullptr
  struct WaveTopkScratch* sc;  // LDS scratch of this wavefront
};

// Lanes r < rounds hold the r-th selected entry in (top_v, top_i, top_c).
__device__ inline int wave_select(const double* vals, int E, uint32_t excl, int rounds,
                                  double& top_v, int& top_i, int& top_c) {
  const int lane = __lane_id();
  const int nper = (E + kWave - 1) / kWave;
  uint32_t sel = 0;  // bit i: expert lane + 64*i selected
  int got = 0;
  for (int r = 0; r < rounds; ++r) {
    int bc = 0, bi = INT_MAX;
    double bv = 0.0;
    for (int i = 0; i < nper; ++i) {
      const int e = lane + kWave * i;
      if (e >= E || ((sel >> i) & 1u) || ((excl >> i) & 1u)) continue;
      const double v = vals[e];
      const int c = (v != v) ? 1 : 2;
      if (key_better(c, v, e, bc, bv, bi)) {
        bc = c;
        bv = v;
        bi = e;
      }
    }
    for (int m = 32; m >= 1; m >>= 1) {
      const int oc = __shfl_xor(bc, m, kWave);
      const double ov = __shfl_xor(bv, m, kWave);
      const int oi = __shfl_xor(bi, m, kWave);
      if (key_better(oc, ov, oi, bc, bv, bi)) {
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
}

// ---------------------------------------------------------------------------
// Block-wide top-k of one token by rank counting: each thread ranks its own
// experts against all others (stopping once k+1 better ones are found), so
// there is no serial round per selected expert.
// ---------------------------------------------------------------------------
constexpr int kTopkThreads = 512;

struct BlockTopkSmem {
  double v[kMaxExperts];            // logits of the token
  unsigned char excl[kMaxExperts];  // 1: not eligible (after a recompute)
  double topv[kMaxTopK + 1];
  int topi[kMaxTopK + 1];
  int topc[kMaxTopK + 1];
  int cand[kMaxExperts];
  uint64_t ckey[kMaxExperts];
  int crank[kMaxExperts];
  double dred[kTopkThreads / kWave];
  uint32_t wthr[kTopkThreads / kWave];
  int ncand;
};

// Unsigned order key of a logit: larger key = ranks earlier.  0 = not
// eligible, 1 = NaN (after every number), numbers in IEEE order with -0 == +0.
__device__ __forceinline__ uint64_t order_key(double v, bool excluded) {
  if (excluded) return 0ull;
  if (v != v) return 1ull;
  if (v == 0.0) v = 0.0;
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// f ranks before e: larger key, or equal key and lower expert id.
__device__ __forceinline__ int ranks_before(uint64_t kf, int f, uint64_t ke, int e) {
  return (kf > ke) | ((kf == ke) & (f < e));
}

// Coarse 32-bit key: the logit rounded to fp32 (a monotone map, so the k-th
// largest coarse key is the coarse key of the k-th largest logit), in the
// same class order as order_key.  Distinct logits may share a coarse key;
// the exact order among candidates is taken on order_key afterwards.
__device__ __forceinline__ uint32_t coarse_key(double v, bool excluded) {
  if (excluded) return 0u;
  if (v != v) return 1u;
  float f = static_cast<float>(v);
  if (f == 0.0f) f = 0.0f;
  const uint32_t u = __float_as_uint(f);
  return (u >> 31) ? ~u : (u | 0x80000000u);  // >= 0x007fffff (-inf) for every number
}

// Sum over the wavefront (DPP: within quads, half rows, rows, then across
// rows with the row broadcasts); the total is returned to every lane.  Lanes
// a broadcast step does not write add 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add_step(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, false));
}

__device__ __forceinline__ float dpp_sum_f(float v) {
  v = dpp_add_step<0xb1, 0xf>(v);   // quad_perm [1,0,3,2]
  v = dpp_add_step<0x4e, 0xf>(v);   // quad_perm [2,3,0,1]
  v = dpp_add_step<0x141, 0xf>(v);  // row_half_mirror
  v = dpp_add_step<0x140, 0xf>(v);  // row_mirror
  v = dpp_add_step<0x142, 0xa>(v);  // row_bcast:15 into rows 1, 3
  v = dpp_add_step<0x143, 0xc>(v);  // row_bcast:31 into rows 2, 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kWave - 1));
}

// The `rounds`-th largest of the wavefront's coarse keys (ties counted), or 0
// when fewer than `rounds` keys are nonzero: the largest t with
// #{keys >= t} >= rounds, built one bit at a time from the top.
template <int N>
__device__ __forceinline__ uint32_t wave_kth_key(const uint32_t (&c)[N], int rounds) {
  uint32_t t = 0u;
#pragma unroll 4
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = t | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) cnt += __popcll(__ballot(c[i] >= cand));
    if (cnt >= rounds) t = cand;
  }
  return t;
}

// Writes the first `rounds` entries of the order into topv/topi/topc.
// (1) Each wavefront finds its `rounds`-th largest coarse key, ties included.
// (2) The largest of these per-wavefront values, thr, is at most the coarse
//     key of the overall `rounds`-th entry (each wavefront alone has that
//     many entries at or above its value), so every member of the overall
//     first `rounds` has coarse key >= thr.
// (3) The candidates (coarse key >= thr) are ranked exactly among themselves
//     on order_key, the comparisons split across the block.
// Needs E <= 2 * blockDim.x; the caller synchronises the block afterwards.
__device__ inline void block_rank(BlockTopkSmem& sm, int E, int rounds) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int nwaves = blockDim.x / kWave;
  const int e0 = threadIdx.x, e1 = threadIdx.x + blockDim.x;
  uint32_t c[2];
  c[0] = (e0 < E) ? coarse_key(sm.v[e0], sm.excl[e0] != 0) : 0u;
  c[1] = (e1 < E) ? coarse_key(sm.v[e1], sm.excl[e1] != 0) : 0u;
  uint32_t wt;
  if (E > (int)blockDim.x) {
    wt = wave_kth_key(c, rounds);
  } else {  // one logit per thread
    const uint32_t c1[1] = {c[0]};
    wt = wave_kth_key(c1, rounds);
  }
  if (lane == 0) sm.wthr[wave] = wt;
  if (threadIdx.x == 0) sm.ncand = 0;
  __syncthreads();
  uint32_t thr = 0u;
  for (int w = 0; w < nwaves; ++w) thr = max(thr, sm.wthr[w]);
  if (thr == 0u) thr = 1u;  // fewer than `rounds` eligible in every wave: all eligible
  // candidates, compacted per wavefront with one LDS atomic each
  const bool q0 = c[0] >= thr, q1 = c[1] >= thr;
  const uint64_t b0 = __ballot(q0), b1 = __ballot(q1);
  const int n0 = __popcll(b0), n = n0 + __popcll(b1);
  int base = 0;
  if (lane == 0 && n > 0) base = atomicAdd(&sm.ncand, n);
  base = __builtin_amdgcn_readfirstlane(base);
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  if (q0) {
    const int slot = base + __popcll(b0 & lt);
    sm.cand[slot] = e0;
    sm.ckey[slot] = order_key(sm.v[e0], false);
    sm.crank[slot] = 0;
  }
  if (q1) {
    const int slot = base + n0 + __popcll(b1 & lt);
    sm.cand[slot] = e1;
    sm.ckey[slot] = order_key(sm.v[e1], false);
    sm.crank[slot] = 0;
  }
  __syncthreads();
  const int nc = sm.ncand;
  if (nc <= (int)blockDim.x) {
    // each candidate's comparisons split over blockDim / nc threads
    const int segs = max(1, (int)blockDim.x / max(nc, 1));
    const int len = (nc + segs - 1) / segs;
    if ((int)threadIdx.x < nc * segs) {
      const int i = threadIdx.x % nc, sgm = threadIdx.x / nc;
      const int e = sm.cand[i];
      const uint64_t ke = sm.ckey[i];
      const int j1 = min(nc, (sgm + 1) * len);
      int cnt = 0;
      for (int j = sgm * len; j < j1; ++j) cnt += ranks_before(sm.ckey[j], sm.cand[j], ke, e);
      if (cnt) atomicAdd(&sm.crank[i], cnt);
    }
  } else {  // more candidates than threads (massive ties): each thread ranks several
    for (int i = threadIdx.x; i < nc; i += blockDim.x) {
      const int e = sm.cand[i];
      const uint64_t ke = sm.ckey[i];
      int cnt = 0;
      for (int j = 0; j < nc; ++j) cnt += ranks_before(sm.ckey[j], sm.cand[j], ke, e);
      sm.crank[i] = cnt;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nc; i += blockDim.x) {
    const int r = sm.crank[i];
    if (r < rounds) {
      const int e = sm.cand[i];
      sm.topv[r] = sm.v[e];
      sm.topi[r] = e;
      sm.topc[r] = (sm.ckey[i] == 1ull) ? 1 : 2;
    }
  }
}

struct BlockTopkArgs {
  int E, k, renorm;
  double bound;  // error bound of the logits (used when certify)
  bool certify;
  const uint16_t* xrow;
  const float* wr;
  const float* bias;
  int H;
  int* ids;  // [k]
  float* w;  // [k]
};

// sm.v must hold the token's logits and be visible to the whole block.
__device__ inline void block_topk(BlockTopkSmem& sm, const BlockTopkArgs& a) {
  const int E = a.E, k = a.k;
  const int K1 = (k + 1 <= E) ? k + 1 : k;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int nwaves = blockDim.x / kWave;
  for (int e = threadIdx.x; e < E; e += blockDim.x) sm.excl[e] = 0;
  __syncthreads();
  block_rank(sm, E, a.certify ? K1 : k);
  __syncthreads();
  if (a.certify) {
    int bad = 0;
    if ((int)threadIdx.x < K1) {
      const int r = threadIdx.x;
      const double vr = sm.topv[r];
      if (sm.topc[r] != 2 || !(vr - vr == 0.0)) bad = 2;  // non-finite or NaN among the top k+1
      else if (r + 1 < K1 && !(vr - sm.topv[r + 1] > 2.0 * a.bound)) bad = 1;
    }
    const int any_bad = __syncthreads_or(bad);
    if (any_bad) {
      // A non-finite bound (possible overflow in the fast sum) says nothing
      // about any logit: recompute all of them.
      const int all = __syncthreads_or(bad == 2) || !(a.bound < __builtin_inf());
      // Every exact top-k member has a fast logit >= (k-th fast value) - 2*bound.
      const double thr = sm.topv[k - 1] - 2.0 * a.bound;
      if (threadIdx.x == 0) sm.ncand = 0;
      __syncthreads();
      for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const double v = sm.v[e];
        const bool cand = all || (v == v && v >= thr);
        if (cand) sm.cand[atomicAdd(&sm.ncand, 1)] = e;
        else sm.excl[e] = 1;
      }
      __syncthreads();
      for (int i = wave; i < sm.ncand; i += nwaves) {
        const int c = sm.cand[i];
        const double val = dd_logit(a.xrow, a.wr, (size_t)E, 1, a.H, c, a.bias);
        if (lane == 0) sm.v[c] = val;
      }
      __syncthreads();
      block_rank(sm, E, k);
      __syncthreads();
    }
  }
  // Weights: softmax over the k selected (renormalised) or over all E, in
  // fp32 (the weights are fp32 outputs; the logit differences are taken in
  // float64 first).
  const double v0 = sm.topv[0];
  if (!a.renorm) {
    float part = 0.f;
    for (int e = threadIdx.x; e < E; e += blockDim.x) part += expf(static_cast<float>(sm.v[e] - v0));
    part = dpp_sum_f(part);
    if (lane == 0) sm.dred[wave] = part;
    __syncthreads();
  }
  if (wave == 0) {
    const float z = (lane < k) ? expf(static_cast<float>(sm.topv[lane] - v0)) : 0.f;
    float denom = 0.f;
    if (a.renorm) {
      denom = dpp_sum_f(z);
    } else {
      for (int i = 0; i < nwaves; ++i) denom += static_cast<float>(sm.dred[i]);
    }
    if (lane < k) {
      a.ids[lane] = sm.topi[lane];
      a.w[lane] = z / denom;
    }
  }
}

// ---------------------------------------------------------------------------
// Wavefront-per-token top-k (large batches): the same selection as block_rank
// inside one wavefront (up to 16 logits per lane).
// ---------------------------------------------------------------------------
struct WaveTopkScratch {
  int cand[kWave];
  uint64_t ckey[kWave];
  double tv[kMaxTopK + 1];
  int ti[kMaxTopK + 1];
  int tc[kMaxTopK + 1];
  unsigned char mark[kMaxExperts];  // 1: logit to recompute
};

constexpr int kMaxPerLane = kMaxExperts / kWave;

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Lanes r < rounds receive the r-th entry of the order in (top_v, top_i,
// top_c); returns how many entries exist (eligible logits, at most rounds).
// The `rounds`-th largest fp32-rounded key is found by bisection; the
// candidates at or above it (at most 64, else the round-by-round selection
// takes over) are ranked exactly on order_key.
// NP: keys per lane, a power of two >= ceil(E / 64).  Keys past E are 0 and
// never reach the threshold (>= 1), so every loop below is fully unrolled
// with no per-element branch.
template <int NP>
__device__ inline int wave_rank_select_np(const double* vals, int E, uint32_t excl, int rounds,
                                          WaveTopkScratch& sc, double& top_v, int& top_i,
                                          int& top_c) {
  const int lane = __lane_id();
  uint32_t c[NP];
  int elig = 0;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int e = lane + kWave * i;
    c[i] = (e < E) ? coarse_key(vals[e], (excl >> i) & 1u) : 0u;
    elig += __popcll(__ballot(c[i] != 0u));
  }
  // Threshold: the `rounds`-th largest of the 64 lane maxima.  Those are
  // `rounds` distinct keys, so the `rounds`-th largest key overall is at least
  // this value, and every member of the first `rounds` (exact order; coarse
  // keys are monotone in it) has a key at or above it.  One key per lane in
  // the bisection instead of NP.
  uint32_t lmax[1] = {0u};
#pragma unroll
  for (int i = 0; i < NP; ++i) lmax[0] = c[i] > lmax[0] ? c[i] : lmax[0];
  uint32_t t = wave_kth_key<1>(lmax, rounds);
  if (t == 0u) t = 1u;  // fewer than `rounds` lanes hold an eligible logit: all eligible
  int nc = 0;
#pragma unroll
  for (int i = 0; i < NP; ++i) nc += __popcll(__ballot(c[i] >= t));
  if (nc > kWave) return wave_select(vals, E, excl, rounds, top_v, top_i, top_c);
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  int base = 0;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const bool q = c[i] >= t;
    const uint64_t b = __ballot(q);
    if (q) {
      const int slot = base + __popcll(b & lt);
      const int e = lane + kWave * i;
      sc.cand[slot] = e;
      sc.ckey[slot] = order_key(vals[e], false);
    }
    base += __popcll(b);
  }
  wave_lds_sync();
  if (lane < nc) {
    const int e = sc.cand[lane];
    const uint64_t ke = sc.ckey[lane];
    int cnt = 0;
    for (int j = 0; j < nc; ++j) cnt += ranks_before(sc.ckey[j], sc.cand[j], ke, e);
    if (cnt < rounds) {
      sc.tv[cnt] = vals[e];
      sc.ti[cnt] = e;
      sc.tc[cnt] = (ke == 1ull) ? 1 : 2;
    }
  }
  wave_lds_sync();
  const int got = min(rounds, elig);
  if (lane < got) {
    top_v = sc.tv[lane];
    top_i = sc.ti[lane];
    top_c = sc.tc[lane];
  }
  wave_lds_sync();
  return got;
}

__device__ inline int wave_rank_select(const double* vals, int E, uint32_t excl, int rounds,
                                       WaveTopkScratch& sc, double& top_v, int& top_i, int& top_c) {
  const int nper = (E + kWave - 1) / kWave;
  if (nper <= 1) return wave_rank_select_np<1>(vals, E, excl, rounds, sc, top_v, top_i, top_c);
  if (nper <= 2) return wave_rank_select_np<2>(vals, E, excl, rounds, sc, top_v, top_i, top_c);
  if (nper <= 4) return wave_rank_select_np<4>(vals, E, excl, rounds, sc, top_v, top_i, top_c);
  if (nper <= 8) return wave_rank_select_np<8>(vals, E, excl, rounds, sc, top_v, top_i, top_c);
  return wave_rank_select_np<kMaxPerLane>(vals, E, excl, rounds, sc, top_v, top_i, top_c);
}

// Select, certify (optionally recompute), and write ids and weights.
__device__ inline void wave_topk(const TopkToken& a) {
  const int lane = __lane_id();
  const int E = a.E, k = a.k;
  const int K1 = (k + 1 <= E) ? k + 1 : k;
  double top_v = 0.0;
  int top_i = 0, top_c = 0;
  uint32_t excl = 0;  // bit i: expert lane + 64*i not eligible (after a recompute)
  int got = wave_rank_select(a.vals, E, 0u, a.certify ? K1 : k, *a.sc, top_v, top_i, top_c);
  if (a.certify) {
    const double next_v = __shfl_down(top_v, 1, kWave);
    const bool fin_r = (lane >= got) || (top_c == 2 && (top_v - top_v == 0.0));
    const bool finite = __all(fin_r);
    const bool gap_ok = (lane + 1 >= got) || (top_v - next_v > 2.0 * a.bound);
    const bool ok = (got == K1) && finite && __all(gap_ok);
    if (a.recomputed != nullptr && lane == 0) *a.recomputed = ok ? 0 : 1;
    if (!ok) {
      // Exact logits are needed only where the fast order is in doubt: the
      // members of close pairs (gap <= 2*bound) among the first k, and, when
      // the k-th and (k+1)-th are close, every logit within 2*bound of the
      // k-th.  Any other logit is more than 2*bound from all of those, so its
      // fast value orders it correctly against their exact values and the
      // selection is rerun on the mixed values.  A non-finite value among
      // the top k+1 or a non-finite bound says nothing: recompute all.
      const bool all = !finite || !(a.bound < __builtin_inf());
      const double two_b = 2.0 * a.bound;
      const bool close_r = (lane + 1 < got) && !(top_v - next_v > two_b);
      // (every lane runs the shuffle: a lane that reads from an inactive lane
      // gets 0)
      const int close_up = __shfl_up(close_r ? 1 : 0, 1, kWave);
      const bool close_prev = (lane > 0) && close_up != 0;
      const bool boundary = __shfl(close_r ? 1 : 0, k - 1, kWave) != 0;
      const double thr = __shfl(top_v, k - 1, kWave) - two_b;
      const int nper = (E + kWave - 1) / kWave;
      WaveTopkScratch& sc = *a.sc;
      for (int i = 0; i < nper; ++i) {
        const int e = lane + kWave * i;
        if (e < E) sc.mark[e] = 0;
      }
      wave_lds_sync();
      if (lane < k && lane < got && (close_r || close_prev)) sc.mark[top_i] = 1;
      wave_lds_sync();
      // Contiguous expert rows: candidates go four at a time (dd_logits4).
      int eb[4] = {-1, -1, -1, -1};
      int nb = 0;
      auto flush = [&]() {
        double v4[4];
        dd_logits4(a.xrow, a.wr, a.wr_se, a.H, eb, a.bias, v4);
        if (lane == 0) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (eb[q] >= 0) a.vals[eb[q]] = v4[q];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) eb[q] = -1;
        nb = 0;
      };
      for (int i = 0; i < nper; ++i) {
        const int e = lane + kWave * i;
        const double v = (e < E) ? a.vals[e] : 0.0;
        const bool cand =
            (e < E) && (all || sc.mark[e] != 0 || (boundary && v == v && v >= thr));
        uint64_t mask = __ballot(cand);
        while (mask) {
          const int l = __builtin_ctzll(mask);
          mask &= mask - 1;
          if (a.wr_sh == 1) {
            const int ec = l + kWave * i;
            if (nb == 0) eb[0] = ec;
            else if (nb == 1) eb[1] = ec;
            else if (nb == 2) eb[2] = ec;
            else eb[3] = ec;
            if (++nb == 4) flush();
          } else {
            const double val = dd_logit(a.xrow, a.wr, a.wr_sh, a.wr_se, a.H, l + kWave * i, a.bias);
            if (lane == 0) a.vals[l + kWave * i] = val;
          }
        }
      }
      if (nb > 0) flush();
      wave_lds_sync();
      got = wave_rank_select(a.vals, E, excl, k, *a.sc, top_v, top_i, top_c);
    }
  }
  // Weights: softmax over the k selected (renormalised) or over all E, in
  // fp32 (the logit differences are taken in float64 first).
  const double v0 = __shfl(top_v, 0, kWave);
  const float z = (lane < k) ? expf(static_cast<float>(top_v - v0)) : 0.f;
  float denom;
  if (a.renorm) {
    denom = dpp_sum_f(z);
  } else {
    float part = 0.f;
    for (int e = lane; e < E; e += kWave) part += expf(static_cast<float>(a.vals[e] - v0));
    denom = dpp_sum_f(part);
  }
  if (lane < k) {
    a.ids[lane] = top_i;
    a.w[lane] = z / denom;
  }
}

// ---------------------------------------------------------------------------
// Certified top-k of one token by a whole workgroup of NTH threads with no
// serial step per selected expert:
//   (1) every wavefront finds the (k+1)-th largest 16-bit coarse key among
//       its lanes' maxima (a 16-step bisection, all wavefronts in parallel);
//       the largest of those is a lower bound for the overall (k+1)-th
//       largest coarse key (each wavefront alone holds k+1 keys at or above
//       its value), so every member of the first k+1 is at or above it;
//   (2) the candidates at or above it are compacted into LDS (one atomic per
//       wavefront) and each ranks itself against all of them on the exact
//       order keys (one thread per candidate, LDS reads in groups of 8);
//   (3) the first k+1 are certified as in wave_topk.
// Returns false, with nothing written, when the fast order cannot be
// certified (close gaps, a non-finite value among the first k+1, more
// candidates than one wavefront holds) or renormalisation is off: the caller
// then runs wave_topk, which recomputes what it must.  The coarse key is the
// top 16 bits of coarse_key (monotone in the logit); a NaN keeps key 1 so
// that it stays eligible below every number.
template <int NTH>
struct BlockFastTopkSmem {
  uint32_t wthr[NTH / kWave];
  int ncand;
  int ok;
  int cand[kWave];  // each thread reads its span of these (nc <= 64)
  uint64_t ckey[kWave];
  double tv[kMaxTopK + 1];
  int ti[kMaxTopK + 1];
};

__device__ __forceinline__ uint32_t coarse16(double v) {
  const uint32_t c = coarse_key(v, false);
  return c == 0u ? 0u : max(c >> 16, 1u);
}

// vals: LDS [E] float64 logits, visible to the block; thread t owns experts
// t + NTH i.  ids / w: [k] outputs.
template <int NTH>
__device__ inline bool block_topk_fast(const double* vals, int E, int k, int renorm, double bound,
                                       BlockFastTopkSmem<NTH>& sm, int* ids, float* w) {
  constexpr int kPer = (kMaxExperts + NTH - 1) / NTH;
  constexpr int kNW = NTH / kWave;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int K1 = (k + 1 <= E) ? k + 1 : k;
  uint32_t c[kPer];
  uint32_t lm = 0u;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = threadIdx.x + NTH * i;
    c[i] = (e < E) ? coarse16(vals[e]) : 0u;
    lm = max(lm, c[i]);
  }
  uint32_t tw = 0u;
#pragma unroll
  for (int bit = 15; bit >= 0; --bit) {
    const uint32_t cand = tw | (1u << bit);
    if (__popcll(__ballot(lm >= cand)) >= K1) tw = cand;
  }
  if (lane == 0) sm.wthr[wave] = tw;
  if (threadIdx.x == 0) sm.ncand = 0;
  __syncthreads();
  uint32_t t = 0u;
#pragma unroll
  for (int i = 0; i < kNW; ++i) t = max(t, sm.wthr[i]);
  if (t == 0u) t = 1u;  // fewer than k+1 eligible in every wavefront: all eligible
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  uint64_t bq[kPer];
  int nw = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    bq[i] = __ballot(c[i] >= t);
    nw += __popcll(bq[i]);
  }
  int base = 0;
  if (lane == 0 && nw > 0) base = atomicAdd(&sm.ncand, nw);
  base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int slot = base + __popcll(bq[i] & lt);
    if (((bq[i] >> lane) & 1ull) && slot < kWave) {
      const int e = threadIdx.x + NTH * i;
      sm.cand[slot] = e;
      sm.ckey[slot] = order_key(vals[e], false);
    }
    base += __popcll(bq[i]);
  }
  __syncthreads();
  const int nc = sm.ncand;
  if (nc > kWave || renorm == 0) return false;  // uniform: every thread read the same nc
  // Rank of each candidate among all nc: the comparisons are split over
  // kParts consecutive threads per candidate (kSpan candidates each), and
  // their counts summed with lane shuffles, so the block does the nc x nc
  // comparisons in kSpan steps instead of one thread doing nc.
  static_assert(NTH % kWave == 0 && NTH / kWave >= 1, "whole wavefronts");
  constexpr int kParts = NTH / kWave;      // threads per candidate
  constexpr int kSpan = kWave / kParts;     // candidates each thread compares with
  static_assert(kParts * kSpan == kWave && (kParts & (kParts - 1)) == 0, "power-of-two split");
  {
    const int ci = threadIdx.x / kParts, part = threadIdx.x % kParts;
    int cnt = 0;
    uint64_t ke = 0ull;
    int e = 0;
    if (ci < nc) {
      e = sm.cand[ci];
      ke = sm.ckey[ci];
      uint64_t kj[kSpan];
      int ej[kSpan];
#pragma unroll
      for (int q = 0; q < kSpan; ++q) {
        kj[q] = sm.ckey[part * kSpan + q];
        ej[q] = sm.cand[part * kSpan + q];
      }
#pragma unroll
      for (int q = 0; q < kSpan; ++q)
        if (part * kSpan + q < nc) cnt += ranks_before(kj[q], ej[q], ke, e);
    }
#pragma unroll
    for (int d = 1; d < kParts; d <<= 1) cnt += __shfl_xor(cnt, d, kWave);
    if (ci < nc && part == 0 && cnt < K1) {
      sm.tv[cnt] = (ke == 1ull) ? __builtin_nan("") : vals[e];
      sm.ti[cnt] = e;
    }
  }
  __syncthreads();
  const int got = min(K1, nc);
  if (wave == 0) {
    const double tv = (lane < got) ? sm.tv[lane] : 0.0;
    const double nv = __shfl_down(tv, 1, kWave);
    const bool fin = (lane >= got) || (tv - tv == 0.0);
    const bool gap = (lane + 1 >= got) || (tv - nv > 2.0 * bound);
    const bool ok = (got == K1) && __all(fin) && __all(gap);
    if (ok) {  // weights as wave_topk computes them (renormalised softmax)
      const double v0 = __shfl(tv, 0, kWave);
      const float z = (lane < k) ? expf(static_cast<float>(tv - v0)) : 0.f;
      const float denom = dpp_sum_f(z);
      if (lane < k) {
        ids[lane] = sm.ti[lane];
        w[lane] = z / denom;
      }
    }
    if (lane == 0) sm.ok = ok ? 1 : 0;
  }
  __syncthreads();
  return sm.ok != 0;
}

// Per-group descriptor the fused decode kernels read in one step.
constexpr int kGroupDescInts = 20;  // e, p0, nrows, spare, 16 input-token rows
constexpr int kGroupDescRows = 16;

// Stable counting sort of P pairs by expert id, by one wavefront.
//   cnt, aidx, off0: LDS scratch [E].  active: [E+1] (count, then ids).
//   desc (optional): [E][kGroupDescInts] group descriptors in active order;
//   the token list holds pair/topk for the first kGroupDescRows rows.
__device__ inline void wave_group(const int* ids, int P, int E, int topk, int* counts,
                                  int* offsets, int* perm_to_pair, int* pair_to_perm, int* active,
                                  int* desc, int* cnt, int* aidx, int* off0) {
  const int lane = __lane_id();
  for (int e = lane; e < E; e += kWave) cnt[e] = 0;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  for (int p = lane; p < P; p += kWave) {
    const int e = ids[p];
    if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __builtin_amdgcn_wave_barrier();
  // offsets (exclusive scan) and the active list, 64 experts at a time
  int run = 0, nact = 0;
  for (int base = 0; base < E; base += kWave) {
    const int e = base + lane;
    const int c = (e < E) ? cnt[e] : 0;
    int x = c;
    for (int d = 1; d < kWave; d <<= 1) {
      const int y = __shfl_up(x, d, kWave);
      if (lane >= d) x += y;
    }
    const int excl_off = run + x - c;
    const uint64_t nz = __ballot(c > 0);
    const int arank = __popcll(nz & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
    if (e < E) {
      if (counts != nullptr) counts[e] = c;
      offsets[e] = excl_off;
      cnt[e] = excl_off;  // next free position of expert e
      off0[e] = excl_off;
      aidx[e] = (c > 0) ? nact + arank : -1;
      if (c > 0) {
        active[1 + nact + arank] = e;
        if (desc != nullptr) {
          int* d = desc + (size_t)(nact + arank) * kGroupDescInts;
          d[0] = e;
          d[1] = excl_off;
          d[2] = c;
          d[3] = 0;
        }
      }
    }
    run += __shfl(x, kWave - 1, kWave);
    nact += __popcll(nz);
  }
  if (lane == 0) {
    offsets[E] = run;
    active[0] = nact;
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __builtin_amdgcn_wave_barrier();
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int s = 0; s < P; s += kWave) {
    const int p = s + lane;
    const int e0 = (p < P) ? ids[p] : -1;
    const bool valid = (p < P) && (unsigned)e0 < (unsigned)E;
    const int e = valid ? e0 : 0;
    uint64_t same = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const uint64_t m = __ballot(valid && ((e >> bit) & 1));
      same &= ((e >> bit) & 1) ? m : ~m;
    }
    const int pos = valid ? cnt[e] + __popcll(same & lt) : 0;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      perm_to_pair[pos] = p;
      pair_to_perm[p] = pos;
      if (desc != nullptr) {
        const int u = aidx[e];
        const int r = pos - off0[e];
        if (u >= 0 && r < kGroupDescRows) desc[(size_t)u * kGroupDescInts + 4 + r] = p / topk;
      }
      if ((same >> lane) == 1ull) cnt[e] = pos + 1;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace moe
