// Router logits for large token batches on the bf16 matrix cores, with a
// rigorous error bound for the certified top-k.
//
// The router is a plain fp32 linear map (the pages keep it outside the
// quantized path: "DGPP" README mirror, supported-models notes), and the
// routing decision is taken on the exact logits (see route.hip).  For
// prefill-sized batches the contraction x[T][H] . Wr[H][E] is large enough
// for MFMA, which takes bf16 operands only.  So:
//
// * Wr is cut by truncation into three bf16 planes, w = hi + mid + lo
//   exactly (hi keeps the top 8 significant bits, mid the next 8, lo the
//   last 8; non-finite w goes whole into hi).  x is bf16 already, so every
//   product x*part is exact in fp32.
// * Each 64-wide K step sums its 192 products (3 planes) on the matrix cores
//   in fp32, starting from zero, and the step sums are added in float64.
//   Whatever order and rounding the matrix core uses inside a step (any
//   faithful fp32 rounding), a step errs by at most
//   g = 192u/(1-192u) (u = 2^-23) times the sum of |products|, and
//   |hi|+|mid|+|lo| <= (1+2^-6)|w|.  With Cauchy-Schwarz,
//       |logit - exact| <= c * ||x_t||_2 * max_e ||w_e||_2
//   where c also covers the float64 additions and the final fp32 rounding.
// * The kernel writes, per token and 64-expert block, the product of upper
//   bounds of ||x_t|| and of the block's largest ||w_e|| (plus tiny terms
//   for flushed subnormals); the top-k multiplies its maximum by c.  When
//   that product could overflow fp32 it writes +inf, which makes the top-k
//   recompute every logit of the token exactly.
#include "moe_launch.h"

namespace moe {
namespace {

constexpr int RBM = 128, RBN = 64, RBK = 64;
// LDS row pitch (bf16): 160-byte rows make the fragment reads conflict-free
// and half as costly in LDS cycles as 144-byte rows on gfx950 (measured); the
// staging writes below keep them conflict-free by writing a step's 8-element
// K pieces in the order piece (h, i) of K half h -> column 8(2i + h), for A
// and B alike, so an MFMA still pairs equal K.
constexpr int RLDS = RBK + 16;
constexpr int kSplitRows = 32;  // router rows per block of the split pass (8 per wavefront)
constexpr int kXcds = 8;

__device__ __forceinline__ void split3(float w, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
  const uint32_t b = __float_as_uint(w);
  if ((b & 0x7f800000u) == 0x7f800000u) {  // inf or NaN: all in hi
    hi = ((b & 0x7fffffu) != 0) ? static_cast<uint16_t>((b >> 16) | 0x40u) : static_cast<uint16_t>(b >> 16);
    mid = lo = 0;
    return;
  }
  hi = static_cast<uint16_t>(b >> 16);
  const float r0 = w - __uint_as_float(b & 0xffff0000u);  // exact (same binade, truncated)
  const uint32_t b0 = __float_as_uint(r0);
  mid = static_cast<uint16_t>(b0 >> 16);
  const float r1 = r0 - __uint_as_float(b0 & 0xffff0000u);  // exact
  lo = static_cast<uint16_t>(__float_as_uint(r1) >> 16);   // exact unless |w| < 2^-110
}

// Wr [H][E] fp32 -> planes [3][E][H] bf16, a transposed fp32 copy wrt [E][H]
// (for the exact recompute of contested logits, read along h), and wsq
// [HB][E] float64 sums of w^2 over router rows [hb*32, +32).
// Block: 64 experts x 32 rows; lane = expert (512 blocks at H = 2048, E = 512).
__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ wr, int H,
                                                           int E, uint16_t* __restrict__ planes,
                                                           float* __restrict__ wrt,
                                                           double* __restrict__ wsq) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + lane;
  const int hb = blockIdx.y;
  const int h0 = hb * kSplitRows + wave * (kSplitRows / 4);
  double sq = 0.0;
  if (e < E) {
    for (int c = 0; c < kSplitRows / 4; c += 8) {
      const int h = h0 + c;
      if (h >= H) break;  // H % 8 == 0: a group of 8 rows is all in or all out
      uint32_t p[3][4];
      float wv[8];
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const float w0 = wr[(size_t)(h + i) * E + e];
        const float w1 = wr[(size_t)(h + i + 1) * E + e];
        wv[i] = w0;
        wv[i + 1] = w1;
        sq = fma(static_cast<double>(w0), static_cast<double>(w0), sq);
        sq = fma(static_cast<double>(w1), static_cast<double>(w1), sq);
        uint16_t a0, a1, a2, c0, c1, c2;
        split3(w0, a0, a1, a2);
        split3(w1, c0, c1, c2);
        p[0][i / 2] = a0 | (uint32_t(c0) << 16);
        p[1][i / 2] = a1 | (uint32_t(c1) << 16);
        p[2][i / 2] = a2 | (uint32_t(c2) << 16);
      }
#pragma unroll
      for (int s = 0; s < 3; ++s)
        *reinterpret_cast<u32x4*>(planes + ((size_t)s * E + e) * H + h) =
            u32x4{p[s][0], p[s][1], p[s][2], p[s][3]};
      float* wt = wrt + (size_t)e * H + h;
      *reinterpret_cast<f32x4*>(wt) = f32x4{wv[0], wv[1], wv[2], wv[3]};
      *reinterpret_cast<f32x4*>(wt + 4) = f32x4{wv[4], wv[5], wv[6], wv[7]};
    }
  }
  __shared__ double red[4][64];
  red[wave][lane] = sq;
  __syncthreads();
  if (wave == 0 && e < E)
    wsq[(size_t)hb * E + e] = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
}

struct RouterMfmaArgs {
  const uint16_t* x;       // [T][H] bf16
  const uint16_t* planes;  // [3][E][H] bf16
  const double* wsq;       // [HB][E]
  int T, H, E, HB;
  float xslack;  // turns the fp32 sum of x^2 into an upper bound of ||x||
  float* logits;  // [T][E]
  float* amax;    // [n_nt][T]
  int n_mt, n_nt;
};

// One LDS stage (50 KB); the next step waits in registers while this one is
// read.  Eight wavefronts of 32 tokens x 32 experts (float64 step sums in 32
// registers a lane) let two workgroups share a CU, so a 512-tile grid runs in
// one round: 80 -> 74 us on 8192 tokens x 512 experts against four
// wavefronts of 64 x 32.
// (16-byte aligned rows: every fragment access is one 128-bit LDS
// instruction; with the element type's 2-byte alignment the compiler splits
// each into two pairs of 32-bit accesses)
struct RouterSmem {
  __attribute__((aligned(16))) uint16_t a[RBM][RLDS];
  __attribute__((aligned(16))) uint16_t b[3][RBN][RLDS];
  float wn[RBN];
};

constexpr int kRThreads = 512;

__global__ __launch_bounds__(kRThreads, 4) void router_mfma_kernel(RouterMfmaArgs a) {
  __shared__ RouterSmem sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // XCD-aware order (workgroup b runs on XCD b % 8): each XCD takes a
  // contiguous range of (token tile, expert tile), expert tiles fastest.
  const int total = a.n_mt * a.n_nt;
  const int per = (total + kXcds - 1) / kXcds;
  const int idx = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  if (idx >= total) return;
  const int mt = idx / a.n_nt, nt = idx % a.n_nt;
  const int t0 = mt * RBM, e0 = nt * RBN;
  const int H = a.H, E = a.E;

  // ||w_e|| upper bounds for this block's experts
  if (tid < RBN) {
    const int e = e0 + tid;
    float wn = 0.f;
    if (e < E) {
      double s = 0.0;
      for (int hb0 = 0; hb0 < a.HB; hb0 += 8) {  // eight loads in flight at a time
        double v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = (hb0 + j < a.HB) ? a.wsq[(size_t)(hb0 + j) * E + e] : 0.0;
#pragma unroll
        for (int j = 0; j < 8; ++j) s += v[j];
      }
      wn = static_cast<float>(sqrt(s) * (1.0 + 0x1p-40)) * (1.0f + 0x1p-21f);
    }
    sm.wn[tid] = wn;
  }

  // staging roles: four threads per token row, two 8-element K pieces each
  const int srow = tid >> 2, squart = tid & 3;
  const uint16_t* xrow = (t0 + srow < a.T) ? a.x + (size_t)(t0 + srow) * H : nullptr;
  float xsq = 0.f;

  u32x4 ra[2], rb[3];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int k = k0 + 8 * (2 * squart + i);
      ra[i] = (xrow != nullptr && k < H) ? *reinterpret_cast<const u32x4*>(xrow + k)
                                         : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int c = tid + kRThreads * i;  // 192 rows x 8 chunks of 8
      const int row = c >> 3, part = c & 7;
      const int s = row / RBN, e = e0 + row % RBN;
      const int k = k0 + 8 * part;
      rb[i] = (e < E && k < H)
                  ? *reinterpret_cast<const u32x4*>(a.planes + ((size_t)s * E + e) * H + k)
                  : u32x4{0, 0, 0, 0};
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int pc = 2 * squart + i;  // K piece (half pc / 4, index pc % 4)
      *reinterpret_cast<u32x4*>(&sm.a[srow][8 * (2 * (pc & 3) + (pc >> 2))]) = ra[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float lo = __uint_as_float(ra[i][j] << 16), hi = __uint_as_float(ra[i][j] & 0xffff0000u);
        xsq = fmaf(lo, lo, xsq);
        xsq = fmaf(hi, hi, xsq);
      }
    }
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int c = tid + kRThreads * i;
      const int row = c >> 3, part = c & 7;  // K piece (half part / 4, index part % 4)
      *reinterpret_cast<u32x4*>(&sm.b[row / RBN][row % RBN][8 * (2 * (part & 3) + (part >> 2))]) = rb[i];
    }
  };

  // MFMA roles: wave (wm, wn) owns tokens [32wm, +32) x experts [32wn, +32)
  const int wm = wave >> 1, wn = wave & 1;
  double dacc[2][2][4];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) dacc[r][c][j] = 0.0;

  const int nk = (H + RBK - 1) / RBK;
  load(0);
  store();
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    const bool more = ks + 1 < nk;
    if (more) load((ks + 1) * RBK);
    f32x4 cacc[2][2];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int c = 0; c < 2; ++c) cacc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < RBK; kk += 32) {
      const int ko = kk + 8 * (lane >> 4);
      bf16x8 af[2];
#pragma unroll
      for (int r = 0; r < 2; ++r)
        af[r] = *reinterpret_cast<const bf16x8*>(&sm.a[32 * wm + 16 * r + (lane & 15)][ko]);
#pragma unroll
      for (int s = 0; s < 3; ++s) {
        bf16x8 bfr[2];
#pragma unroll
        for (int c = 0; c < 2; ++c)
          bfr[c] = *reinterpret_cast<const bf16x8*>(&sm.b[s][32 * wn + 16 * c + (lane & 15)][ko]);
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int c = 0; c < 2; ++c)
            cacc[r][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[r], bfr[c], cacc[r][c], 0, 0, 0);
      }
    }
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) dacc[r][c][j] += static_cast<double>(cacc[r][c][j]);
    __syncthreads();  // every wavefront has read this step
    if (more) store();
    __syncthreads();
  }

  // logits: lane holds tokens 4*(lane/16)+j of each 16-row tile, expert lane%16
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = t0 + 32 * wm + 16 * r + 4 * (lane >> 4) + j;
      if (t >= a.T) continue;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int e = e0 + 32 * wn + 16 * c + (lane & 15);
        if (e < E) a.logits[(size_t)t * E + e] = static_cast<float>(dacc[r][c][j]);
      }
    }

  // per-token bound factor for this expert block
  xsq += __shfl_xor(xsq, 1, kWave);  // the four threads of a token row
  xsq += __shfl_xor(xsq, 2, kWave);
  float wmax = 0.f;
  for (int i = 0; i < RBN; ++i) wmax = fmaxf(wmax, sm.wn[i]);
  if (squart == 0 && t0 + srow < a.T) {
    const float xn = sqrtf(xsq) * a.xslack;
    float f = (xn + 0x1p-40f) * (wmax + 0x1p-40f) * (1.0f + 0x1p-21f);
    if (!(f < 0x1p126f)) f = __builtin_inff();  // also NaN -> inf
    a.amax[(size_t)nt * a.T + t0 + srow] = f;
  }
}

}  // namespace

int router_mfma_cols(int E) { return (E + RBN - 1) / RBN; }

size_t router_mfma_wsq_count(int H, int E) {
  return (size_t)((H + kSplitRows - 1) / kSplitRows) * E;
}

double router_mfma_bound_scale(int H) {
  const double u = 0x1p-23;
  const double n = 3.0 * RBK;
  const double g = n * u / (1.0 - n * u);
  return (g * (1.0 + 0x1p-6) + 0x1p-23 + (H / 64.0 + 4.0) * 0x1p-52) * 1.0001;
}

hipError_t launch_router_mfma(const uint16_t* x, const float* wr, int T, int H, int E,
                              uint16_t* planes, float* wrt, double* wsq, float* logits,
                              float* amax, hipStream_t s) {
  const int HB = (H + kSplitRows - 1) / kSplitRows;
  hipError_t err = launch(router_split_kernel, dim3((E + 63) / 64, HB), dim3(256), 0, s, wr, H, E,
                          planes, wrt, wsq);
  if (err != hipSuccess) return err;
  RouterMfmaArgs a;
  a.x = x;
  a.planes = planes;
  a.wsq = wsq;
  a.T = T;
  a.H = H;
  a.E = E;
  a.HB = HB;
  // fp32 sum of H nonnegative terms errs by at most gamma_H (u = 2^-23);
  // sqrt and the product each add at most a couple of ulps.
  const double gH = H * 0x1p-23 / (1.0 - H * 0x1p-23);
  a.xslack = static_cast<float>((1.0 + gH) * (1.0 + 0x1p-19));
  a.logits = logits;
  a.amax = amax;
  a.n_mt = (T + RBM - 1) / RBM;
  a.n_nt = router_mfma_cols(E);
  const int total = a.n_mt * a.n_nt;
  const int per = (total + kXcds - 1) / kXcds;
  return launch(router_mfma_kernel, dim3(per * kXcds), dim3(kRThreads), 0, s, a);
}

}  // namespace moe
