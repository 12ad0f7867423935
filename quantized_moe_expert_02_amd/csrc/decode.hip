// Decode lowering (T <= 8 rows; up to 32 where every launch has its aligned
// tile) of the whole layer.
//
// Decode is a weight-streaming problem (forum thread "DGPP: a GB10-optimized
// C++/CUDA inference engine", the "Lossless bf12" post: decode kernels read
// the weights at the memory's line rate).  On gfx950 a dependent kernel in the
// same stream starts about 1.5 us after its predecessor ends, while a
// cross-workgroup hand-off inside a kernel needs an agent-scope release
// (an L2 write-back) and costs far more; so the layer runs as a few short
// launches with no intra-kernel hand-off:
//
//   1. router partial sums over (128-row slice x 32 experts) blocks;
//   2. one block per token: sum the slices, select the top-k (coarse
//      threshold, then exact ranking of the candidates), certify it against
//      the exact logits (recomputing near ties), weights;
//   3. each active routed expert's gate/up + SwiGLU, its weights streamed once
//      for all of its tokens (blocks are laid out per routed pair slot; the
//      block of an expert's first pair derives the expert's (token, slot)
//      pairs from the <= 256 routed ids, the others exit); the first blocks
//      compute the shared expert's gate/up + SwiGLU;
//   4. one token: per (token, 16 output columns), the down projections of
//      the token's k slots and of the shared expert, combined in slot order
//      in fp32 and rounded once to bf16;
//      2 to 32 tokens: per (expert group, 64 output rows), the down
//      projection once for all of the expert's tokens into fp32 y (pair
//      order), then
//   5. the slot-order combine (combine.hip).
//
// Rows of h (and y) are indexed by pair (t*k + j), so no permutation is
// needed.
#include "gemv_core.cuh"
#include "topk_core.cuh"

namespace moe {
namespace {

constexpr int kRH = 128;  // router rows per slice
constexpr int kTmax = 8;  // decode rows
constexpr int kPmax = 512;  // (token, slot) pairs of a decode call
constexpr int kRSBatch = 16;

template <int NT>
struct RouterSmem {
  __attribute__((aligned(16))) float xs[kRH][NT];  // the NT tokens of one row together
  double red[8][NT][kRouterCols];
  float reda[8][NT][kRouterCols];
};

// NT: tokens per block (1 for a single token, else groups of 8), so that a
// single-token call carries no per-token guards in its unrolled loops.
// PT: the slice sums' type in memory (float up to 8 tokens, double above:
// see decode_topk_kernel).
template <int NT, typename PT>
__global__ __launch_bounds__(256) void decode_router_kernel(DecodeArgs a) {
  __shared__ RouterSmem<NT> sm;
  const int rb = blockIdx.x;
  const int T = a.T, H = a.H, E = a.E;
  const int cs = rb / a.RS, rs = rb % a.RS;
  // token group: tokens t0 .. t0 + nt - 1 (batches above 8 tokens launch
  // one group of 8 per grid row)
  const int t0 = blockIdx.y * NT, nt = min(NT, T - t0);
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
  for (int i = threadIdx.x; i < NT * kRH; i += 256) {
    const int t = i / kRH, h = i % kRH;
    sm.xs[h][t] = (t < nt && h < nh) ? bf16_to_f32(a.x[(size_t)(t0 + t) * H + h0 + h]) : 0.f;
  }
  __syncthreads();
  double acc[NT];
  float aa[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    acc[t] = 0.0;
    aa[t] = 0.f;
  }
  // Rows of tokens past the batch are zero in LDS, so every token slot runs
  // unguarded (their sums are never stored).
#pragma unroll
  for (int j = 0; j < kRH / 8; ++j) {
    const int h = rg + 8 * j;
    const double wd = wv[j];
    const float wa = fabsf(wv[j]);
    float xv[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) xv[t] = sm.xs[h][t];
#pragma unroll
    for (int t = 0; t < NT; ++t) {  // bf16 * fp32 is exact in float64
      acc[t] = fma(static_cast<double>(xv[t]), wd, acc[t]);
      aa[t] = fmaf(fabsf(xv[t]), wa, aa[t]);
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    sm.red[rg][t][col] = acc[t];
    sm.reda[rg][t][col] = aa[t];
  }
  __syncthreads();
  if (rg < nt && e < E) {  // thread (t = rg, col) folds the 8 row groups
    const int t = rg;
    double s = 0.0;
    float av = 0.f;
    for (int g = 0; g < 8; ++g) {
      s += sm.red[g][t][col];
      av += sm.reda[g][t][col];
    }
    reinterpret_cast<PT*>(a.part)[((size_t)rs * T + t0 + t) * E + e] = static_cast<PT>(s);
    a.apart[((size_t)rs * T + t0 + t) * E + e] = av;
  }
}

template <typename PT>
__global__ __launch_bounds__(kTopkThreads) void decode_topk_kernel(DecodeArgs a) {
  __shared__ double v[kMaxExperts];
  __shared__ WaveTopkScratch wsc;
  __shared__ BlockFastTopkSmem<kTopkThreads> fsm;
  __shared__ float amax_w[kTopkThreads / kWave];
  const int t = blockIdx.x, T = a.T, E = a.E;
  float amax = 0.f;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    double l = 0.0;
    float av = 0.f;
    for (int r0 = 0; r0 < a.RS; r0 += kRSBatch) {
      PT pv[kRSBatch];
      float qv[kRSBatch];
#pragma unroll
      for (int j = 0; j < kRSBatch; ++j) {  // unconditional loads: one round trip per batch
        const int r = min(r0 + j, a.RS - 1);
        pv[j] = reinterpret_cast<const PT*>(a.part)[((size_t)r * T + t) * E + e];
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
    v[e] = l;
    if (a.logits_out != nullptr) a.logits_out[(size_t)t * E + e] = static_cast<float>(l);
    amax = fmaxf(amax, av);
  }
  amax = wave_max_f(amax);
  if ((threadIdx.x & (kWave - 1)) == 0) amax_w[threadIdx.x / kWave] = amax;
  __syncthreads();
  float am = 0.f;
  for (int i = 0; i < (int)(blockDim.x / kWave); ++i) am = fmaxf(am, amax_w[i]);
  // Fast-logit error.  float64 slice sums (128 exact products: 16 fused
  // multiply-adds per thread, then eight partial sums; the RS <= 512 slice
  // additions and the bias in float64 too): at most (16 + 8 + RS + 1) u
  // sum|x||w| (u = 2^-53) < 2^-43 sum|x||w|.  fp32 slice sums add their
  // roundings: < 2^-23 sum|x||w|.  am, the same sum in fp32 (positive
  // terms), is short of it by far less than a factor 2.  With the fp32
  // bound a top-k gap that close needs the recompute (~11 us on one
  // wavefront) on about one token in 64, which a batch of 16 or more
  // tokens nearly always waits for; below 9 tokens the float64 sums' extra
  // bytes cost more (0.5 us) than the rare recompute.
  const double bound = static_cast<double>(am) * (sizeof(PT) == 8 ? 0x1p-40 : 0x1p-23);
  // The whole block selects and certifies; only when that fails (close
  // gaps, non-finite values, many ties) does one wavefront recompute what
  // it must.
  if (block_topk_fast<kTopkThreads>(v, E, a.k, a.renorm, bound, fsm, a.ids + (size_t)t * a.k,
                                    a.w + (size_t)t * a.k))
    return;
  if (threadIdx.x >= kWave) return;
  TopkToken tk;
  tk.vals = v;
  tk.E = E;
  tk.k = a.k;
  tk.renorm = a.renorm;
  tk.bound = bound;
  tk.certify = true;
  tk.xrow = a.x + (size_t)t * a.H;
  tk.wr = a.wr;  // [H][E]
  tk.wr_sh = (size_t)E;
  tk.wr_se = 1;
  tk.bias = a.bias;
  tk.H = a.H;
  tk.ids = a.ids + (size_t)t * a.k;
  tk.w = a.w + (size_t)t * a.k;
  tk.recomputed = nullptr;
  tk.sc = &wsc;
  wave_topk(tk);
}

// Expert group of pair slot q: the expert e = ids[q] and all (token, slot)
// pairs routed to it, in pair order.  Only the first pair of each expert
// proceeds (returns false for the others), so every active expert is
// processed exactly once.  Block-wide (256 threads), two barriers per 256
// pair slots.
struct GroupSmem {
  int16_t pairs[kPmax];  // 16 bits keep the block's LDS within two workgroups per CU
  int16_t toks[kPmax];
  int wcnt[4];
  int wdup[4];
};

__device__ inline bool derive_group(const DecodeArgs& a, int q, GroupSmem& g, int& e_out, int& n_out) {
  if (a.T == 1) {
    // One token: its k experts are distinct, so every slot is its own group.
    const int e = a.ids[q];
    if (threadIdx.x == 0) {
      g.pairs[0] = q;
      g.toks[0] = 0;
    }
    __syncthreads();
    e_out = e;
    n_out = 1;
    return (unsigned)e < (unsigned)a.E;
  }
  const int P = a.T * a.k;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // the slot's id and the first round's ids in one round trip
  const int e = a.ids[q];
  int my = ((int)threadIdx.x < P) ? a.ids[threadIdx.x] : -1;
  if (P <= kWave * 4) {  // one round (straight-line: 0.5 us less at 8 tokens)
    const int j = threadIdx.x;
    const bool m = (j < P) && my == e;
    const uint64_t bal = __ballot(m);
    const uint64_t dup = __ballot(m && j < q);
    if (lane == 0) {
      g.wcnt[wave] = __popcll(bal);
      g.wdup[wave] = dup != 0ull;
    }
    __syncthreads();
    if (g.wdup[0] | g.wdup[1] | g.wdup[2] | g.wdup[3]) return false;  // uniform
    if ((unsigned)e >= (unsigned)a.E) return false;                      // uniform
    int base = 0;
    for (int w = 0; w < wave; ++w) base += g.wcnt[w];
    if (m) {
      const int pos = base + __popcll(bal & lt);
      g.pairs[pos] = (int16_t)j;
      g.toks[pos] = (int16_t)(j / a.k);
    }
    e_out = e;
    n_out = g.wcnt[0] + g.wcnt[1] + g.wcnt[2] + g.wcnt[3];
    __syncthreads();
    return true;
  }
  int n = 0;
  for (int j0 = 0; j0 < P; j0 += kWave * 4) {
    const int j = j0 + (int)threadIdx.x;
    if (j0 > 0) my = (j < P) ? a.ids[j] : -1;
    const bool m = (j < P) && my == e;
    const uint64_t bal = __ballot(m);
    const uint64_t dup = __ballot(m && j < q);
    if (lane == 0) {
      g.wcnt[wave] = __popcll(bal);
      g.wdup[wave] = dup != 0ull;
    }
    __syncthreads();
    if (g.wdup[0] | g.wdup[1] | g.wdup[2] | g.wdup[3]) return false;  // uniform
    if ((unsigned)e >= (unsigned)a.E) return false;                      // uniform
    int base = n;
    for (int w = 0; w < wave; ++w) base += g.wcnt[w];
    if (m) {
      const int pos = base + __popcll(bal & lt);
      g.pairs[pos] = (int16_t)j;
      g.toks[pos] = (int16_t)(j / a.k);
    }
    n += g.wcnt[0] + g.wcnt[1] + g.wcnt[2] + g.wcnt[3];
    __syncthreads();  // pairs visible; wcnt / wdup free for the next round
  }
  e_out = e;
  n_out = n;
  return true;
}

constexpr int kGuWK = GemvShape<kOpGateUp>::WK;  // K split of the gate/up tiles

// ---- aligned FP4 gate/up tile (the common checkpoint layout) ---------------
// For FP4 experts whose K (= H) is a multiple of 2048 with whole-chunk scale
// words (WDesc::wide), a 16-row tile of gate and up is computed with no
// per-load bounds test: wavefront w takes the contiguous K quarter
// [w K/4, (w+1) K/4) in whole batches of four 128-K chunks, every lane's loads of a
// batch share one base address per matrix (immediate offsets), the group's
// input rows (16 at a time) are staged in LDS and read from there
// as the MFMA B operand, and the four quarters are summed in a fixed order.
constexpr int kLeanMaxRows = 16;  // rows per chunk: the MFMA B operand's 16 columns
constexpr int kLeanMaxK = 4096;

struct LeanSmem {
  f32x4 red[kGuWK][2][kWave];
  ScaleXchg sx[kGuWK][2];
  __attribute__((aligned(16))) uint16_t x[kLeanMaxRows * kLeanMaxK];
};

// K quarters made of whole four-chunk batches: every load of a wavefront
// stays inside its own quarter of the row.
constexpr int kLeanKStep = 128 * 4 * kGuWK;

__host__ __device__ __forceinline__ bool lean_fits(const DecodeArgs& a) {
  return a.gate.wide && a.up.wide && a.H % kLeanKStep == 0 && a.H <= kLeanMaxK;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// One token: its input row does not depend on the routing, so each
// wavefront copies its quarter of the row into LDS by DMA (no register round
// trip) before the routed ids are read.
__device__ __forceinline__ void lean_x_dma(const DecodeArgs& a, LeanSmem& sm) {
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.x), (short)0, a.H * 2, 0x00020000);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  for (int i = wave * kWave * 8; i < a.H; i += kWave * kGuWK * 8)  // 512 values per wavefront step
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr_t)(sm.x + i), 16, 2 * i + 16 * lane, 0, 0,
                                             0);
}

// XDMA: the input row is already on its way by lean_x_dma (one token);
// else the rows are moved here.
// SHARED: the shared expert (weights sg / su, expert 0, input rows = all T
// tokens, output row t of hs); else routed expert e's group (rows toks[],
// output rows pairs[] of h).  FP8 (block-128) chunks carry 32 codes per lane
// in two loads and a block scale applied to each chunk's partial sum.
template <int FMT, bool XDMA, bool SHARED>
__device__ inline void gate_up_lean(const DecodeArgs& a, int e, int nrows, const int16_t* toks,
                                    const int16_t* pairs, int tile, LeanSmem& sm) {
  static_assert(FMT == FMT_NVFP4 || FMT == FMT_MXFP4 || FMT == FMT_FP8, "lean layouts");
  constexpr bool kFp8 = FMT == FMT_FP8;
  const WDesc& gw = SHARED ? a.sg : a.gate;
  const WDesc& uw = SHARED ? a.su : a.up;
  const int H = a.H, I = SHARED ? a.I_shared : a.I;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int r = lane & 15, g = lane >> 4;
  const int n0 = tile * 16;
  const int rb = kFp8 ? H : H / 2;  // code bytes per row
  constexpr int cbytes = kFp8 ? 128 : 64;  // code bytes per 128-K chunk and row
  constexpr int lbytes = kFp8 ? 32 : 16;   // of which lane group g loads
  const int spw = H / (128 * kGuWK);  // chunks per wavefront
  const int c0 = wave * spw;
  const uint8_t* gq = gw.codes + e * gw.stride_codes + (size_t)(n0 + r) * rb + lbytes * g;
  const uint8_t* uq = uw.codes + e * uw.stride_codes + (size_t)(n0 + r) * rb + lbytes * g;
  const uint8_t* gs = scale_row_ptr<FMT>(gw, e, n0 + r);
  const uint8_t* us = scale_row_ptr<FMT>(uw, e, n0 + r);
  float tsg = 1.0f, tsu = 1.0f;
  if constexpr (FMT == FMT_NVFP4) {
    tsg = gw.tscale[e];
    tsu = uw.tscale[e];
  }
  // The group's rows in chunks of 16 (the MFMA B operand's columns); the
  // weights of a chunk after the first come from L2.  The reduction barrier
  // of a chunk also orders every wavefront's LDS reads of its rows before
  // the next chunk's DMA overwrites them.
  for (int c0r = 0; c0r < nrows; c0r += kLeanMaxRows) {
    const int nr = min(kLeanMaxRows, nrows - c0r);
    // the group's input rows into LDS by DMA (1 KiB per wavefront
    // instruction, no register round trip): 8-token layers -0.25 us (NVFP4),
    // -0.7 us (MXFP4) against 16-byte loads through registers
    if constexpr (!XDMA) {
      const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(a.x), (short)0, a.T * H * 2, 0x00020000);
      const int ppr = H / (kWave * 8);  // DMA instructions per row
      for (int ii = wave; ii < nr * ppr; ii += kGuWK) {
        const int row = ii / ppr, piece = ii - row * ppr;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rx, (lds_ptr_t)(sm.x + row * H + piece * kWave * 8), 16,
            2 * ((SHARED ? c0r + row : toks[c0r + row]) * H + piece * kWave * 8) + 16 * lane, 0, 0,
            0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's DMA has landed
    __syncthreads();  // x staged
    f32x4 ag = f32x4{0.f, 0.f, 0.f, 0.f}, au = ag;
    const uint16_t* xr = (r < nr) ? sm.x + r * H : nullptr;
    // chunks per batch of loads (FP8: two, which keeps the kernel at 104 VGPRs
    // where four would need 152)
    constexpr int kB = kFp8 ? 2 : 4;
    for (int cb = c0; cb < c0 + spw; cb += kB) {
      ARaw<FMT> pg[kB], pu[kB];
#pragma unroll
      for (int d = 0; d < kB; ++d) {
        if constexpr (kFp8) {
          pg[d].q0 = *reinterpret_cast<const u32x4*>(gq + cbytes * (cb + d));
          pg[d].q1 = *reinterpret_cast<const u32x4*>(gq + cbytes * (cb + d) + 16);
          pu[d].q0 = *reinterpret_cast<const u32x4*>(uq + cbytes * (cb + d));
          pu[d].q1 = *reinterpret_cast<const u32x4*>(uq + cbytes * (cb + d) + 16);
          pg[d].s = reinterpret_cast<const float*>(gs)[cb + d];
          pu[d].s = reinterpret_cast<const float*>(us)[cb + d];
        } else {
          pg[d].q = *reinterpret_cast<const u32x4*>(gq + cbytes * (cb + d));
          pu[d].q = *reinterpret_cast<const u32x4*>(uq + cbytes * (cb + d));
        }
      }
      if constexpr (!kFp8) {
        uint2 swg, swu;
        if constexpr (FMT == FMT_NVFP4) {
          swg = *reinterpret_cast<const uint2*>(gs + 8 * (cb + g));
          swu = *reinterpret_cast<const uint2*>(us + 8 * (cb + g));
        } else {
          swg = make_uint2(*reinterpret_cast<const uint32_t*>(gs + 4 * (cb + g)), 0u);
          swu = make_uint2(*reinterpret_cast<const uint32_t*>(us + 4 * (cb + g)), 0u);
        }
        const uint2 og = exchange_scales<FMT>(swg, sm.sx[wave][0], r, g);
        const uint2 ou = exchange_scales<FMT>(swu, sm.sx[wave][1], r, g);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          pg[d].s = scale_of_chunk<FMT>(og, d);
          pu[d].s = scale_of_chunk<FMT>(ou, d);
        }
      }
#pragma unroll
      for (int d = 0; d < kB; ++d) {
        u32x4 bx[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          bx[i] = xr ? *reinterpret_cast<const u32x4*>(xr + 128 * (cb + d) + 32 * g + 8 * i)
                     : u32x4{0, 0, 0, 0};
        // FP8: each chunk's sum starts from zero and is scaled by its block scale
        f32x4 tg = kFp8 ? f32x4{0.f, 0.f, 0.f, 0.f} : ag, tu = kFp8 ? f32x4{0.f, 0.f, 0.f, 0.f} : au;
        tg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_a<FMT, 0>(pg[d]), as_bf16x8(bx[0]), tg, 0, 0, 0);
        tu = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_a<FMT, 0>(pu[d]), as_bf16x8(bx[0]), tu, 0, 0, 0);
        tg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_a<FMT, 1>(pg[d]), as_bf16x8(bx[1]), tg, 0, 0, 0);
        tu = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_a<FMT, 1>(pu[d]), as_bf16x8(bx[1]), tu, 0, 0, 0);
        tg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_a<FMT, 2>(pg[d]), as_bf16x8(bx[2]), tg, 0, 0, 0);
        tu = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_a<FMT, 2>(pu[d]), as_bf16x8(bx[2]), tu, 0, 0, 0);
        tg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_a<FMT, 3>(pg[d]), as_bf16x8(bx[3]), tg, 0, 0, 0);
        tu = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_a<FMT, 3>(pu[d]), as_bf16x8(bx[3]), tu, 0, 0, 0);
        if constexpr (kFp8) {
          ag = ag + pg[d].s * tg;
          au = au + pu[d].s * tu;
        } else {
          ag = tg;
          au = tu;
        }
      }
    }
    // the four K quarters, summed in order
    sm.red[wave][0][lane] = ag;
    sm.red[wave][1][lane] = au;
    __syncthreads();
    if (wave == 0 && r < nr) {
      f32x4 sg = sm.red[0][0][lane], su = sm.red[0][1][lane];
#pragma unroll
      for (int w = 1; w < kGuWK; ++w) {
        sg = sg + sm.red[w][0][lane];
        su = su + sm.red[w][1][lane];
      }
      // lane (r, g): rows n0 + 4g + j of group row c0r + r
      uint16_t hv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) hv[j] = f32_to_bf16(silu_fast(sg[j] * tsg) * (su[j] * tsu));
      uint16_t* o = SHARED ? a.hs + (size_t)(c0r + r) * I + n0 + 4 * g
                           : a.h + (size_t)pairs[c0r + r] * I + n0 + 4 * g;
      *reinterpret_cast<uint2*>(o) =
          make_uint2(hv[0] | (uint32_t(hv[1]) << 16), hv[2] | (uint32_t(hv[3]) << 16));
    }
  }
}

// The shared expert runs the lean tile too when its format has one and its
// scale rows are whole-chunk words (FP4) or its block scales are per 128 K
// (FP8); other formats keep the generic kernel.
template <int SFMT>
constexpr bool kSharedLean = SFMT == 0 || SFMT == FMT_NVFP4 || SFMT == FMT_MXFP4 || SFMT == FMT_FP8;

template <int SFMT>
__host__ __device__ __forceinline__ bool shared_lean_fits(const DecodeArgs& a) {
  if constexpr (SFMT == FMT_NVFP4 || SFMT == FMT_MXFP4) return a.sg.wide && a.su.wide;
  else return kSharedLean<SFMT>;
}

// LEAN: every block runs the aligned tile (routed FP4 experts, and the shared
// expert when it has one), so the kernel holds none of the generic tile's
// registers: 104 VGPRs instead of 236, four workgroups per CU instead of two.
template <int RFMT, int SFMT, bool LEAN>
__global__ __launch_bounds__(kWave * kGuWK) void decode_gateup_kernel(DecodeArgs a) {
  __shared__ GroupSmem grp;
  // The shared expert's gate/up blocks (independent of routing) come first.
  const int nsg = (SFMT != 0) ? a.I_shared / gemv_rows_per_block<kOpGateUp>() : 0;
  const int ntiles = a.I / gemv_rows_per_block<kOpGateUp>();
  if constexpr (LEAN) {
    static_assert((RFMT == FMT_NVFP4 || RFMT == FMT_MXFP4) && kSharedLean<SFMT>, "lean tiles");
    extern __shared__ __attribute__((aligned(16))) char lean_dyn[];
    LeanSmem& lsm = *reinterpret_cast<LeanSmem*>(lean_dyn);
    if ((int)blockIdx.x < nsg) {
      if constexpr (SFMT != 0)
        gate_up_lean<SFMT, false, true>(a, 0, a.T, nullptr, nullptr, blockIdx.x, lsm);
      return;
    }
    const int b = blockIdx.x - nsg;
    const int q = b / ntiles, tile = b % ntiles;
    if (a.T == 1) lean_x_dma(a, lsm);
    int e, n;
    if (!derive_group(a, q, grp, e, n)) {
      if (a.T == 1) __builtin_amdgcn_s_waitcnt(0x0f70);  // no DMA outlives its block
      return;
    }
    if (a.T == 1)
      gate_up_lean<RFMT, true, false>(a, e, n, grp.toks, grp.pairs, tile, lsm);
    else
      gate_up_lean<RFMT, false, false>(a, e, n, grp.toks, grp.pairs, tile, lsm);
  } else {
    __shared__ GemvSmem<1, kGuWK, 2> sm;
    if ((int)blockIdx.x < nsg) {
      if constexpr (SFMT != 0) {
        GemvIO io{a.x, a.hs, nullptr, a.k, kInShared, a.T};
        gemv_tile<SFMT, kOpGateUp, 1, kGuWK>(a.sg, a.su, io, GemvRows{0, 0, a.T, nullptr, nullptr},
                                             blockIdx.x, sm);
      }
      return;
    }
    const int b = blockIdx.x - nsg;
    const int q = b / ntiles, tile = b % ntiles;
    int e, n;
    if (!derive_group(a, q, grp, e, n)) return;
    GemvIO io{a.x, a.h, nullptr, a.k, kInList, a.T};
    gemv_tile<RFMT, kOpGateUp, 1, kGuWK>(a.gate, a.up, io, GemvRows{e, 0, n, grp.toks, grp.pairs},
                                         tile, sm);
  }
}

// ---- down projection per expert (2 to 32 tokens) -----------------------------
// A block takes 64 output rows (four wavefronts of 16) of one expert's down
// projection over all of K = I, for every row of the expert's group (the
// group's h rows staged in LDS are the MFMA's B operand), so each expert's
// weights are read once for all of its tokens (per-token blocks read a
// popular expert once per token).  y rows go to memory in pair order; the
// combine launch adds them in slot order.  The shared expert's blocks come
// first (all T tokens, y_s).  FP4: batches of four 128-K chunks with the
// whole-chunk scale words; FP8 block-128: batches of two, block scale per
// chunk partial.
constexpr int kDnRows = 16 * kGuWK;  // output rows per block

// Its LDS: the scale exchange and up to 16 h rows (no K reduction across
// wavefronts, so none of LeanSmem's reduction buffers).
struct DownSmem {
  ScaleXchg sx[kGuWK][1];
  __attribute__((aligned(16))) uint16_t x[kLeanMaxRows * kLeanMaxK];
};

template <int FMT>
__host__ __device__ __forceinline__ bool down_lean_fits(const WDesc& w, int K, int H) {
  // whole 512-value DMA pieces per h row; FP4 loads in batches of four chunks
  if (H % kDnRows != 0 || K > kLeanMaxK || K % 512 != 0) return false;
  if constexpr (FMT == FMT_NVFP4 || FMT == FMT_MXFP4) return w.wide;
  else return FMT == FMT_FP8;
}

template <int FMT, bool SHARED>
__device__ inline void down_lean(const DecodeArgs& a, int e, int nrows, const int16_t* pairs, int tile,
                                 DownSmem& sm) {
  static_assert(FMT == FMT_NVFP4 || FMT == FMT_MXFP4 || FMT == FMT_FP8, "lean layouts");
  constexpr bool kFp8 = FMT == FMT_FP8;
  const WDesc& dw = SHARED ? a.sd : a.down;
  const int K = SHARED ? a.I_shared : a.I, H = a.H;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int r = lane & 15, g = lane >> 4;
  const int n0 = tile * kDnRows + 16 * wave;
  const int rb = kFp8 ? K : K / 2;
  constexpr int cbytes = kFp8 ? 128 : 64;
  constexpr int lbytes = kFp8 ? 32 : 16;
  const uint8_t* wq = dw.codes + e * dw.stride_codes + (size_t)(n0 + r) * rb + lbytes * g;
  const uint8_t* ws = scale_row_ptr<FMT>(dw, e, n0 + r);
  float ts = 1.0f;
  if constexpr (FMT == FMT_NVFP4) ts = dw.tscale[e];
  // The group's rows in chunks of 16 (the MFMA B operand's columns); a
  // barrier keeps the next chunk's DMA behind every wavefront's reads.
  for (int c0r = 0; c0r < nrows; c0r += kLeanMaxRows) {
    const int nr = min(kLeanMaxRows, nrows - c0r);
    if (c0r > 0) __syncthreads();
    // the group's h rows into LDS by DMA (1 KiB per wavefront instruction)
    {
      const uint16_t* base = SHARED ? a.hs : a.h;
      const int nsrc = SHARED ? a.T : a.T * a.k;  // rows of the source buffer
      const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(base), (short)0, nsrc * K * 2, 0x00020000);
      const int ppr = K / (kWave * 8);  // DMA instructions per row
      for (int ii = wave; ii < nr * ppr; ii += kGuWK) {
        const int row = ii / ppr, piece = ii - row * ppr;
        const int srow = SHARED ? c0r + row : pairs[c0r + row];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rh, (lds_ptr_t)(sm.x + row * K + piece * kWave * 8),
                                                 16, 2 * (srow * K + piece * kWave * 8) + 16 * lane,
                                                 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's DMA has landed
    __syncthreads();  // h staged
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint16_t* hr = (r < nr) ? sm.x + r * K : nullptr;
    constexpr int kB = kFp8 ? 2 : 4;
    const int nch = K / 128;
    for (int cb = 0; cb < nch; cb += kB) {
      ARaw<FMT> pw[kB];
#pragma unroll
      for (int d = 0; d < kB; ++d) {
        if constexpr (kFp8) {
          pw[d].q0 = *reinterpret_cast<const u32x4*>(wq + cbytes * (cb + d));
          pw[d].q1 = *reinterpret_cast<const u32x4*>(wq + cbytes * (cb + d) + 16);
          pw[d].s = reinterpret_cast<const float*>(ws)[cb + d];
        } else {
          pw[d].q = *reinterpret_cast<const u32x4*>(wq + cbytes * (cb + d));
        }
      }
      if constexpr (!kFp8) {
        uint2 sw;
        if constexpr (FMT == FMT_NVFP4)
          sw = *reinterpret_cast<const uint2*>(ws + 8 * (cb + g));
        else
          sw = make_uint2(*reinterpret_cast<const uint32_t*>(ws + 4 * (cb + g)), 0u);
        const uint2 o = exchange_scales<FMT>(sw, sm.sx[wave][0], r, g);
#pragma unroll
        for (int d = 0; d < kB; ++d) pw[d].s = scale_of_chunk<FMT>(o, d);
      }
#pragma unroll
      for (int d = 0; d < kB; ++d) {
        u32x4 bx[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          bx[i] = hr ? *reinterpret_cast<const u32x4*>(hr + 128 * (cb + d) + 32 * g + 8 * i)
                     : u32x4{0, 0, 0, 0};
        f32x4 t = kFp8 ? f32x4{0.f, 0.f, 0.f, 0.f} : acc;
        t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_a<FMT, 0>(pw[d]), as_bf16x8(bx[0]), t, 0, 0, 0);
        t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_a<FMT, 1>(pw[d]), as_bf16x8(bx[1]), t, 0, 0, 0);
        t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_a<FMT, 2>(pw[d]), as_bf16x8(bx[2]), t, 0, 0, 0);
        t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_a<FMT, 3>(pw[d]), as_bf16x8(bx[3]), t, 0, 0, 0);
        if constexpr (kFp8)
          acc = acc + pw[d].s * t;
        else
          acc = t;
      }
    }
    if (r < nr) {
      // lane (r, g): output rows n0 + 4g + j of group row c0r + r
      float* o = SHARED ? a.ys + (size_t)(c0r + r) * H + n0 + 4 * g
                        : a.y + (size_t)pairs[c0r + r] * H + n0 + 4 * g;
      *reinterpret_cast<f32x4*>(o) = acc * ts;
    }
  }
}

template <int RFMT, int SFMT>
__global__ __launch_bounds__(kWave * kGuWK) void decode_down_kernel(DecodeArgs a) {
  __shared__ GroupSmem grp;
  extern __shared__ __attribute__((aligned(16))) char lean_dyn[];
  DownSmem& lsm = *reinterpret_cast<DownSmem*>(lean_dyn);
  const int ntiles = a.H / kDnRows;
  const int nsd = (SFMT != 0) ? ntiles : 0;
  if ((int)blockIdx.x < nsd) {
    if constexpr (SFMT != 0) down_lean<SFMT, true>(a, 0, a.T, nullptr, blockIdx.x, lsm);
    return;
  }
  const int b = blockIdx.x - nsd;
  const int q = b / ntiles, tile = b % ntiles;
  int e, n;
  if (!derive_group(a, q, grp, e, n)) {
    // a slot with no expert (id out of range) contributes zeros to the combine
    if ((unsigned)a.ids[q] >= (unsigned)a.E && (int)threadIdx.x < kDnRows / 4)
      *reinterpret_cast<f32x4*>(a.y + (size_t)q * a.H + tile * kDnRows + 4 * threadIdx.x) =
          f32x4{0.f, 0.f, 0.f, 0.f};
    return;
  }
  down_lean<RFMT, false>(a, e, n, grp.pairs, tile, lsm);
}

// One 16-row tile (weight rows n0..n0+15 of expert e) times one bf16 input
// row of length K, for the calling wavefront.  The weights are decoded in
// registers as in gemv_tile; the input row is the MFMA's B operand column 0.
// Result: lane 16q holds output rows n0 + 4q + (0..3) (lanes with lane % 16
// != 0 hold zeros), times the NVFP4 tensor scale.  Loads of four 128-wide
// chunks are issued together; the tensor scale is loaded with the first four.
template <int FMT, bool WIDE>
__device__ __forceinline__ f32x4 gemv16_row_impl(const WDesc& w, int e, int n0, const uint16_t* hrow,
                                                 int K, ScaleXchg& sx) {
  const int lane = __lane_id(), r = lane & 15, g = lane >> 4;
  const int row = n0 + r;
  const uint8_t* rp = w.codes + e * w.stride_codes + (size_t)row * row_bytes<FMT>(K);
  const uint8_t* sp = scale_row_ptr<FMT>(w, e, row);
  const uint16_t* brow = (r == 0) ? hrow : nullptr;
  const int nch = (K + 127) / 128;
  constexpr int D = 4;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  float ts = 1.0f;
  constexpr bool wide = WIDE && FMT != FMT_FP8;
  for (int cb = 0; cb < nch; cb += D) {
    ARaw<FMT> ar[D];
    u32x4 bx[D][4];
    uint2 sw = make_uint2(0u, 0u);
    if constexpr (wide) {
#pragma unroll
      for (int d = 0; d < D; ++d)
        ar[d] = load_a<FMT, false>(cb + d < nch ? rp : nullptr, nullptr, cb + d, g, K);
      sw = load_scale_word<FMT>(sp, cb + g, nch);
    } else {
#pragma unroll
      for (int d = 0; d < D; ++d) ar[d] = load_a<FMT>(cb + d < nch ? rp : nullptr, sp, cb + d, g, K);
    }
    if constexpr (FMT == FMT_NVFP4) {
      if (cb == 0) ts = w.tscale[e];
    }
#pragma unroll
    for (int d = 0; d < D; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        bx[d][i] = load_b(cb + d < nch ? brow : nullptr, 128 * (cb + d) + 32 * g + 8 * i, K);
    if constexpr (wide) {
      const uint2 o = exchange_scales<FMT>(sw, sx, r, g);
#pragma unroll
      for (int d = 0; d < D; ++d) ar[d].s = scale_of_chunk<FMT>(o, d);
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (cb + d >= nch) break;
      f32x4 t = (FMT == FMT_FP8) ? f32x4{0.f, 0.f, 0.f, 0.f} : acc;
      t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_a<FMT, 0>(ar[d]), as_bf16x8(bx[d][0]), t, 0, 0, 0);
      t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_a<FMT, 1>(ar[d]), as_bf16x8(bx[d][1]), t, 0, 0, 0);
      t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_a<FMT, 2>(ar[d]), as_bf16x8(bx[d][2]), t, 0, 0, 0);
      t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_a<FMT, 3>(ar[d]), as_bf16x8(bx[d][3]), t, 0, 0, 0);
      if constexpr (FMT == FMT_FP8)
        acc = acc + ar[d].s * t;
      else
        acc = t;
    }
  }
  return acc * ts;
}

template <int FMT>
__device__ __forceinline__ f32x4 gemv16_row(const WDesc& w, int e, int n0, const uint16_t* hrow,
                                            int K, ScaleXchg& sx) {
  if constexpr (FMT != FMT_FP8) {
    if (w.wide) return gemv16_row_impl<FMT, true>(w, e, n0, hrow, K, sx);
  }
  return gemv16_row_impl<FMT, false>(w, e, n0, hrow, K, sx);
}

// Down projection of every routed slot of a token and of the shared expert,
// combined in the same kernel: block (t, 16-column tile of H) of one
// wavefront per slot (at most 12; wavefront w takes slots w, w + 12, ...;
// slot k = the shared expert), each writes its 16
// outputs y_j to LDS, then out[t] = bf16(sum_j w_j * y_j + y_shared) in slot
// order.  No per-pair y goes through memory.
constexpr int kDcCols = 16;
constexpr int kDcMaxWaves = 12;  // one wavefront per slot up to 12 slots (168 VGPRs each)
// On a grid smaller than the GPU (one token), input rows up to this length
// are staged in LDS by the whole wavefront (one 16-byte load per lane per 512
// values) instead of being loaded by the four lanes that feed the MFMA's B
// column (16 load instructions of 4 lanes each per 512 values, which queue in
// the CU's address path): one-token NVFP4 layer 24.9 -> 24.2 us.  On larger
// grids the staging's LDS costs more occupancy than it saves (8-token NVFP4
// layer +3.6 us, 8-token wide-FP8 layer +55 us).
constexpr int kDcStageK = 2048;
constexpr int kDcStageMaxBlocks = 255;

// RFMT / SFMT: the formats of the routed and the shared down projections
// (a layer's down projections may use another format than its gate/up).
// STAGE: input rows staged in LDS (a.dc_stage_k values per wavefront).
template <int RFMT, int SFMT, bool STAGE>
__global__ __launch_bounds__(kDcMaxWaves * kWave) void decode_down_combine_kernel(DecodeArgs a) {
  __shared__ float yp[kMaxTopK + 1][kDcCols];
  __shared__ float wp[kMaxTopK];
  __shared__ ScaleXchg sxd[kDcMaxWaves];
  extern __shared__ __attribute__((aligned(16))) uint16_t hst_dyn[];  // [waves][stage K] when staged
  const int ntiles = a.H / kDcCols;
  const int t = blockIdx.x / ntiles, tile = blockIdx.x % ntiles;
  const int n0 = tile * kDcCols;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int nslots = a.k + ((SFMT != 0) ? 1 : 0);
  const int nwaves = blockDim.x / kWave;
  for (int j = wave; j < nslots; j += nwaves) {
    f32x4 y = f32x4{0.f, 0.f, 0.f, 0.f};
    float wj = 0.f;
    if constexpr (STAGE) {
      // the slot's input row (h of pair t*k+j, or the shared expert's h of
      // token t) staged in LDS, requested before the expert id is read
      const bool routed = j < a.k;
      const int K = routed ? a.I : a.I_shared;
      const uint16_t* hrow =
          routed ? a.h + (size_t)(t * a.k + j) * a.I : a.hs + (size_t)t * a.I_shared;
      uint16_t* hl = hst_dyn + wave * a.dc_stage_k;
      for (int i = lane * 8; i < K; i += kWave * 8)
        *reinterpret_cast<u32x4*>(hl + i) = *reinterpret_cast<const u32x4*>(hrow + i);
      __builtin_amdgcn_wave_barrier();  // this wavefront's LDS reads follow its writes
      if (routed) {
        const int p = t * a.k + j;
        const int e = a.ids[p];
        wj = a.w[p];  // the combine weight, fetched with the expert id
        if ((unsigned)e < (unsigned)a.E) y = gemv16_row<RFMT>(a.down, e, n0, hl, a.I, sxd[wave]);
      } else if constexpr (SFMT != 0) {
        y = gemv16_row<SFMT>(a.sd, 0, n0, hl, a.I_shared, sxd[wave]);
      }
    } else {
      if (j < a.k) {
        const int p = t * a.k + j;
        const int e = a.ids[p];
        wj = a.w[p];  // the combine weight, fetched with the expert id
        if ((unsigned)e < (unsigned)a.E)
          y = gemv16_row<RFMT>(a.down, e, n0, a.h + (size_t)p * a.I, a.I, sxd[wave]);
      } else if constexpr (SFMT != 0) {
        y = gemv16_row<SFMT>(a.sd, 0, n0, a.hs + (size_t)t * a.I_shared, a.I_shared, sxd[wave]);
      }
    }
    if ((lane & 15) == 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) yp[j][4 * (lane >> 4) + q] = y[q];
    }
    if (lane == 0 && j < a.k) wp[j] = wj;
  }
  __syncthreads();
  if ((int)threadIdx.x < kDcCols) {
    const int c = threadIdx.x;
    float acc = 0.f;
    for (int j = 0; j < a.k; ++j) acc = fmaf(wp[j], yp[j][c], acc);
    if constexpr (SFMT != 0) acc = acc + yp[a.k][c];
    a.out[(size_t)t * a.H + n0 + c] = f32_to_bf16(acc);
  }
}

// Gate/up formats (routed, shared) pick the gate/up kernel; down formats
// (routed, shared) pick the down-combine kernel.
struct GateUpLaunch {
  template <int RFMT, int SFMT>
  static hipError_t run(const DecodeArgs& a, hipStream_t s) {
    const int nsg = (SFMT != 0) ? a.I_shared / gemv_rows_per_block<kOpGateUp>() : 0;
    const int ngu = a.T * a.k * (a.I / gemv_rows_per_block<kOpGateUp>());
    if constexpr ((RFMT == FMT_NVFP4 || RFMT == FMT_MXFP4) && kSharedLean<SFMT>) {
      if (lean_fits(a) && shared_lean_fits<SFMT>(a)) {
        // the aligned tile's LDS: reductions, scale exchange, up to 16 input rows
        const size_t dyn = offsetof(LeanSmem, x) + (size_t)std::min(a.T, kLeanMaxRows) * a.H * 2;
        return launch(decode_gateup_kernel<RFMT, SFMT, true>, dim3(nsg + ngu), dim3(kWave * kGuWK),
                      dyn, s, a);
      }
    }
    return launch(decode_gateup_kernel<RFMT, SFMT, false>, dim3(nsg + ngu), dim3(kWave * kGuWK), 0,
                  s, a);
  }
};

// The per-expert down launch and the combine, for 2 to 32 tokens when the
// down projections have lean tiles and the y buffers are given.
template <int RFMT, int SFMT>
constexpr bool kDownLean = (RFMT == FMT_NVFP4 || RFMT == FMT_MXFP4 || RFMT == FMT_FP8) &&
                           (SFMT == 0 || SFMT == FMT_NVFP4 || SFMT == FMT_MXFP4 || SFMT == FMT_FP8);

struct DownLaunch {
  template <int RFMT, int SFMT>
  static hipError_t run(const DecodeArgs& a, hipStream_t s) {
    if constexpr (kDownLean<RFMT, SFMT>) {
      const bool fits = a.T >= 2 && a.y != nullptr && (SFMT == 0 || a.ys != nullptr) &&
                        down_lean_fits<RFMT>(a.down, a.I, a.H) &&
                        (SFMT == 0 || down_lean_fits<SFMT>(a.sd, a.I_shared, a.H));
      if (fits) {
        const int ntiles = a.H / kDnRows;
        const int nsd = (SFMT != 0) ? ntiles : 0;
        const int kmax = std::max(a.I, (SFMT != 0) ? a.I_shared : 0);
        const size_t dyn = offsetof(DownSmem, x) + (size_t)std::min(a.T, kLeanMaxRows) * kmax * 2;
        hipError_t err = launch(decode_down_kernel<RFMT, SFMT>, dim3(nsd + a.T * a.k * ntiles),
                                dim3(kWave * kGuWK), dyn, s, a);
        if (err != hipSuccess) return err;
        return launch_combine(a.y, a.w, nullptr, (SFMT != 0) ? a.ys : nullptr, a.T, a.k, a.H, a.out,
                              s);
      }
    }
    // One wavefront per slot (one round trip per block) when the grid is
    // smaller than the GPU; otherwise 8 per block keep more blocks resident.
    const int nslots = a.k + ((SFMT != 0) ? 1 : 0);
    const int nblocks = a.T * (a.H / kDcCols);
    const int dcw = (nblocks < 256) ? (nslots < kDcMaxWaves ? nslots : kDcMaxWaves)
                                    : (nslots < 8 ? nslots : 8);
    const int kmax = std::max(a.I, (SFMT != 0) ? a.I_shared : 0);
    DecodeArgs b = a;
    b.dc_stage_k = (nblocks <= kDcStageMaxBlocks && kmax <= kDcStageK) ? kmax : 0;
    if (b.dc_stage_k > 0)
      return launch(decode_down_combine_kernel<RFMT, SFMT, true>, dim3(nblocks), dim3(dcw * kWave),
                    (size_t)dcw * b.dc_stage_k * sizeof(uint16_t), s, b);
    return launch(decode_down_combine_kernel<RFMT, SFMT, false>, dim3(nblocks), dim3(dcw * kWave), 0,
                  s, b);
  }
};

// (routed format, shared format or 0) -> L::run<RFMT, SFMT>
template <class L, int RFMT>
hipError_t by_shared_format(int sfmt, const DecodeArgs& a, hipStream_t s) {
  switch (sfmt) {
    case 0: return L::template run<RFMT, 0>(a, s);
    case FMT_NVFP4: return L::template run<RFMT, FMT_NVFP4>(a, s);
    case FMT_MXFP4: return L::template run<RFMT, FMT_MXFP4>(a, s);
    case FMT_FP8: return L::template run<RFMT, FMT_FP8>(a, s);
    case FMT_MXFP8: return L::template run<RFMT, FMT_MXFP8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <class L>
hipError_t by_formats(int rfmt, int sfmt, const DecodeArgs& a, hipStream_t s) {
  switch (rfmt) {
    case FMT_NVFP4: return by_shared_format<L, FMT_NVFP4>(sfmt, a, s);
    case FMT_MXFP4: return by_shared_format<L, FMT_MXFP4>(sfmt, a, s);
    case FMT_FP8: return by_shared_format<L, FMT_FP8>(sfmt, a, s);
    case FMT_MXFP8: return by_shared_format<L, FMT_MXFP8>(sfmt, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool decode_rows_ok(const DecodeArgs& a) {
  if (a.T <= kTmax) return true;
  // 9..32 rows: only the lean gate/up and the per-expert down, which take a
  // group's rows in chunks of the MFMA B operand's 16 columns; pair slots
  // <= 512 (two rounds of derive_group)
  if (a.T > kDecodeMaxRows || a.T * a.k > kPmax) return false;
  if (!(a.gate.fmt == FMT_NVFP4 || a.gate.fmt == FMT_MXFP4) || !lean_fits(a)) return false;
  if (a.has_shared) {
    const int f = a.sg.fmt;
    if (!(f == FMT_FP8 || ((f == FMT_NVFP4 || f == FMT_MXFP4) && a.sg.wide && a.su.wide)))
      return false;
  }
  auto down_ok = [&](const WDesc& w, int K) {
    if (a.H % kDnRows != 0 || K > kLeanMaxK || K % 512 != 0) return false;
    return ((w.fmt == FMT_NVFP4 || w.fmt == FMT_MXFP4) && w.wide) || w.fmt == FMT_FP8;
  };
  return down_ok(a.down, a.I) && (!a.has_shared || down_ok(a.sd, a.I_shared));
}

DecodePlan decode_plan(int T, int H, int E) {
  DecodePlan p;
  p.RS = (H + kRH - 1) / kRH;
  p.CS = (E + kRouterCols - 1) / kRouterCols;
  p.down_tiles = (H + gemv_rows_per_block<kOpDown>() - 1) / gemv_rows_per_block<kOpDown>();
  (void)T;
  return p;
}

hipError_t launch_decode_router(const DecodeArgs& a, hipStream_t s) {
  if (a.T == 1)
    return launch(decode_router_kernel<1, float>, dim3(a.RS * a.CS), dim3(256), 0, s, a);
  const dim3 grid(a.RS * a.CS, (a.T + kTmax - 1) / kTmax);
  if (a.T <= kTmax) return launch(decode_router_kernel<kTmax, float>, grid, dim3(256), 0, s, a);
  return launch(decode_router_kernel<kTmax, double>, grid, dim3(256), 0, s, a);
}

// The top-k on the slice sums the router wrote (fp32 up to 8 tokens).
hipError_t launch_decode_topk(const DecodeArgs& a, hipStream_t s) {
  if (a.T <= kTmax) return launch(decode_topk_kernel<float>, dim3(a.T), dim3(kTopkThreads), 0, s, a);
  return launch(decode_topk_kernel<double>, dim3(a.T), dim3(kTopkThreads), 0, s, a);
}

hipError_t launch_decode_route(const DecodeArgs& a, hipStream_t s) {
  hipError_t err = launch_decode_router(a, s);
  if (err != hipSuccess) return err;
  return launch_decode_topk(a, s);
}

hipError_t launch_decode_gate_up(const DecodeArgs& a, hipStream_t s) {
  return by_formats<GateUpLaunch>(a.gate.fmt, a.has_shared ? a.sg.fmt : 0, a, s);
}

hipError_t launch_decode_experts(const DecodeArgs& a, hipStream_t s) {
  hipError_t err = by_formats<GateUpLaunch>(a.gate.fmt, a.has_shared ? a.sg.fmt : 0, a, s);
  if (err != hipSuccess) return err;
  return by_formats<DownLaunch>(a.down.fmt, a.has_shared ? a.sd.fmt : 0, a, s);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  hipError_t err = launch_decode_router(a, s);
  if (err != hipSuccess) return err;
  err = launch_decode_topk(a, s);
  if (err != hipSuccess) return err;
  err = by_formats<GateUpLaunch>(a.gate.fmt, a.has_shared ? a.sg.fmt : 0, a, s);
  if (err != hipSuccess) return err;
  return by_formats<DownLaunch>(a.down.fmt, a.has_shared ? a.sd.fmt : 0, a, s);
}

}  // namespace moe
