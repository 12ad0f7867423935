// Prefill grouped expert GEMM for FP4 experts (NVFP4, MXFP4) with K a
// multiple of 64: every operand moved global -> LDS by the LDS-DMA loads, and
// each wavefront decodes its own weight fragments from the raw checkpoint
// codes in LDS.
//
// The rows, exact chain and epilogue arithmetic of grouped_gemm_kernel
// (weights decoded to bf16 exactly: NVFP4 E2M1 x E4M3 block scale, MXFP4
// E2M1 x E8M0; v_mfma_f32_16x16x32_bf16, K in steps of 64), on tiles of 128
// permuted rows x 256 weight rows (gate/up: 128 gate + the matching 128 up
// rows), but:
//
// * no staging registers: bf16 activation rows (gathered through
//   perm_to_pair), the packed E2M1 codes and the block-scale words of a step
//   are DMA'd into LDS (global_load_lds), two stages, one bare barrier per
//   step after an explicit vmcnt wait;
// * the weight tile stays packed in LDS (8 KiB per step instead of 32 KiB of
//   bf16); on a 1 x 4 wavefront grid (128 rows x 64 weight rows each) a
//   wavefront reads the 4 bytes (8 codes) and the scale byte of each of its B
//   fragments and decodes them in registers, so every fragment is decoded
//   once;
// * the output tile leaves through LDS as 16-byte row vectors.
//
// LDS rows are unpadded (a DMA instruction fills one contiguous KiB) and the
// 16-byte pieces are XOR-swizzled per row: piece P of a 128-byte activation
// row r at slot P ^ ((r >> 1) & 7), of a 32-byte code row at P ^ ((r >> 3) & 1),
// so the fragment reads of consecutive rows fall in distinct banks.
#include <type_traits>

#include "gemv_core.cuh"

namespace moe {
namespace {

constexpr int BM = kGemmTileM, BN = 256, BK = 64;
constexpr int kXcds = 8;
constexpr int kStages = 2;

template <int FMT>
struct DLayout {
  static constexpr int a_off = 0;                   // [128 rows][128 B] bf16
  static constexpr int b_off = BM * 128;            // [BN rows][32 B] E2M1 codes
  // Scale words of a step: NVFP4 4 bytes, MXFP4 2 bytes per weight row.  A
  // DMA of 4 bytes or fewer lands at a 4-byte pitch per lane (M0 + 4 * lane),
  // so each row has a 4-byte slot whatever the word's size.
  static constexpr int s_off = b_off + BN * 32;
  static constexpr int s_row = (FMT == FMT_NVFP4) ? 4 : 2;  // bytes loaded per row
  static constexpr int s_pitch = 4;                          // LDS bytes per row
  static constexpr int s_bytes = BN * s_pitch;               // one 64-lane region per wave
  static constexpr int stage = s_off + s_bytes;
  static_assert(BN == 4 * 64, "each wavefront DMAs the scale words of 64 weight rows");
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <int SIZE>
__device__ __forceinline__ void dma(const void* src, uint8_t* lds) {
  static_assert(SIZE == 2 || SIZE == 4 || SIZE == 16, "LDS-DMA size");
  if constexpr (SIZE == 16)
    __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds, 16, 0, 0);
  else if constexpr (SIZE == 4)
    __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds, 4, 0, 0);
  else
    __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds, 2, 0, 0);
}

// vmcnt(N) and lgkmcnt(0) (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4));
}

struct DParams {
  WDesc w0, w1;
  const uint16_t* in;
  void* out;
  const int2* tiles;
  const int* n_tiles;
  const int* offsets;
  const int* perm_to_pair;
  int topk, T, in_rows, in_rows_total, max_rt, ntn;
};

template <int OP>
__device__ __forceinline__ int input_row(const DParams& p, int pr, int m0, int m1) {
  const int row = pr < m1 ? pr : m0;
  int ir = (p.tiles != nullptr && OP == kOpGateUp) ? p.perm_to_pair[row] / p.topk : row;
  if ((unsigned)ir >= (unsigned)p.in_rows) ir = 0;
  return ir;
}

// 8 weights of one B fragment (8 consecutive K) from their 4 code bytes.
template <int FMT>
__device__ __forceinline__ bf16x8 decode_frag(uint32_t d, uint32_t sbyte) {
  union {
    bf16x8 v;
    uint32_t u[4];
    bf16x2 h[4];
  } r;
  if constexpr (FMT == FMT_NVFP4) {
    const float s = e4m3x2_to_f32(sbyte)[0];
    const f32x2 f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 0);
    const f32x2 f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 1);
    const f32x2 f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 2);
    const f32x2 f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 3);
    r.u[0] = pack_hi16(f0[0] * s, f0[1] * s);
    r.u[1] = pack_hi16(f1[0] * s, f1[1] * s);
    r.u[2] = pack_hi16(f2[0] * s, f2[1] * s);
    r.u[3] = pack_hi16(f3[0] * s, f3[1] * s);
  } else {
    const float s = __uint_as_float(sbyte << 23);
    r.h[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 0);
    r.h[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 1);
    r.h[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 2);
    r.h[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 3);
  }
  return r.v;
}

template <int FMT>
struct DWaves {
  // 1 x 4 for both formats (measured at T=8192: NVFP4 layer -5..-8%, MXFP4
  // layer -2..-3% against 2 x 2); the grid stays a parameter.
  static constexpr int KWM = 1, KWN = 4 / KWM;
  static constexpr int R = BM / KWM / 16, C = BN / KWN / 16;
};

template <int FMT, int OP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void grouped_gemm_d_kernel(
    DParams p) {
  using D = DLayout<FMT>;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kStages * D::stage];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n_rt = (p.tiles == nullptr) ? (p.T + BM - 1) / BM : min(*p.n_tiles, p.max_rt);
  const int live = n_rt * p.ntn;
  const int per = (live + kXcds - 1) / kXcds;
  const int xcd = blockIdx.x % kXcds, local = blockIdx.x / kXcds;
  const int idx = xcd * per + local;
  if (local >= per || idx >= live) return;
  const int mt = idx / p.ntn, nt = idx % p.ntn;
  int e, m0, m1;
  if (p.tiles == nullptr) {
    e = 0;
    m0 = mt * BM;
    m1 = p.T;
  } else {
    const int2 tl = p.tiles[mt];
    e = tl.x;
    m0 = tl.y;
    m1 = p.offsets[e + 1];
    if (m0 < 0 || m1 > p.in_rows_total || m0 >= m1) return;
  }
  const int N = p.w0.rows, K = p.w0.cols;
  const int n0 = nt * ((OP == kOpGateUp) ? BN / 2 : BN);
  const int nk = K / BK;

  // ---- DMA sources of this lane ----
  // A: 16 KiB-chunks of 8 rows x 128 B; wave w takes chunks 4w .. 4w+3.
  const uint16_t* asrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (4 * wave + i) * 8 + (lane >> 3);
    const int piece = (lane & 7) ^ ((r >> 1) & 7);
    asrc[i] = p.in + (size_t)input_row<OP>(p, m0 + r, m0, m1) * K + 8 * piece;
  }
  // B codes: KiB-chunks of 32 rows x 32 B; wave w takes chunks 2w, 2w+1.
  const uint8_t* bsrc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 64 * wave + 32 * i + (lane >> 1);
    const int piece = (lane & 1) ^ ((r >> 3) & 1);
    const WDesc& wq = (OP == kOpGateUp && r >= BN / 2) ? p.w1 : p.w0;
    const int wr0 = (OP == kOpGateUp) ? n0 + (r & (BN / 2 - 1)) : n0 + r;
    const int wr = wr0 < N ? wr0 : N - 1;
    bsrc[i] = wq.codes + e * wq.stride_codes + (size_t)wr * (K / 2) + 16 * piece;
  }
  // scale words: wave w the weight rows 64w + lane
  const uint8_t* ssrc;
  {
    const int r = 64 * wave + lane;
    const WDesc& wq = (OP == kOpGateUp && r >= BN / 2) ? p.w1 : p.w0;
    const int wr0 = (OP == kOpGateUp) ? n0 + (r & (BN / 2 - 1)) : n0 + r;
    const int wr = wr0 < N ? wr0 : N - 1;
    ssrc = reinterpret_cast<const uint8_t*>(wq.scales) + e * wq.stride_scales +
           (size_t)wr * (K / (FMT == FMT_NVFP4 ? 16 : 32));
  }
  const int sdst = D::s_off + 64 * D::s_pitch * wave;

  auto issue = [&](int ks) {
    uint8_t* st = lds + (ks % kStages) * D::stage;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma<16>(asrc[i] + ks * BK, st + D::a_off + 1024 * (4 * wave + i));
#pragma unroll
    for (int i = 0; i < 2; ++i) dma<16>(bsrc[i] + ks * (BK / 2), st + D::b_off + 1024 * (2 * wave + i));
    dma<D::s_row>(ssrc + ks * D::s_row, st + sdst);
  };

  // Wavefront grid KWM x KWN over the 128 x 128 tile; each wavefront holds R x
  // C fragments of 16 x 16.  1 x 4 (128 rows x 32 weight rows each): every B
  // fragment is decoded by one wavefront only (an NVFP4 decode multiplies by
  // the E4M3 scale in fp32 per weight), at the price of reading each A
  // fragment four times from LDS instead of twice on a 2 x 2 grid.  Gate/up:
  // a wavefront's columns are C/2 gate fragments and the C/2 matching up
  // fragments.
  using L = DWaves<FMT>;
  constexpr int R = L::R, C = L::C;
  const int wm = wave / L::KWN, wn = wave % L::KWN;
  constexpr int kWaveRows = BM / L::KWM, kWaveCols = BN / L::KWN;
  int bcol[C];
#pragma unroll
  for (int c = 0; c < C; ++c)
    bcol[c] = (OP == kOpGateUp)
                  ? ((c < C / 2) ? (kWaveCols / 2) * wn + 16 * c
                                 : BN / 2 + (kWaveCols / 2) * wn + 16 * (c - C / 2))
                  : kWaveCols * wn + 16 * c;
  f32x4 acc[R][C];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < C; ++c) acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int vrows = m1 - m0 - kWaveRows * wm;
  const int vr = vrows <= 0 ? 0 : min(R, (vrows + 15) / 16);
  const int g = lane >> 4, lr = lane & 15;

  auto compute = [&](int ks, auto full_t) {
    constexpr bool FULL = decltype(full_t)::value;
    const uint8_t* st = lds + (ks % kStages) * D::stage;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      // B fragments: row bcol[c] + lr, K kk + 8g .. +8: 4 code bytes at byte
      // 4g of the row's 16-byte piece kk / 32, and the scale byte of that K
      bf16x8 bfr[C];
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const int row = bcol[c] + lr;
        const int slot = (kk >> 5) ^ ((row >> 3) & 1);
        const uint32_t d = *reinterpret_cast<const uint32_t*>(st + D::b_off + row * 32 + 16 * slot + 4 * g);
        const int sb = (FMT == FMT_NVFP4) ? (kk >> 4) + (g >> 1) : (kk >> 5);
        const uint32_t sbyte = st[D::s_off + row * D::s_pitch + sb];
        bfr[c] = decode_frag<FMT>(d, sbyte);
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (!FULL && r >= vr) continue;
        const int row = kWaveRows * wm + 16 * r + lr;
        const int slot = ((kk >> 3) + g) ^ ((row >> 1) & 7);
        const bf16x8 af = *reinterpret_cast<const bf16x8*>(st + D::a_off + row * 128 + 16 * slot);
#pragma unroll
        for (int c = 0; c < C; ++c)
          acc[r][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr[c], acc[r][c], 0, 0, 0);
      }
    }
  };

  // stage 0 up front; at step ks: this wave's loads of stage ks landed (the
  // next stage's may be in flight) and its LDS reads of step ks-1 done,
  // barrier, issue step ks+1 into the buffer of step ks-1, compute step ks.
  auto main_loop = [&](auto full_t) {
    issue(0);
    for (int ks = 0; ks < nk; ++ks) {
      wait_vm_lds<0>();
      __builtin_amdgcn_s_barrier();
      if (ks + 1 < nk) issue(ks + 1);
      compute(ks, full_t);
    }
  };
  if (m1 - m0 >= BM)
    main_loop(std::true_type{});
  else
    main_loop(std::false_type{});

  const float ts0 = (FMT == FMT_NVFP4) ? p.w0.tscale[e] : 1.0f;
  const float ts1 = (FMT == FMT_NVFP4) ? p.w1.tscale[e] : 1.0f;
  // ---- epilogue: the tile goes through LDS so that the stores are 16-byte
  // vectors covering whole row segments (a fragment lane holds one column of
  // four rows; storing from the fragments writes 4-byte pieces).  The K
  // loop's LDS is free once every wavefront has passed the barrier.
  const int col = lane & 15;
  __syncthreads();
  if constexpr (OP == kOpGateUp) {
    // h tile: BM rows x BN/2 bf16 columns, one pass; staged rows of BN/2 + 8
    constexpr int HW = BN / 2, P = HW + 8;
    static_assert(BM * P * 2 <= kStages * D::stage, "staged h tile fits");
    uint16_t* st = reinterpret_cast<uint16_t*>(lds);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int lr = kWaveRows * wm + 16 * r + 4 * (lane >> 4) + j;
#pragma unroll
        for (int c = 0; c < C / 2; ++c) {
          const float hv = silu_fast(acc[r][c][j] * ts0) * (acc[r][c + C / 2][j] * ts1);
          st[lr * P + (kWaveCols / 2) * wn + 16 * c + col] = f32_to_bf16(hv);
        }
      }
    __syncthreads();
    // thread -> (row tid / TPR + RPP q, 8 columns at 8 * (tid % TPR))
    constexpr int TPR = HW / 8, RPP = 256 / TPR;
    const int cb = 8 * (tid % TPR);
    const int n = nt * HW + cb;
#pragma unroll
    for (int q = 0; q < BM / RPP; ++q) {
      const int lr = tid / TPR + RPP * q;
      const int row = m0 + lr;
      if (row >= m1) continue;
      const u32x4 v = *reinterpret_cast<const u32x4*>(st + lr * P + cb);
      uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + (size_t)row * N + n;
      if (n + 7 < N) {
        *reinterpret_cast<u32x4*>(o) = v;
      } else {
        const uint16_t* hs = reinterpret_cast<const uint16_t*>(&v);
        for (int i = 0; i < 8; ++i)
          if (n + i < N) o[i] = hs[i];
      }
    }
  } else {
    // y tile: BM rows x BN fp32 columns in parts of QR rows; staged rows of
    // BN + 4 floats (the fragment writes of the four 16-lane groups land in
    // distinct banks)
    constexpr int P = BN + 4, QR = (BN == 256) ? 32 : 64;
    static_assert(QR * P * 4 <= kStages * D::stage, "staged part of the y tile fits");
    float* st = reinterpret_cast<float*>(lds);
    constexpr int TPR = BN / 4, RPP = 256 / TPR;
    const int cb = 4 * (tid % TPR);
    const int n = n0 + cb;
#pragma unroll
    for (int part = 0; part < BM / QR; ++part) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int r0 = kWaveRows * wm + 16 * r;  // first tile row of fragment row r
        if (r0 / QR != part) continue;
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            st[(r0 - QR * part + 4 * (lane >> 4) + j) * P + kWaveCols * wn + 16 * c + col] =
                acc[r][c][j] * ts0;
      }
      __syncthreads();
      // thread -> (row tid / TPR + RPP q, 4 columns at 4 * (tid % TPR)); N % 4 == 0
#pragma unroll
      for (int q = 0; q < QR / RPP; ++q) {
        const int lr = tid / TPR + RPP * q;
        const int row = m0 + QR * part + lr;
        if (row < m1 && n < N)
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + (size_t)row * N + n) =
              *reinterpret_cast<const f32x4*>(st + lr * P + cb);
      }
      if (part + 1 < BM / QR) __syncthreads();
    }
  }
}

template <int FMT, int OP>
hipError_t launch_d(DParams p, int n_row_tiles, hipStream_t s) {
  const int ntn = (OP == kOpGateUp) ? (p.w0.rows + BN / 2 - 1) / (BN / 2) : (p.w0.rows + BN - 1) / BN;
  p.ntn = ntn;
  p.max_rt = n_row_tiles;
  const int per = (n_row_tiles * ntn + kXcds - 1) / kXcds;
  if (per == 0) return hipSuccess;
  return launch(grouped_gemm_d_kernel<FMT, OP>, dim3(per * kXcds), dim3(256), 0, s, p);
}

}  // namespace

bool grouped_gemm_dma_fits(int op, const WDesc& w0, const WDesc& w1) {
  // FP4 only: the 16-byte code pieces of a step are 64 K of one row.
  const bool fmt_ok = w0.fmt == FMT_MXFP4 || w0.fmt == FMT_NVFP4;
  if (!fmt_ok || w1.fmt != w0.fmt || w0.cols % BK != 0) return false;
  // the epilogue stores aligned 16-byte column groups: 8 bf16 of h, 4 fp32 of y
  if (w0.rows % ((op == kOpGateUp) ? 8 : 4) != 0) return false;
  // the scale word of a step (4 bytes NVFP4, 2 bytes MXFP4) is one aligned DMA
  // and the 16-byte code pieces are aligned DMAs too
  const uintptr_t a = (w0.fmt == FMT_NVFP4) ? 4 : 2;
  for (const WDesc* w : {&w0, &w1}) {
    if (reinterpret_cast<uintptr_t>(w->scales) % a != 0 || w->stride_scales % (long long)a != 0)
      return false;
    if (reinterpret_cast<uintptr_t>(w->codes) % 16 != 0 || w->stride_codes % 16 != 0) return false;
  }
  return true;
}

hipError_t launch_grouped_gemm_dma(int op, const WDesc& w0, const WDesc& w1, const GroupArgs& g,
                                   const int* tiles, const int* n_tiles, int max_tiles,
                                   const uint16_t* in, void* out, hipStream_t s) {
  if (!grouped_gemm_dma_fits(op, w0, w1)) return hipErrorInvalidValue;
  DParams p;
  p.w0 = w0;
  p.w1 = w1;
  p.in = in;
  p.out = out;
  p.topk = g.topk;
  p.T = g.T;
  p.offsets = g.offsets;
  p.perm_to_pair = g.perm_to_pair;
  p.ntn = 0;
  p.max_rt = 0;
  p.in_rows_total = g.T * g.topk;
  int nrt;
  if (g.shared) {
    p.tiles = nullptr;
    p.n_tiles = nullptr;
    nrt = (g.T + BM - 1) / BM;
    p.in_rows = g.T;
  } else {
    p.tiles = reinterpret_cast<const int2*>(tiles);
    p.n_tiles = n_tiles;
    nrt = max_tiles;
    p.in_rows = (op == kOpGateUp) ? g.T : g.T * g.topk;
  }
  const bool gu = op == kOpGateUp;
  if (w0.fmt == FMT_NVFP4)
    return gu ? launch_d<FMT_NVFP4, kOpGateUp>(p, nrt, s) : launch_d<FMT_NVFP4, kOpDown>(p, nrt, s);
  return gu ? launch_d<FMT_MXFP4, kOpGateUp>(p, nrt, s) : launch_d<FMT_MXFP4, kOpDown>(p, nrt, s);
}

}  // namespace moe
