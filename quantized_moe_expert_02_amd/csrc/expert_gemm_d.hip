// Prefill grouped expert GEMM for FP4 experts (NVFP4, MXFP4) with K a
// multiple of 64: every operand moved global -> LDS by the LDS-DMA loads, and
// each wavefront decodes its own weight fragments from the raw checkpoint
// codes in LDS.
//
// The rows, exact chain and epilogue arithmetic of grouped_gemm_kernel
// (weights decoded to bf16 exactly: NVFP4 E2M1 x E4M3 block scale, MXFP4
// E2M1 x E8M0; v_mfma_f32_16x16x32_bf16, K in steps of 64), on tiles of 128
// permuted rows x 256 weight rows (gate/up: 128 gate + the matching 128 up
// rows), four wavefronts, two workgroups per CU, but:
//
// * no staging registers: bf16 activation rows (gathered through
//   perm_to_pair), the packed E2M1 codes and the block-scale words of a step
//   are DMA'd into LDS (buffer loads to LDS), three stages, one bare barrier
//   per step after an explicit vmcnt wait;
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
constexpr int kWaves = 4, kThreads = 64 * kWaves;
constexpr int kXcds = 8;
// Row tiles per run of the tile order (gemm_tile_order): one, i.e. column
// tiles fastest.  Runs of four left the 8192-token FP4 layers' time unchanged
// and raised the gate/up launch's HBM bytes (NVFP4 1.14 -> 1.25 GB): with
// K = 2048 the weights are reused within a run, but the activation rows of
// the tiles in flight no longer fit the L2 together.
constexpr int kRowRun = 1;
// Three stages of 24 KiB and two 4 KiB scale buffers: two steps in flight
// while one is computed, and two workgroups per CU fill the 160 KiB of LDS.
constexpr int kStages = 3;
constexpr int kAPerWave = BM * 128 / 1024 / kWaves;  // KiB-chunks of activations per wave and step
constexpr int kBPerWave = BN * 32 / 1024 / kWaves;   // KiB-chunks of codes per wave and step
// DMA instructions per lane and step when the tile's first 16 RV rows are
// multiplied: only those activation rows are loaded
template <int RV>
constexpr int dma_per_stage() { return RV / 2 + kBPerWave; }

template <int FMT>
struct DLayout {
  // a stage: one step's activations and codes
  static constexpr int a_off = 0;                   // [128 rows][128 B] bf16
  static constexpr int b_off = BM * 128;            // [BN rows][32 B] E2M1 codes
  static constexpr int stage = b_off + BN * 32;
  // Block scales arrive in chunks of kSC = 4 steps, in two buffers after the
  // stages.  A DMA lane moves one step's scale bytes of one row (NVFP4 4,
  // MXFP4 2: the alignment a scale row has with K % 64 == 0) and lands at a
  // 4-byte pitch, so a row holds [step][4 B] and one DMA instruction covers
  // 16 rows, touching one cache line per row where a per-step load would
  // touch one per lane.
  static constexpr int s_row = (FMT == FMT_NVFP4) ? 4 : 2;  // scale bytes per row and step
  static constexpr int kSC = 4;                              // steps per scale chunk
  static constexpr int kLpr = kSC;                           // DMA lanes per row
  static constexpr int kRpi = 64 / kLpr;                     // rows per DMA instruction
  static constexpr int kSpi = 64 / kRpi;                     // instructions per wave and chunk
  static constexpr int s_off = kStages * stage;              // [2][BN rows][16 B]
  static constexpr int s_buf = BN * 16;
  static constexpr int total = s_off + 2 * s_buf;
  static_assert(BN == kWaves * 64, "each wavefront DMAs the scale chunks of 64 weight rows");
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Buffer resource over [base, base + bytes), raw (stride 0) dword access
// (gfx9 word 3).  The DMA loads below take a per-lane offset fixed for the
// whole K loop and the step's offset in an SGPR, so a step's loads cost no
// vector address arithmetic; offsets past `bytes` read zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

template <int SIZE>
__device__ __forceinline__ void dma_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint8_t* lds) {
  static_assert(SIZE == 2 || SIZE == 4 || SIZE == 16, "LDS-DMA size");
  if constexpr (SIZE == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, (int)voff, (int)soff, 0, 0);
  else if constexpr (SIZE == 4)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 4, (int)voff, (int)soff, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 2, (int)voff, (int)soff, 0, 0);
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
  uint32_t in_bytes;  // in_rows * K * 2 < 2^31
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
  // 1 x 4: every B fragment is decoded by one wavefront (measured at T=8192:
  // NVFP4 layer -5..-8%, MXFP4 layer -2..-3% against 2 x 2); the grid stays
  // a parameter.
  static constexpr int KWM = 1, KWN = kWaves / KWM;
  static constexpr int R = BM / KWM / 16, C = BN / KWN / 16;
};

template <int FMT, int OP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void grouped_gemm_d_kernel(
    DParams p) {
  using D = DLayout<FMT>;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[D::total];
  // wave index in an SGPR: the DMA destinations (M0) are scalar arithmetic
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int n_rt = (p.tiles == nullptr) ? (p.T + BM - 1) / BM : min(*p.n_tiles, p.max_rt);
  const int live = n_rt * p.ntn;
  const int per = (live + kXcds - 1) / kXcds;
  const int xcd = blockIdx.x % kXcds, local = blockIdx.x / kXcds;
  const int idx = xcd * per + local;
  if (local >= per || idx >= live) return;
  const int2 tn = gemm_tile_order(idx, p.ntn, n_rt, kRowRun, p.tiles, p.offsets, BM);
  const int mt = tn.x, nt = tn.y;
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

  // ---- DMA sources of this lane: byte offsets in buffers fixed per wave ----
  // A: the first 16 RV tile rows (RV = 8, 4 or 2 by the rows the tile holds)
  // in KiB-chunks of 8 rows x 128 B; wave w takes chunks (RV/2) w ..
  // (RV/2) w + RV/2 - 1.  Set by main_loop.
  const __amdgpu_buffer_rsrc_t ra = buf_rsrc(p.in, p.in_bytes);
  uint32_t aoff[kAPerWave];
  auto set_aoff = [&](auto rv_t) {
    constexpr int NA = decltype(rv_t)::value / 2;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int r = (NA * wave + i) * 8 + (lane >> 3);
      const int piece = (lane & 7) ^ ((r >> 1) & 7);
      aoff[i] = (uint32_t)input_row<OP>(p, m0 + r, m0, m1) * (uint32_t)(2 * K) + 16 * piece;
    }
  };
  // B codes: KiB-chunks of 32 rows x 32 B; wave w takes chunks 2w, 2w+1 (the
  // weight rows 64w .. 64w+63), all rows of one matrix (gate/up: waves 0-1
  // gate rows, waves 2-3 up rows).
  static_assert(kBPerWave == 2, "a wave's code chunks cover its 64 scale rows");
  const WDesc& wq = (OP == kOpGateUp && 64 * wave >= BN / 2) ? p.w1 : p.w0;
  const __amdgpu_buffer_rsrc_t rb = buf_rsrc(wq.codes + e * wq.stride_codes, (uint32_t)N * (K / 2));
  uint32_t boff[kBPerWave];
#pragma unroll
  for (int i = 0; i < kBPerWave; ++i) {
    const int r = 64 * wave + 32 * i + (lane >> 1);
    const int piece = (lane & 1) ^ ((r >> 3) & 1);
    const int wr0 = (OP == kOpGateUp) ? n0 + (r & (BN / 2 - 1)) : n0 + r;
    const int wr = wr0 < N ? wr0 : N - 1;
    boff[i] = (uint32_t)wr * (K / 2) + 16 * piece;
  }
  // scale chunks: wave w the weight rows 64w .. 64w+63
  constexpr int kSpr = (FMT == FMT_NVFP4) ? 16 : 32;  // K per scale byte
  const uint32_t s_pitch = K / kSpr;                   // scale bytes per weight row
  const __amdgpu_buffer_rsrc_t rs =
      buf_rsrc(reinterpret_cast<const uint8_t*>(wq.scales) + e * wq.stride_scales, (uint32_t)N * s_pitch);

  // the stage is a compile-time constant so that every LDS address of a step
  // is a per-lane base plus an immediate offset
  auto issue = [&](int ks, auto stage_t, auto rv_t) {
    constexpr int NA = decltype(rv_t)::value / 2;
    uint8_t* st = lds + decltype(stage_t)::value * D::stage;
#pragma unroll
    for (int i = 0; i < NA; ++i)
      dma_buf<16>(ra, aoff[i], ks * BK * 2, st + D::a_off + 1024 * (NA * wave + i));
#pragma unroll
    for (int i = 0; i < kBPerWave; ++i)
      dma_buf<16>(rb, boff[i], ks * (BK / 2), st + D::b_off + 1024 * (kBPerWave * wave + i));
  };
  // scale chunk q (steps kSC q .. kSC q + kSC - 1) into buffer q % 2: row
  // [r][16 B] with r the tile row.  The chunk's byte offset is part of the
  // lane offset, so bytes past the last row's end read zeros (never used).
  auto issue_scales = [&](int q) {
#pragma unroll
    for (int i = 0; i < D::kSpi; ++i) {
      const int r = 64 * wave + D::kRpi * i + lane / D::kLpr;
      const int wr0 = (OP == kOpGateUp) ? n0 + (r & (BN / 2 - 1)) : n0 + r;
      const int wr = wr0 < N ? wr0 : N - 1;
      const uint32_t off = (uint32_t)wr * s_pitch + (D::kSC * q + lane % D::kLpr) * D::s_row;
      dma_buf<D::s_row>(rs, off, 0, lds + D::s_off + (q & 1) * D::s_buf + 16 * (64 * wave + D::kRpi * i));
    }
  };
  // the scale bytes of step j (buffer, step within the chunk), uniform
  auto sbase = [&](int j) {
    return lds + D::s_off + ((j / D::kSC) & 1) * D::s_buf + (j % D::kSC) * 4;
  };

  // Wavefront grid KWM x KWN over the 128 x 256 tile; each wavefront holds R x
  // C fragments of 16 x 16.  1 x 4 (128 rows x 64 weight rows each): every B
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

  // Per-lane LDS byte offsets within a stage, for the two 32-K halves h of a
  // step.  A wavefront's A fragment rows differ by multiples of 16 and its B
  // fragments start at rows that are multiples of 16, so the XOR swizzles
  // depend on the lane only and each fragment's offset is a lane base plus a
  // compile-time constant.  A fragment r: row 16r + lr, K 32h + 8g .. +8; B
  // fragment c: the 4 code bytes of weight row bcol[c] + lr at K 32h + 8g
  // and the scale byte of that K.
  const int wcol = bcol[0];  // bcol[c] = wcol + ccol(c)
  auto ccol = [](int c) {
    return (OP == kOpGateUp) ? ((c < C / 2) ? 16 * c : BN / 2 + 16 * (c - C / 2)) : 16 * c;
  };
  int a_lane[2], b_lane[2], s_lane[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    a_lane[h] = D::a_off + (kWaveRows * wm + lr) * 128 + 16 * ((4 * h + g) ^ ((lr >> 1) & 7));
    b_lane[h] = D::b_off + (wcol + lr) * 32 + 16 * (h ^ ((lr >> 3) & 1)) + 4 * g;
    s_lane[h] = (wcol + lr) * 16 + ((FMT == FMT_NVFP4) ? 2 * h + (g >> 1) : h);
  }

  // Software pipeline over half-steps.  While the MFMAs of one half run, the
  // wavefront reads the raw codes and scale bytes of the next half (from the
  // next step's stage after half 1), reads the next half's A fragments (each
  // one after the last MFMA on the fragment it replaces) and decodes the next
  // half's B fragments.  Only the first half of a tile waits for its decode.
  bf16x8 acur[R], bcur[C], bnxt[C];
  uint32_t rd[C], rsb[C];  // raw code words and scale bytes of the next half
  auto read_raw = [&](const uint8_t* st, const uint8_t* sp, int h) {
#pragma unroll
    for (int c = 0; c < C; ++c) {
      rd[c] = *reinterpret_cast<const uint32_t*>(st + b_lane[h] + ccol(c) * 32);
      rsb[c] = sp[s_lane[h] + ccol(c) * 16];
    }
  };
  auto read_a = [&](const uint8_t* st, int h, int r) {
    return *reinterpret_cast<const bf16x8*>(st + a_lane[h] + 2048 * r);
  };
  // decode VALU ops per B fragment (NVFP4: E4M3 scale, 4 conversions, 8
  // multiplies, 4 packs; MXFP4: 4 scaled conversions and the scale shift)
  constexpr int kDecV = (FMT == FMT_NVFP4) ? 17 : 5;
  // One half: MFMAs on (acur, bcur); reads of stage `stn` (scales at `spn`),
  // half hn; bnxt
  // decoded.  Instruction order: fragment row 0's MFMAs take the 2C raw reads,
  // every later MFMA but a row's last takes a share of the decode, and each
  // row's A read follows the row's last MFMA.
  auto half = [&](const uint8_t* stn, const uint8_t* spn, int hn, auto rv_t) {
    constexpr int RV = decltype(rv_t)::value;
    read_raw(stn, spn, hn);
#pragma unroll
    for (int r = 0; r < RV; ++r) {
#pragma unroll
      for (int c = 0; c < C; ++c)
        acc[r][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(acur[r], bcur[c], acc[r][c], 0, 0, 0);
      acur[r] = read_a(stn, hn, r);
    }
#pragma unroll
    for (int c = 0; c < C; ++c) {
      bnxt[c] = decode_frag<FMT>(rd[c], rsb[c]);
      // pins the decode to this half: without it the compiler sinks the
      // decode below the step's barrier, next to its first use
      asm volatile("" : "+v"(bnxt[c]));
    }
    static_assert(C == 4, "the instruction order below assumes 4 fragments per row");
    constexpr int kSlots = 3 * (RV - 1), kV = (C * kDecV + kSlots - 1) / kSlots;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, C, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, C, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int r = 1; r < RV; ++r) {
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kV, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#pragma unroll
    for (int c = 0; c < C; ++c) bcur[c] = bnxt[c];
  };

  // Stages: scale chunks 0 and 1 and steps 0, 1 and 2 are issued up front.
  // Step ks: its half 0 reads the last of stage ks (half 1) into registers;
  // then this wave's loads of step ks+1 landed (in-order vmcnt: what was
  // issued after them may be in flight) and all its LDS reads are done,
  // barrier; if step ks was the last of a scale chunk, the chunk after next
  // is issued into its buffer; step ks+3 is issued into the buffer of step
  // ks; half 1 reads half 0 of step ks+1 (at the last step: stale LDS bytes,
  // never used).  A scale chunk is issued kSC >= 4 steps before its first use,
  // so it has landed whenever the step issued after it has.
  static_assert(kStages == 3, "the step loop below is unrolled by three");
  static_assert(D::kSC >= 4, "scale chunks are issued at least 4 steps ahead");
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  // a scale chunk issued at the middle of step j
  auto scales_at = [&](int j) { return j >= 0 && (j + 1) % D::kSC == 0 && (j + 1 + D::kSC) < nk; };
  auto step = [&](int ks, auto stage_t, auto rv_t) {
    constexpr int SC = decltype(stage_t)::value;
    constexpr int kDmaPerStage = dma_per_stage<decltype(rv_t)::value>();
    half(lds + SC * D::stage, sbase(ks), 1, rv_t);
    // issued after step ks+1 (at the middle of step ks-1): a scale chunk, then step ks+2
    const bool s_prev = scales_at(ks - 1);
    if (ks + 2 < nk) {
      if (s_prev)
        wait_vm_lds<kDmaPerStage + D::kSpi>();
      else
        wait_vm_lds<kDmaPerStage>();
    } else {
      if (s_prev)
        wait_vm_lds<D::kSpi>();
      else
        wait_vm_lds<0>();
    }
    __builtin_amdgcn_s_barrier();
    if (scales_at(ks)) issue_scales((ks + 1) / D::kSC + 1);
    if (ks + 3 < nk) issue(ks + 3, stage_t, rv_t);
    half(lds + ((SC + 1) % kStages) * D::stage, sbase(ks + 1), 0, rv_t);
  };
  // RV: the 16-row fragment rows multiplied (a partial tile skips the rest)
  auto main_loop = [&](auto rv_t) {
    constexpr int RV = decltype(rv_t)::value;
    constexpr int kDmaPerStage = dma_per_stage<RV>();
    set_aoff(rv_t);
    issue_scales(0);
    if (D::kSC < nk) issue_scales(1);
    issue(0, S0{}, rv_t);
    if (nk > 1) issue(1, S1{}, rv_t);
    if (nk > 2) issue(2, S2{}, rv_t);
    if (nk > 2)
      wait_vm_lds<2 * kDmaPerStage>();
    else if (nk > 1)
      wait_vm_lds<kDmaPerStage>();
    else
      wait_vm_lds<0>();
    __builtin_amdgcn_s_barrier();
    read_raw(lds, sbase(0), 0);
#pragma unroll
    for (int r = 0; r < RV; ++r) acur[r] = read_a(lds, 0, r);
#pragma unroll
    for (int c = 0; c < C; ++c) bcur[c] = decode_frag<FMT>(rd[c], rsb[c]);
    for (int ks = 0; ks < nk; ks += kStages) {
      step(ks, S0{}, rv_t);
      if (ks + 1 < nk) step(ks + 1, S1{}, rv_t);
      if (ks + 2 < nk) step(ks + 2, S2{}, rv_t);
    }
  };
  static_assert(R == 8, "fragment-row classes 8 / 4 / 2");
  if (vr > 4)
    main_loop(std::integral_constant<int, 8>{});
  else if (vr > 2)
    main_loop(std::integral_constant<int, 4>{});
  else
    main_loop(std::integral_constant<int, 2>{});

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
    constexpr int TPR = HW / 8, RPP = kThreads / TPR;
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
    constexpr int P = BN + 4, QR = 32;
    static_assert(QR * P * 4 <= kStages * D::stage, "staged part of the y tile fits");
    float* st = reinterpret_cast<float*>(lds);
    constexpr int TPR = BN / 4, RPP = kThreads / TPR;
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
  return launch(grouped_gemm_d_kernel<FMT, OP>, dim3(per * kXcds), dim3(kThreads), 0, s, p);
}

}  // namespace

bool grouped_gemm_dma_fits(int op, const WDesc& w0, const WDesc& w1, int in_rows) {
  // FP4 only: the 16-byte code pieces of a step are 64 K of one row.
  const bool fmt_ok = w0.fmt == FMT_MXFP4 || w0.fmt == FMT_NVFP4;
  if (!fmt_ok || w1.fmt != w0.fmt || w0.cols % BK != 0) return false;
  // buffer offsets are 32-bit: the input rows and one expert's codes below 2 GiB
  if ((size_t)in_rows * w0.cols * 2 >= (size_t(1) << 31) ||
      (size_t)w0.rows * w0.cols / 2 >= (size_t(1) << 31))
    return false;
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
  const int in_rows = (g.shared || op == kOpGateUp) ? g.T : g.T * g.topk;
  if (!grouped_gemm_dma_fits(op, w0, w1, in_rows)) return hipErrorInvalidValue;
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
  p.in_bytes = 0;
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
  p.in_bytes = (uint32_t)((size_t)p.in_rows * w0.cols * 2);
  const bool gu = op == kOpGateUp;
  if (w0.fmt == FMT_NVFP4)
    return gu ? launch_d<FMT_NVFP4, kOpGateUp>(p, nrt, s) : launch_d<FMT_NVFP4, kOpDown>(p, nrt, s);
  return gu ? launch_d<FMT_MXFP4, kOpGateUp>(p, nrt, s) : launch_d<FMT_MXFP4, kOpDown>(p, nrt, s);
}

}  // namespace moe
