// Prefill grouped expert GEMM on the gfx950 scaled matrix cores, for the
// opt-in lossy activation modes.
//
// The pages reserve activation quantization for explicit levers: NVFP4 W4A4
// prefill behind an opt-in switch (forum thread "DGPP: a GB10-optimized
// C++/CUDA inference engine", page 5, update post) and an FP8 prefill GEMM
// on per-token 1x128 E4M3 activations against the checkpoint's 128x128
// weight scales (gitee "dgpp" README, "Execution and performance",
// engine.prefill_fp8_gemm).  With both operands in FP8/FP4, the contraction
// runs on v_mfma_scale_f32_16x16x128_f8f6f4:
//
// * MX modes (MXFP4 experts): A = activations (MX E4M3 or E2M1), B = the
//   checkpoint's E2M1 codes; both E8M0 scales per 32 K go straight into the
//   instruction's scale operands, so the weights are never decoded.
// * 1x128 mode (FP8 block-128 experts): A and B E4M3 with unit E8M0 scales;
//   each 128-K step is exactly one scale block of both operands, so the
//   step's partial is scaled by s_a(row) * s_w(block) and added in fp32.
//
// Tiles, rows and epilogues follow the bf16 grouped GEMM: one workgroup of
// 4 wavefronts computes 128 permuted rows x 128 weight rows (gate/up: 64 gate
// + the matching 64 up rows, SwiGLU in the epilogue), each wavefront 64x64
// as 4x4 MFMA tiles of 16x16; K advances 128 per step through two LDS
// buffers fed from two register stages.
//
// Operand layout of the 16x16x128 instruction (measured on gfx950): lane l
// supplies row l % 16; an E2M1 operand holds K [32g, 32g+32) (g = l / 16)
// in its low 4 dwords, two codes per byte, even K in the low nibble; an E4M3
// operand holds K [16g, 16g+16) and [64+16g, 64+16g+16); the scale operand's
// byte 0 is the E8M0 scale of row l % 16 for K block g.  C row i, column j
// sits in lane j + 16 (i / 4), element i % 4.
#include <type_traits>

#include "gemv_core.cuh"

namespace moe {
namespace {

constexpr int BM = kGemmTileM, BN = 128, BK = 128;
constexpr int kXcds = 8;
// Row tiles per run of the tile order (gemm_tile_order).
constexpr int kRowRun = 4;
constexpr int kFmtFp8 = 0, kFmtFp4 = 4;  // operand format codes of the instruction

// LDS rows hold one K step of one tile row in K order, then the row's scale
// word in the padding: the E8M0 bytes of the step (MX) or the row's fp32
// 1x128 scale (A of the 1x128 mode).  Pitches measured with the LDS
// bank-conflict counter on gfx950: with the fragment reads below (row =
// lane % 16; lane group g reads 16 bytes at 16 g, and an E4M3 operand also at
// 64 + 16 g) and staging writes in which the two threads of a row alternate
// 16-byte pieces, both are conflict-free at 160 bytes for 128-byte rows and
// at 96 bytes for 64-byte rows (and conflicted at the other pitches tried).
template <int AM>
struct QCfg {
  static constexpr bool a_fp4 = AM == kActMxfp4;
  static constexpr bool b_fp4 = AM != kActT128;
  static constexpr int a_bytes = a_fp4 ? 64 : 128;  // bytes of one row per K step
  static constexpr int b_bytes = b_fp4 ? 64 : 128;
  static constexpr int a_pitch = a_fp4 ? 96 : 160;
  static constexpr int b_pitch = b_fp4 ? 96 : 160;
  static constexpr int ap = a_bytes / 32;  // 16-byte pieces per staging thread
  static constexpr int bp = b_bytes / 32;
  static constexpr int afmt = a_fp4 ? kFmtFp4 : kFmtFp8;
  static constexpr int bfmt = b_fp4 ? kFmtFp4 : kFmtFp8;
};

template <int AM>
struct QSmem {
  uint8_t a[2][BM][QCfg<AM>::a_pitch];
  uint8_t b[2][BN][QCfg<AM>::b_pitch];
};

template <int AM>
struct QStage {
  u32x4 a[QCfg<AM>::ap];
  u32x4 b[QCfg<AM>::bp];
  uint32_t sc;     // thread < 128: A scale word of its row; else (MX) B scale word
  float ws0, ws1;  // 1x128: the step's weight block scales (w0, w1)
};

struct QParams {
  WDesc w0, w1;
  const uint8_t* codes;   // quantized input rows
  const void* scales;
  int a_pitch_codes;      // bytes per input row
  int a_pitch_scales;     // bytes per input row of scales (4 per 128 K)
  void* out;
  const int2* tiles;
  const int* n_tiles;
  const int* offsets;
  const int* perm_to_pair;
  int topk, T, in_rows, in_rows_total, max_rt, ntn;
};

typedef int i32x4 __attribute__((ext_vector_type(4)));

// An E2M1 operand uses the low 4 dwords; the upper 4 are ignored.
__device__ __forceinline__ i32x8 fp4_operand(u32x4 v) {
  const i32x4 w = __builtin_bit_cast(i32x4, v);
  return __builtin_shufflevector(w, w, 0, 1, 2, 3, -1, -1, -1, -1);
}
__device__ __forceinline__ i32x8 fp8_operand(u32x4 lo, u32x4 hi) {
  return __builtin_shufflevector(__builtin_bit_cast(i32x4, lo), __builtin_bit_cast(i32x4, hi),
                                 0, 1, 2, 3, 4, 5, 6, 7);
}

// Input row of permuted row `pr` (clamped into the group; rows past the
// group read row m0: their outputs are never stored).
template <int OP>
__device__ __forceinline__ int input_row(const QParams& p, int pr, int m0, int m1) {
  const int row = pr < m1 ? pr : m0;
  int ir = (p.tiles != nullptr && OP == kOpGateUp) ? p.perm_to_pair[row] / p.topk : row;
  if ((unsigned)ir >= (unsigned)p.in_rows) ir = 0;
  return ir;
}

template <int AM, int OP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void grouped_gemm_q_kernel(
    QParams p) {
  using C = QCfg<AM>;
  constexpr bool MX = AM != kActT128;
  __shared__ QSmem<AM> sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // XCD-aware order, as in the bf16 grouped GEMM.
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

  // ---- staging roles: thread -> (tile row srow, h); it moves the row's
  // 16-byte pieces h, h+2, h+4, ... of each step ----
  const int srow = tid >> 1, h = tid & 1;
  const uint8_t* arow = p.codes + (size_t)input_row<OP>(p, m0 + srow, m0, m1) * p.a_pitch_codes;
  const WDesc& wq = (OP == kOpGateUp && srow >= BN / 2) ? p.w1 : p.w0;
  const int wr0 = (OP == kOpGateUp) ? n0 + (srow & (BN / 2 - 1)) : n0 + srow;
  const int wr = wr0 < N ? wr0 : N - 1;
  const uint8_t* wrow = wq.codes + e * wq.stride_codes + (size_t)wr * (C::b_fp4 ? K / 2 : K);
  // scale roles: threads 0..127 move the A scale word of tile row tid;
  // threads 128..255 (MX) the B scale word of weight tile row tid - 128.
  const uint32_t* sa_row = nullptr;
  const uint8_t* sb_row = nullptr;
  bool sb_wide = false;
  if (tid < BM) {
    const int ir = input_row<OP>(p, m0 + tid, m0, m1);
    sa_row = reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(p.scales) +
                                               (size_t)ir * p.a_pitch_scales);
  } else if constexpr (MX) {
    const int r = tid - BM;
    const WDesc& wsq = (OP == kOpGateUp && r >= BN / 2) ? p.w1 : p.w0;
    const int n = (OP == kOpGateUp) ? n0 + (r & (BN / 2 - 1)) : n0 + r;
    sb_row = reinterpret_cast<const uint8_t*>(wsq.scales) + e * wsq.stride_scales +
             (size_t)(n < N ? n : N - 1) * (K / 32);
    sb_wide = wsq.wide != 0;
  }
  // 1x128: weight block scales [ceil(N/128)][ceil(K/128)] of this tile's rows
  // (a gate/up tile's 64 rows, and a down tile's 128, lie in one 128-block).
  const int kb_n = (K + 127) / 128;
  const float* ws0p = nullptr;
  const float* ws1p = nullptr;
  if constexpr (!MX) {
    ws0p = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(p.w0.scales) +
                                          e * p.w0.stride_scales) + (size_t)(n0 / 128) * kb_n;
    ws1p = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(p.w1.scales) +
                                          e * p.w1.stride_scales) + (size_t)(n0 / 128) * kb_n;
  }
  const int nk = (K + BK - 1) / BK;

  // FAST: every step is a full 128-K step and the B scale words are aligned.
  auto load_stage = [&](int ks, QStage<AM>& st, auto fast_t) {
    constexpr bool FAST = decltype(fast_t)::value;
    const int k0 = ks * BK;
    const bool full = FAST || k0 + BK <= K;
    const uint8_t* ab = arow + (C::a_fp4 ? k0 / 2 : k0);
    const uint8_t* bb = wrow + (C::b_fp4 ? k0 / 2 : k0);
#pragma unroll
    for (int i = 0; i < C::ap; ++i) {
      const int pb = 16 * (2 * i + h);  // byte of the piece in the step
      st.a[i] = (full || k0 + (C::a_fp4 ? 2 * pb : pb) < K)
                    ? *reinterpret_cast<const u32x4*>(ab + pb) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < C::bp; ++i) {
      const int pb = 16 * (2 * i + h);
      st.b[i] = (full || k0 + (C::b_fp4 ? 2 * pb : pb) < K)
                    ? *reinterpret_cast<const u32x4*>(bb + pb) : u32x4{0, 0, 0, 0};
    }
    st.sc = 0;
    if (tid < BM) {
      // MX: the 4 E8M0 bytes of the step (rows padded to whole steps);
      // 1x128: the fp32 scale of the step's block
      st.sc = sa_row[ks];
    } else if constexpr (MX) {
      if (FAST || (full && sb_wide)) {
        st.sc = reinterpret_cast<const uint32_t*>(sb_row)[ks];
      } else {
        uint32_t v = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kb = 4 * ks + j;  // 32-block
          v |= static_cast<uint32_t>(32 * kb < K ? sb_row[kb] : 127) << (8 * j);
        }
        st.sc = v;
      }
    }
    if constexpr (!MX) {
      st.ws0 = ws0p[ks];
      st.ws1 = (OP == kOpGateUp) ? ws1p[ks] : st.ws0;
    } else {
      st.ws0 = st.ws1 = 1.f;
    }
  };
  auto store_stage = [&](int buf, const QStage<AM>& st) {
#pragma unroll
    for (int i = 0; i < C::ap; ++i)
      *reinterpret_cast<u32x4*>(&sm.a[buf][srow][16 * (2 * i + h)]) = st.a[i];
#pragma unroll
    for (int i = 0; i < C::bp; ++i)
      *reinterpret_cast<u32x4*>(&sm.b[buf][srow][16 * (2 * i + h)]) = st.b[i];
    if (tid < BM)
      *reinterpret_cast<uint32_t*>(&sm.a[buf][tid][C::a_bytes]) = st.sc;
    else if constexpr (MX)
      *reinterpret_cast<uint32_t*>(&sm.b[buf][tid - BM][C::b_bytes]) = st.sc;
  };

  // ---- MFMA roles (as in the bf16 grouped GEMM) ----
  const int wm = wave >> 1, wn = wave & 1;
  int bcol[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
    bcol[c] = (OP == kOpGateUp) ? ((c < 2) ? 32 * wn + 16 * c : 64 + 32 * wn + 16 * (c - 2))
                                : 64 * wn + 16 * c;
  f32x4 acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int vrows = m1 - m0 - 64 * wm;
  const int vr = vrows <= 0 ? 0 : min(4, (vrows + 15) / 16);
  const int g = lane >> 4, lr = lane & 15;

  auto operand = [&](const uint8_t* row, auto fp4_t) {
    if constexpr (decltype(fp4_t)::value)
      return fp4_operand(*reinterpret_cast<const u32x4*>(row + 16 * g));
    else
      return fp8_operand(*reinterpret_cast<const u32x4*>(row + 16 * g),
                         *reinterpret_cast<const u32x4*>(row + 64 + 16 * g));
  };
  using a4 = std::integral_constant<bool, C::a_fp4>;
  using b4 = std::integral_constant<bool, C::b_fp4>;

  auto compute_step = [&](int buf, float ws0, float ws1, auto fast_t) {
    constexpr bool FAST = decltype(fast_t)::value;
    if (!FAST && vr == 0) return;
    i32x8 bf[4];
    int sb[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint8_t* row = &sm.b[buf][bcol[c] + lr][0];
      bf[c] = operand(row, b4{});
      sb[c] = MX ? row[C::b_bytes + g] : 127;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (!FAST && r >= vr) continue;
      const uint8_t* row = &sm.a[buf][64 * wm + 16 * r + lr][0];
      const i32x8 af = operand(row, a4{});
      if constexpr (MX) {
        const int sa = row[C::a_bytes + g];
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[r][c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              af, bf[c], acc[r][c], C::afmt, C::bfmt, 0, sa, 0, sb[c]);
      } else {
        // the fp32 scales of this lane's 4 output rows of tile r (64wm + 16r + 4g + j)
        float rs[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          rs[j] = *reinterpret_cast<const float*>(&sm.a[buf][64 * wm + 16 * r + 4 * g + j][C::a_bytes]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const f32x4 part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              af, bf[c], f32x4{0.f, 0.f, 0.f, 0.f}, C::afmt, C::bfmt, 0, 127, 0, 127);
          const float wsc = (OP == kOpGateUp && c >= 2) ? ws1 : ws0;
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[r][c][j] = fmaf(part[j], rs[j] * wsc, acc[r][c][j]);
        }
      }
    }
  };

  // One register stage in flight: the global loads of step ks+2 are issued
  // once step ks+1 has gone from registers to LDS, and have the MFMAs of
  // step ks+1 to arrive; LDS holds steps ks and ks+1.  The loop is unrolled
  // by two for static buffer names.  wsb0/1[b]: the 1x128 weight scales of
  // the step in LDS buffer b.  The loop exists twice: without conditions for
  // full tiles of whole steps (FAST, MX modes; the 1x128 mode's partials
  // leave no registers for a second copy), and with the guards; its barriers
  // are block-wide and every wavefront of a block takes the same version.
  auto main_loop = [&](auto fast_t) {
    constexpr bool FAST = decltype(fast_t)::value;
    QStage<AM> st;
    float wsb0[2], wsb1[2];
    load_stage(0, st, fast_t);
    store_stage(0, st);
    wsb0[0] = st.ws0;
    wsb1[0] = st.ws1;
    wsb0[1] = wsb1[1] = 0.f;
    if (nk > 1) load_stage(1, st, fast_t);
    __syncthreads();
    int ks = 0;
    if constexpr (FAST) {
      for (; ks + 3 < nk; ks += 2) {
        compute_step(0, wsb0[0], wsb1[0], fast_t);
        store_stage(1, st);
        wsb0[1] = st.ws0;
        wsb1[1] = st.ws1;
        load_stage(ks + 2, st, fast_t);
        __syncthreads();
        compute_step(1, wsb0[1], wsb1[1], fast_t);
        store_stage(0, st);
        wsb0[0] = st.ws0;
        wsb1[0] = st.ws1;
        load_stage(ks + 3, st, fast_t);
        __syncthreads();
      }
    }
    for (; ks < nk; ks += 2) {
      compute_step(0, wsb0[0], wsb1[0], fast_t);
      if (ks + 1 < nk) {
        store_stage(1, st);
        wsb0[1] = st.ws0;
        wsb1[1] = st.ws1;
        if (ks + 2 < nk) load_stage(ks + 2, st, fast_t);
      }
      __syncthreads();
      if (ks + 1 >= nk) break;
      compute_step(1, wsb0[1], wsb1[1], fast_t);
      if (ks + 2 < nk) {
        store_stage(0, st);
        wsb0[0] = st.ws0;
        wsb1[0] = st.ws1;
        if (ks + 3 < nk) load_stage(ks + 3, st, fast_t);
      }
      __syncthreads();
    }
  };
  const bool wide_ok = !MX || (p.w0.wide && p.w1.wide);
  // vr is per wavefront; the version must be the block's: test the block's rows
  if constexpr (MX) {
    if (m1 - m0 >= BM && K % BK == 0 && wide_ok)
      main_loop(std::true_type{});
    else
      main_loop(std::false_type{});
  } else {
    main_loop(std::false_type{});
  }

  // ---- epilogue: lane holds rows 4*(lane/16)+j of each 16-row tile, column lane%16 ----
  const int col = lane & 15;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = m0 + 64 * wm + 16 * r + 4 * (lane >> 4) + j;
      if (row >= m1) continue;
      if constexpr (OP == kOpGateUp) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int n = nt * (BN / 2) + 32 * wn + 16 * c + col;
          if (n >= N) continue;
          const float hv = silu_fast(acc[r][c][j]) * acc[r][c + 2][j];
          reinterpret_cast<uint16_t*>(p.out)[(size_t)row * N + n] = f32_to_bf16(hv);
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int n = n0 + 64 * wn + 16 * c + col;
          if (n >= N) continue;
          reinterpret_cast<float*>(p.out)[(size_t)row * N + n] = acc[r][c][j];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// The same GEMM with every operand moved global -> LDS by the LDS-DMA loads
// (global_load_lds_dwordx4 / _dword): no staging registers, NST stages of LDS
// (one being computed, the next in flight).  Taken when K % 128 == 0 (every step whole) and, for the MX
// modes, the weight scale words are aligned.
//
// A DMA instruction writes 64 lanes x 16 bytes to one contiguous KiB of LDS,
// so rows are unpadded and bank conflicts are avoided by an XOR swizzle of
// the 16-byte pieces within a row: piece P of row r sits at slot
// P ^ ((r >> 1) & 7) in a 128-byte row and at P ^ ((r >> 2) & 3) in a 64-byte
// row.  Eight lanes that read the same piece of eight consecutive rows then
// hit eight distinct 16-byte bank groups, and each lane picks the global
// piece that lands in its LDS slot.  Per stage and wavefront: A codes, B codes
// and one scale word (or, for waves 2-3 of the 1x128 mode, the weight block
// scales) per lane, so every wavefront issues the same number of DMA loads
// and waits for a stage with a fixed vmcnt.
template <int AM>
struct DCfg {
  using C = QCfg<AM>;
  // Stages of LDS in flight.  Measured at T=8192: two stages (50 KB for W4A8,
  // 66 KB for 1x128) beat three or four, whose LDS leaves fewer workgroups
  // per CU: more resident workgroups hide the step latency better than a
  // deeper prefetch within one.
  static constexpr int NST = 2;
  static constexpr int a_chunks = BM * C::a_bytes / 1024;  // KiB pieces per stage
  static constexpr int b_chunks = BN * C::b_bytes / 1024;
  static constexpr int a_per_wave = a_chunks / 4;
  static constexpr int b_per_wave = b_chunks / 4;
  static constexpr int loads_per_stage = a_per_wave + b_per_wave + 1;
  static constexpr int a_off = 0;
  static constexpr int b_off = BM * C::a_bytes;
  static constexpr int s_off = b_off + BN * C::b_bytes;  // 256 dwords: A rows, then B rows / weight scales
  static constexpr int stage_bytes = s_off + 256 * 4;
};

template <int BYTES>
__device__ __forceinline__ int swz_slot(int piece, int row) {
  return BYTES == 128 ? (piece ^ ((row >> 1) & 7)) : (piece ^ ((row >> 2) & 3));
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void dma16(const void* src, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds, 4, 0, 0);
}

// vmcnt(N) and lgkmcnt(0) (gfx9 encoding): this wave's DMA loads older than
// the last N have landed, and its LDS reads are complete.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4));
}

// Wait until at most `later` stages of LOADS loads each are outstanding
// (later in 0 .. MAXL; the wait count must be an immediate).
template <int LOADS, int MAXL>
__device__ __forceinline__ void wait_for_stage(int later) {
  if constexpr (MAXL > 0) {
    if (later >= MAXL) {
      wait_vmcnt_lds<LOADS * MAXL>();
      return;
    }
    wait_for_stage<LOADS, MAXL - 1>(later);
  } else {
    wait_vmcnt_lds<0>();
  }
}

template <int AM, int OP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void grouped_gemm_qd_kernel(
    QParams p) {
  using C = QCfg<AM>;
  using D = DCfg<AM>;
  constexpr bool MX = AM != kActT128;
  constexpr int NST = D::NST;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NST * D::stage_bytes];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
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

  // ---- DMA sources of this lane (fixed tile rows; advanced per step) ----
  constexpr int a_rpc = 1024 / C::a_bytes;  // rows per KiB
  constexpr int b_rpc = 1024 / C::b_bytes;
  const uint8_t* asrc[D::a_per_wave];
#pragma unroll
  for (int i = 0; i < D::a_per_wave; ++i) {
    const int ch = wave * D::a_per_wave + i;
    const int r = ch * a_rpc + lane / (C::a_bytes / 16);
    const int slot = lane % (C::a_bytes / 16);
    const int piece = swz_slot<C::a_bytes>(slot, r);  // the involution maps slot <-> piece
    asrc[i] = p.codes + (size_t)input_row<OP>(p, m0 + r, m0, m1) * p.a_pitch_codes + 16 * piece;
  }
  const uint8_t* bsrc[D::b_per_wave];
#pragma unroll
  for (int i = 0; i < D::b_per_wave; ++i) {
    const int ch = wave * D::b_per_wave + i;
    const int r = ch * b_rpc + lane / (C::b_bytes / 16);
    const int slot = lane % (C::b_bytes / 16);
    const int piece = swz_slot<C::b_bytes>(slot, r);
    const WDesc& wq = (OP == kOpGateUp && r >= BN / 2) ? p.w1 : p.w0;
    const int wr0 = (OP == kOpGateUp) ? n0 + (r & (BN / 2 - 1)) : n0 + r;
    const int wr = wr0 < N ? wr0 : N - 1;
    bsrc[i] = wq.codes + e * wq.stride_codes + (size_t)wr * (C::b_fp4 ? K / 2 : K) + 16 * piece;
  }
  // scale word: waves 0-1 the A rows 64w + lane; waves 2-3 (MX) the weight
  // rows 64(w-2) + lane, (1x128) the two weight block scales of the step.
  const uint8_t* ssrc;
  int sstep;  // bytes per step
  if (wave < 2) {
    ssrc = reinterpret_cast<const uint8_t*>(p.scales) +
           (size_t)input_row<OP>(p, m0 + 64 * wave + lane, m0, m1) * p.a_pitch_scales;
    sstep = 4;
  } else if constexpr (MX) {
    const int r = 64 * (wave - 2) + lane;
    const WDesc& wsq = (OP == kOpGateUp && r >= BN / 2) ? p.w1 : p.w0;
    const int n = (OP == kOpGateUp) ? n0 + (r & (BN / 2 - 1)) : n0 + r;
    ssrc = reinterpret_cast<const uint8_t*>(wsq.scales) + e * wsq.stride_scales +
           (size_t)(n < N ? n : N - 1) * (K / 32);
    sstep = 4;
  } else {
    const WDesc& wsq = (OP == kOpGateUp && lane == 1) ? p.w1 : p.w0;
    ssrc = reinterpret_cast<const uint8_t*>(wsq.scales) + e * wsq.stride_scales +
           (size_t)(n0 / 128) * nk * 4;
    sstep = 4;
  }

  auto issue = [&](int ks) {
    uint8_t* st = lds + (ks % NST) * D::stage_bytes;
    const int ka = ks * (C::a_fp4 ? BK / 2 : BK), kb = ks * (C::b_fp4 ? BK / 2 : BK);
#pragma unroll
    for (int i = 0; i < D::a_per_wave; ++i)
      dma16(asrc[i] + ka, st + D::a_off + 1024 * (wave * D::a_per_wave + i));
#pragma unroll
    for (int i = 0; i < D::b_per_wave; ++i)
      dma16(bsrc[i] + kb, st + D::b_off + 1024 * (wave * D::b_per_wave + i));
    dma4(ssrc + ks * sstep, st + D::s_off + 256 * wave);
  };

  const int wm = wave >> 1, wn = wave & 1;
  int bcol[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
    bcol[c] = (OP == kOpGateUp) ? ((c < 2) ? 32 * wn + 16 * c : 64 + 32 * wn + 16 * (c - 2))
                                : 64 * wn + 16 * c;
  f32x4 acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int vrows = m1 - m0 - 64 * wm;
  const int vr = vrows <= 0 ? 0 : min(4, (vrows + 15) / 16);
  const int g = lane >> 4, lr = lane & 15;

  auto operand = [&](const uint8_t* rowp, int row, auto fp4_t) {
    if constexpr (decltype(fp4_t)::value)
      return fp4_operand(*reinterpret_cast<const u32x4*>(rowp + 16 * swz_slot<64>(g, row)));
    else
      return fp8_operand(*reinterpret_cast<const u32x4*>(rowp + 16 * swz_slot<128>(g, row)),
                         *reinterpret_cast<const u32x4*>(rowp + 16 * swz_slot<128>(4 + g, row)));
  };
  using a4 = std::integral_constant<bool, C::a_fp4>;
  using b4 = std::integral_constant<bool, C::b_fp4>;

  auto compute = [&](int ks, auto full_t) {
    constexpr bool FULL = decltype(full_t)::value;
    const uint8_t* st = lds + (ks % NST) * D::stage_bytes;
    const uint8_t* sw = st + D::s_off;  // scale words: A rows at 0, B rows (MX) at 512
    i32x8 bf[4];
    int sb[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int row = bcol[c] + lr;
      bf[c] = operand(st + D::b_off + row * C::b_bytes, row, b4{});
      sb[c] = MX ? sw[512 + 4 * row + g] : 127;
    }
    float ws0 = 1.f, ws1 = 1.f;
    if constexpr (!MX) {
      ws0 = reinterpret_cast<const float*>(sw + 512)[0];
      ws1 = reinterpret_cast<const float*>(sw + 512)[1];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (!FULL && r >= vr) continue;
      const int row = 64 * wm + 16 * r + lr;
      const i32x8 af = operand(st + D::a_off + row * C::a_bytes, row, a4{});
      if constexpr (MX) {
        const int sa = sw[4 * row + g];
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[r][c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              af, bf[c], acc[r][c], C::afmt, C::bfmt, 0, sa, 0, sb[c]);
      } else {
        const f32x4 rs = *reinterpret_cast<const f32x4*>(sw + 4 * (64 * wm + 16 * r + 4 * g));
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const f32x4 part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              af, bf[c], f32x4{0.f, 0.f, 0.f, 0.f}, C::afmt, C::bfmt, 0, 127, 0, 127);
          const float wsc = (OP == kOpGateUp && c >= 2) ? ws1 : ws0;
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[r][c][j] = fmaf(part[j], rs[j] * wsc, acc[r][c][j]);
        }
      }
    }
  };

  // Pipeline: stages 0 .. NST-2 issued up front; at step ks, wait until this
  // wave's loads of stage ks have landed (the later stages' loads may still
  // be in flight) and its LDS reads of step ks-1 are complete, barrier (all
  // waves' loads of stage ks are visible, and all waves are done with step
  // ks-1), issue stage ks+NST-1 into the buffer of step ks-1, compute step ks.  The barrier is the bare s_barrier: a
  // __syncthreads() fence would wait for every outstanding DMA.
  auto main_loop = [&](auto full_t) {
#pragma unroll
    for (int s0 = 0; s0 < NST - 1; ++s0)
      if (s0 < nk) issue(s0);
    for (int ks = 0; ks < nk; ++ks) {
      const int later = min(NST - 2, nk - 1 - ks);  // stages issued after ks
      wait_for_stage<D::loads_per_stage, NST - 2>(later);
      __builtin_amdgcn_s_barrier();
      if (ks + NST - 1 < nk) issue(ks + NST - 1);
      compute(ks, full_t);
    }
  };
  if (m1 - m0 >= BM)
    main_loop(std::true_type{});
  else
    main_loop(std::false_type{});

  const int col = lane & 15;
  if constexpr (OP == kOpGateUp) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = m0 + 64 * wm + 16 * r + 4 * (lane >> 4) + j;
        if (row >= m1) continue;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int n = nt * (BN / 2) + 32 * wn + 16 * c + col;
          if (n >= N) continue;
          const float hv = silu_fast(acc[r][c][j]) * acc[r][c + 2][j];
          reinterpret_cast<uint16_t*>(p.out)[(size_t)row * N + n] = f32_to_bf16(hv);
        }
      }
    }
  } else {
    // fp32 y through the K loop's LDS, two halves of 64 rows x 132-float
    // rows, stored as 16-byte vectors over whole row segments (a fragment
    // lane holds one column of four rows: storing from the fragments writes
    // 4-byte pieces); N not a multiple of 4 falls back to elements.
    constexpr int P = 132;
    static_assert(64 * P * 4 <= NST * D::stage_bytes, "staged half tile fits");
    float* st = reinterpret_cast<float*>(lds);
    const int cb = 4 * (tid & 31);
    const int n = n0 + cb;
    const bool vec = N % 4 == 0;
    __syncthreads();
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (wm == half) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              st[(16 * r + 4 * (lane >> 4) + j) * P + 64 * wn + 16 * c + col] = acc[r][c][j];
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int lr = (tid >> 5) + 8 * q;
        const int row = m0 + 64 * half + lr;
        if (row >= m1 || n >= N) continue;
        const f32x4 v = *reinterpret_cast<const f32x4*>(st + lr * P + cb);
        float* o = reinterpret_cast<float*>(p.out) + (size_t)row * N + n;
        if (vec && n + 3 < N) {
          *reinterpret_cast<f32x4*>(o) = v;
        } else {
          for (int i = 0; i < 4; ++i)
            if (n + i < N) o[i] = v[i];
        }
      }
      if (half == 0) __syncthreads();
    }
  }
}

template <int AM, int OP>
hipError_t launch_q(QParams p, int n_row_tiles, hipStream_t s) {
  const int ntn = (OP == kOpGateUp) ? (p.w0.rows + BN / 2 - 1) / (BN / 2) : (p.w0.rows + BN - 1) / BN;
  p.ntn = ntn;
  p.max_rt = n_row_tiles;
  const int per = (n_row_tiles * ntn + kXcds - 1) / kXcds;
  if (per == 0) return hipSuccess;
  const bool dma = p.w0.cols % BK == 0 && (AM == kActT128 || (p.w0.wide && p.w1.wide));
  if (dma) return launch(grouped_gemm_qd_kernel<AM, OP>, dim3(per * kXcds), dim3(256), 0, s, p);
  return launch(grouped_gemm_q_kernel<AM, OP>, dim3(per * kXcds), dim3(256), 0, s, p);
}

template <int AM>
hipError_t launch_mode(int op, const QParams& p, int nrt, hipStream_t s) {
  return op == kOpGateUp ? launch_q<AM, kOpGateUp>(p, nrt, s) : launch_q<AM, kOpDown>(p, nrt, s);
}

}  // namespace

hipError_t launch_grouped_gemm_q(int mode, int op, const WDesc& w0, const WDesc& w1,
                                 const GroupArgs& g, const int* tiles, const int* n_tiles,
                                 int max_tiles, const uint8_t* in_codes, const void* in_scales,
                                 void* out, hipStream_t s) {
  const bool mx = mode == kActMxfp8 || mode == kActMxfp4;
  if (mx ? (w0.fmt != FMT_MXFP4 || w1.fmt != FMT_MXFP4)
         : (mode != kActT128 || w0.fmt != FMT_FP8 || w1.fmt != FMT_FP8))
    return hipErrorInvalidValue;
  if (w0.cols % 32 != 0) return hipErrorInvalidValue;
  QParams p;
  p.w0 = w0;
  p.w1 = w1;
  p.codes = in_codes;
  p.scales = in_scales;
  const int K = w0.cols;
  p.a_pitch_codes = (mode == kActMxfp4) ? K / 2 : K;
  p.a_pitch_scales = act_scale_pitch(K);  // bytes: 4 per 128 K (MX bytes or one fp32)
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
  switch (mode) {
    case kActMxfp8: return launch_mode<kActMxfp8>(op, p, nrt, s);
    case kActMxfp4: return launch_mode<kActMxfp4>(op, p, nrt, s);
    default: return launch_mode<kActT128>(op, p, nrt, s);
  }
}

}  // namespace moe
