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
constexpr int kFmtFp8 = 0, kFmtFp4 = 4;  // operand format codes of the instruction

template <int AM>
struct QCfg {
  static constexpr bool a_fp4 = AM == kActMxfp4;
  static constexpr bool b_fp4 = AM != kActT128;
  static constexpr int a_bytes = a_fp4 ? 64 : 128;  // bytes of one row per K step
  static constexpr int b_bytes = b_fp4 ? 64 : 128;
  // LDS row pitch: 16 bytes of padding (row = lane % 16 reads hit distinct banks)
  static constexpr int a_pitch = a_bytes + 16;
  static constexpr int b_pitch = b_bytes + 16;
  static constexpr int ap = a_bytes / 32;  // 16-byte pieces per thread per step
  static constexpr int bp = b_bytes / 32;
  static constexpr int afmt = a_fp4 ? kFmtFp4 : kFmtFp8;
  static constexpr int bfmt = b_fp4 ? kFmtFp4 : kFmtFp8;
};

template <int AM>
struct QSmem {
  uint8_t a[2][BM][QCfg<AM>::a_pitch];
  uint8_t b[2][BN][QCfg<AM>::b_pitch];
  uint32_t as[2][BM];  // MX: 4 E8M0 bytes of the step; T128: fp32 scale bits
  uint32_t bs[2][BN];  // MX: 4 E8M0 bytes of the step (weights)
};

template <int AM>
struct QStage {
  u32x4 a[QCfg<AM>::ap];
  u32x4 b[QCfg<AM>::bp];
  uint32_t sc;     // thread < 128: A scale of its row; else (MX) B scale of its weight row
  float ws0, ws1;  // T128: the step's weight block scales (w0, w1)
};

struct QParams {
  WDesc w0, w1;
  const uint8_t* codes;   // quantized input rows
  const void* scales;
  int a_pitch_codes;      // bytes per input row
  int a_pitch_scales;     // MX: bytes per row; T128: floats per row
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
  __shared__ QSmem<AM> sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // XCD-aware order, as in the bf16 grouped GEMM.
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

  // ---- staging roles: thread -> (tile row srow, half of the step's bytes) ----
  const int srow = tid >> 1, shalf = tid & 1;
  const uint8_t* arow = p.codes + (size_t)input_row<OP>(p, m0 + srow, m0, m1) * p.a_pitch_codes;
  const WDesc& wq = (OP == kOpGateUp && srow >= BN / 2) ? p.w1 : p.w0;
  const int wr0 = (OP == kOpGateUp) ? n0 + (srow & (BN / 2 - 1)) : n0 + srow;
  const int wr = wr0 < N ? wr0 : N - 1;
  const int wrb = C::b_fp4 ? K / 2 : K;
  const uint8_t* wrow = wq.codes + e * wq.stride_codes + (size_t)wr * wrb;
  // scale roles: threads 0..127 own the A scale of tile row tid; threads
  // 128..255 (MX) the B scale of weight tile row tid - 128.
  const uint8_t* sa_row = nullptr;
  const uint8_t* sb_row = nullptr;
  bool sb_wide = false;
  if (tid < BM) {
    const int ir = input_row<OP>(p, m0 + tid, m0, m1);
    sa_row = reinterpret_cast<const uint8_t*>(p.scales) +
             (size_t)ir * p.a_pitch_scales * (AM == kActT128 ? 4 : 1);
  } else if constexpr (AM != kActT128) {
    const int r = tid - BM;
    const WDesc& wsq = (OP == kOpGateUp && r >= BN / 2) ? p.w1 : p.w0;
    const int n = (OP == kOpGateUp) ? n0 + (r & (BN / 2 - 1)) : n0 + r;
    sb_row = reinterpret_cast<const uint8_t*>(wsq.scales) + e * wsq.stride_scales +
             (size_t)(n < N ? n : N - 1) * (K / 32);
    sb_wide = wsq.wide != 0;
  }
  // T128: weight block scales [ceil(N/128)][ceil(K/128)] of this tile's rows
  // (a gate/up tile's 64 rows, and a down tile's 128, lie in one 128-block).
  const int kb_n = (K + 127) / 128;
  const float* ws0p = nullptr;
  const float* ws1p = nullptr;
  if constexpr (AM == kActT128) {
    ws0p = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(p.w0.scales) +
                                          e * p.w0.stride_scales) + (size_t)(n0 / 128) * kb_n;
    ws1p = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(p.w1.scales) +
                                          e * p.w1.stride_scales) + (size_t)(n0 / 128) * kb_n;
  }
  const int nk = (K + BK - 1) / BK;

  auto load_stage = [&](int ks, QStage<AM>& st) {
    const int k0 = ks * BK;
    const bool full = k0 + BK <= K;
    // pieces: A byte offset (within the step) 16 * (ap * shalf + i)
#pragma unroll
    for (int i = 0; i < C::ap; ++i) {
      const int pb = 16 * (C::ap * shalf + i);                   // byte in the step
      const int kk = k0 + (C::a_fp4 ? 2 * pb : pb);              // first K of the piece
      const size_t off = (size_t)(C::a_fp4 ? k0 / 2 : k0) + pb;
      st.a[i] = (full || kk < K) ? *reinterpret_cast<const u32x4*>(arow + off) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < C::bp; ++i) {
      const int pb = 16 * (C::bp * shalf + i);
      const int kk = k0 + (C::b_fp4 ? 2 * pb : pb);
      const size_t off = (size_t)(C::b_fp4 ? k0 / 2 : k0) + pb;
      st.b[i] = (full || kk < K) ? *reinterpret_cast<const u32x4*>(wrow + off) : u32x4{0, 0, 0, 0};
    }
    st.sc = 0;
    if (tid < BM) {
      // MX: the 4 E8M0 bytes of the step (rows padded to whole steps);
      // T128: the fp32 scale of the step's block
      st.sc = reinterpret_cast<const uint32_t*>(sa_row)[ks];
    } else if constexpr (AM != kActT128) {
      if (full && sb_wide) {
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
    if constexpr (AM == kActT128) {
      st.ws0 = ws0p[ks];
      st.ws1 = (OP == kOpGateUp) ? ws1p[ks] : st.ws0;
    } else {
      st.ws0 = st.ws1 = 1.f;
    }
  };
  // LDS order of an E4M3 row: byte piece P (16 B) of the step sits at slot
  // 2 (P % 4) + P / 4, so lane group g finds its two pieces (g and 4 + g) in
  // one 32-byte run, and the two staging threads of a row interleave their
  // 16-byte writes.  E2M1 rows keep the K order (lane group g reads 16 bytes
  // at 16 g).
  auto a_slot = [](int P) { return C::a_fp4 ? P : 2 * (P & 3) + (P >> 2); };
  auto b_slot = [](int P) { return C::b_fp4 ? P : 2 * (P & 3) + (P >> 2); };
  auto store_stage = [&](int buf, const QStage<AM>& st) {
#pragma unroll
    for (int i = 0; i < C::ap; ++i)
      *reinterpret_cast<u32x4*>(&sm.a[buf][srow][16 * a_slot(C::ap * shalf + i)]) = st.a[i];
#pragma unroll
    for (int i = 0; i < C::bp; ++i)
      *reinterpret_cast<u32x4*>(&sm.b[buf][srow][16 * b_slot(C::bp * shalf + i)]) = st.b[i];
    if (tid < BM)
      sm.as[buf][tid] = st.sc;
    else
      sm.bs[buf][tid - BM] = st.sc;
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

  auto compute_step = [&](int buf, float ws0, float ws1) {
    if (vr == 0) return;
    i32x8 bf[4];
    int sb[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint8_t* src = &sm.b[buf][bcol[c] + lr][0];
      if constexpr (C::b_fp4) {
        bf[c] = fp4_operand(*reinterpret_cast<const u32x4*>(src + 16 * g));
        sb[c] = reinterpret_cast<const uint8_t*>(&sm.bs[buf][bcol[c] + lr])[g];
      } else {
        bf[c] = fp8_operand(*reinterpret_cast<const u32x4*>(src + 32 * g),
                            *reinterpret_cast<const u32x4*>(src + 32 * g + 16));
        sb[c] = 127;
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (r >= vr) continue;
      const int arow_l = 64 * wm + 16 * r + lr;
      const uint8_t* src = &sm.a[buf][arow_l][0];
      i32x8 af;
      int sa;
      if constexpr (C::a_fp4) {
        af = fp4_operand(*reinterpret_cast<const u32x4*>(src + 16 * g));
      } else {
        af = fp8_operand(*reinterpret_cast<const u32x4*>(src + 32 * g),
                         *reinterpret_cast<const u32x4*>(src + 32 * g + 16));
      }
      if constexpr (AM == kActT128) {
        sa = 127;
        // this lane's 4 output rows of tile r: 64wm + 16r + 4g + j
        const f32x4 rs = *reinterpret_cast<const f32x4*>(&sm.as[buf][64 * wm + 16 * r + 4 * g]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const f32x4 part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              af, bf[c], f32x4{0.f, 0.f, 0.f, 0.f}, C::afmt, C::bfmt, 0, sa, 0, sb[c]);
          const float wsc = (OP == kOpGateUp && c >= 2) ? ws1 : ws0;
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[r][c][j] = fmaf(part[j], rs[j] * wsc, acc[r][c][j]);
        }
      } else {
        sa = reinterpret_cast<const uint8_t*>(&sm.as[buf][arow_l])[g];
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[r][c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              af, bf[c], acc[r][c], C::afmt, C::bfmt, 0, sa, 0, sb[c]);
      }
    }
  };

  // Two register stages in flight (steps ks+1, ks+2) while step ks is
  // computed from LDS; the loop is unrolled by two for static stage names.
  // The T128 weight scales of the step held by LDS buffer b: wsb0[b], wsb1[b].
  {
    QStage<AM> s0, s1;
    float wsb0[2], wsb1[2];
    load_stage(0, s0);
    store_stage(0, s0);
    wsb0[0] = s0.ws0;
    wsb1[0] = s0.ws1;
    wsb0[1] = wsb1[1] = 0.f;
    if (nk > 1) load_stage(1, s0);
    if (nk > 2) load_stage(2, s1);
    __syncthreads();
    for (int ks = 0; ks < nk; ks += 2) {
      compute_step(0, wsb0[0], wsb1[0]);
      if (ks + 1 < nk) {
        store_stage(1, s0);
        wsb0[1] = s0.ws0;
        wsb1[1] = s0.ws1;
        if (ks + 3 < nk) load_stage(ks + 3, s0);
      }
      __syncthreads();
      if (ks + 1 >= nk) break;
      compute_step(1, wsb0[1], wsb1[1]);
      if (ks + 2 < nk) {
        store_stage(0, s1);
        wsb0[0] = s1.ws0;
        wsb1[0] = s1.ws1;
        if (ks + 4 < nk) load_stage(ks + 4, s1);
      }
      __syncthreads();
    }
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
          const float h = silu_fast(acc[r][c][j]) * acc[r][c + 2][j];
          reinterpret_cast<uint16_t*>(p.out)[(size_t)row * N + n] = f32_to_bf16(h);
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

template <int AM, int OP>
hipError_t launch_q(QParams p, int n_row_tiles, hipStream_t s) {
  const int ntn = (OP == kOpGateUp) ? (p.w0.rows + BN / 2 - 1) / (BN / 2) : (p.w0.rows + BN - 1) / BN;
  p.ntn = ntn;
  p.max_rt = n_row_tiles;
  const int per = (n_row_tiles * ntn + kXcds - 1) / kXcds;
  if (per == 0) return hipSuccess;
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
  p.a_pitch_scales = mx ? act_scale_pitch(K) : (K + 127) / 128;
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
