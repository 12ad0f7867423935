// Prefill grouped expert GEMM (row groups larger than a decode batch).
//
// The pages run prefill expert GEMMs "over a compact list of the routed
// segments' tiles instead of a grid over the longest segment" and run the gate
// and up projections in one launch (gitee "dgpp" README, "Execution and
// performance", engine.expert_tile_list and engine.expert_gemm_pair).  Here:
//
// * one workgroup (4 wavefronts) computes a 128-row tile of one expert's group
//   (rows = permuted (token, slot) pairs) against 128 weight rows: for
//   gate/up, 64 gate rows and the matching 64 up rows (SwiGLU in the
//   epilogue, 64 h columns out); for down, 128 output columns;
// * K advances 64 at a time; the weight tile is decoded once per step from its
//   checkpoint format into bf16 in LDS (NVFP4: E2M1 x E4M3, exact in bf16;
//   MXFP4: E2M1 x E8M0; FP8: E4M3, with each 128x128 block scale applied to the
//   partial sum of its K block) and shared by all 128 rows; activations are
//   gathered into LDS; both are double-buffered in registers across steps;
// * each wavefront computes a 64x64 sub-tile with v_mfma_f32_16x16x32_bf16
//   (bf16 products exact in fp32, fp32 accumulation);
// * blocks are ordered so that every column tile of one row tile lands on the
//   same XCD (its activation rows stay in that XCD's L2).
#include <type_traits>

#include "gemv_core.cuh"

namespace moe {
namespace {

constexpr int BM = kGemmTileM, BN = 128, BK = 64;
// LDS row pitch (bf16 elements).  160-byte rows: measured with the LDS
// bank-conflict counter on gfx950, the fragment reads below (row = lane % 16,
// 16-byte column = lane / 16) are conflict-free and take half the LDS cycles
// of any other pitch from 136 to 192 bytes, and the staging writes are
// conflict-free when the two threads of a row interleave their 16-byte pieces.
constexpr int LDSW = BK + 16;
constexpr int kXcds = 8;
// Row tiles per run of the tile order (gemm_tile_order).
constexpr int kRowRun = 4;

struct GemmParams {
  WDesc w0, w1;           // gate, up (gate/up) or down (both)
  const uint16_t* in;     // x [T][H] (gate/up) or h [rows][I] (down)
  void* out;              // h bf16 [rows][I] or y fp32 [rows][H]
  const int2* tiles;      // (expert, first permuted row) per row tile; nullptr: shared expert
  const int* n_tiles;
  const int* offsets;     // [E+1] group bounds (routed)
  const int* perm_to_pair;
  int topk;
  int T;                  // shared expert rows
  int in_rows;            // rows of `in`
  int in_rows_total;      // permuted rows (T*k)
  int max_rt;             // row tiles the grid was sized for
  int ntn;                // column tiles
};

struct GemmSmem {
  uint16_t a[2][BM][LDSW];
  uint16_t b[2][BN][LDSW];
};

// Per-thread staging of one K step: 32 activations and 32 weights.
template <int FMT>
struct Stage {
  u32x4 a[4];   // 32 bf16 activations
  u32x4 q[2];   // FP4: q[0] = 32 codes; FP8: q[0..1] = 32 codes
  uint32_t s;   // NVFP4: two E4M3 scales; MXFP4: one E8M0
};

template <int FMT>
__device__ __forceinline__ void decode32(const Stage<FMT>& st, uint32_t (&w)[16]) {
  if constexpr (FMT == FMT_NVFP4) {
    const f32x2 sc = e4m3x2_to_f32(st.s);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const float s = (d < 2) ? sc[0] : sc[1];
      const uint32_t v = st.q[0][d];
      const f32x2 f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 0);
      const f32x2 f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 1);
      const f32x2 f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 2);
      const f32x2 f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 3);
      w[4 * d + 0] = pack_hi16(f0[0] * s, f0[1] * s);
      w[4 * d + 1] = pack_hi16(f1[0] * s, f1[1] * s);
      w[4 * d + 2] = pack_hi16(f2[0] * s, f2[1] * s);
      w[4 * d + 3] = pack_hi16(f3[0] * s, f3[1] * s);
    }
  } else if constexpr (FMT == FMT_MXFP4) {
    const float s = __uint_as_float(st.s << 23);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t v = st.q[0][d];
      union {
        bf16x2 h;
        uint32_t u;
      } c0, c1, c2, c3;
      c0.h = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 0);
      c1.h = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 1);
      c2.h = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 2);
      c3.h = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 3);
      w[4 * d + 0] = c0.u;
      w[4 * d + 1] = c1.u;
      w[4 * d + 2] = c2.u;
      w[4 * d + 3] = c3.u;
    }
  } else {
    // FP8: the block scale multiplies the 128-K partial; MXFP8: the E8M0 of
    // the thread's 32-K block as the converter's scale (exact in bf16)
    const float s = (FMT == FMT_MXFP8) ? __uint_as_float(st.s << 23) : 1.0f;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const uint32_t v = st.q[d / 4][d % 4];
      union {
        bf16x2 h;
        uint32_t u;
      } c0, c1;
      c0.h = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, s, false);
      c1.h = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, s, true);
      w[2 * d + 0] = c0.u;
      w[2 * d + 1] = c1.u;
    }
  }
}

template <int FMT, int OP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void grouped_gemm_kernel(
    GemmParams p) {
  __shared__ GemmSmem sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // XCD-aware order: workgroup b runs on XCD b % 8.  Each XCD takes a
  // contiguous range of the live (row tile, column tile) pairs in the order
  // of gemm_tile_order (runs of up to four row tiles of one expert, row tiles
  // fastest), so a run's workgroups share each weight column tile and its
  // activation rows in that XCD's L2 (wide FP8 prefill gate/up 6.31 -> 6.15
  // ms against column tiles fastest, its 1x128 mode 3.48 -> 3.22 ms).
  const int n_rt = (p.tiles == nullptr) ? (p.T + BM - 1) / BM : min(*p.n_tiles, p.max_rt);
  const int live = n_rt * p.ntn;
  const int per = (live + kXcds - 1) / kXcds;
  const int xcd = blockIdx.x % kXcds, local = blockIdx.x / kXcds;
  const int idx = xcd * per + local;
  if (local >= per || idx >= live) return;
  const int2 tn = gemm_tile_order(idx, p.ntn, n_rt, kRowRun, p.tiles, p.offsets, BM);
  const int mt = tn.x, nt = tn.y;
  int e, m0, m1;
  if (p.tiles == nullptr) {  // shared expert over rows 0..T-1
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
  const int n0 = nt * ((OP == kOpGateUp) ? BN / 2 : BN);  // first weight row of this tile

  // ---- staging roles: thread -> (tile row, K half) ----
  const int srow = tid >> 1, shalf = tid & 1;
  // Activation row.  Rows past the group (and, defensively, rows whose index
  // is out of range) read row m0 / row 0 instead of zeros: an MFMA output
  // row depends on its own A row only, and padding rows are never stored,
  // so every full K step loads unconditionally.
  const uint16_t* arow;
  bool arow_ok;
  {
    const int pr = m0 + srow;
    const bool in_group = pr < m1;
    const int row = in_group ? pr : m0;  // m0 < m1: a valid row of the group
    int ir = (p.tiles != nullptr && OP == kOpGateUp) ? p.perm_to_pair[row] / p.topk : row;
    arow_ok = in_group && (unsigned)ir < (unsigned)p.in_rows;
    if ((unsigned)ir >= (unsigned)p.in_rows) ir = 0;
    arow = p.in + (size_t)ir * K;
  }
  // Weight row: gate/up tiles hold 64 gate rows then the matching 64 up rows.
  // Rows past N read row N-1 (their output columns are never stored).
  const WDesc& wq = (OP == kOpGateUp && srow >= BN / 2) ? p.w1 : p.w0;
  const int wr0 = (OP == kOpGateUp) ? n0 + (srow & (BN / 2 - 1)) : n0 + srow;
  const bool wvalid = wr0 < N;
  const int wr = wvalid ? wr0 : N - 1;
  const int rb = row_bytes<FMT>(K);
  const uint8_t* wrow = wq.codes + e * wq.stride_codes + (size_t)wr * rb;
  const uint8_t* wsrow = scale_row_ptr<FMT>(wq, e, wr);

  // A full K step (k0 + BK <= K): no guards.
  auto load_full = [&](int k0, Stage<FMT>& st) {
    const int kb = k0 + 32 * shalf;
#pragma unroll
    for (int i = 0; i < 4; ++i) st.a[i] = *reinterpret_cast<const u32x4*>(arow + kb + 8 * i);
    if constexpr (fmt_is_fp8(FMT)) {
      st.q[0] = *reinterpret_cast<const u32x4*>(wrow + kb);
      st.q[1] = *reinterpret_cast<const u32x4*>(wrow + kb + 16);
      st.s = (FMT == FMT_MXFP8) ? wsrow[kb / 32] : 0u;
    } else {
      st.q[0] = *reinterpret_cast<const u32x4*>(wrow + kb / 2);
      st.q[1] = u32x4{0, 0, 0, 0};
      if constexpr (FMT == FMT_NVFP4)
        st.s = *reinterpret_cast<const uint16_t*>(wsrow + kb / 16);
      else
        st.s = wsrow[kb / 32];
    }
  };
  // The last, partial K step: zeros past K on both operands.
  auto load_tail = [&](int k0, Stage<FMT>& st) {
    const int kb = k0 + 32 * shalf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = kb + 8 * i;
      st.a[i] = (arow_ok && k < K) ? *reinterpret_cast<const u32x4*>(arow + k)
                                   : u32x4{0, 0, 0, 0};
    }
    st.q[0] = u32x4{0, 0, 0, 0};
    st.q[1] = u32x4{0, 0, 0, 0};
    st.s = 0;
    if (wvalid && kb < K) {
      if constexpr (FMT == FMT_MXFP8) {  // K % 32 == 0: the 32-K block is whole
        st.q[0] = *reinterpret_cast<const u32x4*>(wrow + kb);
        st.q[1] = *reinterpret_cast<const u32x4*>(wrow + kb + 16);
        st.s = wsrow[kb / 32];
      } else if constexpr (FMT == FMT_FP8) {
        st.q[0] = *reinterpret_cast<const u32x4*>(wrow + kb);
        if (kb + 16 < K) st.q[1] = *reinterpret_cast<const u32x4*>(wrow + kb + 16);
      } else {
        st.q[0] = *reinterpret_cast<const u32x4*>(wrow + kb / 2);
        if constexpr (FMT == FMT_NVFP4)
          st.s = *reinterpret_cast<const uint16_t*>(wsrow + kb / 16);
        else
          st.s = wsrow[kb / 32];
      }
    }
  };
  // FAST (see the main loop): every K step is full, no guard.
  auto load_stage = [&](int k0, Stage<FMT>& st, auto fast_t) {
    if constexpr (decltype(fast_t)::value) {
      load_full(k0, st);
    } else {
      if (k0 + BK <= K)
        load_full(k0, st);
      else
        load_tail(k0, st);
    }
  };
  // K order inside a step's LDS rows: the 8-element piece i of K half h
  // (step offset 32h + 8i) sits at column 8(2i + h).  A and B use the same
  // order, so each MFMA still pairs equal K; a step's MFMAs cover all 64 K.
  auto store_stage = [&](int buf, const Stage<FMT>& st) {
    uint16_t* ad = &sm.a[buf][srow][8 * shalf];
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(ad + 16 * i) = st.a[i];
    uint32_t w[16];
    decode32<FMT>(st, w);
    uint16_t* bd = &sm.b[buf][srow][8 * shalf];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4*>(bd + 16 * i) = u32x4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
  };

  // ---- MFMA roles: wave (wm, wn) owns rows [64wm, +64) and four 16-wide
  // column tiles: down -> B rows 64wn + 16c; gate/up -> gate rows 32wn + 16c
  // (c = 0,1) and the matching up rows 64 + 32wn + 16c (c = 2,3).
  const int wm = wave >> 1, wn = wave & 1;
  int bcol[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
    bcol[c] = (OP == kOpGateUp) ? ((c < 2) ? 32 * wn + 16 * c : 64 + 32 * wn + 16 * (c - 2))
                                : 64 * wn + 16 * c;
  f32x4 acc[4][4];
  f32x4 tmp[4][4];  // FP8: the current 128-wide K block
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
      tmp[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  // 16-row MFMA tiles of this wave that hold rows of the group (a short
  // group's tile is mostly padding: skip the padding's MFMAs and reads)
  const int vrows = m1 - m0 - 64 * wm;
  const int vr = vrows <= 0 ? 0 : min(4, (vrows + 15) / 16);
  const int nk = (K + BK - 1) / BK;

  // MFMAs of step ks on LDS buffer buf, and (FP8) the 128-wide K block close.
  // FAST: all four 16-row tiles of the wave hold group rows (no per-tile
  // branches, so the compiler can interleave these MFMAs with the next
  // step's decode).
  auto compute_step = [&](int buf, int ks, auto fast_t) {
    constexpr bool FAST = decltype(fast_t)::value;
    if (FAST || vr > 0) {
#pragma unroll
      for (int kk = 0; kk < BK; kk += 32) {
        bf16x8 af[4], bfr[4];
        const int ko = kk + 8 * (lane >> 4);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          bfr[c] = *reinterpret_cast<const bf16x8*>(&sm.b[buf][bcol[c] + (lane & 15)][ko]);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (FAST || r < vr)
            af[r] = *reinterpret_cast<const bf16x8*>(&sm.a[buf][64 * wm + 16 * r + (lane & 15)][ko]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (!FAST && r >= vr) continue;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            if constexpr (FMT == FMT_FP8)
              tmp[r][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[r], bfr[c], tmp[r][c], 0, 0, 0);
            else
              acc[r][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[r], bfr[c], acc[r][c], 0, 0, 0);
          }
        }
      }
    }
    if constexpr (FMT == FMT_FP8) {
      // close a 128-wide K block: acc += s(block) * partial
      const int kend = (ks + 1) * BK;
      if ((kend % 128) == 0 || ks + 1 == nk) {
        const int kblk = (ks * BK) / 128;
        const int cb = (K + 127) / 128;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const WDesc& wc = (OP == kOpGateUp && c >= 2) ? p.w1 : p.w0;
          const int row = n0 + ((OP == kOpGateUp) ? (bcol[c] & (BN / 2 - 1)) : bcol[c]);
          float s = 0.f;
          if (row < N) {
            const float* sp = reinterpret_cast<const float*>(
                reinterpret_cast<const uint8_t*>(wc.scales) + e * wc.stride_scales);
            s = sp[(size_t)(row / 128) * cb + kblk];
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            acc[r][c] = acc[r][c] + s * tmp[r][c];
            tmp[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
        }
      }
    }
  };

  // Two register stages in flight: while step ks is computed from LDS, the
  // global loads of steps ks+1 and ks+2 are outstanding, so each load has two
  // compute steps to arrive.  The loop is unrolled by two so that the
  // stages keep static register names.
  // The loop body exists twice: a fast version for the common case (full
  // 128-row tile half for this wave, K a multiple of BK), with no branch
  // between the MFMAs, and the general one.  Both barriers are block-wide,
  // so every wavefront of the block takes its own version safely.
  auto main_loop = [&](auto fast_t) {
    Stage<FMT> s0, s1;
    load_stage(0, s0, fast_t);
    store_stage(0, s0);
    if (nk > 1) load_stage(BK, s0, fast_t);
    if (nk > 2) load_stage(2 * BK, s1, fast_t);
    __syncthreads();
    int ks = 0;
    if constexpr (decltype(fast_t)::value) {
      // Steady state without conditions (steps ks+1 .. ks+4 exist): each
      // half-step is one basic block, which the scheduler can interleave.
      for (; ks + 4 < nk; ks += 2) {
        compute_step(0, ks, fast_t);
        store_stage(1, s0);
        load_stage((ks + 3) * BK, s0, fast_t);
        __syncthreads();
        compute_step(1, ks + 1, fast_t);
        store_stage(0, s1);
        load_stage((ks + 4) * BK, s1, fast_t);
        __syncthreads();
      }
    }
    for (; ks < nk; ks += 2) {
      // step ks on buffer 0; s0 holds step ks+1, s1 holds step ks+2
      compute_step(0, ks, fast_t);
      if (ks + 1 < nk) {
        store_stage(1, s0);
        if (ks + 3 < nk) load_stage((ks + 3) * BK, s0, fast_t);
      }
      __syncthreads();
      if (ks + 1 >= nk) break;
      // step ks+1 on buffer 1; s1 holds step ks+2, s0 holds step ks+3
      compute_step(1, ks + 1, fast_t);
      if (ks + 2 < nk) {
        store_stage(0, s1);
        if (ks + 4 < nk) load_stage((ks + 4) * BK, s1, fast_t);
      }
      __syncthreads();
    }
  };
  if (vr == 4 && K % BK == 0)
    main_loop(std::true_type{});
  else
    main_loop(std::false_type{});

  // ---- epilogue: lane holds rows 4*(lane/16)+j of each 16-row tile, column lane%16 ----
  const float ts0 = (FMT == FMT_NVFP4) ? p.w0.tscale[e] : 1.0f;
  const float ts1 = (FMT == FMT_NVFP4) ? p.w1.tscale[e] : 1.0f;
  const int col = lane & 15;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = m0 + 64 * wm + 16 * r + 4 * (lane >> 4) + j;
      if (row >= m1) continue;
      const int orow = row;
      if constexpr (OP == kOpGateUp) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int n = nt * (BN / 2) + 32 * wn + 16 * c + col;
          if (n >= N) continue;
          const float g = acc[r][c][j] * ts0;
          const float u = acc[r][c + 2][j] * ts1;
          const float h = silu_fast(g) * u;
          reinterpret_cast<uint16_t*>(p.out)[(size_t)orow * N + n] = f32_to_bf16(h);
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int n = n0 + 64 * wn + 16 * c + col;
          if (n >= N) continue;
          reinterpret_cast<float*>(p.out)[(size_t)orow * N + n] = acc[r][c][j] * ts0;
        }
      }
    }
  }
}

template <int FMT, int OP>
hipError_t launch_t(GemmParams p, int n_row_tiles, hipStream_t s) {
  const int ntn = (OP == kOpGateUp) ? (p.w0.rows + BN / 2 - 1) / (BN / 2) : (p.w0.rows + BN - 1) / BN;
  p.ntn = ntn;
  p.max_rt = n_row_tiles;
  const int per = (n_row_tiles * ntn + kXcds - 1) / kXcds;
  if (per == 0) return hipSuccess;
  return launch(grouped_gemm_kernel<FMT, OP>, dim3(per * kXcds), dim3(256), 0, s, p);
}

template <int FMT>
hipError_t launch_fmt(int op, const GemmParams& p, int n_row_tiles, hipStream_t s) {
  return op == kOpGateUp ? launch_t<FMT, kOpGateUp>(p, n_row_tiles, s)
                         : launch_t<FMT, kOpDown>(p, n_row_tiles, s);
}

}  // namespace

hipError_t launch_grouped_gemm(int op, const WDesc& w0, const WDesc& w1, const GroupArgs& g,
                               const int* tiles, const int* n_tiles, int max_tiles,
                               const uint16_t* in, void* out, hipStream_t s) {
  const int dma_rows = (g.shared || op == kOpGateUp) ? g.T : g.T * g.topk;
  if (grouped_gemm_dma_fits(op, w0, w1, dma_rows) && reinterpret_cast<uintptr_t>(in) % 16 == 0)
    return launch_grouped_gemm_dma(op, w0, w1, g, tiles, n_tiles, max_tiles, in, out, s);
  GemmParams p;
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
  switch (w0.fmt) {
    case FMT_NVFP4: return launch_fmt<FMT_NVFP4>(op, p, nrt, s);
    case FMT_MXFP4: return launch_fmt<FMT_MXFP4>(op, p, nrt, s);
    case FMT_FP8: return launch_fmt<FMT_FP8>(op, p, nrt, s);
    case FMT_MXFP8: return launch_fmt<FMT_MXFP8>(op, p, nrt, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
