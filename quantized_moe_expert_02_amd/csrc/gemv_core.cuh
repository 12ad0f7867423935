// Expert GEMV core for small row groups (decode): weights streamed once per
// group, decoded in registers, contracted on the bf16 matrix cores.
//
// Decode is bound by memory bandwidth, and the decode kernels read the
// weights at the memory's line rate (forum thread "DGPP: a GB10-optimized
// C++/CUDA inference engine", the "Lossless bf12" post); the
// expert kernels are written per weight format and read the checkpoint bytes
// with no dequantized copy ("DGPP" README, intro bullet on checkpoint formats).
//
// Design for gfx950:
// * One 16-row tile of an expert projection per wave, one MFMA
//   (v_mfma_f32_16x16x32_bf16) per 32-wide K slice; the B operand is the
//   group's input rows (up to 16, zero-padded).  The K order inside a 128-wide
//   chunk is permuted so that each lane's 16-byte load of packed codes feeds
//   its own MFMA operands directly (lane r+16g holds K = 128c+32g+8i.. for MFMA
//   i), and the four lanes of a row read 64 contiguous bytes.
// * All loads of a batch of chunks (weights, scales, activations) are issued
//   before any of them is used, so a wave waits one memory round trip per
//   batch rather than one per chunk.
// * NVFP4: E2M1 x E4M3 has at most 6 significant bits, so the decoded weight
//   q*s is exact in bf16; the per-expert fp32 tensor scale multiplies the fp32
//   accumulator.  MXFP4: the E8M0 power of two is applied by the converter.
//   FP8: E4M3 is exact in bf16; the 128x128 block scale multiplies each
//   chunk's partial sum (a chunk never straddles a 128-wide K block).
// * Products of bf16 operands are exact in fp32; accumulation is fp32.
// * Gate and up run in one pass (gitee "dgpp" README, "Execution and
//   performance", engine.expert_gemm_pair: both projections in one launch) and
//   SwiGLU runs in the epilogue, writing h in bf16.
#pragma once
#include "moe_launch.h"

namespace moe {

constexpr int kOpGateUp = 0;
constexpr int kOpDown = 1;

// Raw per-lane data of one 128-wide K chunk of one 16-row tile.
template <int FMT>
struct ARaw;
template <>
struct ARaw<FMT_NVFP4> {
  u32x4 q;     // 32 E2M1 codes
  uint32_t s;  // two E4M3 scale bytes (low 16 bits)
};
template <>
struct ARaw<FMT_MXFP4> {
  u32x4 q;
  uint32_t s;  // one E8M0 byte
};
template <>
struct ARaw<FMT_FP8> {
  u32x4 q0, q1;  // 32 E4M3 codes
  float s;       // the 128x128 block scale of this chunk
};
template <>
struct ARaw<FMT_MXFP8> {
  u32x4 q0, q1;  // 32 E4M3 codes: one MX block
  uint32_t s;    // its E8M0 byte
};

template <int FMT>
__device__ __forceinline__ int row_bytes(int K) {
  return fmt_is_fp8(FMT) ? K : K / 2;
}

// Load the lane's part of chunk c for weight row `row` (nullptr = zero row).
// SC = false: FP4 codes only (the scales come from exchange_scales).
template <int FMT, bool SC = true>
__device__ __forceinline__ ARaw<FMT> load_a(const uint8_t* __restrict__ row,
                                            const uint8_t* __restrict__ srow, int c, int g, int K) {
  ARaw<FMT> a;
  const int k0 = 128 * c + 32 * g;
  if constexpr (FMT == FMT_FP8) {
    a.q0 = u32x4{0, 0, 0, 0};
    a.q1 = u32x4{0, 0, 0, 0};
    a.s = 0.f;
    if (row != nullptr) {
      if (k0 < K) a.q0 = *reinterpret_cast<const u32x4*>(row + k0);
      if (k0 + 16 < K) a.q1 = *reinterpret_cast<const u32x4*>(row + k0 + 16);
      a.s = reinterpret_cast<const float*>(srow)[c];
    }
  } else if constexpr (FMT == FMT_MXFP8) {
    a.q0 = u32x4{0, 0, 0, 0};
    a.q1 = u32x4{0, 0, 0, 0};
    if constexpr (SC) a.s = 0;
    if (row != nullptr && k0 < K) {  // K % 32 == 0: the block is whole
      a.q0 = *reinterpret_cast<const u32x4*>(row + k0);
      a.q1 = *reinterpret_cast<const u32x4*>(row + k0 + 16);
      if constexpr (SC) a.s = srow[k0 / 32];
    }
  } else {
    a.q = u32x4{0, 0, 0, 0};
    // SC = false: s is written by the caller (exchange_scales); leaving it
    // unwritten here keeps the compiler from waiting on every load in flight
    // before the zeroing (the registers double as the 2-byte loads' targets).
    if constexpr (SC) a.s = 0;
    if (row != nullptr && k0 < K) {
      a.q = *reinterpret_cast<const u32x4*>(row + k0 / 2);
      if constexpr (SC) {
        if constexpr (FMT == FMT_NVFP4)
          a.s = *reinterpret_cast<const uint16_t*>(srow + k0 / 16);
        else
          a.s = srow[k0 / 32];
      }
    }
  }
  return a;
}

// Decode the 8 weights of MFMA I (0..3) of a chunk into bf16.
template <int FMT, int I>
__device__ __forceinline__ bf16x8 decode_a(const ARaw<FMT>& a) {
  union {
    bf16x8 v;
    uint32_t u[4];
    bf16x2 h[4];
  } r;
  if constexpr (FMT == FMT_NVFP4) {
    const uint32_t d = a.q[I];
    const f32x2 sc = e4m3x2_to_f32(a.s);
    const float s = (I < 2) ? sc[0] : sc[1];
    const f32x2 f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 0);
    const f32x2 f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 1);
    const f32x2 f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 2);
    const f32x2 f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 3);
    r.u[0] = pack_hi16(f0[0] * s, f0[1] * s);
    r.u[1] = pack_hi16(f1[0] * s, f1[1] * s);
    r.u[2] = pack_hi16(f2[0] * s, f2[1] * s);
    r.u[3] = pack_hi16(f3[0] * s, f3[1] * s);
  } else if constexpr (FMT == FMT_MXFP4) {
    const uint32_t d = a.q[I];
    const float s = __uint_as_float(a.s << 23);  // 2^(code-127) as the converter's scale
    r.h[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 0);
    r.h[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 1);
    r.h[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 2);
    r.h[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 3);
  } else {
    // FP8: the block scale multiplies the chunk's partial sum later; MXFP8:
    // the E8M0 scale as the converter's scale (E4M3 x 2^e is exact in bf16)
    float s = 1.0f;
    if constexpr (FMT == FMT_MXFP8) s = __uint_as_float(a.s << 23);
    const uint32_t d0 = (I < 2) ? a.q0[2 * I] : a.q1[2 * I - 4];
    const uint32_t d1 = (I < 2) ? a.q0[2 * I + 1] : a.q1[2 * I - 3];
    r.h[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, s, false);
    r.h[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, s, true);
    r.h[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, s, false);
    r.h[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, s, true);
  }
  return r.v;
}

// 8 bf16 activations of one MFMA slice (zeros past K or for a padding row).
__device__ __forceinline__ u32x4 load_b(const uint16_t* __restrict__ brow, int k, int K) {
  u32x4 r = u32x4{0, 0, 0, 0};
  if (brow != nullptr && k < K) r = *reinterpret_cast<const u32x4*>(brow + k);
  return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& u) {
  union {
    u32x4 u;
    bf16x8 v;
  } r;
  r.u = u;
  return r.v;
}

template <int FMT>
__device__ __forceinline__ const uint8_t* scale_row_ptr(const WDesc& w, int e, int n) {
  if constexpr (FMT == FMT_NVFP4)
    return reinterpret_cast<const uint8_t*>(w.scales) + e * w.stride_scales +
           (size_t)n * (w.cols / 16);
  else if constexpr (FMT == FMT_MXFP4 || FMT == FMT_MXFP8)
    return reinterpret_cast<const uint8_t*>(w.scales) + e * w.stride_scales +
           (size_t)n * (w.cols / 32);
  else  // FP8: the row of 128x128 block scales covering output row n
    return reinterpret_cast<const uint8_t*>(w.scales) + e * w.stride_scales +
           (size_t)(n / 128) * ((w.cols + 127) / 128) * 4;
}

// FP4 block scales by whole chunks (WDesc::wide).  The lane (r, g) that
// needs the two NVFP4 (one MXFP4) scale bytes of K piece 32g..32g+31 of four
// chunks would otherwise issue four 2-byte loads that each touch 16 rows'
// scale lines; instead it loads the whole scale word (8 E4M3 / 4 E8M0 bytes)
// of one chunk of its row, and a wave-local LDS transpose hands every lane
// the bytes of its own K piece of each chunk.
struct alignas(8) ScaleXchg {
  uint16_t v[16][4][4];  // [row][K piece][chunk of the batch]
};

template <int FMT>
__device__ __forceinline__ uint2 load_scale_word(const uint8_t* __restrict__ srow, int c, int nch) {
  uint2 w = make_uint2(0u, 0u);
  if (srow != nullptr && c < nch) {
    if constexpr (FMT == FMT_NVFP4)
      w = *reinterpret_cast<const uint2*>(srow + 8 * c);
    else
      w.x = *reinterpret_cast<const uint32_t*>(srow + 4 * c);
  }
  return w;
}

// Lane (r, g) passes the scale word of chunk g of a four-chunk batch (row r)
// and receives, for chunk d of the batch, the ARaw::s of its K piece g in
// bits [16d, 16d + 16) (NVFP4) or [8d, 8d + 8) (MXFP4).  Wave-local: the
// lanes r + 16g of one row are in one wavefront.
template <int FMT>
__device__ __forceinline__ uint2 exchange_scales(uint2 w, ScaleXchg& x, int r, int g) {
  if constexpr (FMT == FMT_NVFP4) {
    x.v[r][0][g] = static_cast<uint16_t>(w.x);
    x.v[r][1][g] = static_cast<uint16_t>(w.x >> 16);
    x.v[r][2][g] = static_cast<uint16_t>(w.y);
    x.v[r][3][g] = static_cast<uint16_t>(w.y >> 16);
  } else {
    uint8_t* b = reinterpret_cast<uint8_t*>(&x.v[r][0][0]);  // [K piece][chunk] bytes
#pragma unroll
    for (int p = 0; p < 4; ++p) b[4 * p + g] = static_cast<uint8_t>(w.x >> (8 * p));
  }
  // LDS accesses of one wavefront complete in order; this only keeps the
  // compiler from moving the reads above the writes of the other lanes.
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  __asm__ volatile("" ::: "memory");
  uint2 o;
  if constexpr (FMT == FMT_NVFP4) {
    o = *reinterpret_cast<const uint2*>(&x.v[r][g][0]);
  } else {
    o.x = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(&x.v[r][0][0]) + 4 * g);
    o.y = 0u;
  }
  __asm__ volatile("" ::: "memory");
  return o;
}

template <int FMT>
__device__ __forceinline__ uint32_t scale_of_chunk(uint2 o, int d) {
  if constexpr (FMT == FMT_NVFP4)
    return ((d < 2 ? o.x : o.y) >> (16 * (d & 1))) & 0xffffu;
  else
    return (o.x >> (8 * d)) & 0xffu;
}

// Where a group's rows come from and go to.
struct GemvRows {
  int e;                // expert index within the projection
  int p0;               // first output row (permuted position, or 0 for the shared expert)
  int nrows;            // rows in the group
  const int16_t* rows_in;   // kInList: input row of each group row
  const int16_t* rows_out;  // kInList: output row of each group row
};

// How group row j maps to an input row of `in`.
enum : int {
  kInShared = 0,  // j (the shared expert over every row); output row j
  kInPerm = 1,    // perm_to_pair[p0 + j] / topk; output row p0 + j
  kInDirect = 2,  // p0 + j; output row p0 + j
  kInList = 3,    // rows_in[j]; output row rows_out[j]
};

struct GemvIO {
  const uint16_t* in;       // bf16 input rows
  void* out;                // bf16 h or fp32 y
  const int* perm_to_pair;  // kInPerm
  int topk;
  int mode;                 // kIn*
  int in_rows;              // rows of `in` (an input row outside is read as zeros)
};

template <int WN, int WK, int NT>
struct GemvSmem {
  f32x4 red[WN * WK][NT][64];
  ScaleXchg sx[WN * WK][NT];
};

// One workgroup (64*WN*WK threads): output rows [tile*16*WN, +16*WN) of one
// expert projection for every row of the group.  `sm` must be block-shared.
// WIDE: FP4 scales by whole chunks (exchange_scales); a separate copy of the
// body, so that neither copy carries the other's registers or load waits.
template <int FMT, int OP, int WN, int WK, bool WIDE>
__device__ __forceinline__ void gemv_tile_impl(const WDesc& w0, const WDesc& w1, const GemvIO& io,
                                               const GemvRows& gr, int tile,
                                               GemvSmem<WN, WK, (OP == kOpGateUp) ? 2 : 1>& sm) {
  constexpr int NT = (OP == kOpGateUp) ? 2 : 1;  // weight tiles per wave
  constexpr int D = 4;                            // chunks in flight per wave
  static_assert(D == 4, "exchange_scales maps lane group g to chunk g of a batch");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wn = wave / WK, wk = wave % WK;
  const int e = gr.e, p0 = gr.p0, nrows = gr.nrows;
  const int N = w0.rows, K = w0.cols;
  const int n0 = (tile * WN + wn) * 16;
  const bool wave_on = n0 < N;  // waves past N only join the barriers
  const int r = lane & 15, g = lane >> 4;
  const int nrow = n0 + r;
  const int rb = row_bytes<FMT>(K);
  const WDesc* wd[NT];
  wd[0] = &w0;
  if constexpr (NT == 2) wd[1] = &w1;
  const uint8_t* arow[NT];
  const uint8_t* srow[NT];
#pragma unroll
  for (int q = 0; q < NT; ++q) {
    const bool on = wave_on && nrow < N;
    arow[q] = on ? wd[q]->codes + e * wd[q]->stride_codes + (size_t)nrow * rb : nullptr;
    srow[q] = on ? scale_row_ptr<FMT>(*wd[q], e, nrow) : nullptr;
  }
  const int nch = (K + 127) / 128;
  constexpr bool wide = WIDE && FMT != FMT_FP8;
  // NVFP4 per-expert tensor scales: loaded with the first weight batch (not
  // in the epilogue, where the load would cost one more memory round trip).
  float ts[NT];
#pragma unroll
  for (int q = 0; q < NT; ++q) ts[q] = 1.0f;

  for (int pass = 0; pass < nrows; pass += 16) {
    const int grow = pass + r;
    const bool row_ok = grow < nrows;
    // Issue the row-index load first; it is consumed after the weight loads.
    int idx = 0;
    if (row_ok) {
      if (io.mode == kInPerm)
        idx = io.perm_to_pair[p0 + grow];
      else if (io.mode == kInList)
        idx = gr.rows_in[grow];
    }
    const uint16_t* brow = nullptr;
    f32x4 acc[NT];
#pragma unroll
    for (int q = 0; q < NT; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (wave_on) {
      bool first = true;
      for (int cb = wk; cb < nch; cb += WK * D) {
        ARaw<FMT> ar[D][NT];
        uint2 sw[NT];
#pragma unroll
        for (int q = 0; q < NT; ++q) sw[q] = make_uint2(0u, 0u);
        if constexpr (wide) {
#pragma unroll
          for (int d = 0; d < D; ++d) {
            const int c = cb + d * WK;
#pragma unroll
            for (int q = 0; q < NT; ++q)
              ar[d][q] = load_a<FMT, false>(c < nch ? arow[q] : nullptr, nullptr, c, g, K);
          }
#pragma unroll
          for (int q = 0; q < NT; ++q) sw[q] = load_scale_word<FMT>(srow[q], cb + g * WK, nch);
        } else {
#pragma unroll
          for (int d = 0; d < D; ++d) {
            const int c = cb + d * WK;
#pragma unroll
            for (int q = 0; q < NT; ++q)
              ar[d][q] = load_a<FMT>(c < nch ? arow[q] : nullptr, srow[q], c, g, K);
          }
        }
        if (first) {
          first = false;
          if constexpr (FMT == FMT_NVFP4) {
            if (pass == 0) {
#pragma unroll
              for (int q = 0; q < NT; ++q) ts[q] = wd[q]->tscale[e];
            }
          }
          if (row_ok) {
            int in_row;
            if (io.mode == kInShared)
              in_row = grow;
            else if (io.mode == kInPerm)
              in_row = idx / io.topk;
            else if (io.mode == kInDirect)
              in_row = p0 + grow;
            else
              in_row = idx;
            if ((unsigned)in_row < (unsigned)io.in_rows) brow = io.in + (size_t)in_row * K;
          }
        }
        u32x4 bx[D][4];
#pragma unroll
        for (int d = 0; d < D; ++d) {
          const int c = cb + d * WK;
          const int kb = 128 * c + 32 * g;
#pragma unroll
          for (int i = 0; i < 4; ++i) bx[d][i] = load_b(c < nch ? brow : nullptr, kb + 8 * i, K);
        }
        if constexpr (wide) {
#pragma unroll
          for (int q = 0; q < NT; ++q) {
            const uint2 o = exchange_scales<FMT>(sw[q], sm.sx[wave][q], r, g);
#pragma unroll
            for (int d = 0; d < D; ++d) ar[d][q].s = scale_of_chunk<FMT>(o, d);
          }
        }
#pragma unroll
        for (int d = 0; d < D; ++d) {
          const int c = cb + d * WK;
          if (c >= nch) break;
#pragma unroll
          for (int q = 0; q < NT; ++q) {
            f32x4 t = (FMT == FMT_FP8) ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[q];
            t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_a<FMT, 0>(ar[d][q]), as_bf16x8(bx[d][0]), t, 0, 0, 0);
            t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_a<FMT, 1>(ar[d][q]), as_bf16x8(bx[d][1]), t, 0, 0, 0);
            t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_a<FMT, 2>(ar[d][q]), as_bf16x8(bx[d][2]), t, 0, 0, 0);
            t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_a<FMT, 3>(ar[d][q]), as_bf16x8(bx[d][3]), t, 0, 0, 0);
            if constexpr (FMT == FMT_FP8) {
              acc[q] = acc[q] + ar[d][q].s * t;
            } else {
              acc[q] = t;
            }
          }
        }
      }
    }

    // Reduce the K-split waves in a fixed order.
    if constexpr (WK > 1) {
#pragma unroll
      for (int q = 0; q < NT; ++q) sm.red[wave][q][lane] = acc[q];
      __syncthreads();
      if (wk == 0) {
#pragma unroll
        for (int q = 0; q < NT; ++q) {
          f32x4 s = sm.red[wave][q][lane];
          for (int j = 1; j < WK; ++j) s = s + sm.red[wave + j][q][lane];
          acc[q] = s;
        }
      }
      __syncthreads();
    }

    // Epilogue: lane holds rows n0 + 4*g + (0..3) for group row pass + r.
    if (wk == 0 && wave_on && row_ok) {
      const int nb = n0 + 4 * g;
      const int orow = (io.mode == kInShared) ? grow
                       : (io.mode == kInList) ? gr.rows_out[grow] : p0 + grow;
      if constexpr (OP == kOpGateUp) {
        uint16_t h[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float gv = acc[0][j] * ts[0];
          const float uv = acc[1][j] * ts[1];
          h[j] = f32_to_bf16(silu_fast(gv) * uv);
        }
        uint16_t* o = reinterpret_cast<uint16_t*>(io.out) + (size_t)orow * N + nb;
        if (nb + 3 < N) {
          *reinterpret_cast<uint2*>(o) =
              make_uint2(h[0] | (uint32_t(h[1]) << 16), h[2] | (uint32_t(h[3]) << 16));
        } else {
          for (int j = 0; j < 4; ++j)
            if (nb + j < N) o[j] = h[j];
        }
      } else {
        float* o = reinterpret_cast<float*>(io.out) + (size_t)orow * N + nb;
        const f32x4 y = acc[0] * ts[0];
        if (nb + 3 < N) {
          *reinterpret_cast<f32x4*>(o) = y;
        } else {
          for (int j = 0; j < 4; ++j)
            if (nb + j < N) o[j] = y[j];
        }
      }
    }
  }
}

template <int FMT, int OP, int WN, int WK>
__device__ __forceinline__ void gemv_tile(const WDesc& w0, const WDesc& w1, const GemvIO& io,
                                          const GemvRows& gr, int tile,
                                          GemvSmem<WN, WK, (OP == kOpGateUp) ? 2 : 1>& sm) {
  if constexpr (FMT != FMT_FP8) {
    if (w0.wide && (OP != kOpGateUp || w1.wide)) {
      gemv_tile_impl<FMT, OP, WN, WK, true>(w0, w1, io, gr, tile, sm);
      return;
    }
  }
  gemv_tile_impl<FMT, OP, WN, WK, false>(w0, w1, io, gr, tile, sm);
}

// Tile shapes: gate/up splits K across 4 waves of one 16-row tile; down
// gives each of 4 waves its own 16-row tile over the full K.
template <int OP>
struct GemvShape;
template <>
struct GemvShape<kOpGateUp> {
  static constexpr int WN = 1, WK = 4;
};
template <>
struct GemvShape<kOpDown> {
  static constexpr int WN = 4, WK = 1;
};

template <int OP>
__host__ __device__ constexpr int gemv_rows_per_block() {
  return 16 * GemvShape<OP>::WN;
}

}  // namespace moe
