// Expert GEMV for small row groups (decode): weights streamed once per group,
// decoded in registers, contracted on the bf16 matrix cores.
//
// "Decode on the Spark is a memory-bandwidth problem" and the decode kernels
// read the weights at the memory's line rate (forum thread "DGPP: a
// GB10-optimized C++/CUDA inference engine", the "Lossless bf12" post); the
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
// * NVFP4: E2M1 x E4M3 has at most 6 significant bits, so the decoded weight
//   q*s is exact in bf16; the per-expert fp32 tensor scale multiplies the fp32
//   accumulator.  MXFP4: the E8M0 power of two is applied by the converter.
//   FP8: E4M3 is exact in bf16; the 128x128 block scale multiplies each
//   chunk's partial sum (a chunk never straddles a 128-wide K block).
// * Products of bf16 operands are exact in fp32; accumulation is fp32.
// * Gate and up are fused in one pass (gitee "dgpp" README, "Execution and
//   performance", engine.expert_gemm_pair: both projections in one launch) and
//   SwiGLU runs in the epilogue, writing h in bf16.
#include "moe_launch.h"

namespace moe {
namespace {

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
};

template <int FMT>
__device__ __forceinline__ int row_bytes(int K) {
  return FMT == FMT_FP8 ? K : K / 2;
}

// Load the lane's part of chunk c for weight row `row` (nullptr = zero row).
template <int FMT>
__device__ __forceinline__ ARaw<FMT> load_a(const uint8_t* __restrict__ row,
                                            const uint8_t* __restrict__ srow, int c, int g, int K) {
  ARaw<FMT> a;
  const int k0 = 128 * c + 32 * g;
  if constexpr (FMT == FMT_FP8) {
    a.q0 = u32x4{0, 0, 0, 0};
    a.q1 = u32x4{0, 0, 0, 0};
    if (row != nullptr) {
      if (k0 < K) a.q0 = *reinterpret_cast<const u32x4*>(row + k0);
      if (k0 + 16 < K) a.q1 = *reinterpret_cast<const u32x4*>(row + k0 + 16);
    }
  } else {
    a.q = u32x4{0, 0, 0, 0};
    a.s = 0;
    if (row != nullptr && k0 < K) {
      a.q = *reinterpret_cast<const u32x4*>(row + k0 / 2);
      if constexpr (FMT == FMT_NVFP4)
        a.s = *reinterpret_cast<const uint16_t*>(srow + k0 / 16);
      else
        a.s = srow[k0 / 32];
    }
  }
  return a;
}

// Decode the 8 weights of MFMA i (I = 0..3) into bf16.
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
    const uint32_t d0 = (I < 2) ? a.q0[2 * I] : a.q1[2 * I - 4];
    const uint32_t d1 = (I < 2) ? a.q0[2 * I + 1] : a.q1[2 * I - 3];
    r.h[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false);
    r.h[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true);
    r.h[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false);
    r.h[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true);
  }
  return r.v;
}

__device__ __forceinline__ bf16x8 load_b(const uint16_t* __restrict__ brow, int k, int K) {
  union {
    bf16x8 v;
    u32x4 u;
  } r;
  r.u = u32x4{0, 0, 0, 0};
  if (brow != nullptr && k < K) r.u = *reinterpret_cast<const u32x4*>(brow + k);
  return r.v;
}

struct GemvParams {
  WDesc w0, w1;
  GroupArgs grp;
  const uint16_t* in;
  void* out;
};

template <int FMT>
__device__ __forceinline__ const uint8_t* scale_row_ptr(const WDesc& w, int e, int n) {
  if constexpr (FMT == FMT_NVFP4)
    return reinterpret_cast<const uint8_t*>(w.scales) + e * w.stride_scales + (size_t)n * (w.cols / 16);
  else if constexpr (FMT == FMT_MXFP4)
    return reinterpret_cast<const uint8_t*>(w.scales) + e * w.stride_scales + (size_t)n * (w.cols / 32);
  else
    return nullptr;
}

__device__ __forceinline__ float fp8_block_scale(const WDesc& w, int e, int n0, int c) {
  const int cb = (w.cols + 127) / 128;
  const float* s = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(w.scales) +
                                                  e * w.stride_scales);
  return s[(n0 / 128) * cb + c];
}

// WN waves along N (16 rows each) x WK waves along K per block.
template <int FMT, int OP, int WN, int WK>
__global__ __launch_bounds__(64 * WN * WK) void expert_gemv_kernel(GemvParams p) {
  constexpr int NT = (OP == kOpGateUp) ? 2 : 1;  // weight tiles per wave
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wn = wave / WK, wk = wave % WK;
  const GroupArgs& G = p.grp;
  const int u = blockIdx.y;
  int e, p0, nrows;
  if (G.shared) {
    e = 0;
    p0 = 0;
    nrows = G.T;
  } else {
    if (u >= *G.n_act) return;
    e = G.act[u];
    p0 = G.offsets[e];
    nrows = G.offsets[e + 1] - p0;
  }
  const int N = p.w0.rows, K = p.w0.cols;
  const int n0 = (blockIdx.x * WN + wn) * 16;
  const bool wave_on = n0 < N;  // waves past N only join the barrier
  const int r = lane & 15, g = lane >> 4;
  const int nrow = n0 + r;
  const int rb = row_bytes<FMT>(K);
  const uint8_t* arow[NT];
  const uint8_t* srow[NT];
  const WDesc* wd[NT];
  wd[0] = &p.w0;
  if constexpr (NT == 2) wd[1] = &p.w1;
#pragma unroll
  for (int q = 0; q < NT; ++q) {
    arow[q] = (wave_on && nrow < N) ? wd[q]->codes + e * wd[q]->stride_codes + (size_t)nrow * rb
                                    : nullptr;
    srow[q] = (wave_on && nrow < N) ? scale_row_ptr<FMT>(*wd[q], e, nrow) : nullptr;
  }
  const int nch = (K + 127) / 128;
  __shared__ f32x4 red[WN * WK][NT][64];

  for (int pass = 0; pass < nrows; pass += 16) {
    // B operand: group row `pass + r` of this pass
    const int grow = pass + r;
    const uint16_t* brow = nullptr;
    if (grow < nrows) {
      int in_row;
      if (G.shared)
        in_row = grow;
      else if (OP == kOpGateUp)
        in_row = G.perm_to_pair[p0 + grow] / G.topk;
      else
        in_row = p0 + grow;
      brow = p.in + (size_t)in_row * K;
    }
    f32x4 acc[NT];
#pragma unroll
    for (int q = 0; q < NT; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (wave_on) {
      constexpr int D = 4;  // chunks in flight per wave
      for (int cb = wk; cb < nch; cb += WK * D) {
        ARaw<FMT> ar[D][NT];
#pragma unroll
        for (int d = 0; d < D; ++d) {
          const int c = cb + d * WK;
#pragma unroll
          for (int q = 0; q < NT; ++q)
            ar[d][q] = load_a<FMT>(c < nch ? arow[q] : nullptr, srow[q], c, g, K);
        }
#pragma unroll
        for (int d = 0; d < D; ++d) {
          const int c = cb + d * WK;
          if (c >= nch) break;
          const int kb = 128 * c + 32 * g;
          const bf16x8 b0 = load_b(brow, kb, K);
          const bf16x8 b1 = load_b(brow, kb + 8, K);
          const bf16x8 b2 = load_b(brow, kb + 16, K);
          const bf16x8 b3 = load_b(brow, kb + 24, K);
#pragma unroll
          for (int q = 0; q < NT; ++q) {
            f32x4 t = (FMT == FMT_FP8) ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[q];
            t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_a<FMT, 0>(ar[d][q]), b0, t, 0, 0, 0);
            t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_a<FMT, 1>(ar[d][q]), b1, t, 0, 0, 0);
            t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_a<FMT, 2>(ar[d][q]), b2, t, 0, 0, 0);
            t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(decode_a<FMT, 3>(ar[d][q]), b3, t, 0, 0, 0);
            if constexpr (FMT == FMT_FP8) {
              const float s = fp8_block_scale(*wd[q], e, n0, c);
              acc[q] = acc[q] + s * t;
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
      for (int q = 0; q < NT; ++q) red[wave][q][lane] = acc[q];
      __syncthreads();
      if (wk == 0) {
#pragma unroll
        for (int q = 0; q < NT; ++q) {
          f32x4 s = red[wave][q][lane];
          for (int j = 1; j < WK; ++j) s = s + red[wave + j][q][lane];
          acc[q] = s;
        }
      }
      __syncthreads();
    }

    // Epilogue: lane holds rows n0 + 4*g + (0..3) for group row pass + r.
    if (wk == 0 && wave_on && grow < nrows) {
      const int nb = n0 + 4 * g;
      const int orow = G.shared ? grow : p0 + grow;
      float ts[NT];
#pragma unroll
      for (int q = 0; q < NT; ++q) ts[q] = (FMT == FMT_NVFP4) ? wd[q]->tscale[e] : 1.0f;
      if constexpr (OP == kOpGateUp) {
        uint16_t h[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float gv = acc[0][j] * ts[0];
          const float uv = acc[1][j] * ts[1];
          const float sg = gv / (1.0f + expf(-gv));
          h[j] = f32_to_bf16(sg * uv);
        }
        uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + (size_t)orow * N + nb;
        if (nb + 3 < N) {
          const uint2 v = make_uint2(h[0] | (uint32_t(h[1]) << 16), h[2] | (uint32_t(h[3]) << 16));
          *reinterpret_cast<uint2*>(o) = v;
        } else {
          for (int j = 0; j < 4; ++j)
            if (nb + j < N) o[j] = h[j];
        }
      } else {
        float* o = reinterpret_cast<float*>(p.out) + (size_t)orow * N + nb;
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
hipError_t launch_t(const GemvParams& p, hipStream_t s) {
  const int N = p.w0.rows;
  dim3 grid((N + 16 * WN - 1) / (16 * WN), p.grp.shared ? 1 : p.grp.max_groups);
  return launch(expert_gemv_kernel<FMT, OP, WN, WK>, grid, dim3(64 * WN * WK), 0, s, p);
}

template <int FMT>
hipError_t launch_fmt(int op, const GemvParams& p, hipStream_t s) {
  if (op == kOpGateUp) return launch_t<FMT, kOpGateUp, 1, 4>(p, s);
  return launch_t<FMT, kOpDown, 4, 1>(p, s);
}

}  // namespace

hipError_t launch_expert_gemv(int op, const WDesc& w0, const WDesc& w1, const GroupArgs& g,
                              const uint16_t* in, void* out, hipStream_t s) {
  GemvParams p{w0, w1, g, in, out};
  switch (w0.fmt) {
    case FMT_NVFP4:
      return launch_fmt<FMT_NVFP4>(op, p, s);
    case FMT_MXFP4:
      return launch_fmt<FMT_MXFP4>(op, p, s);
    case FMT_FP8:
      return launch_fmt<FMT_FP8>(op, p, s);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace moe
