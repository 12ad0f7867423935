// Activation quantizers of the opt-in lossy GEMM modes.
//
// The pages' activation-quantizing levers (NVFP4 W4A4 prefill, gated behind
// an opt-in switch: forum thread "DGPP: a GB10-optimized C++/CUDA inference
// engine", page 5, update post; the FP8 prefill GEMM with per-token 1x128
// E4M3 activations: gitee "dgpp" README, "Execution and performance",
// engine.prefill_fp8_gemm) give no arithmetic.  The conversions here are:
//
// * MX (E4M3 or E2M1 elements, E8M0 scale per 32 consecutive K): the OCP
//   Microscaling Formats v1.0 conversion of a scalar block.  shared exponent
//   = floor(log2 amax) - emax(element) clamped to [-127, 127], elements
//   RNE(clamp(v / 2^shared)).  All-zero block: scale code 0; a non-finite
//   value: scale 0xFF and zero codes.
// * per-token 1x128 (E4M3 elements, fp32 scale per 128 K):
//   s = max(amax, 2^-64) / 448 and e = RNE(clamp(v / s, +-448)), both
//   divisions IEEE fp32; a non-finite value gives s = NaN and zero codes.
//
// One thread converts 32 consecutive elements; the 4 threads of one 128-wide
// block are adjacent lanes (rows are padded to whole 128-blocks of threads),
// so the 1x128 amax is a 4-lane reduction.  Element rounding is done on the
// fp32 bit pattern (the value grid's quantum follows the exponent field).
#include "moe_device.cuh"
#include "moe_launch.h"

namespace moe {
namespace {

// |q| <= 448, finite.  Sign from the fp32 sign bit (so -0 and negative values
// that round to zero give 0x80).
__device__ __forceinline__ uint32_t e4m3_rne(float q) {
  uint32_t u = __float_as_uint(q);
  const uint32_t sgn = (u >> 24) & 0x80u;
  u &= 0x7fffffffu;
  uint32_t c;
  if (__uint_as_float(u) < 0x1p-6f) {
    // subnormal quantum 2^-9; a result of 8 is the smallest normal (code 8)
    c = static_cast<uint32_t>(__builtin_rintf(__uint_as_float(u) * 512.0f));
  } else {
    u += 0x7ffffu + ((u >> 20) & 1u);  // keep 3 mantissa bits, ties to even
    c = (((u >> 23) - 120u) << 3) | ((u >> 20) & 7u);
  }
  return c | sgn;
}

// |q| <= 6, finite.
__device__ __forceinline__ uint32_t e2m1_rne(float q) {
  uint32_t u = __float_as_uint(q);
  const uint32_t sgn = (u >> 28) & 0x8u;
  u &= 0x7fffffffu;
  uint32_t c;
  if (__uint_as_float(u) < 1.0f) {
    c = static_cast<uint32_t>(__builtin_rintf(__uint_as_float(u) * 2.0f));  // 0, 0.5, 1.0
  } else {
    u += 0x1fffffu + ((u >> 22) & 1u);  // keep 1 mantissa bit, ties to even
    c = (((u >> 23) - 126u) << 1) | ((u >> 22) & 1u);
  }
  return c | sgn;
}

struct QuantArgs {
  const uint16_t* in;  // bf16 [rows][K]
  int rows, K;
  int nb;              // 128-blocks per row: ceil(K / 128)
  uint8_t* codes;      // [rows][K] (E4M3) or [rows][K/2] (E2M1)
  void* scales;        // MX: uint8 [rows][4*nb]; T128: fp32 [rows][nb]
};

template <int MODE>
__global__ __launch_bounds__(256) void quantize_kernel(QuantArgs a) {
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int per_row = 4 * a.nb;
  const long long row = t / per_row;
  const int c = static_cast<int>(t % per_row);  // 32-chunk of the row
  // Every thread of the launch reaches the 4-lane reduction below; threads
  // past the last row or K only contribute zeros and store nothing.
  const bool live = row < a.rows && 32 * c < a.K;
  float v[32];
  float amax = 0.f;
  bool finite = true;
  if (live) {
    const u32x4* src = reinterpret_cast<const u32x4*>(a.in + row * a.K + 32 * c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 w = src[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
        v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
      }
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float m = fabsf(v[i]);
      finite = finite && (m <= 0x1.fffffep127f);  // false for inf and NaN
      amax = fmaxf(amax, finite ? m : 0.f);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = 0.f;
  }

  if constexpr (MODE == kActT128) {
    // 1x128 block = 4 adjacent lanes
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    int fin = finite ? 1 : 0;
    fin &= __shfl_xor(fin, 1);
    fin &= __shfl_xor(fin, 2);
    if (!live) return;
    const float s = fmaxf(amax, 0x1p-64f) / 448.0f;
    uint32_t out[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t w = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float q = fminf(fmaxf(v[4 * i + j] / s, -448.0f), 448.0f);
        w |= (fin ? e4m3_rne(q) : 0u) << (8 * j);
      }
      out[i] = w;
    }
    u32x4* dst = reinterpret_cast<u32x4*>(a.codes + row * a.K + 32 * c);
    dst[0] = u32x4{out[0], out[1], out[2], out[3]};
    dst[1] = u32x4{out[4], out[5], out[6], out[7]};
    if ((c & 3) == 0)
      reinterpret_cast<float*>(a.scales)[row * a.nb + c / 4] =
          fin ? s : __uint_as_float(0x7fc00000u);
  } else {
    if (row >= a.rows) return;
    uint8_t* srow = reinterpret_cast<uint8_t*>(a.scales) + row * per_row;
    if (!live) {  // padding chunk of the last 128-block: unit scale
      srow[c] = 127;
      return;
    }
    constexpr int emax = (MODE == kActMxfp8) ? 8 : 2;
    constexpr float qmax = (MODE == kActMxfp8) ? 448.0f : 6.0f;
    // floor(log2 amax) from the exponent field; a zero or subnormal amax
    // lands below the E8M0 range and clamps to -127.
    const int ef = static_cast<int>(__float_as_uint(amax) >> 23);
    const int shared = (ef == 0) ? -127 : max(ef - 127 - emax, -127);
    const float inv = __uint_as_float(static_cast<uint32_t>(127 - shared) << 23);  // 2^-shared
    uint32_t code[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float q = fminf(fmaxf(v[i] * inv, -qmax), qmax);
      code[i] = finite ? ((MODE == kActMxfp8) ? e4m3_rne(q) : e2m1_rne(q)) : 0u;
    }
    if constexpr (MODE == kActMxfp8) {
      uint32_t out[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        out[i] = code[4 * i] | (code[4 * i + 1] << 8) | (code[4 * i + 2] << 16) |
                 (code[4 * i + 3] << 24);
      u32x4* dst = reinterpret_cast<u32x4*>(a.codes + row * a.K + 32 * c);
      dst[0] = u32x4{out[0], out[1], out[2], out[3]};
      dst[1] = u32x4{out[4], out[5], out[6], out[7]};
    } else {
      uint32_t out[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t w = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) w |= code[8 * i + j] << (4 * j);  // even K in the low nibble
        out[i] = w;
      }
      *reinterpret_cast<u32x4*>(a.codes + row * (a.K / 2) + 16 * c) =
          u32x4{out[0], out[1], out[2], out[3]};
    }
    srow[c] = finite ? static_cast<uint8_t>(shared + 127) : 0xFF;
  }
}

}  // namespace

hipError_t launch_quantize_act(int mode, const uint16_t* in, int rows, int K, uint8_t* codes,
                               void* scales, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  QuantArgs a;
  a.in = in;
  a.rows = rows;
  a.K = K;
  a.nb = (K + 127) / 128;
  a.codes = codes;
  a.scales = scales;
  const long long threads = (long long)rows * 4 * a.nb;
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
  switch (mode) {
    case kActMxfp8: return launch(quantize_kernel<kActMxfp8>, grid, dim3(256), 0, s, a);
    case kActMxfp4: return launch(quantize_kernel<kActMxfp4>, grid, dim3(256), 0, s, a);
    case kActT128: return launch(quantize_kernel<kActT128>, grid, dim3(256), 0, s, a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
