// Device-side helpers shared by the gfx950 kernels of the MoE layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

enum : int { FMT_NVFP4 = 1, FMT_MXFP4 = 2, FMT_FP8 = 3, FMT_MXFP8 = 4 };

// Formats whose codes are one byte per weight (E4M3).
constexpr bool fmt_is_fp8(int f) { return f == FMT_FP8 || f == FMT_MXFP8; }

// Activation modes of the expert GEMMs: the exact chain (bf16 inputs) and the
// opt-in lossy ones (inputs quantized per row: MX E4M3 or E2M1 with an E8M0
// scale per 32 K; E4M3 with an fp32 scale per 128 K).
enum : int { kActExact = 0, kActMxfp8 = 1, kActMxfp4 = 2, kActT128 = 3 };
typedef int i32x8 __attribute__((ext_vector_type(8)));

// One projection of E stacked experts as the kernels see it.
struct WDesc {
  int fmt;  // FMT_*
  const uint8_t* codes;
  const void* scales;
  const float* tscale;  // NVFP4 per-expert tensor scale, else nullptr
  long long stride_codes;   // bytes between experts
  long long stride_scales;  // bytes between experts
  int rows, cols;
  // NVFP4 / MXFP4 / MXFP8: cols % 128 == 0 and every scale row starts
  // 8-byte (NVFP4) or 4-byte (MX) aligned, so the block scales of a 128-wide
  // K chunk of a row are one aligned word.
  int wide;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// SiLU for the SwiGLU epilogues: g * sigmoid(g) with the hardware exp and
// reciprocal (a few fp32 ulps, far below the bf16 rounding of h that
// follows).  g = -inf gives NaN, +inf gives +inf, as g / (1 + exp(-g)) does.
__device__ __forceinline__ float silu_fast(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// Pack the upper halves of two floats that are exactly bf16-representable.
__device__ __forceinline__ uint32_t pack_hi16(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// Two E4M3 bytes (low 16 bits of w) -> two floats, via the gfx950 converter.
__device__ __forceinline__ f32x2 e4m3x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
}

// Wave-wide helpers --------------------------------------------------------
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ double shfl_xor_d(double v, int m) {
  return __shfl_xor(v, m, kWave);
}

__device__ __forceinline__ float wave_sum_f(float v) {
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ float wave_max_f(float v) {
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

// Order of a grouped GEMM's (row tile, column tile) pairs.  The row tiles of
// one expert are cut into runs of at most `run` consecutive tiles, and a run
// takes every column tile with its row tiles fastest: the run's workgroups
// read each weight column tile together (one HBM fetch per run, not one per
// row tile) while its activation rows stay in L2.  idx in [0, n_rt * ntn)
// maps one to one onto (row tile, column tile) in [0, n_rt) x [0, ntn); run
// 1 is column tiles fastest.  tiles: int2 (expert, first permuted row) in
// expert order, tile_m rows each, as the grouping writes them from offsets;
// nullptr: one expert whose rows are all n_rt tiles.
__device__ inline int2 gemm_tile_order(int idx, int ntn, int n_rt, int run, const int2* tiles,
                                       const int* offsets, int tile_m) {
  const int lin = idx / ntn;  // a row tile of idx's run
  if (run <= 1) return make_int2(lin, idx - lin * ntn);
  int j = lin, R = n_rt;  // lin's place among its expert's tiles, their count
  if (tiles != nullptr) {
    const int2 tl = tiles[lin];
    const int a = offsets[tl.x], b = offsets[tl.x + 1];
    if (tl.y < a || b <= tl.y) return make_int2(lin, idx - lin * ntn);  // not from these offsets
    j = (tl.y - a) / tile_m;
    R = (b - a + tile_m - 1) / tile_m;
    if (j > lin) return make_int2(lin, idx - lin * ntn);
  }
  const int c = j / run;
  const int start = lin - j + c * run;
  const int size = min(min(run, R - c * run), n_rt - start);
  const int rem = idx - start * ntn;
  return make_int2(start + rem % size, rem / size);
}

// Launch a kernel and return the status of this launch alone (not the
// thread's sticky last-error state, which other libraries may have left set).
template <typename... KArgs, typename... Args, size_t... Is>
hipError_t launch_impl(void (*k)(KArgs...), dim3 grid, dim3 block, size_t shmem, hipStream_t s,
                       std::index_sequence<Is...>, Args&&... args) {
  std::tuple<KArgs...> held(std::forward<Args>(args)...);
  void* argv[] = {static_cast<void*>(&std::get<Is>(held))..., nullptr};
  return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, argv, shmem, s);
}

template <typename... KArgs, typename... Args>
hipError_t launch(void (*k)(KArgs...), dim3 grid, dim3 block, size_t shmem, hipStream_t s,
                  Args&&... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  return launch_impl(k, grid, block, shmem, s, std::index_sequence_for<KArgs...>{},
                     std::forward<Args>(args)...);
}

}  // namespace moe
