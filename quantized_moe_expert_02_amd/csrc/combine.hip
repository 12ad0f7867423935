// Weighted combine of the per-expert partials.
//
// The default chain keeps expert partial sums in fp32; summing them from bf16
// is an explicit lossy lever (gitee "dgpp" README, "Execution and
// performance", engine.prefill_bf16_partials).  Each output element sums its
// k partials in slot order, then the shared expert, then rounds once to bf16:
// a fixed order, so the result does not depend on scheduling.
#include "moe_launch.h"

namespace moe {
namespace {

// PAIR: y rows in pair order (row t*k+j, the decode lowering): the rows'
// addresses need no load, so the weights and y go out in one round trip.
template <bool PAIR>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const float* __restrict__ w,
                                                      const int* __restrict__ p2p,
                                                      const float* __restrict__ ys, int T, int k,
                                                      int H, uint16_t* __restrict__ out) {
  const int t = blockIdx.y;
  const int n = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (n >= H) return;
  // All slots of a batch of 16 (every slot for k <= 16) in two round trips:
  // the slots' rows and weights, then their y; the sum stays in slot order.
  constexpr int B = 16;
  // the shared expert's row, loaded with the first batch (added last)
  const f32x4 yv = (ys != nullptr) ? *reinterpret_cast<const f32x4*>(ys + (size_t)t * H + n)
                                   : f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < k; j0 += B) {
    int pp[B];
    float wj[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      pp[b] = -1;
      wj[b] = 0.f;
      if (j0 + b < k) {  // wave-uniform
        pp[b] = PAIR ? t * k + j0 + b : p2p[(size_t)t * k + j0 + b];
        wj[b] = w[(size_t)t * k + j0 + b];
      }
    }
    // y is read once: non-temporal loads keep it from displacing cached
    // lines (measured on the 8192-token layer: 171 -> 124 us)
    f32x4 v[B];
#pragma unroll
    for (int b = 0; b < B; ++b)  // a dropped pair (pair_to_perm -1) contributes nothing
      v[b] = (pp[b] >= 0) ? __builtin_nontemporal_load(
                                reinterpret_cast<const f32x4*>(y + (size_t)pp[b] * H + n))
                          : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < B; ++b) {
      if (j0 + b < k) {
        const float wb = (pp[b] >= 0) ? wj[b] : 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] = fmaf(wb, v[b][q], acc[q]);
      }
    }
  }
  if (ys != nullptr) acc = acc + yv;
  const uint2 o = make_uint2(f32_to_bf16(acc[0]) | (uint32_t(f32_to_bf16(acc[1])) << 16),
                             f32_to_bf16(acc[2]) | (uint32_t(f32_to_bf16(acc[3])) << 16));
  *reinterpret_cast<uint2*>(out + (size_t)t * H + n) = o;
}

}  // namespace

hipError_t launch_combine(const float* y, const float* w, const int* pair_to_perm, const float* ys,
                          int T, int k, int H, uint16_t* out, hipStream_t s) {
  dim3 grid((H / 4 + 255) / 256, T);
  if (pair_to_perm == nullptr)
    return launch(combine_kernel<true>, grid, dim3(256), 0, s, y, w, pair_to_perm, ys, T, k, H, out);
  return launch(combine_kernel<false>, grid, dim3(256), 0, s, y, w, pair_to_perm, ys, T, k, H, out);
}

}  // namespace moe
