// Standalone expert GEMV launch (the moe_expert_gemm entry point for small
// row groups).  The kernel body lives in gemv_core.cuh and is shared with
// the fused decode kernels.
#include "gemv_core.cuh"

namespace moe {
namespace {

struct GemvKParams {
  WDesc w0, w1;
  GroupArgs grp;
  const int2* tiles;  // routed: (expert, first permuted row) per chunk of kGemvChunk rows,
  const int* n_tiles; // or nullptr: one block row per active expert (grp.act / grp.n_act)
  int max_tiles;
  const uint16_t* in;
  void* out;
};

// With a chunk list, each block computes one chunk of at most kGemvChunk rows
// (one 16-row pass) of one expert: the chunks of a large group run in
// parallel blocks, and the weights of its later chunks come from L2.
// Without one (a caller-supplied active-expert list), each block takes a
// whole group in consecutive passes.
template <int FMT, int OP>
__global__ __launch_bounds__(512) void expert_gemv_kernel(GemvKParams p) {
  constexpr int WN = GemvShape<OP>::WN, WK = GemvShape<OP>::WK;
  __shared__ GemvSmem<WN, WK, (OP == kOpGateUp) ? 2 : 1> sm;
  const GroupArgs& G = p.grp;
  GemvRows gr;
  gr.rows_in = gr.rows_out = nullptr;
  const int u = blockIdx.y;
  if (G.shared) {
    gr.e = 0;
    gr.p0 = u * kGemvChunk;
    gr.nrows = min(kGemvChunk, G.T - gr.p0);
    if (gr.nrows <= 0) return;
  } else if (p.tiles != nullptr) {
    // both loads issued before either is used
    const int nt = *p.n_tiles;
    const int2 tl = p.tiles[u < p.max_tiles ? u : 0];
    if (u >= min(nt, p.max_tiles)) return;
    const int P = G.T * G.topk;
    gr.e = tl.x;
    if ((unsigned)gr.e >= (unsigned)G.E) return;
    gr.p0 = tl.y;
    const int end = G.offsets[gr.e + 1];
    gr.nrows = min(kGemvChunk, end - gr.p0);
    if (gr.p0 < 0 || gr.nrows <= 0 || end > P) return;
  } else {
    // both loads issued before either is used (act holds max_groups >= gridDim.y entries)
    const int na = *G.n_act;
    gr.e = G.act[u];
    if (u >= na) return;
    const int P = G.T * G.topk;
    if ((unsigned)gr.e >= (unsigned)G.E) return;
    gr.p0 = G.offsets[gr.e];
    gr.nrows = G.offsets[gr.e + 1] - gr.p0;
    if (gr.p0 < 0 || gr.nrows < 0 || gr.p0 + gr.nrows > P) return;
  }
  const int in_rows = G.shared ? G.T : (OP == kOpGateUp ? G.T : G.T * G.topk);
  const int mode = G.shared ? kInDirect : (OP == kOpGateUp ? kInPerm : kInDirect);
  GemvIO io{p.in, p.out, G.perm_to_pair, G.topk, mode, in_rows};
  gemv_tile<FMT, OP, WN, WK>(p.w0, p.w1, io, gr, blockIdx.x, sm);
}

template <int FMT, int OP>
hipError_t launch_t(const GemvKParams& p, hipStream_t s) {
  constexpr int RPB = gemv_rows_per_block<OP>();
  const int chunks = p.grp.shared ? (p.grp.T + kGemvChunk - 1) / kGemvChunk
                     : (p.tiles != nullptr ? p.max_tiles : p.grp.max_groups);
  if (chunks <= 0) return hipSuccess;
  dim3 grid((p.w0.rows + RPB - 1) / RPB, chunks);
  constexpr int threads = kWave * GemvShape<OP>::WN * GemvShape<OP>::WK;
  return launch(expert_gemv_kernel<FMT, OP>, grid, dim3(threads), 0, s, p);
}

template <int FMT>
hipError_t launch_fmt(int op, const GemvKParams& p, hipStream_t s) {
  return op == kOpGateUp ? launch_t<FMT, kOpGateUp>(p, s) : launch_t<FMT, kOpDown>(p, s);
}

}  // namespace

hipError_t launch_expert_gemv(int op, const WDesc& w0, const WDesc& w1, const GroupArgs& g,
                              const int* tiles, const int* n_tiles, int max_tiles,
                              const uint16_t* in, void* out, hipStream_t s) {
  GemvKParams p{w0, w1, g, reinterpret_cast<const int2*>(tiles), n_tiles, max_tiles, in, out};
  switch (w0.fmt) {
    case FMT_NVFP4: return launch_fmt<FMT_NVFP4>(op, p, s);
    case FMT_MXFP4: return launch_fmt<FMT_MXFP4>(op, p, s);
    case FMT_FP8: return launch_fmt<FMT_FP8>(op, p, s);
    case FMT_MXFP8: return launch_fmt<FMT_MXFP8>(op, p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
