// Host-side launchers of the MoE kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_device.cuh"

namespace moe {

// ---- routing --------------------------------------------------------------
// Rows of the router per partial-sum slice and experts per block.
constexpr int kRouterCols = 32;
constexpr int kRouterTokens = 8;
// Batches of at most this many tokens take the sliced router.
constexpr int kRouterSlicedRows = 64;
constexpr int kMaxExperts = 1024;  // top-k keeps up to 16 logits per lane
constexpr int kMaxTopK = 32;

struct RouterPlan {
  int RH;  // router rows per slice
  int RS;  // number of slices
  int CS;  // number of column blocks
};
RouterPlan router_plan(int T, int H, int E);

hipError_t launch_router_logits(const uint16_t* x, const float* wr, int T, int H, int E,
                                const RouterPlan& rp, float* part, float* amax, hipStream_t s);

struct TopkArgs {
  const float* part;  // mode 1: partial logits [RS][T][E]; mode 0: given logits [T][E]
  int RS;
  const float* amax;  // mode 1: [RS][CS][T]
  int CS;
  const float* bias;  // [E] or nullptr (mode 1)
  const uint16_t* x;  // mode 1: activations for the certified recompute
  const float* wr;
  int mode;
  int T, H, E, k, renorm;
  float* logits_out;  // [T][E] or nullptr
  int* ids;           // [T][k]
  float* w;           // [T][k]
  int* recomputed;    // [T] or nullptr
  // mode 1: per-logit error bound = bound_scale * max(amax over blocks, |bias|) + bound_abs
  double bound_scale, bound_abs;
  // One wavefront per token (large T) instead of one block; in mode 1 this
  // needs wrt, the router weights transposed to [E][H], for the recompute.
  int wave;
  const float* wrt;
};
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);

// Router logits on the matrix cores (large T): Wr split into three exact bf16
// planes, fp32 step sums added in float64.  Writes logits [T][E] (no bias)
// and amax [router_mfma_cols(E)][T]; the top-k bound is
// router_mfma_bound_scale(H) times the maximum of amax over blocks.
// planes: [3][E][H] bf16 scratch; wrt: [E][H] fp32 (Wr transposed, written
// for the top-k recompute); wsq: router_mfma_wsq_count(H, E) doubles.
int router_mfma_cols(int E);
size_t router_mfma_wsq_count(int H, int E);
double router_mfma_bound_scale(int H);
hipError_t launch_router_mfma(const uint16_t* x, const float* wr, int T, int H, int E,
                              uint16_t* planes, float* wrt, double* wsq, float* logits,
                              float* amax, hipStream_t s);

// ---- grouping -------------------------------------------------------------
constexpr int kPermChunk = 1024;
struct PermPlan {
  int P, NB;
};
inline PermPlan perm_plan(int T, int k) {
  PermPlan p;
  p.P = T * k;
  p.NB = (p.P + kPermChunk - 1) / kPermChunk;
  return p;
}
// ws: hist [NB][E] int32 (each chunk's rank base within its expert, written in place)
hipError_t launch_permute(const int* ids, int T, int k, int E, int* counts, int* offsets,
                          int* perm_to_pair, int* pair_to_perm, int* hist, int* act,
                          int* n_act, int tile_m, int* tiles, int* n_tiles, int max_tiles,
                          hipStream_t s);
// Active-expert list (and tile list) from offsets only.
hipError_t launch_groups_from_offsets(const int* offsets, int E, int* act, int* n_act, int tile_m,
                                      int* tiles, int* n_tiles, int max_tiles, hipStream_t s);

// ---- experts ----------------------------------------------------------------
struct GroupArgs {
  const int* offsets;       // [E+1] (routed)
  const int* perm_to_pair;  // routed GATE_UP input-row map
  const int* act;           // active expert ids
  const int* n_act;
  int topk;
  int shared;  // 1: single expert over rows 0..T-1
  int T;
  int E;
  int max_groups;  // grid bound on active experts
};
// Expert GEMV over chunks of at most kGemvChunk rows: routed chunks come from
// the tile list of launch_permute / launch_groups_from_offsets built with
// tile_m = kGemvChunk (int2 (expert, first permuted row)), or, with tiles ==
// nullptr, one block row per active expert of g.act / g.n_act takes the
// whole group; the shared expert (g.shared) is cut into chunks of its T rows.
constexpr int kGemvChunk = 16;
hipError_t launch_expert_gemv(int op, const WDesc& w0, const WDesc& w1, const GroupArgs& g,
                              const int* tiles, const int* n_tiles, int max_tiles,
                              const uint16_t* in, void* out, hipStream_t s);
// Tiled grouped GEMM (row groups of any size) over the tile list of
// launch_permute / launch_groups_from_offsets: tiles int2 (expert, first
// permuted row) of kGemmTileM rows.  Shared expert (g.shared): tiles unused.
constexpr int kGemmTileM = 128;
hipError_t launch_grouped_gemm(int op, const WDesc& w0, const WDesc& w1, const GroupArgs& g,
                               const int* tiles, const int* n_tiles, int max_tiles,
                               const uint16_t* in, void* out, hipStream_t s);
// The same GEMM for FP4 experts (NVFP4, MXFP4) with
// K % 64 == 0, output rows a multiple of 8 (gate/up) or 4 (down) and aligned
// codes, scale words and activations (`in` 16-byte aligned): operands moved by
// LDS-DMA, weight fragments decoded per wavefront, the output tile stored
// through LDS (launch_grouped_gemm takes it when it fits; in_rows: the rows of
// `in`, whose bytes and one expert's codes must stay below 2 GiB).
bool grouped_gemm_dma_fits(int op, const WDesc& w0, const WDesc& w1, int in_rows);
hipError_t launch_grouped_gemm_dma(int op, const WDesc& w0, const WDesc& w1, const GroupArgs& g,
                                   const int* tiles, const int* n_tiles, int max_tiles,
                                   const uint16_t* in, void* out, hipStream_t s);

// ---- opt-in lossy activation modes -----------------------------------------
// Quantize bf16 rows [rows][K] (K % 32 == 0) for mode kActMxfp8 / kActMxfp4 /
// kActT128: codes [rows][K] (E4M3) or [rows][K/2] (E2M1, even K in the low
// nibble); scales MX: uint8 E8M0 [rows][act_scale_pitch(K)] (entries past K/32
// are 127), T128: fp32 [rows][ceil(K/128)].
inline int act_scale_pitch(int K) { return 4 * ((K + 127) / 128); }
hipError_t launch_quantize_act(int mode, const uint16_t* in, int rows, int K, uint8_t* codes,
                               void* scales, hipStream_t s);
// Grouped GEMM on the scaled matrix cores over quantized inputs (codes and
// scales laid out as launch_quantize_act writes them).  Weight format: MXFP4
// for the MX modes, FP8 block-128 for kActT128.  Same tiles, rows and outputs
// as launch_grouped_gemm.
hipError_t launch_grouped_gemm_q(int mode, int op, const WDesc& w0, const WDesc& w1,
                                 const GroupArgs& g, const int* tiles, const int* n_tiles,
                                 int max_tiles, const uint8_t* in_codes, const void* in_scales,
                                 void* out, hipStream_t s);

// ---- fused decode lowering (T <= 8; up to 32 on aligned shapes) -------------
struct DecodePlan {
  int RS, CS, down_tiles;
};
DecodePlan decode_plan(int T, int H, int E);

struct DecodeArgs {
  const uint16_t* x;
  int T, H, I, E, k, renorm, I_shared, has_shared, max_groups;
  const float* wr;
  const float* bias;
  WDesc gate, up, down, sg, su, sd;
  int RS, CS;
  // workspace
  double* part;       // [RS][T][E] slice sums of x.Wr: fp32 (T <= 8) or fp64 (T > 8)
  float* apart;       // [RS][T][E] fp32 slice sums of |x||Wr|
  float* logits_out;  // [T][E] debug copy or nullptr
  int* ids;           // [T][k]
  float* w;           // [T][k]
  uint16_t* h;        // [T*k][I], row = pair t*k+j
  uint16_t* hs;       // [T][I_shared]
  uint16_t* out;      // [T][H]
  int dc_stage_k;     // down-combine launch: input rows staged in LDS, per-wave row length (0: not)
  float* y;           // [T*k][H] fp32 partials (row = pair t*k+j) for the per-expert down, or nullptr
  float* ys;          // [T][H] fp32 shared expert's down output, or nullptr
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
// Rows the decode lowering takes: every T <= 8, and 9..32 (T*k <= 512) when
// every launch has its aligned (lean) tile for these weights (the layer then
// sets a.y / a.ys, which the per-expert down needs).
constexpr int kDecodeMaxRows = 32;
bool decode_rows_ok(const DecodeArgs& a);
// Routing alone with the decode router (128-row slices, token groups of 8)
// and the decode top-k, for batches up to kRouterSlicedRows tokens: reads x,
// wr, bias; writes part/apart (workspace), logits_out (optional), ids, w.
hipError_t launch_decode_route(const DecodeArgs& a, hipStream_t s);
// The fused decode's expert launches alone (gate/up + SwiGLU, down + combine)
// on the routing in a.ids / a.w.
hipError_t launch_decode_experts(const DecodeArgs& a, hipStream_t s);
// Its first launch alone: routed gate/up + SwiGLU into a.h (row t*k+j) and
// the shared expert's into a.hs, on the routing in a.ids.
hipError_t launch_decode_gate_up(const DecodeArgs& a, hipStream_t s);
// Token-table routing on given logits [T][E] (k <= 64).
hipError_t launch_table_route(const int* tok, const int* table, int V, int T, int k, int E,
                              const float* logits, int renorm, int* ids, float* w, hipStream_t s);

// ---- combine ----------------------------------------------------------------
// pair_to_perm nullptr: y rows are in pair order (row t*k+j).
hipError_t launch_combine(const float* y, const float* w, const int* pair_to_perm, const float* ys,
                          int T, int k, int H, uint16_t* out, hipStream_t s);

}  // namespace moe
