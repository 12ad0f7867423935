// The C ABI: host-side validation, workspace planning and launch sequencing.
//
// Bad configuration is rejected before anything runs and never falls back
// silently (gitee "dgpp" README, "Configuration": unknown keys and invalid
// types are rejected; the startup memory plan is checked before allocation).
// Here that means: every descriptor and size is checked on the host, a
// negative status comes back before any launch, and the caller sizes the
// workspace from moe_workspace_size() up front.
#include <algorithm>
#include <cstring>
#include <mutex>

#include "../../include/moe.h"
#include "moe_launch.h"

using namespace moe;

namespace {

// Workspace of moe_layer_forward_noalloc: one array per GPU the library runs
// on, held until the process ends.  Host code never uses the array's name
// as an address (on the host it is a stand-in, not device memory): the
// device address is resolved once per device with hipGetSymbolAddress and
// kept in scratch_addr.
constexpr size_t kNoAllocBytes = size_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int fmt_of(int32_t f) {
  switch (f) {
    case MOE_FMT_NVFP4: return FMT_NVFP4;
    case MOE_FMT_MXFP4: return FMT_MXFP4;
    case MOE_FMT_FP8_B128: return FMT_FP8;
    case MOE_FMT_MXFP8: return FMT_MXFP8;
    default: return 0;
  }
}

size_t codes_bytes(const moe_qweight& q) {
  const size_t rb = (q.format == MOE_FMT_FP8_B128 || q.format == MOE_FMT_MXFP8)
                        ? (size_t)q.cols : (size_t)q.cols / 2;
  return rb * q.rows;
}
size_t scales_bytes(const moe_qweight& q) {
  switch (q.format) {
    case MOE_FMT_NVFP4: return (size_t)q.rows * (q.cols / 16);
    case MOE_FMT_MXFP4:
    case MOE_FMT_MXFP8: return (size_t)q.rows * (q.cols / 32);
    default: return (size_t)((q.rows + 127) / 128) * ((q.cols + 127) / 128) * 4;
  }
}

// One projection: expected shape [E][rows][cols].
int32_t check_qweight(const moe_qweight& q, int E, int rows, int cols) {
  if (fmt_of(q.format) == 0) return MOE_ERR_UNSUPPORTED;
  if (q.num_experts != E || q.rows != rows || q.cols != cols) return MOE_ERR_INVALID_ARG;
  if (rows <= 0 || cols <= 0) return MOE_ERR_INVALID_ARG;
  if (rows % 16 != 0) return MOE_ERR_UNSUPPORTED;
  if (q.format == MOE_FMT_FP8_B128 ? (cols % 16 != 0) : (cols % 32 != 0)) return MOE_ERR_UNSUPPORTED;
  if (q.codes == nullptr || q.scales == nullptr) return MOE_ERR_INVALID_ARG;
  if ((q.format == MOE_FMT_NVFP4) != (q.tensor_scale != nullptr)) return MOE_ERR_INVALID_ARG;
  if (!aligned(q.codes, 16)) return MOE_ERR_INVALID_ARG;
  const size_t salign = (q.format == MOE_FMT_FP8_B128) ? 4 : (q.format == MOE_FMT_NVFP4 ? 2 : 1);
  if (!aligned(q.scales, salign)) return MOE_ERR_INVALID_ARG;
  if (q.tensor_scale != nullptr && !aligned(q.tensor_scale, 4)) return MOE_ERR_INVALID_ARG;
  if (E > 1) {
    if (q.expert_stride_codes < (int64_t)codes_bytes(q) || q.expert_stride_codes % 16 != 0)
      return MOE_ERR_INVALID_ARG;
    if (q.expert_stride_scales < (int64_t)scales_bytes(q) ||
        q.expert_stride_scales % (int64_t)salign != 0)
      return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

WDesc wdesc(const moe_qweight& q) {
  WDesc w;
  w.fmt = fmt_of(q.format);
  w.codes = q.codes;
  w.scales = q.scales;
  w.tscale = q.tensor_scale;
  w.stride_codes = q.expert_stride_codes;
  w.stride_scales = q.expert_stride_scales;
  w.rows = q.rows;
  w.cols = q.cols;
  const size_t word = (q.format == MOE_FMT_NVFP4)                                  ? 8
                      : (q.format == MOE_FMT_MXFP4 || q.format == MOE_FMT_MXFP8) ? 4
                                                                                 : 0;
  w.wide = word != 0 && q.cols % 128 == 0 && aligned(q.scales, word) &&
           (q.num_experts == 1 || q.expert_stride_scales % (int64_t)word == 0);
  return w;
}

bool act_mode_valid(int32_t m) {
  return m == MOE_ACT_MXFP8 || m == MOE_ACT_MXFP4 || m == MOE_ACT_FP8_T128;
}

// Does lossy mode m quantize the inputs of a projection in weight format f?
bool mode_applies(int32_t m, int32_t f) {
  if (m == MOE_ACT_MXFP8 || m == MOE_ACT_MXFP4) return f == MOE_FMT_MXFP4;
  if (m == MOE_ACT_FP8_T128) return f == MOE_FMT_FP8_B128;
  return false;
}

int act_kernel_mode(int32_t m) {
  return m == MOE_ACT_MXFP8 ? kActMxfp8 : (m == MOE_ACT_MXFP4 ? kActMxfp4 : kActT128);
}

int32_t check_layer(const moe_layer_desc* L) {
  if (L == nullptr) return MOE_ERR_INVALID_ARG;
  if (L->H <= 0 || L->I <= 0 || L->E <= 0 || L->top_k <= 0) return MOE_ERR_INVALID_ARG;
  if (L->top_k > L->E) return MOE_ERR_INVALID_ARG;
  if (L->E > kMaxExperts || L->top_k > kMaxTopK) return MOE_ERR_UNSUPPORTED;
  if (L->renormalize != 0 && L->renormalize != 1) return MOE_ERR_INVALID_ARG;
  if (L->router_w == nullptr || !aligned(L->router_w, 4)) return MOE_ERR_INVALID_ARG;
  if (L->router_bias != nullptr && !aligned(L->router_bias, 4)) return MOE_ERR_INVALID_ARG;
  int32_t st;
  if ((st = check_qweight(L->gate, L->E, L->I, L->H)) != MOE_OK) return st;
  if ((st = check_qweight(L->up, L->E, L->I, L->H)) != MOE_OK) return st;
  if ((st = check_qweight(L->down, L->E, L->H, L->I)) != MOE_OK) return st;
  if (L->gate.format != L->up.format) return MOE_ERR_UNSUPPORTED;
  if (L->has_shared != 0 && L->has_shared != 1) return MOE_ERR_INVALID_ARG;
  if (L->has_shared) {
    if (L->I_shared <= 0) return MOE_ERR_INVALID_ARG;
    if ((st = check_qweight(L->sh_gate, 1, L->I_shared, L->H)) != MOE_OK) return st;
    if ((st = check_qweight(L->sh_up, 1, L->I_shared, L->H)) != MOE_OK) return st;
    if ((st = check_qweight(L->sh_down, 1, L->H, L->I_shared)) != MOE_OK) return st;
    if (L->sh_gate.format != L->sh_up.format) return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

// Workspace sections for (L, T).
struct WsPlan {
  RouterPlan rp;
  DecodePlan dp;
  int P, NB, max_tiles, tile_m;  // tile list: chunks of tile_m rows (GEMM tile or GEMV pass)
  size_t part, amax, ids, w, counts, offsets, p2pair, pair2p, hist, act, nact, tiles, ntiles, h,
      hs, y, ys, total;
  // matrix-core router (T > kGemvMaxRows): split router planes and w^2 sums
  bool mfma_router;
  size_t planes, wrt, wsq;
  // decode router (T <= kRouterSlicedRows): slice sums
  size_t dpart, dapart;
  // lossy activation modes (T > kGemvMaxRows): quantized x, h and shared h
  // (codes sized for E4M3, scales 4 bytes per 128 K per row)
  size_t xq, xqs, hq, hqs, hsq, hsqs;
  size_t tlog;
};


constexpr int kTileM = kGemmTileM;  // rows per grouped-GEMM tile
// Calls with at most this many tokens run the expert GEMV lowering: each
// active expert's weights are streamed by its own blocks, in passes of 16
// rows (a token picks an expert at most once, so a group has at most this
// many rows; the passes after the first read the weights from L2); larger
// calls run the tiled grouped GEMM.
constexpr int kGemvMaxRows = 64;
// The matrix-core router's error bound assumes H * 2^-23 << 1.
constexpr int kMfmaRouterMaxH = 1 << 16;

// Row counts the kernels index with 32-bit integers: at most 2^24 (token,
// slot) pairs, and every token-major buffer (T rows of H, I, I_shared or E
// elements) below 2^31 elements.  Larger T is MOE_ERR_UNSUPPORTED.
constexpr int64_t kMaxPairs = int64_t(1) << 24;

bool rows_ok(const moe_layer_desc* L, int T) {
  if (T < 0) return false;
  const int64_t w = std::max({L->H, L->I, L->E, L->has_shared ? L->I_shared : 0});
  return (int64_t)T * L->top_k <= kMaxPairs && (int64_t)T * w < (int64_t(1) << 31);
}

// Only for T with rows_ok (its int products stay in range).
WsPlan plan(const moe_layer_desc* L, int T) {
  WsPlan p;
  const int E = L->E, k = L->top_k;
  p.rp = router_plan(T, L->H, E);
  p.P = T * k;
  p.NB = (p.P + kPermChunk - 1) / kPermChunk;
  p.tile_m = (T > kGemvMaxRows) ? kTileM : kGemvChunk;
  p.max_tiles = p.P / p.tile_m + (p.P < E ? p.P : E) + 1;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes);
    return at;
  };
  p.dp = decode_plan(T, L->H, E);
  p.mfma_router = T > kGemvMaxRows && L->H <= kMfmaRouterMaxH;
  const size_t amax_n = p.mfma_router ? (size_t)router_mfma_cols(E) * T
                                      : (size_t)p.rp.RS * p.rp.CS * T;
  p.part = take((size_t)p.rp.RS * T * E * 4);
  p.amax = take(amax_n * 4);
  p.ids = take((size_t)p.P * 4);
  p.w = take((size_t)p.P * 4);
  p.counts = take((size_t)E * 4);
  p.offsets = take((size_t)(E + 1) * 4);
  p.p2pair = take((size_t)p.P * 4);
  p.pair2p = take((size_t)p.P * 4);
  p.hist = take((size_t)p.NB * E * 4);
  p.nact = take((size_t)(E + 1) * 4);  // [0] = count, then ids
  p.act = p.nact + 4;
  p.tiles = take((size_t)p.max_tiles * 8);
  p.ntiles = take(4);
  p.h = take((size_t)p.P * L->I * 2);
  p.hs = take(L->has_shared ? (size_t)T * L->I_shared * 2 : 0);
  p.y = take((size_t)p.P * L->H * 4);
  p.ys = take(L->has_shared ? (size_t)T * L->H * 4 : 0);
  p.planes = p.wrt = p.wsq = 0;
  if (p.mfma_router) {
    p.planes = take((size_t)3 * E * L->H * 2);
    p.wrt = take((size_t)E * L->H * 4);
    p.wsq = take(router_mfma_wsq_count(L->H, E) * 8);
  }
  p.dpart = p.dapart = 0;
  if (T <= kRouterSlicedRows) {  // decode router slices (fused decode and the sliced router)
    p.dpart = take((size_t)p.dp.RS * T * E * 8);
    p.dapart = take((size_t)p.dp.RS * T * E * 4);
  }
  p.tlog = take((size_t)T * E * 4);  // router logits for token-table routing
  p.xq = p.xqs = p.hq = p.hqs = p.hsq = p.hsqs = 0;
  if (T > kGemvMaxRows) {
    auto sb = [](int K) { return (size_t)act_scale_pitch(K); };
    p.xq = take((size_t)T * L->H);
    p.xqs = take((size_t)T * sb(L->H));
    p.hq = take((size_t)p.P * L->I);
    p.hqs = take((size_t)p.P * sb(L->I));
    if (L->has_shared) {
      p.hsq = take((size_t)T * L->I_shared);
      p.hsqs = take((size_t)T * sb(L->I_shared));
    }
  }
  p.total = o;
  return p;
}

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(reinterpret_cast<char*>(ws) + off);
}

thread_local const char* g_last_error = "";

int32_t hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_error = hipGetErrorString(e);
  return MOE_ERR_HIP;
}

int32_t run_route(const moe_layer_desc* L, const uint16_t* x, float* logits, int T, int* ids,
                  float* w, void* ws, const WsPlan& p, hipStream_t s) {
  TopkArgs a;
  std::memset(&a, 0, sizeof(a));
  a.T = T;
  a.H = L->H;
  a.E = L->E;
  a.k = L->top_k;
  a.renorm = L->renormalize;
  a.ids = ids;
  a.w = w;
  if (x == nullptr) {
    a.mode = 0;
    a.part = logits;
    a.RS = 1;
    a.wave = T > kGemvMaxRows;
  } else if (T <= kRouterSlicedRows) {
    // the decode router (128-row slices of fp64 sums, token groups of 8) and
    // the decode top-k, certified with the per-expert sums of |x||w|
    DecodeArgs d;
    std::memset(&d, 0, sizeof(d));
    d.x = x;
    d.T = T;
    d.H = L->H;
    d.E = L->E;
    d.k = L->top_k;
    d.renorm = L->renormalize;
    d.wr = L->router_w;
    d.bias = L->router_bias;
    d.RS = p.dp.RS;
    d.CS = p.dp.CS;
    d.part = at<double>(ws, p.dpart);
    d.apart = at<float>(ws, p.dapart);
    d.logits_out = logits;
    d.ids = ids;
    d.w = w;
    return hip_status(launch_decode_route(d, s));
  } else {
    a.mode = 1;
    a.part = at<float>(ws, p.part);
    a.amax = at<float>(ws, p.amax);
    if (p.mfma_router) {
      hipError_t e = launch_router_mfma(x, L->router_w, T, L->H, L->E, at<uint16_t>(ws, p.planes),
                                        at<float>(ws, p.wrt), at<double>(ws, p.wsq),
                                        at<float>(ws, p.part), at<float>(ws, p.amax), s);
      if (e != hipSuccess) return hip_status(e);
      a.wave = 1;
      a.wrt = at<float>(ws, p.wrt);
      a.RS = 1;
      a.CS = router_mfma_cols(L->E);
      a.bound_scale = router_mfma_bound_scale(L->H);
    } else {
      // float64 slice sums rounded once to fp32: error <= 2^-23 * sum|x||w|
      hipError_t e = launch_router_logits(x, L->router_w, T, L->H, L->E, p.rp,
                                          at<float>(ws, p.part), at<float>(ws, p.amax), s);
      if (e != hipSuccess) return hip_status(e);
      a.RS = p.rp.RS;
      a.CS = p.rp.CS;
      a.bound_scale = 0x1p-22;
    }
    a.bound_abs = 0.0;
    a.bias = L->router_bias;
    a.x = x;
    a.wr = L->router_w;
    a.logits_out = logits;
  }
  return hip_status(launch_topk(a, s));
}

// tiles_ready: the tile list in ws was written by launch_permute for these
// offsets (moe_layer_forward); otherwise it is rebuilt here when needed.
int32_t run_experts(int op, const moe_layer_desc* L, int shared, const int* offsets,
                    const int* perm_to_pair, const int* active, int T, const uint16_t* in,
                    void* out, void* ws, const WsPlan& p, bool tiles_ready, hipStream_t s) {
  GroupArgs g;
  g.offsets = offsets;
  g.perm_to_pair = perm_to_pair;
  const bool gemm = T > kGemvMaxRows;
  // The GEMV takes a caller's active-expert list as is (a block row per
  // group, no extra launch); otherwise both lowerings use the tile list,
  // built from offsets unless the layer's permute wrote it.
  const bool by_groups = !gemm && !shared && !tiles_ready && active != nullptr;
  const bool groups_ready = shared || tiles_ready || by_groups;
  g.act = by_groups ? active + 1 : nullptr;
  g.n_act = by_groups ? active : nullptr;
  g.topk = L->top_k;
  g.shared = shared;
  g.T = T;
  g.E = L->E;
  g.max_groups = p.P < L->E ? p.P : L->E;
  if (!shared && !groups_ready) {
    hipError_t e = launch_groups_from_offsets(offsets, L->E, at<int>(ws, p.act),
                                              at<int>(ws, p.nact), p.tile_m, at<int>(ws, p.tiles),
                                              at<int>(ws, p.ntiles), p.max_tiles, s);
    if (e != hipSuccess) return hip_status(e);
  }
  WDesc w0, w1;
  if (op == MOE_OP_GATE_UP_SWIGLU) {
    w0 = wdesc(shared ? L->sh_gate : L->gate);
    w1 = wdesc(shared ? L->sh_up : L->up);
  } else {
    w0 = wdesc(shared ? L->sh_down : L->down);
    w1 = w0;
  }
  if (gemm)
    return hip_status(launch_grouped_gemm(op, w0, w1, g, at<int>(ws, p.tiles),
                                          at<int>(ws, p.ntiles), p.max_tiles, in, out, s));
  if (by_groups)
    return hip_status(launch_expert_gemv(op, w0, w1, g, nullptr, nullptr, 0, in, out, s));
  return hip_status(launch_expert_gemv(op, w0, w1, g, at<int>(ws, p.tiles), at<int>(ws, p.ntiles),
                                       p.max_tiles, in, out, s));
}

// The grouped GEMM on quantized inputs (any T).
int32_t run_experts_q(int32_t mode, int op, const moe_layer_desc* L, int shared, const int* offsets,
                      const int* perm_to_pair, const int* active, int T, const uint8_t* codes,
                      const void* scales, void* out, void* ws, const WsPlan& p, bool tiles_ready,
                      hipStream_t s) {
  GroupArgs g;
  g.offsets = offsets;
  g.perm_to_pair = perm_to_pair;
  g.topk = L->top_k;
  g.shared = shared;
  g.T = T;
  g.E = L->E;
  g.max_groups = p.P < L->E ? p.P : L->E;
  g.act = nullptr;
  g.n_act = nullptr;
  // This GEMM always runs on 128-row tiles (a ready tile list exists only on
  // the layer's prefill lowering, where the plan's tiles are 128 rows); the
  // workspace's list holds at least this many entries.
  const int max_tiles = p.P / kTileM + (p.P < L->E ? p.P : L->E) + 1;
  if (!shared && !tiles_ready) {
    hipError_t e = launch_groups_from_offsets(offsets, L->E, at<int>(ws, p.act),
                                              at<int>(ws, p.nact), kTileM, at<int>(ws, p.tiles),
                                              at<int>(ws, p.ntiles), max_tiles, s);
    if (e != hipSuccess) return hip_status(e);
  }
  (void)active;
  WDesc w0, w1;
  if (op == MOE_OP_GATE_UP_SWIGLU) {
    w0 = wdesc(shared ? L->sh_gate : L->gate);
    w1 = wdesc(shared ? L->sh_up : L->up);
  } else {
    w0 = wdesc(shared ? L->sh_down : L->down);
    w1 = w0;
  }
  return hip_status(launch_grouped_gemm_q(act_kernel_mode(mode), op, w0, w1, g,
                                          at<int>(ws, p.tiles), at<int>(ws, p.ntiles),
                                          max_tiles, codes, scales, out, s));
}

// The decode lowering's arguments for (L, T) without its buffers.
DecodeArgs decode_args(const moe_layer_desc* L, const uint16_t* x, int T, const WsPlan& p) {
  DecodeArgs a;
  std::memset(&a, 0, sizeof(a));
  a.x = x;
  a.T = T;
  a.H = L->H;
  a.I = L->I;
  a.E = L->E;
  a.k = L->top_k;
  a.renorm = L->renormalize;
  a.I_shared = L->has_shared ? L->I_shared : 0;
  a.has_shared = L->has_shared;
  a.max_groups = p.P < L->E ? p.P : L->E;
  a.wr = L->router_w;
  a.bias = L->router_bias;
  a.gate = wdesc(L->gate);
  a.up = wdesc(L->up);
  a.down = wdesc(L->down);
  if (L->has_shared) {
    a.sg = wdesc(L->sh_gate);
    a.su = wdesc(L->sh_up);
    a.sd = wdesc(L->sh_down);
  }
  a.RS = p.dp.RS;
  a.CS = p.dp.CS;
  return a;
}

// The layer.  given_ids / given_w: a routing to use instead of the router
// (moe_layer_forward_routed), else nullptr.
int32_t layer_impl(const moe_layer_desc* L, const uint16_t* x, int32_t T, uint16_t* out, void* ws,
                   size_t ws_bytes, int32_t act_mode, float* dbg_logits, int32_t* dbg_ids,
                   float* dbg_w, const int32_t* given_ids, const float* given_w, void* stream) {
  int32_t st = check_layer(L);
  if (st != MOE_OK) return st;
  if (act_mode != MOE_ACT_EXACT) {
    if (!act_mode_valid(act_mode)) return MOE_ERR_INVALID_ARG;
    const bool any = mode_applies(act_mode, L->gate.format) ||
                     mode_applies(act_mode, L->down.format) ||
                     (L->has_shared && (mode_applies(act_mode, L->sh_gate.format) ||
                                        mode_applies(act_mode, L->sh_down.format)));
    if (!any) return MOE_ERR_UNSUPPORTED;
    // the quantizer works on whole 32-element blocks of K
    auto k_ok = [&](const moe_qweight& q) {
      return !mode_applies(act_mode, q.format) || q.cols % 32 == 0;
    };
    if (!k_ok(L->gate) || !k_ok(L->down) ||
        (L->has_shared && (!k_ok(L->sh_gate) || !k_ok(L->sh_down))))
      return MOE_ERR_UNSUPPORTED;
  }
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (!rows_ok(L, T)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (x == nullptr || out == nullptr || !aligned(x, 16) || !aligned(out, 16))
    return MOE_ERR_INVALID_ARG;
  const WsPlan p = plan(L, T);
  if (ws == nullptr || ws_bytes < p.total || !aligned(ws, kAlign)) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool routed = given_ids != nullptr;
  // (the kernels only read a given routing)
  int* ids = routed ? const_cast<int*>(given_ids) : (dbg_ids ? dbg_ids : at<int>(ws, p.ids));
  float* w = routed ? const_cast<float*>(given_w) : (dbg_w ? dbg_w : at<float>(ws, p.w));
  if (T <= kDecodeMaxRows) {
    DecodeArgs a = decode_args(L, x, T, p);
    a.part = at<double>(ws, p.dpart);
    a.apart = at<float>(ws, p.dapart);
    a.logits_out = dbg_logits;
    a.ids = ids;
    a.w = w;
    a.h = at<uint16_t>(ws, p.h);
    a.hs = L->has_shared ? at<uint16_t>(ws, p.hs) : nullptr;
    a.y = at<float>(ws, p.y);
    a.ys = L->has_shared ? at<float>(ws, p.ys) : nullptr;
    a.out = out;
    if (decode_rows_ok(a))  // else the 9-64-row lowering below
      return hip_status(routed ? launch_decode_experts(a, s) : launch_decode(a, s));
  }
  if (!routed && (st = run_route(L, x, dbg_logits, T, ids, w, ws, p, s)) != MOE_OK) return st;
  int* offsets = at<int>(ws, p.offsets);
  int* p2pair = at<int>(ws, p.p2pair);
  int* pair2p = at<int>(ws, p.pair2p);
  if ((st = hip_status(launch_permute(ids, T, L->top_k, L->E, at<int>(ws, p.counts), offsets,
                                      p2pair, pair2p, at<int>(ws, p.hist), at<int>(ws, p.act),
                                      at<int>(ws, p.nact), p.tile_m, at<int>(ws, p.tiles),
                                      at<int>(ws, p.ntiles), p.max_tiles, s))) != MOE_OK)
    return st;
  uint16_t* h = at<uint16_t>(ws, p.h);
  float* y = at<float>(ws, p.y);
  const int* active = at<int>(ws, p.nact);
  // Lossy modes (prefill lowering only): which projections quantize their inputs.
  const bool lossy = act_mode != MOE_ACT_EXACT && T > kGemvMaxRows;
  const bool q_gu = lossy && mode_applies(act_mode, L->gate.format);
  const bool q_d = lossy && mode_applies(act_mode, L->down.format);
  const bool q_sgu = lossy && L->has_shared && mode_applies(act_mode, L->sh_gate.format);
  const bool q_sd = lossy && L->has_shared && mode_applies(act_mode, L->sh_down.format);
  const int km = act_kernel_mode(act_mode);
  uint8_t* xq = at<uint8_t>(ws, p.xq);
  void* xqs = at<void>(ws, p.xqs);
  if ((q_gu || q_sgu) &&
      (st = hip_status(launch_quantize_act(km, x, T, L->H, xq, xqs, s))) != MOE_OK)
    return st;
  st = q_gu ? run_experts_q(act_mode, MOE_OP_GATE_UP_SWIGLU, L, 0, offsets, p2pair, active, T, xq,
                            xqs, h, ws, p, true, s)
            : run_experts(MOE_OP_GATE_UP_SWIGLU, L, 0, offsets, p2pair, active, T, x, h, ws, p,
                          true, s);
  if (st != MOE_OK) return st;
  if (q_d) {
    uint8_t* hq = at<uint8_t>(ws, p.hq);
    void* hqs = at<void>(ws, p.hqs);
    if ((st = hip_status(launch_quantize_act(km, h, p.P, L->I, hq, hqs, s))) != MOE_OK) return st;
    st = run_experts_q(act_mode, MOE_OP_DOWN, L, 0, offsets, p2pair, active, T, hq, hqs, y, ws, p,
                       true, s);
  } else {
    st = run_experts(MOE_OP_DOWN, L, 0, offsets, p2pair, active, T, h, y, ws, p, true, s);
  }
  if (st != MOE_OK) return st;
  float* ys = nullptr;
  if (L->has_shared) {
    uint16_t* hs = at<uint16_t>(ws, p.hs);
    ys = at<float>(ws, p.ys);
    st = q_sgu ? run_experts_q(act_mode, MOE_OP_GATE_UP_SWIGLU, L, 1, nullptr, nullptr, nullptr, T,
                               xq, xqs, hs, ws, p, true, s)
               : run_experts(MOE_OP_GATE_UP_SWIGLU, L, 1, nullptr, nullptr, nullptr, T, x, hs, ws,
                             p, true, s);
    if (st != MOE_OK) return st;
    if (q_sd) {
      uint8_t* hsq = at<uint8_t>(ws, p.hsq);
      void* hsqs = at<void>(ws, p.hsqs);
      if ((st = hip_status(launch_quantize_act(km, hs, T, L->I_shared, hsq, hsqs, s))) != MOE_OK)
        return st;
      st = run_experts_q(act_mode, MOE_OP_DOWN, L, 1, nullptr, nullptr, nullptr, T, hsq, hsqs, ys,
                         ws, p, true, s);
    } else {
      st = run_experts(MOE_OP_DOWN, L, 1, nullptr, nullptr, nullptr, T, hs, ys, ws, p, true, s);
    }
    if (st != MOE_OK) return st;
  }
  return hip_status(launch_combine(y, w, pair2p, ys, T, L->top_k, L->H, out, s));
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_last_error(void) { return g_last_error; }

const char* moe_status_string(int32_t status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or format";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int32_t moe_validate_layer(const moe_layer_desc* L) { return check_layer(L); }

size_t moe_workspace_size(const moe_layer_desc* L, int32_t T) {
  if (check_layer(L) != MOE_OK || !rows_ok(L, T)) return 0;
  if (T == 0) return kAlign;
  return plan(L, T).total;
}

int32_t moe_route_topk(const moe_layer_desc* L, const uint16_t* x, float* logits, int32_t T,
                       int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes, void* stream) {
  int32_t st = check_layer(L);
  if (st != MOE_OK) return st;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (!rows_ok(L, T)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (logits == nullptr || topk_ids == nullptr || topk_w == nullptr) return MOE_ERR_INVALID_ARG;
  if (x != nullptr && (!aligned(x, 16) || L->H % 8 != 0)) return MOE_ERR_INVALID_ARG;
  const WsPlan p = plan(L, T);
  if (x != nullptr && (ws == nullptr || ws_bytes < p.total || !aligned(ws, kAlign)))
    return MOE_ERR_WORKSPACE;
  return run_route(L, x, logits, T, topk_ids, topk_w, ws, p, static_cast<hipStream_t>(stream));
}

size_t moe_permute_workspace_size(int32_t T, int32_t k, int32_t E) {
  if (T < 0 || k <= 0 || E <= 0 || E > kMaxExperts) return 0;
  if ((int64_t)T * k > kMaxPairs) return 0;
  const PermPlan pp = perm_plan(T, k);
  return align_up((size_t)pp.NB * E * 4) + align_up((size_t)(E + 1) * 4);
}

int32_t moe_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E, int32_t* counts,
                    int32_t* offsets, int32_t* perm_to_pair, int32_t* pair_to_perm,
                    int32_t* active_experts, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || k <= 0 || E <= 0 || k > E) return MOE_ERR_INVALID_ARG;
  if (E > kMaxExperts || (int64_t)T * k > kMaxPairs) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!topk_ids || !counts || !offsets || !perm_to_pair || !pair_to_perm) return MOE_ERR_INVALID_ARG;
  const size_t need = moe_permute_workspace_size(T, k, E);
  if (ws == nullptr || ws_bytes < need || !aligned(ws, kAlign)) return MOE_ERR_WORKSPACE;
  const PermPlan pp = perm_plan(T, k);
  int* hist = at<int>(ws, 0);
  int* active = active_experts ? active_experts : at<int>(ws, align_up((size_t)pp.NB * E * 4));
  return hip_status(launch_permute(topk_ids, T, k, E, counts, offsets, perm_to_pair, pair_to_perm,
                                   hist, active + 1, active, kTileM, nullptr, nullptr, 0,
                                   static_cast<hipStream_t>(stream)));
}

int32_t moe_expert_gemm(int32_t op, const moe_layer_desc* L, int32_t shared,
                        const int32_t* offsets, const int32_t* perm_to_pair,
                        const int32_t* active_experts, int32_t T, const uint16_t* in, void* out,
                        void* ws, size_t ws_bytes, void* stream) {
  int32_t st = check_layer(L);
  if (st != MOE_OK) return st;
  if (op != MOE_OP_GATE_UP_SWIGLU && op != MOE_OP_DOWN) return MOE_ERR_INVALID_ARG;
  if (shared != 0 && shared != 1) return MOE_ERR_INVALID_ARG;
  if (shared && !L->has_shared) return MOE_ERR_INVALID_ARG;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (!rows_ok(L, T)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (in == nullptr || out == nullptr || !aligned(in, 16) || !aligned(out, 16))
    return MOE_ERR_INVALID_ARG;
  if (!shared && (offsets == nullptr || (op == MOE_OP_GATE_UP_SWIGLU && perm_to_pair == nullptr)))
    return MOE_ERR_INVALID_ARG;
  const WsPlan p = plan(L, T);
  if (!shared && (ws == nullptr || ws_bytes < p.total || !aligned(ws, kAlign)))
    return MOE_ERR_WORKSPACE;
  return run_experts(op, L, shared, offsets, perm_to_pair, shared ? nullptr : active_experts, T,
                     in, out, ws, p, false, static_cast<hipStream_t>(stream));
}

int32_t moe_combine(const float* y_perm, const float* topk_w, const int32_t* pair_to_perm,
                    const float* y_shared, int32_t T, int32_t k, int32_t H, uint16_t* out,
                    void* stream) {
  if (T < 0 || k <= 0 || H <= 0) return MOE_ERR_INVALID_ARG;
  if (H % 4 != 0) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!y_perm || !topk_w || !pair_to_perm || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned(y_perm, 16) || !aligned(out, 8) || (y_shared && !aligned(y_shared, 16)))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_combine(y_perm, topk_w, pair_to_perm, y_shared, T, k, H, out,
                                   static_cast<hipStream_t>(stream)));
}

int32_t moe_layer_forward_ex(const moe_layer_desc* L, const uint16_t* x, int32_t T, uint16_t* out,
                             void* ws, size_t ws_bytes, int32_t act_mode, float* dbg_logits,
                             int32_t* dbg_ids, float* dbg_w, void* stream) {
  return layer_impl(L, x, T, out, ws, ws_bytes, act_mode, dbg_logits, dbg_ids, dbg_w, nullptr,
                    nullptr, stream);
}

int32_t moe_layer_forward(const moe_layer_desc* L, const uint16_t* x, int32_t T, uint16_t* out,
                          void* ws, size_t ws_bytes, float* dbg_logits, int32_t* dbg_ids,
                          float* dbg_w, void* stream) {
  return layer_impl(L, x, T, out, ws, ws_bytes, MOE_ACT_EXACT, dbg_logits, dbg_ids, dbg_w, nullptr,
                    nullptr, stream);
}

int32_t moe_decode_gate_up(const moe_layer_desc* L, const uint16_t* x, int32_t T,
                           const int32_t* topk_ids, uint16_t* h, uint16_t* h_shared, void* stream) {
  int32_t st = check_layer(L);
  if (st != MOE_OK) return st;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (!rows_ok(L, T)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (x == nullptr || topk_ids == nullptr || h == nullptr || !aligned(x, 16) || !aligned(h, 16) ||
      !aligned(topk_ids, 4))
    return MOE_ERR_INVALID_ARG;
  if (L->has_shared && (h_shared == nullptr || !aligned(h_shared, 16))) return MOE_ERR_INVALID_ARG;
  const WsPlan p = plan(L, T);
  DecodeArgs a = decode_args(L, x, T, p);
  // the rows moe_layer_forward gives to the decode lowering
  if (T > kDecodeMaxRows || !decode_rows_ok(a)) return MOE_ERR_UNSUPPORTED;
  a.ids = const_cast<int32_t*>(topk_ids);  // only read
  a.h = h;
  a.hs = L->has_shared ? h_shared : nullptr;
  return hip_status(launch_decode_gate_up(a, static_cast<hipStream_t>(stream)));
}

size_t moe_noalloc_workspace_limit(void) { return kNoAllocBytes; }

int32_t moe_layer_forward_noalloc(const moe_layer_desc* L, const uint16_t* x, int32_t T,
                                  uint16_t* out, void* stream) {
  int32_t st = check_layer(L);
  if (st != MOE_OK) return st;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (!rows_ok(L, T)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (x == nullptr || out == nullptr || !aligned(x, 16) || !aligned(out, 16))
    return MOE_ERR_INVALID_ARG;
  const size_t need = plan(L, T).total;
  if (need > kNoAllocBytes) {
    g_last_error = "moe_layer_forward_noalloc: the layer needs more workspace than the fixed array";
    return MOE_ERR_WORKSPACE;
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_addr[dev] == nullptr) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_status(e);
      g_scratch_addr[dev] = p;
    }
    ws = g_scratch_addr[dev];
  }
  return layer_impl(L, x, T, out, ws, kNoAllocBytes, MOE_ACT_EXACT, nullptr, nullptr, nullptr,
                    nullptr, nullptr, stream);
}

int32_t moe_layer_forward_routed(const moe_layer_desc* L, const uint16_t* x, int32_t T,
                                 const int32_t* topk_ids, const float* topk_w, uint16_t* out,
                                 void* ws, size_t ws_bytes, int32_t act_mode, void* stream) {
  if (T <= 0)  // checks of L and T only; nothing runs
    return layer_impl(L, x, T, out, ws, ws_bytes, act_mode, nullptr, nullptr, nullptr, nullptr,
                      nullptr, stream);
  if (topk_ids == nullptr || topk_w == nullptr || !aligned(topk_ids, 4) || !aligned(topk_w, 4))
    return MOE_ERR_INVALID_ARG;
  return layer_impl(L, x, T, out, ws, ws_bytes, act_mode, nullptr, nullptr, nullptr, topk_ids,
                    topk_w, stream);
}

int32_t moe_route_table(const moe_layer_desc* L, const uint16_t* x, float* logits,
                        const int32_t* token_ids, const int32_t* table, int32_t V, int32_t T,
                        int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes,
                        void* stream) {
  int32_t st = check_layer(L);
  if (st != MOE_OK) return st;
  if (T < 0 || V <= 0) return MOE_ERR_INVALID_ARG;
  if (!rows_ok(L, T)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (token_ids == nullptr || table == nullptr || topk_ids == nullptr || topk_w == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (x == nullptr && logits == nullptr) return MOE_ERR_INVALID_ARG;
  if (x != nullptr && (!aligned(x, 16) || L->H % 8 != 0)) return MOE_ERR_INVALID_ARG;
  const WsPlan p = plan(L, T);
  if (ws == nullptr || ws_bytes < p.total || !aligned(ws, kAlign)) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float* lg = logits;
  if (x != nullptr) {
    // the router's logits (its own top-k goes to scratch and is not used)
    float* lo = logits ? logits : at<float>(ws, p.tlog);
    if ((st = run_route(L, x, lo, T, at<int>(ws, p.ids), at<float>(ws, p.w), ws, p, s)) != MOE_OK)
      return st;
    lg = lo;
  }
  return hip_status(launch_table_route(token_ids, table, V, T, L->top_k, L->E, lg,
                                       L->renormalize, topk_ids, topk_w, s));
}

int32_t moe_quantize_act(int32_t mode, const uint16_t* in, int32_t rows, int32_t K,
                         uint8_t* codes, void* scales, void* stream) {
  if (!act_mode_valid(mode) || rows < 0 || K <= 0 || K % 32 != 0) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if (in == nullptr || codes == nullptr || scales == nullptr || !aligned(in, 16) ||
      !aligned(codes, 16) || !aligned(scales, 4))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_quantize_act(act_kernel_mode(mode), in, rows, K, codes, scales,
                                        static_cast<hipStream_t>(stream)));
}

int32_t moe_expert_gemm_q(int32_t mode, int32_t op, const moe_layer_desc* L, int32_t shared,
                          const int32_t* offsets, const int32_t* perm_to_pair,
                          const int32_t* active_experts, int32_t T, const uint8_t* in_codes,
                          const void* in_scales, void* out, void* ws, size_t ws_bytes,
                          void* stream) {
  int32_t st = check_layer(L);
  if (st != MOE_OK) return st;
  if (!act_mode_valid(mode)) return MOE_ERR_INVALID_ARG;
  if (op != MOE_OP_GATE_UP_SWIGLU && op != MOE_OP_DOWN) return MOE_ERR_INVALID_ARG;
  if (shared != 0 && shared != 1) return MOE_ERR_INVALID_ARG;
  if (shared && !L->has_shared) return MOE_ERR_INVALID_ARG;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (!rows_ok(L, T)) return MOE_ERR_UNSUPPORTED;
  const moe_qweight& wq = (op == MOE_OP_GATE_UP_SWIGLU) ? (shared ? L->sh_gate : L->gate)
                                                        : (shared ? L->sh_down : L->down);
  if (!mode_applies(mode, wq.format) || wq.cols % 32 != 0) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (in_codes == nullptr || in_scales == nullptr || out == nullptr || !aligned(in_codes, 16) ||
      !aligned(in_scales, 4) || !aligned(out, 16))
    return MOE_ERR_INVALID_ARG;
  if (!shared && (offsets == nullptr || (op == MOE_OP_GATE_UP_SWIGLU && perm_to_pair == nullptr)))
    return MOE_ERR_INVALID_ARG;
  const WsPlan p = plan(L, T);
  if (!shared && (ws == nullptr || ws_bytes < p.total || !aligned(ws, kAlign)))
    return MOE_ERR_WORKSPACE;
  return run_experts_q(mode, op, L, shared, offsets, perm_to_pair, active_experts, T, in_codes,
                       in_scales, out, ws, p, false, static_cast<hipStream_t>(stream));
}

}  // extern "C"
