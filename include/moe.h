/*
 * moe.h — C ABI of the routed mixture-of-experts layer for AMD MI355X (gfx950).
 *
 * The layer runs an LLM's routed MoE block directly on checkpoint-format
 * quantized expert weights: NVFP4, MXFP4 and FP8 E4M3 with 128x128 block
 * scales, BF16 activations, FP32 accumulation, no dequantized weight copy.
 * Serving checkpoints as published, with kernels written per weight format and
 * no conversion step, is the premise of the DGPP pages ("DGPP" README, intro
 * bullet on checkpoint formats; forum thread "DGPP: a GB10-optimized C++/CUDA
 * inference engine", opening post, quantization table).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named *in the descriptor and in the calls* are DEVICE pointers,
 *   owned by the caller; the library never allocates, frees or keeps them.
 *   The descriptor structs themselves are read on the host during the call.
 * - All work is queued on `stream` (a hipStream_t; NULL = the default
 *   stream).  No entry point synchronises the stream, so every call may be
 *   captured into a HIP graph.
 * - Argument and shape checks run on the host before anything is queued and
 *   return a negative MOE_ERR_* code; nothing is launched then.  A failed
 *   launch returns MOE_ERR_HIP.  Faults inside kernels surface at the
 *   caller's next synchronisation.
 * - No silent fallback: an unsupported shape or format returns
 *   MOE_ERR_UNSUPPORTED; there is no slow path.
 * - T = 0 is a no-op returning MOE_OK.
 * - bf16 values are passed as uint16_t bit patterns.
 * - Results are deterministic: the same inputs give bit-identical outputs run
 *   after run (no floating-point atomics; fixed reduction orders).  The pages
 *   hold the serving chain to the same contract ("DGPP" README, the paragraph
 *   on the default chain being exact and repeatable).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

/* ---- status codes ------------------------------------------------------ */
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG (-1) /* null pointer, bad size, bad descriptor */
#define MOE_ERR_UNSUPPORTED (-2) /* valid request this library does not run */
#define MOE_ERR_WORKSPACE (-3)   /* workspace missing or smaller than required */
#define MOE_ERR_HIP (-4)         /* a HIP launch failed */

/* ---- weight formats (one projection of E stacked experts) --------------- */
/* NVFP4: codes uint8 [E][rows][cols/2], two E2M1 codes per byte with the
 *   even K index in the low nibble; scales uint8 E4M3 [E][rows][cols/16]
 *   (one per 16 consecutive K of a row); tensor_scale fp32 [E].
 *   W[n,k] = e2m1(q[n,k]) * e4m3(S[n,k/16]) * tensor_scale[e].
 *   Requires cols % 32 == 0.
 * MXFP4: codes as NVFP4; scales uint8 E8M0 [E][rows][cols/32];
 *   tensor_scale NULL.  W[n,k] = e2m1(q[n,k]) * 2^(S[n,k/32]-127).
 *   Requires cols % 32 == 0.
 * FP8_B128: codes uint8 E4M3 ("fn") [E][rows][cols]; scales fp32
 *   [E][ceil(rows/128)][ceil(cols/128)]; tensor_scale NULL.
 *   W[n,k] = e4m3(Q[n,k]) * S[n/128][k/128].  Requires cols % 16 == 0.
 * MXFP8: codes uint8 E4M3 [E][rows][cols]; scales uint8 E8M0
 *   [E][rows][cols/32]; tensor_scale NULL.  W[n,k] = e4m3(Q[n,k]) *
 *   2^(S[n,k/32]-127) (OCP MX v1.0 MXFP8 E4M3).  Requires cols % 32 == 0.
 *   The pages list MXFP8 among the checkpoint formats read as published
 *   ("DGPP" README, intro bullet on checkpoint formats) and serve shared
 *   experts in their shipped MXFP8 (README variant, supported-models table).
 * Element and scale encodings are those of the OCP Microscaling Formats v1.0
 * (E2M1, E8M0) and OCP 8-bit Floating Point (E4M3) specifications.         */
#define MOE_FMT_NVFP4 1
#define MOE_FMT_MXFP4 2
#define MOE_FMT_FP8_B128 3
#define MOE_FMT_MXFP8 4

typedef struct moe_qweight {
  int32_t format;      /* MOE_FMT_* */
  int32_t rows;        /* output features (logical [rows][cols], K = cols contiguous) */
  int32_t cols;        /* input features (the contraction dimension) */
  int32_t num_experts; /* E stacked experts */
  const uint8_t* codes;
  const void* scales;
  const float* tensor_scale;    /* NVFP4 only, else NULL */
  int64_t expert_stride_codes;  /* bytes between experts in `codes`, 16-byte multiple */
  int64_t expert_stride_scales; /* bytes between experts in `scales` */
} moe_qweight;

/* One layer.  Router weight fp32 [H][E] row-major; optional fp32 [E]
 * per-expert logit offsets.  Routed projections: gate and up [E][I][H],
 * down [E][H][I].  Optional always-on shared expert (weight 1): sh_gate,
 * sh_up [1][I_shared][H], sh_down [1][H][I_shared].                        */
typedef struct moe_layer_desc {
  int32_t H, I, E, top_k;
  int32_t renormalize; /* 1: softmax over the k selected logits; 0: full softmax gathered */
  const float* router_w;
  const float* router_bias;
  moe_qweight gate, up, down;
  int32_t has_shared, I_shared;
  moe_qweight sh_gate, sh_up, sh_down;
} moe_layer_desc;

/* ---- expert-GEMM operations ---------------------------------------------- */
#define MOE_OP_GATE_UP_SWIGLU 0 /* in bf16 [rows][H] -> h bf16 [rows][I]: h = bf16(silu(x.Wg^T)*(x.Wu^T)) */
#define MOE_OP_DOWN 1           /* in bf16 [rows][I] -> y fp32 [rows][H]: y = h.Wd^T */

int32_t moe_abi_version(void);
const char* moe_status_string(int32_t status);

/* Text of the last HIP error this library saw on the calling thread (after a
 * MOE_ERR_HIP), or "" if none.  The string is owned by the library. */
const char* moe_last_error(void);

/* Host-only check of a layer descriptor (no HIP call): MOE_OK or a negative code. */
int32_t moe_validate_layer(const moe_layer_desc* L);

/* Workspace bytes every entry point below needs for this layer and T tokens:
 * the memory a call uses is planned and sized before anything is allocated
 * or launched (gitee "dgpp" README, "Highlights": the startup memory plan is
 * checked before allocation; "Request capacity and memory").  A workspace of
 * at least this size (256-byte aligned device memory) serves any call with
 * the same (L, T) or smaller T; it needs no initialisation (no kernel reads a
 * workspace byte the same call has not written).  Calls that share a
 * workspace must not overlap in time.  Returns 0 when the descriptor is
 * invalid, T < 0, or T is beyond the row limit every entry point shares (at
 * most 2^24 (token, slot) pairs, T times each of H, I, I_shared and E below
 * 2^31; above it the entry points return MOE_ERR_UNSUPPORTED); T == 0 gives
 * one 256-byte unit. */
size_t moe_workspace_size(const moe_layer_desc* L, int32_t T);

/* Router softmax + top-k (the router function, top-k and tie rule are not on
 * the pages; this follows a softmax router with k largest logits, ties to the
 * lower expert id, outputs in descending logit order).
 *   x        bf16 [T][H] or NULL.
 *   logits   fp32 [T][E].  If x is NULL: input, and routing is decided on
 *            these values exactly.  Else: output, l = x.Wr + b rounded to fp32;
 *            routing is then decided on the exact logits rounded once to
 *            float64 (a rigorous error bound certifies the fast sum; uncertain
 *            tokens are recomputed with a compensated float64 sum).
 *   topk_ids int32 [T][k]; topk_w fp32 [T][k] (softmax over the k selected,
 *            or over all E when renormalize == 0).
 * NaN logits rank after every number. */
int32_t moe_route_topk(const moe_layer_desc* L, const uint16_t* x, float* logits, int32_t T,
                       int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes,
                       void* stream);

/* Grouping of the T*k (token, slot) pairs by expert, the step that lets the
 * expert GEMMs run over a compact list of the routed segments instead of a
 * grid over the longest one (gitee "dgpp" README, "Configuration", "Execution
 * and performance": engine.expert_tile_list): a stable counting sort (pairs
 * in t-major, slot order within each expert).
 *   topk_ids int32 [T][k] with values in [0, E) (out-of-range ids are dropped).
 *   counts [E]; offsets [E+1] (exclusive scan of counts);
 *   perm_to_pair [T*k]: permuted row -> pair t*k+j (the first offsets[E]
 *            entries); pair_to_perm [T*k]: inverse, -1 for a dropped pair.
 *   active_experts int32 [E+1] or NULL: element 0 = number of experts with at
 *            least one row, then their ids in increasing order.
 * At most 2^24 pairs (T*k); more returns MOE_ERR_UNSUPPORTED (and a
 * workspace size of 0).
 * Workspace: moe_permute_workspace_size(T, k, E) bytes. */
size_t moe_permute_workspace_size(int32_t T, int32_t k, int32_t E);
int32_t moe_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E, int32_t* counts,
                    int32_t* offsets, int32_t* perm_to_pair, int32_t* pair_to_perm,
                    int32_t* active_experts, void* ws, size_t ws_bytes, void* stream);

/* One expert projection pass over grouped rows.
 *   shared = 0: routed experts; rows are the T*k permuted pairs grouped by
 *     `offsets` [E+1]; for op GATE_UP the input row of permuted row p is
 *     token perm_to_pair[p]/k of `in` (x bf16 [T][H]); for op DOWN the input
 *     row is p of `in` (h bf16 [T*k][I]).  Output row p in permuted order.
 *   active_experts: routed only, the [E+1] list moe_permute writes (count,
 *     then ids), or NULL.  With T <= 64 and a list, one block row per active
 *     expert takes its whole group; otherwise the call derives a list of row
 *     chunks from `offsets` with one extra launch (16-row chunks of a group
 *     run in parallel blocks for T <= 64, 128-row tiles above).
 *   shared = 1: the shared expert over T rows of `in`; offsets, perm_to_pair
 *     and active_experts unused.
 *   out: GATE_UP -> bf16 [rows][I or I_shared]; DOWN -> fp32 [rows][H].
 * Accumulation is fp32; products of the decoded weight and the bf16 input are
 * exact.  The intermediate h is BF16 (activations stay BF16, forum opening
 * post).  The kernel variant follows the row count (row-aware lowering, gitee
 * "dgpp" README, "Highlights"): calls with T <= 64 stream each active
 * expert's weights with its own blocks, 16 rows per pass; larger calls run the
 * tiled grouped GEMM. */
int32_t moe_expert_gemm(int32_t op, const moe_layer_desc* L, int32_t shared,
                        const int32_t* offsets, const int32_t* perm_to_pair,
                        const int32_t* active_experts, int32_t T, const uint16_t* in, void* out,
                        void* ws, size_t ws_bytes, void* stream);

/* Weighted combine (partials kept in fp32, summed in slot order; bf16
 * partials are a lossy lever on the pages, gitee "dgpp" README, "Execution
 * and performance", engine.prefill_bf16_partials):
 *   out[t] = bf16( sum_{j<k} w[t,j] * y_perm[pair_to_perm[t*k+j]] + y_shared[t] ),
 *   a pair with pair_to_perm -1 (dropped by the grouping) contributing nothing.
 *   y_perm fp32 [T*k][H]; topk_w fp32 [T][k]; y_shared fp32 [T][H] or NULL;
 *   out bf16 [T][H]. */
int32_t moe_combine(const float* y_perm, const float* topk_w, const int32_t* pair_to_perm,
                    const float* y_shared, int32_t T, int32_t k, int32_t H, uint16_t* out,
                    void* stream);

/* The whole layer on checkpoint-format expert weights with no dequantized
 * copy (the "DGPP" README intro: checkpoints served as published; forum
 * thread "DGPP: a GB10-optimized C++/CUDA inference engine", opening post:
 * NVFP4 / MXFP4 routed experts, FP8 block-128 experts and shared experts,
 * activations BF16): route, group, gate/up + SwiGLU, down, shared expert,
 * combine.  x bf16 [T][H] -> out bf16 [T][H], both 16-byte aligned device
 * memory owned by the caller.  Optional debug outputs (NULL to skip): logits
 * fp32 [T][E], ids int32 [T][k], weights fp32 [T][k].  The lowering follows
 * the row count (gitee "dgpp" README, "Highlights": row-aware execution):
 * T <= 8 runs the decode lowering (each active expert's weights streamed once
 * for all its tokens), and so does T <= 32 with T*k <= 512 when every
 * projection has the aligned tile (FP4 gate/up with H a multiple of 2048 and
 * H <= 4096; FP4 or FP8 down projections with I a multiple of 512, I <= 4096
 * and H a multiple of 64; whole-chunk FP4 scale words); otherwise 9..64 rows
 * run the expert GEMV, larger T the grouped GEMM over a tile list.
 * Errors: MOE_ERR_INVALID_ARG (T < 0, null or misaligned x / out),
 * MOE_ERR_WORKSPACE (ws null, misaligned or below
 * moe_workspace_size(L, T)), MOE_ERR_UNSUPPORTED (a shape or format the
 * descriptor check rejects), MOE_ERR_HIP (a launch failed; moe_last_error
 * gives the text).  T == 0 returns MOE_OK and launches nothing. */
int32_t moe_layer_forward(const moe_layer_desc* L, const uint16_t* x, int32_t T, uint16_t* out,
                          void* ws, size_t ws_bytes, float* dbg_logits, int32_t* dbg_ids,
                          float* dbg_w, void* stream);

/* ---- opt-in lossy activation modes ---------------------------------------
 * The default chain keeps activations BF16.  The pages name activation
 * quantization only as explicit levers, off by default: NVFP4 W4A4 prefill
 * behind an opt-in switch (forum thread "DGPP: a GB10-optimized C++/CUDA
 * inference engine", page 5, the update post), and an FP8 prefill GEMM on
 * per-token 1x128 E4M3 activations against the checkpoint's 128x128 weight
 * scales, not bitwise (gitee "dgpp" README, "Execution and performance",
 * engine.prefill_fp8_gemm).  These modes quantize each expert GEMM input
 * row from its BF16 form and run the contraction on the gfx950 scaled
 * FP8/FP4 matrix cores:
 *   MOE_ACT_MXFP8    (W4A8, MXFP4 experts): E4M3 elements, E8M0 scale per 32 K.
 *   MOE_ACT_MXFP4    (W4A4, MXFP4 experts): E2M1 elements, E8M0 scale per 32 K.
 *     MX conversion (OCP Microscaling Formats v1.0): shared exponent
 *     floor(log2 max|v|) - emax(element) (8 for E4M3, 2 for E2M1), clamped
 *     to [-127, 127]; elements round to nearest even after v / 2^shared,
 *     saturating.  All-zero block: scale code 0; a non-finite value: scale
 *     0xFF and zero codes.
 *   MOE_ACT_FP8_T128 (FP8 block-128 experts): E4M3 elements, fp32 scale per
 *     128 K: s = max(amax, 2^-64) / 448, e = RNE(clamp(v / s, +-448)), both
 *     divisions IEEE fp32; a non-finite value: s = NaN and zero codes.
 * A mode quantizes the inputs of the projections whose weight format it
 * names (MXFP4 for the MX modes, FP8_B128 for FP8_T128); other projections
 * keep the exact chain.  NVFP4 experts have no lossy mode here: their
 * 16-wide E4M3 block scales do not fit the matrix cores' E8M0-per-32 scale
 * operand.  Results are deterministic but not those of the exact chain.  */
#define MOE_ACT_EXACT 0
#define MOE_ACT_MXFP8 1
#define MOE_ACT_MXFP4 2
#define MOE_ACT_FP8_T128 3

/* Quantize bf16 rows for a lossy mode.
 *   in     bf16 [rows][K], 16-byte aligned; K % 32 == 0.
 *   codes  MXFP8 / FP8_T128: uint8 E4M3 [rows][K];
 *          MXFP4: uint8 [rows][K/2], two E2M1 codes per byte, even K in the
 *          low nibble; 16-byte aligned.
 *   scales [rows][4*ceil(K/128)] bytes, 4-byte aligned:
 *          MX modes: E8M0 codes, entry j for K [32j, 32j+32); entries at and
 *          past K/32 are written 127 (unit scale, padding to whole 128-K
 *          steps); FP8_T128: fp32 [rows][ceil(K/128)], entry j for
 *          K [128j, 128j+128).
 * Returns MOE_ERR_INVALID_ARG for a bad mode, size or pointer. */
int32_t moe_quantize_act(int32_t mode, const uint16_t* in, int32_t rows, int32_t K,
                         uint8_t* codes, void* scales, void* stream);

/* moe_expert_gemm on quantized inputs (always the tiled grouped GEMM on the
 * scaled matrix cores, at any T).  in_codes / in_scales as moe_quantize_act
 * writes them for the projection's input: x rows [T][H] for op GATE_UP
 * (routed rows read token perm_to_pair[p]/k), the permuted h rows [T*k][I]
 * for op DOWN (shared: [T][I_shared]).  The projection's weight format must
 * be the one the mode names, else MOE_ERR_UNSUPPORTED.  Other arguments and
 * outputs as moe_expert_gemm. */
int32_t moe_expert_gemm_q(int32_t mode, int32_t op, const moe_layer_desc* L, int32_t shared,
                          const int32_t* offsets, const int32_t* perm_to_pair,
                          const int32_t* active_experts, int32_t T, const uint8_t* in_codes,
                          const void* in_scales, void* out, void* ws, size_t ws_bytes,
                          void* stream);

/* moe_layer_forward with an activation mode (MOE_ACT_*).  The mode applies to
 * the prefill lowering (T > 64, the tiled grouped GEMM); decode-sized calls
 * (T <= 64) stream the weights once per active expert, where quantizing the
 * few activation rows saves nothing, and compute the exact chain.  A mode
 * that names no projection format of the layer, or applies to a projection
 * whose K (cols) is not a multiple of 32, returns MOE_ERR_UNSUPPORTED.
 * The workspace of moe_workspace_size(L, T) serves every mode.  MOE_ACT_EXACT
 * is moe_layer_forward. */
int32_t moe_layer_forward_ex(const moe_layer_desc* L, const uint16_t* x, int32_t T, uint16_t* out,
                             void* ws, size_t ws_bytes, int32_t act_mode, float* dbg_logits,
                             int32_t* dbg_ids, float* dbg_w, void* stream);

/* ---- routing from a token table, and the layer on a given routing --------
 * The pages route the first layers of one served model by a token table
 * ("DGPP" README variant, supported-models notes on DeepSeek-V4-Flash;
 * source layout, the dsv4 model directory) and give no more detail.  The
 * reading taken: the experts of token t are row token_ids[t] of `table`, in
 * table order, and the weights are the layer's own router function at those
 * experts (the softmax over the k selected logits, or with renormalize == 0
 * the full softmax gathered).
 *   token_ids int32 [T]; table int32 [V][k] (k = L->top_k).
 *   x bf16 [T][H] or NULL; logits fp32 [T][E]: with x NULL the input, else
 *     the router's logits are written there (NULL: kept in the workspace).
 *   topk_ids int32 [T][k], topk_w fp32 [T][k] (weights computed in float64).
 * A token id outside [0, V) selects nothing (ids -1, weights 0); a table
 * entry outside [0, E) is passed through with weight 0 and no part in the
 * normalisation (the grouping drops it).  NaN logits: unspecified.
 * Workspace: moe_workspace_size(L, T). */
int32_t moe_route_table(const moe_layer_desc* L, const uint16_t* x, float* logits,
                        const int32_t* token_ids, const int32_t* table, int32_t V, int32_t T,
                        int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes,
                        void* stream);

/* moe_layer_forward_ex on a given routing (topk_ids int32 [T][k], topk_w fp32
 * [T][k], device, e.g. from moe_route_topk or moe_route_table) instead of the
 * router: grouping, experts, shared expert and combine.  Expert ids outside
 * [0, E) are dropped (their slots contribute nothing).  Where
 * moe_layer_forward takes the decode lowering only its expert launches run. */
int32_t moe_layer_forward_routed(const moe_layer_desc* L, const uint16_t* x, int32_t T,
                                 const int32_t* topk_ids, const float* topk_w, uint16_t* out,
                                 void* ws, size_t ws_bytes, int32_t act_mode, void* stream);

/* The decode lowering's gate/up stage alone (the rows moe_layer_forward
 * gives to it: T <= 8, up to 32 on aligned shapes), on a given routing:
 * each active routed expert's gate and up projections streamed once for all
 * of its tokens, both in one pass with SwiGLU in the epilogue (the pages pair
 * gate and up in one launch: gitee "dgpp" README, "Execution and
 * performance", engine.expert_gemm_pair), and the shared expert's.
 *   topk_ids int32 [T][k] (ids outside [0, E) are skipped);
 *   h        bf16 [T*k][I]: row t*k+j = bf16(silu(x_t.Wg_e^T) * (x_t.Wu_e^T)),
 *            e = topk_ids[t][j] (rows of skipped pairs are not written);
 *   h_shared bf16 [T][I_shared] (the shared expert), NULL without one.
 * Other T returns MOE_ERR_UNSUPPORTED.  This is the first of the decode
 * lowering's expert launches, exposed so that it can be timed and checked on
 * its own; moe_layer_forward runs it wherever it takes the decode lowering. */
int32_t moe_decode_gate_up(const moe_layer_desc* L, const uint16_t* x, int32_t T,
                           const int32_t* topk_ids, uint16_t* h, uint16_t* h_shared, void* stream);

/* ---- the layer without a caller workspace ------------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture that must not call hipMalloc, tight serving loops, harnesses that
 * forbid allocation.  moe_layer_forward (MOE_ACT_EXACT, no debug outputs)
 * with its workspace taken from one fixed array inside the library, of
 * moe_noalloc_workspace_limit() bytes (32 MiB) per GPU, held by each GPU the
 * call runs on until the process ends.  The call allocates and frees
 * nothing (no hipMalloc, hipFree or allocating library routine).
 *   Returns MOE_ERR_WORKSPACE, before any launch, when the layer at this T
 *   needs more workspace than the array holds (moe_workspace_size(L, T) >
 *   moe_noalloc_workspace_limit(); at H = 2048, E = 512, I = 512, top-10
 *   that is above roughly T = 350 tokens); other errors as moe_layer_forward.
 *   Every call on a GPU shares that GPU's array, which keeps the last call's
 *   contents (no kernel reads a workspace byte before writing it in the same
 *   call): calls that overlap in time on one GPU, on any streams, race. */
size_t moe_noalloc_workspace_limit(void);
int32_t moe_layer_forward_noalloc(const moe_layer_desc* L, const uint16_t* x, int32_t T,
                                  uint16_t* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
