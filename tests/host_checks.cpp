// Host-side checks of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code of every library source (see
// tests/test_host_sanitize.py).  Only validation, workspace planning and the
// argument checks of the entry points run: every pointer is a fake device
// address that no host code may dereference, and on a machine without a GPU
// any call that gets past its checks stops at its first HIP call
// (MOE_ERR_HIP).  The driver exits non-zero on a wrong status; the sanitizers
// abort on any memory error or undefined behaviour.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../include/moe.h"

static int g_fail = 0;

#define EXPECT(cond, ...)                                   \
  do {                                                      \
    if (!(cond)) {                                          \
      std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      std::fprintf(stderr, __VA_ARGS__);                    \
      std::fprintf(stderr, "\n");                           \
      ++g_fail;                                             \
    }                                                       \
  } while (0)

// a fake, 256-byte aligned device address (never dereferenced on the host)
static const void* fake(uintptr_t k) { return reinterpret_cast<const void*>((k + 1) << 20); }

static moe_qweight qw(int fmt, int E, int rows, int cols, uintptr_t tag) {
  moe_qweight q;
  std::memset(&q, 0, sizeof(q));
  q.format = fmt;
  q.rows = rows;
  q.cols = cols;
  q.num_experts = E;
  q.codes = static_cast<const uint8_t*>(fake(tag));
  q.scales = fake(tag + 1);
  q.tensor_scale = (fmt == MOE_FMT_NVFP4) ? static_cast<const float*>(fake(tag + 2)) : nullptr;
  const int64_t rb = (fmt == MOE_FMT_FP8_B128 || fmt == MOE_FMT_MXFP8) ? cols : cols / 2;
  q.expert_stride_codes = ((int64_t)rows * rb + 15) / 16 * 16;
  if (fmt == MOE_FMT_NVFP4)
    q.expert_stride_scales = (int64_t)rows * (cols / 16);
  else if (fmt == MOE_FMT_FP8_B128)
    q.expert_stride_scales = (int64_t)((rows + 127) / 128) * ((cols + 127) / 128) * 4;
  else
    q.expert_stride_scales = (int64_t)rows * ((cols + 31) / 32);
  return q;
}

static moe_layer_desc layer(int fmt, int H, int I, int E, int k, bool shared, int sfmt, int Is) {
  moe_layer_desc L;
  std::memset(&L, 0, sizeof(L));
  L.H = H;
  L.I = I;
  L.E = E;
  L.top_k = k;
  L.renormalize = 1;
  L.router_w = static_cast<const float*>(fake(1));
  L.router_bias = nullptr;
  L.gate = qw(fmt, E, I, H, 10);
  L.up = qw(fmt, E, I, H, 20);
  L.down = qw(fmt, E, H, I, 30);
  L.has_shared = shared ? 1 : 0;
  L.I_shared = shared ? Is : 0;
  if (shared) {
    L.sh_gate = qw(sfmt, 1, Is, H, 40);
    L.sh_up = qw(sfmt, 1, Is, H, 50);
    L.sh_down = qw(sfmt, 1, H, Is, 60);
  }
  return L;
}

// xorshift64*: a seeded stream for the descriptor fuzz
static uint64_t g_rng = 0x9E3779B97F4A7C15ull;
static uint64_t rnd() {
  g_rng ^= g_rng >> 12;
  g_rng ^= g_rng << 25;
  g_rng ^= g_rng >> 27;
  return g_rng * 2685821657736338717ull;
}
static int pick(const int* v, int n) { return v[rnd() % (uint64_t)n]; }

int main() {
  EXPECT(moe_abi_version() == MOE_ABI_VERSION, "abi version");
  for (int st = -6; st <= 1; ++st) EXPECT(moe_status_string(st) != nullptr, "status string %d", st);
  EXPECT(moe_last_error() != nullptr, "last error");

  const int fmts[] = {MOE_FMT_NVFP4, MOE_FMT_MXFP4, MOE_FMT_FP8_B128, MOE_FMT_MXFP8};

  // valid layers of every format, with and without a shared expert
  for (int f : fmts)
    for (int sf : fmts) {
      moe_layer_desc L = layer(f, 2048, 512, 512, 10, true, sf, 512);
      EXPECT(moe_validate_layer(&L) == MOE_OK, "valid layer fmt %d shared %d", f, sf);
      const int Ts[] = {0, 1, 5, 8, 9, 40, 64, 65, 150, 8192};
      size_t prev = 0;
      for (int T : Ts) {
        const size_t ws = moe_workspace_size(&L, T);
        EXPECT(ws > 0 && ws % 256 == 0, "workspace size T=%d: %zu", T, ws);
        (void)prev;
        prev = ws;
      }
      EXPECT(moe_workspace_size(&L, -1) == 0, "negative T");
    }

  // descriptor errors: each must be reported, never crash
  {
    moe_layer_desc L = layer(MOE_FMT_NVFP4, 2048, 512, 64, 4, false, 0, 0);
    EXPECT(moe_validate_layer(nullptr) == MOE_ERR_INVALID_ARG, "null desc");
    moe_layer_desc B = L;
    B.top_k = 65;
    EXPECT(moe_validate_layer(&B) == MOE_ERR_INVALID_ARG, "top_k > E");
    B = L;
    B.gate.rows = 500;
    EXPECT(moe_validate_layer(&B) == MOE_ERR_INVALID_ARG, "gate rows != I");
    B = L;
    B.gate.codes = nullptr;
    EXPECT(moe_validate_layer(&B) == MOE_ERR_INVALID_ARG, "null codes");
    B = L;
    B.up.expert_stride_codes = 8;
    EXPECT(moe_validate_layer(&B) == MOE_ERR_INVALID_ARG, "short expert stride");
    B = L;
    B.down.tensor_scale = nullptr;
    EXPECT(moe_validate_layer(&B) == MOE_ERR_INVALID_ARG, "NVFP4 without tensor scale");
    B = L;
    B.renormalize = 2;
    EXPECT(moe_validate_layer(&B) == MOE_ERR_INVALID_ARG, "renormalize flag");
    B = layer(MOE_FMT_NVFP4, 2048 + 16, 512, 64, 4, false, 0, 0);
    EXPECT(moe_validate_layer(&B) == MOE_ERR_UNSUPPORTED, "NVFP4 K %% 32 != 0");
    B = layer(MOE_FMT_FP8_B128, 2048 + 16, 512, 64, 4, false, 0, 0);
    EXPECT(moe_validate_layer(&B) == MOE_OK, "FP8 K %% 16 == 0");
    B = layer(MOE_FMT_MXFP4, 2048, 512 + 8, 64, 4, false, 0, 0);
    EXPECT(moe_validate_layer(&B) == MOE_ERR_UNSUPPORTED, "rows %% 16 != 0");
    B = L;
    B.gate.format = 9;
    EXPECT(moe_validate_layer(&B) == MOE_ERR_UNSUPPORTED, "unknown format");
  }

  // entry points reject bad arguments before any launch
  {
    moe_layer_desc L = layer(MOE_FMT_MXFP4, 2048, 512, 64, 4, true, MOE_FMT_FP8_B128, 256);
    const size_t ws = moe_workspace_size(&L, 150);
    uint16_t* x = (uint16_t*)fake(100);
    uint16_t* out = (uint16_t*)fake(200);
    void* w = (void*)fake(300);
    EXPECT(moe_layer_forward(&L, x, 150, out, w, ws - 256, nullptr, nullptr, nullptr, nullptr) ==
               MOE_ERR_WORKSPACE, "small workspace");
    EXPECT(moe_layer_forward(&L, x, 150, out, nullptr, ws, nullptr, nullptr, nullptr, nullptr) ==
               MOE_ERR_WORKSPACE, "null workspace");
    EXPECT(moe_layer_forward(&L, x, -1, out, w, ws, nullptr, nullptr, nullptr, nullptr) ==
               MOE_ERR_INVALID_ARG, "negative T");
    EXPECT(moe_layer_forward(&L, x, 0, out, w, ws, nullptr, nullptr, nullptr, nullptr) == MOE_OK,
           "T == 0");
    EXPECT(moe_layer_forward(&L, x + 1, 150, out, w, ws, nullptr, nullptr, nullptr, nullptr) ==
               MOE_ERR_INVALID_ARG, "misaligned x");
    EXPECT(moe_layer_forward(&L, nullptr, 150, out, w, ws, nullptr, nullptr, nullptr, nullptr) ==
               MOE_ERR_INVALID_ARG, "null x");
    EXPECT(moe_layer_forward_ex(&L, x, 150, out, w, ws, 77, nullptr, nullptr, nullptr, nullptr) ==
               MOE_ERR_INVALID_ARG, "unknown activation mode");
    const size_t lim = moe_noalloc_workspace_limit();
    EXPECT(lim > 0, "no-alloc limit");
    EXPECT(moe_layer_forward_noalloc(&L, x, 100000, out, nullptr) == MOE_ERR_WORKSPACE,
           "no-alloc beyond its array");
    EXPECT(moe_layer_forward_noalloc(&L, x, 1 << 20, out, nullptr) == MOE_ERR_UNSUPPORTED,
           "rows beyond the limit");
    EXPECT(moe_layer_forward(&L, x, 1 << 20, out, w, ws, nullptr, nullptr, nullptr, nullptr) ==
               MOE_ERR_UNSUPPORTED, "rows beyond the limit");
    EXPECT(moe_workspace_size(&L, 1 << 20) == 0, "no workspace beyond the row limit");
    EXPECT(moe_permute_workspace_size(8192, 10, 512) > 0, "permute workspace");
    EXPECT(moe_permute_workspace_size(0x7fffffff, 64, 4096) == 0, "permute beyond the pair limit");
    EXPECT(moe_permute(nullptr, 0x7fffffff, 64, 4096, nullptr, nullptr, nullptr, nullptr, nullptr,
                       nullptr, 0, nullptr) == MOE_ERR_UNSUPPORTED, "permute beyond the pair limit");
    EXPECT(moe_combine(nullptr, nullptr, nullptr, nullptr, 4, 2, 256, nullptr, nullptr) ==
               MOE_ERR_INVALID_ARG, "combine null pointers");
  }

  // workspace planning at extreme T: no overflow, either a size or 0
  {
    moe_layer_desc L = layer(MOE_FMT_NVFP4, 7168, 2048, 256, 8, true, MOE_FMT_FP8_B128, 2048);
    const int Ts[] = {1 << 16, 1 << 20, 1 << 24, 0x7fffffff};
    for (int T : Ts) {
      const size_t ws = moe_workspace_size(&L, T);
      EXPECT(ws == 0 || ws % 256 == 0, "T=%d size %zu", T, ws);
    }
  }

  // descriptor fuzz: random shapes, formats and strides, seeded
  {
    const int Hs[] = {0, 16, 64, 128, 256, 384, 512, 2048, 2064, 6144, 7168, -128};
    const int Is[] = {0, 16, 48, 128, 192, 512, 520, 2048, 4096};
    const int Es[] = {1, 2, 8, 64, 257, 512, 1024, 4096, -1};
    const int ks[] = {1, 2, 8, 10, 16, 17, 64, 0};
    const int fm[] = {MOE_FMT_NVFP4, MOE_FMT_MXFP4, MOE_FMT_FP8_B128, MOE_FMT_MXFP8, 0, 7};
    const int Tv[] = {0, 1, 3, 8, 9, 33, 64, 65, 300, 4096};
    int ok = 0;
    for (int it = 0; it < 20000; ++it) {
      const int f = pick(fm, 6);
      const bool sh = (rnd() & 1) != 0;
      moe_layer_desc L = layer(f, pick(Hs, 12), pick(Is, 9), pick(Es, 9), pick(ks, 8), sh,
                               pick(fm, 6), pick(Is, 9));
      switch (rnd() % 8) {
        case 0: L.down.expert_stride_scales -= (int64_t)(rnd() % 5); break;
        case 1: L.gate.codes = (const uint8_t*)((uintptr_t)L.gate.codes + rnd() % 32); break;
        case 2: L.up.num_experts += (int)(rnd() % 3) - 1; break;
        case 3: L.router_w = (rnd() & 1) ? nullptr : L.router_w; break;
        default: break;
      }
      const int32_t st = moe_validate_layer(&L);
      EXPECT(st == MOE_OK || st == MOE_ERR_INVALID_ARG || st == MOE_ERR_UNSUPPORTED,
             "fuzz %d status %d", it, st);
      const int T = pick(Tv, 10);
      const size_t ws = moe_workspace_size(&L, T);
      EXPECT((st == MOE_OK) == (ws != 0), "fuzz %d: status %d but workspace %zu", it, st, ws);
      if (st == MOE_OK) ++ok;
    }
    EXPECT(ok > 100, "fuzz reached few valid descriptors (%d)", ok);
  }

  if (g_fail) {
    std::fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  std::printf("host checks passed\n");
  return 0;
}
