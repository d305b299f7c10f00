// Host-side run of every argument check of the C ABI (csrc/fa_api.hip) under the
// address and undefined-behaviour sanitizers. fa_api.hip is compiled with hipcc's host
// pass only; the kernel launchers it calls (kernels.h) and the few HIP runtime entry
// points it uses are replaced by the stubs below, which record the calls that get past
// validation. Every FA_ERR_* path of every entry point is driven, then valid calls
// that reach a launcher (FA_OK), a launcher that fails (FA_ERR_LAUNCH) and the
// scratch lookup of fa_bwd_noalloc. Prints "ok" or the first failing check and exits
// non-zero. Built and run by tests/test_abi_sanitize.py.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>

#include "fa.h"
#include "kernels.h"

// ---- stubs -----------------------------------------------------------------------
static int g_launches = 0;                   // launcher calls that reached a stub
static hipError_t g_launch_result = hipSuccess;
static int g_symbol_lookups = 0;
static hipError_t g_get_device_result = hipSuccess;
static float g_scratch_stub[64];             // what the stubbed symbol lookup returns
static const float* g_last_dvec = nullptr;   // workspace the backward launcher got

namespace fa {
hipError_t launch_fwd_bf16(const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, float*,
                           const AttnShape&, hipStream_t) { ++g_launches; return g_launch_result; }
hipError_t launch_fwd_bf16_variant(const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*,
                                   float*, const AttnShape&, int, hipStream_t) {
  ++g_launches; return g_launch_result;
}
size_t fwd_v1_workspace_floats(const AttnShape& s) {
  return (size_t)s.B * s.Hq * ((s.Nq + 127) / 128) * (128 * (size_t)s.d + 512);
}
hipError_t launch_fwd_v1(const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, float*,
                         float*, const AttnShape&, hipStream_t) { ++g_launches; return g_launch_result; }
hipError_t launch_fwd_fp8(const uint8_t*, const uint8_t*, const uint8_t*, uint16_t*, float*, float,
                          float, float, const AttnShape&, hipStream_t) {
  ++g_launches; return g_launch_result;
}
hipError_t launch_fwd_f32(const float*, const float*, const float*, float*, float*,
                          const AttnShape&, hipStream_t) { ++g_launches; return g_launch_result; }
hipError_t launch_fwd_splitkv(const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, float*,
                              float*, float*, int, const AttnShape&, hipStream_t) {
  ++g_launches; return g_launch_result;
}
hipError_t launch_bwd(const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*,
                      const uint16_t*, const float*, uint16_t*, uint16_t*, uint16_t*, float* dvec,
                      const AttnShape&, int, hipStream_t) {
  ++g_launches; g_last_dvec = dvec; return g_launch_result;
}
hipError_t launch_mfma_probe(float*, int, int, int, hipStream_t) { ++g_launches; return g_launch_result; }
}  // namespace fa

extern "C" {
hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return g_get_device_result;
}
hipError_t hipGetSymbolAddress(void** p, const void*) {
  ++g_symbol_lookups;
  *p = g_scratch_stub;
  return hipSuccess;
}
// registration of the library's device array (host pass only: nothing to register)
void** __hipRegisterFatBinary(const void*) { static void* h = nullptr; return &h; }
void __hipUnregisterFatBinary(void**) {}
void __hipRegisterVar(void**, char*, char*, const char*, int, size_t, int, int) {}
}
// the fat binary the host pass refers to (no device code in this build)
extern "C" const char FA_FATBIN_SYMBOL[16] = {0};

// ---- checks ----------------------------------------------------------------------
static int g_fail = 0;
#define EXPECT(cond, ...)                      \
  do {                                         \
    if (!(cond) && !g_fail) {                  \
      std::printf("FAIL line %d: ", __LINE__); \
      std::printf(__VA_ARGS__);                \
      std::printf("\n");                       \
      g_fail = 1;                              \
    }                                          \
  } while (0)

alignas(256) static char g_buf[1 << 16];
static void* const P = g_buf;        // aligned, never dereferenced by the library
static void* const PU = g_buf + 2;   // misaligned
static const float kNan = std::numeric_limits<float>::quiet_NaN();
static const float kInf = std::numeric_limits<float>::infinity();

static int fwd(const char* which, void* q, void* o, float* lse, int B, int Hq, int Hkv, int Nq,
               int Nk, int d, float scale) {
  if (!std::strcmp(which, "bf16"))
    return fa_fwd(q, P, P, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, 1, nullptr);
  if (!std::strcmp(which, "f32"))
    return fa_fwd_f32((const float*)q, (const float*)P, (const float*)P, (float*)o, lse, B, Hq,
                      Hkv, Nq, Nk, d, scale, 1, nullptr);
  return fa_fwd_fp8(q, P, P, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, 1.f, 1.f, 1.f, 1, nullptr);
}

static void check_forwards() {
  float* L = (float*)P;
  for (const char* w : {"bf16", "f32", "fp8"}) {
    EXPECT(fwd(w, nullptr, P, L, 1, 2, 1, 8, 8, 64, .1f) == FA_ERR_NULL, "%s null q", w);
    EXPECT(fwd(w, P, nullptr, L, 1, 2, 1, 8, 8, 64, .1f) == FA_ERR_NULL, "%s null o", w);
    EXPECT(fwd(w, P, P, nullptr, 1, 2, 1, 8, 8, 64, .1f) == FA_ERR_NULL, "%s null lse", w);
    const int bad[][6] = {{0, 2, 1, 8, 8, 64}, {1, 0, 1, 8, 8, 64}, {1, 2, 0, 8, 8, 64},
                          {1, 2, 1, 0, 8, 64}, {1, 2, 1, 8, 0, 64}, {1, 2, 1, 8, 8, 0},
                          {-1, 2, 1, 8, 8, 64}, {1, 2, 1, -5, 8, 64},
                          {1, 2, 1, 8, std::numeric_limits<int>::min(), 64}};
    for (auto& b : bad)
      EXPECT(fwd(w, P, P, L, b[0], b[1], b[2], b[3], b[4], b[5], .1f) == FA_ERR_SHAPE, "%s shape", w);
    EXPECT(fwd(w, P, P, L, 1, 3, 2, 8, 8, 64, .1f) == FA_ERR_HEADS, "%s heads", w);
    for (float s : {0.f, -1.f, kNan, kInf, -kInf})
      EXPECT(fwd(w, P, P, L, 1, 2, 1, 8, 8, 64, s) == FA_ERR_SCALE, "%s scale %g", w, s);
    EXPECT(fwd(w, PU, P, L, 1, 2, 1, 8, 8, 64, .1f) == FA_ERR_ALIGN, "%s align q", w);
    EXPECT(fwd(w, P, PU, L, 1, 2, 1, 8, 8, 64, .1f) == FA_ERR_ALIGN, "%s align o", w);
    EXPECT(fwd(w, P, P, L, 1 << 20, 1 << 12, 1, 1 << 10, 8, 64, .1f) == FA_ERR_TOO_LARGE,
           "%s too large", w);
    EXPECT(fwd(w, P, P, L, 1 << 16, 1, 1, 8, 1 << 16, 64, .1f) == FA_ERR_TOO_LARGE,
           "%s too large (keys)", w);
  }
  for (int d : {32, 96, 100, 257, 512})
    EXPECT(fwd("bf16", P, P, (float*)P, 1, 2, 1, 8, 8, d, .1f) == FA_ERR_HEAD_DIM, "bf16 d %d", d);
  for (int d : {2, 6, 260, 512})
    EXPECT(fwd("f32", P, P, (float*)P, 1, 2, 1, 8, 8, d, .1f) == FA_ERR_HEAD_DIM, "f32 d %d", d);
  for (int d : {32, 100})
    EXPECT(fwd("fp8", P, P, (float*)P, 1, 2, 1, 8, 8, d, .1f) == FA_ERR_HEAD_DIM, "fp8 d %d", d);
  // FP8 descales, and a product that overflows once folded together
  EXPECT(fa_fwd_fp8(P, P, P, P, (float*)P, 1, 2, 1, 8, 8, 64, .1f, 0.f, 1.f, 1.f, 1, nullptr) ==
             FA_ERR_SCALE, "fp8 descale 0");
  EXPECT(fa_fwd_fp8(P, P, P, P, (float*)P, 1, 2, 1, 8, 8, 64, .1f, 1.f, kNan, 1.f, 1, nullptr) ==
             FA_ERR_SCALE, "fp8 descale nan");
  EXPECT(fa_fwd_fp8(P, P, P, P, (float*)P, 1, 2, 1, 8, 8, 64, 1e30f, 1e30f, 1e30f, 1.f, 1,
                    nullptr) == FA_ERR_SCALE, "fp8 folded overflow");
  // valid calls reach the launcher; a failing launcher maps to FA_ERR_LAUNCH
  for (const char* w : {"bf16", "f32", "fp8"}) {
    const int before = g_launches;
    EXPECT(fwd(w, P, P, (float*)P, 2, 4, 2, 100, 130, 128, .1f) == FA_OK, "%s valid", w);
    EXPECT(g_launches == before + 1, "%s launch count", w);
    g_launch_result = hipErrorInvalidValue;
    EXPECT(fwd(w, P, P, (float*)P, 2, 4, 2, 100, 130, 128, .1f) == FA_ERR_LAUNCH, "%s launch err", w);
    g_launch_result = hipSuccess;
  }
}

static void check_splitkv() {
  float* L = (float*)P;
  EXPECT(fa_splitkv_default_splits(0, 1, 1, 1, 1, 64) == 1, "default splits of bad shape");
  EXPECT(fa_splitkv_default_splits(8, 8, 8, 1, 32768, 128) >= 1, "default splits");
  EXPECT(fa_splitkv_default_splits(1, 1, 1, 1, 1 << 30, 128) <= 1024, "split cap");
  EXPECT(fa_fwd_splitkv_workspace_bytes(0, 1, 1, 1, 1, 64, 4) == 0, "ws of bad shape");
  const size_t ws = fa_fwd_splitkv_workspace_bytes(2, 4, 1, 1, 4096, 128, 8);
  EXPECT(ws == 2 * 4 * 8 * 128 * 4 + 256, "split workspace bytes %zu", ws);
  auto call = [&](void* w, size_t wb, int Hq, int Nq, int d, int splits) {
    return fa_fwd_splitkv(P, P, P, P, L, 2, Hq, 1, Nq, 4096, d, .1f, 1, splits, w, wb, nullptr);
  };
  EXPECT(call(P, ws, 4, 1, 128, 8) == FA_OK, "split valid");
  EXPECT(call(nullptr, ws, 4, 1, 128, 8) == FA_ERR_WORKSPACE, "split null ws");
  EXPECT(call(P, ws - 1, 4, 1, 128, 8) == FA_ERR_WORKSPACE, "split small ws");
  EXPECT(call(PU, ws, 4, 1, 128, 8) == FA_ERR_WORKSPACE, "split misaligned ws");
  EXPECT(call(P, ws, 4, 1, 128, -1) == FA_ERR_SPLITS, "split -1");
  EXPECT(call(P, ws, 4, 1, 128, 1025) == FA_ERR_SPLITS, "split 1025");
  EXPECT(fa_fwd_splitkv(P, P, P, P, L, 1, 1, 1, 1, 7, 128, .1f, 1, 8, P, 1 << 16, nullptr) ==
             FA_ERR_SPLITS, "more splits than keys");
  EXPECT(call(P, ws, 17, 1, 128, 8) == FA_ERR_SHAPE, "split rows");
  EXPECT(fa_fwd_splitkv(P, P, P, P, L, 1, 16, 1, 2, 4096, 128, .1f, 1, 8, P, 1 << 16, nullptr) ==
             FA_ERR_SHAPE, "split more than 16 rows");
  EXPECT(call(P, ws, 4, 1, 96, 8) == FA_ERR_HEAD_DIM, "split d");
  EXPECT(fa_fwd_splitkv(nullptr, P, P, P, L, 2, 4, 1, 1, 4096, 128, .1f, 1, 8, P, ws, nullptr) ==
             FA_ERR_NULL, "split null");
}

static void check_backward() {
  const float* L = (const float*)P;
  EXPECT(fa_bwd_workspace_bytes(2, 32, 8, 8192, 8192, 128) == 2u * 2 * 32 * 8192 * 4, "bwd ws");
  EXPECT(fa_bwd_workspace_bytes(1, 1, 1, 3, 3, 64) == 256, "bwd ws rounding");
  EXPECT(fa_bwd_workspace_bytes(1, 0, 1, 3, 3, 64) == 0, "bwd ws bad");
  const size_t ws = fa_bwd_workspace_bytes(1, 2, 1, 8, 8, 128);
  auto bwd = [&](const void* q, void* dv, void* w, size_t wb, int Hq, int Hkv, int d, float s) {
    return fa_bwd(q, P, P, P, P, L, P, P, dv, w, wb, 1, Hq, Hkv, 8, 8, d, s, 1, nullptr);
  };
  EXPECT(bwd(P, P, P, ws, 2, 1, 128, .1f) == FA_OK, "bwd valid");
  EXPECT(g_last_dvec == (const float*)P, "bwd workspace passed through");
  EXPECT(bwd(nullptr, P, P, ws, 2, 1, 128, .1f) == FA_ERR_NULL, "bwd null q");
  EXPECT(bwd(P, nullptr, P, ws, 2, 1, 128, .1f) == FA_ERR_NULL, "bwd null dv");
  EXPECT(bwd(P, P, nullptr, ws, 2, 1, 128, .1f) == FA_ERR_WORKSPACE, "bwd null ws");
  EXPECT(bwd(P, P, P, ws - 1, 2, 1, 128, .1f) == FA_ERR_WORKSPACE, "bwd small ws");
  EXPECT(bwd(P, P, PU, ws, 2, 1, 128, .1f) == FA_ERR_WORKSPACE, "bwd misaligned ws");
  EXPECT(bwd(PU, P, P, ws, 2, 1, 128, .1f) == FA_ERR_ALIGN, "bwd align");
  EXPECT(bwd(P, PU, P, ws, 2, 1, 128, .1f) == FA_ERR_ALIGN, "bwd align dv");
  EXPECT(bwd(P, P, P, ws, 3, 2, 128, .1f) == FA_ERR_HEADS, "bwd heads");
  EXPECT(bwd(P, P, P, ws, 2, 1, 80, .1f) == FA_ERR_HEAD_DIM, "bwd d");
  EXPECT(bwd(P, P, P, ws, 2, 1, 128, kNan) == FA_ERR_SCALE, "bwd scale");
  for (int stage : {-2, -1, 2, 7})
    EXPECT(fa_bwd_stage(stage, P, P, P, P, P, L, P, P, P, P, ws, 1, 2, 1, 8, 8, 128, .1f, 1,
                        nullptr) == FA_ERR_STAGE, "stage %d", stage);
  for (int stage : {0, 1})
    EXPECT(fa_bwd_stage(stage, P, P, P, P, P, L, P, P, P, P, ws, 1, 2, 1, 8, 8, 128, .1f, 1,
                        nullptr) == FA_OK, "stage %d valid", stage);
  g_launch_result = hipErrorInvalidValue;
  EXPECT(bwd(P, P, P, ws, 2, 1, 128, .1f) == FA_ERR_LAUNCH, "bwd launch err");
  g_launch_result = hipSuccess;

  // fa_bwd_noalloc: same checks, the row limit of its scratch, one symbol lookup per device
  auto na = [&](const void* q, int B, int Hq, int Hkv, int Nq, int d) {
    return fa_bwd_noalloc(q, P, P, P, P, L, P, P, P, B, Hq, Hkv, Nq, 8, d, .1f, 1, nullptr);
  };
  const int lookups = g_symbol_lookups;
  EXPECT(na(nullptr, 1, 2, 1, 8, 128) == FA_ERR_NULL, "noalloc null");
  EXPECT(na(PU, 1, 2, 1, 8, 128) == FA_ERR_ALIGN, "noalloc align");
  EXPECT(na(P, 1, 3, 2, 8, 128) == FA_ERR_HEADS, "noalloc heads");
  EXPECT(na(P, 1, 2, 1, 8, 96) == FA_ERR_HEAD_DIM, "noalloc d");
  EXPECT(na(P, 1, 1, 1, FA_BWD_NOALLOC_MAX_ROWS + 1, 64) == FA_ERR_SCRATCH, "noalloc rows");
  EXPECT(na(P, 2, 32, 8, FA_BWD_NOALLOC_MAX_ROWS / 64 + 1, 64) == FA_ERR_SCRATCH, "noalloc rows");
  EXPECT(g_symbol_lookups == lookups, "no HIP call before validation passes");
  g_get_device_result = hipErrorNoDevice;
  EXPECT(na(P, 1, 2, 1, 8, 128) == FA_ERR_LAUNCH, "noalloc without device");
  g_get_device_result = hipSuccess;
  EXPECT(na(P, 1, 1, 1, FA_BWD_NOALLOC_MAX_ROWS, 64) == FA_OK, "noalloc at the limit");
  EXPECT(g_last_dvec == g_scratch_stub, "noalloc passes the looked-up scratch address");
  EXPECT(na(P, 2, 32, 8, 8192, 128) == FA_OK, "noalloc GQA training shape");
  EXPECT(g_symbol_lookups == lookups + 1, "one lookup per device (%d)", g_symbol_lookups - lookups);
}

static void check_variants_and_probe() {
  float* L = (float*)P;
  for (int var : {-1, 4, 100})
    EXPECT(fa_fwd_variant(P, P, P, P, L, P, 1 << 16, 1, 2, 1, 8, 8, 64, .1f, 1, var, nullptr) ==
               FA_ERR_VARIANT, "variant %d", var);
  EXPECT(fa_fwd_variant_workspace_bytes(1, 2, 1, 8, 8, 64, 1) == 0, "variant 1 ws");
  const size_t ws = fa_fwd_variant_workspace_bytes(1, 2, 1, 300, 300, 64, 2);
  EXPECT(ws >= (size_t)1 * 2 * 3 * (128 * 64 + 512) * 4, "variant 2 ws %zu", ws);
  EXPECT(fa_fwd_variant(P, P, P, P, L, nullptr, 0, 1, 2, 1, 300, 300, 64, .1f, 1, 2, nullptr) ==
             FA_ERR_WORKSPACE, "variant 2 no ws");
  EXPECT(fa_fwd_variant(P, P, P, P, L, P, ws - 1, 1, 2, 1, 300, 300, 64, .1f, 1, 2, nullptr) ==
             FA_ERR_WORKSPACE, "variant 2 small ws");
  EXPECT(fa_fwd_variant(P, P, P, P, L, P, ws, 1, 2, 1, 300, 300, 256, .1f, 1, 1, nullptr) ==
             FA_ERR_HEAD_DIM, "variant d");
  for (int var : {0, 1, 3})
    EXPECT(fa_fwd_variant(P, P, P, P, L, nullptr, 0, 1, 2, 1, 300, 300, 64, .1f, 1, var,
                          nullptr) == FA_OK, "variant %d valid", var);
  EXPECT(fa_fwd_variant(P, P, P, P, L, P, ws, 1, 2, 1, 300, 300, 64, .1f, 1, 2, nullptr) == FA_OK,
         "variant 2 valid");
  EXPECT(fa_mfma_probe(nullptr, 1, 1, 0, nullptr) == FA_ERR_NULL, "probe null");
  EXPECT(fa_mfma_probe((float*)PU, 1, 1, 0, nullptr) == FA_ERR_ALIGN, "probe align");
  for (int b : {0, (1 << 20) + 1})
    EXPECT(fa_mfma_probe((float*)P, b, 1, 0, nullptr) == FA_ERR_SHAPE, "probe blocks");
  EXPECT(fa_mfma_probe((float*)P, 1, 1, 2, nullptr) == FA_ERR_SHAPE, "probe kind");
  EXPECT(fa_mfma_probe((float*)P, 4, 4, 1, nullptr) == FA_OK, "probe valid");
}

int main() {
  EXPECT(fa_version() == 10000, "version");
  for (int c = 1; c >= -13; --c) {
    const char* s = fa_status_string(c);
    EXPECT(s && std::strlen(s) > 0, "status %d", c);
    if (c <= 0) EXPECT(std::strncmp(s, "FA_", 3) == 0, "status %d named", c);
  }
  check_forwards();
  check_splitkv();
  check_backward();
  check_variants_and_probe();
  if (g_fail) return 1;
  std::printf("ok\n");
  return 0;
}
