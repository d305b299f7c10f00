// C-ABI entry points of libfa.so (declared and documented in include/fa.h).
// Every entry point validates its arguments on the host before touching the HIP
// runtime, then enqueues the kernels of kernels.h on the caller's stream.
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "fa.h"
#include "kernels.h"

namespace {

constexpr int kVersion = 10000;  // 1.0.0

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_bf16_dim(int d) { return d == 64 || d == 128 || d == 256; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int check_shape(int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || d <= 0) return FA_ERR_SHAPE;
  if (Hq % Hkv != 0) return FA_ERR_HEADS;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
  // Kernels index rows with 32-bit ints and elements with 64-bit offsets.
  const long long rows_q = (long long)B * Hq * Nq, rows_k = (long long)B * Hkv * Nk;
  if (rows_q > 0x7fffffffLL || rows_k > 0x7fffffffLL) return FA_ERR_TOO_LARGE;
  return FA_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH; }

fa::AttnShape shape(int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal) {
  fa::AttnShape s;
  s.B = B; s.Hq = Hq; s.Hkv = Hkv; s.Nq = Nq; s.Nk = Nk; s.d = d;
  s.scale = scale; s.causal = causal != 0;
  return s;
}

constexpr int kMaxSplits = 1024;
constexpr int kSplitMaxRows = 16;  // (Hq/Hkv) * Nq handled by one split workgroup

size_t splitkv_part_o_bytes(int B, int Hq, int Nq, int d, int splits) {
  return align256((size_t)B * Hq * Nq * splits * d * sizeof(float));
}
size_t splitkv_part_lse_bytes(int B, int Hq, int Nq, int splits) {
  return align256((size_t)B * Hq * Nq * splits * sizeof(float));
}

// Device-resident scratch of fa_bwd_noalloc: D_i and the log2-scaled lse of up to
// FA_BWD_NOALLOC_MAX_ROWS query rows (the workspace fa_bwd takes from its caller).
// Every GPU the library runs on holds its own copy until the process ends.
static __device__ __align__(256) float scratch[2 * (size_t)FA_BWD_NOALLOC_MAX_ROWS];

// Device address of `scratch` on each device, looked up once per device with that
// device current. In host code the array's name is only a host-side stand-in; every
// kernel argument uses the address kept here.
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
float* scratch_ptr[kMaxDevices] = {};

int scratch_on_current_device(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FA_ERR_LAUNCH;
    scratch_ptr[dev] = (float*)p;
  }
  *out = scratch_ptr[dev];
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_version(void) { return kVersion; }

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: a size is <= 0";
    case FA_ERR_HEADS: return "FA_ERR_HEADS: Hq is not a multiple of Hkv";
    case FA_ERR_HEAD_DIM: return "FA_ERR_HEAD_DIM: head dimension d not supported by this entry point";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: a tensor pointer is not 16-byte aligned";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace NULL or too small";
    case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH: the HIP runtime rejected a kernel launch";
    case FA_ERR_TOO_LARGE: return "FA_ERR_TOO_LARGE: problem exceeds the library's index range";
    case FA_ERR_SPLITS: return "FA_ERR_SPLITS: num_splits out of range";
    case FA_ERR_SCALE: return "FA_ERR_SCALE: scale (and every FP8 descale) must be finite and > 0";
    case FA_ERR_STAGE: return "FA_ERR_STAGE: backward stage must be 0 or 1";
    case FA_ERR_VARIANT: return "FA_ERR_VARIANT: forward variant must be 0, 1, 2 or 3";
    case FA_ERR_SCRATCH:
      return "FA_ERR_SCRATCH: B * Hq * Nq exceeds FA_BWD_NOALLOC_MAX_ROWS (fa_bwd_noalloc's "
             "fixed scratch); use fa_bwd with a workspace";
    default: return "unknown fa status code";
  }
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
           int Hkv, int Nq, int Nk, int d, float scale, int causal, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  int st = check_shape(B, Hq, Hkv, Nq, Nk, d, scale);
  if (st != FA_OK) return st;
  if (!supported_bf16_dim(d)) return FA_ERR_HEAD_DIM;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  return launch_status(fa::launch_fwd_bf16(
      (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse,
      shape(B, Hq, Hkv, Nq, Nk, d, scale, causal), (hipStream_t)stream));
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B,
               int Hq, int Hkv, int Nq, int Nk, int d, float scale, float descale_q,
               float descale_k, float descale_v, int causal, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  int st = check_shape(B, Hq, Hkv, Nq, Nk, d, scale);
  if (st != FA_OK) return st;
  for (float x : {descale_q, descale_k, descale_v})
    if (!(x > 0.f) || !isfinite(x)) return FA_ERR_SCALE;
  // the kernel folds scale * descale_q * descale_k into one float
  const float c = scale * descale_q * descale_k;
  if (!(c > 0.f) || !isfinite(c * 1.4426950408889634f)) return FA_ERR_SCALE;
  if (!supported_bf16_dim(d)) return FA_ERR_HEAD_DIM;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  return launch_status(fa::launch_fwd_fp8(
      (const uint8_t*)q, (const uint8_t*)k, (const uint8_t*)v, (uint16_t*)o, lse, descale_q,
      descale_k, descale_v, shape(B, Hq, Hkv, Nq, Nk, d, scale, causal), (hipStream_t)stream));
}

int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B,
               int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  int st = check_shape(B, Hq, Hkv, Nq, Nk, d, scale);
  if (st != FA_OK) return st;
  if (d % 4 != 0 || d > 256) return FA_ERR_HEAD_DIM;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  return launch_status(fa::launch_fwd_f32(q, k, v, o, lse,
                                          shape(B, Hq, Hkv, Nq, Nk, d, scale, causal),
                                          (hipStream_t)stream));
}

int fa_splitkv_default_splits(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || d <= 0 || Hq % Hkv) return 1;
  // About 512 chunk workgroups (two per compute unit), each at least 1024 keys long
  // with one query row per kv-head (vector chunk kernel) or 512 with several (matrix-
  // core chunk kernel). Measured at d = 128 over split counts 1-256 (MI355X): within
  // 5 % of the best count on eight decode shapes (B1-B64, 8-512 (batch, kv-head)
  // groups, 2048-65536 keys); against four workgroups per compute unit and 256 keys:
  // B8 H8 Nk32768 -2 %, B1 H8 Nk32768 -42 %, B1 Hq32 Hkv8 Nk65536 -16 %, B2 Hq64 Hkv8
  // Nk32768 -7 %, B16 Hq32 Hkv4 Nk8192 unchanged.
  const long long groups = (long long)B * Hkv;
  long long s = (512 + groups - 1) / groups;
  const long long min_chunk = (long long)(Hq / Hkv) * Nq <= 1 ? 1024 : 512;
  const long long by_len = Nk / min_chunk;
  if (s > by_len) s = by_len;
  if (s < 1) s = 1;
  if (s > kMaxSplits) s = kMaxSplits;
  return (int)s;
}

size_t fa_fwd_splitkv_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d,
                                      int num_splits) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || d <= 0) return 0;
  const int s = num_splits > 0 ? num_splits
                               : fa_splitkv_default_splits(B, Hq, Hkv, Nq, Nk, d);
  return splitkv_part_o_bytes(B, Hq, Nq, d, s) + splitkv_part_lse_bytes(B, Hq, Nq, s);
}

int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                   int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                   int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  int st = check_shape(B, Hq, Hkv, Nq, Nk, d, scale);
  if (st != FA_OK) return st;
  if (!supported_bf16_dim(d)) return FA_ERR_HEAD_DIM;
  if ((Hq / Hkv) * (long long)Nq > kSplitMaxRows) return FA_ERR_SHAPE;
  if (num_splits < 0 || num_splits > kMaxSplits) return FA_ERR_SPLITS;
  const int s = num_splits > 0 ? num_splits : fa_splitkv_default_splits(B, Hq, Hkv, Nq, Nk, d);
  if (s > Nk) return FA_ERR_SPLITS;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  const size_t need = fa_fwd_splitkv_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, s);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return FA_ERR_WORKSPACE;
  float* part_o = (float*)workspace;
  float* part_lse = (float*)((char*)workspace + splitkv_part_o_bytes(B, Hq, Nq, d, s));
  return launch_status(fa::launch_fwd_splitkv(
      (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse, part_o,
      part_lse, s, shape(B, Hq, Hkv, Nq, Nk, d, scale, causal), (hipStream_t)stream));
}

size_t fa_bwd_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || d <= 0) return 0;
  return align256(2 * (size_t)B * Hq * Nq * sizeof(float));
}

static int bwd_check(const void* q, const void* k, const void* v, const void* o,
                     const void* dO, const float* lse, void* dq, void* dk, void* dv, int B,
                     int Hq, int Hkv, int Nq, int Nk, int d, float scale) {
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
  int st = check_shape(B, Hq, Hkv, Nq, Nk, d, scale);
  if (st != FA_OK) return st;
  if (!supported_bf16_dim(d)) return FA_ERR_HEAD_DIM;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dO) ||
      !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return FA_ERR_ALIGN;
  return FA_OK;
}

static int bwd_common(const void* q, const void* k, const void* v, const void* o,
                      const void* dO, const float* lse, void* dq, void* dk, void* dv,
                      void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                      int Nq, int Nk, int d, float scale, int causal, int stage,
                      void* stream) {
  int st = bwd_check(q, k, v, o, dO, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, scale);
  if (st != FA_OK) return st;
  if (!workspace || !aligned16(workspace) ||
      workspace_bytes < fa_bwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, d))
    return FA_ERR_WORKSPACE;
  return launch_status(fa::launch_bwd(
      (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)o,
      (const uint16_t*)dO, lse, (uint16_t*)dq, (uint16_t*)dk, (uint16_t*)dv, (float*)workspace,
      shape(B, Hq, Hkv, Nq, Nk, d, scale, causal), stage, (hipStream_t)stream));
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
           const float* lse, void* dq, void* dk, void* dv, void* workspace,
           size_t workspace_bytes, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
           int causal, void* stream) {
  return bwd_common(q, k, v, o, dO, lse, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv,
                    Nq, Nk, d, scale, causal, -1, stream);
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                   const void* dO, const float* lse, void* dq, void* dk, void* dv, int B,
                   int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                   void* stream) {
  int st = bwd_check(q, k, v, o, dO, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, scale);
  if (st != FA_OK) return st;
  if ((long long)B * Hq * Nq > FA_BWD_NOALLOC_MAX_ROWS) return FA_ERR_SCRATCH;
  float* ws = nullptr;
  st = scratch_on_current_device(&ws);
  if (st != FA_OK) return st;
  // Nothing in the scratch needs clearing: the dQ kernel writes D and the scaled lse of
  // every row before the dK/dV kernel, queued after it on the same stream, reads them.
  return launch_status(fa::launch_bwd(
      (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)o,
      (const uint16_t*)dO, lse, (uint16_t*)dq, (uint16_t*)dk, (uint16_t*)dv, ws,
      shape(B, Hq, Hkv, Nq, Nk, d, scale, causal), -1, (hipStream_t)stream));
}

int fa_bwd_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                 const void* dO, const float* lse, void* dq, void* dk, void* dv,
                 void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int Nq,
                 int Nk, int d, float scale, int causal, void* stream) {
  if (stage < 0 || stage > 1) return FA_ERR_STAGE;
  return bwd_common(q, k, v, o, dO, lse, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv,
                    Nq, Nk, d, scale, causal, stage, stream);
}

size_t fa_fwd_variant_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d,
                                      int variant) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || d <= 0) return 0;
  if (variant != 2) return 0;
  return align256(fa::fwd_v1_workspace_floats(shape(B, Hq, Hkv, Nq, Nk, d, 1.f, 0)) *
                  sizeof(float));
}

int fa_fwd_variant(const void* q, const void* k, const void* v, void* o, float* lse,
                   void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int Nq,
                   int Nk, int d, float scale, int causal, int variant, void* stream) {
  if (variant < 0 || variant > 3) return FA_ERR_VARIANT;
  if (variant == 0) return fa_fwd(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, stream);
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  int st = check_shape(B, Hq, Hkv, Nq, Nk, d, scale);
  if (st != FA_OK) return st;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  const fa::AttnShape s = shape(B, Hq, Hkv, Nq, Nk, d, scale, causal);
  if (variant == 1 || variant == 3)
    return launch_status(fa::launch_fwd_bf16_variant((const uint16_t*)q, (const uint16_t*)k,
                                                     (const uint16_t*)v, (uint16_t*)o, lse, s,
                                                     variant, (hipStream_t)stream));
  const size_t need = fa_fwd_variant_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, variant);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return FA_ERR_WORKSPACE;
  return launch_status(fa::launch_fwd_v1((const uint16_t*)q, (const uint16_t*)k,
                                         (const uint16_t*)v, (uint16_t*)o, lse,
                                         (float*)workspace, s, (hipStream_t)stream));
}

int fa_mfma_probe(float* out, int blocks, int iters, int kind, void* stream) {
  if (!out) return FA_ERR_NULL;
  if (!aligned16(out)) return FA_ERR_ALIGN;
  if (blocks < 1 || blocks > (1 << 20) || iters < 1 || iters > (1 << 20) ||
      (kind != 0 && kind != 1))
    return FA_ERR_SHAPE;
  return launch_status(fa::launch_mfma_probe(out, blocks, iters, kind, (hipStream_t)stream));
}

}  // extern "C"
