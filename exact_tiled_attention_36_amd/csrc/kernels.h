// Internal launch interface between the C-ABI layer (fa_api.hip) and the kernels.
// Shapes have been validated by the caller; these functions only enqueue work.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct AttnShape {
  int B, Hq, Hkv, Nq, Nk, d;
  float scale;
  int causal;
};

// Forward, bf16 in/out (d in {64,128,256}).
hipError_t launch_fwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           uint16_t* o, float* lse, const AttnShape& s, hipStream_t st);

// Ablation forwards (d in {64,128}), same outputs as launch_fwd_bf16:
// variant 1: production grid, O renormalised after every key block;
// variant 3: production kernel with every eighth exponential computed in software;
// v1: K/V-block outer loop, Q-block inner loop, one workgroup per (batch, head), with
// an fp32 workspace of fwd_v1_workspace_floats(s) floats.
hipError_t launch_fwd_bf16_variant(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   uint16_t* o, float* lse, const AttnShape& s, int variant,
                                   hipStream_t st);
size_t fwd_v1_workspace_floats(const AttnShape& s);
hipError_t launch_fwd_v1(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                         float* lse, float* ws, const AttnShape& s, hipStream_t st);

// Forward, FP8 E4M3 (OCP) q/k/v bytes with per-tensor descales, bf16 o, fp32 lse
// (d in {64,128,256}).
hipError_t launch_fwd_fp8(const uint8_t* q, const uint8_t* k, const uint8_t* v, uint16_t* o,
                          float* lse, float descale_q, float descale_k, float descale_v,
                          const AttnShape& s, hipStream_t st);

// Forward, fp32 in/out (d % 4 == 0, d <= 256).
hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o,
                          float* lse, const AttnShape& s, hipStream_t st);

// Split-KV forward + merge. `part_o` [B,Hq,Nq,splits,d] fp32, `part_lse`
// [B,Hq,Nq,splits] fp32.
hipError_t launch_fwd_splitkv(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              uint16_t* o, float* lse, float* part_o, float* part_lse,
                              int splits, const AttnShape& s, hipStream_t st);

// Backward. `dvec` is fp32 scratch of 2 * B*Hq*Nq floats: D_i = rowsum(dO * O), then
// the log2-domain LSE used by the recompute.
// stage: -1 all, 0 D preprocess, 1 dK/dV, 2 dQ.
hipError_t launch_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const uint16_t* o, const uint16_t* dO, const float* lse,
                      uint16_t* dq, uint16_t* dk, uint16_t* dv, float* dvec,
                      const AttnShape& s, int stage, hipStream_t st);

// Matrix-core rate probe: `blocks` workgroups of 256 threads, each wave running
// iters x 16 bf16 32x32x16 products on register operands (kind 0 zeros, 1 normal-like
// bf16); one float per thread is written to out (blocks * 256 floats).
hipError_t launch_mfma_probe(float* out, int blocks, int iters, int kind, hipStream_t st);

}  // namespace fa
