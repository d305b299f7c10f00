/*
 * fa.h — C ABI of the exact tiled attention library (libfa.so), MI355X / gfx950.
 *
 * What is computed. For every batch b and query head h, with key/value head
 * kvh = h / (Hq / Hkv):
 *     s_ij = scale * q_i . k_j              (scores; the pages' value of scale is 1/sqrt(d))
 *     p_ij = exp(s_ij - lse_i)              (row softmax of the visible scores)
 *     lse_i = log(sum_j exp(s_ij))          (natural log, of the scaled scores)
 *     o_i   = sum_j p_ij v_j
 * ("FlashAttention" (ruizhehou.github.io), §一: scores Q K^T / sqrt(d), softmax,
 * times V; FlashAttention1 article (gitcode.csdn.net), §一: the same formula.)
 * The forward pass forms the scores tile by tile with online softmax — running row
 * max m and row sum l, rescale by exp(m_old - m_new), one division at the end — so
 * no N x N matrix is ever written to memory ("FlashAttention" (ruizhehou.github.io),
 * §二.1 tiling, §二.2 online softmax, §四.1 deferred normalisation). It keeps one
 * float per row, lse = m + ln(l), for the backward pass, which rebuilds P from it
 * (§二.3 recomputation).
 *
 * Causal masking (causal != 0) is aligned to the bottom-right corner: query row i
 * sees key j iff j <= i + (Nk - Nq). With Nq == Nk this is the lower triangle; with
 * Nq == 1 (decode) the row sees every key. A row that sees no key (only possible
 * when Nq > Nk) gets o = 0 and lse = -inf. Grouped/multi-query attention
 * ("FlashAttention" (newton.com.tw wiki), 發展歷程, FlashAttention-2 paragraph):
 * Hq must be a multiple of Hkv; query head h uses key/value head h / (Hq / Hkv).
 *
 * Layouts. All tensors are dense and row-major with the head dimension fastest:
 *     q, o, dO, dq : [B, Hq,  Nq, d]
 *     k, v, dk, dv : [B, Hkv, Nk, d]
 *     lse          : [B, Hq,  Nq]   float32
 * bf16 entry points take IEEE bfloat16 bit patterns (2 bytes per element);
 * fa_fwd_f32 takes float32. Every tensor pointer must be 16-byte aligned.
 *
 * Ownership and errors. Pointers are device pointers owned by the caller; the
 * library keeps no pointer after a call returns and allocates nothing. Outputs are
 * fully overwritten (no zeroing needed). Calls are asynchronous: work is enqueued
 * on `stream` (a hipStream_t; NULL means the default stream) and the library never
 * synchronises. Arguments are validated before any HIP call; on a bad argument the
 * call returns a negative FA_ERR_* code and enqueues nothing. FA_ERR_LAUNCH means a
 * kernel launch was rejected by the runtime. fa_status_string() names every code.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,       /* a required pointer is NULL                          */
  FA_ERR_SHAPE = -2,      /* a size is <= 0 (Nk may not be 0 either)             */
  FA_ERR_HEADS = -3,      /* Hq is not a multiple of Hkv                         */
  FA_ERR_HEAD_DIM = -4,   /* d not supported by this entry point                 */
  FA_ERR_ALIGN = -5,      /* a tensor pointer is not 16-byte aligned             */
  FA_ERR_WORKSPACE = -6,  /* workspace NULL or smaller than the size asked for   */
  FA_ERR_LAUNCH = -7,     /* the HIP runtime rejected a kernel launch            */
  FA_ERR_TOO_LARGE = -8,  /* an index would overflow 32/64-bit addressing limits */
  FA_ERR_SPLITS = -9,     /* num_splits out of range                             */
  FA_ERR_SCALE = -10,     /* scale (or an FP8 descale) is not a finite number > 0 */
  FA_ERR_STAGE = -11,     /* fa_bwd_stage: stage not in {0, 1}                   */
  FA_ERR_VARIANT = -12,   /* fa_fwd_variant: variant not in {0, 1, 2, 3}         */
  FA_ERR_SCRATCH = -13    /* fa_bwd_noalloc: B * Hq * Nq > FA_BWD_NOALLOC_MAX_ROWS */
};

/* Largest B * Hq * Nq that fa_bwd_noalloc accepts (its scratch: 8 MiB per GPU). */
#define FA_BWD_NOALLOC_MAX_ROWS 1048576

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int fa_version(void);

/* Human-readable name of a status code (static string, never NULL). */
const char* fa_status_string(int status);

/*
 * Forward pass, bfloat16 inputs and output, float32 accumulation.
 * Writes o (bf16) and lse (float32). d must be 64, 128 or 256.
 * Work is gridded over (batch, head, block of query rows): the sequence-dimension
 * parallelism of "FlashAttention" (ruizhehou.github.io), §四.2. Causal calls skip
 * key tiles that lie wholly above the diagonal.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
           void* stream);

/*
 * Forward pass, float32 inputs and output, float32 arithmetic throughout.
 * Same contract as fa_fwd; d must be a multiple of 4 in [4, 256].
 */
int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
               int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
               void* stream);

/*
 * Forward pass with FP8 inputs: q, k, v hold OCP E4M3 bytes (1 sign, 4 exponent bits
 * with bias 7, 3 mantissa bits; no infinities; 0x7f and 0xff are NaN; largest finite
 * value 448) with one scale per tensor, so the attention computed is that of
 *     q = descale_q * Q8,  k = descale_k * K8,  v = descale_v * V8
 * with the given `scale` on the scores, exactly as fa_fwd defines it. This is the
 * low-precision forward the wiki lists for the third version ("FlashAttention"
 * (newton.com.tw), 發展歷程); the pages do not give its scaling recipe, so the plain
 * per-tensor form is used. Both products run on FP8 matrix instructions with fp32
 * accumulation; the softmax weights are rounded to E4M3 (nearest even) before the
 * product with V: for a row i and column c, |o_ic - exact| <= sum_j |P8_ij - P_ij| |v_jc|,
 * where the weight's rounding error |P8 - P| is at most max(P / 16, 2^-10 P_max_i).
 * The FP8 matrix instruction also sums its products with less than float32 accuracy
 * (measured: up to about 2^-15 of sum_d |q_d k_d| per score), which moves scores, lse
 * and weights slightly. lse is the float32 log-sum-exp of the unrounded weights, o is
 * bf16. Output layouts, alignment, ownership and errors as
 * fa_fwd (layouts count elements: q/k/v rows are d bytes); d must be 64, 128 or 256.
 * FA_ERR_SCALE if a descale or scale * descale_q * descale_k * log2(e) is not a finite
 * number > 0. NaN codes in the inputs propagate to the outputs of the rows they reach.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, float descale_q,
               float descale_k, float descale_v, int causal, void* stream);

/*
 * Split-KV forward for short query blocks (decode). Same result and layouts as
 * fa_fwd, but the keys of every (batch, kv-head) are cut into num_splits chunks that
 * run in separate workgroups; each chunk leaves a normalised partial output and its
 * log-sum-exp in `workspace`, and a second kernel merges the chunks by the online-
 * softmax rescale rule ("FlashAttention" (ruizhehou.github.io), §二.2, applied to
 * whole chunks). This fills the GPU when B * Hq * Nq is small and Nk is long.
 * Requires (Hq / Hkv) * Nq <= 16 and d in {64, 128, 256}. num_splits in
 * [1, 1024]; pass 0 to let the library choose (fa_splitkv_default_splits).
 * workspace must hold fa_fwd_splitkv_workspace_bytes(...) bytes (16-byte aligned,
 * contents ignored on entry).
 */
int fa_splitkv_default_splits(int B, int Hq, int Hkv, int Nq, int Nk, int d);
size_t fa_fwd_splitkv_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d,
                                      int num_splits);
int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                   int causal, int num_splits, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * Backward pass by recomputation ("FlashAttention" (ruizhehou.github.io), §二.3):
 * from q, k, v, the forward's o and lse, and the upstream gradient dO, rebuild each
 * block of P = exp(s - lse) and write dq, dk, dv (bf16, same layouts as q, k, v).
 * The chain rule used (the pages give no backward formulas): D_i = sum_c dO_ic o_ic,
 * dP = dO V^T, dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO,
 * with dK and dV summed over the query heads that share a kv-head.
 * workspace must hold fa_bwd_workspace_bytes(...) bytes (16-byte aligned; contents
 * ignored on entry; it receives D_i and a log2-scaled copy of lse). d must be 64,
 * 128 or 256.
 */
size_t fa_bwd_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d);
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
           const float* lse, void* dq, void* dk, void* dv, void* workspace,
           size_t workspace_bytes, int B, int Hq, int Hkv, int Nq, int Nk, int d,
           float scale, int causal, void* stream);

/*
 * fa_bwd without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation). Same arguments, results and errors as fa_bwd minus the workspace; the
 * call allocates nothing (no hipMalloc, hipFree or allocating library routine). D_i
 * and the log2-scaled lse live in a fixed device array of the library instead, 8 MiB
 * on every GPU it runs on, held until the process ends: B * Hq * Nq must not exceed
 * FA_BWD_NOALLOC_MAX_ROWS, else FA_ERR_SCRATCH (nothing is enqueued). The array's
 * address on the current device is looked up on the first call there (a HIP query,
 * not an allocation). `stream` must belong to the current device. All calls on one GPU
 * share that array and it keeps the last call's contents (nothing in it needs to start
 * at zero): calls that overlap in time on one GPU (different streams, or another
 * thread) race on it and must be ordered by the caller.
 */
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                   const void* dO, const float* lse, void* dq, void* dk, void* dv, int B,
                   int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                   void* stream);

/*
 * One stage of fa_bwd, same arguments plus `stage`, for callers that schedule or
 * time the two kernels separately. fa_bwd == stage 0, then 1 on one stream.
 *   stage 0: dq, and D_i = sum_c dO_ic o_ic and a log2-scaled copy of lse into the
 *            workspace (must run first);
 *   stage 1: dk and dv (reads both from the workspace).
 * Returns FA_ERR_STAGE for other values.
 */
int fa_bwd_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                 const void* dO, const float* lse, void* dq, void* dk, void* dv,
                 void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int Nq,
                 int Nk, int d, float scale, int causal, void* stream);

/*
 * Forward-pass variants for the comparison of the first and second versions of the
 * method ("FlashAttention" (ruizhehou.github.io): §二.2 and §三 for the first, §四.1 and
 * §四.2 for what the second changes). All three return the same O (bf16) and lse
 * (float32) as fa_fwd, up to rounding; only how the work is organised differs:
 *   variant 0: fa_fwd itself (deferred normalisation, grid over (batch, head, row
 *              block)); workspace unused, may be NULL.
 *   variant 1: fa_fwd's grid and pipeline, but O renormalised after every key block
 *              (the first version's update, §二.2): isolates the cost of the extra
 *              rescaling the second version removes. workspace unused.
 *   variant 2: the first version's loop order: one workgroup per (batch, head), K/V
 *              blocks in the outer loop, 128-row Q blocks in the inner loop, O, m and
 *              l read from and written back to `workspace` (fp32) for every pair of
 *              blocks, then a final pass writes o and lse.
 *   variant 3: fa_fwd with every eighth exponential computed by a polynomial on the
 *              FMA units (range reduction to [-1/2, 1/2], degree-3 minimax, relative
 *              error < 1e-4) instead of the transcendental unit: the partial software
 *              exponential the wiki names for the fourth version ("FlashAttention"
 *              (newton.com.tw), 核心技術). workspace unused.
 * Variants 1 to 3 take d in {64, 128} (FA_ERR_HEAD_DIM otherwise). Other arguments,
 * layouts, alignment and errors as fa_fwd; workspace must hold
 * fa_fwd_variant_workspace_bytes(...) bytes, 16-byte aligned (FA_ERR_WORKSPACE), and
 * its contents need no initialisation. Unknown variant: FA_ERR_VARIANT.
 */
size_t fa_fwd_variant_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d,
                                      int variant);
int fa_fwd_variant(const void* q, const void* k, const void* v, void* o, float* lse,
                   void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int Nq,
                   int Nk, int d, float scale, int causal, int variant, void* stream);

/*
 * fa_mfma_probe — measurement helper (not part of the attention computation): the
 * sustained rate of the bf16 matrix instruction the kernels use
 * (v_mfma_f32_32x32x16_bf16), so that a kernel's achieved TFLOP/s can be read
 * against what the matrix cores deliver at the clock the chip actually runs.
 * Launches `blocks` workgroups of 256 threads; every wave runs iters x 16 products
 * (32*32*16*2 flop each) on operands held in registers: kind 0 fills them with
 * zeros, kind 1 with bf16 values drawn from an approximately standard normal
 * distribution (the attention workloads' input distribution; the chip's clock under
 * matrix load depends on the operand bits). Total work: blocks * 4 * iters * 16 *
 * 32768 flop; the caller times the call (e.g. with events on `stream`).
 * out: device buffer of blocks * 256 floats (written, values meaningless), 16-byte
 * aligned. Errors: FA_ERR_NULL, FA_ERR_ALIGN, FA_ERR_SHAPE (blocks not in
 * [1, 1 << 20], iters not in [1, 1 << 20], kind not 0 or 1), FA_ERR_LAUNCH.
 */
int fa_mfma_probe(float* out, int blocks, int iters, int kind, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
