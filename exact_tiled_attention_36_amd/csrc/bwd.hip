// Backward attention by recomputation, bf16 in/out, fp32 accumulation, for gfx950.
//
// The forward pass keeps only the per-row statistics; the backward pass rebuilds
// every block of P from them instead of reading a stored N x N matrix
// ("FlashAttention" (ruizhehou.github.io), §二.3 recomputation; the statistics m and
// l are folded into lse = m + ln l, so P = exp(s - lse)). The pages give no formulas
// for the gradients; these kernels use the chain rule of softmax attention:
//     D_i  = sum_c dO_ic O_ic        (equals sum_j P_ij dP_ij)
//     dP   = dO V^T,  dS = P * (dP - D)
//     dV   = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K
// with dK, dV summed over the query heads that share a key/value head.
//
// Two kernels on one stream:
//  1. bwd_dq (bwd_dq.h; first): one workgroup per (batch, head, 128 queries: 4 waves of
//     32, or on small grids 8 waves in two groups that split the key tiles; d = 64 and
//     128 from bwd_dq_small.hip); Q and dO stay in registers, K/V tiles are triple
//     buffered in LDS; S^T and dP^T put one query per lane, so LSE and D are per-lane
//     scalars, and dQ^T += K^T dS^T reads K^T with LDS transpose loads. Its prologue
//     forms D_i from its rows of O and dO (dO is in registers already) and stores D
//     and LSE * log2(e) for the second kernel.
//  2. bwd_dkdv (bwd_dkdv.h; bwd_dkdv_rs.h at d = 256, 64 keys per workgroup, the
//     products of each 32 keys split between two waves): one workgroup per (batch,
//     kv-head, 128 keys); each wave
//     keeps 32 keys of K and V in registers and loops over the group's query heads and
//     the query blocks that can see its keys (diagonal blocks first, then the unmasked
//     ones block by block from the last down, all heads of the group per block, so the
//     group's waves share Q/dO tiles in L2), with Q/dO/LSE/D tiles triple buffered in
//     LDS.
//     S = Q K^T and dP = dO V^T come out with one key per lane, so P and dS (rounded
//     to bf16) feed dV^T += dO^T P and dK^T += Q^T dS directly as B operands; dO^T
//     and Q^T are read with LDS transpose loads.
// No atomics: every output element is written by exactly one workgroup, so results
// are bitwise reproducible.
#include "bwd_dq.h"
#include "bwd_dkdv_rs.h"

namespace fa {
namespace {

// dQ grids of at most this many 128-row workgroups (two per compute unit fill 512) run
// the key-split form (bwd_dq.h, KS = 2: 8 waves, two groups taking half of the key
// tiles each). Against the 4-wave form: B1 H8 N2048 d128 causal -11 % (128
// workgroups), B1 H16 -7 %, B4 H8 N1024 d64 causal -10 % (256), B1 H24 -14 % (384),
// B1 H32 N2048 -19 % (512); but B2 H24 N2048 +10 % (768) and +5 to +20 % at 1024.
constexpr long long kDqKeySplitMaxGrid = 512;

// stage 0: dQ (and D, LSE * log2(e) into the workspace); stage 1: dK, dV; stage -1: both.
template <int D, int BMQ, int BN, int NWQ, bool CAUSAL>
hipError_t run(const BwdParams& p, int B, int stage, hipStream_t st) {
  if (stage == -1 || stage == 0) {
    const int nqb = (p.Nq + 32 * NWQ - 1) / (32 * NWQ);
    const long long n = (long long)nqb * p.Hq * B;
    if (n > 0x7fffffffLL) return hipErrorInvalidValue;
    hipError_t e;
    if constexpr (NWQ == 4 && D <= 128) {
      e = launch_bwd_dq_small(p, nqb, (int)n, D, CAUSAL, n <= kDqKeySplitMaxGrid, st);
    } else {
      hipLaunchKernelGGL((bwd_dq_kernel<D, BN, NWQ, CAUSAL>), dim3((int)n), dim3(64 * NWQ), 0, st, p, nqb);
      e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
  }
  if (stage == -1 || stage == 1) {
    // Grids of at most 256 workgroups of 128 keys leave compute units idle (one
    // workgroup each, and under a causal mask the first keys' workgroups take twice the
    // average): there each workgroup takes 64 keys, its two wave pairs splitting every
    // query tile (d = 64, 128). At exactly 256: B2 Hq32 Hkv8 N2048 causal -20 %, B1
    // Hq32 Hkv8 N4096 -25 %; at 384 and 512 the 128-key form is mostly ahead.
    const long long wg128 = (long long)((p.Nk + 127) / 128) * p.Hkv * B;
    const bool split = BMQ == 64 && wg128 <= 256;
    const int bnk = split || D == 256 ? 64 : 128;
    const int nkb = (p.Nk + bnk - 1) / bnk;
    const long long n = (long long)nkb * p.Hkv * B;
    if (n > 0x7fffffffLL) return hipErrorInvalidValue;
    hipError_t e;
    if constexpr (D == 128 && BMQ == 64) {
      e = launch_bwd_dkdv_d128(p, nkb, (int)n, CAUSAL, split, st);
    } else if constexpr (BMQ == 64) {
      if (split)
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, BMQ, CAUSAL, true>), dim3((int)n), dim3(256), 0, st, p, nkb);
      else
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, BMQ, CAUSAL>), dim3((int)n), dim3(256), 0, st, p, nkb);
      e = hipGetLastError();
    } else {
      static_assert(D == 256, "32-query tiles are the d = 256 form");
      hipLaunchKernelGGL((bwd_dkdv_rs_kernel<CAUSAL>), dim3((int)n), dim3(256), 0, st, p, nkb);
      e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const uint16_t* o, const uint16_t* dO, const float* lse,
                      uint16_t* dq, uint16_t* dk, uint16_t* dv, float* dvec,
                      const AttnShape& s, int stage, hipStream_t st) {
  BwdParams p;
  p.lse2v = dvec + (size_t)s.B * s.Hq * s.Nq;
  p.q = q; p.k = k; p.v = v; p.o = o; p.dO = dO; p.lse = lse;
  p.dq = dq; p.dk = dk; p.dv = dv; p.dvec = dvec;
  p.Hq = s.Hq; p.Hkv = s.Hkv; p.Nq = s.Nq; p.Nk = s.Nk; p.g = s.Hq / s.Hkv;
  p.causal_off = s.Nk - s.Nq;
  p.scale = s.scale;
  p.scale_log2 = s.scale * kLog2e;
  const bool c = s.causal != 0;
  // dQ runs in 128-row workgroups of 4 waves at every head size: two of them share a
  // compute unit (61 KB of LDS and 254 registers per wave at d = 128), so one's start
  // and end overlap the other's key loop. Measured against 256-row workgroups of 8
  // waves: B2 Hq32 Hkv8 N8192 d128 causal -1.5 %, B4 H32 N4096 d128 causal -1 to -6 %,
  // N2048 -9 to -11 %, B4 H32 d64 causal N2048 -17 %, N4096 -10 %.
  switch (s.d) {
    case 64: return c ? run<64, 64, 32, 4, true>(p, s.B, stage, st) : run<64, 64, 32, 4, false>(p, s.B, stage, st);
    case 128: return c ? run<128, 64, 32, 4, true>(p, s.B, stage, st) : run<128, 64, 32, 4, false>(p, s.B, stage, st);
    case 256: return c ? run<256, 32, 32, 4, true>(p, s.B, stage, st) : run<256, 32, 32, 4, false>(p, s.B, stage, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
