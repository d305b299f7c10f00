// Forward attention, bf16: launches of the software-pipelined kernel in fwd_bf16.h
// (d = 64, and d = 128 for shorter sequences: 8-wave workgroups) and of the two-group
// kernel in fwd_pp.h (d = 256, and d = 128 for long sequences or, with GQA, from 2048
// rows), and the first-version comparison forms; small grids (the key-split form) and
// short key ranges (d = 64, and causal d = 128: 4-wave workgroups) go to the 128-row
// kernels of fwd_bf16_small.hip.
#include "fwd_bf16.h"
#include "fwd_pp.h"

namespace fa {
namespace {

#ifndef FWD_SMALL_GRID
#define FWD_SMALL_GRID 256
#endif
constexpr long long kSmallGrid = FWD_SMALL_GRID;
// query rows from which the d = 128 two-group kernel runs: head pairs causal (as 4-wave
// workgroups below kHp8MinRowsCausal), 64 rows of one head causal, either form non-causal
constexpr int kHpMinRowsCausal = 2048, kHp8MinRowsCausal = 8192, kRowsMinRowsCausal = 8192,
              kPpMinRowsNonCausal = 1024;
constexpr int kSmallKeys64 = 4096, kSmallKeys128 = 3072;

}  // namespace

hipError_t launch_fwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           uint16_t* o, float* lse, const AttnShape& s, hipStream_t st) {
  FwdParams p;
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.Hq = s.Hq; p.Hkv = s.Hkv; p.Nq = s.Nq; p.Nk = s.Nk; p.g = s.Hq / s.Hkv;
  p.causal_off = s.Nk - s.Nq;
  p.scale_log2 = s.scale * kLog2e;
  const bool c = s.causal != 0;
  // Grids too small to give every compute unit a 256-row workgroup (short sequences,
  // few heads) use 128-row workgroups instead: twice the workgroups, each less
  // efficient per unit of work, but no compute unit left idle. Each has 8 waves in two
  // groups that take half of the key tiles each (fwd_bf16.h, KS = 2), so every SIMD
  // holds two waves and a wave's chain of key tiles is half as long; against 4-wave
  // workgroups over all keys: B2 H16 N1024 d64 non-causal -14 %, B1 H8 N2048 d64 -22 %
  // (causal -27 %), d128 -11 % (causal -13 %), B2 H8 N1024 d128 causal -9 %. Causal
  // grids of exactly 256 such workgroups too (B1 H32 N2048 d128 -17 %, B2 H16 N2048 d64
  // -25 %; non-causal there +15 %, causal d128 at 384 or 512 +9 to +14 %).
  const long long wg256 = (long long)((s.Nq + 255) / 256) * s.Hq * s.B;
  if ((c ? wg256 <= kSmallGrid : wg256 < kSmallGrid) && (s.d == 64 || s.d == 128)) {
    return launch_fwd_bf16_small(p, s.B, s.d, c, true, st);
  }
  // d = 256 (fwd_pp.h): two waves per SIMD, each alternating a matrix phase and a
  // vector phase; measured 1.7x the one-wave-per-SIMD software-pipelined kernel (B2 H16
  // N4096 causal: 490 -> 285 us). Causal and on small grids as 4-wave workgroups, two per
  // compute unit (B2 H16 N4096 causal -1.5 to -3 %, B4 H16 N2048 -8 %, B1 H4 N1024
  // -23 %); non-causal on large grids as 8-wave workgroups whose two groups take turns
  // on the matrix cores (2 % faster there). At d <= 128 a key tile's softmax takes about
  // as long as its products, and the software-pipelined kernel below is 6-7 % faster.
  // Small grids: two such 4-wave groups in one workgroup, each over half of the key
  // tiles (fwd_pp.h KS = 2): B2 H8 N2048 causal -15 %, B1 Hq8 Hkv2 N4000 causal -18 %,
  // B1 H4 N1024 -10 %, B2 H8 N2048 non-causal -6 %.
  if (s.d == 256) {
    if (wg256 < kSmallGrid)
      return c ? run_pp<256, 32, true, 1, false, 4, 2>(p, s.B, st)
               : run_pp<256, 32, false, 1, false, 4, 2>(p, s.B, st);
    if (c) return run_pp<256, 32, true, 1, false, 4>(p, s.B, st);
    return run_pp<256, 32, false, 1, false, 8>(p, s.B, st);
  }
  // d = 128, long enough sequences: the two-group kernel with two 32-row query blocks
  // per wave (fwd_pp.h), so each K / V^T operand read from LDS feeds two products, when
  // it still gives every compute unit a workgroup.
  //  - an even number of query heads per kv-head: the two blocks are the same rows of
  //    two heads of one group (256-row workgroups). Time against the other kernels: B2
  //    Hq32 Hkv8 N8192 causal -8 % (-3.7 % against 64 consecutive rows), B4 Hq32 Hkv8
  //    N4096 causal -11 %, N3072 -7 %, non-causal N2048 -8.5 %, B8 Hq32 Hkv8 N1024
  //    non-causal -7.6 %. Causal below 8192 rows as one group of 4 waves (128 rows of
  //    each head, 80 KB of LDS, two workgroups per compute unit): against the 8-wave
  //    form B4 Hq32 Hkv8 N3072 -3 %, N4096 -1.8 %, B2 N6144 -0.4 %, but B2 N8192
  //    +1.8 % (and non-causal +1.5 to +2 %); B4 N2048 -1.4 % against the 32-row 4-wave
  //    kernel.
  //  - otherwise 64 consecutive rows of one head (512-row workgroups): B1 H8 N32768
  //    causal -8 %, B2 H32 N4096 and B1 H8 N16384 non-causal -9 %, B8 H32 N2048 and B16
  //    H32 N1024 non-causal -9 %, but B4 H32 N4096 causal +1 % (a 512-row workgroup walks
  //    the diagonal tiles for all of its rows, a larger share of the work there), so
  //    causal from 8192 rows only.
  const long long wghp = (long long)((s.Nq + 255) / 256) * (s.Hq / 2) * s.B;
  if (s.d == 128 && (s.Hq / s.Hkv) % 2 == 0 && s.Nq >= (c ? kHpMinRowsCausal : kPpMinRowsNonCausal) &&
      wghp >= kSmallGrid) {
    if (!c) return run_pp<128, 32, false, 2, true>(p, s.B, st);
    return s.Nq >= kHp8MinRowsCausal ? run_pp<128, 32, true, 2, true>(p, s.B, st)
                                     : run_pp<128, 32, true, 2, true, 4>(p, s.B, st);
  }
  const long long wg512 = (long long)((s.Nq + 511) / 512) * s.Hq * s.B;
  if (s.d == 128 && s.Nq >= (c ? kRowsMinRowsCausal : kPpMinRowsNonCausal) && wg512 >= kSmallGrid)
    return c ? run_pp<128, 32, true, 2>(p, s.B, st) : run_pp<128, 32, false, 2>(p, s.B, st);
  // For short key ranges the 4-wave kernel is also the faster one on large grids: two
  // of its 128-row workgroups share a compute unit (80 KB of LDS and 252 registers per
  // wave each), so one's start and end overlap the other's key loop. Measured against
  // the 8-wave kernel (B4 H32): d64 causal N2048 -11 %, N4096 -4 to -6 %, d64
  // non-causal N4096 -3.5 %, d128 causal N2048 -5 %, N3072 -3 %; but d128 causal N4096
  // +0-2 %, d128 non-causal N2048 +3.5 % and N4096 +14 %, N6144 d128 and N8192 d64
  // causal +2-3 %.
  if ((s.d == 64 && s.Nk <= kSmallKeys64) || (s.d == 128 && c && s.Nk <= kSmallKeys128))
    return launch_fwd_bf16_small(p, s.B, s.d, c, false, st);
  switch (s.d) {
#ifndef FWD_CFG128
#define FWD_CFG128 64, 8, 1
#endif
#ifndef FWD_CFG64
#define FWD_CFG64 64, 8, 1
#endif
    case 64: return c ? run<64, FWD_CFG64, true>(p, s.B, st) : run<64, FWD_CFG64, false>(p, s.B, st);
    case 128: return c ? run<128, FWD_CFG128, true>(p, s.B, st) : run<128, FWD_CFG128, false>(p, s.B, st);
    default: return hipErrorInvalidValue;
  }
}


hipError_t launch_fwd_bf16_variant(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   uint16_t* o, float* lse, const AttnShape& s, int variant,
                                   hipStream_t st) {
  FwdParams p;
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.Hq = s.Hq; p.Hkv = s.Hkv; p.Nq = s.Nq; p.Nk = s.Nk; p.g = s.Hq / s.Hkv;
  p.causal_off = s.Nk - s.Nq;
  p.scale_log2 = s.scale * kLog2e;
  const bool c = s.causal != 0;
  if (variant == 1) {
    switch (s.d) {
      case 64: return c ? run<64, 64, 8, 1, true, true>(p, s.B, st) : run<64, 64, 8, 1, false, true>(p, s.B, st);
      case 128: return c ? run<128, 64, 8, 1, true, true>(p, s.B, st) : run<128, 64, 8, 1, false, true>(p, s.B, st);
      default: return hipErrorInvalidValue;
    }
  }
  if (variant == 3) {
    switch (s.d) {
      case 64: return c ? run<64, 64, 8, 1, true, false, true>(p, s.B, st) : run<64, 64, 8, 1, false, false, true>(p, s.B, st);
      case 128: return c ? run<128, 64, 8, 1, true, false, true>(p, s.B, st) : run<128, 64, 8, 1, false, false, true>(p, s.B, st);
      default: return hipErrorInvalidValue;
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
