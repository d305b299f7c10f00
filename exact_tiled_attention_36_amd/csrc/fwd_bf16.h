// Forward attention, bf16 inputs, fp32 accumulation, for gfx950.
//
// The method ("FlashAttention" (ruizhehou.github.io)): Q is cut into row blocks
// (outer loop) and K/V into column blocks (inner loop), §二.1 and §三; each block of
// scores updates a running row max m and row sum l with the rescale factor
// exp(m_old - m_new), §二.2; the output accumulator stays unnormalised and is divided
// by l once after the last block, §四.1 (the FlashAttention-2 form); blocks of one
// head's rows run in separate workgroups, §四.2.
//
// MI355X mapping:
//  * one workgroup = NW waves x 32 query rows; wave w owns rows 32w..32w+31 for the
//    whole loop, so m, l and the output never need a cross-wave reduce.
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: K (A operand) comes from LDS with
//    16-byte reads, Q^T (B operand) sits in registers for the whole kernel. In the
//    result each lane holds one query (its column) and 16 of the 32 keys of a block,
//    so the row max/sum are in-lane reductions plus one v_permlane32_swap.
//  * O^T += V^T P^T: the exponentiated scores, rounded to bf16, are already laid out
//    as the B operand; V^T (A operand) is read from V's natural [key][d] LDS tile
//    with ds_read_b64_tr_b16.
//  * scores are scaled into the base-2 domain (scale * log2 e folded into one FMA)
//    and exponentiated with v_exp_f32.
//  * lazy rescale: the exponent base m of a wave moves only when some row sees a
//    score more than kRescaleSlack (log2 units) above it; otherwise weights up to
//    2^kRescaleSlack accumulate against the stale base. O / l and lse = m + log l use
//    the same base, so the result is unchanged, and the rescale of O is a rare branch.
//  * software pipeline, one barrier per key tile t:
//      region A: O += V_{t-1}^T P_{t-1} (matrix)  with  row max of S_t (vector)
//      [rare branch: rescale O]
//      region B: S_{t+1} = K_{t+1} Q^T (matrix)  with  exp / row sum of S_t (vector)
//    so each wave's vector work runs under its own matrix instructions. K runs two
//    tiles ahead of V in the LDS buffers.
//  * tiles that no row of the workgroup needs masked for (causal diagonal, key tail)
//    run in a loop without mask code; the rest in a masked loop.
//  * grid: one workgroup per (batch, head, row block). Non-causal ids are remapped so
//    consecutive ids stay on one XCD (one L2); causal grids follow causal_order: the
//    longest row blocks first, balanced over the 8 XCDs, two heads interleaved per
//    XCD.
//
// This header holds the kernel and its launch template; fwd_bf16.hip launches it
// (8-wave workgroups, d = 64 and 128; d = 256 goes to fwd_pp.h) and
// fwd_bf16_small.hip launches the 128-row forms (small grids: 8 waves splitting the
// keys; short key ranges: 4 waves, two workgroups per compute unit) with a compiler
// option of their own.
#pragma once
#include "common.h"
#include "kernels.h"

namespace fa {

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int Hq, Hkv, Nq, Nk, g, nqb, causal_off;
  float scale_log2;
};

// 128-row forward, d = 64 or 128 (fwd_bf16_small.hip): 4-wave workgroups, or with
// key_split 8-wave workgroups whose two halves take half of the key tiles each.
hipError_t launch_fwd_bf16_small(FwdParams p, long long B, int d, bool causal, bool key_split,
                                 hipStream_t st);

namespace {

// Headroom (in log2 units) the running max may lag behind the true row max before
// the accumulators are rescaled: weights stay below 2^8, far inside fp32/bf16 range.
constexpr float kRescaleSlack = 8.f;

template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

// One workgroup = NW waves; wave w owns QS blocks of 32 query rows (BM = 32*QS*NW
// rows per workgroup). Every K operand and every V^T operand read from LDS feeds the
// QS blocks, so LDS reads per matrix op fall as 1/QS.
// RENORM (ablation only, not the production path): the FlashAttention-1 update of
// "FlashAttention" (ruizhehou.github.io) §二.2, which keeps O normalised after every
// key block: the running max is exact (no slack), and each tile scales O by
// alpha * l_old / l_new and P by 1 / l_new before the product, so the epilogue does
// not divide. Same grid and pipeline as the deferred (§四.1) form, so timing the two
// isolates the cost of renormalising every block.
// POLY (ablation only): every eighth weight 2^x is computed by poly_exp2 on the FMA
// units instead of v_exp_f32, the partial software exponential that the wiki lists
// for FlashAttention-4 (核心技術), to move work off the transcendental unit.
// KS = 2 (grids too small to fill the GPU): the NW waves form two groups
// that own the same rows and take one half of the key tiles each, in LDS buffers of
// their own (the key/value-block split of §四.3 inside one workgroup); at the end the
// second group hands its O, running max and row sums to the first through LDS, which
// merges them with the rescale rule of §二.2 before the one division. Each wave's
// chain of dependent key tiles is half as long and every SIMD holds two waves.
template <int D, int BN, int NW, int QS, bool CAUSAL, bool RENORM = false, bool POLY = false,
          int KS = 1>
__global__ __launch_bounds__(64 * NW, 1) void fwd_bf16_kernel(FwdParams p) {
  using TL = TileLayout<D>;
  static_assert(KS == 1 || (KS == 2 && QS == 1 && !RENORM && NW == 8),
                "the key split is a one-block form of 8 waves");
  constexpr int WG = NW / KS;    // waves per key group
  constexpr int RPW = 32 * QS;   // query rows per wave
  constexpr int BM = RPW * WG;   // query rows per workgroup
  constexpr int TILE = TL::elems(BN);
  constexpr int NKB = BN / 32;   // 32-key blocks per tile
  constexpr int NDC = D / 16;    // 16-wide chunks of d (reduction of S)
  constexpr int NCB = D / 32;    // 32-wide column blocks of O
  static_assert(TL::shifts_ok(BN), "LDS reads add row offsets as constants");

  __shared__ __attribute__((aligned(16))) uint16_t smem[KS * 4 * TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wall = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ks = KS == 1 ? 0 : wall / WG;  // key group (uniform)
  const int wu = KS == 1 ? wall : wall % WG;  // wave within its group
  const int l32 = lane & 31, hi = lane >> 5;

  int L = xcd_remap(blockIdx.x, gridDim.x);
  int qb, bh;
  if (CAUSAL) {
    causal_order<2>(blockIdx.x, gridDim.x, p.nqb, bh, qb);
  } else {
    qb = L % p.nqb;
    bh = L / p.nqb;
  }
  const int h = bh % p.Hq, b = bh / p.Hq;
  const int kvh = h / p.g;
  const int q0 = qb * BM;
  const int w0 = q0 + RPW * wu;  // first query row of this wave

  const uint16_t* Qg = p.q + (size_t)(b * p.Hq + h) * p.Nq * D;
  const uint16_t* Kg = p.k + (size_t)(b * p.Hkv + kvh) * p.Nk * D;
  const uint16_t* Vg = p.v + (size_t)(b * p.Hkv + kvh) * p.Nk * D;

  bf16x8_t qreg[QS][NDC];
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    const int qrow = w0 + 32 * qs + l32;
    const int qr = qrow < p.Nq ? qrow : p.Nq - 1;
    const u32x4_t* src = (const u32x4_t*)(Qg + (size_t)qr * D + 8 * hi);
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) qreg[qs][dc] = __builtin_bit_cast(bf16x8_t, src[2 * dc]);
  }
  // nothing may be outstanding in the loops below except the tile copies they issue
  wait_vmem();

  int kend = p.Nk;
  if (CAUSAL) {
    const int lim = q0 + BM + p.causal_off;  // keys < lim may be visible to some row
    kend = lim < kend ? lim : kend;
  }
  const int ntiles_all = kend > 0 ? (kend + BN - 1) / BN : 0;
  // tiles [0, tfull) are wholly visible to every row of the workgroup
  int tfull_all = p.Nk / BN;
  if (CAUSAL) {
    const int lim = q0 + p.causal_off + 1;  // keys < lim are visible to every row
    tfull_all = min(tfull_all, lim > 0 ? lim / BN : 0);
  }
  tfull_all = min(tfull_all, ntiles_all);
  // KS = 2: group g takes global tiles [g*nh, g*nh + nh) as its local tiles 0..nh-1 (the
  // second group's last one may lie past the keys: copied from the last key row and
  // masked away). Both groups run the same steps (their barriers are shared): the
  // unmasked loop covers the local tiles unmasked in both groups.
  const int ntiles = KS == 1 ? ntiles_all : (ntiles_all + 1) / 2;
  const int t0 = ks * ntiles;  // global index of local tile 0
  const int tfull = KS == 1 ? tfull_all : min(min(tfull_all, ntiles), max(tfull_all - ntiles, 0));

  f32x16_t oacc[QS][NCB];
  float m[QS], lsum[QS], m_use[QS], alpha[QS];
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) oacc[qs][cb] = zero16();
    m[qs] = -INFINITY;
    lsum[qs] = 0.f;
    m_use[qs] = 0.f;
    alpha[qs] = 1.f;
  }
  const float c2 = p.scale_log2;

  auto Kb = [&](int i) FA_INLINE { return smem + (4 * ks + (i & 1)) * TILE; };
  auto Vb = [&](int i) FA_INLINE { return smem + (4 * ks + 2 + (i & 1)) * TILE; };
  // Rows past the last key re-read the last key row: always finite, and masked to
  // zero weight before they can contribute (tiles past the end are never used).
  const uint32_t lane_off = 4u * lane;
  // local tile t of this wave's key group (each group copies its own tiles)
  auto load = [&](const uint16_t* G, int tl, uint16_t* dst) FA_INLINE {
    const int t = t0 + tl;
    if constexpr (D <= 128) {
      if ((t + 1) * BN <= p.Nk) {  // whole tile present: scalar-addressed copies
        // the 4-wave and non-causal kernels keep too many scalar values for the
        // per-piece LDS addresses the compiler would hoist (they spilled into vector
        // lanes: small-grid d = 128 forward 10 % faster without); the causal 8-wave
        // kernels did not spill and keep the hoisted form (1-3 % faster there)
        if constexpr (CAUSAL && NW == 8 && KS == 1)
          tile_load_full<D, BN, WG>(G, t * BN, dst, wu, lane_off);
        else
          tile_load_full_o<D, BN, WG>(G, t * BN, dst, wu, lane_off);
        return;
      }
    }
    tile_load_async<D, BN, WG>(G, t * BN, p.Nk, dst, wu, lane);
  };

  // per-lane LDS byte offsets inside a tile: K operand rows, V^T transposed reads
  // (source lane j = lane % 16 points at key row 4*hi + j/4, column 16*((lane/16)%2) +
  // 4*(j%4), see common.h)
  const int tr_row = 4 * hi + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const uint32_t srow = 2 * (TL::row(l32) + 8 * hi);
  const uint32_t trow = 2 * (TL::row(tr_row) + tr_col);

  // S^T = K Q^T for one tile of BN keys
  auto compute_s = [&](f32x16_t (&sc)[QS][NKB], const uint16_t* Ks) FA_INLINE {
    const uint32_t base = opaque(lds_addr(Ks) + srow);
#pragma unroll
    for (int qs = 0; qs < QS; ++qs)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sc[qs][kb] = zero16();
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const bf16x8_t a = lds_read8_at(base + 2 * (TL::row(32 * kb) + 16 * dc));
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) sc[qs][kb] = mfma32x32x16(a, qreg[qs][dc], sc[qs][kb]);
      }
  };

  // O^T += V^T P^T for one tile
  auto pv = [&](const uint32_t (&pk)[QS][NKB][8], const uint16_t* Vs) FA_INLINE {
    const uint32_t base = opaque(lds_addr(Vs) + trow);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8_t bop[QS];
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) {
          const u32x4_t bu = {pk[qs][kb][4 * kk], pk[qs][kb][4 * kk + 1], pk[qs][kb][4 * kk + 2],
                              pk[qs][kb][4 * kk + 3]};
          bop[qs] = __builtin_bit_cast(bf16x8_t, bu);
        }
        const int R = 32 * kb + 16 * kk;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const bf16x8_t a = join8(lds_read_tr4_at(base + 2 * (TL::row(R) + 32 * cb)),
                                   lds_read_tr4_at(base + 2 * (TL::row(R + 8) + 32 * cb)));
#pragma unroll
          for (int qs = 0; qs < QS; ++qs) oacc[qs][cb] = mfma32x32x16(a, bop[qs], oacc[qs][cb]);
        }
      }
  };

  // causal / key-tail mask of the scores of local tile t
  auto mask = [&](f32x16_t (&sc)[QS][NKB], int t) FA_INLINE {
    const int j0 = (t0 + t) * BN;
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
      const int lim = CAUSAL ? w0 + 32 * qs + l32 + p.causal_off : 0x7fffffff;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (j >= p.Nk || j > lim) sc[qs][kb][r] = -INFINITY;
        }
    }
  };

  // Row maxima and the lazy-rescale decision; returns whether the base of some block
  // moved (the rescale branch covers all blocks; unmoved rows have alpha = 1).
  auto smax = [&](f32x16_t (&sc)[QS][NKB]) FA_INLINE {
    bool any = false;
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[qs][kb][r]);
      mx = xhalf_max(mx) * c2;
      const bool move = __any(mx > m[qs] + (RENORM ? 0.f : kRescaleSlack));
      const float m_next = move ? fmaxf(m[qs], mx) : m[qs];
      m_use[qs] = (m_next == -INFINITY) ? 0.f : m_next;
      alpha[qs] = fast_exp2(m[qs] - m_use[qs]);  // 1 if the base did not move, 0 on first use
      m[qs] = m_next;
      any |= move;
    }
    return any;
  };
  // weights, their row sums and their bf16 packing
  auto sexp = [&](f32x16_t (&sc)[QS][NKB], uint32_t (&pk)[QS][NKB][8]) FA_INLINE {
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
      float rs = 0.f;
      if constexpr (!RENORM) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const float x0 = fmaf(sc[qs][kb][r], c2, -m_use[qs]);
            const float x1 = fmaf(sc[qs][kb][r + 1], c2, -m_use[qs]);
            const float p0 = fast_exp2(x0);
            const float p1 = (POLY && (r + 1) % 8 == 7) ? poly_exp2(x1) : fast_exp2(x1);
            rs += p0 + p1;
            pk[qs][kb][r >> 1] = pack_bf16x2(p0, p1);
          }
        lsum[qs] = fmaf(lsum[qs], alpha[qs], rs);
      } else {
        float pv[NKB][16];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            pv[kb][r] = fast_exp2(fmaf(sc[qs][kb][r], c2, -m_use[qs]));
            rs += pv[kb][r];
          }
        const float l_old = lsum[qs];
        lsum[qs] = fmaf(l_old, alpha[qs], rs);
        // O <- O * alpha * l_old / l_new, P <- P / l_new (whole-row sums)
        const float lt_old = xhalf_sum(l_old), lt_new = xhalf_sum(lsum[qs]);
        const float pscale = lt_new > 0.f ? 1.f / lt_new : 0.f;
        const float oscale = alpha[qs] * lt_old * pscale;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[qs][cb][r] *= oscale;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; r += 2)
            pk[qs][kb][r >> 1] = pack_bf16x2(pv[kb][r] * pscale, pv[kb][r + 1] * pscale);
      }
    }
  };
  auto rescale = [&]() FA_INLINE {
#pragma unroll
    for (int qs = 0; qs < QS; ++qs)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[qs][cb][r] *= alpha[qs];
  };

  // Step t. Entering: S_t in cur with its mask, row max and rescale decision applied
  // (m, m_use, alpha, move), K_{t+1} in K buffer (t+1)%2 and V_t in V buffer t%2. A
  // pending rescale of O (O holds P_{..t-1} V at the old base) comes first; it is the
  // only branch of the step, before its one scheduling region:
  //   copies of K_{t+2} and V_{t+1} into the free buffers,
  //   S_{t+1} = K_{t+1} Q^T (matrix)  with  P_t = exp(S_t) and its row sum (vector),
  //   O += V_t^T P_t (matrix)          with  mask and row max of S_{t+1} (vector),
  // then the copies' wait and a barrier. MASK: tile t+1 needs the mask; LAST: there is
  // no tile t+1.
  f32x16_t sA[QS][NKB], sB[QS][NKB];
  uint32_t pk[QS][NKB][8];
  bool move = false;
  auto step = [&](auto mask_tag, auto last_tag, f32x16_t (&cur)[QS][NKB],
                  f32x16_t (&nxt)[QS][NKB], int t) FA_INLINE {
    constexpr bool MASK = decltype(mask_tag)::value, LAST = decltype(last_tag)::value;
    if (!RENORM && move) rescale();
    if constexpr (!LAST) {
      load(Kg, t + 2, Kb(t));
      load(Vg, t + 1, Vb(t + 1));
    }
    __builtin_amdgcn_sched_barrier(0);
    debug_sync();
    if constexpr (!LAST) compute_s(nxt, Kb(t + 1));
    sexp(cur, pk);
    pv(pk, Vb(t));
    if constexpr (!LAST) {
      if constexpr (MASK) mask(nxt, t + 1);
      move = smax(nxt);
    }
    __builtin_amdgcn_sched_barrier(0);
    debug_sync();
    if constexpr (!LAST) {
      wait_vmem();
      __syncthreads();
    }
  };

  if (ntiles > 0) {
    load(Kg, 0, Kb(0));
    load(Kg, 1, Kb(1));
    load(Vg, 0, Vb(0));
    wait_vmem();
    __syncthreads();
    compute_s(sA, Kb(0));
    if (tfull == 0) mask(sA, 0);
    move = smax(sA);
    __syncthreads();  // K_0's buffer is refilled in step 0
    // S_t in sA at the top of each pair
    int t = 0;
    for (; t + 2 < tfull && t + 2 < ntiles; t += 2) {
      step(BoolC<false>(), BoolC<false>(), sA, sB, t);
      step(BoolC<false>(), BoolC<false>(), sB, sA, t + 1);
    }
    for (; t + 2 < ntiles; t += 2) {
      step(BoolC<true>(), BoolC<false>(), sA, sB, t);
      step(BoolC<true>(), BoolC<false>(), sB, sA, t + 1);
    }
    if (t + 1 < ntiles) {
      step(BoolC<true>(), BoolC<false>(), sA, sB, t);
      step(BoolC<false>(), BoolC<true>(), sB, sA, t + 1);
    } else {
      step(BoolC<false>(), BoolC<true>(), sA, sB, t);
    }
  }

  if constexpr (KS == 2) {
    // the second key group's O, base m and row sums to the first (tile buffers free:
    // every wave is past its last step)
    constexpr int XF = NCB * 16 + 2;  // floats per lane
    float* xf = (float*)smem + (size_t)wu * XF * 64 + lane;
    __syncthreads();
    if (ks == 1) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) xf[(16 * cb + r) * 64] = oacc[0][cb][r];
      xf[(NCB * 16) * 64] = m[0];
      xf[(NCB * 16 + 1) * 64] = lsum[0];
    }
    __syncthreads();
    if (ks == 1) return;
    const float m1 = xf[(NCB * 16) * 64], l1 = xf[(NCB * 16 + 1) * 64];
    const float mt = fmaxf(m[0], m1);
    const float mb = mt == -INFINITY ? 0.f : mt;
    const float a0 = fast_exp2(m[0] - mb), a1 = fast_exp2(m1 - mb);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[0][cb][r] = oacc[0][cb][r] * a0 + xf[(16 * cb + r) * 64] * a1;
    lsum[0] = lsum[0] * a0 + l1 * a1;
    m[0] = mt;
  }
  // Epilogue: combine the two half-row sums, normalise once, store O and LSE.
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    const int qrow = w0 + 32 * qs + l32;
    const float ltot = xhalf_sum(lsum[qs]);
    if (qrow < p.Nq) {
      const float inv = RENORM ? 1.f : (ltot > 0.f ? 1.f / ltot : 0.f);
      if (hi == 0) {
        p.lse[(size_t)(b * p.Hq + h) * p.Nq + qrow] =
            ltot > 0.f ? (m[qs] + log2f(ltot)) * kLn2 : -INFINITY;
      }
      uint16_t* orow = p.o + ((size_t)(b * p.Hq + h) * p.Nq + qrow) * D;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int c0 = 32 * cb + 8 * rg + 4 * hi;
          u32x2_t val = {pack_bf16x2(oacc[qs][cb][4 * rg] * inv, oacc[qs][cb][4 * rg + 1] * inv),
                         pack_bf16x2(oacc[qs][cb][4 * rg + 2] * inv, oacc[qs][cb][4 * rg + 3] * inv)};
          *(u32x2_t*)(orow + c0) = val;
        }
    }
  }
}

template <int D, int BN, int NW, int QS, bool CAUSAL, bool RENORM = false, bool POLY = false,
          int KS = 1>
hipError_t run(FwdParams p, long long B, hipStream_t st) {
  constexpr int BM = 32 * (NW / KS) * QS;
  p.nqb = (p.Nq + BM - 1) / BM;
  const long long nb = (long long)p.nqb * p.Hq * B;
  if (nb > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, BN, NW, QS, CAUSAL, RENORM, POLY, KS>), dim3((int)nb),
                     dim3(64 * NW), 0, st, p);
  return hipGetLastError();
}

}  // namespace
}  // namespace fa
