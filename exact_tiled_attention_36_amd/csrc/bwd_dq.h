// The dQ kernel of the recompute backward (the first of its two kernels), for gfx950.
// Included by bwd.hip (d = 256) and by bwd_dq_small.hip (d = 64 and 128, built with a
// compiler option of their own: see that file); 4-wave workgroups at every head size.
#pragma once
#include "bwd_dkdv.h"

namespace fa {

// Launch of bwd_dq_kernel<d, 32, 4, causal> (d = 64 or 128) on `grid` workgroups, or
// with key_split of its 8-wave form whose two wave groups take half of the key tiles
// each (bwd_dq_small.hip).
hipError_t launch_bwd_dq_small(const BwdParams& p, int nqb, int grid, int d, bool causal,
                               bool key_split, hipStream_t st);

namespace {
// ---------------------------------------------------------------------------------
// 1. dQ, with D
// ---------------------------------------------------------------------------------
// One workgroup = NW waves x 32 query rows; Q and dO stay in registers, each wave
// owns its rows' dQ. Key tiles of BN rows (K and V) are triple buffered in LDS and
// copied two tiles ahead. Step t is one scheduling region:
//   S, dP of tile t+1 (matrix)       with  dS of tile t (vector),
//   dQ^T += K_t^T dS^T (matrix)      with  mask of tile t+1 (vector),
// then the copies' wait and a barrier. S^T and dP^T put one query per lane, so LSE
// and D are per-lane scalars; dS^T comes out in the B-operand layout of the dQ
// product, and K^T is read with LDS transpose loads.
//
// KS = 2 (grids too small to fill the GPU): the NW waves form two groups that own the
// same rows and take one half of the key tiles each, in LDS buffers of their own; at
// the end the second group adds its partial dQ into the first's through LDS (dQ is a
// plain sum over key tiles). Each wave's chain of key tiles is half as long and every
// SIMD holds two waves.
template <int D, int BN, int NW, bool CAUSAL, int KS = 1>
__global__ __launch_bounds__(64 * NW, 1) void bwd_dq_kernel(BwdParams p, int nqb) {
  using TL = TileLayout<D>;
  constexpr int TILE = TL::elems(BN);
  constexpr int NDC = D / 16, NCB = D / 32, NKB = BN / 32;
  static_assert(KS == 1 || (KS == 2 && D <= 128 && NW == 8), "the key split is an 8-wave form");
  constexpr int WG = NW / KS;    // waves per key group
  constexpr int BM = 32 * WG;    // query rows per workgroup (one 32-row block per wave)
  constexpr int NB = 3;
  static_assert(TL::shifts_ok(BN), "LDS reads add row offsets as constants");

  __shared__ __attribute__((aligned(16))) uint16_t smem[KS * NB * 2 * TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wall = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ks = KS == 1 ? 0 : wall / WG;     // key group (uniform)
  const int wu = KS == 1 ? wall : wall % WG;  // wave within its group
  const int l32 = lane & 31, hi = lane >> 5;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  int qb, bh;
  if (CAUSAL) {
    causal_order<2>(blockIdx.x, gridDim.x, nqb, bh, qb);
  } else {
    qb = L % nqb;
    bh = L / nqb;
  }
  const int h = bh % p.Hq, b = bh / p.Hq, kvh = h / p.g;
  const int q0 = qb * BM;
  const int w0 = q0 + 32 * wu;
  const int qrow = w0 + l32;
  const bool qvalid = qrow < p.Nq;
  const size_t rowidx = (size_t)(b * p.Hq + h) * p.Nq + (qvalid ? qrow : p.Nq - 1);

  bf16x8_t qreg[NDC], doreg[NDC];
  {
    const u32x4_t* qs = (const u32x4_t*)(p.q + rowidx * D + 8 * hi);
    const u32x4_t* os = (const u32x4_t*)(p.dO + rowidx * D + 8 * hi);
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      qreg[dc] = __builtin_bit_cast(bf16x8_t, qs[2 * dc]);
      doreg[dc] = __builtin_bit_cast(bf16x8_t, os[2 * dc]);
    }
  }
  // D_i = sum_c dO_ic O_ic: this lane's half of the row of O, read in the layout of
  // dO, then the two halves combined. D and LSE * log2(e) also go to the workspace
  // for the dK/dV kernel.
  float dpart = 0.f;
  {
    const u32x4_t* os = (const u32x4_t*)(p.o + rowidx * D + 8 * hi);
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      const u32x4_t ov = os[2 * dc];
      const u32x4_t dv = __builtin_bit_cast(u32x4_t, doreg[dc]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dpart = fmaf(bf16_lo(ov[i]), bf16_lo(dv[i]), dpart);
        dpart = fmaf(bf16_hi(ov[i]), bf16_hi(dv[i]), dpart);
      }
    }
  }
  const float dsum = xhalf_sum(dpart);
  const float lraw = p.lse[rowidx];
  const float Dv = qvalid ? dsum : 0.f;
  const float lse2 = (!qvalid || lraw == -INFINITY) ? INFINITY : lraw * kLog2e;
  if (qvalid && hi == 0 && ks == 0) {
    p.dvec[rowidx] = Dv;
    p.lse2v[rowidx] = lse2;
  }
  // nothing may be outstanding in the loops below except the tile copies they issue
  wait_vmem();

  const uint16_t* Kg = p.k + (size_t)(b * p.Hkv + kvh) * p.Nk * D;
  const uint16_t* Vg = p.v + (size_t)(b * p.Hkv + kvh) * p.Nk * D;
  int kend = p.Nk;
  if (CAUSAL) {
    const int lim = q0 + BM + p.causal_off;
    kend = lim < kend ? lim : kend;
  }
  const int ntiles_all = kend > 0 ? (kend + BN - 1) / BN : 0;
  // tiles [0, tfull) are wholly visible to every row of the workgroup
  int tfull_all = p.Nk / BN;
  if (CAUSAL) {
    const int lim = q0 + p.causal_off + 1;
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

  f32x16_t dqacc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) dqacc[cb] = zero16();
  const float c2 = p.scale_log2;

  // buffer t%3 (of this wave's key group) holds the K tile of local key tile t, followed
  // by its V tile
  auto Kb = [&](int t) FA_INLINE { return smem + (ks * NB + t % NB) * 2 * TILE; };
  // rows past Nk re-read the last key row; the key-tail mask zeroes their weight
  const uint32_t lane_off = 4u * lane;
  auto load_tile = [&](int tl) FA_INLINE {
    const int t = t0 + tl;
    uint16_t* const buf = Kb(tl);
    if constexpr (D == 256) {
      const uint32_t m0 = lds_addr(buf);
      tile_load_m0<D, BN, WG>(Kg, t * BN, p.Nk, m0, wu, lane_off);
      tile_load_m0<D, BN, WG>(Vg, t * BN, p.Nk, m0 + 2 * TILE, wu, lane_off);
      return;
    }
    if constexpr (D <= 128) {
      if ((t + 1) * BN <= p.Nk) {  // whole tile present: scalar-addressed copies
        // (from one opaque LDS base: the hoisted per-piece addresses spilled into
        // vector lanes)
        tile_load_full_o<D, BN, WG>(Kg, t * BN, buf, wu, lane_off);
        tile_load_full_o<D, BN, WG>(Vg, t * BN, buf + TILE, wu, lane_off);
        return;
      }
    }
    tile_load_async<D, BN, WG>(Kg, t * BN, p.Nk, buf, wu, lane);
    tile_load_async<D, BN, WG>(Vg, t * BN, p.Nk, buf + TILE, wu, lane);
  };

  const int tr_row = 4 * hi + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const uint32_t srow = 2 * (TL::row(l32) + 8 * hi);
  const uint32_t trow = 2 * (TL::row(tr_row) + tr_col);

  // S^T = K Q^T and dP^T = V dO^T for key tile t
  auto compute_sp = [&](f32x16_t (&S)[NKB], f32x16_t (&dP)[NKB], int t) FA_INLINE {
    const uint32_t kbase = opaque(lds_addr(Kb(t)) + srow);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      S[kb] = zero16();
      dP[kb] = zero16();
    }
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const uint32_t a = kbase + 2 * (TL::row(32 * kb) + 16 * dc);
        S[kb] = mfma32x32x16(lds_read8_at(a), qreg[dc], S[kb]);
        dP[kb] = mfma32x32x16(lds_read8_at(a + 2 * TILE), doreg[dc], dP[kb]);
      }
  };
  // causal / key-tail mask of local key tile t: masked scores give P = dS = 0
  auto mask = [&](f32x16_t (&S)[NKB], int t) FA_INLINE {
    const int j0 = (t0 + t) * BN;
    const int lim = CAUSAL ? qrow + p.causal_off : 0x7fffffff;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = j0 + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (j >= p.Nk || j > lim) S[kb][r] = -INFINITY;
      }
  };
  // dS = P * (dP - D) with P = exp2(S * scale * log2e - LSE2), bf16 pairs
  auto dsoft = [&](f32x16_t (&S)[NKB], f32x16_t (&dP)[NKB], uint32_t (&dspk)[NKB][8]) FA_INLINE {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float ds2[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float pr = fast_exp2(fmaf(S[kb][r + e], c2, -lse2));
          ds2[e] = pr * (dP[kb][r + e] - Dv);
        }
        dspk[kb][r >> 1] = pack_bf16x2(ds2[0], ds2[1]);
      }
  };
  // dQ^T += K_t^T dS^T
  auto dq_mm = [&](const uint32_t (&dspk)[NKB][8], int t) FA_INLINE {
    const uint32_t tb = opaque(lds_addr(Kb(t)) + trow);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const u32x4_t du = {dspk[kb][4 * kk], dspk[kb][4 * kk + 1], dspk[kb][4 * kk + 2], dspk[kb][4 * kk + 3]};
        const bf16x8_t db = __builtin_bit_cast(bf16x8_t, du);
        const int R = 32 * kb + 16 * kk;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const bf16x8_t a = join8(lds_read_tr4_at(tb + 2 * (TL::row(R) + 32 * cb)),
                                   lds_read_tr4_at(tb + 2 * (TL::row(R + 8) + 32 * cb)));
          dqacc[cb] = mfma32x32x16(a, db, dqacc[cb]);
        }
      }
  };

  // Step t: entering, S/dP of tile t (masked) in (sc, pc), tiles t and t+1 in LDS.
  // MASK: tile t+1 needs the mask; LAST: there is no tile t+1.
  f32x16_t sA[NKB], pA[NKB], sB[NKB], pB[NKB];
  uint32_t dspk[NKB][8];
  auto step = [&](auto mask_tag, auto last_tag, f32x16_t (&sc)[NKB], f32x16_t (&pc)[NKB],
                  f32x16_t (&sn)[NKB], f32x16_t (&pn)[NKB], int t) FA_INLINE {
    constexpr bool MASK = decltype(mask_tag)::value, LAST = decltype(last_tag)::value;
    if constexpr (!LAST) load_tile(t + 2);  // into the buffer of tile t-1, done with
    __builtin_amdgcn_sched_barrier(0);
    debug_sync();
    if constexpr (!LAST) compute_sp(sn, pn, t + 1);
    dsoft(sc, pc, dspk);
    dq_mm(dspk, t);
    if constexpr (!LAST && MASK) mask(sn, t + 1);
    __builtin_amdgcn_sched_barrier(0);
    debug_sync();
    if constexpr (!LAST) {
      wait_vmem();
      __syncthreads();
    }
  };

  if (ntiles > 0) {
    load_tile(0);
    load_tile(1);
    wait_vmem();
    __syncthreads();
    compute_sp(sA, pA, 0);
    if (tfull == 0) mask(sA, 0);
    int t = 0;
    for (; t + 2 < tfull && t + 2 < ntiles; t += 2) {
      step(BoolC<false>(), BoolC<false>(), sA, pA, sB, pB, t);
      step(BoolC<false>(), BoolC<false>(), sB, pB, sA, pA, t + 1);
    }
    for (; t + 2 < ntiles; t += 2) {
      step(BoolC<true>(), BoolC<false>(), sA, pA, sB, pB, t);
      step(BoolC<true>(), BoolC<false>(), sB, pB, sA, pA, t + 1);
    }
    if (t + 1 < ntiles) {
      step(BoolC<true>(), BoolC<false>(), sA, pA, sB, pB, t);
      step(BoolC<false>(), BoolC<true>(), sB, pB, sA, pA, t + 1);
    } else {
      step(BoolC<false>(), BoolC<true>(), sA, pA, sB, pB, t);
    }
  }

  if constexpr (KS == 2) {
    // the second key group's partial dQ into the first's (tile buffers free: every
    // wave is past its last step)
    float* xf = (float*)smem + (size_t)wu * (NCB * 16) * 64 + lane;
    __syncthreads();
    if (ks == 1) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) xf[(16 * cb + r) * 64] = dqacc[cb][r];
    }
    __syncthreads();
    if (ks == 1) return;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) dqacc[cb][r] += xf[(16 * cb + r) * 64];
  }
  if (qvalid) {
    uint16_t* orow = p.dq + rowidx * D;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int c0 = 32 * cb + 8 * rg + 4 * hi;
        const u32x2_t val = {pack_bf16x2(dqacc[cb][4 * rg] * p.scale, dqacc[cb][4 * rg + 1] * p.scale),
                             pack_bf16x2(dqacc[cb][4 * rg + 2] * p.scale, dqacc[cb][4 * rg + 3] * p.scale)};
        *(u32x2_t*)(orow + c0) = val;
      }
  }
}

}  // namespace
}  // namespace fa
