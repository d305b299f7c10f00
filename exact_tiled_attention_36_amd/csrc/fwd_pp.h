// Forward attention, bf16, with two wave groups that take turns on the matrix cores
// ("ping-pong"), for gfx950.
//
// Same method and result as fwd_bf16.h ("FlashAttention" (ruizhehou.github.io): tiles
// of Q rows in the outer loop and of K/V in the inner loop, §二.1 and §三; running row
// max and row sum with the rescale factor exp(m_old - m_new), §二.2; the output divided
// by the row sum once at the end, §四.1; row blocks of a head in separate workgroups,
// §四.2). What differs is how the work of one workgroup is laid out in time.
//
// A workgroup has 8 waves of QB blocks of 32 query rows; waves 0-3 form group A and
// waves 4-7 group B, so every SIMD holds one wave of each group. A wave's key-tile
// step has a matrix phase (S_{t+1} = K_{t+1} Q^T and O^T += V_t^T P_t^T) and a vector
// phase (mask, row max, lazy rescale of O, exponentials, row sums and bf16 packing of
// S_{t+1} into P_{t+1}). The two groups are half a step apart: while the wave of group
// A on a SIMD runs its matrix phase, the wave of group B runs its vector phase, then
// they swap. On gfx950 a vector-only wave and a matrix-only wave on one SIMD overlap
// (measured: paired they take 65 % of the sum of their separate times), so each SIMD's
// matrix unit is fed by one wave while the other wave's softmax runs beside it.
// (Raising the matrix-phase wave's issue priority with s_setprio measured no faster,
// so both waves keep the default priority.)
//
// Phases are separated by workgroup barriers (two per key tile). K and V tiles are
// double buffered in LDS: K_{t+1} and V_t are read by group A in the first phase of
// step t and by group B in the second; the copies of K_{t+2} and V_{t+1} are issued at
// the start of step t into the buffers that K_t and V_{t-1} left, and waited for at the
// step's end barrier. Each wave needs only one score tile and one packed-weight tile
// per query block in registers (no in-wave software pipeline).
//
// NW = 4: one group of 4 waves (no turn-taking; 128 rows per workgroup at QB = 1, or
// 128 rows of each of two heads with HP): two workgroups share a compute unit (72 KB of
// LDS each at d = 256, 80 KB for d = 128 head pairs), so each SIMD still holds two
// waves, of different workgroups, that overlap by themselves.
//
// QB = 1 (d = 256): 32 rows per wave, Q in registers.
// QB = 2 (d = 128, large grids): 64 rows per wave, 512 per workgroup, so every K or
// V^T operand read from LDS feeds two products instead of one (LDS bytes per product
// 0.75 KB instead of 1 KB at d = 128, and half as many workgroups for the same rows).
// The registers (256 per wave at two waves per SIMD) hold Q of the first block and
// the 128 output accumulators; the second block's Q rows sit in a tile of the wave's
// own in LDS. With this many live accumulators the loop must have a single producer
// of O: every key tile, the last included, runs through one loop (the last step's
// scores come from a stale buffer and are never used). The form with a separate last
// step made the compiler keep a second copy of O across the loop and spill.
#pragma once
#pragma once
#include "fwd_bf16.h"

#ifndef FWD_PP_LOOK
#define FWD_PP_LOOK 4
#endif
#ifndef FWD_PP2_LOOK
#define FWD_PP2_LOOK 3
#endif

namespace fa {
namespace {

// starting value of the running max: finite, so a row that has seen no key yet needs
// no special case (its weights are exp2(-inf) = 0, its first rescale factor 0)
constexpr float kNoMax = -1e30f;

//
// KS = 2 (one-block 4-wave form, grids too small to fill the GPU): two such groups of 4
// waves in one workgroup own the same rows and take one half of the key tiles each, in
// LDS buffers of their own; at the end the second hands O, its base m and its row sums
// to the first through LDS, which merges them (§二.2 rescale) before the one division.
template <int D, int BN, bool CAUSAL, int QB, bool HP = false, int NW = 8, int KS = 1>
__global__ __launch_bounds__(64 * NW * KS, (NW == 8 || KS == 2) ? 1 : 2) void fwd_pp_kernel(FwdParams p) {
  using TL = TileLayout<D>;
  static_assert(NW == 8 || NW == 4, "two wave groups of 4, or one group of 4 waves");
  static_assert(KS == 1 || (KS == 2 && NW == 4 && QB == 1 && !HP), "key split of the 4-wave form");
  static_assert(!HP || QB == 2, "head pairs take two query blocks");
  // HP: the two blocks of a wave are the same 32 rows of two query heads that share a
  // kv-head; otherwise QB consecutive 32-row blocks of one head
  constexpr int RW = HP ? 32 : 32 * QB;  // query rows per wave
  constexpr int BM = RW * NW;            // query rows per workgroup (per head)
  constexpr int QSTEP = HP ? 0 : 32;     // row offset of block qb = QSTEP * qb
  constexpr int TILE = TL::elems(BN);
  constexpr int NKB = BN / 32;   // 32-key blocks per tile
  constexpr int NDC = D / 16;    // 16-wide chunks of d (reduction of S)
  constexpr int NCB = D / 32;    // 32-wide column blocks of O
  static_assert(TL::shifts_ok(BN), "LDS reads add row offsets as constants");
  static_assert(QB == 1 || QB == 2, "one or two query blocks per wave");
  // with two blocks, the second block's Q rows stay in LDS (a tile per wave): the
  // registers hold Q of the first block only
  constexpr int QT = TL::elems(32);

  __shared__ __attribute__((aligned(16))) uint16_t smem[KS * (4 * TILE + (QB - 1) * NW * QT)];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wall = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ks = KS == 1 ? 0 : wall / NW;     // key group (uniform)
  const int wu = KS == 1 ? wall : wall % NW;  // wave within its group
  const bool grp_b = NW == 8 && wu >= 4;   // wave-uniform
  const int l32 = lane & 31, hi = lane >> 5;

  int qb, bh;
  if (CAUSAL) {
    causal_order<2>(blockIdx.x, gridDim.x, p.nqb, bh, qb);
  } else {
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    qb = L % p.nqb;
    bh = L / p.nqb;
  }
  const int hpb = HP ? p.Hq / 2 : p.Hq;  // head slots per batch (pairs with HP)
  const int h = HP ? 2 * (bh % hpb) : bh % hpb, b = bh / hpb;
  const int kvh = h / p.g;
  const int q0 = qb * BM;
  const int w0 = q0 + RW * wu;  // first query row of this wave

  const uint16_t* Qg = p.q + (size_t)(b * p.Hq + h) * p.Nq * D;
  const uint16_t* Kg = p.k + (size_t)(b * p.Hkv + kvh) * p.Nk * D;
  const uint16_t* Vg = p.v + (size_t)(b * p.Hkv + kvh) * p.Nk * D;

  bf16x8_t qreg[NDC];
  {
    const int qrow = w0 + l32;
    const int qr = qrow < p.Nq ? qrow : p.Nq - 1;
    const u32x4_t* src = (const u32x4_t*)(Qg + (size_t)qr * D + 8 * hi);
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) qreg[dc] = __builtin_bit_cast(bf16x8_t, src[2 * dc]);
  }
  uint16_t* const q1t = smem + 4 * TILE + wu * QT;  // this wave's second Q block (QB = 2)
  if constexpr (QB == 2)
    tile_load_async<D, 32, 1>(HP ? Qg + (size_t)p.Nq * D : Qg, w0 + QSTEP, p.Nq, q1t, 0, lane);
  // nothing may be outstanding in the loop below except the tile copies it issues
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
  // masked away); both groups run the same steps, since they share the barriers
  const int ntiles = KS == 1 ? ntiles_all : (ntiles_all + 1) / 2;
  const int t0 = ks * ntiles;  // global index of local tile 0
  const int tfull = KS == 1 ? tfull_all : min(min(tfull_all, ntiles), max(tfull_all - ntiles, 0));

  f32x16_t oacc[QB][NCB];
  float m[QB], lsum[QB];  // running max (log2 units) and row sum per block
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) oacc[qb][cb] = zero16();
    m[qb] = kNoMax;
    lsum[qb] = 0.f;
  }
  const float c2 = p.scale_log2;

  auto Kb = [&](int i) FA_INLINE { return smem + (4 * ks + (i & 1)) * TILE; };
  auto Vb = [&](int i) FA_INLINE { return smem + (4 * ks + 2 + (i & 1)) * TILE; };
  // Rows past the last key re-read the last key row: always finite, and masked to
  // zero weight before they can contribute.
  const uint32_t lane_off = 4u * lane;
  auto load8 = [&](const uint16_t* G, int tl, uint16_t* dst) FA_INLINE {
    const int t = t0 + tl;
    if ((t + 1) * BN <= p.Nk) {  // whole tile present: scalar-addressed copies
      tile_load_full<D, BN, NW>(G, t * BN, dst, wu, lane_off);
      return;
    }
    tile_load_async<D, BN, NW>(G, t * BN, p.Nk, dst, wu, lane);
  };
  auto load4 = [&](const uint16_t* G, int tl, uint16_t* dst) FA_INLINE {  // group A only
    const int t = t0 + tl;
    if ((t + 1) * BN <= p.Nk) {
      tile_load_full<D, BN, 4>(G, t * BN, dst, wu, lane_off);
      return;
    }
    tile_load_async<D, BN, 4>(G, t * BN, p.Nk, dst, wu, lane);
  };

  // per-lane LDS byte offsets inside a tile: K operand rows, V^T transposed reads
  const int tr_row = 4 * hi + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const uint32_t srow = 2 * (TL::row(l32) + 8 * hi);
  const uint32_t trow = 2 * (TL::row(tr_row) + tr_col);

  f32x16_t S[QB][NKB];
  u32x4_t pk[QB][NKB][2];  // packed bf16 weights, one MFMA B operand per 16 keys

  // S^T = K Q^T for one tile of BN keys; every K operand read feeds the QB blocks (the
  // second block's Q^T operand is a 16-byte row read of its LDS tile)
  auto compute_s = [&](const uint16_t* Ks) FA_INLINE {
    const uint32_t base = opaque(lds_addr(Ks) + srow);
    const uint32_t qbase = QB == 2 ? opaque(lds_addr(q1t) + srow) : 0u;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) S[qb][kb] = zero16();
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const bf16x8_t a = lds_read8_at(base + 2 * (TL::row(32 * kb) + 16 * dc));
        S[0][kb] = mfma32x32x16(a, qreg[dc], S[0][kb]);
        if constexpr (QB == 2) {
          const bf16x8_t q1 = lds_read8_at(qbase + 2 * 16 * dc);
          S[1][kb] = mfma32x32x16(a, q1, S[1][kb]);
        }
      }
  };
  // O^T += V^T P^T for one tile; every V^T operand read feeds the QB blocks
  auto pv = [&](const uint16_t* Vs) FA_INLINE {
    const uint32_t base = opaque(lds_addr(Vs) + trow);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8_t bop[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          bop[qb] = __builtin_bit_cast(bf16x8_t, pk[qb][kb][kk]);
        }
        const int R = 32 * kb + 16 * kk;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const bf16x8_t a = join8(lds_read_tr4_at(base + 2 * (TL::row(R) + 32 * cb)),
                                   lds_read_tr4_at(base + 2 * (TL::row(R + 8) + 32 * cb)));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) oacc[qb][cb] = mfma32x32x16(a, bop[qb], oacc[qb][cb]);
        }
      }
  };
  // Matrix phase of step t: S_{t+1} (NEXT: there is a next tile) and O += V_t P_t.
  // The LDS operand reads are kept a few reads ahead of the products that use them
  // (left to itself the compiler hoists all of them and runs out of registers).
  auto mat_phase = [&](int t, auto next_tag, auto pv_tag) FA_INLINE {
    constexpr bool NEXT = decltype(next_tag)::value, PV = decltype(pv_tag)::value;
    __builtin_amdgcn_sched_barrier(0);
    debug_sync();
    constexpr int NS = NEXT ? NDC * NKB : 0, NP = PV ? 2 * NKB * NCB : 0;
    if constexpr (QB == 1) {
      if constexpr (NEXT) compute_s(Kb(t + 1));
      if constexpr (PV) pv(Vb(t));
      ReadAheadG<FWD_PP_LOOK, NS, 1, NP, 2>::emit();
    } else {
      // O += V_t P_t first: the weights die before the next scores are made
      if constexpr (PV) pv(Vb(t));
      if constexpr (NEXT) compute_s(Kb(t + 1));
      ReadAheadG<FWD_PP2_LOOK, NP, 2, NS, 2, QB>::emit();
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // vector phase: S_j (in S) into P_j (in pk), with m, l and the lazy rescale of O
  auto vec_phase = [&](int j) FA_INLINE {
    if (j >= tfull) {  // causal diagonal or key tail
      // key j*BN + 4*hi + c (c a per-register constant) is visible to this lane's row
      // iff c <= T, with T the last visible key less the lane's base (j local)
      const int base = (t0 + j) * BN + 4 * hi;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        int last = p.Nk - 1;
        if (CAUSAL) last = min(last, w0 + QSTEP * qb + l32 + p.causal_off);
        const int T = last - base;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * kb + 8 * (r >> 2) + (r & 3) > T) S[qb][kb][r] = -INFINITY;
      }
    }
    float mx[QB];
    bool up = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      mx[qb] = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx[qb] = fmaxf(mx[qb], S[qb][kb][r]);
      mx[qb] = xhalf_max(mx[qb]) * c2;
      up = up || mx[qb] > m[qb] + kRescaleSlack;
    }
    // the base moves only when some row's max passes it by more than the slack
    if (__any(up)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float m_next = fmaxf(m[qb], mx[qb]);
        const float alpha = fast_exp2(m[qb] - m_next);  // 0 on first use, 1 if unchanged
        m[qb] = m_next;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[qb][cb][r] *= alpha;
        lsum[qb] *= alpha;
      }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = fast_exp2(fmaf(S[qb][kb][r], c2, -m[qb]));
          const float p1 = fast_exp2(fmaf(S[qb][kb][r + 1], c2, -m[qb]));
          rs += p0 + p1;
          pk[qb][kb][r >> 3][(r >> 1) & 3] = pack_bf16x2(p0, p1);
        }
      lsum[qb] += rs;
    }
  };
  // Both groups run the same instruction stream; group B passes one extra barrier at
  // the start and group A one at the end, which puts B half a step behind A. Barrier
  // k of one group is barrier k of the other, so between two barriers one group runs
  // a matrix phase while the other runs a vector phase. Group A issues every tile copy
  // (at the start of its matrix phase of step t: K_{t+2} and V_{t+1}) and waits for
  // them at the end of step t, before group A's next matrix phase and before group
  // B's, which comes a phase later. Buffers: K_{t+1} and V_t are read by A in one phase
  // and by B in the next; K_{t+2} replaces K_t and V_{t+1} replaces V_{t-1}, which B
  // finished reading a phase before A issues the copies.
  if (ntiles > 0) {
    load8(Kg, 0, Kb(0));
    if (ntiles > 1) load8(Kg, 1, Kb(1));
    load8(Vg, 0, Vb(0));
    wait_vmem();
    __syncthreads();
    if (grp_b) __syncthreads();
    // S_0 and P_0
    mat_phase(-1, BoolC<true>(), BoolC<false>());
    __syncthreads();
    vec_phase(0);
    __syncthreads();
    if constexpr (QB == 2) {
      // every step in one loop (the last one's scores are made from a stale buffer and
      // never used), so the output accumulators have one producer in the loop
      for (int t = 0; t < ntiles; ++t) {
        if (!grp_b) {
          if (t + 2 < ntiles) load4(Kg, t + 2, Kb(t));
          if (t + 1 < ntiles) load4(Vg, t + 1, Vb(t + 1));
        }
        mat_phase(t, BoolC<true>(), BoolC<true>());
        __syncthreads();
        if (t + 1 < ntiles) vec_phase(t + 1);
        wait_vmem();
        __syncthreads();
      }
      if (!grp_b) __syncthreads();
    } else {
      int t = 0;
      for (; t + 1 < ntiles; ++t) {
        if (!grp_b) {
          if (t + 2 < ntiles) load4(Kg, t + 2, Kb(t));
          load4(Vg, t + 1, Vb(t + 1));
        }
        mat_phase(t, BoolC<true>(), BoolC<true>());
        __syncthreads();
        vec_phase(t + 1);
        wait_vmem();
        __syncthreads();
      }
      // last step: only O += V_t P_t
      mat_phase(t, BoolC<false>(), BoolC<true>());
      __syncthreads();
      if (!grp_b) __syncthreads();
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
    const float mt = fmaxf(m[0], m1);  // both bases finite (kNoMax before any key)
    const float a0 = fast_exp2(m[0] - mt), a1 = fast_exp2(m1 - mt);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[0][cb][r] = oacc[0][cb][r] * a0 + xf[(16 * cb + r) * 64] * a1;
    lsum[0] = lsum[0] * a0 + l1 * a1;
    m[0] = mt;
  }
  // Epilogue: combine the two half-row sums, normalise once, store O and LSE.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qrow = w0 + QSTEP * qb + l32;
    const int hq = HP ? h + qb : h;
    const float ltot = xhalf_sum(lsum[qb]);
    if (qrow < p.Nq) {
      const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
      if (hi == 0) {
        p.lse[(size_t)(b * p.Hq + hq) * p.Nq + qrow] =
            ltot > 0.f ? (m[qb] + log2f(ltot)) * kLn2 : -INFINITY;
      }
      uint16_t* orow = p.o + ((size_t)(b * p.Hq + hq) * p.Nq + qrow) * D;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int c0 = 32 * cb + 8 * rg + 4 * hi;
          u32x2_t val = {pack_bf16x2(oacc[qb][cb][4 * rg] * inv, oacc[qb][cb][4 * rg + 1] * inv),
                         pack_bf16x2(oacc[qb][cb][4 * rg + 2] * inv, oacc[qb][cb][4 * rg + 3] * inv)};
          *(u32x2_t*)(orow + c0) = val;
        }
    }
  }
}

template <int D, int BN, bool CAUSAL, int QB = 1, bool HP = false, int NW = 8, int KS = 1>
hipError_t run_pp(FwdParams p, long long B, hipStream_t st) {
  constexpr int BM = (HP ? 32 : 32 * QB) * NW;
  p.nqb = (p.Nq + BM - 1) / BM;
  const long long nb = (long long)p.nqb * (HP ? p.Hq / 2 : p.Hq) * B;
  if (nb > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_pp_kernel<D, BN, CAUSAL, QB, HP, NW, KS>), dim3((int)nb), dim3(64 * NW * KS),
                     0, st, p);
  return hipGetLastError();
}

}  // namespace
}  // namespace fa
