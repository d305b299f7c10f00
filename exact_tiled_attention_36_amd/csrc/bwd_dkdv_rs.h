// dK/dV of the recompute backward for head size 256, with the products of a key slot
// split between two waves (gfx950).
//
// Same products as bwd_dkdv.h ("FlashAttention" (ruizhehou.github.io), §二.3: P is
// rebuilt from Q, K and the forward's LSE, then dV = P^T dO, dS = P * (dP - D) with
// dP = dO V^T, dK = scale * dS^T Q, summed over the query heads that share the
// kv-head). At d = 256 one wave cannot hold K and V of its 32 keys (128 registers) and
// their dK and dV accumulators (256) and still have room for its operands: the
// one-wave kernel spilled, and the reloads' waits also waited for the step's tile
// copies. Here a workgroup of 4 waves (one per SIMD) covers 64 keys in two 32-key
// slots, and the two waves of a slot split the products:
//   the weight wave: K in registers; per 32-query step S = Q K^T, the weights P
//                    (masked, bf16), dV += dO^T P; it hands P to its partner in LDS;
//   the dS wave:     V in registers; dP = dO V^T, dS = P * (dP - D) with the
//                    partner's P, dK += Q^T dS, one step behind.
// Each wave holds 64 operand (K or V) and 128 accumulator registers, about 320 in all:
// no scratch. Q/dO tiles and their LSE2/D rows are triple buffered (step s: the weight
// waves read tile s, the dS waves tile s-1, the copies of tile s+1 land in the third
// buffer), the exchanged weights double buffered; one barrier per step orders it all.
// The last eight products of a step (dV/dK of its second 16 queries, registers only)
// run after the barrier, beside the next step's row reads.
//
// The dS wave multiplies dP - D by the bf16 weight the dV product uses too (the
// one-wave kernel uses the float32 weight): the results differ within one bf16
// rounding of P.
#pragma once
#include "bwd_dkdv.h"

namespace fa {
namespace {

template <bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_rs_kernel(BwdParams p, int nkb) {
  constexpr int D = 256, BMQ = 32, NQS = 1;
  using TL = TileLayout<D>;
  constexpr int TILE = TL::elems(BMQ);
  constexpr int NDC = D / 16, NCB = D / 32, HD = NDC / 2;
  constexpr int NW = 4, NS = NW / 2;  // waves, 32-key slots
  constexpr int BNK = 32 * NS, NB = 3, SV = 64;

  __shared__ __attribute__((aligned(16))) uint16_t smem[NB * 2 * TILE];
  __shared__ __attribute__((aligned(16))) float svec[NB * 2 * SV];
  // exchanged weights: [key slot][buffer][16-query half][lane]
  __shared__ u32x4_t xbuf[NS][2][2][64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool role_b = wu >= NS;  // wave-uniform: dP/dS/dK wave
  const int kw = wu % NS;        // key slot
  const int l32 = lane & 31, hi = lane >> 5;
  int kb, bkv;
  if (CAUSAL) {
    causal_order<1>(blockIdx.x, gridDim.x, nkb, bkv, kb);
    kb = nkb - 1 - kb;
  } else {
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    kb = L % nkb;
    bkv = L / nkb;
  }
  const int kvh = bkv % p.Hkv, b = bkv / p.Hkv;
  const int k0 = kb * BNK;
  const int key = k0 + 32 * kw + l32;
  const size_t kbase = ((size_t)(b * p.Hkv + kvh) * p.Nk + (key < p.Nk ? key : p.Nk - 1)) * D;

  // K (weight waves) or V (dS waves) of this lane's key, as MFMA B operands
  bf16x8_t kv[NDC];
  {
    const u32x4_t* src = (const u32x4_t*)((role_b ? p.v : p.k) + kbase + 8 * hi);
    const u32x4_t z = {0, 0, 0, 0};
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) kv[dc] = __builtin_bit_cast(bf16x8_t, key < p.Nk ? src[2 * dc] : z);
  }
  // nothing may be outstanding in the loops below except the tile copies they issue
  wait_vmem();

  // Query tiles (as bwd_dkdv.h): [qb0, nqb) can see some key of this workgroup; tiles
  // [qb0, qd) touch the causal diagonal and a ragged last tile [qe, nqb) holds rows
  // past Nq: those steps need masking and run first, then the unmasked tiles [qd, qe)
  // from the top down.
  int i_start = 0;
  if (CAUSAL) {
    i_start = k0 - p.causal_off;
    if (i_start < 0) i_start = 0;
  }
  const int nqb = (p.Nq + BMQ - 1) / BMQ;
  const int qb0 = min(i_start / BMQ, nqb);
  int qd = qb0;
  if (CAUSAL) {
    const int lim = k0 + BNK - 1 - p.causal_off;  // first row that sees every key here
    qd = lim <= 0 ? 0 : (lim + BMQ - 1) / BMQ;
    qd = max(qb0, min(qd, nqb));
  }
  const int qe = p.Nq % BMQ ? nqb - 1 : nqb;
  const int nu = qe > qd ? qe - qd : 0;
  const int nm = (nqb - qb0) - nu;
  const int total_m = nm * p.g, total = (nm + nu) * p.g;
  struct Cur {
    int s, hs, j;
  };
  auto cur_i0 = [&](const Cur& c) FA_INLINE {
    if (c.s < total_m)
      return (c.j < qd - qb0 ? qb0 + c.j : max(qd, qe) + (c.j - (qd - qb0))) * BMQ;
    return (qe - 1 - c.j) * BMQ;
  };
  auto cur_next = [&](Cur& c) FA_INLINE {
    if (c.s < total_m) {
      if (++c.j == nm) {
        c.j = 0;
        ++c.hs;
      }
      if (c.s + 1 == total_m) c.hs = c.j = 0;
    } else if (++c.hs == p.g) {
      c.hs = 0;
      ++c.j;
    }
    ++c.s;
  };

  f32x16_t acc[NCB];  // dV^T (weight waves) or dK^T (dS waves)
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = zero16();
  const float c2 = p.scale_log2;

  auto qtile = [&](int s) FA_INLINE { return smem + (s % NB) * 2 * TILE; };
  auto stats = [&](int s) FA_INLINE { return svec + (s % NB) * 2 * SV; };
  const uint32_t lane_off = 4u * lane;
  // copies of the tiles of step s (Q, dO; rows past Nq re-read the last row) and of
  // their LSE2 (wave 0) and D (wave 1) rows, spread over the 4 waves
  auto issue = [&](int s, const Cur& c) FA_INLINE {
    const size_t hbase = (size_t)(b * p.Hq + kvh * p.g + c.hs) * p.Nq;
    const int i0 = cur_i0(c);
    const uint32_t m0t = lds_addr(qtile(s));
    tile_load_m0<D, BMQ, NW>(p.q + hbase * D, i0, p.Nq, m0t, wu, lane_off);
    tile_load_m0<D, BMQ, NW>(p.dO + hbase * D, i0, p.Nq, m0t + 2 * TILE, wu, lane_off);
    if (wu < 2) vec_load_async((wu ? p.dvec : p.lse2v) + hbase, i0, p.Nq - 1, stats(s) + wu * SV, lane);
  };

  // Both roles: LDS byte offsets of the row operand (Q for S, dO for dP) and of the
  // transposed operand (dO^T for dV, Q^T for dK) within a step's pair of tiles.
  const uint32_t rowoff = role_b ? 2u * TILE : 0u, troff = role_b ? 0u : 2u * TILE;
  const int tr_row = 4 * hi + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  static_assert(TL::shifts_ok(BMQ), "LDS reads add row offsets as constants");

  // dV/dK operands of the second 16 queries of the previous step, carried into the
  // next one (zero before the first step)
  bf16x8_t gcar[NCB], pcar;
  {
    const u32x4_t z = {0, 0, 0, 0};
    pcar = __builtin_bit_cast(bf16x8_t, z);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) gcar[cb] = pcar;
  }

  // One step: the 32-query slice of one tile. MASK: the weight wave masks (causal
  // diagonal, rows past Nq); the dS wave needs no mask (masked weights are 0).
  auto step = [&](auto role_tag, auto mask_tag, int s, int i0) FA_INLINE {
    constexpr bool RB = decltype(role_tag)::value;
    constexpr bool MASK = decltype(mask_tag)::value;
    const uint16_t* T = qtile(s);
    const uint32_t sbase = opaque(lds_addr(T) + 2 * TL::row(l32) + 16 * hi + rowoff);
    const uint32_t tbase = opaque(lds_addr(T) + 2 * (TL::row(tr_row) + tr_col) + troff);
    const uint32_t lbase = opaque(lds_addr(stats(s)) + 16 * hi + (RB ? 4 * SV : 0));
    u32x4_t* xb = &xbuf[kw][s & 1][0][0];

    bf16x8_t ra[NDC];     // row operands of S or dP
    bf16x8_t ga[2][NCB];  // transposed operands of a 16-query half
    f32x16_t X;           // S or dP
    f32x4_t st[4];        // LSE2 or D of the slice's rows
    bf16x8_t pc[2];       // P or dS (bf16, B-operand layout)

    auto rd_row = [&](int j0, int n) FA_INLINE {
#pragma unroll
      for (int j = j0; j < j0 + n; ++j) ra[j] = lds_read8_at(sbase + 2 * 16 * j);
    };
    auto mm_x = [&](int j0, int n) FA_INLINE {
      if (j0 == 0) X = zero16();
#pragma unroll
      for (int j = j0; j < j0 + n; ++j) X = mfma32x32x16(ra[j], kv[j], X);
    };
    auto rd_st = [&]() FA_INLINE {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) st[rg] = lds_read_f4_at(lbase + 4 * 8 * rg);
    };
    auto rd_g = [&](int kk, int slot) FA_INLINE {
      const int R = 16 * kk;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const uint32_t o0 = tbase + 2 * (TL::row(R) + 32 * cb), o1 = tbase + 2 * (TL::row(R + 8) + 32 * cb);
        ga[slot][cb] = join8(lds_read_tr4_at(o0), lds_read_tr4_at(o1));
      }
    };
    auto mm_g = [&](int kk, int slot) FA_INLINE {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[cb] = mfma32x32x16(ga[slot][cb], pc[kk], acc[cb]);
    };
    // rows 8kk .. 8kk+7 of the slice: weights (weight wave) or dS (dS wave), bf16
    auto vec = [&](int kk) FA_INLINE {
      uint32_t pp[4];
      u32x4_t pw = {0, 0, 0, 0};
      if constexpr (RB) pw = xb[kk * 64 + lane];
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int rg = 2 * kk + rr;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * rg + e;
          if constexpr (!RB) {
            float pr = fast_exp2(fmaf(X[r], c2, -st[rg][e]));
            if (MASK) {
              const int i = i0 + 8 * rg + 4 * hi + e;
              if ((CAUSAL && key > i + p.causal_off) || i >= p.Nq) pr = 0.f;
            }
            v[e] = pr;
          } else {
            const uint32_t wd = pw[2 * rr + (e >> 1)];
            const float pr = __uint_as_float((e & 1) ? (wd & 0xffff0000u) : (wd << 16));
            v[e] = pr * (X[r] - st[rg][e]);
          }
        }
        pp[2 * rr] = pack_bf16x2(v[0], v[1]);
        pp[2 * rr + 1] = pack_bf16x2(v[2], v[3]);
      }
      const u32x4_t pu = {pp[0], pp[1], pp[2], pp[3]};
      if constexpr (!RB) xb[kk * 64 + lane] = pu;
      pc[kk] = __builtin_bit_cast(bf16x8_t, pu);
    };
    auto interleave = [&](auto n_tag) FA_INLINE {
#pragma unroll
      for (int i = 0; i < decltype(n_tag)::value; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one matrix op
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // vector ops
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    using IHD = std::integral_constant<int, HD>;
    using INCB = std::integral_constant<int, NCB>;

    // The row reads of this step beside dV/dK of the previous step's second 16 queries
    // (registers only), then S/dP over the two halves of d, the vector work of the
    // first 16 queries, and dV/dK of those beside the vector work of the other 16.
    // The products of those 16 go to the next step (or to the end of the loop).
    rd_row(0, NDC);
    rd_st();
    debug_sync();
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[cb] = mfma32x32x16(gcar[cb], pcar, acc[cb]);
    interleave(INCB());
    mm_x(0, HD);
    rd_g(0, 0);
    interleave(IHD());
    mm_x(HD, HD);
    rd_g(1, 1);
    interleave(IHD());
    vec(0);
    __builtin_amdgcn_sched_barrier(0);
    pin(pc[0]);
    mm_g(0, 0);
    vec(1);
    interleave(INCB());
    pin(pc[1]);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) gcar[cb] = ga[1][cb];
    pcar = pc[1];
    debug_sync();
  };
  // the carried products of the last step
  auto flush = [&]() FA_INLINE {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[cb] = mfma32x32x16(gcar[cb], pcar, acc[cb]);
  };

  Cur cur = {0, 0, 0};
  if (total > 0) {
    issue(0, cur);
    wait_vmem();
  }
  __syncthreads();
  Cur nxt = cur;
  cur_next(nxt);

  // Step s: the weight waves take tile s, the dS waves tile s-1; copies of tile s+1.
  // Both roles pass total + 1 step barriers (and, in the debug build, the same number
  // of extra ones in each step, idle steps included).
  if (!role_b) {
    int s = 0;
    for (; s < total_m; ++s) {
      if (s + 1 < total) issue(s + 1, nxt);
      step(BoolC<false>(), BoolC<true>(), s, cur_i0(cur));
      cur = nxt;
      cur_next(nxt);
      wait_vmem();
      __syncthreads();
    }
    for (; s < total; ++s) {
      if (s + 1 < total) issue(s + 1, nxt);
      step(BoolC<false>(), BoolC<false>(), s, cur_i0(cur));
      cur = nxt;
      cur_next(nxt);
      wait_vmem();
      __syncthreads();
    }
    flush();
    if (total > 0) {  // the dS waves' last step
      debug_sync();
      debug_sync();
      __syncthreads();
    }
  } else {
    if (total > 0) {  // the weight waves' first step
      if (1 < total) issue(1, nxt);
      cur = nxt;
      cur_next(nxt);
      debug_sync();
      debug_sync();
      wait_vmem();
      __syncthreads();
    }
    for (int s = 1; s <= total; ++s) {
      if (s + 1 < total) issue(s + 1, nxt);
      step(BoolC<true>(), BoolC<false>(), s - 1, 0);
      cur = nxt;
      cur_next(nxt);
      wait_vmem();
      __syncthreads();
    }
    flush();
  }

  if (key < p.Nk) {
    uint16_t* out = (role_b ? p.dk : p.dv) + kbase;
    const float f = role_b ? p.scale : 1.f;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int c0 = 32 * cb + 8 * rg + 4 * hi;
        const u32x2_t val = {pack_bf16x2(acc[cb][4 * rg] * f, acc[cb][4 * rg + 1] * f),
                             pack_bf16x2(acc[cb][4 * rg + 2] * f, acc[cb][4 * rg + 3] * f)};
        *(u32x2_t*)(out + c0) = val;
      }
  }
}

}  // namespace
}  // namespace fa
