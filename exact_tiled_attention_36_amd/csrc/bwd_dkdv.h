// The dK/dV kernel of the recompute backward and the parameter block the backward
// kernels share, for gfx950. Included by bwd_dq.h (and so by bwd.hip, which launches
// every head size but 128) and by bwd_dkdv_d128.hip (head size 128, built with a
// compiler option of its own: see that file).
#pragma once
#include "common.h"
#include "kernels.h"

namespace fa {

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dO;
  const float* lse;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* dvec;   // D_i, [B, Hq, Nq]
  float* lse2v;  // lse_i * log2(e), +inf for rows that saw no key, [B, Hq, Nq]
  int Hq, Hkv, Nq, Nk, g, causal_off;
  float scale, scale_log2;
};

// Launch of bwd_dkdv_kernel<128, 64, causal, split> on `grid` workgroups
// (bwd_dkdv_d128.hip).
hipError_t launch_bwd_dkdv_d128(const BwdParams& p, int nkb, int grid, bool causal, bool split,
                                hipStream_t st);

namespace {

// Asynchronous copy of 64 consecutive floats (indices clamped to `last`) into LDS by
// one wave: one direct global->LDS load of 4 bytes per lane.
__device__ __forceinline__ void vec_load_async(const float* G, int i0, int last, float* lds,
                                               int lane) {
  lds_dma_dword(G + min(i0 + lane, last), lds);
}

// ---------------------------------------------------------------------------------
// 2. dK, dV
// ---------------------------------------------------------------------------------
template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

// One workgroup = 4 waves x 32 keys. Each wave keeps its K and V rows in registers
// and walks the (query head, 64-query tile) steps that can see its keys. Q/dO tiles
// and their LSE2/D values are triple buffered in LDS and loaded one step ahead by
// direct global->LDS copies. A step is software-pipelined in 4 sub-phases per
// 32-query slice:
//   S/dP of the slice (d halves 0 and 1), then
//   dV/dK of the previous slice (its 16-query halves) together with the softmax of
//   this slice,
// so the softmax of every slice runs under matrix ops of the wave itself, and only
// one slice's S/dP accumulators are live at a time. The previous slice of a step's
// first slice is the last slice of the step before, which is why tiles stay in LDS
// for two steps. Each sub-phase also reads the LDS operands of the next one.
//
// SPLIT (grids too small to fill the GPU with 128-key workgroups): a workgroup covers
// 64 keys; waves w and w+2 own the same 32 keys and take one 32-query slice each of
// every tile (wave w+2 the upper one), and at the end wave w+2 hands its dK/dV partial
// sums to wave w through LDS. Twice the workgroups for the same work, every SIMD busy.
template <int D, int BMQ, bool CAUSAL, bool SPLIT = false>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BwdParams p, int nkb) {
  using TL = TileLayout<D>;
  constexpr int TILE = TL::elems(BMQ);
  constexpr int NDC = D / 16, NCB = D / 32, HD = NDC / 2;
  static_assert(!SPLIT || BMQ == 64, "split slices need two 32-query slices per tile");
  constexpr int NQS = SPLIT ? 1 : BMQ / 32;  // query slices per wave and tile
  constexpr int BNK = SPLIT ? 64 : 128, NB = 3;
  constexpr int SV = BMQ < 64 ? 64 : BMQ;  // statistics slots per buffer and kind
  static_assert(SV % 64 == 0, "statistics rows per step");

  __shared__ __attribute__((aligned(16))) uint16_t smem[NB * 2 * TILE];
  __shared__ __attribute__((aligned(16))) float svec[NB * 2 * SV];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int l32 = lane & 31, hi = lane >> 5;
  // key block kb is seen by the most query rows at kb = 0
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
  const int key = k0 + 32 * (SPLIT ? (w & 1) : w) + l32;
  const int qoff = SPLIT ? 32 * (wu >> 1) : 0;  // this wave's slice within a tile

  bf16x8_t kreg[NDC], vreg[NDC];
  {
    const size_t base = ((size_t)(b * p.Hkv + kvh) * p.Nk + (key < p.Nk ? key : p.Nk - 1)) * D;
    const u32x4_t* ks = (const u32x4_t*)(p.k + base + 8 * hi);
    const u32x4_t* vs = (const u32x4_t*)(p.v + base + 8 * hi);
    const u32x4_t z = {0, 0, 0, 0};
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      kreg[dc] = __builtin_bit_cast(bf16x8_t, key < p.Nk ? ks[2 * dc] : z);
      vreg[dc] = __builtin_bit_cast(bf16x8_t, key < p.Nk ? vs[2 * dc] : z);
    }
  }
  // nothing may be outstanding in the loops below except the tile copies they issue
  wait_vmem();

  // Query tiles of every head: [qb0, nqb) can see some key of this workgroup. Tiles
  // [qb0, qd) touch the causal diagonal and a ragged last tile [qe, nqb) holds rows
  // past Nq: those steps need masking and run first, in a loop of their own, then the
  // unmasked tiles [qd, qe) from the top down.
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
  const int nu = qe > qd ? qe - qd : 0;        // unmasked tiles per head
  const int nm = (nqb - qb0) - nu;             // masked tiles per head
  const int total_m = nm * p.g, total = (nm + nu) * p.g;
  // Step cursor: step s, head hs in the group and tile counter j, advanced one step at
  // a time without divisions. Masked steps run head by head over the nm masked tiles
  // of each head (j = masked tile); unmasked steps run tile-major from the last tile
  // down, all heads of the group per tile (j = tiles done): the workgroups of a
  // (batch, kv-head) then read the same Q/dO tiles at about the same time, so most
  // copies hit in L2.
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

  f32x16_t dkacc[NCB], dvacc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    dkacc[cb] = zero16();
    dvacc[cb] = zero16();
  }
  const float c2 = p.scale_log2;

  auto qtile = [&](int s) FA_INLINE { return smem + (s % NB) * 2 * TILE; };
  auto stats = [&](int s) FA_INLINE { return svec + (s % NB) * 2 * SV; };
  // Copies of step s: Q and dO tiles (PPW pieces of 256 bytes per wave each) and the
  // LSE2/D rows. Rows past Nq re-read the last row; the softmax of a step that
  // reaches past Nq zeroes their P and dS. dma_piece(s, ..., j) issues this wave's
  // j-th piece, j < 2*PPW, so a step can spread the copies of the next one over its
  // sub-phases.
  constexpr int PPW = BMQ * D / 128 / 4;
  const uint32_t lane_off = 4u * lane;
  struct StepPos {
    const uint16_t* q;   // first row of the head's Q / dO
    const uint16_t* dO;
    const float* lse2;
    const float* dvec;
    int i0;
  };
  auto pos_of = [&](const Cur& c) FA_INLINE {
    const size_t hbase = (size_t)(b * p.Hq + kvh * p.g + c.hs) * p.Nq;
    StepPos sp;
    sp.q = p.q + hbase * D;
    sp.dO = p.dO + hbase * D;
    sp.lse2 = p.lse2v + hbase;
    sp.dvec = p.dvec + hbase;
    sp.i0 = cur_i0(c);
    return sp;
  };
  // D = 128: the LDS address of row wu + 4i is that of row wu plus a constant (checked
  // below); the base passes through opaque_s() once per step (m0q), so the compiler
  // does not keep one scalar register per row and buffer (they spilled into vector
  // lanes in the split form)
  constexpr auto wave_independent = []() {
    for (int w = 0; w < 4; ++w)
      for (int i = 0; i < PPW; ++i)
        if (TL::row(w + 4 * i) - TL::row(w) != TL::row(4 * i) - TL::row(0)) return false;
    return true;
  };
  static_assert(D != 128 || wave_independent(), "row offsets of a wave's pieces depend on the wave");
  auto dma_piece = [&](int s, const StepPos& ps, int j, uint32_t m0q) FA_INLINE {
    const uint16_t* G = j < PPW ? ps.q : ps.dO;
    uint16_t* tile = qtile(s) + (j < PPW ? 0 : TILE);
    const int k = wu + 4 * (j % PPW);  // piece of the tile (uniform)
    if constexpr (D == 64) {
      // piece k = rows 2k and 2k+1
      const int r = 2 * k + (lane >> 5);
      lds_dma_dword(G + (size_t)min(ps.i0 + r, p.Nq - 1) * D + 2 * (lane & 31),
                    tile + TL::row(2 * k));
    } else {
      static_assert(D == 128, "one piece per row");
      const int jj = j % PPW;
      const uint32_t m0 = m0q + (j < PPW ? 0u : 2u * TILE) + 2u * (TL::row(4 * jj) - TL::row(0));
      lds_dma_row_imm<0>(G + (size_t)min(ps.i0 + k, p.Nq - 1) * D, lane_off, m0);
    }
  };
  // LSE2 rows by waves 0 and 2, D rows by waves 1 and 3 (identical duplicate copies
  // keep the code free of branches)
  auto dma_stats = [&](int s, const StepPos& ps) FA_INLINE {
    float* sv = stats(s) + (wu & 1) * SV;
    const float* src = (wu & 1) ? ps.dvec : ps.lse2;
#pragma unroll
    for (int c = 0; c < SV / 64; ++c) vec_load_async(src, ps.i0 + 64 * c, p.Nq - 1, sv + 64 * c, lane);
  };
  auto issue_at = [&](int s, const StepPos& ps) FA_INLINE {
    const uint32_t m0q = D == 128 ? opaque_s(lds_addr(qtile(s)) + 2u * TL::row(wu)) : 0u;
#pragma unroll
    for (int j = 0; j < 2 * PPW; ++j) dma_piece(s, ps, j, m0q);
    dma_stats(s, ps);
  };
  // Copies of a tile whose rows all lie below Nq, for D = 128: wave w copies rows
  // w + 16a + 4c (a, c < 4) of Q and dO. The four rows of one a share one M0 value (the
  // LDS address of row w + 16a): row c sits 1296c bytes above it in LDS (4 rows of 256
  // bytes plus 272 of padding, the same for every wave) and 1024c bytes above it in
  // global memory, so the immediate offset is 1296c and the per-lane offset 272c
  // smaller; the global base is lowered by 1024 to keep those offsets non-negative.
  // Each group of four copies costs one M0 write and a few scalar adds.
  static_assert(D != 128 || (TL::row(4) - TL::row(0) == 648 && TL::row(12) - TL::row(8) == 648 &&
                             TL::row(19) - TL::row(3) == 2560),
                "row offsets the grouped copies assume");
  const uint32_t vo0 = lane_off + 1024u, vo1 = lane_off + 1024u - 272u,
                 vo2 = lane_off + 1024u - 544u, vo3 = lane_off + 1024u - 816u;
  auto issue_full = [&](int s, const StepPos& ps) FA_INLINE {
    if constexpr (D == 128 && BMQ == 64) {
      // (the split form passes the base through opaque_s(): its hoisted per-buffer
      // addresses spilled into vector lanes)
      const uint32_t qb0 = (uint32_t)(uintptr_t)(const FA_LDS void*)qtile(s) + 320u * wu;
      const uint32_t qb = SPLIT ? opaque_s(qb0) : qb0;
      const char* gq = (const char*)(ps.q + (size_t)(ps.i0 + wu) * D) - 1024;
      const char* go = (const char*)(ps.dO + (size_t)(ps.i0 + wu) * D) - 1024;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const uint32_t m = qb + 5120u * a;
        lds_dma_row_x4<0, 1296, 2592, 3888>(gq + 4096 * a, vo0, vo1, vo2, vo3, m);
        lds_dma_row_x4<0, 1296, 2592, 3888>(go + 4096 * a, vo0, vo1, vo2, vo3, m + 2 * TILE);
      }
      dma_stats(s, ps);
    } else {
      issue_at(s, ps);
    }
  };

  const int tr_row = 4 * hi + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  // P and dS (bf16, MFMA B-operand layout) of the previous step's last slice
  bf16x8_t pprev[2], dprev[2];
  {
    const u32x4_t z = {0, 0, 0, 0};
    pprev[0] = pprev[1] = dprev[0] = dprev[1] = __builtin_bit_cast(bf16x8_t, z);
  }

  static_assert(TL::shifts_ok(BMQ), "LDS reads add row offsets as constants");
  // byte address of this lane's transposed reads in a Q tile (dO: + 2*TILE bytes)
  auto tr_base = [&](const uint16_t* T) FA_INLINE {
    return opaque(lds_addr(T) + 2 * (TL::row(tr_row + qoff) + tr_col));
  };
  // dV += dO^T P, dK += Q^T dS for rows 16kk.. of slice `sl` of the tile at tb
  auto rd_g = [&](uint32_t tb, int sl, int kk, bf16x8_t* ga, bf16x8_t* gb) FA_INLINE {
    const int R = 32 * sl + 16 * kk;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const uint32_t o0 = tb + 2 * (TL::row(R) + 32 * cb), o1 = tb + 2 * (TL::row(R + 8) + 32 * cb);
      ga[cb] = join8(lds_read_tr4_at(o0 + 2 * TILE), lds_read_tr4_at(o1 + 2 * TILE));
      gb[cb] = join8(lds_read_tr4_at(o0), lds_read_tr4_at(o1));
    }
  };
  auto mm_g = [&](const bf16x8_t* ga, const bf16x8_t* gb, bf16x8_t pbv, bf16x8_t dbv) FA_INLINE {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      dvacc[cb] = mfma32x32x16(ga[cb], pbv, dvacc[cb]);
      dkacc[cb] = mfma32x32x16(gb[cb], dbv, dkacc[cb]);
    }
  };

  // MASK: the step touches the causal diagonal or reaches past the last query row.
  // issue_next: the copies of the next step's tiles, issued right behind the step's
  // first operand reads, so their address work overlaps the reads' latency (issued
  // before the reads, after the barrier, they delayed the step's first products)
  auto step = [&](auto mask_tag, int s, int i0, auto&& issue_next) FA_INLINE {
    constexpr bool MASK = decltype(mask_tag)::value;
    const uint16_t* Qs = qtile(s);
    const uint16_t* Qp = s > 0 ? qtile(s - 1) : Qs;  // with P = dS = 0 at s = 0
    // per-lane LDS byte bases of this step's reads (constants are added to them)
    const uint32_t sbase = opaque(lds_addr(Qs) + 2 * TL::row(l32 + qoff) + 16 * hi);
    const uint32_t tcur = tr_base(Qs), tprev = tr_base(Qp);
    const uint32_t lbase = opaque(lds_addr(stats(s)) + 16 * hi + 4 * qoff);

    bf16x8_t sa[2][HD], sb[2][HD];    // Q and dO row operands of an S/dP sub-phase
    bf16x8_t ga[2][NCB], gb[2][NCB];  // dO^T and Q^T operands of a dV/dK sub-phase
    f32x4_t lv[2][2], dv[2][2];       // LSE2 and D of the rows of a softmax quarter
    f32x16_t S, dP;
    bf16x8_t pc[NQS][2], dsc[NQS][2];

    auto rd_s = [&](int qs, int half) FA_INLINE {
#pragma unroll
      for (int j = 0; j < HD; ++j) {
        const uint32_t a = sbase + 2 * (TL::row(32 * qs) + 16 * (half * HD + j));
        sa[half][j] = lds_read8_at(a);
        sb[half][j] = lds_read8_at(a + 2 * TILE);
      }
    };
    auto mm_s = [&](int half) FA_INLINE {
      if (half == 0) {
        S = zero16();
        dP = zero16();
      }
#pragma unroll
      for (int j = 0; j < HD; ++j) {
        S = mfma32x32x16(sa[half][j], kreg[half * HD + j], S);
        dP = mfma32x32x16(sb[half][j], vreg[half * HD + j], dP);
      }
    };
    auto rd_ld = [&](int qs, int kk) FA_INLINE {
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int rg = 2 * kk + rr;
        lv[kk][rr] = lds_read_f4_at(lbase + 4 * (32 * qs + 8 * rg));
        dv[kk][rr] = lds_read_f4_at(lbase + 4 * (SV + 32 * qs + 8 * rg));
      }
    };
    // accumulator rows 8kk .. 8kk+7 of the slice: P and dS rounded to bf16
    auto soft = [&](int qs, int kk) FA_INLINE {
      uint32_t pp[4], dd[4];
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int rg = 2 * kk + rr;
        float pv[4], dsv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * rg + e;
          float pr = fast_exp2(fmaf(S[r], c2, -lv[kk][rr][e]));
          if (MASK) {
            const int i = i0 + qoff + 32 * qs + 8 * rg + 4 * hi + e;
            if ((CAUSAL && key > i + p.causal_off) || i >= p.Nq) pr = 0.f;
          }
          pv[e] = pr;
          dsv[e] = pr * (dP[r] - dv[kk][rr][e]);
        }
        pp[2 * rr] = pack_bf16x2(pv[0], pv[1]);
        pp[2 * rr + 1] = pack_bf16x2(pv[2], pv[3]);
        dd[2 * rr] = pack_bf16x2(dsv[0], dsv[1]);
        dd[2 * rr + 1] = pack_bf16x2(dsv[2], dsv[3]);
      }
      const u32x4_t pu = {pp[0], pp[1], pp[2], pp[3]};
      const u32x4_t du = {dd[0], dd[1], dd[2], dd[3]};
      pc[qs][kk] = __builtin_bit_cast(bf16x8_t, pu);
      dsc[qs][kk] = __builtin_bit_cast(bf16x8_t, du);
    };
    auto interleave = [&]() FA_INLINE {
#pragma unroll
      for (int i = 0; i < NDC; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one matrix op
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // vector ops
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    rd_s(0, 0);
    issue_next();
    __builtin_amdgcn_sched_barrier(0);
    debug_sync();
#pragma unroll
    for (int qs = 0; qs < NQS; ++qs) {
      // previous slice: the last one of the step before, or qs-1 of this step
      const uint32_t tg = qs == 0 ? tprev : tcur;
      const int sg = qs == 0 ? NQS - 1 : qs - 1;
      mm_s(0);
      rd_s(qs, 1);
      interleave();
      mm_s(1);
      rd_g(tg, sg, 0, ga[0], gb[0]);
      rd_ld(qs, 0);
      interleave();
      mm_g(ga[0], gb[0], qs == 0 ? pprev[0] : pc[qs - 1][0], qs == 0 ? dprev[0] : dsc[qs - 1][0]);
      rd_g(tg, sg, 1, ga[1], gb[1]);
      rd_ld(qs, 1);
      soft(qs, 0);
      interleave();
      // keep the softmax in this region: its results are used only in the next
      // step, and the compiler would otherwise sink it past the loop's branches
      pin(pc[qs][0]);
      pin(dsc[qs][0]);
      mm_g(ga[1], gb[1], qs == 0 ? pprev[1] : pc[qs - 1][1], qs == 0 ? dprev[1] : dsc[qs - 1][1]);
      if (qs + 1 < NQS) rd_s(qs + 1, 0);
      soft(qs, 1);
      interleave();
      pin(pc[qs][1]);
      pin(dsc[qs][1]);
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      pprev[kk] = pc[NQS - 1][kk];
      dprev[kk] = dsc[NQS - 1][kk];
    }
    debug_sync();
  };

  Cur cur = {0, 0, 0};
  if (total > 0) {
    issue_at(0, pos_of(cur));
    wait_vmem();
  }
  __syncthreads();

  // Step s copies the tiles of step s+1 into buffer (s+1)%3, behind its own first
  // operand reads (tiles of the unmasked loop lie wholly below Nq). cur positions step
  // s, nxt step s+1.
  Cur nxt = cur;
  cur_next(nxt);
  int s = 0;
  for (; s < total_m; ++s) {
    step(BoolC<true>(), s, cur_i0(cur), [&]() FA_INLINE {
      if (s + 1 < total) issue_at(s + 1, pos_of(nxt));
    });
    cur = nxt;
    cur_next(nxt);
    wait_vmem();
    __syncthreads();
  }
  for (; s < total; ++s) {
    step(BoolC<false>(), s, cur_i0(cur), [&]() FA_INLINE {
      if (s + 1 < total) issue_full(s + 1, pos_of(nxt));
    });
    cur = nxt;
    cur_next(nxt);
    wait_vmem();
    __syncthreads();
  }
  // dV/dK of the last slice of the last step
  if (total > 0) {
    const uint32_t tb = tr_base(qtile(total - 1));
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8_t ga[NCB], gb[NCB];
      rd_g(tb, NQS - 1, kk, ga, gb);
      mm_g(ga, gb, pprev[kk], dprev[kk]);
    }
  }

  if constexpr (SPLIT) {
    // waves 2, 3 hand their partial sums to waves 0, 1 (the tiles are no longer read)
    __syncthreads();
    f32x16_t* xfer = (f32x16_t*)smem + ((w & 1) * 2 * NCB) * 64 + lane;
    if (wu >= 2) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        xfer[cb * 64] = dkacc[cb];
        xfer[(NCB + cb) * 64] = dvacc[cb];
      }
    }
    __syncthreads();
    if (wu >= 2) return;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      dkacc[cb] += xfer[cb * 64];
      dvacc[cb] += xfer[(NCB + cb) * 64];
    }
  }
  if (key < p.Nk) {
    const size_t base = ((size_t)(b * p.Hkv + kvh) * p.Nk + key) * D;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int c0 = 32 * cb + 8 * rg + 4 * hi;
        const u32x2_t kv = {pack_bf16x2(dkacc[cb][4 * rg] * p.scale, dkacc[cb][4 * rg + 1] * p.scale),
                            pack_bf16x2(dkacc[cb][4 * rg + 2] * p.scale, dkacc[cb][4 * rg + 3] * p.scale)};
        const u32x2_t vv = {pack_bf16x2(dvacc[cb][4 * rg], dvacc[cb][4 * rg + 1]),
                            pack_bf16x2(dvacc[cb][4 * rg + 2], dvacc[cb][4 * rg + 3])};
        *(u32x2_t*)(p.dk + base + c0) = kv;
        *(u32x2_t*)(p.dv + base + c0) = vv;
      }
  }
}

}  // namespace
}  // namespace fa
