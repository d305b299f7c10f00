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
// Three kernels on one stream:
//  1. bwd_pre:  D for every query row (HBM-bound row dot products).
//  2. bwd_dkdv: one workgroup per (batch, kv-head, 128 keys); each wave keeps 32 keys
//     of K and V in registers and loops over the group's query heads and the query
//     blocks that can see its keys (diagonal blocks first, then the unmasked ones
//     block by block from the last down, all heads of the group per block, so the
//     group's waves share Q/dO tiles in L2), with Q/dO/LSE/D tiles triple buffered in
//     LDS.
//     S = Q K^T and dP = dO V^T come out with one key per lane, so P and dS (rounded
//     to bf16) feed dV^T += dO^T P and dK^T += Q^T dS directly as B operands; dO^T
//     and Q^T are read with LDS transpose loads.
//  3. bwd_dq:   one workgroup per (batch, head, 32 queries per wave: 256 at d <= 128,
//     128 at d = 256); Q and dO stay in registers, K/V tiles are triple buffered in
//     LDS; S^T and dP^T put one query per lane, so LSE and D are per-lane scalars, and
//     dQ^T += K^T dS^T reads K^T with LDS transpose loads.
// No atomics: every output element is written by exactly one workgroup, so results
// are bitwise reproducible.
#include "common.h"
#include "kernels.h"

namespace fa {
namespace {

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

// ---------------------------------------------------------------------------------
// 1. D_i = sum_c dO_ic * O_ic
// ---------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p, int rows) {
  constexpr int LPR = D / 8;        // lanes per row, 8 elements (16 bytes) each
  constexpr int RPB = 256 / LPR;    // rows per workgroup pass
  const int tid = threadIdx.x, sub = tid % LPR;
  for (int row = blockIdx.x * RPB + tid / LPR; row < rows; row += gridDim.x * RPB) {
    const u32x4_t a = ((const u32x4_t*)(p.o + (size_t)row * D))[sub];
    const u32x4_t b = ((const u32x4_t*)(p.dO + (size_t)row * D))[sub];
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = fmaf(bf16_lo(a[i]), bf16_lo(b[i]), acc);
      acc = fmaf(bf16_hi(a[i]), bf16_hi(b[i]), acc);
    }
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) acc += __shfl_xor(acc, off);
    if (sub == 0) {
      p.dvec[row] = acc;
      const float l = p.lse[row];
      p.lse2v[row] = l == -INFINITY ? INFINITY : l * kLog2e;
    }
  }
}

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
template <int D, int BMQ, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BwdParams p, int nkb) {
  using TL = TileLayout<D>;
  constexpr int TILE = TL::elems(BMQ);
  constexpr int NDC = D / 16, NCB = D / 32, NQS = BMQ / 32, HD = NDC / 2;
  constexpr int BNK = 128, NB = 3;
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
  const int key = k0 + 32 * w + l32;

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
  auto dma_piece = [&](int s, const StepPos& ps, int j) FA_INLINE {
    const uint16_t* G = j < PPW ? ps.q : ps.dO;
    uint16_t* tile = qtile(s) + (j < PPW ? 0 : TILE);
    const int k = wu + 4 * (j % PPW);  // piece of the tile (uniform)
    if constexpr (D == 64) {
      // piece k = rows 2k and 2k+1
      const int r = 2 * k + (lane >> 5);
      lds_dma_dword(G + (size_t)min(ps.i0 + r, p.Nq - 1) * D + 2 * (lane & 31),
                    tile + TL::row(2 * k));
    } else {
      constexpr int PPR = D / 128;  // pieces per row
      const int r = k / PPR, c0 = (k % PPR) * 128;
      lds_dma_row(G + (size_t)min(ps.i0 + r, p.Nq - 1) * D + c0, lane_off, tile + TL::row(r) + c0);
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
#pragma unroll
    for (int j = 0; j < 2 * PPW; ++j) dma_piece(s, ps, j);
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
      const uint32_t qb = (uint32_t)(uintptr_t)(const FA_LDS void*)qtile(s) + 320u * wu;
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
    return opaque(lds_addr(T) + 2 * (TL::row(tr_row) + tr_col));
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
  auto step = [&](auto mask_tag, int s, int i0) FA_INLINE {
    constexpr bool MASK = decltype(mask_tag)::value;
    const uint16_t* Qs = qtile(s);
    const uint16_t* Qp = s > 0 ? qtile(s - 1) : Qs;  // with P = dS = 0 at s = 0
    // per-lane LDS byte bases of this step's reads (constants are added to them)
    const uint32_t sbase = opaque(lds_addr(Qs) + 2 * TL::row(l32) + 16 * hi);
    const uint32_t tcur = tr_base(Qs), tprev = tr_base(Qp);
    const uint32_t lbase = opaque(lds_addr(stats(s)) + 16 * hi);

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
            const int i = i0 + 32 * qs + 8 * rg + 4 * hi + e;
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
    __builtin_amdgcn_sched_barrier(0);
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
  };

  Cur cur = {0, 0, 0};
  if (total > 0) {
    issue_at(0, pos_of(cur));
    wait_vmem();
  }
  __syncthreads();

  // Step s copies the tiles of step s+1 into buffer (s+1)%3 first (tiles of the
  // unmasked loop lie wholly below Nq). cur positions step s, nxt step s+1.
  Cur nxt = cur;
  cur_next(nxt);
  int s = 0;
  for (; s < total_m; ++s) {
    if (s + 1 < total) issue_at(s + 1, pos_of(nxt));
    step(BoolC<true>(), s, cur_i0(cur));
    cur = nxt;
    cur_next(nxt);
    wait_vmem();
    __syncthreads();
  }
  for (; s < total; ++s) {
    if (s + 1 < total) issue_full(s + 1, pos_of(nxt));
    step(BoolC<false>(), s, cur_i0(cur));
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

// ---------------------------------------------------------------------------------
// 3. dQ
// ---------------------------------------------------------------------------------
// One workgroup = NW waves x 32 query rows; Q and dO stay in registers, each wave
// owns its rows' dQ. Key tiles of BN rows (K and V) are triple buffered in LDS and
// copied two tiles ahead. Step t is one scheduling region:
//   S, dP of tile t+1 (matrix)       with  dS of tile t (vector),
//   dQ^T += K_t^T dS^T (matrix)      with  mask of tile t+1 (vector),
// then the copies' wait and a barrier. S^T and dP^T put one query per lane, so LSE
// and D are per-lane scalars; dS^T comes out in the B-operand layout of the dQ
// product, and K^T is read with LDS transpose loads.
template <int D, int BN, int NW, bool CAUSAL>
__global__ __launch_bounds__(64 * NW, 1) void bwd_dq_kernel(BwdParams p, int nqb) {
  using TL = TileLayout<D>;
  constexpr int TILE = TL::elems(BN);
  constexpr int NDC = D / 16, NCB = D / 32, NKB = BN / 32;
  constexpr int BM = 32 * NW;    // query rows per workgroup (one 32-row block per wave)
  constexpr int NB = 3;
  static_assert(TL::shifts_ok(BN), "LDS reads add row offsets as constants");

  __shared__ __attribute__((aligned(16))) uint16_t smem[NB * 2 * TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const float lse2 = qvalid ? p.lse2v[rowidx] : INFINITY;
  const float Dv = qvalid ? p.dvec[rowidx] : 0.f;
  // nothing may be outstanding in the loops below except the tile copies they issue
  wait_vmem();

  const uint16_t* Kg = p.k + (size_t)(b * p.Hkv + kvh) * p.Nk * D;
  const uint16_t* Vg = p.v + (size_t)(b * p.Hkv + kvh) * p.Nk * D;
  int kend = p.Nk;
  if (CAUSAL) {
    const int lim = q0 + BM + p.causal_off;
    kend = lim < kend ? lim : kend;
  }
  const int ntiles = kend > 0 ? (kend + BN - 1) / BN : 0;
  // tiles [0, tfull) are wholly visible to every row of the workgroup
  int tfull = p.Nk / BN;
  if (CAUSAL) {
    const int lim = q0 + p.causal_off + 1;
    tfull = min(tfull, lim > 0 ? lim / BN : 0);
  }
  tfull = min(tfull, ntiles);

  f32x16_t dqacc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) dqacc[cb] = zero16();
  const float c2 = p.scale_log2;

  // buffer t%3 holds the K tile of key tile t, followed by its V tile
  auto Kb = [&](int t) FA_INLINE { return smem + (t % NB) * 2 * TILE; };
  // rows past Nk re-read the last key row; the key-tail mask zeroes their weight
  const uint32_t lane_off = 4u * lane;
  auto load_tile = [&](int t) FA_INLINE {
    if constexpr (D <= 128) {
      if ((t + 1) * BN <= p.Nk) {  // whole tile present: scalar-addressed copies
        tile_load_full<D, BN, NW>(Kg, t * BN, Kb(t), wu, lane_off);
        tile_load_full<D, BN, NW>(Vg, t * BN, Kb(t) + TILE, wu, lane_off);
        return;
      }
    }
    tile_load_async<D, BN, NW>(Kg, t * BN, p.Nk, Kb(t), wu, lane);
    tile_load_async<D, BN, NW>(Vg, t * BN, p.Nk, Kb(t) + TILE, wu, lane);
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
  // causal / key-tail mask of key tile t: masked scores give P = dS = 0
  auto mask = [&](f32x16_t (&S)[NKB], int t) FA_INLINE {
    const int j0 = t * BN;
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
    if constexpr (!LAST) compute_sp(sn, pn, t + 1);
    dsoft(sc, pc, dspk);
    dq_mm(dspk, t);
    if constexpr (!LAST && MASK) mask(sn, t + 1);
    __builtin_amdgcn_sched_barrier(0);
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

// stage 0: D = rowsum(dO * O); stage 1: dK, dV; stage 2: dQ; stage -1: all three.
template <int D, int BMQ, int BN, int NWQ, bool CAUSAL>
hipError_t run(const BwdParams& p, int B, int stage, hipStream_t st) {
  if (stage == -1 || stage == 0) {
    const int rows = B * p.Hq * p.Nq;
    constexpr int RPB = 256 / (D / 8);
    int nb = (rows + RPB - 1) / RPB;
    if (nb > 65536) nb = 65536;
    hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3(nb), dim3(256), 0, st, p, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stage == -1 || stage == 1) {
    const int nkb = (p.Nk + 127) / 128;
    const long long n = (long long)nkb * p.Hkv * B;
    if (n > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, BMQ, CAUSAL>), dim3((int)n), dim3(256), 0, st, p, nkb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stage == -1 || stage == 2) {
    const int nqb = (p.Nq + 32 * NWQ - 1) / (32 * NWQ);
    const long long n = (long long)nqb * p.Hq * B;
    if (n > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_dq_kernel<D, BN, NWQ, CAUSAL>), dim3((int)n), dim3(64 * NWQ), 0, st, p, nqb);
    hipError_t e = hipGetLastError();
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
  // dQ grids too small for one 256-row workgroup per compute unit use 128-row ones (4
  // waves): twice the workgroups, no compute unit left idle (dK/dV is unchanged)
  const long long dq256 = (long long)((s.Nq + 255) / 256) * s.Hq * s.B;
  if (dq256 < 256 && (s.d == 64 || s.d == 128)) {
    if (s.d == 64) return c ? run<64, 64, 32, 4, true>(p, s.B, stage, st) : run<64, 64, 32, 4, false>(p, s.B, stage, st);
    return c ? run<128, 64, 32, 4, true>(p, s.B, stage, st) : run<128, 64, 32, 4, false>(p, s.B, stage, st);
  }
  switch (s.d) {
    case 64: return c ? run<64, 64, 32, 8, true>(p, s.B, stage, st) : run<64, 64, 32, 8, false>(p, s.B, stage, st);
    case 128: return c ? run<128, 64, 32, 8, true>(p, s.B, stage, st) : run<128, 64, 32, 8, false>(p, s.B, stage, st);
    case 256: return c ? run<256, 32, 32, 4, true>(p, s.B, stage, st) : run<256, 32, 32, 4, false>(p, s.B, stage, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
