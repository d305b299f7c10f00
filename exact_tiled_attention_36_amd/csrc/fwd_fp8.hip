// Forward attention with FP8 (OCP E4M3) Q, K, V and per-tensor scales, for gfx950.
//
// Same method and pipeline as the bf16 forward (tiling, online softmax with deferred
// normalisation and the lazy rescale: "FlashAttention" (ruizhehou.github.io) §二 and
// §四.1), with both products on v_mfma_scale_f32_32x32x64_f8f6f4 (FP8 operands, unit
// block scales): four times the bf16 instruction's work in twice its cycles. The
// low-precision forward the wiki lists for the third version ("FlashAttention"
// (newton.com.tw), 發展歷程) is the motivation; its scaling recipe is not on the pages,
// so this entry point takes plain per-tensor scales: the true inputs are
// q = descale_q * Q8, k = descale_k * K8, v = descale_v * V8.
//
// Lane layouts (v_mfma_scale_f32_32x32x64_f8f6f4 with FP8 A and B): lane l holds 32
// bytes of A row l%32 and 32 bytes of B column l%32; the 64 reduction positions split
// 32/32 between the lane halves h = l/32 (which 32 is free as long as A and B agree);
// D has the bf16 instruction's layout, D[8(r/4)+4h+r%4][l%32].
//  * S^T = K Q^T: A = K rows (two 16-byte LDS reads per lane: bytes 64c + 32h .. +31),
//    B = Q^T (the same 32 bytes of the lane's query row, in registers).
//  * O^T += V^T P^T: B = P^T. After S a lane holds the weights of keys 8u + 4h + 0..3
//    (u = 0..3) of each 32-key block, packed four FP8 to a dword; two v_permlane32_swap
//    per block leave lane half h holding keys 16h .. 16h+15 in order. A = V^T comes
//    from V's natural [key][d] LDS tile by ds_read_b64_tr_b8: within each 16 lanes,
//    destination lane i receives byte i%8 of source lanes 2e + i/8 (e = 0..7), so with
//    source lane j pointing at row r0 + j/2, column c0 + 8(j%2), lane i gets column
//    c0 + i of rows r0 .. r0+7. Two such reads give a lane's 16 keys of one block.
//  * P is rounded to E4M3 (round to nearest even) before the product; the lazy rescale
//    keeps weights at most 2^8, inside E4M3's range (448). Row sums use the unrounded
//    fp32 weights, so lse is the fp32 one; O carries the rounding of P.
#include "common.h"
#include "kernels.h"

namespace fa {
namespace {

constexpr float kRescaleSlackF8 = 8.f;

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));

template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

// LDS layout of a [rows][RB] byte tile (RB = head dim in bytes, rows a multiple of 16).
// Two access patterns, on the bank model of 64 four-byte banks serving 16 lanes of a
// 16-byte read or 32 lanes of an 8-byte read per cycle:
//   (a) 16-byte reads, 16 lanes at 16 consecutive rows and one 16-byte column chunk;
//   (b) transposed 8-byte reads, 32 lanes covering 8 consecutive rows (aligned to 8)
//       by 32 bytes (two adjacent chunks).
// Rows are grouped in 256-byte pieces (256/RB rows each, contiguous as in global
// memory, so one direct global->LDS copy per wave fills a piece). Within 16 rows, piece
// m starts at 16-byte slot t(m) = 2m (first half of the pieces) or 2m - 1 (second
// half), mod 16: the first 8 rows start on even slots, the next 8 on odd ones, which
// makes (a) and (b) conflict-free. Pieces never overlap because t only grows; the
// pattern repeats every 16 rows (1280, 2304 or 4608 bytes for RB = 64, 128, 256).
template <int RB>
struct F8Tile {
  static_assert(RB == 64 || RB == 128 || RB == 256, "head dim in bytes");
  static constexpr int RPP = 256 / RB;   // rows per piece
  static constexpr int P = 16 / RPP;     // pieces per 16 rows
  // end of the last piece, 256 (P - 1) + 16 t(P - 1) + 256, rounded up to 256 bytes
  static constexpr int PERIOD = (288 * P - 48 + 255) / 256 * 256;
  static constexpr int bytes(int rows) { return (rows / 16) * PERIOD; }
  __host__ __device__ static constexpr int row(int r) {
    const int m = (r & 15) / RPP;
    const int t = m < P / 2 ? 2 * m : 2 * m - 1;
    return (r >> 4) * PERIOD + 256 * m + 16 * t + (r % RPP) * RB;
  }
  // row(R + r) - row(r) for the lane rows r in [r0, r0 + n), or -1 if not constant
  static constexpr int shift(int R, int r0, int n) {
    const int d = row(R + r0) - row(r0);
    for (int r = r0; r < r0 + n; ++r)
      if (row(R + r) - row(r) != d) return -1;
    return d;
  }
};

// Asynchronous copy of a [ROWS][RB] byte tile (rows j0.. of G, clamped to nrows-1) into
// an F8Tile, one 256-byte piece per wave instruction; waves take every NW-th piece.
// The LDS address of piece i of wave wu is that of the wave's first piece plus a
// constant (checked for every wave at compile time). At d = 64 and 256 the first one
// passes through opaque_s(), so the compiler forms each piece's address in the loop
// instead of keeping one scalar register per piece and buffer: at d = 256 those spilled
// (62-65 scalar registers into vector lanes, 16-28 bytes of scratch per lane; now 8-16,
// outside the loop), and the forward runs 4.5 % faster at B2 H16 N4096 d256 causal and
// 2 % at d = 64. At d = 128 the hoisted form is 1 % faster and is kept.
template <int RB, int NW, int NI>
struct F8PieceOffsets {
  using TL = F8Tile<RB>;
  static constexpr int off(int w, int i) { return TL::row((w + NW * i) * TL::RPP) - TL::row(w * TL::RPP); }
  static constexpr bool wave_independent() {
    for (int i = 0; i < NI; ++i)
      for (int w = 1; w < NW; ++w)
        if (off(w, i) != off(0, i)) return false;
    return true;
  }
};
template <int RB, int ROWS, int NW>
__device__ __forceinline__ void f8_tile_load(const uint8_t* G, int j0, int nrows, uint8_t* lds,
                                             int wu, int lane) {
  using TL = F8Tile<RB>;
  constexpr int NSEG = ROWS * RB / 256;
  constexpr int LPR = RB / 4;  // lanes per row
  static_assert(NSEG % NW == 0, "pieces must split evenly over the waves");
  using PO = F8PieceOffsets<RB, NW, NSEG / NW>;
  static_assert(PO::wave_independent(), "LDS offsets must not depend on the wave");
  if constexpr (RB == 128) {
#pragma unroll
    for (int i = 0; i < NSEG / NW; ++i) {
      const int k = wu + NW * i;
      const int r = k * TL::RPP + lane / LPR;
      const uint8_t* src = G + (size_t)min(j0 + r, nrows - 1) * RB + 4 * (lane % LPR);
      lds_dma_dword(src, lds + TL::row(k * TL::RPP));
    }
  } else {
    const uint32_t m0w = opaque_s(lds_addr(lds) + (uint32_t)TL::row(wu * TL::RPP));
#pragma unroll
    for (int i = 0; i < NSEG / NW; ++i) {
      const int k = wu + NW * i;
      const int r = k * TL::RPP + lane / LPR;
      const uint8_t* src = G + (size_t)min(j0 + r, nrows - 1) * RB + 4 * (lane % LPR);
      lds_dma_dword_m0(src, m0w + (uint32_t)PO::off(0, i));
    }
  }
}

struct Fp8Params {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  uint16_t* o;
  float* lse;
  int Hq, Hkv, Nq, Nk, g, nqb, causal_off;
  float c2;         // scale * descale_q * descale_k * log2(e)
  float descale_v;
};

__device__ __forceinline__ f32x16_t mfma_f8(i32x8_t a, i32x8_t b, f32x16_t c) {
  // cbsz = blgp = 0: both operands FP8 E4M3; E8M0 block scales 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0x7f7f7f7f, 0,
                                                         0x7f7f7f7f);
}

// The compiler pads a vector read of v_mfma_scale_f32_32x32x64_f8f6f4's result (FP8
// operands) with as few as 19 wait states; measured on the GPU, the accumulator register
// read first after the kernel's last product then sometimes still held its old value.
// Where a result is read right after the product with no barrier between (after the
// last tile, and the first tile's scores), 32 more wait states are added explicitly.
__device__ __forceinline__ void mfma_result_guard() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7");
}

__device__ __forceinline__ i32x2_t lds_read_tr8_at(uint32_t a) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((FA_LDS i32x2_t*)(uintptr_t)a);
}
__device__ __forceinline__ u32x4_t lds_read16_at(uint32_t a) {
  return *(const FA_LDS u32x4_t*)(uintptr_t)a;
}

// KS = 2 (d <= 128, grids too small to fill the GPU): the NW waves form two groups that
// own the same rows and take one half of the key tiles each, in LDS buffers of their
// own; at the end the second group hands its O, base m and row sums to the first through
// LDS, which merges them (rescale to the larger base) before the one division.
template <int D, int BN, int NW, bool CAUSAL, int KS = 1>
__global__ __launch_bounds__(64 * NW, 1) void fwd_fp8_kernel(Fp8Params p) {
  using TL = F8Tile<D>;
  static_assert(KS == 1 || (KS == 2 && NW == 8 && D <= 128), "key split of the 8-wave form");
  constexpr int WG = NW / KS;  // waves per key group
  constexpr int BM = 32 * WG;
  constexpr int TILE = TL::bytes(BN);
  constexpr int NKB = BN / 32;   // 32-key blocks per tile
  constexpr int NDQ = D / 64;    // 64-byte chunks of d (reduction of S)
  constexpr int NCB = D / 32;    // 32-wide column blocks of O
  static_assert(BN == 64, "one PV product covers the 64 keys of a tile");
  // operand reads add row offsets as constants to a per-lane base
  static_assert(TL::shift(32, 0, 32) >= 0, "32-row shift");
  static_assert(TL::shift(8, 0, 8) >= 0 && TL::shift(8, 16, 8) == TL::shift(8, 0, 8),
                "8-row shift of the transposed reads");
  static_assert(TL::row(16) == TL::PERIOD, "16-row period");

  __shared__ __attribute__((aligned(16))) uint8_t smem[KS * 4 * TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wall = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ks = KS == 1 ? 0 : wall / WG;     // key group (uniform)
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
  const int w0 = q0 + 32 * wu;

  const uint8_t* Qg = p.q + (size_t)(b * p.Hq + h) * p.Nq * D;
  const uint8_t* Kg = p.k + (size_t)(b * p.Hkv + kvh) * p.Nk * D;
  const uint8_t* Vg = p.v + (size_t)(b * p.Hkv + kvh) * p.Nk * D;

  // Q^T operand: lane (query l32, half h) holds bytes 64c + 32h .. +31 of its row
  i32x8_t qreg[NDQ];
  {
    const int qrow = w0 + l32;
    const int qr = qrow < p.Nq ? qrow : p.Nq - 1;
    const u32x4_t* src = (const u32x4_t*)(Qg + (size_t)qr * D + 32 * hi);
#pragma unroll
    for (int c = 0; c < NDQ; ++c) {
      const u32x4_t lo = src[4 * c], hv = src[4 * c + 1];
      qreg[c] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                        (int)hv[0], (int)hv[1], (int)hv[2], (int)hv[3]};
    }
  }
  wait_vmem();

  int kend = p.Nk;
  if (CAUSAL) {
    const int lim = q0 + BM + p.causal_off;  // keys < lim may be visible to some row
    kend = lim < kend ? lim : kend;
  }
  const int ntiles_all = kend > 0 ? (kend + BN - 1) / BN : 0;
  int tfull_all = p.Nk / BN;  // tiles [0, tfull) are visible to every row of the workgroup
  if (CAUSAL) {
    const int lim = q0 + p.causal_off + 1;
    tfull_all = min(tfull_all, lim > 0 ? lim / BN : 0);
  }
  tfull_all = min(tfull_all, ntiles_all);
  // KS = 2: group g takes global tiles [g*nh, g*nh + nh) as its local tiles 0..nh-1 (the
  // second group's last one may lie past the keys: copied from the last key row and
  // masked away); both groups run the same steps, since they share the barriers
  const int ntiles = KS == 1 ? ntiles_all : (ntiles_all + 1) / 2;
  const int t0 = ks * ntiles;  // global index of local tile 0
  const int tfull = KS == 1 ? tfull_all : min(min(tfull_all, ntiles), max(tfull_all - ntiles, 0));

  f32x16_t oacc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) oacc[cb] = zero16();
  float m = -INFINITY, lsum = 0.f, m_use = 0.f, alpha = 1.f;
  const float c2 = p.c2;

  auto Kb = [&](int i) FA_INLINE { return smem + (4 * ks + (i & 1)) * TILE; };
  auto Vb = [&](int i) FA_INLINE { return smem + (4 * ks + 2 + (i & 1)) * TILE; };
  // rows past the last key re-read the last key row; their scores are masked (t local)
  auto load = [&](const uint8_t* G, int t, uint8_t* dst) FA_INLINE {
    f8_tile_load<D, BN, WG>(G, (t0 + t) * BN, p.Nk, dst, wu, lane);
  };

  // per-lane LDS byte offsets inside a tile
  const uint32_t srow = TL::row(l32) + 32 * hi;
  const int jj = lane & 15;
  const uint32_t trow = TL::row(16 * hi + (jj >> 1)) + 8 * (jj & 1) + 16 * ((lane >> 4) & 1);

  // S^T = K Q^T for one tile
  auto compute_s = [&](f32x16_t (&sc)[NKB], const uint8_t* Ks) FA_INLINE {
    const uint32_t base = opaque(lds_addr(Ks) + srow);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) sc[kb] = zero16();
#pragma unroll
    for (int c = 0; c < NDQ; ++c)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const uint32_t a = base + TL::shift(32 * kb, 0, 32) + 64 * c;
        const u32x4_t lo = lds_read16_at(a), hv = lds_read16_at(a + 16);
        const i32x8_t av = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                            (int)hv[0], (int)hv[1], (int)hv[2], (int)hv[3]};
        sc[kb] = mfma_f8(av, qreg[c], sc[kb]);
      }
  };

  // O^T += V^T P^T for one tile. pk[kb][u]: FP8 weights of keys 32kb + 8u + 4h + 0..3.
  auto pv = [&](const uint32_t (&pk)[NKB][4], const uint8_t* Vs) FA_INLINE {
    // v_permlane32_swap(x, y) exchanges x of the upper half with y of the lower half:
    // swapping (u=0 | u=2) and (u=1 | u=3) gives half 0 keys 0-3, 4-7 | 8-11, 12-15
    // and half 1 keys 16-19, 20-23 | 24-27, 28-31.
    uint32_t bq[NKB][4];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const auto s0 = __builtin_amdgcn_permlane32_swap(pk[kb][0], pk[kb][2], false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(pk[kb][1], pk[kb][3], false, false);
      bq[kb][0] = s0[0];
      bq[kb][1] = s0[1];
      bq[kb][2] = s1[0];
      bq[kb][3] = s1[1];
    }
    static_assert(NKB == 2, "one MFMA takes two 32-key blocks");
    const i32x8_t bop = {(int)bq[0][0], (int)bq[0][1], (int)bq[0][2], (int)bq[0][3],
                         (int)bq[1][0], (int)bq[1][1], (int)bq[1][2], (int)bq[1][3]};
    const uint32_t base = opaque(lds_addr(Vs) + trow);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      // keys 32kb + 16h + 8x + 0..7, x = 0, 1: the order of the B operand's bytes
      i32x2_t r[NKB][2];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int x = 0; x < 2; ++x)
          r[kb][x] = lds_read_tr8_at(base + TL::shift(32 * kb, 0, 32) +
                                     (x ? TL::shift(8, 0, 8) : 0) + 32 * cb);
      const i32x8_t aop = {r[0][0][0], r[0][0][1], r[0][1][0], r[0][1][1],
                           r[1][0][0], r[1][0][1], r[1][1][0], r[1][1][1]};
      oacc[cb] = mfma_f8(aop, bop, oacc[cb]);
    }
  };

  auto mask = [&](f32x16_t (&sc)[NKB], int t) FA_INLINE {  // t local
    const int j0 = (t0 + t) * BN;
    const int lim = CAUSAL ? w0 + l32 + p.causal_off : 0x7fffffff;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = j0 + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (j >= p.Nk || j > lim) sc[kb][r] = -INFINITY;
      }
  };
  auto smax = [&](f32x16_t (&sc)[NKB]) FA_INLINE {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
    mx = xhalf_max(mx) * c2;
    const bool move = __any(mx > m + kRescaleSlackF8);
    const float m_next = move ? fmaxf(m, mx) : m;
    m_use = (m_next == -INFINITY) ? 0.f : m_next;
    alpha = fast_exp2(m - m_use);
    m = m_next;
    return move;
  };
  // weights 2^(s c2 - m_use), their fp32 row sum, and their FP8 packing
  auto sexp = [&](f32x16_t (&sc)[NKB], uint32_t (&pk)[NKB][4]) FA_INLINE {
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w[e] = fast_exp2(fmaf(sc[kb][4 * u + e], c2, -m_use));
          rs += w[e];
        }
        uint32_t x = __builtin_amdgcn_cvt_pk_fp8_f32(w[0], w[1], 0, false);
        x = __builtin_amdgcn_cvt_pk_fp8_f32(w[2], w[3], x, true);
        pk[kb][u] = x;
      }
    lsum = fmaf(lsum, alpha, rs);
  };
  auto rescale = [&]() FA_INLINE {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[cb][r] *= alpha;
  };

  // Step t, as in the bf16 forward: a pending rescale of O, then one scheduling region
  // with the copies of K_{t+2} and V_{t+1}, S_{t+1} (matrix) beside P_t (vector), and
  // O += V_t^T P_t (matrix) beside the mask and row max of S_{t+1} (vector); then the
  // copies' wait and a barrier.
  f32x16_t sA[NKB], sB[NKB];
  uint32_t pk[NKB][4];
  bool move = false;
  auto step = [&](auto mask_tag, auto last_tag, f32x16_t (&cur)[NKB], f32x16_t (&nxt)[NKB],
                  int t) FA_INLINE {
    constexpr bool MASK = decltype(mask_tag)::value, LAST = decltype(last_tag)::value;
    if (move) rescale();
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
    } else {
      mfma_result_guard();
    }
  };

  if (ntiles > 0) {
    load(Kg, 0, Kb(0));
    load(Kg, 1, Kb(1));
    load(Vg, 0, Vb(0));
    wait_vmem();
    __syncthreads();
    compute_s(sA, Kb(0));
    __builtin_amdgcn_sched_barrier(0);
    mfma_result_guard();
    if (tfull == 0) mask(sA, 0);
    move = smax(sA);
    __syncthreads();  // K_0's buffer is refilled in step 0
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
        for (int r = 0; r < 16; ++r) xf[(16 * cb + r) * 64] = oacc[cb][r];
      xf[(NCB * 16) * 64] = m;
      xf[(NCB * 16 + 1) * 64] = lsum;
    }
    __syncthreads();
    if (ks == 1) return;
    const float m1 = xf[(NCB * 16) * 64], l1 = xf[(NCB * 16 + 1) * 64];
    const float mt = fmaxf(m, m1);
    const float mb = mt == -INFINITY ? 0.f : mt;
    const float a0 = fast_exp2(m - mb), a1 = fast_exp2(m1 - mb);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[cb][r] = oacc[cb][r] * a0 + xf[(16 * cb + r) * 64] * a1;
    lsum = lsum * a0 + l1 * a1;
    m = mt;
  }
  // Epilogue: combine the half-row sums, normalise once (with the V descale), store.
  {
    const int qrow = w0 + l32;
    const float ltot = xhalf_sum(lsum);
    if (qrow < p.Nq) {
      const float inv = ltot > 0.f ? p.descale_v / ltot : 0.f;
      if (hi == 0) {
        p.lse[(size_t)(b * p.Hq + h) * p.Nq + qrow] =
            ltot > 0.f ? (m + log2f(ltot)) * kLn2 : -INFINITY;
      }
      uint16_t* orow = p.o + ((size_t)(b * p.Hq + h) * p.Nq + qrow) * D;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int c0 = 32 * cb + 8 * rg + 4 * hi;
          u32x2_t val = {pack_bf16x2(oacc[cb][4 * rg] * inv, oacc[cb][4 * rg + 1] * inv),
                         pack_bf16x2(oacc[cb][4 * rg + 2] * inv, oacc[cb][4 * rg + 3] * inv)};
          *(u32x2_t*)(orow + c0) = val;
        }
    }
  }
}

// 8 waves (two per SIMD) up to d = 128; d = 256 needs one wave per SIMD for its registers.
// Grids too small to give every compute unit a 256-row workgroup (SMALL) take 128-row
// workgroups at d <= 128: 8 waves in two groups over half of the key tiles each (KS = 2).
// Measured at B1 H8 N2048 d128 causal: 46.7 us with 256-row workgroups, 36.9 with
// 4-wave 128-row ones, 29.2 with the key split (small grids at d = 64 and 128 -36 to
// -40 % in all).
template <int D, bool CAUSAL, bool SMALL = false>
hipError_t run_fp8(Fp8Params p, long long B, hipStream_t st) {
  constexpr bool KS2 = SMALL && D <= 128;
  constexpr int NW = D == 256 ? 4 : 8, BM = KS2 ? 128 : 32 * NW;
  p.nqb = (p.Nq + BM - 1) / BM;
  const long long nb = (long long)p.nqb * p.Hq * B;
  if (nb > 0x7fffffffLL) return hipErrorInvalidValue;
  if constexpr (KS2)
    hipLaunchKernelGGL((fwd_fp8_kernel<D, 64, 8, CAUSAL, 2>), dim3((int)nb), dim3(512), 0, st, p);
  else
    hipLaunchKernelGGL((fwd_fp8_kernel<D, 64, NW, CAUSAL>), dim3((int)nb), dim3(64 * NW), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const uint8_t* q, const uint8_t* k, const uint8_t* v, uint16_t* o,
                          float* lse, float descale_q, float descale_k, float descale_v,
                          const AttnShape& s, hipStream_t st) {
  Fp8Params p;
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.Hq = s.Hq; p.Hkv = s.Hkv; p.Nq = s.Nq; p.Nk = s.Nk; p.g = s.Hq / s.Hkv;
  p.causal_off = s.Nk - s.Nq;
  p.c2 = s.scale * descale_q * descale_k * kLog2e;
  p.descale_v = descale_v;
  const bool c = s.causal != 0;
  const bool small = (long long)((s.Nq + 255) / 256) * s.Hq * s.B < 256;
  switch (s.d) {
    case 64:
      if (small) return c ? run_fp8<64, true, true>(p, s.B, st) : run_fp8<64, false, true>(p, s.B, st);
      return c ? run_fp8<64, true>(p, s.B, st) : run_fp8<64, false>(p, s.B, st);
    case 128:
      if (small) return c ? run_fp8<128, true, true>(p, s.B, st) : run_fp8<128, false, true>(p, s.B, st);
      return c ? run_fp8<128, true>(p, s.B, st) : run_fp8<128, false>(p, s.B, st);
    case 256: return c ? run_fp8<256, true>(p, s.B, st) : run_fp8<256, false>(p, s.B, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
