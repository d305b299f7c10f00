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
//  * one workgroup = 4 waves = 128 query rows; wave w owns rows 32w..32w+31 and keeps
//    them for the whole loop, so m, l and the output never need a cross-wave reduce.
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: K (A operand) comes from LDS with
//    16-byte reads, Q^T (B operand) sits in registers for the whole kernel. In the
//    result each lane holds one query (its column) and 16 of the 32 keys, so the row
//    max/sum are in-lane reductions plus one v_permlane32_swap with lane ^ 32.
//  * O^T += V^T P^T: the exponentiated scores, rounded to bf16, are already laid out
//    as the B operand; V^T (A operand) is read from V's natural [key][d] LDS tile
//    with ds_read_b64_tr_b16. The rescale by exp(m_old - m_new) is a per-lane scalar.
//  * scores are scaled into the base-2 domain (scale * log2 e folded into one FMA)
//    and exponentiated with v_exp_f32.
//  * K/V tiles are double buffered in LDS: the global loads of tile t+1 are issued
//    before tile t is computed and written to the other buffer afterwards; one
//    barrier per tile.
//  * causal: key tiles wholly above the diagonal are never visited; only the tiles
//    that cross the diagonal or the key tail are masked.
//  * grid: one workgroup per (batch, head, row block), ids remapped so consecutive
//    ids stay on one XCD (one L2) and, for causal, the longest row blocks go first.
#include "common.h"
#include "kernels.h"

namespace fa {
namespace {

// Headroom (in log2 units) the running max may lag behind the true row max before
// the accumulators are rescaled: weights stay below 2^8, far inside fp32/bf16 range.
constexpr float kRescaleSlack = 8.f;

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int Hq, Hkv, Nq, Nk, g, nqb, causal_off;
  float scale_log2;
};

template <int D, int BN>
struct FwdTile {
  static constexpr int BM = 128;
  static constexpr int TILE = TileLayout<D>::elems(BN);  // elements per K or V tile
  static constexpr int LPT = BN * D / 8 / 256;      // 16-byte chunks per thread per tensor
  static constexpr int LDS_BYTES = 2 * 2 * TILE * 2;
  static_assert(LPT * 256 * 8 == BN * D, "tile must split evenly over 256 threads");
};

template <int D, int BN, bool CAUSAL>
__global__ __launch_bounds__(256, D == 256 ? 1 : 2) void fwd_bf16_kernel(FwdParams p) {
  using T = FwdTile<D, BN>;
  using TL = TileLayout<D>;
  constexpr int BM = T::BM, LPT = T::LPT;
  constexpr int NKB = BN / 32;   // 32-key sub-blocks per tile
  constexpr int NDC = D / 16;    // 16-wide chunks of d (reduction of S)
  constexpr int NCB = D / 32;    // 32-wide column blocks of O
  constexpr int CPR = D / 8;     // 16-byte chunks per row

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * 2 * T::TILE];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  int L = xcd_remap(blockIdx.x, gridDim.x);
  int qb = L % p.nqb;
  const int bh = L / p.nqb;
  if (CAUSAL) qb = p.nqb - 1 - qb;
  const int h = bh % p.Hq, b = bh / p.Hq;
  const int kvh = h / p.g;
  const int q0 = qb * BM;

  const uint16_t* Qg = p.q + (size_t)(b * p.Hq + h) * p.Nq * D;
  const uint16_t* Kg = p.k + (size_t)(b * p.Hkv + kvh) * p.Nk * D;
  const uint16_t* Vg = p.v + (size_t)(b * p.Hkv + kvh) * p.Nk * D;

  const int qrow = q0 + w * 32 + l32;
  bf16x8_t qreg[NDC];
  {
    const int qr = qrow < p.Nq ? qrow : p.Nq - 1;
    const u32x4_t* src = (const u32x4_t*)(Qg + (size_t)qr * D + 8 * hi);
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) qreg[dc] = __builtin_bit_cast(bf16x8_t, src[2 * dc]);
  }

  int kend = p.Nk;
  if (CAUSAL) {
    const int lim = q0 + BM + p.causal_off;  // keys < lim may be visible to some row
    kend = lim < kend ? lim : kend;
  }
  const int ntiles = kend > 0 ? (kend + BN - 1) / BN : 0;

  f32x16_t oacc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) oacc[cb] = zero16();
  float m = -INFINITY, lsum = 0.f;
  const float c2 = p.scale_log2;

  u32x4_t kreg[LPT], vreg[LPT];
  // Rows past the last key re-read the last key row: always finite, and masked to
  // zero weight before they can contribute, so no branch is needed here.
  auto gload = [&](int t) {
    const int j0 = t * BN;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int c = tid + 256 * i, row = c / CPR, col = c % CPR;
      const int j = min(j0 + row, p.Nk - 1);
      kreg[i] = ((const u32x4_t*)(Kg + (size_t)j * D))[col];
      vreg[i] = ((const u32x4_t*)(Vg + (size_t)j * D))[col];
    }
  };
  auto lstore = [&](int buf) {
    uint16_t* Ks = smem + buf * 2 * T::TILE;
    uint16_t* Vs = Ks + T::TILE;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int c = tid + 256 * i, row = c / CPR, col = c % CPR;
      *(FA_LDS u32x4_t*)(Ks + TL::off(row, col * 8)) = kreg[i];
      *(FA_LDS u32x4_t*)(Vs + TL::off(row, col * 8)) = vreg[i];
    }
  };

  if (ntiles > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();

  // Transposed-read addressing of V^T inside a 16-key chunk (see common.h):
  // source lane j = lane % 16 points at key row 4*hi + j/4, column 16*((lane/16)%2) + 4*(j%4).
  const int tr_row = 4 * hi + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) gload(t + 1);
    const uint16_t* Ks = smem + buf * 2 * T::TILE;
    const uint16_t* Vs = Ks + T::TILE;
    const int j0 = t * BN;

    // S^T = K Q^T for this wave's 32 queries and the tile's BN keys.
    f32x16_t s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = zero16();
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        s[kb] = mfma32x32x16(lds_read8(Ks + TL::off(32 * kb + l32, 16 * dc + 8 * hi)), qreg[dc], s[kb]);

    const bool need_mask = (j0 + BN > p.Nk) || (CAUSAL && (j0 + BN - 1 > q0 + p.causal_off));
    if (need_mask) {
      const int lim = CAUSAL ? qrow + p.causal_off : 0x7fffffff;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (j >= p.Nk || j > lim) s[kb][r] = -INFINITY;
        }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = xhalf_max(mx) * c2;
    // Lazy rescale: the exponent base m only moves when some row of the wave sees a
    // score more than kRescaleSlack (log2 units) above it. Otherwise the stale base is
    // kept and weights up to 2^kRescaleSlack are accumulated; the final O / l and
    // lse = m + log l use the same base, so the result is unchanged.
    if (__any(mx > m + kRescaleSlack)) {
      const float m_new = fmaxf(m, mx);
      const float alpha = fast_exp2(m - (m_new == -INFINITY ? 0.f : m_new));
      lsum *= alpha;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[cb][r] *= alpha;
      m = m_new;
    }
    const float m_use = (m == -INFINITY) ? 0.f : m;

    float rs = 0.f;
    uint32_t pk[NKB][8];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = fast_exp2(fmaf(s[kb][r], c2, -m_use));
        const float p1 = fast_exp2(fmaf(s[kb][r + 1], c2, -m_use));
        rs += p0 + p1;
        pk[kb][r >> 1] = pack_bf16x2(p0, p1);
      }
    lsum += rs;

    // O^T += V^T P^T, one 16-key chunk at a time.
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const u32x4_t bu = {pk[kb][4 * kk], pk[kb][4 * kk + 1], pk[kb][4 * kk + 2], pk[kb][4 * kk + 3]};
        const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, bu);
        const int vr = 32 * kb + 16 * kk + tr_row;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const bf16x8_t a = join8(lds_read_tr4(Vs + TL::off(vr, tr_col + 32 * cb)),
                                   lds_read_tr4(Vs + TL::off(vr + 8, tr_col + 32 * cb)));
          oacc[cb] = mfma32x32x16(a, bop, oacc[cb]);
        }
      }

    if (t + 1 < ntiles) lstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: combine the two half-row sums, normalise once, store O and LSE.
  const float ltot = xhalf_sum(lsum);
  if (qrow < p.Nq) {
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
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

template <int D, int BN, bool CAUSAL>
hipError_t run(const FwdParams& p, int nblocks, hipStream_t st) {
  hipLaunchKernelGGL((fwd_bf16_kernel<D, BN, CAUSAL>), dim3(nblocks), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           uint16_t* o, float* lse, const AttnShape& s, hipStream_t st) {
  FwdParams p;
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.Hq = s.Hq; p.Hkv = s.Hkv; p.Nq = s.Nq; p.Nk = s.Nk; p.g = s.Hq / s.Hkv;
  p.nqb = (s.Nq + 127) / 128;
  p.causal_off = s.Nk - s.Nq;
  p.scale_log2 = s.scale * kLog2e;
  const long long nb = (long long)p.nqb * s.Hq * s.B;
  if (nb > 0x7fffffffLL) return hipErrorInvalidValue;
  const int n = (int)nb;
  const bool c = s.causal != 0;
  switch (s.d) {
    case 64: return c ? run<64, 64, true>(p, n, st) : run<64, 64, false>(p, n, st);
    case 128: return c ? run<128, 64, true>(p, n, st) : run<128, 64, false>(p, n, st);
    case 256: return c ? run<256, 32, true>(p, n, st) : run<256, 32, false>(p, n, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
