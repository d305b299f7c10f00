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

// One workgroup = NW waves, each owning QS x 32 query rows, so BM = NW * QS * 32 rows
// share every K/V tile (the per-CU load path from L2 into LDS is a limit at smaller
// BM). Each wave overlaps its own matrix and vector work: on gfx950 the matrix
// instructions of one wave do not overlap the vector instructions of another wave on
// the same SIMD, but do overlap the same wave's independent vector instructions.
template <int D, int BN, int NW, int QS, bool PIPE, bool CAUSAL>
__global__ __launch_bounds__(64 * NW, 1) void fwd_bf16_kernel(FwdParams p) {
  using TL = TileLayout<D>;
  constexpr int RPW = 32 * QS;   // query rows per wave
  constexpr int BM = NW * RPW;   // query rows per workgroup
  constexpr int TILE = TL::elems(BN);
  constexpr int NKB = BN / 32;   // 32-key sub-blocks per tile
  constexpr int NDC = D / 16;    // 16-wide chunks of d (reduction of S)
  constexpr int NCB = D / 32;    // 32-wide column blocks of O

  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;

  int L = xcd_remap(blockIdx.x, gridDim.x);
  int qb = L % p.nqb;
  const int bh = L / p.nqb;
  if (CAUSAL) qb = p.nqb - 1 - qb;
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

  int kend = p.Nk;
  if (CAUSAL) {
    const int lim = q0 + BM + p.causal_off;  // keys < lim may be visible to some row
    kend = lim < kend ? lim : kend;
  }
  const int ntiles = kend > 0 ? (kend + BN - 1) / BN : 0;

  f32x16_t oacc[QS][NCB];
  float m[QS], lsum[QS];
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) oacc[qs][cb] = zero16();
    m[qs] = -INFINITY;
    lsum[qs] = 0.f;
  }
  const float c2 = p.scale_log2;

  auto Kb = [&](int i) { return smem + (i & 1) * TILE; };
  auto Vb = [&](int i) { return smem + (2 + (i & 1)) * TILE; };
  // Rows past the last key re-read the last key row: always finite, and masked to
  // zero weight before they can contribute.
  auto load = [&](const uint16_t* G, int t, uint16_t* dst) {
    tile_load_async<D, BN, NW>(G, t * BN, p.Nk, dst, wu, lane);
  };

  // Transposed-read addressing of V^T inside a 16-key chunk (see common.h):
  // source lane j = lane % 16 points at key row 4*hi + j/4, column 16*((lane/16)%2) + 4*(j%4).
  const int tr_row = 4 * hi + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  // S^T = K Q^T for this wave's rows and one tile of BN keys; each K operand read from
  // LDS feeds the QS query sub-blocks.
  auto compute_s = [&](f32x16_t (&sc)[QS][NKB], const uint16_t* Ks) {
#pragma unroll
    for (int qs = 0; qs < QS; ++qs)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sc[qs][kb] = zero16();
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const bf16x8_t a = lds_read8(Ks + TL::off(32 * kb + l32, 16 * dc + 8 * hi));
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) sc[qs][kb] = mfma32x32x16(a, qreg[qs][dc], sc[qs][kb]);
      }
  };

  // Causal / key-tail mask of tile t (only tiles that cross the diagonal or the end).
  auto mask = [&](f32x16_t (&sc)[QS][NKB], int t) {
    const int j0 = t * BN;
    const bool need_mask = (j0 + BN > p.Nk) || (CAUSAL && (j0 + BN - 1 > w0 + p.causal_off));
    if (need_mask) {
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
    }
  };

  // Online-softmax update with the scores sc, in two parts. softmax_max: row maxima and
  // the lazy-rescale decision (the exponent base m only moves when some row of the wave
  // sees a score more than kRescaleSlack log2 units above it; otherwise the stale base
  // is kept and weights up to 2^kRescaleSlack are accumulated; the final O / l and
  // lse = m + log l use the same base, so the result is unchanged). softmax_exp: the
  // weights, their row sums and their bf16 packing, with no branches, so the caller's
  // independent matrix work can be interleaved with it.
  float m_use[QS];
  auto softmax_max = [&](f32x16_t (&sc)[QS][NKB], float (&alpha)[QS]) {
    bool any_move = false;
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[qs][kb][r]);
      mx = xhalf_max(mx) * c2;
      const bool move = __any(mx > m[qs] + kRescaleSlack);
      any_move |= move;
      const float m_next = move ? fmaxf(m[qs], mx) : m[qs];
      m_use[qs] = (m_next == -INFINITY) ? 0.f : m_next;
      alpha[qs] = fast_exp2(m[qs] - m_use[qs]);  // 1 if the base did not move, 0 on first use
      m[qs] = m_next;
    }
    return any_move;
  };
  auto softmax_exp = [&](f32x16_t (&sc)[QS][NKB], uint32_t (&pk)[QS][NKB][8], const float (&alpha)[QS]) {
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = fast_exp2(fmaf(sc[qs][kb][r], c2, -m_use[qs]));
          const float p1 = fast_exp2(fmaf(sc[qs][kb][r + 1], c2, -m_use[qs]));
          rs += p0 + p1;
          pk[qs][kb][r >> 1] = pack_bf16x2(p0, p1);
        }
      lsum[qs] = fmaf(lsum[qs], alpha[qs], rs);
    }
  };

  auto rescale_o = [&](const float (&alpha)[QS]) {
#pragma unroll
    for (int qs = 0; qs < QS; ++qs)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[qs][cb][r] *= alpha[qs];
  };

  // O^T += V^T P^T for one tile; each V^T operand read from LDS feeds the QS sub-blocks.
  auto pv = [&](const uint32_t (&pk)[QS][NKB][8], const uint16_t* Vs) {
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
        const int vr = 32 * kb + 16 * kk + tr_row;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const bf16x8_t a = join8(lds_read_tr4(Vs + TL::off(vr, tr_col + 32 * cb)),
                                   lds_read_tr4(Vs + TL::off(vr + 8, tr_col + 32 * cb)));
#pragma unroll
          for (int qs = 0; qs < QS; ++qs) oacc[qs][cb] = mfma32x32x16(a, bop[qs], oacc[qs][cb]);
        }
      }
  };

  // Software pipeline, one barrier per step. Entering step t: S_t is in registers,
  // K_{t+1} sits in K buffer (t+1)%2 and V_t in V buffer t%2; the other two buffers
  // are free. Step t starts the direct loads of V_{t+1} and K_{t+2} into them, then
  // issues the matrix products of S_{t+1} together with the vector-ALU softmax of S_t
  // (one basic block, so the two overlap inside the wave), rescales O if the exponent
  // base moved, accumulates V_t^T P_t^T and waits for its loads.
  // A wave skips tiles that lie wholly above its own rows' diagonal; it still takes
  // part in every load and barrier of the workgroup.
  const int wlim = w0 + RPW - 1 + p.causal_off;  // last key any row of this wave sees
  auto visible = [&](int t) { return !CAUSAL || t * BN <= wlim; };

  // Software pipeline, one barrier per step. Entering step t: S_t is in registers,
  // K_{t+1} sits in K buffer (t+1)%2 and V_t in V buffer t%2; the other two buffers
  // are free. Step t starts the direct loads of V_{t+1} and K_{t+2} into them, issues
  // the products of S_{t+1}, runs the softmax of S_t on the vector ALUs (the compiler
  // interleaves the independent parts), accumulates V_t^T P_t^T, and waits for its
  // loads.
  f32x16_t sA[QS][NKB], sB[QS][NKB];
  uint32_t pk[QS][NKB][8];
  if constexpr (!PIPE) {
    // Plain double buffering (one score tile live, for the widest head dim): step t
    // loads tile t+1 into the other buffers while computing S_t, softmax and PV.
    if (ntiles > 0) {
      load(Kg, 0, Kb(0));
      load(Vg, 0, Vb(0));
      wait_vmem();
      __syncthreads();
    }
    for (int t = 0; t < ntiles; ++t) {
      if (t + 1 < ntiles) {
        load(Kg, t + 1, Kb(t + 1));
        load(Vg, t + 1, Vb(t + 1));
      }
      if (visible(t)) {
        compute_s(sA, Kb(t));
        mask(sA, t);
        float alpha[QS];
        if (softmax_max(sA, alpha)) rescale_o(alpha);
        softmax_exp(sA, pk, alpha);
        pv(pk, Vb(t));
      }
      wait_vmem();
      __syncthreads();
    }
  }
  auto step = [&](f32x16_t (&cur)[QS][NKB], f32x16_t (&nxt)[QS][NKB], int t, bool has_next) {
    if (has_next) {
      load(Vg, t + 1, Vb(t + 1));
      if (t + 2 < ntiles) load(Kg, t + 2, Kb(t + 2));
    }
    if (has_next && visible(t + 1)) compute_s(nxt, Kb(t + 1));
    if (visible(t)) {
      mask(cur, t);
      float alpha[QS];
      if (softmax_max(cur, alpha)) rescale_o(alpha);
      softmax_exp(cur, pk, alpha);
      pv(pk, Vb(t));
    }
    if (has_next) {
      wait_vmem();
      __syncthreads();
    }
  };
  if (PIPE && ntiles > 0) {
    load(Kg, 0, Kb(0));
    load(Vg, 0, Vb(0));
    if (ntiles > 1) load(Kg, 1, Kb(1));
    wait_vmem();
    __syncthreads();
    if (visible(0)) compute_s(sA, Kb(0));
    __syncthreads();  // K_0's buffer is refilled in step 0
    int t = 0;
    for (; t + 2 < ntiles; t += 2) {
      step(sA, sB, t, true);
      step(sB, sA, t + 1, true);
    }
    if (t + 1 < ntiles) {
      step(sA, sB, t, true);
      step(sB, sA, t + 1, false);
    } else {
      step(sA, sB, t, false);
    }
  }

  // Epilogue: combine the two half-row sums, normalise once, store O and LSE.
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    const int qrow = w0 + 32 * qs + l32;
    const float ltot = xhalf_sum(lsum[qs]);
    if (qrow < p.Nq) {
      const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
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

template <int D, int BN, int NW, int QS, bool PIPE, bool CAUSAL>
hipError_t run(FwdParams p, long long B, hipStream_t st) {
  constexpr int BM = 32 * NW * QS;
  p.nqb = (p.Nq + BM - 1) / BM;
  const long long nb = (long long)p.nqb * p.Hq * B;
  if (nb > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, BN, NW, QS, PIPE, CAUSAL>), dim3((int)nb), dim3(64 * NW), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           uint16_t* o, float* lse, const AttnShape& s, hipStream_t st) {
  FwdParams p;
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.Hq = s.Hq; p.Hkv = s.Hkv; p.Nq = s.Nq; p.Nk = s.Nk; p.g = s.Hq / s.Hkv;
  p.causal_off = s.Nk - s.Nq;
  p.scale_log2 = s.scale * kLog2e;
  const bool c = s.causal != 0;
  switch (s.d) {
    case 64: return c ? run<64, 64, 8, 1, true, true>(p, s.B, st) : run<64, 64, 8, 1, true, false>(p, s.B, st);
    case 128: return c ? run<128, 64, 8, 1, true, true>(p, s.B, st) : run<128, 64, 8, 1, true, false>(p, s.B, st);
    case 256: return c ? run<256, 32, 4, 1, false, true>(p, s.B, st) : run<256, 32, 4, 1, false, false>(p, s.B, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
