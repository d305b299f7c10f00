// Ablation forward: the FlashAttention-1 loop order (not the production path).
//
// "FlashAttention" (ruizhehou.github.io) §二 / §三 describe the first version: the
// outer loop runs over K/V blocks and the inner loop over Q blocks; for every (K/V
// block, Q block) pair the Q block, the output block O_i and its statistics m_i, l_i
// are read from HBM, updated with the online-softmax rule of §二.2 (O kept normalised
// after every block), and written back. Work is parallel over batch and head only
// (§四.2 names this as what the second version fixes). This kernel reproduces that
// structure on gfx950 so that its time can be set beside the production kernel's:
//   * grid: one workgroup (4 waves) per (batch, query head);
//   * K/V block j (64 keys) sits in LDS, block j+1 is copied in meanwhile;
//   * inner loop over 128-row Q blocks, wave w owning rows 32w..32w+31: Q from global
//     memory, O (fp32) and m, l from a workspace, S = K_j Q^T and O^T += V^T P^T on
//     MFMA exactly as in the production kernel, then O, m, l back to the workspace;
//   * a final pass writes O in bf16 and LSE = m + ln l.
// The workspace keeps O in the accumulator's register order, so every lane reads and
// writes only its own elements.
#include "common.h"
#include "kernels.h"

namespace fa {
namespace {

struct V1Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  float* ow;   // [B*Hq][nqb][4 waves][D/8 chunks][64 lanes][4] fp32
  float* mw;   // [B*Hq][nqb][4][64] running max (log2 units), one copy per lane
  float* lw;   // [B*Hq][nqb][4][64] running row sum, one copy per lane
  int Hq, Hkv, Nq, Nk, g, causal_off, nqb;
  float scale_log2;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void fwd_v1_kernel(V1Params p) {
  using TL = TileLayout<D>;
  constexpr int NW = 4, BM = 32 * NW, BN = 64;
  constexpr int TILE = TL::elems(BN);
  constexpr int NKB = BN / 32, NDC = D / 16, NCB = D / 32, NE4 = NCB * 4;
  static_assert(TL::shifts_ok(BN), "LDS reads add row offsets as constants");

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * 2 * TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int bh = blockIdx.x;
  const int h = bh % p.Hq, b = bh / p.Hq, kvh = h / p.g;
  const uint16_t* Qg = p.q + (size_t)bh * p.Nq * D;
  const uint16_t* Kg = p.k + (size_t)(b * p.Hkv + kvh) * p.Nk * D;
  const uint16_t* Vg = p.v + (size_t)(b * p.Hkv + kvh) * p.Nk * D;
  const int nkb = (p.Nk + BN - 1) / BN;
  const float c2 = p.scale_log2;

  auto Kb = [&](int j) FA_INLINE { return smem + (j & 1) * 2 * TILE; };
  auto load_kv = [&](int j) FA_INLINE {
    tile_load_async<D, BN, NW>(Kg, j * BN, p.Nk, Kb(j), wu, lane);
    tile_load_async<D, BN, NW>(Vg, j * BN, p.Nk, Kb(j) + TILE, wu, lane);
  };
  const int tr_row = 4 * hi + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const uint32_t srow = 2 * (TL::row(l32) + 8 * hi);
  const uint32_t trow = 2 * (TL::row(tr_row) + tr_col);

  // workspace slots of (Q block i, this wave)
  auto slot = [&](int i) FA_INLINE { return ((size_t)bh * p.nqb + i) * NW + wu; };

  load_kv(0);
  wait_vmem();
  __syncthreads();
  for (int j = 0; j < nkb; ++j) {
    if (j + 1 < nkb) load_kv(j + 1);
    const uint32_t kbase = opaque(lds_addr(Kb(j)) + srow);
    const uint32_t vbase = opaque(lds_addr(Kb(j) + TILE) + trow);
    for (int i = 0; i < p.nqb; ++i) {
      const int r0 = i * BM + 32 * wu;
      // block pairs wholly above the diagonal are skipped (never at j = 0, where every
      // Q block's workspace is initialised)
      if (CAUSAL && j > 0 && j * BN > i * BM + BM - 1 + p.causal_off) continue;
      const int qrow = r0 + l32;
      bf16x8_t qreg[NDC];
      {
        const int qr = qrow < p.Nq ? qrow : p.Nq - 1;
        const u32x4_t* src = (const u32x4_t*)(Qg + (size_t)qr * D + 8 * hi);
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) qreg[dc] = __builtin_bit_cast(bf16x8_t, src[2 * dc]);
      }
      const size_t sl = slot(i);
      f32x16_t oacc[NCB];
      float m = -INFINITY, l = 0.f;
      if (j > 0) {
        const f32x4_t* src = (const f32x4_t*)(p.ow + sl * NE4 * 256) + lane;
#pragma unroll
        for (int e4 = 0; e4 < NE4; ++e4) {
          const f32x4_t x = src[e4 * 64];
#pragma unroll
          for (int u = 0; u < 4; ++u) oacc[e4 >> 2][4 * (e4 & 3) + u] = x[u];
        }
        m = p.mw[sl * 64 + lane];
        l = p.lw[sl * 64 + lane];
      } else {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) oacc[cb] = zero16();
      }
      // S^T = K_j Q^T
      f32x16_t sc[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sc[kb] = zero16();
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          sc[kb] = mfma32x32x16(lds_read8_at(kbase + 2 * (TL::row(32 * kb) + 16 * dc)), qreg[dc], sc[kb]);
      // causal / key-tail mask
      const int lim = CAUSAL ? qrow + p.causal_off : 0x7fffffff;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j * BN + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (key >= p.Nk || key > lim) sc[kb][r] = -INFINITY;
        }
      // online-softmax update, O kept normalised (§二.2)
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
      mx = xhalf_max(mx) * c2;
      const float m_new = fmaxf(m, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m - m_use);
      float pv[NKB][16], rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          pv[kb][r] = fast_exp2(fmaf(sc[kb][r], c2, -m_use));
          rs += pv[kb][r];
        }
      const float l_new = fmaf(alpha, l, xhalf_sum(rs));
      const float inv = l_new > 0.f ? 1.f / l_new : 0.f;
      const float oscale = alpha * l * inv;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[cb][r] *= oscale;
      // O^T += V_j^T (P / l_new)^T
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          uint32_t pk[4];
#pragma unroll
          for (int u = 0; u < 4; ++u)
            pk[u] = pack_bf16x2(pv[kb][8 * kk + 2 * u] * inv, pv[kb][8 * kk + 2 * u + 1] * inv);
          const u32x4_t bu = {pk[0], pk[1], pk[2], pk[3]};
          const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, bu);
          const int R = 32 * kb + 16 * kk;
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            const bf16x8_t a = join8(lds_read_tr4_at(vbase + 2 * (TL::row(R) + 32 * cb)),
                                     lds_read_tr4_at(vbase + 2 * (TL::row(R + 8) + 32 * cb)));
            oacc[cb] = mfma32x32x16(a, bop, oacc[cb]);
          }
        }
      // back to the workspace
      {
        f32x4_t* dst = (f32x4_t*)(p.ow + sl * NE4 * 256) + lane;
#pragma unroll
        for (int e4 = 0; e4 < NE4; ++e4) {
          f32x4_t x;
#pragma unroll
          for (int u = 0; u < 4; ++u) x[u] = oacc[e4 >> 2][4 * (e4 & 3) + u];
          dst[e4 * 64] = x;
        }
        p.mw[sl * 64 + lane] = m_new;
        p.lw[sl * 64 + lane] = l_new;
      }
    }
    wait_vmem();
    __syncthreads();
  }

  // final pass: O (already normalised) in bf16, LSE = m + ln l
  for (int i = 0; i < p.nqb; ++i) {
    const int qrow = i * BM + 32 * wu + l32;
    const size_t sl = slot(i);
    const float m = p.mw[sl * 64 + lane], l = p.lw[sl * 64 + lane];
    if (qrow < p.Nq) {
      if (hi == 0) p.lse[(size_t)bh * p.Nq + qrow] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
      const f32x4_t* src = (const f32x4_t*)(p.ow + sl * NE4 * 256) + lane;
      uint16_t* orow = p.o + ((size_t)bh * p.Nq + qrow) * D;
#pragma unroll
      for (int e4 = 0; e4 < NE4; ++e4) {
        const f32x4_t x = src[e4 * 64];
        const int c0 = 32 * (e4 >> 2) + 8 * (e4 & 3) + 4 * hi;
        const u32x2_t val = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
        *(u32x2_t*)(orow + c0) = val;
      }
    }
  }
}

template <int D, bool CAUSAL>
hipError_t run_v1(const V1Params& p, int B, hipStream_t st) {
  const long long nb = (long long)B * p.Hq;
  if (nb > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_v1_kernel<D, CAUSAL>), dim3((int)nb), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace

// O: 128 rows x d per Q block; m and l: 4 waves x 64 lanes per Q block each
size_t fwd_v1_workspace_floats(const AttnShape& s) {
  const size_t nqb = (size_t)(s.Nq + 127) / 128;
  return (size_t)s.B * s.Hq * nqb * (128 * (size_t)s.d + 2 * 256);
}

hipError_t launch_fwd_v1(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                         float* lse, float* ws, const AttnShape& s, hipStream_t st) {
  V1Params p;
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.Hq = s.Hq; p.Hkv = s.Hkv; p.Nq = s.Nq; p.Nk = s.Nk; p.g = s.Hq / s.Hkv;
  p.causal_off = s.Nk - s.Nq;
  p.nqb = (s.Nq + 127) / 128;
  p.scale_log2 = s.scale * kLog2e;
  const size_t n_o = (size_t)s.B * s.Hq * p.nqb * 128 * s.d;
  const size_t n_s = (size_t)s.B * s.Hq * p.nqb * 256;
  p.ow = ws;
  p.mw = ws + n_o;
  p.lw = ws + n_o + n_s;
  const bool c = s.causal != 0;
  switch (s.d) {
    case 64: return c ? run_v1<64, true>(p, s.B, st) : run_v1<64, false>(p, s.B, st);
    case 128: return c ? run_v1<128, true>(p, s.B, st) : run_v1<128, false>(p, s.B, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
