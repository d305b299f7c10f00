// Split-KV forward for short query blocks (decode), bf16 in/out, for gfx950.
//
// With one query row per head the tiled forward launches only B*Hq workgroups and
// leaves most of the 256 compute units idle while K and V (the whole cost) stream
// from HBM. Here the keys of each (batch, kv-head) are cut into chunks that run in
// separate workgroups (the key/value-block split of "FlashAttention"
// (ruizhehou.github.io), §四.3, taken across workgroups), and a second kernel merges
// the chunk results with the online-softmax rescale rule of §二.2: chunk c leaves a
// normalised output O_c and its log-sum-exp L_c; the merged result is
// O = sum_c exp(L_c - L) O_c with L = log sum_c exp(L_c).
//
// Work is HBM-bound (about one flop per byte per query row). All query rows of the
// kv-head (the GQA group times Nq, at most 16) are handled by the same chunk, so K and
// V are read once. With one row the chunk stays on the vector ALUs
// (splitkv_chunk_kernel): every key row is read by d/8 lanes (16 bytes each,
// coalesced), scores are lane-group dot products finished with xor-shuffles, each lane
// group runs its own online softmax over its share of the keys, and the group states
// are merged through LDS at the end. With several rows that vector work grows with the
// row count and the chunk runs on the matrix cores instead (splitkv_mfma_kernel).
#include "common.h"
#include "kernels.h"

namespace fa {
namespace {

struct SplitParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  float* part_o;    // [B, Hq, Nq, S, D]
  float* part_lse;  // [B, Hq, Nq, S]
  int Hq, Hkv, Nq, Nk, g, rows, splits, chunk, causal_off;
  float scale_log2;
};

constexpr int kUnroll = 4;

template <int D, int RM>
__global__ __launch_bounds__(256) void splitkv_chunk_kernel(SplitParams p) {
  constexpr int LPK = D / 8;            // lanes per key row
  constexpr int NG = 256 / LPK;         // lane groups per workgroup
  __shared__ float gm[NG], gl[NG];
  __shared__ float go[NG * D];          // one row's per-group unnormalised outputs

  const int tid = threadIdx.x, sub = tid % LPK, grp = tid / LPK;
  const int split = blockIdx.x % p.splits;
  const int bkv = blockIdx.x / p.splits;
  const int kvh = bkv % p.Hkv, b = bkv / p.Hkv;
  const int j_begin = split * p.chunk;
  const int j_end = min(p.Nk, j_begin + p.chunk);
  const int R = p.rows;

  // q rows of this kv-head: row r -> head kvh*g + r / Nq, query r % Nq.
  float qv[RM][8];
  int lim[RM];
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    const int rr = r < R ? r : R - 1;
    const int h = kvh * p.g + rr / p.Nq, i = rr % p.Nq;
    const u32x4_t u = ((const u32x4_t*)(p.q + ((size_t)(b * p.Hq + h) * p.Nq + i) * D))[sub];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qv[r][2 * e] = bf16_lo(u[e]) * p.scale_log2;
      qv[r][2 * e + 1] = bf16_hi(u[e]) * p.scale_log2;
    }
    lim[r] = i + p.causal_off;  // causal limit (caller passes a huge offset if non-causal)
  }

  float m[RM], l[RM], acc[RM][8];
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
  }

  const uint16_t* Kg = p.k + (size_t)(b * p.Hkv + kvh) * p.Nk * D;
  const uint16_t* Vg = p.v + (size_t)(b * p.Hkv + kvh) * p.Nk * D;

  for (int jb = j_begin + grp; jb < j_end; jb += NG * kUnroll) {
    u32x4_t kr[kUnroll], vr[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int j = jb + u * NG;
      ok[u] = j < j_end;
      const int jj = ok[u] ? j : j_begin;
      kr[u] = ((const u32x4_t*)(Kg + (size_t)jj * D))[sub];
      vr[u] = ((const u32x4_t*)(Vg + (size_t)jj * D))[sub];
    }
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      if (r >= R) break;
      float s[kUnroll];
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a = fmaf(qv[r][2 * e], bf16_lo(kr[u][e]), a);
          a = fmaf(qv[r][2 * e + 1], bf16_hi(kr[u][e]), a);
        }
#pragma unroll
        for (int off = 1; off < LPK; off <<= 1) a += __shfl_xor(a, off);
        const int j = jb + u * NG;
        s[u] = (ok[u] && j <= lim[r]) ? a : -INFINITY;
        mx = fmaxf(mx, s[u]);
      }
      const float m_new = fmaxf(m[r], mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m[r] - m_use);
      m[r] = m_new;
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[r][e] *= alpha;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const float pu = fast_exp2(s[u] - m_use);
        ps += pu;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[r][2 * e] = fmaf(pu, bf16_lo(vr[u][e]), acc[r][2 * e]);
          acc[r][2 * e + 1] = fmaf(pu, bf16_hi(vr[u][e]), acc[r][2 * e + 1]);
        }
      }
      l[r] = l[r] * alpha + ps;
    }
  }

  // merge the NG lane-group states of this chunk, one query row at a time
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    if (r >= R) break;
    if (sub == 0) {
      gm[grp] = m[r];
      gl[grp] = l[r];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) go[grp * D + sub * 8 + e] = acc[r][e];
    __syncthreads();
    const int h = kvh * p.g + r / p.Nq, i = r % p.Nq;
    const size_t row = (size_t)(b * p.Hq + h) * p.Nq + i;
    for (int c = tid; c < D; c += 256) {
      float M = -INFINITY;
      for (int gI = 0; gI < NG; ++gI) M = fmaxf(M, gm[gI]);
      const float Mu = M == -INFINITY ? 0.f : M;
      float Ls = 0.f, Os = 0.f;
      for (int gI = 0; gI < NG; ++gI) {
        const float wgt = fast_exp2(gm[gI] - Mu);
        Ls = fmaf(gl[gI], wgt, Ls);
        Os = fmaf(go[gI * D + c], wgt, Os);
      }
      p.part_o[(row * p.splits + split) * D + c] = Ls > 0.f ? Os / Ls : 0.f;
      if (c == 0) p.part_lse[row * p.splits + split] = Ls > 0.f ? (Mu + log2f(Ls)) * kLn2 : -INFINITY;
    }
    __syncthreads();
  }
}

// The same chunk results on the matrix cores, for several query rows per kv-head (GQA
// groups, small query blocks): one wave per chunk holds the group's rows as the 32
// columns of Sᵀ = K Qᵀ (rows past the group's are zeros and never stored), streams the
// chunk's keys in tiles of 32 through its own double-buffered LDS tiles (direct copies,
// no barriers: a wave waits only for its own copies), and runs the forward kernel's
// per-tile steps: scores on v_mfma_f32_32x32x16_bf16, masking at the chunk end and the
// causal limit of each row, the online softmax with the lazy rescale, and Oᵀ += Vᵀ Pᵀ
// with Vᵀ read by LDS transpose loads. Row r of a kv-head is query head kvh*g + r/Nq,
// query r % Nq.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(64) void splitkv_mfma_kernel(SplitParams p) {
  using TL = TileLayout<D>;
  constexpr int BN = 32;
  constexpr int TILE = TL::elems(BN);
  constexpr int NDC = D / 16, NCB = D / 32;
  static_assert(TL::shifts_ok(BN), "LDS reads add row offsets as constants");
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * TILE];  // K0 V0 K1 V1

  const int lane = threadIdx.x, l32 = lane & 31, hi = lane >> 5;
  const int split = blockIdx.x % p.splits;
  const int bkv = blockIdx.x / p.splits;
  const int kvh = bkv % p.Hkv, b = bkv / p.Hkv;
  const int j_begin = split * p.chunk;
  const int j_end = min(p.Nk, j_begin + p.chunk);

  const bool rvalid = l32 < p.rows;
  const int rr = rvalid ? l32 : 0;
  const int h = kvh * p.g + rr / p.Nq, qi = rr % p.Nq;
  const int lim = qi + p.causal_off;  // keys j <= lim are visible to this row
  bf16x8_t qreg[NDC];
  {
    const u32x4_t* src = (const u32x4_t*)(p.q + ((size_t)(b * p.Hq + h) * p.Nq + qi) * D + 8 * hi);
    const u32x4_t z = {0, 0, 0, 0};
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) qreg[dc] = __builtin_bit_cast(bf16x8_t, rvalid ? src[2 * dc] : z);
  }

  const uint16_t* Kg = p.k + (size_t)(b * p.Hkv + kvh) * p.Nk * D;
  const uint16_t* Vg = p.v + (size_t)(b * p.Hkv + kvh) * p.Nk * D;
  const int ntiles = j_end > j_begin ? (j_end - j_begin + BN - 1) / BN : 0;
  auto Kb = [&](int t) FA_INLINE { return smem + (t & 1) * 2 * TILE; };
  const uint32_t lane_off = 4u * lane;
  // rows past Nk re-read the last key row; keys at or past the chunk end are masked
  auto load = [&](int t) FA_INLINE {
    const int j0 = j_begin + t * BN;
    if constexpr (D <= 128) {
      if (j0 + BN <= p.Nk) {
        tile_load_full<D, BN, 1>(Kg, j0, Kb(t), 0, lane_off);
        tile_load_full<D, BN, 1>(Vg, j0, Kb(t) + TILE, 0, lane_off);
        return;
      }
    }
    tile_load_async<D, BN, 1>(Kg, j0, p.Nk, Kb(t), 0, lane);
    tile_load_async<D, BN, 1>(Vg, j0, p.Nk, Kb(t) + TILE, 0, lane);
  };

  const int tr_row = 4 * hi + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const uint32_t srow = 2 * (TL::row(l32) + 8 * hi);
  const uint32_t trow = 2 * (TL::row(tr_row) + tr_col);

  f32x16_t oacc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) oacc[cb] = zero16();
  float m = -INFINITY, lsum = 0.f;
  const float c2 = p.scale_log2;

  if (ntiles > 0) load(0);
  for (int t = 0; t < ntiles; ++t) {
    wait_vmem();  // tile t is in LDS; the buffer of t+1 was last read in step t-1
    if (t + 1 < ntiles) load(t + 1);
    const uint16_t* Ks = Kb(t);
    // Sᵀ = K Qᵀ: one row per lane, keys 8(r/4) + 4*hi + r%4 of the tile
    f32x16_t sc = zero16();
    {
      const uint32_t base = opaque(lds_addr(Ks) + srow);
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) sc = mfma32x32x16(lds_read8_at(base + 32 * dc), qreg[dc], sc);
    }
    const int j0 = j_begin + t * BN;
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = j0 + 8 * (r >> 2) + 4 * hi + (r & 3);
      if (j >= j_end || (CAUSAL && j > lim)) sc[r] = -INFINITY;
      mx = fmaxf(mx, sc[r]);
    }
    mx = xhalf_max(mx) * c2;
    // lazy rescale: the base moves only when some row's max passes it by more than 8
    const bool move = __any(mx > m + 8.f);
    const float m_next = move ? fmaxf(m, mx) : m;
    const float m_use = m_next == -INFINITY ? 0.f : m_next;
    if (move) {
      const float alpha = fast_exp2(m - m_use);
      lsum *= alpha;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[cb][r] *= alpha;
    }
    m = m_next;
    uint32_t pk[8];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = fast_exp2(fmaf(sc[r], c2, -m_use));
      const float p1 = fast_exp2(fmaf(sc[r + 1], c2, -m_use));
      lsum += p0 + p1;
      pk[r >> 1] = pack_bf16x2(p0, p1);
    }
    // Oᵀ += Vᵀ Pᵀ
    const uint32_t vbase = opaque(lds_addr(Ks + TILE) + trow);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const u32x4_t bu = {pk[4 * kk], pk[4 * kk + 1], pk[4 * kk + 2], pk[4 * kk + 3]};
      const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, bu);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const bf16x8_t a = join8(lds_read_tr4_at(vbase + 2 * (TL::row(16 * kk) + 32 * cb)),
                                 lds_read_tr4_at(vbase + 2 * (TL::row(16 * kk + 8) + 32 * cb)));
        oacc[cb] = mfma32x32x16(a, bop, oacc[cb]);
      }
    }
  }

  // normalised chunk output and its log-sum-exp
  const float ltot = xhalf_sum(lsum);
  if (rvalid) {
    const size_t row = (size_t)(b * p.Hq + h) * p.Nq + qi;
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    float* po = p.part_o + (row * p.splits + split) * D;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const f32x4_t v4 = {oacc[cb][4 * rg] * inv, oacc[cb][4 * rg + 1] * inv,
                            oacc[cb][4 * rg + 2] * inv, oacc[cb][4 * rg + 3] * inv};
        *(f32x4_t*)(po + 32 * cb + 8 * rg + 4 * hi) = v4;
      }
    if (hi == 0)
      p.part_lse[row * p.splits + split] = ltot > 0.f ? (m + log2f(ltot)) * kLn2 : -INFINITY;
  }
}

// One wave per output row: merge the chunk results with weights exp(L_c - L).
template <int D>
__global__ __launch_bounds__(256) void splitkv_merge_kernel(SplitParams p, int nrows) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= nrows) return;
  const float* pl = p.part_lse + (size_t)row * p.splits;
  float M = -INFINITY;
  for (int c = lane; c < p.splits; c += 64) M = fmaxf(M, pl[c]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  const float Mu = M == -INFINITY ? 0.f : M;
  float S = 0.f;
  for (int c = lane; c < p.splits; c += 64) S += __expf(pl[c] - Mu);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) S += __shfl_xor(S, off);
  const float inv = S > 0.f ? 1.f / S : 0.f;
  constexpr int PER = D / 64;
  float o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;
  const float* po = p.part_o + (size_t)row * p.splits * D;
  for (int c = 0; c < p.splits; ++c) {
    const float wgt = __expf(pl[c] - Mu) * inv;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = fmaf(wgt, po[(size_t)c * D + lane + 64 * e], o[e]);
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const __bf16 bv = (__bf16)o[e];
    p.o[(size_t)row * D + lane + 64 * e] = __builtin_bit_cast(uint16_t, bv);
  }
  if (lane == 0) p.lse[row] = S > 0.f ? Mu + __logf(S) : -INFINITY;
}

template <int D, int RM>
hipError_t run(const SplitParams& p, int B, hipStream_t st) {
  const long long n = (long long)B * p.Hkv * p.splits;
  if (n > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((splitkv_chunk_kernel<D, RM>), dim3((int)n), dim3(256), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nrows = B * p.Hq * p.Nq;
  hipLaunchKernelGGL((splitkv_merge_kernel<D>), dim3((nrows + 3) / 4), dim3(256), 0, st, p, nrows);
  return hipGetLastError();
}

template <int D>
hipError_t run_mfma(const SplitParams& p, int B, hipStream_t st) {
  const long long n = (long long)B * p.Hkv * p.splits;
  if (n > 0x7fffffffLL || p.rows > 32) return hipErrorInvalidValue;
  if (p.causal_off < 0x3fffffff)
    hipLaunchKernelGGL((splitkv_mfma_kernel<D, true>), dim3((int)n), dim3(64), 0, st, p);
  else
    hipLaunchKernelGGL((splitkv_mfma_kernel<D, false>), dim3((int)n), dim3(64), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nrows = B * p.Hq * p.Nq;
  hipLaunchKernelGGL((splitkv_merge_kernel<D>), dim3((nrows + 3) / 4), dim3(256), 0, st, p, nrows);
  return hipGetLastError();
}

// Measured on MI355X (d = 128): one row per kv-head, B8 H8 Nk32768: vector 5.7 TB/s,
// matrix 5.4; four rows (Hq32 Hkv8, Nk65536): 4.5 vs 5.4; eight rows (Hq32 Hkv4,
// Nk8192): 0.72 vs 5.2.
template <int D>
hipError_t run_rows(const SplitParams& p, int B, hipStream_t st) {
  if (p.rows <= 1) return run<D, 1>(p, B, st);
  return run_mfma<D>(p, B, st);
}

}  // namespace

hipError_t launch_fwd_splitkv(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              uint16_t* o, float* lse, float* part_o, float* part_lse,
                              int splits, const AttnShape& s, hipStream_t st) {
  SplitParams p;
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse; p.part_o = part_o; p.part_lse = part_lse;
  p.Hq = s.Hq; p.Hkv = s.Hkv; p.Nq = s.Nq; p.Nk = s.Nk; p.g = s.Hq / s.Hkv;
  p.rows = p.g * s.Nq;
  p.splits = splits;
  p.chunk = (s.Nk + splits - 1) / splits;
  p.causal_off = s.causal ? s.Nk - s.Nq : 0x3fffffff;
  p.scale_log2 = s.scale * kLog2e;
  switch (s.d) {
    case 64: return run_rows<64>(p, s.B, st);
    case 128: return run_rows<128>(p, s.B, st);
    case 256: return run_rows<256>(p, s.B, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
