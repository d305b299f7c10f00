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
// Work is HBM-bound (about one flop per byte), so it stays on the vector ALUs: in a
// chunk workgroup every key row is read by d/8 lanes (16 bytes each, coalesced),
// scores are lane-group dot products finished with xor-shuffles, and each lane group
// runs its own online softmax over its share of the keys. The group states are
// merged through LDS at the end. All query rows of the kv-head (the GQA group times
// Nq, at most 16) are handled by the same workgroup, so K and V are read once.
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
hipError_t run_rows(const SplitParams& p, int B, hipStream_t st) {
  if (p.rows <= 1) return run<D, 1>(p, B, st);
  if (p.rows <= 4) return run<D, 4>(p, B, st);
  return run<D, 16>(p, B, st);
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
