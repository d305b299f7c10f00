// Forward attention with float32 inputs and float32 arithmetic (no rounding of the
// probabilities), for callers that need fp32 accuracy. Same algorithm as the bf16
// kernel ("FlashAttention" (ruizhehou.github.io), §二.1 tiling, §二.2 online softmax,
// §四.1 deferred normalisation), on the vector ALUs:
//  * one workgroup = 64 query rows; four lanes share a row, each holding a quarter
//    of its d columns (column c belongs to lane c % 4 of the quad), so one score is a
//    quad-wide dot product finished by two xor-shuffles;
//  * 32-key tiles of K and V are staged through LDS, zero-padded to a multiple of 4
//    columns; the tile's scores go through LDS as well, so the quad can split the
//    exponentials and every lane can read all 32 weights for its output columns.
#include "common.h"
#include "kernels.h"

namespace fa {
namespace {

constexpr int kF32Rows = 64;
constexpr int kF32Keys = 32;

struct F32Params {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int Hq, Hkv, Nq, Nk, d, g, nqb, causal_off, causal;
  float scale_log2;
};

template <int NC>
__global__ __launch_bounds__(256) void fwd_f32_kernel(F32Params p) {
  constexpr int W = 4 * NC;  // padded row width in LDS
  __shared__ float Ks[kF32Keys * W];
  __shared__ float Vs[kF32Keys * W];
  __shared__ float Ps[kF32Rows * (kF32Keys + 1)];
  const int tid = threadIdx.x, part = tid & 3, qi = tid >> 2;
  const int d = p.d, d4 = d >> 2;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  int qb = L % p.nqb;
  const int bh = L / p.nqb;
  if (p.causal) qb = p.nqb - 1 - qb;
  const int h = bh % p.Hq, b = bh / p.Hq, kvh = h / p.g;
  const int q0 = qb * kF32Rows;
  const int qrow = q0 + qi;
  const float* Qg = p.q + (size_t)(b * p.Hq + h) * p.Nq * d;
  const float* Kg = p.k + (size_t)(b * p.Hkv + kvh) * p.Nk * d;
  const float* Vg = p.v + (size_t)(b * p.Hkv + kvh) * p.Nk * d;

  float qv[NC], acc[NC];
  {
    const int qr = qrow < p.Nq ? qrow : p.Nq - 1;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = part + 4 * i;
      qv[i] = c < d ? Qg[(size_t)qr * d + c] * p.scale_log2 : 0.f;
      acc[i] = 0.f;
    }
  }
  int kend = p.Nk;
  if (p.causal) {
    const int lim = q0 + kF32Rows + p.causal_off;
    kend = lim < kend ? lim : kend;
  }
  const int lim_row = p.causal ? qrow + p.causal_off : 0x7fffffff;
  float m = -INFINITY, l = 0.f;
  float* prow = Ps + qi * (kF32Keys + 1);

  for (int j0 = 0; j0 < kend; j0 += kF32Keys) {
    __syncthreads();
    for (int c = tid; c < kF32Keys * NC; c += 256) {
      const int r = c / NC, col = c % NC, j = j0 + r;
      f32x4_t kk = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (j < p.Nk && col < d4) {
        kk = ((const f32x4_t*)(Kg + (size_t)j * d))[col];
        vv = ((const f32x4_t*)(Vg + (size_t)j * d))[col];
      }
      *(f32x4_t*)(Ks + r * W + 4 * col) = kk;
      *(f32x4_t*)(Vs + r * W + 4 * col) = vv;
    }
    __syncthreads();
    // scores (base-2 scaled): each quad lane takes a quarter of the columns
    float mx = -INFINITY;
    for (int jj = 0; jj < kF32Keys; ++jj) {
      const float* kr = Ks + jj * W + part;
      float sp = 0.f;
#pragma unroll
      for (int i = 0; i < NC; ++i) sp = fmaf(qv[i], kr[4 * i], sp);
      sp += __shfl_xor(sp, 1);
      sp += __shfl_xor(sp, 2);
      const int j = j0 + jj;
      const float sv = (j < p.Nk && j <= lim_row) ? sp : -INFINITY;
      mx = fmaxf(mx, sv);
      if (part == (jj & 3)) prow[jj] = sv;
    }
    const float m_new = fmaxf(m, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m - m_use);
    m = m_new;
    __syncthreads();
    float rs = 0.f;
    for (int jj = part; jj < kF32Keys; jj += 4) {
      const float pv = exp2f(prow[jj] - m_use);
      prow[jj] = pv;
      rs += pv;
    }
    rs += __shfl_xor(rs, 1);
    rs += __shfl_xor(rs, 2);
    l = l * alpha + rs;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NC; ++i) acc[i] *= alpha;
    for (int jj = 0; jj < kF32Keys; ++jj) {
      const float pv = prow[jj];
      const float* vr = Vs + jj * W + part;
#pragma unroll
      for (int i = 0; i < NC; ++i) acc[i] = fmaf(pv, vr[4 * i], acc[i]);
    }
  }
  if (qrow < p.Nq) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* orow = p.o + ((size_t)(b * p.Hq + h) * p.Nq + qrow) * d;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = part + 4 * i;
      if (c < d) orow[c] = acc[i] * inv;
    }
    if (part == 0)
      p.lse[(size_t)(b * p.Hq + h) * p.Nq + qrow] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
  }
}

template <int NC>
hipError_t run(const F32Params& p, int n, hipStream_t st) {
  hipLaunchKernelGGL((fwd_f32_kernel<NC>), dim3(n), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o,
                          float* lse, const AttnShape& s, hipStream_t st) {
  F32Params p;
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.Hq = s.Hq; p.Hkv = s.Hkv; p.Nq = s.Nq; p.Nk = s.Nk; p.d = s.d; p.g = s.Hq / s.Hkv;
  p.nqb = (s.Nq + kF32Rows - 1) / kF32Rows;
  p.causal_off = s.Nk - s.Nq;
  p.causal = s.causal != 0;
  p.scale_log2 = s.scale * kLog2e;
  const long long nb = (long long)p.nqb * s.Hq * s.B;
  if (nb > 0x7fffffffLL) return hipErrorInvalidValue;
  const int n = (int)nb;
  if (s.d <= 64) return run<16>(p, n, st);
  if (s.d <= 128) return run<32>(p, n, st);
  return run<64>(p, n, st);
}

}  // namespace fa
