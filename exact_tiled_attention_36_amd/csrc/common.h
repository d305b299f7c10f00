// Device helpers shared by the attention kernels (gfx950 / CDNA4 only).
//
// MFMA used throughout: v_mfma_f32_32x32x16_bf16, D[32x32] += A[32x16] * B[16x32].
// Lane layout (64 lanes, h = lane / 32, n = lane % 32):
//   A operand: lane holds A[n][8h + e], e = 0..7         (row n, 8 consecutive k)
//   B operand: lane holds B[8h + e][n], e = 0..7         (column n, 8 consecutive k)
//   D result : lane holds D[8(r/4) + 4h + (r%4)][n], r = 0..15
// The k index of one MFMA may be any permutation of the 16 reduction positions as
// long as A and B agree; the kernels use that to feed a D result straight back in
// as the next product's B operand.
//
// ds_read_b64_tr_b16 (LDS transpose read, 4 x 16-bit per lane): inside every group
// of 16 lanes, if source lane j supplies the address of 4 consecutive elements
// x_j[0..3], destination lane i receives x_{4e + i/4}[i % 4] for e = 0..3. Pointing
// source lane j at row (r0 + j/4), column (c0 + 4 (j%4)) of a row-major tile hands
// lane i the column c0 + i, rows r0..r0+3: a transposed operand read from a tile
// stored in its natural [row][d] layout.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

#define FA_LDS __attribute__((address_space(3)))
// kernels are written with local lambdas; they must never become real calls
#define FA_INLINE __attribute__((always_inline))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16_t mfma32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Round two floats to bf16 (nearest-even) and pack them, first one in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// 16-byte LDS read (ds_read_b128); `p` must point into a __shared__ array.
__device__ __forceinline__ bf16x8_t lds_read8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *(const FA_LDS u32x4_t*)(p));
}

// Transposed LDS read (ds_read_b64_tr_b16) of 4 bf16; see the header comment.
__device__ __forceinline__ u32x2_t lds_read_tr4(const uint16_t* p) {
  s16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, r);
}

// LDS reads at a byte address. Kernels form a few per-lane base addresses per tile
// and pass them through opaque(), so the compiler cannot re-associate base and
// constant parts (it would otherwise keep one register per distinct address and
// redo the buffer offset for each); the constants then fold into the instructions'
// 16-bit offset field.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const FA_LDS void*)p;
}
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm("" : "+v"(x));
  return x;
}
// The same for a wave-uniform value kept in a scalar register.
__device__ __forceinline__ uint32_t opaque_s(uint32_t x) {
  asm("" : "+s"(x));
  return x;
}
// Marks x as needed here: volatile asm is never moved, so the computation of x cannot
// be sunk past this point (e.g. across a barrier into the next loop iteration).
__device__ __forceinline__ void pin(uint32_t x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void pin(float x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void pin(bf16x8_t x) { asm volatile("" ::"v"(x)); }

__device__ __forceinline__ bf16x8_t lds_read8_at(uint32_t a) {
  return __builtin_bit_cast(bf16x8_t, *(const FA_LDS u32x4_t*)(uintptr_t)a);
}
__device__ __forceinline__ u32x2_t lds_read_tr4_at(uint32_t a) {
  s16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4_t*)(uintptr_t)a);
  return __builtin_bit_cast(u32x2_t, r);
}
__device__ __forceinline__ f32x4_t lds_read_f4_at(uint32_t a) {
  return *(const FA_LDS f32x4_t*)(uintptr_t)a;
}

__device__ __forceinline__ bf16x8_t join8(u32x2_t lo, u32x2_t hi) {
  u32x4_t v = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(bf16x8_t, v);
}

// Exchange with lane (lane ^ 32) and combine: one v_permlane32_swap.
__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 2^x on the FMA units instead of the transcendental unit: x = n + f with n = rint(x),
// |f| <= 1/2 (Cody-Waite style reduction), 2^f by a degree-3 polynomial with minimax
// relative error 8.4e-5 on [-1/2, 1/2] (coefficients fitted by csrc/fit_exp2_poly.py),
// scaled by 2^n with ldexp. x is clamped at -200 first, so -inf (a masked score) gives
// exactly 0 and never a NaN.
__device__ __forceinline__ float poly_exp2(float x) {
  x = fmaxf(x, -200.f);
  const float n = __builtin_rintf(x);
  const float f = x - n;
  float p = fmaf(0.055212993f, f, 0.24271414f);
  p = fmaf(p, f, 0.69326216f);
  p = fmaf(p, f, 0.99991959f);
  return __builtin_amdgcn_ldexpf(p, (int)n);
}

// LDS layout of a [rows][D] bf16 tile (rows a multiple of 16). Every tile is read
// two ways: 16-byte row reads (lanes 0..31 read 32 different rows at one column
// chunk: MFMA A operands) and transposed reads (each 16-lane group reads 4
// consecutive rows x 32 bytes: ds_read_b64_tr_b16). Measured bank-conflict counts on
// gfx950 follow a model of 64 four-byte banks serving 16 lanes of a 16-byte read or
// 32 lanes of an 8-byte read per cycle. In units of 16-byte slots (16 per bank
// cycle), row r is started at slot 4*(r%4) + (r/4)%4 (mod 16): 16 consecutive rows
// then start on 16 different slots (row reads), and 4 consecutive rows x 64 bytes
// cover 16 different slots (transposed reads of two 16-lane groups). Rows stay
// contiguous (for d=64, row pairs), so whole 256-byte pieces can be filled by one
// direct global->LDS load, and every offset is "per-lane row base + constant".
// Padding: 1 KiB per 16 rows (d >= 128) or 512 bytes per 16 rows (d = 64).
template <int D>
struct TileLayout {
  static_assert(D == 64 || D == 128 || D == 256, "head dim");
  static constexpr int elems(int rows) {
    return D == 64 ? (rows / 16) * 1280 : (rows / 16) * (16 * D + 512);
  }
  // element offset of row r. The pattern repeats every 16 rows (8 for the transposed
  // reads' 8-row groups), so row(R + r) - row(r) is the same for every lane row r of
  // the kernels' access patterns; they add it as a constant (checked by shift()).
  __host__ __device__ static constexpr int row(int r) {
    if constexpr (D == 64) {
      const int m = r >> 1;  // row pair, stored contiguously
      const int a = 4 * (m & 1) + 9 * ((m >> 1) & 3) + 32 * (m >> 3);
      return m * 128 + 8 * a + 64 * (r & 1);
    } else {
      const int sl = 4 * (r & 3) + 17 * ((r >> 2) & 3) + 64 * (r >> 4);
      return r * D + 8 * sl;
    }
  }
  __device__ __forceinline__ static int off(int r, int e) { return row(r) + e; }
  // row(R + r) - row(r) for lane rows r < n, or -1 if it depends on r
  static constexpr int shift(int R, int n) {
    const int d = row(R) - row(0);
    for (int r = 0; r < n; ++r)
      if (row(R + r) - row(r) != d) return -1;
    return d;
  }
  // the kernels' patterns in a tile of `rows` rows: 32-row operand reads at multiples
  // of 32, transposed reads of 8-row groups at multiples of 8
  static constexpr bool shifts_ok(int rows) {
    for (int R = 0; R + 32 <= rows; R += 32)
      if (shift(R, 32) < 0) return false;
    for (int R = 0; R + 8 <= rows; R += 8)
      if (shift(R, 8) < 0) return false;
    return row(0) == 0;
  }
};

// Direct global->LDS copy of one dword per lane (global_load_lds_dword): lane i's 4
// bytes from `src` land at LDS byte address lds_base + 4*i; `lds_base` must be
// wave-uniform. Written as inline assembly so that the compiler does not treat the
// copy as an LDS store of unknown address: it would otherwise wait for every such
// copy to land before the next LDS read of the wave, i.e. expose the full memory
// latency of a prefetch that targets a different buffer. Completion is therefore
// the caller's business: wait_vmem() and a workgroup barrier before the buffer is
// read. M0 holds the LDS base; one wait state separates its write from the load.
__device__ __forceinline__ void lds_dma_dword_m0(const void* src, uint32_t m0v) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %0, off"
      :
      : "v"(src), "s"(m0v)
      : "memory", "m0");
}
__device__ __forceinline__ void lds_dma_dword(const void* src, const void* lds_base) {
  lds_dma_dword_m0(src, (uint32_t)(uintptr_t)(const FA_LDS void*)lds_base);
}

// Same copy with a wave-uniform global base and a per-lane byte offset (the saddr
// form): lane i reads gbase + lane_off. With lane_off = 4*lane a wave copies 256
// contiguous bytes at no vector-ALU cost. The caller guarantees that nothing reads the
// destination before its wait_vmem() and barrier, and that no wave still reads it when
// the copy is issued; the memory clobber keeps every other memory access of the wave on
// its side of the copy as well, so that order never rests on how the compiler treats
// volatile asm next to ordinary loads and stores.
__device__ __forceinline__ void lds_dma_row(const void* gbase, uint32_t lane_off,
                                            const void* lds_base) {
  const uint32_t m0v = (uint32_t)(uintptr_t)(const FA_LDS void*)lds_base;
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %0, %1"
      :
      : "v"(lane_off), "s"(gbase), "s"(m0v)
      : "memory", "m0");
}

// Same copy with a scalar base, a per-lane byte offset and an immediate offset IMM
// that the hardware adds to both addresses: lane i reads gbase + lane_off + IMM and
// writes LDS byte lds_m0 + IMM + 4*i.
template <int IMM>
__device__ __forceinline__ void lds_dma_row_imm(const void* gbase, uint32_t lane_off,
                                                uint32_t lds_m0) {
  static_assert(IMM >= 0 && IMM < 4096, "immediate offset range");
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %0, %1 offset:%3"
      :
      : "v"(lane_off), "s"(gbase), "s"(lds_m0), "i"(IMM)
      : "memory", "m0");
}

// Four copies of the saddr form that share one M0 write: copy c reads
// gbase + voff_c + IMM_c and writes LDS lds_m0 + IMM_c + 4*lane. With row strides that
// differ between global memory and LDS, voff_c absorbs the difference.
template <int I0, int I1, int I2, int I3>
__device__ __forceinline__ void lds_dma_row_x4(const void* gbase, uint32_t v0, uint32_t v1,
                                               uint32_t v2, uint32_t v3, uint32_t lds_m0) {
  static_assert(I0 >= 0 && I3 < 4096 && I0 <= I1 && I1 <= I2 && I2 <= I3, "offset range");
  asm volatile(
      "s_mov_b32 m0, %5\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %0, %4 offset:%6\n\t"
      "global_load_lds_dword %1, %4 offset:%7\n\t"
      "global_load_lds_dword %2, %4 offset:%8\n\t"
      "global_load_lds_dword %3, %4 offset:%9"
      :
      : "v"(v0), "v"(v1), "v"(v2), "v"(v3), "s"(gbase), "s"(lds_m0), "i"(I0), "i"(I1), "i"(I2),
        "i"(I3)
      : "memory", "m0");
}

// Asynchronous copy of a [ROWS][D] bf16 tile (global rows j0.. of G, clamped to
// nrows-1) into an LDS tile, by direct global->LDS loads of 4 bytes per lane: each
// wave instruction fills one contiguous 256-byte piece (128 elements). The NW waves of
// the workgroup take every NW-th piece; `wu` is the wave index made wave-uniform
// (readfirstlane), so piece and row arithmetic stays scalar and the only per-lane
// term is the lane's byte offset. Completion is tracked by vmcnt: wait_vmem() and a
// barrier must follow before any wave reads the tile.
template <int D, int ROWS, int NW>
__device__ __forceinline__ void tile_load_async(const uint16_t* G, int j0, int nrows,
                                                uint16_t* lds, int wu, int lane) {
  constexpr int NSEG = ROWS * D / 128;
  static_assert(NSEG % NW == 0, "pieces must split evenly over the waves");
#pragma unroll
  for (int i = 0; i < NSEG / NW; ++i) {
    const int k = wu + NW * i;  // piece index (uniform)
    const uint16_t* src;
    uint16_t* dst;
    if constexpr (D == 64) {
      // piece k = rows 2k and 2k+1, contiguous in global memory and in LDS
      const int r = 2 * k + (lane >> 5);
      src = G + (size_t)min(j0 + r, nrows - 1) * D + 2 * (lane & 31);
      dst = lds + TileLayout<D>::row(2 * k);
    } else {
      constexpr int PPR = D / 128;  // pieces per row
      const int r = k / PPR, c0 = (k % PPR) * 128;
      src = G + (size_t)min(j0 + r, nrows - 1) * D + c0 + 2 * lane;
      dst = lds + TileLayout<D>::row(r) + c0;
    }
    lds_dma_dword(src, dst);
  }
}

// The same copy for a tile whose ROWS rows all exist (j0 + ROWS <= nrows), in fewer
// instructions. L describes the LDS layout in 256-byte pieces, which are contiguous in
// global memory and in LDS: L::pieces(rows) pieces hold `rows` rows, and
// L::piece_bytes(u) is the LDS byte offset of piece u. Piece i of wave wu lies
// 256*(wu + NW*i) bytes past the tile's first row in global memory, so one scalar base
// per 4 KiB serves every piece and the rest goes into the instruction's immediate
// offset (which the hardware also adds to the LDS address, so M0 is lowered by it);
// the LDS offset of piece i from the wave's first piece is the same for every wave
// (checked at compile time), a constant added to M0. About three scalar instructions
// per piece, no vector ones.
template <class L, int ROWS, int NW>
struct PieceCopy {
  static constexpr int NSEG = L::pieces(ROWS);
  static constexpr int NI = NSEG / NW;
  static_assert(NSEG % NW == 0, "pieces must split evenly over the waves");
  // byte offset in LDS of piece i of wave w, relative to the wave's first piece
  static constexpr int lds_off(int w, int i) {
    return L::piece_bytes(w + NW * i) - L::piece_bytes(w);
  }
  static constexpr bool wave_independent() {
    for (int i = 0; i < NI; ++i)
      for (int w = 1; w < NW; ++w)
        if (lds_off(w, i) != lds_off(0, i)) return false;
    return true;
  }
  static_assert(wave_independent(), "LDS offsets must not depend on the wave");

  template <int I>
  __device__ __forceinline__ static void piece(const char* g0, uint32_t lane_off, uint32_t m0) {
    constexpr int GOFF = 256 * NW * I;
    constexpr int IMM = GOFF % 4096;
    static_assert(lds_off(0, I) >= IMM, "M0 stays at or above the tile's first piece");
    lds_dma_row_imm<IMM>(g0 + (GOFF - IMM), lane_off, m0 + (uint32_t)(lds_off(0, I) - IMM));
  }
  template <int... I>
  __device__ __forceinline__ static void all(const char* g0, uint32_t lane_off, uint32_t m0,
                                             std::integer_sequence<int, I...>) {
    (piece<I>(g0, lane_off, m0), ...);
  }
  // row0: the tile's first row in global memory; lds: the tile; wu: wave index
  // (uniform); lane_off = 4*lane
  __device__ __forceinline__ static void run(const void* row0, void* lds, int wu,
                                             uint32_t lane_off) {
    const char* g0 = (const char*)row0 + 256 * wu;
    const uint32_t m0 = lds_addr(lds) + L::piece_bytes(wu);
    all(g0, lane_off, m0, std::make_integer_sequence<int, NI>());
  }
};

// A bf16 TileLayout<D> in 256-byte pieces: a row pair (d = 64), a row (d = 128) or
// half a row (d = 256).
template <int D>
struct BfRows {
  static constexpr int pieces(int rows) { return rows * D / 128; }
  static constexpr int piece_bytes(int u) {
    if constexpr (D == 64) return 2 * TileLayout<D>::row(2 * u);
    else if constexpr (D == 128) return 2 * TileLayout<D>::row(u);
    else return 2 * TileLayout<D>::row(u / 2) + 256 * (u % 2);
  }
};

// Whole bf16 tile: rows j0 .. j0+ROWS-1 of G, all present.
template <int D, int ROWS, int NW>
__device__ __forceinline__ void tile_load_full(const uint16_t* G, int j0, uint16_t* lds, int wu,
                                               uint32_t lane_off) {
  PieceCopy<BfRows<D>, ROWS, NW>::run(G + (size_t)j0 * D, lds, wu, lane_off);
}
// The same, with the wave's first LDS address passed through opaque_s() (see
// tile_load_m0): for kernels where the hoisted per-piece addresses spill.
template <int D, int ROWS, int NW>
__device__ __forceinline__ void tile_load_full_o(const uint16_t* G, int j0, uint16_t* lds, int wu,
                                                 uint32_t lane_off) {
  using PC = PieceCopy<BfRows<D>, ROWS, NW>;
  const uint32_t m0w = opaque_s(lds_addr(lds) + (uint32_t)BfRows<D>::piece_bytes(wu));
  PC::all((const char*)(G + (size_t)j0 * D) + 256 * wu, lane_off, m0w,
          std::make_integer_sequence<int, PC::NI>());
}

// The same copy (d = 128 or 256) for kernels that keep many scalar values live: the LDS
// address of each piece is formed in the loop from one scalar base that passes through
// opaque_s(), so the compiler does not keep one scalar register per piece and buffer
// (which spills to vector lanes and costs a read per piece). lds_m0: LDS byte address
// of the tile. A tile that reaches past nrows re-reads row nrows-1 for the rows beyond,
// with one scalar base per piece.
template <int D, int ROWS, int NW>
__device__ __forceinline__ void tile_load_m0(const uint16_t* G, int j0, int nrows,
                                             uint32_t lds_m0, int wu, uint32_t lane_off) {
  static_assert(D == 128 || D == 256, "pieces of whole or half rows");
  using PC = PieceCopy<BfRows<D>, ROWS, NW>;
  constexpr int PPR = D / 128;  // pieces per row
  static_assert(NW % PPR == 0, "a wave's pieces share their column half");
  const uint32_t m0w = opaque_s(lds_m0 + (uint32_t)BfRows<D>::piece_bytes(wu));
  if (j0 + ROWS <= nrows) {
    PC::all((const char*)(G + (size_t)j0 * D) + 256 * wu, lane_off, m0w,
            std::make_integer_sequence<int, PC::NI>());
  } else {
#pragma unroll
    for (int i = 0; i < PC::NI; ++i) {
      const int r = min(j0 + wu / PPR + (NW / PPR) * i, nrows - 1);
      lds_dma_row_imm<0>(G + (size_t)r * D + 128 * (wu % PPR), lane_off,
                         m0w + (uint32_t)PC::lds_off(0, i));
    }
  }
}

// Scheduling hint for a run of N1 operand groups of R1 LDS reads followed by N2 groups
// of R2 reads, each group feeding QB consecutive products: the reads are issued LOOK
// ahead of the products that use them (sched_group_barrier groups, in program order).
template <int LOOK, int N1, int R1, int N2, int R2, int QB = 1>
struct ReadAheadG {
  static constexpr int NR = R1 * N1 + R2 * N2;
  // reads wanted once product i has been issued
  static constexpr int want(int i) {
    const int need =
        i < 0 ? 0 : (i < QB * N1 ? R1 * (i / QB + 1) : R1 * N1 + R2 * ((i - QB * N1) / QB + 1));
    return need + LOOK < NR ? need + LOOK : NR;
  }
  template <int I>
  __device__ __forceinline__ static void one() {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one matrix product
    if constexpr (want(I) > want(I - 1))
      __builtin_amdgcn_sched_group_barrier(0x100, want(I) - want(I - 1), 0);  // LDS reads
  }
  template <int... I>
  __device__ __forceinline__ static void all(std::integer_sequence<int, I...>) {
    (one<I>(), ...);
  }
  __device__ __forceinline__ static void emit() {
    __builtin_amdgcn_sched_group_barrier(0x100, want(-1), 0);
    all(std::make_integer_sequence<int, QB * (N1 + N2)>());
  }
};
// NS products that read one LDS operand each, then NP that read two
template <int LOOK, int NS, int NP>
using ReadAhead = ReadAheadG<LOOK, NS, 1, NP, 2, 1>;

// Wait until this wave's vector memory operations (including direct LDS loads) are done.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Debug build (FA_DEBUG_BARRIERS=1, built as libfa_sync.so): every kernel step also
// completes its copies and passes a workgroup barrier at the points that call this.
// Barriers change only timing, so its results must equal the normal build's bit for
// bit; a difference means some LDS access is not ordered by the kernel's own waits
// and barriers (a race). Every wave of a workgroup calls it the same number of times.
#ifndef FA_DEBUG_BARRIERS
#define FA_DEBUG_BARRIERS 0
#endif
__device__ __forceinline__ void debug_sync() {
  if constexpr (FA_DEBUG_BARRIERS != 0) {
    wait_vmem();
    __syncthreads();
  }
}

// Workgroup ids are dealt round-robin to the 8 XCDs (each with its own L2). Map the
// hardware id to a logical id so that consecutive logical ids run on one XCD.
__host__ __device__ __forceinline__ int xcd_remap(int hw, int n) {
  const int x = hw & 7, slot = hw >> 3;
  const int per = n >> 3, rem = n & 7;
  return x * per + (x < rem ? x : rem) + slot;
}

// (batch*head, row block) of workgroup `hw` of a causal launch of n = nbh * nqb
// workgroups, longest row blocks (the last ones, which see the most keys) first.
// Workgroup hw runs on XCD hw % 8 as the (hw / 8)-th of that XCD.
//  * nbh a multiple of 8: each XCD owns nbh / 8 whole (batch, head) pairs (their K/V
//    stay in its L2) and takes their row blocks C heads at a time, alternating
//    between them from the longest down. With C = 1 the long blocks of an XCD's last
//    head start when most compute units are already finishing short ones (about 9 %
//    of tail at 16 row blocks per head); C = 2 hands them out in the first half. A
//    kernel whose concurrent workgroups share tiles of one head in L2 (dK/dV) keeps
//    C = 1.
//  * otherwise a head's blocks cannot stay on one XCD without giving some XCDs only
//    long blocks and others only short ones: ids run over every head at one
//    row-block level, longest level first, so each XCD gets the same mix.
template <int C>
__host__ __device__ __forceinline__ void causal_order(int hw, int n, int nqb, int& bh,
                                                      int& qb) {
  static_assert(C == 1 || C == 2, "one or two heads at a time");
  const int nbh = n / nqb;
  if ((nbh & 7) == 0) {
    const int k = nbh >> 3, x = hw & 7, slot = hw >> 3;
    const int pair = slot / (C * nqb);
    const int nh = C < k - C * pair ? C : k - C * pair;
    const int r = slot - pair * C * nqb;
    bh = x * k + C * pair + (nh == 2 ? (r & 1) : 0);
    qb = nqb - 1 - (nh == 2 ? (r >> 1) : r);
  } else {
    bh = hw % nbh;
    qb = nqb - 1 - hw / nbh;
  }
}

}  // namespace fa
