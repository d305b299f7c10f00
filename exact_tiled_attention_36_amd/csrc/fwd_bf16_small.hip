// Forward attention, bf16, 128-row workgroups, d = 64 or 128, in a translation unit of
// its own: for grids too small to give every compute unit a 256-row workgroup (short
// sequences, few heads) as 8 waves whose two halves take half of the key tiles each,
// and for short key ranges as 4 waves (two of these workgroups share a compute unit;
// see fwd_bf16.hip).
//
// These kernels keep O in the accumulation registers, so the compiler also puts every
// score product there and copies each element out before the softmax
// (v_accvgpr_read). build.py compiles this file alone with
// -mllvm --amdgpu-mfma-vgpr-form: products write ordinary vector registers and the
// kernels need fewer registers (d = 128: 252 instead of 336, d = 64: about 163 instead
// of 208), without scratch. Measured on MI355X: B1 H8 N2048 d128 causal 8 % faster,
// B2 H16 N1024 d64 1.5 %. The option is not used for the other forward kernels (the
// 8-wave ones compile identically with it, the d = 256 one ran 1.5 % slower).
#include "fwd_bf16.h"

namespace fa {

hipError_t launch_fwd_bf16_small(FwdParams p, long long B, int d, bool causal, bool key_split,
                                 hipStream_t st) {
  if (key_split) {
    if (d == 64)
      return causal ? run<64, 64, 8, 1, true, false, false, 2>(p, B, st)
                    : run<64, 64, 8, 1, false, false, false, 2>(p, B, st);
    if (d == 128)
      return causal ? run<128, 64, 8, 1, true, false, false, 2>(p, B, st)
                    : run<128, 64, 8, 1, false, false, false, 2>(p, B, st);
    return hipErrorInvalidValue;
  }
  if (d == 64) return causal ? run<64, 64, 4, 1, true>(p, B, st) : run<64, 64, 4, 1, false>(p, B, st);
  if (d == 128) return causal ? run<128, 64, 4, 1, true>(p, B, st) : run<128, 64, 4, 1, false>(p, B, st);
  return hipErrorInvalidValue;
}

}  // namespace fa
