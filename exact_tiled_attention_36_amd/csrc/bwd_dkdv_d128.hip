// dK/dV kernel, head size 128, in a translation unit of its own.
//
// The compiler puts the results of every matrix product of a kernel that uses the
// accumulation registers (here dK and dV, 128 of them per lane) in accumulation
// registers too, so each S and dP element the softmax reads first costs a
// v_accvgpr_read: 64 of the 235 vector instructions of a step. build.py compiles this
// file alone with -mllvm --amdgpu-mfma-vgpr-form: products write ordinary vector
// registers and the compiler keeps values that do not fit in the accumulation
// registers, without scratch (324 registers per lane). The step then issues 171 vector
// instructions; measured 1.3-1.7 % less time for dK/dV on MI355X. Only this
// instantiation gets the option (the file with every head size did not compile with it).
#include "bwd_dkdv.h"

namespace fa {

hipError_t launch_bwd_dkdv_d128(const BwdParams& p, int nkb, int grid, bool causal, bool split,
                                hipStream_t st) {
  if (split) {
    if (causal)
      hipLaunchKernelGGL((bwd_dkdv_kernel<128, 64, true, true>), dim3(grid), dim3(256), 0, st, p, nkb);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<128, 64, false, true>), dim3(grid), dim3(256), 0, st, p, nkb);
  } else if (causal) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<128, 64, true>), dim3(grid), dim3(256), 0, st, p, nkb);
  } else {
    hipLaunchKernelGGL((bwd_dkdv_kernel<128, 64, false>), dim3(grid), dim3(256), 0, st, p, nkb);
  }
  return hipGetLastError();
}

}  // namespace fa
