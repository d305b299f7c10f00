// dQ kernels for d = 64 and 128 (128 query rows per workgroup: 4 waves, two workgroups
// per compute unit, or on small grids 8 waves in two groups that take half of the key
// tiles each) in a translation unit of their own. build.py compiles this file with
// -mllvm --amdgpu-mfma-vgpr-form: the matrix products write ordinary vector registers,
// so the softmax reads S and dP without a v_accvgpr_read per element (a step of these
// kernels issues 193 vector instructions instead of 257). The option is kept off the
// d = 256 dQ build, which it makes spill.
#include "bwd_dq.h"

namespace fa {

hipError_t launch_bwd_dq_small(const BwdParams& p, int nqb, int grid, int d, bool causal,
                               bool key_split, hipStream_t st) {
  if (key_split) {
    if (d == 64) {
      if (causal)
        hipLaunchKernelGGL((bwd_dq_kernel<64, 32, 8, true, 2>), dim3(grid), dim3(512), 0, st, p, nqb);
      else
        hipLaunchKernelGGL((bwd_dq_kernel<64, 32, 8, false, 2>), dim3(grid), dim3(512), 0, st, p, nqb);
    } else if (d == 128) {
      if (causal)
        hipLaunchKernelGGL((bwd_dq_kernel<128, 32, 8, true, 2>), dim3(grid), dim3(512), 0, st, p, nqb);
      else
        hipLaunchKernelGGL((bwd_dq_kernel<128, 32, 8, false, 2>), dim3(grid), dim3(512), 0, st, p, nqb);
    } else {
      return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (d == 64) {
    if (causal)
      hipLaunchKernelGGL((bwd_dq_kernel<64, 32, 4, true>), dim3(grid), dim3(256), 0, st, p, nqb);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<64, 32, 4, false>), dim3(grid), dim3(256), 0, st, p, nqb);
  } else if (d == 128) {
    if (causal)
      hipLaunchKernelGGL((bwd_dq_kernel<128, 32, 4, true>), dim3(grid), dim3(256), 0, st, p, nqb);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<128, 32, 4, false>), dim3(grid), dim3(256), 0, st, p, nqb);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fa
