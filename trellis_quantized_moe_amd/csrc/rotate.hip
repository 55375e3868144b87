// Input rotation kernel (the per-unit work is rotate_unit).
#include "rotate_dev.hpp"

namespace exl3 {

// One lane quad per (item, 128-block), 64 quads per block.
__global__ void __launch_bounds__(256) rotate_kernel(RotParams p) {
  if (p.ctrl_clear && blockIdx.x == 0 && threadIdx.x == 0) {
    p.ctrl_clear[0] = 0;  // dropped pairs (none in a linear call)
    p.ctrl_clear[1] = 0;  // bad stage entries
    p.ctrl_clear[2] = 0;  // waits that gave up
  }
  if (p.zero) {  // completion counts of the GEMMs that follow
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < p.nzero;
         i += (int64_t)gridDim.x * blockDim.x)
      p.zero[i] = 0;
  }
  rotate_unit(p, (int64_t)blockIdx.x * 64 + (threadIdx.x >> 2), threadIdx.x & 3);
}

hipError_t launch_rotate(const RotParams &p, hipStream_t s) {
  const int64_t groups = (int64_t)p.nitems * (p.H >> 7);
  if (groups <= 0) return hipSuccess;
  if (p.nproj < 1 || p.nproj > 2) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rotate_kernel, dim3((unsigned)((groups + 63) / 64)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace exl3
