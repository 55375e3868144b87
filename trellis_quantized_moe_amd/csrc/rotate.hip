// Input rotation x~ = fp16_rne(H128(x * suh) / sqrt(128)) for the GEMM A
// operands, stored in the kSigma k-order the decoded B operands use.
// exllamav3 PR #284 "MoE: Add fused additive EXL3 kernels" (API contract:
// each projection's suh/svh rotations, reused by residual stages) and
// TensorFold PR #837 (What this changes: the input rotation, each expert's
// rotation for gate and up).
#include "common.hpp"
#include "kernels.hpp"

namespace exl3 {

// One 16-lane group per (item, 128-block), 16 groups per block; the group
// loads the x block once and writes it rotated for every projection. Lane i
// loads entries 8i..8i+7 (16 bytes), transforms, and stores them as one
// 16-byte run in the kSigma order: slots 0..7 of its half-group hold entries
// {0,4,1,5,2,6,3,7} of the lane's 8.
__global__ void __launch_bounds__(256) rotate_kernel(RotParams p) {
  const int nblk = p.H >> 7;
  const int64_t gid = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int i = threadIdx.x & 15;
  if (p.ctrl_clear && blockIdx.x == 0 && threadIdx.x == 0) {
    p.ctrl_clear[1] = 0;  // bad stage entries
  }
  if (p.zero) {  // narrow-tile completion counts of the GEMM that follows
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < p.nzero;
         i += (int64_t)gridDim.x * blockDim.x)
      p.zero[i] = 0;
  }
  if (gid >= (int64_t)p.nitems * nblk) return;
  const int item = (int)(gid / nblk);
  const int blk = (int)(gid - (int64_t)item * nblk);

  int row, e;
  if (p.pair_of_pos != nullptr) {
    const int pos = p.pass_base + item;
    if (pos >= min(*p.total_valid, p.pairs)) return;  // uniform per group
    const int q = p.pair_of_pos[pos];
    if (q < 0 || q >= p.pairs) return;  // inconsistent metadata: drop
    row = q / p.topk;
    e = p.expert_of_pos[pos];
  } else {
    row = item;
    e = 0;
  }
  const int64_t col = blk * 128 + 8 * i;
  const u32x4 xv = *(const u32x4 *)(p.x + (int64_t)row * p.H + col);
  u32x4 sv[2];
#pragma unroll
  for (int pj = 0; pj < 2; ++pj)
    if (pj < p.nproj) sv[pj] = *(const u32x4 *)(p.suh[pj] + (int64_t)e * p.H + col);
#pragma unroll
  for (int pj = 0; pj < 2; ++pj) {
    if (pj >= p.nproj) break;
    // halves are unpacked with shifts: this compiler mis-compiles a bit_cast
    // of a vector element taken inside an unrolled loop (it reuses element 0)
    float v[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t xw = xv[j], sw = sv[pj][j];
      v[2 * j] = f16_bits_to_f32((uint16_t)(xw & 0xFFFFu)) * f16_bits_to_f32((uint16_t)(sw & 0xFFFFu));
      v[2 * j + 1] = f16_bits_to_f32((uint16_t)(xw >> 16)) * f16_bits_to_f32((uint16_t)(sw >> 16));
    }
    fwht128_lane8(v);
    uint16_t h[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) h[j] = f32_to_f16_bits(v[j] * kRsqrt128);
    const u32x4 o = {(uint32_t)h[0] | ((uint32_t)h[4] << 16), (uint32_t)h[1] | ((uint32_t)h[5] << 16),
                     (uint32_t)h[2] | ((uint32_t)h[6] << 16), (uint32_t)h[3] | ((uint32_t)h[7] << 16)};
    *(u32x4 *)(p.xt + ((int64_t)item * p.nproj + pj) * p.H + col) = o;
  }
}

hipError_t launch_rotate(const RotParams &p, hipStream_t s) {
  const int64_t groups = (int64_t)p.nitems * (p.H >> 7);
  if (groups <= 0) return hipSuccess;
  if (p.nproj < 1 || p.nproj > 2) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rotate_kernel, dim3((unsigned)((groups + 15) / 16)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace exl3
