// Ordered top-k combine kernels (the per-row work of a pass range is
// combine_row).
#include "combine_dev.hpp"

namespace exl3 {

// One workgroup of 256 threads per row (rows with no pair in the pass range
// return at once).
__global__ void __launch_bounds__(256) combine_kernel(CombineParams p) {
  combine_row(p, blockIdx.x);
}

// Single pass (every kept position in it): one workgroup of 512 threads per
// row, so the row's positions are known after one load (pos_of_pair) instead
// of two, and the d loads of up to 8 positions are in flight together. Same
// fp32 additions in the same order as combine_kernel.
constexpr int kRowThreads = 512;

__global__ void __launch_bounds__(kRowThreads) combine_rows_kernel(CombineParams p) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x;
  const int end = min(*p.total_valid, p.pairs);
  const int q = (lane < p.topk) ? p.pos_of_pair[r * p.topk + lane] : -1;
  const bool valid = q >= 0 && q < end;
  const uint64_t vmask = __ballot(valid);
  if (vmask == 0) return;  // dropped row: the pack wrote its zeros
  int rank = 0;
  for (uint64_t m = vmask; m; m &= m - 1) {
    const int l = __ffsll((long long)m) - 1;
    const int ql = __shfl(q, l, 64);
    rank += (valid && ql < q) ? 1 : 0;
  }
  const int cnt = __popcll(vmask);
  // position of rank k; rank 0 always has a lane (the smallest position)
  const int pos0 = __shfl(q, __ffsll((long long)__ballot(valid && rank == 0)) - 1, 64);
  // a rank no lane holds (past cnt, or positions repeated by inconsistent
  // metadata): -1, loaded from pos0 and not added
  auto pos_of_rank = [&](int k) {
    const uint64_t sel = __ballot(valid && rank == k);
    return (k < cnt && sel) ? __shfl(q, __ffsll((long long)sel) - 1, 64) : -1;
  };
  const int64_t rowoff = (int64_t)r * p.H;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  const f32x4 nz = {-0.f, -0.f, -0.f, -0.f};  // x + (-0) == x exactly
  for (int c0 = threadIdx.x * 4; c0 < p.H; c0 += 2 * kRowThreads * 4) {
    const int c1 = c0 + kRowThreads * 4;
    const bool two = c1 < p.H;
    f32x4 a0 = zero, a1 = zero;
    for (int kb = 0; kb < cnt; kb += 8) {
      f32x4 v0[8], v1[8];
      bool ok[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int pk = pos_of_rank(kb + u);
        ok[u] = pk >= 0;
        const float *dk = p.d + (int64_t)(ok[u] ? pk : pos0) * p.H;
        v0[u] = *(const f32x4 *)(dk + c0);
        v1[u] = two ? *(const f32x4 *)(dk + c1) : zero;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        a0 += ok[u] ? v0[u] : nz;
        a1 += ok[u] ? v1[u] : nz;
      }
    }
    auto emit = [&](int c, f32x4 acc) {
      if (p.out_f32) {
        *(f32x4 *)((float *)p.out + rowoff + c) = acc;
      } else {
        const uint32_t lo = (uint32_t)f32_to_out16(acc[0], p.out_bf16) |
                           ((uint32_t)f32_to_out16(acc[1], p.out_bf16) << 16);
        const uint32_t hi = (uint32_t)f32_to_out16(acc[2], p.out_bf16) |
                           ((uint32_t)f32_to_out16(acc[3], p.out_bf16) << 16);
        *(uint2 *)((uint16_t *)p.out + rowoff + c) = make_uint2(lo, hi);
      }
    };
    emit(c0, a0);
    if (two) emit(c1, a1);
  }
}

hipError_t launch_combine(const CombineParams &p, int npos, hipStream_t s) {
  if (npos <= 0 || p.rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3(p.rows), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_combine_rows(const CombineParams &p, hipStream_t s) {
  if (p.rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(combine_rows_kernel, dim3(p.rows), dim3(kRowThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace exl3
