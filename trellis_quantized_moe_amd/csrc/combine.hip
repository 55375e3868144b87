// Ordered top-k combine: y_r = sum of the row's weighted per-pair outputs d,
// added in fp32 in ascending packed position (expert, then pair index), pass
// after pass. TensorFold PR #837 (What this changes: the weighted combine;
// an expert's member count never changes a row's bits) — the fixed order
// makes the row's bytes independent of other rows, capacity and chunking.
#include "common.hpp"
#include "kernels.hpp"

namespace exl3 {

// One block per packed position of the pass; only the row's lowest position
// in the pass does the work (the "owner"), so each row is written once.
__global__ void __launch_bounds__(256) combine_kernel(CombineParams p) {
  __shared__ int spos[32];
  const int pos = p.pass_base + blockIdx.x;
  const int end = min(min(p.pass_end, *p.total_valid), p.pairs);
  if (pos >= end) return;
  const int q0 = p.pair_of_pos[pos];
  if (q0 < 0 || q0 >= p.pairs) return;  // inconsistent metadata: drop
  const int r = q0 / p.topk;
  if (threadIdx.x < p.topk) spos[threadIdx.x] = p.pos_of_pair[r * p.topk + threadIdx.x];
  __syncthreads();

  int owner = 0x7fffffff;
  bool first = true, last = true;
  for (int j = 0; j < p.topk; ++j) {
    const int q = spos[j];
    if (q < 0) continue;
    if (q < p.pass_base) first = false;
    else if (q >= end) last = false;
    else owner = min(owner, q);
  }
  if (owner != pos) return;

  // this row's positions inside the pass, ascending (at most topk <= 32)
  __shared__ int order[32];
  __shared__ int s_cnt;
  if (threadIdx.x == 0) {
    int cnt = 0;
    for (int prev = -1;;) {
      int nxt = 0x7fffffff;
      for (int j = 0; j < p.topk; ++j) {
        const int q = spos[j];
        if (q > prev && q >= p.pass_base && q < end) nxt = min(nxt, q);
      }
      if (nxt == 0x7fffffff) break;
      order[cnt++] = nxt - p.pass_base;
      prev = nxt;
    }
    s_cnt = cnt;
  }
  __syncthreads();
  const int cnt = s_cnt;
  for (int c = threadIdx.x * 4; c < p.H; c += 256 * 4) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (!first) acc = *(const f32x4 *)(p.yacc + (int64_t)r * p.H + c);
    for (int k = 0; k < cnt; ++k) acc += *(const f32x4 *)(p.d + (int64_t)order[k] * p.H + c);
    if (!last) {
      *(f32x4 *)(p.yacc + (int64_t)r * p.H + c) = acc;
    } else if (p.out_f32) {
      *(f32x4 *)((float *)p.out + (int64_t)r * p.H + c) = acc;
    } else {
      const uint32_t lo = (uint32_t)f32_to_f16_bits(acc[0]) | ((uint32_t)f32_to_f16_bits(acc[1]) << 16);
      const uint32_t hi = (uint32_t)f32_to_f16_bits(acc[2]) | ((uint32_t)f32_to_f16_bits(acc[3]) << 16);
      *(uint2 *)((uint16_t *)p.out + (int64_t)r * p.H + c) = make_uint2(lo, hi);
    }
  }
}

hipError_t launch_combine(const CombineParams &p, int npos, hipStream_t s) {
  if (npos <= 0) return hipSuccess;
  const dim3 grid(npos);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace exl3
