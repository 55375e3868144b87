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

  const int c = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (c >= p.H) return;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (!first) acc = *(const f32x4 *)(p.yacc + (int64_t)r * p.H + c);
  int prev = -1;
  for (;;) {  // ascending positions of this row inside the pass
    int nxt = 0x7fffffff;
    for (int j = 0; j < p.topk; ++j) {
      const int q = spos[j];
      if (q > prev && q >= p.pass_base && q < end) nxt = min(nxt, q);
    }
    if (nxt == 0x7fffffff) break;
    const f32x4 d = *(const f32x4 *)(p.d + (int64_t)(nxt - p.pass_base) * p.H + c);
    acc += d;
    prev = nxt;
  }
  if (!last) {
    *(f32x4 *)(p.yacc + (int64_t)r * p.H + c) = acc;
  } else if (p.out_f32) {
    *(f32x4 *)((float *)p.out + (int64_t)r * p.H + c) = acc;
  } else {
    uint16_t *o = (uint16_t *)p.out + (int64_t)r * p.H + c;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = f32_to_f16_bits(acc[k]);
  }
}

hipError_t launch_combine(const CombineParams &p, int npos, hipStream_t s) {
  if (npos <= 0) return hipSuccess;
  const dim3 grid(npos, (p.H + 1023) / 1024);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace exl3
