// Ordered top-k combine of one packed position, shared by the combine kernel
// and the pipelined expert kernel (which combines an earlier pass while
// later passes compute).
// y_r = sum of the row's weighted per-pair outputs d, added in fp32 in
// ascending packed position (expert, then pair index), pass after pass.
// TensorFold PR #837 (What this changes: the weighted combine; an expert's
// how many rows an expert serves must not alter any row's result) — the
// fixed order makes the row's
// bytes independent of other rows, capacity and chunking.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace exl3 {

// One workgroup per packed position of the pass. Only the workgroup of the
// row's lowest position inside the pass (its "owner") does the work, so each
// row is written once per pass. In every wave, lane j < topk holds the
// position of the row's pair j; the wave ranks those inside the pass with
// ballots (no shared memory, no serial loop) and the 4 waves add the d rows
// in ascending position over interleaved 16-byte column chunks.
__device__ __forceinline__ void combine_position(const CombineParams &p, int item) {
  const int lane = threadIdx.x & 63;
  const int pos = p.pass_base + item;
  const int end = min(min(p.pass_end, *p.total_valid), p.pairs);
  if (pos >= end) return;  // uniform per workgroup
  const int q0 = p.pair_of_pos[pos];
  if (q0 < 0 || q0 >= p.pairs) return;  // inconsistent metadata: drop
  const int r = q0 / p.topk;
  const int q = (lane < p.topk) ? p.pos_of_pair[r * p.topk + lane] : -1;
  const bool in_pass = q >= p.pass_base && q < end;
  // the row's pairs before and after this pass decide whether yacc is read
  // (earlier passes contributed) and whether the result is final
  const bool first = __ballot(q >= 0 && q < p.pass_base) == 0;
  const bool last = __ballot(q >= end) == 0;
  const uint64_t inmask = __ballot(in_pass);
  // owner: the lowest in-pass position of the row
  int owner = in_pass ? q : 0x7fffffff;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) owner = min(owner, __shfl_xor(owner, d, 64));
  if (owner != pos) return;

  // positions in ascending order: lane j's rank among in-pass positions
  int rank = 0;
  for (uint64_t m = inmask; m; m &= m - 1) {
    const int l = __ffsll((long long)m) - 1;
    const int ql = __shfl(q, l, 64);
    rank += (in_pass && ql < q) ? 1 : 0;
  }
  const int cnt = __popcll(inmask);
  // order[k] = k-th smallest in-pass position (relative); a rank no lane
  // holds (positions repeated by inconsistent metadata) is skipped (-1)
  int order[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    if (k < cnt) {
      const uint64_t sel = __ballot(in_pass && rank == k);
      const int l = __ffsll((long long)sel) - 1;
      order[k] = sel ? __shfl(q, l, 64) - p.pass_base : -1;
    }
  }

  const int64_t rowoff = (int64_t)r * p.H;
  auto emit = [&](int c, f32x4 acc) {
    if (!last) {
      *(f32x4 *)(p.yacc + rowoff + c) = acc;
    } else if (p.out_f32) {
      *(f32x4 *)((float *)p.out + rowoff + c) = acc;
    } else {
      const uint32_t lo = (uint32_t)f32_to_out16(acc[0], p.out_bf16) |
                           ((uint32_t)f32_to_out16(acc[1], p.out_bf16) << 16);
      const uint32_t hi = (uint32_t)f32_to_out16(acc[2], p.out_bf16) |
                           ((uint32_t)f32_to_out16(acc[3], p.out_bf16) << 16);
      *(uint2 *)((uint16_t *)p.out + rowoff + c) = make_uint2(lo, hi);
    }
  };
  // H is a multiple of 128: columns [c, c + 4) and [c + 1024, c + 1028) per
  // lane and step (both in range whenever c + 1024 < H)
  for (int c = threadIdx.x * 4; c < p.H; c += 2048) {
    const int c2 = c + 1024;
    const bool two = c2 < p.H;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = acc;
    if (!first) {
      acc = *(const f32x4 *)(p.yacc + rowoff + c);
      if (two) acc2 = *(const f32x4 *)(p.yacc + rowoff + c2);
    }
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      if (k < cnt && order[k] >= 0) {
        const float *dk = p.d + (int64_t)order[k] * p.H;
        acc += *(const f32x4 *)(dk + c);
        if (two) acc2 += *(const f32x4 *)(dk + c2);
      }
    }
    emit(c, acc);
    if (two) emit(c2, acc2);
  }
}

}  // namespace exl3
