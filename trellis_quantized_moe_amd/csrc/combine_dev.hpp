// Ordered top-k combine of one row over one pass range, shared by the
// combine kernel and the pipelined expert kernel (which combines an earlier
// pass while later passes compute).
// y_r = sum of the row's weighted per-pair outputs d, added in fp32 in
// ascending packed position (expert, then pair index), pass after pass.
// TensorFold PR #837 (What this changes: the weighted combine; how many rows
// an expert serves must not alter any row's result) — the fixed order makes
// the row's bytes independent of other rows, capacity and chunking.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace exl3 {

// One workgroup per row. Lane j < topk of every wave holds the position of
// the row's pair j; the wave ranks the positions inside the pass range with
// ballots (no shared memory, no serial loop). A row with no position in the
// range has nothing to do. Otherwise the workgroup's threads add, for
// interleaved 16-byte column chunks, the running sum of earlier passes
// (yacc, unless no earlier pass holds a pair of the row) and then the d rows
// in ascending position; the result goes to yacc, or to the output when no
// later pass holds a pair of the row. The loads of up to kRanks positions
// for kChunks column chunks per thread are in flight together, so a row
// costs about one memory latency at the hidden sizes of the layer.
__device__ __forceinline__ void combine_row(const CombineParams &p, int r) {
  constexpr int kChunks = 6;  // 16-byte column chunks per thread and step
  constexpr int kRanks = 4;   // positions whose loads are in flight together
  const int lane = threadIdx.x & 63;
  if (r >= p.rows) return;
  const int end = min(min(p.pass_end, *p.total_valid), p.pairs);
  const int q = (lane < p.topk) ? p.pos_of_pair[r * p.topk + lane] : -1;
  const bool in_pass = q >= p.pass_base && q < end;
  const uint64_t inmask = __ballot(in_pass);
  if (inmask == 0) return;  // uniform per workgroup
  // the row's pairs before and after this range decide whether yacc is read
  // (earlier passes contributed) and whether the result is final
  const bool first = __ballot(q >= 0 && q < p.pass_base) == 0;
  const bool last = __ballot(q >= end) == 0;
  int rank = 0;
  for (uint64_t m = inmask; m; m &= m - 1) {
    const int l = __ffsll((long long)m) - 1;
    const int ql = __shfl(q, l, 64);
    rank += (in_pass && ql < q) ? 1 : 0;
  }
  const int cnt = __popcll(inmask);
  // position (relative to the range) of rank k; rank 0 always has a lane.
  // A rank no lane holds (past cnt, or positions repeated by inconsistent
  // metadata): -1, loaded from rank 0's row and not added
  const int pos0 = __shfl(q, __ffsll((long long)__ballot(in_pass && rank == 0)) - 1, 64) -
                   p.pass_base;
  auto pos_of_rank = [&](int k) {
    const uint64_t sel = __ballot(in_pass && rank == k);
    return (k < cnt && sel) ? __shfl(q, __ffsll((long long)sel) - 1, 64) - p.pass_base : -1;
  };

  const int64_t rowoff = (int64_t)r * p.H;
  const int span = 4 * (int)blockDim.x;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  const f32x4 nz = {-0.f, -0.f, -0.f, -0.f};  // x + (-0) == x exactly
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
  // H is a multiple of 128: chunk j of a step covers columns
  // [c0 + j span, c0 + j span + 4) when that is below H
  for (int c0 = threadIdx.x * 4; c0 < p.H; c0 += kChunks * span) {
    f32x4 acc[kChunks];
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
      const int c = c0 + j * span;
      acc[j] = (!first && c < p.H) ? *(const f32x4 *)(p.yacc + rowoff + c) : zero;
    }
    for (int kb = 0; kb < cnt; kb += kRanks) {
      f32x4 v[kRanks][kChunks];
      bool ok[kRanks];
#pragma unroll
      for (int u = 0; u < kRanks; ++u) {
        const int pk = pos_of_rank(kb + u);
        ok[u] = pk >= 0;
        const float *dk = p.d + (int64_t)(ok[u] ? pk : pos0) * p.H;
#pragma unroll
        for (int j = 0; j < kChunks; ++j) {
          const int c = c0 + j * span;
          v[u][j] = c < p.H ? *(const f32x4 *)(dk + c) : zero;
        }
      }
#pragma unroll
      for (int u = 0; u < kRanks; ++u)
#pragma unroll
        for (int j = 0; j < kChunks; ++j) acc[j] += ok[u] ? v[u][j] : nz;
    }
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
      const int c = c0 + j * span;
      if (c < p.H) emit(c, acc[j]);
    }
  }
}

}  // namespace exl3
