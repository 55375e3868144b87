// Input rotation of one (item, 128-block) by one 16-lane group (x in fp16 or
// bf16, read exactly; x~ rounded once to fp16 from an exact fp64 transform,
// so it is the correctly rounded rotated value), shared by the
// rotate kernel and the per-pass expert kernel (which rotates the next pass's
// inputs while its own down work finishes).
// x~ = fp16_rne(H128(x * suh) / sqrt(128)) for the GEMM A operands, stored in
// the kSigma k-order the decoded B operands use. exllamav3 PR #284 "MoE: Add
// fused additive EXL3 kernels" (API contract: each projection's suh/svh
// rotations, reused by residual stages) and TensorFold PR #837 (What this
// changes: the input rotation, each expert's rotation for gate and up).
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace exl3 {

// One (item, 128-block) unit whose source row and expert are known. Lane i
// (0..15 of the group) loads entries 8i..8i+7 (16 bytes) of the x block
// once, transforms it for every projection, and stores each result as one
// 16-byte run in the kSigma order: slots 0..7 of its half-group hold entries
// {0,4,1,5,2,6,3,7} of the lane's 8. Every lane of the group must call this
// with the same unit.
__device__ __forceinline__ void rotate_block(const RotParams &p, int item, int blk, int row, int e,
                                             int i) {
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
    double v[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t xw = xv[j], sw = sv[pj][j];
      const float x0 = p.x_bf16 ? bf16_bits_to_f32((uint16_t)(xw & 0xFFFFu))
                                : f16_bits_to_f32((uint16_t)(xw & 0xFFFFu));
      const float x1 = p.x_bf16 ? bf16_bits_to_f32((uint16_t)(xw >> 16))
                                : f16_bits_to_f32((uint16_t)(xw >> 16));
      v[2 * j] = (double)(x0 * f16_bits_to_f32((uint16_t)(sw & 0xFFFFu)));
      v[2 * j + 1] = (double)(x1 * f16_bits_to_f32((uint16_t)(sw >> 16)));
    }
    // exact butterflies and one rounding: x~ is the fp16 value nearest to
    // Hhat(x * suh) itself
    fwht128_lane8(v);
    uint16_t h[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) h[j] = f64_to_f16_bits(v[j] * kRsqrt128d);
    const u32x4 o = {(uint32_t)h[0] | ((uint32_t)h[4] << 16), (uint32_t)h[1] | ((uint32_t)h[5] << 16),
                     (uint32_t)h[2] | ((uint32_t)h[6] << 16), (uint32_t)h[3] | ((uint32_t)h[7] << 16)};
    *(u32x4 *)(p.xt + ((int64_t)item * p.nproj + pj) * p.H + col) = o;
  }
}

// Unit gid = item * (H / 128) + block: the row and expert of the item come
// from the pack (MoE) or are the item itself (linear).
__device__ __forceinline__ void rotate_unit(const RotParams &p, int64_t gid, int i) {
  const int nblk = p.H >> 7;
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
  rotate_block(p, item, blk, row, e, i);
}

}  // namespace exl3
