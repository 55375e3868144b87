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

// A 64-bit value from lane (l ^ D) of the same group of four lanes (D = 1
// or 2), by two DPP quad permutes: no LDS traffic, unlike a bpermute.
template <int D>
__device__ __forceinline__ double quad_xor(double v) {
  static_assert(D == 1 || D == 2, "quad lanes");
  constexpr int ctrl = (D == 1) ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] / [2,3,0,1]
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)u, ctrl, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), ctrl, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// One (item, 128-block) unit whose source row and expert are known, done by
// the 4 lanes of a lane quad. Lane i (0..3 of the quad) loads entries
// 32i .. 32i + 31 (64 bytes) of the x block once and, for every projection,
// multiplies by suh (exact: the signs are +-1), runs the five butterfly
// levels of distances 1..16 in its registers and the two of distances 32
// and 64 across the quad (DPP), all in fp64 (exact for fp16 inputs: any sum
// of 128 of them spans at most 47 significant bits), scales by 1/sqrt(128)
// and rounds once to fp16. Each 16-entry group is stored in the kSigma
// order (slot p holds entry kSigma[p]). Every lane of the quad must call this
// with the same unit.
template <bool BF16>
__device__ __forceinline__ void rotate_block_t(const RotParams &p, int item, int blk, int row,
                                               int e, int i) {
  const int64_t col = blk * 128 + 32 * i;
  const u32x4 *xp = (const u32x4 *)(p.x + (int64_t)row * p.H + col);
  const bool upper1 = (i & 1) != 0, upper2 = (i & 2) != 0;
#pragma unroll 1
  for (int pj = 0; pj < p.nproj; ++pj) {
    // x is loaded again for the second projection (from the cache): not
    // keeping it live across the butterflies leaves room for 4 waves/SIMD
    const u32x4 *sp = (const u32x4 *)(p.suh[pj] + (int64_t)e * p.H + col);
    u32x4 xv[4], sv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      xv[c] = xp[c];
      sv[c] = sp[c];
    }
    // x stays packed: each product widens its two fp16 (or bf16) operands
    // itself, which keeps 32 widened copies of x out of the registers
    double v[32];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t xw = xv[j >> 2][j & 3], sw = sv[j >> 2][j & 3];
      if constexpr (BF16) {
        v[2 * j] = (double)mul_f32_by_f16<false>(__builtin_bit_cast(float, xw << 16), sw,
                                                  kNegZeroBits);
        v[2 * j + 1] = (double)mul_f32_by_f16<true>(
            __builtin_bit_cast(float, xw & 0xFFFF0000u), sw, kNegZeroBits);
      } else {
        v[2 * j] = (double)mul_f16_by_f16<false>(xw, sw, kNegZeroBits);
        v[2 * j + 1] = (double)mul_f16_by_f16<true>(xw, sw, kNegZeroBits);
      }
    }
#pragma unroll
    for (int d = 1; d < 32; d <<= 1) {
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        if ((j & d) == 0) {
          const double lo = v[j], hi = v[j + d];
          v[j] = lo + hi;
          v[j + d] = lo - hi;
        }
      }
    }
    // across the quad: the lower lane of a pair keeps v + o, the upper o - v
    const double s1 = upper1 ? -1.0 : 1.0, s2 = upper2 ? -1.0 : 1.0;
#pragma unroll
    for (int j = 0; j < 32; ++j) v[j] = fma(v[j], s1, quad_xor<1>(v[j]));
#pragma unroll
    for (int j = 0; j < 32; ++j) v[j] = fma(v[j], s2, quad_xor<2>(v[j]));
    u32x4 *op = (u32x4 *)(p.xt + ((int64_t)item * p.nproj + pj) * p.H + col);
#pragma unroll
    for (int g = 0; g < 4; ++g) {  // 8 entries: slots {0,4,1,5,2,6,3,7}
      const double *q = v + 8 * g;
      op[g] = (u32x4){f64x2_to_f16x2_bits(q[0] * kRsqrt128d, q[4] * kRsqrt128d),
                      f64x2_to_f16x2_bits(q[1] * kRsqrt128d, q[5] * kRsqrt128d),
                      f64x2_to_f16x2_bits(q[2] * kRsqrt128d, q[6] * kRsqrt128d),
                      f64x2_to_f16x2_bits(q[3] * kRsqrt128d, q[7] * kRsqrt128d)};
    }
  }
}

__device__ __forceinline__ void rotate_block(const RotParams &p, int item, int blk, int row, int e,
                                             int i) {
  if (p.x_bf16) rotate_block_t<true>(p, item, blk, row, e, i);
  else rotate_block_t<false>(p, item, blk, row, e, i);
}

// The same unit by 16 lanes of 8 entries each (lane i: entries 8i .. 8i+7):
// three butterfly levels in registers and four across the 16 lanes. Less
// work per lane than the quad form, for the latency-bound decode-size launch
// (pack_rotate_small_kernel). Same arithmetic (exact fp64 sums, one
// rounding), so the same bits.
template <bool BF16>
__device__ __forceinline__ void rotate_block16_t(const RotParams &p, int item, int blk, int row,
                                                 int e, int i) {
  const int64_t col = blk * 128 + 8 * i;
  const u32x4 xv = *(const u32x4 *)(p.x + (int64_t)row * p.H + col);
#pragma unroll 1
  for (int pj = 0; pj < p.nproj; ++pj) {
    const u32x4 sv = *(const u32x4 *)(p.suh[pj] + (int64_t)e * p.H + col);
    double v[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t xw = xv[j], sw = sv[j];
      const float x0 = BF16 ? bf16_bits_to_f32((uint16_t)(xw & 0xFFFFu))
                            : f16_bits_to_f32((uint16_t)(xw & 0xFFFFu));
      const float x1 = BF16 ? bf16_bits_to_f32((uint16_t)(xw >> 16))
                            : f16_bits_to_f32((uint16_t)(xw >> 16));
      v[2 * j] = (double)mul_f32_by_f16<false>(x0, sw, kNegZeroBits);
      v[2 * j + 1] = (double)mul_f32_by_f16<true>(x1, sw, kNegZeroBits);
    }
#pragma unroll
    for (int d = 1; d < 8; d <<= 1) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if ((j & d) == 0) {
          const double lo = v[j], hi = v[j + d];
          v[j] = lo + hi;
          v[j + d] = lo - hi;
        }
      }
    }
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      const double s = (i & d) ? -1.0 : 1.0;
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = fma(v[j], s, __shfl_xor(v[j], d, 64));
    }
    *(u32x4 *)(p.xt + ((int64_t)item * p.nproj + pj) * p.H + col) =
        (u32x4){f64x2_to_f16x2_bits(v[0] * kRsqrt128d, v[4] * kRsqrt128d),
                f64x2_to_f16x2_bits(v[1] * kRsqrt128d, v[5] * kRsqrt128d),
                f64x2_to_f16x2_bits(v[2] * kRsqrt128d, v[6] * kRsqrt128d),
                f64x2_to_f16x2_bits(v[3] * kRsqrt128d, v[7] * kRsqrt128d)};
  }
}

__device__ __forceinline__ void rotate_block16(const RotParams &p, int item, int blk, int row,
                                               int e, int i) {
  if (p.x_bf16) rotate_block16_t<true>(p, item, blk, row, e, i);
  else rotate_block16_t<false>(p, item, blk, row, e, i);
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
    if (pos >= min(*p.total_valid, p.pairs)) return;  // uniform per quad
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
