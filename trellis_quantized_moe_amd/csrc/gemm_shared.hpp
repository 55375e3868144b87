// Device code shared by the narrow and wide grouped-GEMM kernels: the
// buffer-resource helper, work-tile lookup and the epilogue. Both kernels use
// this one epilogue so a row's output bytes never depend on the tile shape it
// was computed with (TensorFold PR #837 "cuda: EXL3 linear and grouped routed
// experts, every codebook and width, a width per expert", What this changes:
// row-invariant linear; the number of rows routed to an expert does not alter
// any row's result).
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace exl3 {

// Raw buffer resource (gfx9 dword 3 = 0x00020000): SGPR base, 32-bit
// per-lane offsets, out-of-range reads return 0.
// The base and size are wave-uniform; readfirstlane keeps the descriptor in
// SGPRs even when the compiler computed them with vector instructions.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  void *ub = (void *)(uintptr_t)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0,
                                           __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// ---------------------------------------------------------------- epilogue
// Shared by every tile shape, so a row's bytes never depend on the tile it
// was computed in. T is an LDS tile of fp32 pre-rotation accumulators:
// T[pj * proj_stride + row * ld + c], c = 0 .. 128*nblk-1 (columns relative
// to colbase). One 16-lane group handles one (row, 128-block) at a time.
// COH: a~ (gate/up) and d (down) are written with device-coherent stores, for
// a reader in the same launch.
// The per-column vectors of one 128-column block, staged in LDS by a caller
// that loaded them ahead of time (16-row kernels): svh and chscale of gate
// and up (or of the one projection), the down input signs (gate/up), and the
// route weights of the tile's rows (down). Columns relative to colbase.
// Layout at v (fp16): svh of projection q at v[256 q + c], its chscale at
// v[256 q + 128 + c], the down input signs at v[512 + c].
struct EpiVec {
  const uint16_t *v;
  const float *wt;
};

template <int EPI, bool COH = false, bool LDSV = false>
__device__ __forceinline__ void epilogue(const GemmParams &p, float *T, int ld, int proj_stride,
                                         int e, int row0, int nrows, int colbase, int nblk,
                                         const EpiVec &ev = EpiVec{}) {
  const int ngroups = blockDim.x >> 4;
  const int grp = threadIdx.x >> 4;
  const int i = threadIdx.x & 15;
  // svh / chscale of projection q at column c (relative to colbase)
  auto svh_at = [&](int q, int c) -> float {
    if constexpr (LDSV) return f16_bits_to_f32(ev.v[256 * q + c]);
    else return f16_bits_to_f32(p.proj[q].svh[(size_t)e * p.out_f + colbase + c]);
  };
  auto cs_at = [&](int q, int c) -> float {
    if constexpr (LDSV) return f16_bits_to_f32(ev.v[256 * q + 128 + c]);
    else return f16_bits_to_f32(p.proj[q].cs[(size_t)e * p.out_f + colbase + c]);
  };
  if constexpr (EPI == EPI_GATEUP) {
    // y = H(acc)/sqrt(128) * svh * cs for gate (pj 0) and up (pj 1)
    for (int it = grp; it < 2 * nrows; it += ngroups) {
      const int q = it / nrows, row = it - q * nrows;
      float *t = T + q * proj_stride + row * ld;
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = t[i + 16 * j];
      fwht128_group16(v);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = i + 16 * j;
        t[c] = ((v[j] * kRsqrt128) * svh_at(q, c)) * cs_at(q, c);
      }
    }
    __syncthreads();
    // a = silu(g) * u; a~ = fp16(H(a * suh_down)/sqrt(128)) in kSigma order
    for (int row = grp; row < nrows; row += ngroups) {
      const size_t sb = (size_t)e * p.out_f + colbase;
      const float *tg = T + row * ld, *tu = T + proj_stride + row * ld;
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = i + 16 * j;
        const float sd = LDSV ? f16_bits_to_f32(ev.v[512 + c]) : f16_bits_to_f32(p.suh_down[sb + c]);
        v[j] = (silu(tg[c]) * tu[c]) * sd;
      }
      fwht128_group16(v);
      uint16_t *o = p.out_h + (int64_t)(row0 + row) * p.ldo + colbase;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint16_t h = f32_to_f16_bits(v[j] * kRsqrt128);
        if constexpr (COH)
          __hip_atomic_store(o + 16 * j + sigma_inv(i), h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
          o[16 * j + sigma_inv(i)] = h;
      }
    }
  } else {
    for (int it = grp; it < nrows * nblk; it += ngroups) {
      const int row = it / nblk, blk = it - row * nblk;
      const float *t = T + row * ld + blk * 128;
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = t[i + 16 * j];
      fwht128_group16(v);
      const int cb = colbase + blk * 128;
      float wt = 1.0f;
      if constexpr (EPI == EPI_DOWN)
        wt = LDSV ? ev.wt[row] : p.weight_of_pos[p.pass_base + row0 + row];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = i + 16 * j;
        const float y = ((v[j] * kRsqrt128) * svh_at(0, blk * 128 + c)) * cs_at(0, blk * 128 + c);
        const int64_t o = (int64_t)(row0 + row) * p.ldo + cb + c;
        if constexpr (EPI == EPI_DOWN) {
          if constexpr (COH)
            __hip_atomic_store(p.out_f32 + o, y * wt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          else
            p.out_f32[o] = y * wt;
        } else {
          if (p.out_f32) p.out_f32[o] = y;
          else p.out_h[o] = f32_to_out16(y, p.out_bf16);
        }
      }
    }
  }
}

__device__ __forceinline__ bool tile_of_block(const GemmParams &p, int bm, int bx, int &e,
                                              int &row0, int &nrows) {
  if (p.plan_tiles == nullptr) {
    e = 0;
    row0 = bx * bm;
    nrows = min(bm, p.rows - row0);
    return nrows > 0;
  }
  if (bx >= uload_i32(p.plan_ntiles)) return false;
  const int32_t *t = p.plan_tiles + 3 * bx;
  e = uload_i32(t);
  row0 = uload_i32(t + 1);
  nrows = uload_i32(t + 2);
  return true;
}

constexpr int kLdsStride = 132;  // 128 columns + 4 floats of padding

}  // namespace exl3
