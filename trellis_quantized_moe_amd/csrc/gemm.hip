// Grouped EXL3 GEMM for gfx950: trellis decode straight into MFMA B operands,
// fp16 MFMA with fp32 accumulation, additive stages, and three fused
// epilogues (plain linear, gate/up -> SwiGLU -> down-input rotation, and
// down -> weighted per-pair output).
//
// What is computed follows TensorFold PR #837 "cuda: EXL3 linear and grouped
// routed experts, every codebook and width, a width per expert" (What this
// changes: decode straight into the matrix-core operands, input rotation,
// row-invariant linear, grouped experts with SwiGLU and down) and exllamav3
// PR #284 "MoE: Add fused additive EXL3 kernels" (Summary: FP32 accumulation
// and output scaling; stage tables with zero-scale sparse entries).
//
// Arithmetic contract (makes a row's bytes independent of the other rows,
// the tile it lands in, the capacity and the chunking):
//   P_t[row][n] = v_mfma_f32_16x16x32_f16 chain over k in ascending 64-blocks
//                 (two 32-steps each), starting from 0
//   acc         = fmaf(s_t, P_t, acc) over stages in order, from acc = 0,
//                 stages with s_t == 0 skipped
//   epilogue    = fixed-order fp32 FWHT per 128-block, then per-element
//                 scalings, identical code for every tile shape.
#include "common.hpp"
#include "kernels.hpp"

namespace exl3 {

// Rows per tile are 16 (one MFMA row block); each wave owns one 16-column
// strip (one tile column nt) over the whole input dimension. Two register
// buffers of kGroup k-blocks (64 inputs each) alternate: one is in flight
// while the other is decoded and multiplied. Every load is issued
// unconditionally (tail groups re-read the last group) so the compiler can
// count outstanding loads exactly.
constexpr int kGroup = 2;

template <int K>
struct ChainBuf {
  uint32_t raw[kGroup][Geom<K>::kLoadDw];
  u32x4 a[kGroup][2];
};

// Raw buffer resource (gfx9 dword 3 = 0x00020000): SGPR base, 32-bit
// per-lane offsets, out-of-range reads return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}

template <int K>
__device__ __forceinline__ void chain_load(ChainBuf<K> &b, __amdgpu_buffer_rsrc_t wr,
                                           const uint32_t (&voff)[Geom<K>::kLoadDw],
                                           __amdgpu_buffer_rsrc_t ar, uint32_t avoff, int kb0) {
  constexpr int TD = Geom<K>::kTileDw;
#pragma unroll
  for (int u = 0; u < kGroup; ++u) {
    const int kb = kb0 + u;
    const int koff = kb * 4 * TD * 4;  // bytes of four tiles per k-block
#pragma unroll
    for (int j = 0; j < Geom<K>::kLoadDw; ++j)
      b.raw[u][j] = __builtin_amdgcn_raw_buffer_load_b32(wr, voff[j], koff, 0);
    b.a[u][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ar, avoff, kb * 128, 0));
    b.a[u][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ar, avoff + 16, kb * 128, 0));
  }
}

template <int K>
__device__ __forceinline__ void chain_compute(const ChainBuf<K> &b, uint32_t shift, uint32_t mask,
                                              int nvalid, f32x4 &acc) {
#pragma unroll
  for (int u = 0; u < kGroup; ++u) {
    if (u < nvalid) {
      uint32_t w[8];
      decode_column<K>(b.raw[u], shift, mask, w);
      const f16x8 b0 = __builtin_bit_cast(f16x8, (u32x4){w[0], w[1], w[2], w[3]});
      const f16x8 b1 = __builtin_bit_cast(f16x8, (u32x4){w[4], w[5], w[6], w[7]});
      acc = mfma16x16x32(__builtin_bit_cast(f16x8, b.a[u][0]), b0, acc);
      acc = mfma16x16x32(__builtin_bit_cast(f16x8, b.a[u][1]), b1, acc);
    }
  }
}

// P = MFMA chain of one stage over all inputs for this wave's strip.
// strip: the 16-column strip's tiles (in_f/16 tiles of 32K bytes);
// ar/avoff: A rows (kSigma order) and this lane's byte offset of its row and
// k-group. in_f is a multiple of 128.
template <int K>
__device__ __forceinline__ f32x4 stage_chain(const uint32_t *strip, int in_f,
                                             __amdgpu_buffer_rsrc_t ar, uint32_t avoff, int lane) {
  constexpr int ND = Geom<K>::kLoadDw, TD = Geom<K>::kTileDw;
  const int g = lane >> 4;
  const ColumnWindow<K> cw(lane & 15);
  uint32_t voff[ND];
#pragma unroll
  for (int j = 0; j < ND; ++j) voff[j] = (uint32_t)(g * TD + cw.idx[j]) * 4u;
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(strip, (uint32_t)(in_f / 16) * 32u * K);
  avoff += 32u * g;  // 16 halves per k-group
  const uint32_t mask = codebook_mask();
  const int nkb = in_f >> 6;
  const int last = nkb - kGroup;  // start of the last full group
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  ChainBuf<K> A, B;
  chain_load<K>(A, wr, voff, ar, avoff, 0);
  for (int kb0 = 0; kb0 < nkb; kb0 += 2 * kGroup) {
    chain_load<K>(B, wr, voff, ar, avoff, min(kb0 + kGroup, last));
    chain_compute<K>(A, cw.shift, mask, nkb - kb0, acc);
    chain_load<K>(A, wr, voff, ar, avoff, min(kb0 + 2 * kGroup, last));
    chain_compute<K>(B, cw.shift, mask, nkb - kb0 - kGroup, acc);
  }
  return acc;
}

// Stage loop of one projection for one wave: acc = sum fmaf(s_t, P_t, acc).
__device__ __forceinline__ f32x4 project_strip(const ProjDev &pd, int E, int e,
                                               int in_f, int nt,
                                               __amdgpu_buffer_rsrc_t ar, uint32_t avoff,
                                               int lane, int32_t *ctrl, bool report) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const size_t strip_dw_per_bit = (size_t)nt * (in_f / 16) * 8;  // x K
  for (int t = 0; t < pd.num_stages; ++t) {
    const float s = pd.scale[t * E + e];
    if (s == 0.0f) continue;  // zero scale: the stage is skipped entirely
    const int64_t addr = pd.trellis[t * E + e];
    const int K = pd.bits[t * E + e];
    if (addr == 0 || K < 2 || K > 8) {
      if (report && lane == 0) atomicAdd(ctrl + 1, 1);
      continue;
    }
    const uint32_t *strip = (const uint32_t *)(uintptr_t)addr + strip_dw_per_bit * K;
    f32x4 p;
    switch (K) {
      case 2: p = stage_chain<2>(strip, in_f, ar, avoff, lane); break;
      case 3: p = stage_chain<3>(strip, in_f, ar, avoff, lane); break;
      case 4: p = stage_chain<4>(strip, in_f, ar, avoff, lane); break;
      case 5: p = stage_chain<5>(strip, in_f, ar, avoff, lane); break;
      case 6: p = stage_chain<6>(strip, in_f, ar, avoff, lane); break;
      case 7: p = stage_chain<7>(strip, in_f, ar, avoff, lane); break;
      default: p = stage_chain<8>(strip, in_f, ar, avoff, lane); break;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = fmaf(s, p[r], acc[r]);
  }
  return acc;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

constexpr int kLdsStride = 132;  // 128 columns + 4 floats of padding

template <int EPI>
__global__ void __launch_bounds__(EPI == EPI_GATEUP ? 1024 : 512)
    gemm_narrow_kernel(GemmParams p) {
  constexpr int NPROJ = (EPI == EPI_GATEUP) ? 2 : 1;
  __shared__ float tile[NPROJ][kBM][kLdsStride];

  int e, row0, nrows;
  if (p.plan_tiles == nullptr) {
    e = 0;
    row0 = blockIdx.x * kBM;
    nrows = min(kBM, p.rows - row0);
  } else {
    if ((int)blockIdx.x >= *p.plan_ntiles) return;
    const int32_t *t = p.plan_tiles + 3 * blockIdx.x;
    e = t[0];
    row0 = t[1];
    nrows = t[2];
  }
  const int nb = blockIdx.y;  // 128-column output block
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int pj = (EPI == EPI_GATEUP) ? (w >> 3) : 0;
  const int c16 = w & 7;
  const int nt = nb * 8 + c16;

  // Lanes of rows past the tile's end read the last valid row (same cache
  // lines, no extra traffic); their results are never stored.
  const int arow = min(lane & 15, nrows - 1);
  const uint16_t *a_tile = p.A + (int64_t)row0 * p.lda + pj * p.a_proj_stride;
  const __amdgpu_buffer_rsrc_t ar =
      make_rsrc(a_tile, (uint32_t)((int64_t)(nrows - 1) * p.lda * 2 + 2 * p.in_f));
  const uint32_t avoff = (uint32_t)(arow * p.lda * 2);

  const f32x4 acc = project_strip(p.proj[pj], p.E, e, p.in_f, nt, ar, avoff, lane, p.ctrl,
                                  nb == 0 && c16 == 0);

  // MFMA layout -> LDS tile[row][col]
#pragma unroll
  for (int r = 0; r < 4; ++r) tile[pj][4 * (lane >> 4) + r][c16 * 16 + (lane & 15)] = acc[r];
  __syncthreads();

  const int grp = threadIdx.x >> 4;  // 16-lane group
  const int i = threadIdx.x & 15;
  const int colbase = nb * 128;

  if constexpr (EPI == EPI_GATEUP) {
    // Phase 1: output rotation of gate and up: y = H(acc) / sqrt(128) * svh * cs
    {
      const int q = grp >> 4, row = grp & 15;  // 64 groups: 2 proj x 16 rows x 2
      if ((grp < 32) && row < nrows) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = tile[q][row][i + 16 * j];
        fwht128_group16(v);
        const ProjDev &pd = p.proj[q];
        const size_t ob = (size_t)e * p.out_f + colbase;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int c = i + 16 * j;
          tile[q][row][c] = ((v[j] * kRsqrt128) * f16_bits_to_f32(pd.svh[ob + c])) *
                            f16_bits_to_f32(pd.cs[ob + c]);
        }
      }
    }
    __syncthreads();
    // Phase 2: a = silu(g) * u; a~ = fp16(H(a * suh_down) / sqrt(128))
    {
      const int row = grp;
      if (grp < 16 && row < nrows) {
        const size_t sb = (size_t)e * p.out_f + colbase;
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int c = i + 16 * j;
          const float gt = tile[0][row][c], up = tile[1][row][c];
          v[j] = (silu(gt) * up) * f16_bits_to_f32(p.suh_down[sb + c]);
        }
        fwht128_group16(v);
        uint16_t *o = p.out_h + (int64_t)(row0 + row) * p.ldo + colbase;
#pragma unroll
        for (int j = 0; j < 8; ++j) o[16 * j + sigma_inv(i)] = f32_to_f16_bits(v[j] * kRsqrt128);
      }
    }
  } else {
    const int row = grp;
    if (grp < 16 && row < nrows) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = tile[0][row][i + 16 * j];
      fwht128_group16(v);
      const ProjDev &pd = p.proj[0];
      const size_t ob = (size_t)e * p.out_f + colbase;
      float wt = 1.0f;
      if constexpr (EPI == EPI_DOWN) wt = p.weight_of_pos[p.pass_base + row0 + row];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = i + 16 * j;
        float y = ((v[j] * kRsqrt128) * f16_bits_to_f32(pd.svh[ob + c])) *
                  f16_bits_to_f32(pd.cs[ob + c]);
        if constexpr (EPI == EPI_DOWN) {
          p.out_f32[(int64_t)(row0 + row) * p.ldo + colbase + c] = y * wt;
        } else {
          if (p.out_f32)
            p.out_f32[(int64_t)(row0 + row) * p.ldo + colbase + c] = y;
          else
            p.out_h[(int64_t)(row0 + row) * p.ldo + colbase + c] = f32_to_f16_bits(y);
        }
      }
    }
  }
}

hipError_t launch_gemm(int epi, const GemmParams &p, int tiles, int nblocks,
                       hipStream_t s) {
  if (tiles <= 0 || nblocks <= 0) return hipSuccess;
  const dim3 grid(tiles, nblocks);
  switch (epi) {
    case EPI_GATEUP:
      hipLaunchKernelGGL(gemm_narrow_kernel<EPI_GATEUP>, grid, dim3(1024), 0, s, p);
      break;
    case EPI_DOWN:
      hipLaunchKernelGGL(gemm_narrow_kernel<EPI_DOWN>, grid, dim3(512), 0, s, p);
      break;
    default:
      hipLaunchKernelGGL(gemm_narrow_kernel<EPI_LINEAR>, grid, dim3(512), 0, s, p);
      break;
  }
  return hipGetLastError();
}

// Diagnostic decode of whole tiles with the same column decoder: one wave per
// tile, lane n (< 16) decodes column n; output [tile][k][n] fp16 in natural k.
template <int K>
__device__ void decode_tile_wave(const uint16_t *words, uint16_t *out, int lane) {
  if (lane >= 16) return;
  const uint32_t *t = (const uint32_t *)words;
  const ColumnWindow<K> cw(lane);
  uint32_t raw[Geom<K>::kLoadDw];
#pragma unroll
  for (int j = 0; j < Geom<K>::kLoadDw; ++j) raw[j] = t[cw.idx[j]];
  uint32_t b[8];
  decode_column<K>(raw, cw.shift, codebook_mask(), b);
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const int j = (v & 3) + 8 * (v >> 2);
    out[j * 16 + lane] = (uint16_t)(b[v] & 0xFFFFu);
    out[(j + 4) * 16 + lane] = (uint16_t)(b[v] >> 16);
  }
}

__global__ void decode_tiles_kernel(const uint16_t *words, int ntiles, int K,
                                    uint16_t *out) {
  const int tile = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tile >= ntiles) return;
  const int lane = threadIdx.x & 63;
  const uint16_t *w = words + (size_t)tile * 16 * K;
  uint16_t *o = out + (size_t)tile * 256;
  switch (K) {
    case 2: decode_tile_wave<2>(w, o, lane); break;
    case 3: decode_tile_wave<3>(w, o, lane); break;
    case 4: decode_tile_wave<4>(w, o, lane); break;
    case 5: decode_tile_wave<5>(w, o, lane); break;
    case 6: decode_tile_wave<6>(w, o, lane); break;
    case 7: decode_tile_wave<7>(w, o, lane); break;
    default: decode_tile_wave<8>(w, o, lane); break;
  }
}

hipError_t launch_decode_tiles(const uint16_t *words, int ntiles, int K,
                               uint16_t *out, hipStream_t s) {
  if (ntiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(decode_tiles_kernel, dim3((ntiles + 3) / 4), dim3(256), 0, s,
                     words, ntiles, K, out);
  return hipGetLastError();
}

}  // namespace exl3
