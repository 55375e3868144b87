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
//   P_t[row][n] = v_mfma_f32_16x16x32_f16 chain over ascending 32-input
//                 k-steps (each two whole trellis tiles along k), from 0
//   acc         = fmaf(s_t, P_t, acc) over stages in order, from acc = 0,
//                 stages with s_t == 0 skipped
//   epilogue    = fixed-order fp32 FWHT per 128-block, then per-element
//                 scalings, identical code for every tile shape.
#include <algorithm>
#include <utility>

#include "gemm_shared.hpp"

namespace exl3 {

// Narrow tiles: rows per tile are 16 (one MFMA row block); each wave owns one
// 16-column strip (one tile column nt) over the whole input dimension. Two
// register buffers of kGroup k-blocks (64 inputs each) alternate: one is in
// flight while the other is decoded and multiplied. Every load is issued
// unconditionally (tail groups re-read the last group) so the compiler can
// count outstanding loads exactly.
//
// MFMA k-step s (0, 1) of k-block kb covers inputs 64 kb + 32 s .. +31, i.e.
// trellis tiles 4 kb + 2 s and 4 kb + 2 s + 1 along k. Lane (g, n) supplies
// states 8 (g & 1) .. +7 of column n of tile 4 kb + 2 s + (g >> 1) (a half
// column) and the matching 8 rotated inputs. The 128-row kernel uses the same
// k-steps, so both run one MFMA chain per output.
constexpr int kGroup = 2;

template <int K>
struct ChainBuf {
  uint32_t raw[kGroup][2][HalfGeom<K>::kLoadDw];
  u32x4 a[kGroup][2];
};

template <int K>
__device__ __forceinline__ void chain_load(ChainBuf<K> &b, __amdgpu_buffer_rsrc_t wr,
                                           const uint32_t (&voff)[HalfGeom<K>::kLoadDw],
                                           __amdgpu_buffer_rsrc_t ar, uint32_t avoff, int kb0) {
  constexpr int TD = Geom<K>::kTileDw;
#pragma unroll
  for (int u = 0; u < kGroup; ++u) {
    const int kb = kb0 + u;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int koff = (kb * 4 + 2 * s) * TD * 4;  // bytes of the k-step's first tile
#pragma unroll
      for (int j = 0; j < HalfGeom<K>::kLoadDw; ++j)
        b.raw[u][s][j] = __builtin_amdgcn_raw_buffer_load_b32(wr, voff[j], koff, 0);
      b.a[u][s] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(ar, avoff, kb * 128 + 64 * s, 0));
    }
  }
}

template <int K>
__device__ __forceinline__ void chain_compute(const ChainBuf<K> &b, uint32_t shift, uint32_t mask,
                                              int nvalid, f32x4 &acc) {
  constexpr int NN = HalfGeom<K>::kNormDw;
#pragma unroll
  for (int u = 0; u < kGroup; ++u) {
    if (u < nvalid) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        uint32_t N[NN];
        normalize(b.raw[u][s], shift, N);
        const u32x4 w = {half_reg<K, 0>(N, mask), half_reg<K, 1>(N, mask),
                         half_reg<K, 2>(N, mask), half_reg<K, 3>(N, mask)};
        acc = mfma16x16x32(__builtin_bit_cast(f16x8, b.a[u][s]), __builtin_bit_cast(f16x8, w), acc);
      }
    }
  }
}

// P = MFMA chain of one stage over all inputs for this wave's strip.
// strip: the 16-column strip's tiles (in_f/16 tiles of 32K bytes);
// ar/avoff: A rows (kSigma order) and this lane's byte offset of its row.
// in_f is a multiple of 128.
template <int K>
__device__ __forceinline__ f32x4 stage_chain(const uint32_t *strip, int in_f,
                                             __amdgpu_buffer_rsrc_t ar, uint32_t avoff, int lane) {
  constexpr int ND = HalfGeom<K>::kLoadDw, TD = Geom<K>::kTileDw;
  const int g = lane >> 4, n = lane & 15;
  // window of states 8h .. 8h+7 of column n: first bit 16nK + 8hK + K - 16
  const int b = 16 * n * K + 8 * (g & 1) * K + K - 16;
  const int d0 = b >> 5;  // floor
  const uint32_t shift = (uint32_t)(b & 31);
  uint32_t voff[ND];
#pragma unroll
  for (int j = 0; j < ND; ++j) {
    int d = d0 + j;
    d += (d < 0) ? TD : 0;
    d -= (d >= TD) ? TD : 0;
    voff[j] = (uint32_t)((g >> 1) * TD + d) * 4u;
  }
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(strip, (uint32_t)(in_f / 16) * 32u * K);
  avoff += 16u * g;  // 8 halves per k-group
  const uint32_t mask = codebook_mask();
  const int nkb = in_f >> 6;
  const int last = nkb - kGroup;  // start of the last full group
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  ChainBuf<K> A, B;
  chain_load<K>(A, wr, voff, ar, avoff, 0);
  for (int kb0 = 0; kb0 < nkb; kb0 += 2 * kGroup) {
    chain_load<K>(B, wr, voff, ar, avoff, min(kb0 + kGroup, last));
    chain_compute<K>(A, shift, mask, nkb - kb0, acc);
    chain_load<K>(A, wr, voff, ar, avoff, min(kb0 + 2 * kGroup, last));
    chain_compute<K>(B, shift, mask, nkb - kb0 - kGroup, acc);
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
    const float s = uload_f32(pd.scale + t * E + e);
    if (s == 0.0f) continue;  // zero scale: the stage is skipped entirely
    const uint32_t *tens = uload_ptr(pd.trellis + t * E + e);
    const int K = uload_i32(pd.bits + t * E + e);
    if (tens == nullptr || K < 2 || K > 8) {
      if (report && lane == 0) atomicAdd(ctrl + 1, 1);
      continue;
    }
    const uint32_t *strip = tens + strip_dw_per_bit * K;
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

// ------------------------------------------------------------ narrow tiles
// 16 rows; one wave per 16-column strip over the whole input dimension.
template <int EPI>
__global__ void __launch_bounds__(EPI == EPI_GATEUP ? 1024 : 512)
    gemm_narrow_kernel(GemmParams p) {
  constexpr int NPROJ = (EPI == EPI_GATEUP) ? 2 : 1;
  __shared__ float tile[NPROJ][kBM][kLdsStride];

  int e, row0, nrows;
  if (!tile_of_block(p, kBM, blockIdx.x, e, row0, nrows)) return;
  const int nb = blockIdx.y;  // 128-column output block
  const int lane = threadIdx.x & 63;
  const int w = wave_id();
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

  const ProjDev pd = (pj == 0) ? p.proj[0] : p.proj[1];
  const f32x4 acc = project_strip(pd, p.E, e, p.in_f, nt, ar, avoff, lane, p.ctrl,
                                  nb == 0 && c16 == 0);

#pragma unroll
  for (int r = 0; r < 4; ++r) tile[pj][4 * (lane >> 4) + r][c16 * 16 + (lane & 15)] = acc[r];
  __syncthreads();
  epilogue<EPI>(p, &tile[0][0][0], kLdsStride, kBM * kLdsStride, e, row0, nrows, nb * 128, 1);
}

hipError_t launch_gemm(int epi, const GemmParams &p, int tiles, int nblocks, hipStream_t s,
                       bool wide) {
  if (tiles <= 0 || nblocks <= 0) return hipSuccess;
  if (wide) return launch_gemm_wide(epi, p, tiles, nblocks, s);
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
