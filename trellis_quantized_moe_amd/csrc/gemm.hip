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
#include <algorithm>
#include <utility>

#include "common.hpp"
#include "kernels.hpp"

namespace exl3 {

// Narrow tiles: rows per tile are 16 (one MFMA row block); each wave owns one 16-column
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

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// ---------------------------------------------------------------- epilogue
// Shared by every tile shape, so a row's bytes never depend on the tile it
// was computed in. T is an LDS tile of fp32 pre-rotation accumulators:
// T[pj * proj_stride + row * ld + c], c = 0 .. 128*nblk-1 (columns relative
// to colbase). One 16-lane group handles one (row, 128-block) at a time.
template <int EPI>
__device__ __forceinline__ void epilogue(const GemmParams &p, float *T, int ld, int proj_stride,
                                         int e, int row0, int nrows, int colbase, int nblk) {
  const int ngroups = blockDim.x >> 4;
  const int grp = threadIdx.x >> 4;
  const int i = threadIdx.x & 15;
  if constexpr (EPI == EPI_GATEUP) {
    // y = H(acc)/sqrt(128) * svh * cs for gate (pj 0) and up (pj 1)
    for (int it = grp; it < 2 * nrows; it += ngroups) {
      const int q = it / nrows, row = it - q * nrows;
      float *t = T + q * proj_stride + row * ld;
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = t[i + 16 * j];
      fwht128_group16(v);
      const ProjDev &pd = p.proj[q];
      const size_t ob = (size_t)e * p.out_f + colbase;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = i + 16 * j;
        t[c] = ((v[j] * kRsqrt128) * f16_bits_to_f32(pd.svh[ob + c])) *
               f16_bits_to_f32(pd.cs[ob + c]);
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
        v[j] = (silu(tg[c]) * tu[c]) * f16_bits_to_f32(p.suh_down[sb + c]);
      }
      fwht128_group16(v);
      uint16_t *o = p.out_h + (int64_t)(row0 + row) * p.ldo + colbase;
#pragma unroll
      for (int j = 0; j < 8; ++j) o[16 * j + sigma_inv(i)] = f32_to_f16_bits(v[j] * kRsqrt128);
    }
  } else {
    const ProjDev &pd = p.proj[0];
    for (int it = grp; it < nrows * nblk; it += ngroups) {
      const int row = it / nblk, blk = it - row * nblk;
      const float *t = T + row * ld + blk * 128;
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = t[i + 16 * j];
      fwht128_group16(v);
      const int cb = colbase + blk * 128;
      const size_t ob = (size_t)e * p.out_f + cb;
      float wt = 1.0f;
      if constexpr (EPI == EPI_DOWN) wt = p.weight_of_pos[p.pass_base + row0 + row];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = i + 16 * j;
        const float y = ((v[j] * kRsqrt128) * f16_bits_to_f32(pd.svh[ob + c])) *
                        f16_bits_to_f32(pd.cs[ob + c]);
        const int64_t o = (int64_t)(row0 + row) * p.ldo + cb + c;
        if constexpr (EPI == EPI_DOWN) {
          p.out_f32[o] = y * wt;
        } else {
          if (p.out_f32) p.out_f32[o] = y;
          else p.out_h[o] = f32_to_f16_bits(y);
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

// -------------------------------------------------------------- wide tiles
// 128 rows x 256 columns per workgroup of 4 waves; each wave owns 64 columns
// (4 strips) over all 128 rows (8 MFMA row blocks). GATEUP: waves 0-1 gate,
// 2-3 up (128 columns each); otherwise 256 consecutive output columns.
//
// Software pipeline over 64-input k-blocks. A rows and trellis words are
// copied global->LDS by DMA (SGPR base + per-lane offset) into rings of
// three buffers: at k-block kb a wave issues A[kb+2] and T[kb+3], multiplies
// A[kb] by the B operands decoded one iteration earlier, and meanwhile
// decodes T[kb+1] into the other B register set. Every wave issues the same
// number of DMAs per iteration (tails re-copy the last k-block), so the wait
// for the data of iteration kb is an exact vmcnt with one iteration of DMAs
// still in flight, followed by one barrier.
constexpr int kWBM = 128;
constexpr int kRing = 3;
constexpr int kAbuf = 128 * 128;        // bytes: one projection's A k-block
constexpr int kTslot = 1024;            // bytes: one strip's 4 tiles (K <= 8)
constexpr int kTbuf = 4 * 4 * kTslot;   // bytes: 4 waves x 4 strips

template <int EPI>
struct WideLds {
  static constexpr int NPROJ = (EPI == EPI_GATEUP) ? 2 : 1;
  static constexpr int kCols = (EPI == EPI_GATEUP) ? 128 : 256;  // per projection
  static constexpr int kLd = kCols + 4;
  static constexpr int kTileBytes = NPROJ * kWBM * kLd * 4;
  static constexpr int kAOff = 0;
  static constexpr int kTOff = kRing * NPROJ * kAbuf;
  static constexpr int kRingBytes = kTOff + kRing * kTbuf;
  static constexpr int kBytes = kTileBytes > kRingBytes ? kTileBytes : kRingBytes;
  static constexpr int kAChunks = NPROJ * 16 / 4;  // 1 KB A chunks per wave per k-block
  static constexpr int kDmaPerIter = kAChunks + 4;
};

// 16-byte chunk swizzle of A row r (0..15 inside its 16-row block). A row is
// 128 bytes; the 16 lanes of a fragment read (rows 0..15, one chunk index)
// land on 16 distinct 16-byte bank groups of a 256-byte bank window, and any
// 8 consecutive rows on 8 distinct groups of a 128-byte window.
__device__ __forceinline__ int a_swizzle(int r) { return (r ^ (r >> 3)) & 7; }

// 16-byte-per-lane global->LDS copy: lane L reads sbase + voff and writes
// LDS byte m0 + 16 L. The wave's LDS destination goes through m0.
__device__ __forceinline__ void dma16(uint32_t voff, const void *sbase, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "s"(lds_base)
      : "memory");
}

// dma16 with only the lanes in `lanes` active. The exec mask is narrowed and
// restored inside one asm block, so the caller's code stays one basic block
// (a branch would split the scheduling units of the pipelined loop).
__device__ __forceinline__ void dma16_lanes(uint32_t voff, const void *sbase, uint32_t lds_base,
                                            uint64_t lanes) {
  uint64_t saved;
  asm volatile(
      "s_mov_b64 %0, exec\n\t"
      "s_and_b64 exec, exec, %4\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b64 exec, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds_base), "s"(lanes)
      : "memory");
}

__device__ __forceinline__ const char *uniform_ptr(const char *ptr) {
  const uint64_t b = (uint64_t)(uintptr_t)ptr;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  return (const char *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Column window of lane column n for width K: dword indices and bit shift.
template <int K>
__device__ __forceinline__ void column_window_k(int n, int (&idx)[Geom<K>::kLoadDw],
                                                uint32_t &shift) {
  constexpr int td = 8 * K;
  const int b = 16 * n * K + K - 16;
  const int d0 = b >> 5;
  shift = (uint32_t)(b & 31);
#pragma unroll
  for (int j = 0; j < Geom<K>::kLoadDw; ++j) {
    int d = d0 + j;
    d += (d < 0) ? td : 0;
    d -= (d >= td) ? td : 0;
    idx[j] = d;
  }
}

// One scheduling unit of a pipelined wide iteration: decode register V of
// strip NS of the next k-block and issue this unit's share of the current
// k-block's MFMAs (MFMA m: step m / (4 MS), row block (m / 4) % MS, strip
// m % 4). Units are separated by scheduling barriers so that the in-order
// issue alternates MFMAs with decode VALU work.
// DMA d of an iteration (G per iteration) is issued in unit (32 d) / G.
template <int G, int U>
constexpr int dma_of_unit() {
  for (int d = 0; d < G; ++d)
    if (d * 32 / G == U) return d;
  return -1;
}

template <int K, int MS, int G, int U, typename Dma>
__device__ __forceinline__ void wide_unit(const uint32_t (&N)[4][Geom<K>::kNormDw],
                                          uint32_t mask, const f16x8 (&af)[2][MS],
                                          const f16x8 (&bf)[2][4], f32x4 (&pacc)[8][4],
                                          uint32_t (&nxt)[4][8], Dma &dma) {
  constexpr int NS = U / 8, V = U % 8;
  constexpr int D = dma_of_unit<G, U>();
  if constexpr (D >= 0) dma(D);
  nxt[NS][V] = column_reg<K, V>(N[NS], mask);
  constexpr int M = 8 * MS, m0 = U * M / 32, m1 = (U + 1) * M / 32;
#pragma unroll
  for (int m = m0; m < m1; ++m) {
    const int s = m / (4 * MS), ms = (m / 4) % MS, ns = m % 4;
    pacc[ms][ns] = mfma16x16x32(af[s][ms], bf[s][ns], pacc[ms][ns]);
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <int K, int MS, int G, typename Dma, int... Us>
__device__ __forceinline__ void wide_units(const uint32_t (&N)[4][Geom<K>::kNormDw],
                                           uint32_t mask, const f16x8 (&af)[2][MS],
                                           const f16x8 (&bf)[2][4], f32x4 (&pacc)[8][4],
                                           uint32_t (&nxt)[4][8], Dma &dma,
                                           std::integer_sequence<int, Us...>) {
  (wide_unit<K, MS, G, Us>(N, mask, af, bf, pacc, nxt, dma), ...);
}

struct WideArgs {
  int e, row0, nrows, nb, w, pj, lane, nkb, colbase;
  const char *abase;     // A rows of the tile (uniform)
  uint32_t avoff[8];     // per A chunk: lane's byte offset from abase
  uint32_t adst[8];      // per A chunk: LDS byte offset inside an A buffer
  uint32_t lds0;         // LDS address of smem
};

// One projection stage over all k-blocks for one wave: pacc += A x W_t.
// MS = number of 16-row blocks multiplied (the tile's valid rows rounded up).
template <int EPI, int K, int MS>
__device__ __forceinline__ void wide_stage(const WideArgs &c, char *smem, const char *tens,
                                           int nt0, int ktiles, f32x4 (&pacc)[8][4]) {
  using L = WideLds<EPI>;
  constexpr int NPROJ = L::NPROJ;
  constexpr int ND = Geom<K>::kLoadDw;
  constexpr int TD = Geom<K>::kTileDw;
  constexpr int SEG = 128 * K;               // bytes of a strip's k-block (4 tiles)
  constexpr uint64_t kSegLanes = (SEG >= 1024) ? ~0ull : ((1ull << (SEG / 16)) - 1);
  const int lane = c.lane, g = lane >> 4, n = lane & 15;
  const int nkb = c.nkb;

  // trellis DMA: lane L copies 16 bytes at 16 min(L, SEG/16 - 1) of each
  // strip's k-block segment (lanes past the segment repeat its last chunk
  // into the unused tail of the 1 KB slot)
  uint32_t tvoff[4];
#pragma unroll
  for (int ns = 0; ns < 4; ++ns)
    tvoff[ns] = (uint32_t)((nt0 + ns) * ktiles * 32 * K + 16 * min(lane, SEG / 16 - 1));
  const uint32_t tdst = (uint32_t)(L::kTOff + c.w * 4 * kTslot);

  // decode reads: dword idx of the lane's column inside tile g of a strip slot
  int idx[ND];
  uint32_t shift;
  column_window_k<K>(n, idx, shift);
  uint32_t traddr[ND];
#pragma unroll
  for (int j = 0; j < ND; ++j)
    traddr[j] = (uint32_t)(L::kTOff + c.w * 4 * kTslot + g * 32 * K + 4 * idx[j]);
  // A fragment reads: row 16 ms + n, 16-byte chunk (2g + s) ^ a_swizzle(n)
  uint32_t afrag[2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
    afrag[s] = (uint32_t)(L::kAOff + c.pj * kAbuf + n * 128 + (((2 * g + s) ^ a_swizzle(n)) * 16));
  const uint32_t mask = codebook_mask();

  // DMA d of k-block (ka, kt): d < kAChunks copies A chunk d, the others
  // the trellis segment of strip d - kAChunks (lanes past the segment idle)
  auto dma_one = [&](int d, int ka, int kt, int abuf, int tbuf) {
    if (d < L::kAChunks) {
      const char *ab = uniform_ptr(c.abase + (size_t)ka * 128);
      dma16(c.avoff[d], ab, c.lds0 + c.adst[d] + abuf * NPROJ * kAbuf);
    } else {
      const int ns = d - L::kAChunks;
      const char *tb = uniform_ptr(tens + (size_t)kt * 4 * 32 * K);
      if constexpr (SEG >= 1024) dma16(tvoff[ns], tb, c.lds0 + tdst + tbuf * kTbuf + ns * kTslot);
      else dma16_lanes(tvoff[ns], tb, c.lds0 + tdst + tbuf * kTbuf + ns * kTslot, kSegLanes);
    }
  };
  auto issue = [&](int ka, int kt, int abuf, int tbuf) {
#pragma unroll
    for (int d = 0; d < L::kDmaPerIter; ++d) dma_one(d, ka, kt, abuf, tbuf);
  };
  auto decode = [&](int tbuf, uint32_t (&bw)[4][8]) {
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
      uint32_t r[ND];
#pragma unroll
      for (int j = 0; j < ND; ++j)
        r[j] = *(const uint32_t *)(smem + traddr[j] + tbuf * kTbuf + ns * kTslot);
      decode_column<K>(r, shift, mask, bw[ns]);
    }
  };
  // multiply A[abuf] by the current B registers while decoding the next
  // k-block from T[tbuf] into nxt, interleaved unit by unit
  // issuing k-block (ka, kt) into (dabuf, dtbuf) one DMA at a time
  auto step = [&](int abuf, int tbuf, const uint32_t (&cur)[4][8], uint32_t (&nxt)[4][8],
                  int ka, int kt, int dabuf, int dtbuf) {
    uint32_t r[4][ND];
#pragma unroll
    for (int ns = 0; ns < 4; ++ns)
#pragma unroll
      for (int j = 0; j < ND; ++j)
        r[ns][j] = *(const uint32_t *)(smem + traddr[j] + tbuf * kTbuf + ns * kTslot);
    f16x8 af[2][MS];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int ms = 0; ms < MS; ++ms)
        af[st][ms] = *(const f16x8 *)(smem + afrag[st] + abuf * NPROJ * kAbuf + ms * 2048);
    f16x8 bf[2][4];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int ns = 0; ns < 4; ++ns)
        bf[st][ns] = __builtin_bit_cast(f16x8, (u32x4){cur[ns][4 * st], cur[ns][4 * st + 1],
                                                        cur[ns][4 * st + 2], cur[ns][4 * st + 3]});
    uint32_t N[4][Geom<K>::kNormDw];
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) column_normalize<K>(r[ns], shift, N[ns]);
    __builtin_amdgcn_sched_barrier(0);
    auto dma = [&](int d) { dma_one(d, ka, kt, dabuf, dtbuf); };
    wide_units<K, MS, L::kDmaPerIter>(N, mask, af, bf, pacc, nxt, dma,
                                      std::make_integer_sequence<int, 32>{});
  };

  uint32_t bA[4][8], bB[4][8];
  const int last = nkb - 1;
  __syncthreads();  // the LDS rings are free
  // prologue: T[0]; A[0] + T[1]; A[1] + T[2]
  const char *t0 = uniform_ptr(tens);
#pragma unroll
  for (int ns = 0; ns < 4; ++ns)
    dma16_lanes(tvoff[ns], t0, c.lds0 + tdst + 0 * kTbuf + ns * kTslot, kSegLanes);
  issue(0, min(1, last), 0, 1);
  issue(min(1, last), min(2, last), 1, 2);
  wait_vmcnt<2 * L::kDmaPerIter>();
  __syncthreads();
  decode(0, bA);

  // iteration kb: A[kb] in abuf kb%3, T[kb+1] in tbuf (kb+1)%3; issue
  // A[kb+2] -> abuf (kb+2)%3 and T[kb+3] -> tbuf kb%3, spread over the
  // iteration's units (both buffers were last read in iteration kb-1)
#define EXL3_WIDE_ITER(KB, AB, TB_NEXT, CUR, NXT)                                       \
  {                                                                                     \
    wait_vmcnt<L::kDmaPerIter>();                                                       \
    __syncthreads();                                                                    \
    step((AB), (TB_NEXT), CUR, NXT, min((KB) + 2, last), min((KB) + 3, last),           \
         ((AB) + 2) % 3, (AB));                                                         \
  }
  int kb = 0;
  for (; kb + 6 <= nkb; kb += 6) {
    EXL3_WIDE_ITER(kb + 0, 0, 1, bA, bB)
    EXL3_WIDE_ITER(kb + 1, 1, 2, bB, bA)
    EXL3_WIDE_ITER(kb + 2, 2, 0, bA, bB)
    EXL3_WIDE_ITER(kb + 3, 0, 1, bB, bA)
    EXL3_WIDE_ITER(kb + 4, 1, 2, bA, bB)
    EXL3_WIDE_ITER(kb + 5, 2, 0, bB, bA)
  }
  // remainder (nkb is even): 0, 2 or 4 k-blocks, buffers continue from 0
  if (kb + 2 <= nkb) {
    EXL3_WIDE_ITER(kb + 0, 0, 1, bA, bB)
    EXL3_WIDE_ITER(kb + 1, 1, 2, bB, bA)
    kb += 2;
    if (kb + 2 <= nkb) {
      EXL3_WIDE_ITER(kb + 0, 2, 0, bA, bB)
      EXL3_WIDE_ITER(kb + 1, 0, 1, bB, bA)
    }
  }
#undef EXL3_WIDE_ITER
  wait_vmcnt<0>();  // drain tail DMAs before the LDS is reused
}

// A wave with no work for this stage still takes part in the DMA/barrier
// cadence of its workgroup (same counts, data never read).
template <int EPI>
__device__ __forceinline__ void wide_idle_stage(const WideArgs &c) {
  using L = WideLds<EPI>;
  const int nkb = c.nkb;
  const uint32_t tdst = (uint32_t)(L::kTOff + c.w * 4 * kTslot);
  auto issue = [&](int ka, int abuf, int tbuf) {
    const char *ab = uniform_ptr(c.abase + (size_t)ka * 128);
#pragma unroll
    for (int ch = 0; ch < L::kAChunks; ++ch)
      dma16(c.avoff[ch], ab, c.lds0 + c.adst[ch] + abuf * L::NPROJ * kAbuf);
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) dma16(c.avoff[0], ab, c.lds0 + tdst + tbuf * kTbuf + ns * kTslot);
  };
  const int last = nkb - 1;
  __syncthreads();
  const char *a0 = uniform_ptr(c.abase);
#pragma unroll
  for (int ns = 0; ns < 4; ++ns) dma16(c.avoff[0], a0, c.lds0 + tdst + ns * kTslot);
  issue(0, 0, 1);
  issue(min(1, last), 1, 2);
  wait_vmcnt<2 * L::kDmaPerIter>();
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    wait_vmcnt<L::kDmaPerIter>();
    __syncthreads();
    const int ab = kb % 3;
    issue(min(kb + 2, last), (ab + 2) % 3, ab);
  }
  wait_vmcnt<0>();
}

template <int EPI, int K>
__device__ __forceinline__ void wide_stage_rows(const WideArgs &c, char *smem, const char *tens,
                                                int nt0, int ktiles, int msub,
                                                f32x4 (&pacc)[8][4]) {
  if (msub <= 2) wide_stage<EPI, K, 2>(c, smem, tens, nt0, ktiles, pacc);
  else if (msub <= 4) wide_stage<EPI, K, 4>(c, smem, tens, nt0, ktiles, pacc);
  else wide_stage<EPI, K, 8>(c, smem, tens, nt0, ktiles, pacc);
}

// One work item: rows of tile `bx` times 256-column block `by`.
template <int EPI, bool MULTI>
__device__ __forceinline__ void wide_item(const GemmParams &p, char *smem, int bx, int by) {
  using L = WideLds<EPI>;
  constexpr int NPROJ = L::NPROJ;

  WideArgs c;
  if (!tile_of_block(p, kWBM, bx, c.e, c.row0, c.nrows)) return;
  c.nb = by;
  c.lane = threadIdx.x & 63;
  c.w = wave_id();
  c.pj = (EPI == EPI_GATEUP) ? (c.w >> 1) : 0;
  c.colbase = (EPI == EPI_GATEUP) ? c.nb * 128 : c.nb * 256;
  c.nkb = p.in_f >> 6;
  c.lds0 = (uint32_t)(uintptr_t)smem;
  const int w = c.w, lane = c.lane, g = lane >> 4, n = lane & 15;
  const int colw = c.colbase + ((EPI == EPI_GATEUP) ? 64 * (w & 1) : 64 * w);
  const bool col_ok = colw < p.out_f;
  const int nt0 = colw >> 4;
  const int ktiles = p.in_f >> 4;
  const int msub = (c.nrows + 15) >> 4;

  // A chunk ch of this wave: 8 rows x 128 B; lane L -> row 8 rg + L/8, LDS
  // slot L%8 holding the global 16-byte chunk (L%8) ^ a_swizzle(row & 15).
  c.abase = (const char *)(p.A + (int64_t)c.row0 * p.lda);
#pragma unroll
  for (int ch = 0; ch < L::kAChunks; ++ch) {
    const int f = w * L::kAChunks + ch;
    const int q = f >> 4, rg = f & 15;
    const int r = 8 * rg + (lane >> 3);
    const int rs = min(r, c.nrows - 1);
    const int gc = (lane & 7) ^ a_swizzle(r & 15);
    c.avoff[ch] = (uint32_t)(2 * ((int64_t)rs * p.lda + q * p.a_proj_stride + gc * 8));
    c.adst[ch] = (uint32_t)(L::kAOff + q * kAbuf + rg * 1024);
  }

  f32x4 acc[MULTI ? 8 : 1][4];
  f32x4 pacc[8][4];
#pragma unroll
  for (int ms = 0; ms < (MULTI ? 8 : 1); ++ms)
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) acc[ms][ns] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const ProjDev pd = (c.pj == 0) ? p.proj[0] : p.proj[NPROJ - 1];
  const int nst = MULTI ? max(p.proj[0].num_stages, p.proj[NPROJ - 1].num_stages) : 1;
  for (int t = 0; t < nst; ++t) {
    float sc = 0.0f;
    int K = 0;
    const char *tens = nullptr;
    if (t < pd.num_stages && col_ok) {
      sc = uload_f32(pd.scale + t * p.E + c.e);
      K = uload_i32(pd.bits + t * p.E + c.e);
      tens = (const char *)uload_ptr(pd.trellis + t * p.E + c.e);
      if (sc != 0.0f && (tens == nullptr || K < 2 || K > 8)) {
        if (c.nb == 0 && (w & 1) == 0 && lane == 0) atomicAdd(p.ctrl + 1, 1);
        sc = 0.0f;
      }
    }
    const bool active = __builtin_amdgcn_readfirstlane(sc != 0.0f ? 1 : 0) != 0;
#pragma unroll
    for (int ms = 0; ms < 8; ++ms)
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) pacc[ms][ns] = (f32x4){0.f, 0.f, 0.f, 0.f};
    if (!active) {
      wide_idle_stage<EPI>(c);
    } else {
      switch (K) {
        case 2: wide_stage_rows<EPI, 2>(c, smem, tens, nt0, ktiles, msub, pacc); break;
        case 3: wide_stage_rows<EPI, 3>(c, smem, tens, nt0, ktiles, msub, pacc); break;
        case 4: wide_stage_rows<EPI, 4>(c, smem, tens, nt0, ktiles, msub, pacc); break;
        case 5: wide_stage_rows<EPI, 5>(c, smem, tens, nt0, ktiles, msub, pacc); break;
        case 6: wide_stage_rows<EPI, 6>(c, smem, tens, nt0, ktiles, msub, pacc); break;
        case 7: wide_stage_rows<EPI, 7>(c, smem, tens, nt0, ktiles, msub, pacc); break;
        default: wide_stage_rows<EPI, 8>(c, smem, tens, nt0, ktiles, msub, pacc); break;
      }
    }
    // acc = fmaf(s_t, P_t, acc) from acc = 0; a skipped stage leaves acc alone
#pragma unroll
    for (int ms = 0; ms < 8; ++ms)
#pragma unroll
      for (int ns = 0; ns < 4; ++ns)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (MULTI) {
            if (active) acc[ms][ns][r] = fmaf(sc, pacc[ms][ns][r], acc[ms][ns][r]);
          } else {
            pacc[ms][ns][r] = active ? fmaf(sc, pacc[ms][ns][r], 0.0f) : 0.0f;
          }
        }
  }
  const f32x4(&fin)[8][4] =
      *reinterpret_cast<const f32x4(*)[8][4]>(MULTI ? &acc[0][0] : &pacc[0][0]);

  // ---- epilogue: accumulators -> LDS tile -> shared epilogue
  __syncthreads();
  float *T = (float *)smem;
  const int cw = (EPI == EPI_GATEUP) ? 64 * (w & 1) : 64 * w;  // column of the wave in T
#pragma unroll
  for (int ms = 0; ms < 8; ++ms)
#pragma unroll
    for (int ns = 0; ns < 4; ++ns)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        T[c.pj * (kWBM * L::kLd) + (16 * ms + 4 * g + r) * L::kLd + cw + 16 * ns + n] =
            fin[ms][ns][r];
  __syncthreads();
  const int nblk = (EPI == EPI_GATEUP) ? 1 : min(2, (p.out_f - c.colbase) / 128);
  epilogue<EPI>(p, T, L::kLd, kWBM * L::kLd, c.e, c.row0, c.nrows, c.colbase, nblk);
}

// One workgroup per (tile, 256-column block) on a 1-D grid of groups of 8
// tiles x nb column blocks. Workgroups are dealt to the 8 XCDs round-robin by
// linear id, so tile 8 G + (id % 8) keeps all its column blocks on one XCD
// (sharing its L2 copy of the tile's A rows), and the dispatch order walks
// the tiles front to back: tiles past the device's tile count (the launch is
// sized for the worst case) come last and exit at once.
template <int EPI, bool MULTI>
__global__ void __launch_bounds__(256, 1) gemm_wide_kernel(GemmParams p, int nb) {
  __shared__ __attribute__((aligned(16))) char smem[WideLds<EPI>::kBytes];
  const int id = blockIdx.x, per = 8 * nb;
  const int grp = id / per, r = id - grp * per;
  wide_item<EPI, MULTI>(p, smem, 8 * grp + (r & 7), r >> 3);
}

hipError_t launch_gemm(int epi, const GemmParams &p, int tiles, int nblocks, hipStream_t s,
                       bool wide) {
  if (tiles <= 0 || nblocks <= 0) return hipSuccess;
  const dim3 grid(tiles, nblocks);
  const bool multi = p.proj[0].num_stages > 1 || (epi == EPI_GATEUP && p.proj[1].num_stages > 1);
  if (wide) {
    const dim3 wgrid((unsigned)((tiles + 7) / 8 * 8 * nblocks));
#define EXL3_WIDE(E, M) \
  hipLaunchKernelGGL((gemm_wide_kernel<E, M>), wgrid, dim3(256), 0, s, p, nblocks)
    switch (epi) {
      case EPI_GATEUP: if (multi) EXL3_WIDE(EPI_GATEUP, true); else EXL3_WIDE(EPI_GATEUP, false); break;
      case EPI_DOWN: if (multi) EXL3_WIDE(EPI_DOWN, true); else EXL3_WIDE(EPI_DOWN, false); break;
      default: if (multi) EXL3_WIDE(EPI_LINEAR, true); else EXL3_WIDE(EPI_LINEAR, false); break;
    }
#undef EXL3_WIDE
    return hipGetLastError();
  }
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
