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
// Pipeline: the A rows and the trellis words of a 64-input k-block are
// copied global->LDS by the DMA form of the global loads into a ring of
// kRing buffers, kRing-1 k-blocks ahead of the k-block being decoded and
// multiplied. The wait for a k-block is an exact vmcnt (every wave issues the
// same number of DMAs per k-block; tails re-issue the last k-block), followed
// by a barrier, so loads stay in flight across iterations.
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
  static constexpr int kDmaPerKb = NPROJ * 16 / 4 + 4;  // per wave: A chunks + strips
};

// One 16-byte-per-lane global->LDS DMA: lane L writes lds_base + 16 L.
// m0 is saved and restored around the copy.
__device__ __forceinline__ void dma16(const void *gaddr, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gaddr), "s"(lds_base)
      : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int K>
__device__ __forceinline__ void decode_lds(const char *tbase, const int (&idx)[5], uint32_t shift,
                                           uint32_t mask, uint32_t (&w)[8]) {
  uint32_t r[Geom<K>::kLoadDw];
#pragma unroll
  for (int j = 0; j < Geom<K>::kLoadDw; ++j) r[j] = *(const uint32_t *)(tbase + 4 * idx[j]);
  decode_column<K>(r, shift, mask, w);
}

__device__ __forceinline__ void decode_lds_k(int K, const char *tbase, const int (&idx)[5],
                                             uint32_t shift, uint32_t mask, uint32_t (&w)[8]) {
  switch (K) {
    case 2: decode_lds<2>(tbase, idx, shift, mask, w); break;
    case 3: decode_lds<3>(tbase, idx, shift, mask, w); break;
    case 4: decode_lds<4>(tbase, idx, shift, mask, w); break;
    case 5: decode_lds<5>(tbase, idx, shift, mask, w); break;
    case 6: decode_lds<6>(tbase, idx, shift, mask, w); break;
    case 7: decode_lds<7>(tbase, idx, shift, mask, w); break;
    default: decode_lds<8>(tbase, idx, shift, mask, w); break;
  }
}

// Column window of lane column n for width K (runtime K): 5 dword indices
// (extra ones wrap inside the tile and are never used) and the bit shift.
__device__ __forceinline__ void column_window(int K, int n, int (&idx)[5], uint32_t &shift) {
  const int td = 8 * K;
  const int b = 16 * n * K + K - 16;
  const int d0 = b >> 5;
  shift = (uint32_t)(b & 31);
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    int d = d0 + j;
    d += (d < 0) ? td : 0;
    d -= (d >= td) ? td : 0;
    d -= (d >= td) ? td : 0;
    idx[j] = d;
  }
}

template <int EPI, bool MULTI>
__global__ void __launch_bounds__(256, 1) gemm_wide_kernel(GemmParams p) {
  using L = WideLds<EPI>;
  constexpr int NPROJ = L::NPROJ;
  constexpr int kAChunks = NPROJ * 16 / 4;  // 1 KB A chunks per wave per k-block
  __shared__ __attribute__((aligned(16))) char smem[L::kBytes];

  int e, row0, nrows;
  if (!tile_of_block(p, kWBM, blockIdx.x, e, row0, nrows)) return;
  const int nb = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int pj = (EPI == EPI_GATEUP) ? (w >> 1) : 0;
  const int colbase = (EPI == EPI_GATEUP) ? nb * 128 : nb * 256;
  const int colw = colbase + ((EPI == EPI_GATEUP) ? 64 * (w & 1) : 64 * w);
  const bool col_ok = colw < p.out_f;
  const int nt0 = colw >> 4;
  const int g = lane >> 4, n = lane & 15;
  const int msub_act = (nrows + 15) >> 4;
  const int nkb = p.in_f >> 6;
  const int ktiles = p.in_f >> 4;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  // A chunk c of this wave: 8 rows x 128 B; lane L -> row 8 rg + L/8, slot
  // L%8 holding global 16-byte chunk (L%8) ^ (row & 7) (bank swizzle).
  const uint16_t *asrc[kAChunks];
  uint32_t adst[kAChunks];
#pragma unroll
  for (int c = 0; c < kAChunks; ++c) {
    const int f = w * kAChunks + c;
    const int q = f >> 4, rg = f & 15;
    const int r = 8 * rg + (lane >> 3);
    const int rs = min(r, nrows - 1);
    const int gc = (lane & 7) ^ (r & 7);
    asrc[c] = p.A + (int64_t)(row0 + rs) * p.lda + q * p.a_proj_stride + gc * 8;
    adst[c] = (uint32_t)(L::kAOff + q * kAbuf + rg * 1024);
  }
  auto a_frag = [&](int buf, int ms, int s) -> f16x8 {
    const int r = 16 * ms + n;
    const int c = (2 * g + s) ^ (r & 7);
    return *(const f16x8 *)(smem + L::kAOff + (buf * NPROJ + pj) * kAbuf + r * 128 + c * 16);
  };

  const uint32_t mask = codebook_mask();
  // acc: running stage sum (only with several stages); pacc: one stage's chain
  f32x4 acc[MULTI ? 8 : 1][4];
  f32x4 pacc[8][4];
#pragma unroll
  for (int ms = 0; ms < (MULTI ? 8 : 1); ++ms)
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) acc[ms][ns] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const ProjDev pd = (pj == 0) ? p.proj[0] : p.proj[NPROJ - 1];
  const int nst = MULTI ? max(p.proj[0].num_stages, p.proj[NPROJ - 1].num_stages) : 1;
  for (int t = 0; t < nst; ++t) {
    float sc = 0.0f;
    int K = 4;
    const uint32_t *tens = nullptr;
    if (t < pd.num_stages && col_ok) {
      sc = uload_f32(pd.scale + t * p.E + e);
      K = uload_i32(pd.bits + t * p.E + e);
      tens = uload_ptr(pd.trellis + t * p.E + e);
      if (sc != 0.0f && (tens == nullptr || K < 2 || K > 8)) {
        if (nb == 0 && (w & 1) == 0 && lane == 0) atomicAdd(p.ctrl + 1, 1);
        sc = 0.0f;
      }
    }
    const bool active = __builtin_amdgcn_readfirstlane(sc != 0.0f ? 1 : 0) != 0;
    if (!active) K = 4;
    int idx[5];
    uint32_t shift;
    column_window(K, n, idx, shift);
    const int seg = 128 * K;  // bytes of one strip's 4 tiles of a k-block
    // trellis DMA source of this lane for strip ns: 16 bytes at 16*min(L, seg/16-1)
    // of the strip's k-block segment (lanes past the segment repeat its last
    // chunk into the unused tail of the 1 KB slot). Inactive waves copy from
    // their A rows instead (never decoded).
    const char *tsrc[4];
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
      const int ch = min(lane, seg / 16 - 1);
      tsrc[ns] = active ? (const char *)tens + (size_t)(nt0 + ns) * ktiles * 32 * K + 16 * ch
                        : (const char *)asrc[0];
    }
    const uint32_t tdst = (uint32_t)(L::kTOff + w * 4 * kTslot);
    const int kstride = active ? 4 * 32 * K : 0;  // bytes per k-block in a strip

    auto issue = [&](int kb, int buf) {
#pragma unroll
      for (int c = 0; c < kAChunks; ++c)
        dma16(asrc[c] + kb * 64, lds0 + adst[c] + buf * NPROJ * kAbuf);
#pragma unroll
      for (int ns = 0; ns < 4; ++ns)
        dma16(tsrc[ns] + (size_t)kb * kstride, lds0 + tdst + buf * kTbuf + ns * kTslot);
    };

#pragma unroll
    for (int ms = 0; ms < 8; ++ms)
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) pacc[ms][ns] = (f32x4){0.f, 0.f, 0.f, 0.f};

    __syncthreads();  // previous users of the ring are done
#pragma unroll
    for (int d = 0; d < kRing - 1; ++d) issue(min(d, nkb - 1), d);
    int buf = 0;
    for (int kb = 0; kb < nkb; ++kb) {
      // DMAs of k-block kb are done once at most (kRing-2) later k-blocks'
      // worth of DMAs are still outstanding
      wait_vmcnt<(kRing - 2) * L::kDmaPerKb>();
      __syncthreads();
      const int nbuf = (buf + kRing - 1) % kRing;
      issue(min(kb + kRing - 1, nkb - 1), nbuf);
      if (active) {
        uint32_t bw[4][8];
        const char *tb = smem + L::kTOff + buf * kTbuf + w * 4 * kTslot + g * 32 * K;
#pragma unroll
        for (int ns = 0; ns < 4; ++ns)
          decode_lds_k(K, tb + ns * kTslot, idx, shift, mask, bw[ns]);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          f16x8 bf[4];
#pragma unroll
          for (int ns = 0; ns < 4; ++ns)
            bf[ns] = __builtin_bit_cast(f16x8, (u32x4){bw[ns][4 * s], bw[ns][4 * s + 1],
                                                        bw[ns][4 * s + 2], bw[ns][4 * s + 3]});
          f16x8 af[8];
#pragma unroll
          for (int ms = 0; ms < 8; ++ms) af[ms] = a_frag(buf, ms, s);
          if (msub_act == 8) {
#pragma unroll
            for (int ms = 0; ms < 8; ++ms)
#pragma unroll
              for (int ns = 0; ns < 4; ++ns)
                pacc[ms][ns] = mfma16x16x32(af[ms], bf[ns], pacc[ms][ns]);
          } else {
#pragma unroll
            for (int ms = 0; ms < 8; ++ms) {
              if (ms < msub_act) {
#pragma unroll
                for (int ns = 0; ns < 4; ++ns)
                  pacc[ms][ns] = mfma16x16x32(af[ms], bf[ns], pacc[ms][ns]);
              }
            }
          }
        }
      }
      buf = (buf + 1 == kRing) ? 0 : buf + 1;
    }
    wait_vmcnt<0>();  // drain the tail DMAs before the ring is reused
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
  const f32x4(&fin)[8][4] = *reinterpret_cast<const f32x4(*)[8][4]>(MULTI ? &acc[0][0] : &pacc[0][0]);

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
        T[pj * (kWBM * L::kLd) + (16 * ms + 4 * g + r) * L::kLd + cw + 16 * ns + n] =
            fin[ms][ns][r];
  __syncthreads();
  const int nblk = (EPI == EPI_GATEUP) ? 1 : min(2, (p.out_f - colbase) / 128);
  epilogue<EPI>(p, T, L::kLd, kWBM * L::kLd, e, row0, nrows, colbase, nblk);
}

hipError_t launch_gemm(int epi, const GemmParams &p, int tiles, int nblocks, hipStream_t s,
                       bool wide) {
  if (tiles <= 0 || nblocks <= 0) return hipSuccess;
  const dim3 grid(tiles, nblocks);
  const bool multi = p.proj[0].num_stages > 1 || (epi == EPI_GATEUP && p.proj[1].num_stages > 1);
  if (wide) {
#define EXL3_WIDE(E, M) hipLaunchKernelGGL((gemm_wide_kernel<E, M>), grid, dim3(256), 0, s, p)
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
