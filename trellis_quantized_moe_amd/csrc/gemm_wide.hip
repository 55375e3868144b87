// Grouped EXL3 GEMM on 128-row tiles (prefill-size work) for gfx950: the
// trellis is decoded straight into MFMA B operands and multiplied with fp16
// MFMA into fp32 accumulators. Additive stages and the shared epilogues are
// handled here too.
//
// What is computed follows TensorFold PR #837 "cuda: EXL3 linear and grouped
// routed experts, every codebook and width, a width per expert" (What this
// changes: decode straight into the matrix-core operands; grouped experts with
// SwiGLU and down) and exllamav3 PR #284 "MoE: Add fused additive EXL3
// kernels" (Summary: FP32 accumulation and output scaling; stage tables with
// per-stage tables in which a stage may be absent). The per-element
// arithmetic is the one the
// narrow kernel uses: for each output, an MFMA chain over ascending 32-input
// k-steps (each two whole trellis tiles) starting from 0, then
// acc = fmaf(s_t, P_t, acc) over the stages, then the shared epilogue.
//
// Tile: 128 rows x 256 columns per workgroup of 4 waves. Wave w owns 64
// output columns (4 strips of 16) over all 128 rows (8 MFMA row blocks): 32
// 16x16 fp32 accumulator blocks (in VGPRs; the multi-stage variant keeps a
// second set in AGPRs). GATEUP: waves 0-1 compute gate and waves 2-3 compute
// up (128 columns each), so the epilogue has both halves of SwiGLU in one
// workgroup.
//
// Two workgroups share a CU (80 KB of LDS and at most 256 registers per wave
// each). On gfx950 a wave's own VALU work hides under its MFMAs only in part
// (about two VALU instructions per 16x16x32 MFMA); the VALU decode of one
// wave also runs under the MFMAs of the other wave on the same SIMD.
//
// Launch forms: gemm_wide_kernel (one projection kind per launch: linear
// calls), gemm_wide_pass_kernel (gate/up and down of a single pass in one
// launch) and gemm_wide_pipe_kernel (several passes pipelined across
// launches), all built from wide_item below.
//
// Pipeline over 32-input stages (one MFMA k-step; 2 trellis tiles along k):
//  - A (rotated activations) is copied global->LDS by DMA into a ring of 3
//    slots. Each wave copies its share of the rows the tile's MFMAs read
//    (AMap) and all waves read all of it, so one barrier per stage
//    publishes it.
//  - Trellis words are copied global->LDS by DMA into a ring of 4 slots per
//    wave. A wave copies and reads only its own strips, so its own vmcnt
//    wait is enough (no barrier).
//  - In stage ks a wave multiplies A[ks] by B[ks], which it decoded in the
//    previous stage into registers. Meanwhile it decodes T[ks+1] into the
//    other register set and issues the DMAs of A[ks+2] and then T[ks+4].
//    The work is cut into units of two MFMAs plus a share of the decode,
//    separated by scheduling barriers.
//  - Lane (g, n) of a strip decodes states 8(g & 1) .. 8(g & 1) + 7 of column
//    n of tile g >> 1: the 8 k-entries the MFMA takes from that lane, in the
//    kSigma order of the rotated activations.
//  - Every wave issues the same DMAs in every stage (past the end it
//    re-copies the last stage). The wait for A[ks] and T[ks+1] is therefore an
//    exact vmcnt that leaves T[ks+2], A[ks+1] and T[ks+3] in flight.
#include <utility>

#include "gemm_shared.hpp"
#include "rotate_dev.hpp"
#include "combine_dev.hpp"

namespace exl3 {

constexpr int kWBM = 128;
constexpr int kARing = 3;
constexpr int kTRing = 4;
constexpr int kArow = 64;             // bytes of one A row per stage (32 fp16)
constexpr int kAbuf = kWBM * kArow;   // one projection's A stage: 8 KB
constexpr int kTstrip = 512;          // one strip's stage: 2 tiles of 32K bytes (K <= 8)
constexpr int kTwave = 4 * kTstrip;   // one wave's 4 strips
constexpr int kTstage = 4 * kTwave;   // 4 waves

template <int EPI>
struct WideLds {
  static constexpr int NPROJ = (EPI == EPI_GATEUP) ? 2 : 1;
  static constexpr int kCols = (EPI == EPI_GATEUP) ? 128 : 256;  // per projection
  static constexpr int kLd = kCols + 4;
  static constexpr int kHalf = 64;  // epilogue rows per round
  static constexpr int kTileBytes = NPROJ * kHalf * kLd * 4;
  static constexpr int kAStage = NPROJ * kAbuf;
  static constexpr int kAOff = 0;
  static constexpr int kTOff = kARing * kAStage;
  static constexpr int kRingBytes = kTOff + kTRing * kTstage;
  static constexpr int kBytes = kTileBytes > kRingBytes ? kTileBytes : kRingBytes;
};
static_assert(WideLds<EPI_GATEUP>::kBytes <= 80 * 1024, "two workgroups per CU");
static_assert(WideLds<EPI_LINEAR>::kBytes <= 80 * 1024, "two workgroups per CU");

// 16-byte chunk swizzle of A row r (0..15 inside its 16-row block); a row is
// 64 bytes (4 chunks), and lane (g, r) of an A-fragment read takes chunk g of
// row r. gfx950 serves a 64-lane ds_read_b128 as 4 groups of 16 lanes over 64
// four-byte banks; with this swizzle the LDS bank-conflict counter reads zero
// for the fragment reads (without it, or with (r>>1)^(r>>3), every read costs
// 4 extra cycles).
__device__ __forceinline__ int a_swizzle(int r) { return (r >> 1) & 3; }

// 16-byte-per-lane global->LDS copy: lane L reads sbase + voff and writes
// LDS byte m0 + 16 L. The wave's LDS destination goes through m0. Each of
// these asm blocks spends five wait states (SALU instructions plus s_nop)
// before its vector memory instruction: the compiler may write the SGPR
// operands with a VALU instruction (v_readfirstlane) just before the block,
// CDNA requires five wait states between such a write and a vector memory
// read of the SGPR, and the compiler's hazard check does not look inside
// inline asm.
__device__ __forceinline__ void dma16(uint32_t voff, const void *sbase, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 3\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "s"(lds_base)
      : "memory");
}

// dma16 with device-coherent loads (sc1): never served by a stale L2 line,
// for data another workgroup of the same launch wrote.
__device__ __forceinline__ void dma16_coh(uint32_t voff, const void *sbase, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 3\n\t"
      "global_load_lds_dwordx4 %0, %1 sc1"
      :
      : "v"(voff), "s"(sbase), "s"(lds_base)
      : "memory");
}

template <bool COH>
__device__ __forceinline__ void dma16_a(uint32_t voff, const void *sbase, uint32_t lds_base) {
  if constexpr (COH) dma16_coh(voff, sbase, lds_base);
  else dma16(voff, sbase, lds_base);
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
      "s_nop 1\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b64 exec, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds_base), "s"(lanes)
      : "memory", "scc");
}

// dma16_lanes with device-coherent loads (sc1).
__device__ __forceinline__ void dma16_lanes_coh(uint32_t voff, const void *sbase,
                                                uint32_t lds_base, uint64_t lanes) {
  uint64_t saved;
  asm volatile(
      "s_mov_b64 %0, exec\n\t"
      "s_and_b64 exec, exec, %4\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 1\n\t"
      "global_load_lds_dwordx4 %1, %2 sc1\n\t"
      "s_mov_b64 exec, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds_base), "s"(lanes)
      : "memory", "scc");
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

__device__ __forceinline__ uint32_t uniform_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

struct WideArgs {
  int e, row0, nrows, nb, w, pj, lane, nks, colbase;
  const char *abase;     // A rows of the tile (uniform)
  int64_t lda, aps;      // A row stride and projection stride (elements)
  uint32_t lds0;         // LDS address of smem
};

// The A copies of one wave for a tile of MS row blocks: a stage needs the
// NPROJ x MS 16-row chunks (1 KB each: 16 rows x 64 B) its MFMAs read, and
// the 4 waves share them evenly, so every wave issues AD copies a stage (a
// constant per MS, which keeps each vmcnt wait exact); one projection at
// MS = 2 is copied as 8-row halves, one per wave. Chunk f covers rows
// 16 (f % MS) .. +15 of projection f / MS; lane L copies row 16 rg + L / 4
// (+ 8 for the second half), LDS slot L % 4 holding the global 16-byte
// chunk (L % 4) ^ a_swizzle(row & 15). Rows past the tile's end re-read its
// last row (never stored).
template <int EPI, int MS, bool COH>
struct AMap {
  using L = WideLds<EPI>;
  static constexpr int TC = L::NPROJ * MS;       // 16-row chunks a stage needs
  static constexpr bool kHalf = TC < 4;          // 8-row halves
  static constexpr int AD = kHalf ? 1 : TC / 4;  // copies per wave and stage
  static_assert(kHalf ? TC * 2 == 4 : TC % 4 == 0, "the waves share the chunks evenly");
  uint32_t voff[AD];  // lane's byte offset from the stage's A rows
  uint32_t dst[AD];   // LDS byte offset inside an A slot (uniform)

  __device__ __forceinline__ explicit AMap(const WideArgs &c) {
    const int lane = c.lane;
#pragma unroll
    for (int d = 0; d < AD; ++d) {
      const int f = kHalf ? (c.w >> 1) : c.w * AD + d;
      const int half = kHalf ? (c.w & 1) : 0;
      const int q = f / MS, rg = f % MS;
      const int r = 16 * rg + 8 * half + ((kHalf ? (lane & 31) : lane) >> 2);
      const int rs = min(r, c.nrows - 1);
      const int gc = (lane & 3) ^ a_swizzle(r & 15);
      voff[d] = (uint32_t)(2 * ((int64_t)rs * c.lda + q * c.aps + gc * 8));
      dst[d] = uniform_u32((uint32_t)(L::kAOff + q * kAbuf + rg * 1024 + half * 512));
    }
  }
  // copy d of stage ka into A slot sa
  __device__ __forceinline__ void copy(const WideArgs &c, int d, int ka, int sa) const {
    const char *ab = uniform_ptr(c.abase + (size_t)ka * kArow);
    const uint32_t to = uniform_u32(c.lds0 + dst[d] + sa * L::kAStage);
    if constexpr (kHalf) {
      if constexpr (COH) dma16_lanes_coh(voff[d], ab, to, 0xFFFFFFFFull);
      else dma16_lanes(voff[d], ab, to, 0xFFFFFFFFull);
    } else {
      dma16_a<COH>(voff[d], ab, to);
    }
  }
};

// Decoded B registers of one stage: one MFMA B operand per strip.
typedef u32x4 BRegs[4];

// Per-stage context of one wave.
template <int EPI, int K, int MS, bool COH>
struct WideIter {
  using L = WideLds<EPI>;
  static constexpr int ND = HalfGeom<K>::kLoadDw, NN = HalfGeom<K>::kNormDw;
  static constexpr int U = 2 * MS;     // units per stage, two MFMAs each
  static constexpr int PPU = 16 / U;   // decode pairs per unit
  static constexpr int SEG = 64 * K;   // bytes of a strip's stage
  // A 64-lane trellis copy moves 16 bytes a lane: 16 lanes carry a strip's
  // stage for K <= 4 (4 strips a copy), 32 lanes otherwise (2 strips); a
  // strip's LDS slot is as wide as its lanes.
  static constexpr int LPS = (SEG <= 256) ? 16 : 32;  // lanes per strip
  static constexpr int SPD = 64 / LPS;                // strips per copy
  static constexpr int TDMA = 4 / SPD;                // trellis copies per wave and stage
  using AM = AMap<EPI, MS, COH>;
  static constexpr int AD = AM::AD;                   // A copies per wave and stage
  static constexpr int DMA = AD + TDMA;               // copies per wave and stage
  static constexpr int TSTR = 16 * LPS;               // LDS bytes of a strip's slot
  static constexpr uint64_t kStripLanes =
      (SEG == TSTR) ? ((1ull << LPS) - 1) : ((1ull << (SEG / 16)) - 1);
  static constexpr uint64_t kSegLanes =
      (LPS == 32) ? (kStripLanes | (kStripLanes << 32))
                  : (kStripLanes | (kStripLanes << 16) | (kStripLanes << 32) | (kStripLanes << 48));

  const WideArgs &c;
  const AM am;
  const char *smem;
  const char *tens;
  uint32_t shift, mask;
  uint32_t tvoff[TDMA];
  uint32_t traddr[ND];
  uint32_t afrag;
  uint32_t tdst;  // LDS address of this wave's T region (uniform)

  // one stage's working set
  uint32_t raw[4][ND];
  uint32_t N[NN];
  f16x8 af[MS];
  uint32_t ar;  // A fragment address in the current slot

  __device__ __forceinline__ WideIter(const WideArgs &c_, const char *smem_, const char *tens_,
                                      int nt0, int ktiles)
      : c(c_), am(c_), smem(smem_), tens(tens_) {
    const int lane = c.lane, g = lane >> 4, n = lane & 15;
    const int sl = lane % LPS;
#pragma unroll
    for (int d = 0; d < TDMA; ++d) {
      const int ns = SPD * d + lane / LPS;
      tvoff[d] = (uint32_t)((nt0 + ns) * ktiles * 32 * K + 16 * min(sl, SEG / 16 - 1));
    }
    tdst = uniform_u32(c.lds0 + L::kTOff + c.w * kTwave);
    const HalfWindow<K> hw(lane);
    shift = hw.shift;
#pragma unroll
    for (int j = 0; j < ND; ++j) traddr[j] = (uint32_t)(L::kTOff + c.w * kTwave) + hw.off[j];
    afrag = (uint32_t)(L::kAOff + c.pj * kAbuf + n * kArow + ((g ^ a_swizzle(n)) * 16));
    mask = codebook_mask();
  }

  // DMA d (0 .. DMA-1) of stages (ka, kt) into slots (sa, st): A chunks
  // first, then the trellis (SPD strips per DMA).
  __device__ __forceinline__ void dma(int d, int ka, int kt, int sa, int st) const {
    if (d < AD) {
      am.copy(c, d, ka, sa);
    } else {
      const int td = d - AD;
      const char *tb = uniform_ptr(tens + (size_t)kt * 2 * 32 * K);
      const uint32_t dst = uniform_u32(tdst + st * kTstage + td * SPD * TSTR);
      if constexpr (SEG == TSTR) dma16(tvoff[td], tb, dst);
      else dma16_lanes(tvoff[td], tb, dst, kSegLanes);
    }
  }

  __device__ __forceinline__ void read_raw(int st) {
    const uint32_t off = (uint32_t)(st * kTstage);
#pragma unroll
    for (int ns = 0; ns < 4; ++ns)
#pragma unroll
      for (int j = 0; j < ND; ++j)
        raw[ns][j] = *(const uint32_t *)(smem + traddr[j] + off + ns * TSTR);
  }

  template <int Q>
  __device__ __forceinline__ void decode_pair(BRegs &bn) {
    constexpr int ns = Q / 4, r = Q % 4;
    bn[ns][r] = half_column_reg<K, r>(raw[ns], shift, N, mask);
  }
  template <int... Qs>
  __device__ __forceinline__ void decode_seq(BRegs &bn, std::integer_sequence<int, Qs...>) {
    (decode_pair<Qs>(bn), ...);
  }
  template <int Q0, int CNT>
  __device__ __forceinline__ void decode_range(BRegs &bn) {
    decode_off<Q0>(bn, std::make_integer_sequence<int, CNT>{});
  }
  template <int Q0, int... Is>
  __device__ __forceinline__ void decode_off(BRegs &bn, std::integer_sequence<int, Is...>) {
    (decode_pair<Q0 + Is>(bn), ...);
  }

  __device__ __forceinline__ void load_af(int slot_ms, int ms) {
    af[slot_ms] = *(const f16x8 *)(smem + ar + ms * 16 * kArow);
  }

  // Unit u: its DMAs, PPU decode pairs, two MFMAs.
  template <int u>
  __device__ __forceinline__ void unit(const BRegs &bc, BRegs &bn, f32x4 (&pacc)[8][4], int ka,
                                       int kt, int sa_w, int st_w) {
    constexpr int ms = u / 2, ns0 = (u & 1) * 2;
#pragma unroll
    for (int d = 0; d < DMA; ++d)
      if ((d * U) / DMA == u) dma(d, ka, kt, sa_w, st_w);
    decode_range<u * PPU, PPU>(bn);
    pacc[ms][ns0] = mfma16x16x32(af[ms], __builtin_bit_cast(f16x8, bc[ns0]), pacc[ms][ns0]);
    pacc[ms][ns0 + 1] =
        mfma16x16x32(af[ms], __builtin_bit_cast(f16x8, bc[ns0 + 1]), pacc[ms][ns0 + 1]);
    __builtin_amdgcn_sched_barrier(0);
  }
  template <int... Us>
  __device__ __forceinline__ void units(const BRegs &bc, BRegs &bn, f32x4 (&pacc)[8][4], int ka,
                                        int kt, int sa_w, int st_w,
                                        std::integer_sequence<int, Us...>) {
    (unit<Us>(bc, bn, pacc, ka, kt, sa_w, st_w), ...);
  }

  // Stage ks: A[ks] in A slot ks % 3 (= sa), T[ks+1] in T slot (ks+1) % 4.
  __device__ __forceinline__ void iteration(int ks, int sa, const BRegs &bc, BRegs &bn,
                                            f32x4 (&pacc)[8][4]) {
    const int last = c.nks - 1;
    wait_vmcnt<DMA + TDMA>();
    __syncthreads();
    ar = afrag + (uint32_t)(sa * L::kAStage);
    // every A fragment of the stage at once: under load an LDS read takes a
    // few hundred cycles, so only the first MFMA waits for one
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) load_af(ms, ms);
    read_raw((ks + 1) & 3);
    const int sa_w = (sa == 0) ? 2 : sa - 1;  // (ks + 2) % 3
    units(bc, bn, pacc, min(ks + 2, last), min(ks + 4, last), sa_w, ks & 3,
          std::make_integer_sequence<int, U>{});
  }

  // One projection stage over all k: pacc += A x W.
  __device__ __forceinline__ void run(f32x4 (&pacc)[8][4]) {
    const int nks = c.nks, last = nks - 1;
    BRegs b0, b1;
    __syncthreads();  // the LDS rings are free
    // prologue, in the order of the steady state: T[0], T[1], A[0] T[2],
    // A[1] T[3]
#pragma unroll
    for (int d = AD; d < DMA; ++d) dma(d, 0, 0, 0, 0);
#pragma unroll
    for (int d = AD; d < DMA; ++d) dma(d, 0, min(1, last), 0, 1);
#pragma unroll
    for (int d = 0; d < AD; ++d) dma(d, 0, 0, 0, 0);
#pragma unroll
    for (int d = AD; d < DMA; ++d) dma(d, 0, min(2, last), 0, 2);
#pragma unroll
    for (int d = 0; d < AD; ++d) dma(d, min(1, last), 0, 1, 0);
#pragma unroll
    for (int d = AD; d < DMA; ++d) dma(d, 0, min(3, last), 0, 3);
    wait_vmcnt<3 * TDMA + 2 * AD>();  // T[0] (this wave's own copy)
    read_raw(0);
    decode_seq(b0, std::make_integer_sequence<int, 16>{});
    int sa = 0;
    for (int ks = 0; ks < nks; ks += 2) {  // nks is a multiple of 4
      iteration(ks, sa, b0, b1, pacc);
      sa = (sa == 2) ? 0 : sa + 1;
      iteration(ks + 1, sa, b1, b0, pacc);
      sa = (sa == 2) ? 0 : sa + 1;
    }
    wait_vmcnt<0>();  // no DMA may land after the LDS is reused
  }
};

// A wave with no work for this stage still copies its share of A and takes
// part in the barrier cadence of its workgroup (1 + nks barriers).
template <int EPI, bool COH, int MS>
__device__ __forceinline__ void wide_idle_stage(const WideArgs &c) {
  using AM = AMap<EPI, MS, COH>;
  const AM am(c);
  const int nks = c.nks, last = nks - 1;
  auto issue = [&](int ka, int sa) {
#pragma unroll
    for (int d = 0; d < AM::AD; ++d) am.copy(c, d, ka, sa);
  };
  __syncthreads();
  issue(0, 0);
  issue(min(1, last), 1);
  int sa = 0;
  for (int ks = 0; ks < nks; ++ks) {
    wait_vmcnt<AM::AD>();
    __syncthreads();
    issue(min(ks + 2, last), (sa == 0) ? 2 : sa - 1);
    sa = (sa == 2) ? 0 : sa + 1;
  }
  wait_vmcnt<0>();
}

template <int EPI, bool COH>
__device__ __forceinline__ void wide_idle_rows(const WideArgs &c, int msub) {
  if (msub <= 2) wide_idle_stage<EPI, COH, 2>(c);
  else if (msub <= 4) wide_idle_stage<EPI, COH, 4>(c);
  else wide_idle_stage<EPI, COH, 8>(c);
}

template <int EPI, int K, bool COH>
__device__ __forceinline__ void wide_stage_rows(const WideArgs &c, char *smem, const char *tens,
                                                int nt0, int ktiles, int msub,
                                                f32x4 (&pacc)[8][4]) {
  if (msub <= 2) {
    WideIter<EPI, K, 2, COH> it(c, smem, tens, nt0, ktiles);
    it.run(pacc);
  } else if (msub <= 4) {
    WideIter<EPI, K, 4, COH> it(c, smem, tens, nt0, ktiles);
    it.run(pacc);
  } else {
    WideIter<EPI, K, 8, COH> it(c, smem, tens, nt0, ktiles);
    it.run(pacc);
  }
}

// One work item: rows of tile `bx` times 256-column block `by`.
// COH (within one launch, for the pass kernel): the down projection reads its
// A rows with device-coherent loads, the gate/up epilogue writes a~ with
// device-coherent stores. Returns false when the tile does not exist.
template <int EPI, bool MULTI, bool COH = false>
__device__ __forceinline__ bool wide_item(const GemmParams &p, char *smem, int bx, int by) {
  using L = WideLds<EPI>;
  constexpr int NPROJ = L::NPROJ;
  constexpr bool kCohLoad = COH && EPI == EPI_DOWN;
  constexpr bool kCohStore = COH && EPI == EPI_GATEUP;

  WideArgs c;
  if (!tile_of_block(p, kWBM, bx, c.e, c.row0, c.nrows)) return false;
  c.nb = by;
  c.lane = threadIdx.x & 63;
  c.w = wave_id();
  c.pj = (EPI == EPI_GATEUP) ? (c.w >> 1) : 0;
  c.colbase = (EPI == EPI_GATEUP) ? c.nb * 128 : c.nb * 256;
  c.nks = p.in_f >> 5;
  c.lds0 = (uint32_t)(uintptr_t)smem;
  const int w = c.w, lane = c.lane, g = lane >> 4, n = lane & 15;
  const int colw = c.colbase + ((EPI == EPI_GATEUP) ? 64 * (w & 1) : 64 * w);
  const bool col_ok = colw < p.out_f;
  const int nt0 = colw >> 4;
  const int ktiles = p.in_f >> 4;
  const int msub = (c.nrows + 15) >> 4;

  // the A rows of the tile (the copies per stage: AMap)
  c.abase = (const char *)(p.A + (int64_t)c.row0 * p.lda);
  c.lda = p.lda;
  c.aps = p.a_proj_stride;

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
      wide_idle_rows<EPI, kCohLoad>(c, msub);
    } else {
      switch (K) {
        case 2: wide_stage_rows<EPI, 2, kCohLoad>(c, smem, tens, nt0, ktiles, msub, pacc); break;
        case 3: wide_stage_rows<EPI, 3, kCohLoad>(c, smem, tens, nt0, ktiles, msub, pacc); break;
        case 4: wide_stage_rows<EPI, 4, kCohLoad>(c, smem, tens, nt0, ktiles, msub, pacc); break;
        case 5: wide_stage_rows<EPI, 5, kCohLoad>(c, smem, tens, nt0, ktiles, msub, pacc); break;
        case 6: wide_stage_rows<EPI, 6, kCohLoad>(c, smem, tens, nt0, ktiles, msub, pacc); break;
        case 7: wide_stage_rows<EPI, 7, kCohLoad>(c, smem, tens, nt0, ktiles, msub, pacc); break;
        default: wide_stage_rows<EPI, 8, kCohLoad>(c, smem, tens, nt0, ktiles, msub, pacc); break;
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

  // ---- epilogue: accumulators -> LDS tile -> shared epilogue, in two
  // rounds of 64 rows (row blocks 0-3, then 4-7)
  float *T = (float *)smem;
  const int cw = (EPI == EPI_GATEUP) ? 64 * (w & 1) : 64 * w;  // column of the wave in T
  const int nblk = (EPI == EPI_GATEUP) ? 1 : min(2, (p.out_f - c.colbase) / 128);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int hrows = min(L::kHalf, c.nrows - L::kHalf * half);
    if (hrows <= 0) break;  // uniform
    __syncthreads();
#pragma unroll
    for (int ms = 4 * half; ms < 4 * half + 4; ++ms)
#pragma unroll
      for (int ns = 0; ns < 4; ++ns)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          T[c.pj * (L::kHalf * L::kLd) + (16 * (ms - 4 * half) + 4 * g + r) * L::kLd + cw +
            16 * ns + n] = fin[ms][ns][r];
    __syncthreads();
    epilogue<EPI, kCohStore>(p, T, L::kLd, L::kHalf * L::kLd, c.e, c.row0 + L::kHalf * half,
                             hrows, c.colbase, nblk);
  }
  return true;
}

// One workgroup per (tile, 256-column block) on a 1-D grid of groups of 8
// tiles x nb column blocks. Workgroups are dealt to the 8 XCDs round-robin by
// linear id, so tile 8 G + (id % 8) keeps all its column blocks on one XCD
// (sharing its L2 copy of the tile's A rows), and the dispatch order walks
// the tiles front to back: tiles past the device's tile count (the launch is
// sized for the worst case) come last and exit at once.
template <int EPI, bool MULTI>
__global__ void __launch_bounds__(256, MULTI ? 1 : 2) gemm_wide_kernel(GemmParams p, int nb) {
  __shared__ __attribute__((aligned(16))) char smem[WideLds<EPI>::kBytes];
  const int id = blockIdx.x, per = 8 * nb;
  const int grp = id / per, r = id - grp * per;
  wide_item<EPI, MULTI>(p, smem, 8 * grp + (r & 7), r >> 3);
}

// One pass of the routed experts in one launch (calls with a single pass;
// several passes run pipelined, gemm_wide_pipe_kernel). Items, in dispatch
// order: gate/up (tile x 128-column block of the intermediate, ids [0, g1)),
// then down (tile x 256-column block of the hidden size, tiles in reverse
// plan order), in the XCD-aware order of gemm_wide_kernel. A down item needs
// only the a~ rows of its own tile, which that tile's nb_gu gate/up items
// write with device-coherent stores; each waits until its stores are
// complete and counts itself in q[tile]. The down item waits for q[tile] ==
// nb_gu and reads a~ with device-coherent loads, so the down work of finished
// tiles runs while slower tiles are still in gate/up. The plan puts heavy
// tiles first, so the first down items dispatched belong to tiles that finish
// early. Workgroups are dispatched in id order on every XCD and gate/up items
// never wait, so every item a down item waits on is resident or finished and
// the wait ends; it is bounded anyway (a timeout is counted in ctrl[2]).
// (Handing down work out in the order tiles finish, through a claim counter,
// measured slower.) q holds `slots` ints, zero at launch.
template <bool MULTI>
__global__ void __launch_bounds__(256, MULTI ? 1 : 2)
    gemm_wide_pass_kernel(GemmParams gu, GemmParams dn, int nb_gu, int nb_dn, int g1, int slots,
                          int32_t *q) {
  constexpr int kBytes = WideLds<EPI_GATEUP>::kBytes > WideLds<EPI_DOWN>::kBytes
                             ? WideLds<EPI_GATEUP>::kBytes
                             : WideLds<EPI_DOWN>::kBytes;
  __shared__ __attribute__((aligned(16))) char smem[kBytes];
  int id = blockIdx.x;
  if (id < g1) {
    const int per = 8 * nb_gu, grp = id / per, r = id - grp * per;
    const int bx = 8 * grp + (r & 7);
    if (bx >= slots || !wide_item<EPI_GATEUP, MULTI, true>(gu, smem, bx, r >> 3)) return;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's a~ stores
    __syncthreads();                                     // ... and every wave's
    if (threadIdx.x == 0)
      __hip_atomic_fetch_add(q + bx, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  id -= g1;
  const int per = 8 * nb_dn, grp = id / per, r = id - grp * per;
  const int ntiles = min(uload_i32(dn.plan_ntiles), slots);
  const int bx = ntiles - 1 - (8 * grp + (r & 7));
  if (bx < 0) return;
  if (threadIdx.x == 0) {
    int spins = 0;
    while (__hip_atomic_load(q + bx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < nb_gu) {
      if (++spins > (1 << 22)) {
        atomicAdd(dn.ctrl + 2, 1);
        break;
      }
      __builtin_amdgcn_s_sleep(4);
    }
  }
  __syncthreads();
  wide_item<EPI_DOWN, MULTI, true>(dn, smem, bx, r >> 3);
}

hipError_t launch_gemm_wide_pass(const GemmParams &gu, const GemmParams &dn, int tiles,
                                 int slots, int nb_gu, int nb_dn, int32_t *q, hipStream_t s) {
  if (tiles <= 0 || nb_gu <= 0 || nb_dn <= 0) return hipSuccess;
  const bool multi = gu.proj[0].num_stages > 1 || gu.proj[1].num_stages > 1 ||
                     dn.proj[0].num_stages > 1;
  const int t8 = (tiles + 7) / 8 * 8;
  const int g1 = t8 * nb_gu;
  const dim3 grid((unsigned)(g1 + t8 * nb_dn));
  if (multi)
    hipLaunchKernelGGL(gemm_wide_pass_kernel<true>, grid, dim3(256), 0, s, gu, dn, nb_gu, nb_dn,
                       g1, slots, q);
  else
    hipLaunchKernelGGL(gemm_wide_pass_kernel<false>, grid, dim3(256), 0, s, gu, dn, nb_gu, nb_dn,
                       g1, slots, q);
  return hipGetLastError();
}

// Routed experts over several passes, software-pipelined across launches:
// launch k holds the gate/up items of pass k, the down items of pass k - 1,
// the rotation of pass k + 1 and the combine of pass k - 2. x~, a~ and d have
// two buffers each (by pass parity), so within one launch no item reads what
// another writes (gate/up reads x~[k] and writes a~[k]; down reads a~[k-1]
// and writes d[k-1]; the rotation writes x~[k+1]; the combine reads d[k-2] =
// d[k]), and every value an item reads was written by an earlier launch. No
// item waits for another: the launch fills the machine with whatever work is
// left of four passes, instead of idling through one pass's stragglers.
// Items, in dispatch order (longest first): gate/up (tile x 128-column
// block, heavy tiles first), down (tile x 256-column block), rotation
// (64 (position, 128-block) units, one per lane quad), combine (one row;
// rows without a pair in the unit return at once).
constexpr int kRotUnitsPerItem = 64;

template <bool MULTI>
__global__ void __launch_bounds__(256, MULTI ? 1 : 2)
    gemm_wide_pipe_kernel(GemmParams gu, GemmParams dn, RotParams rn, CombineParams cb,
                          int nb_gu, int nb_dn, int g1, int g2, int g3) {
  constexpr int kBytes = WideLds<EPI_GATEUP>::kBytes > WideLds<EPI_DOWN>::kBytes
                             ? WideLds<EPI_GATEUP>::kBytes
                             : WideLds<EPI_DOWN>::kBytes;
  __shared__ __attribute__((aligned(16))) char smem[kBytes];
  int id = blockIdx.x;
  if (id < g1) {
    const int per = 8 * nb_gu, grp = id / per, r = id - grp * per;
    wide_item<EPI_GATEUP, MULTI>(gu, smem, 8 * grp + (r & 7), r >> 3);
    return;
  }
  id -= g1;
  if (id < g2) {
    const int per = 8 * nb_dn, grp = id / per, r = id - grp * per;
    wide_item<EPI_DOWN, MULTI>(dn, smem, 8 * grp + (r & 7), r >> 3);
    return;
  }
  id -= g2;
  if (id < g3) {
    rotate_unit(rn, (int64_t)id * kRotUnitsPerItem + (threadIdx.x >> 2), threadIdx.x & 3);
    return;
  }
  combine_row(cb, id - g3);
}

hipError_t launch_gemm_wide_pipe(const GemmParams &gu, int tiles_gu, const GemmParams &dn,
                                 int tiles_dn, const RotParams &rn, const CombineParams &cb,
                                 int rows_cb, int nb_gu, int nb_dn, hipStream_t s) {
  if (rn.nitems > 0 && (rn.nproj < 1 || rn.nproj > 2)) return hipErrorInvalidValue;
  const bool multi = (tiles_gu > 0 && (gu.proj[0].num_stages > 1 || gu.proj[1].num_stages > 1)) ||
                     (tiles_dn > 0 && dn.proj[0].num_stages > 1);
  const int g1 = tiles_gu > 0 ? (tiles_gu + 7) / 8 * 8 * nb_gu : 0;
  const int g2 = tiles_dn > 0 ? (tiles_dn + 7) / 8 * 8 * nb_dn : 0;
  const int64_t units = rn.nitems > 0 ? (int64_t)rn.nitems * (rn.H >> 7) : 0;
  const int g3 = (int)((units + kRotUnitsPerItem - 1) / kRotUnitsPerItem);
  const int g4 = rows_cb > 0 ? rows_cb : 0;
  const int64_t total = (int64_t)g1 + g2 + g3 + g4;
  if (total <= 0) return hipSuccess;
  const dim3 grid((unsigned)total);
  if (multi)
    hipLaunchKernelGGL(gemm_wide_pipe_kernel<true>, grid, dim3(256), 0, s, gu, dn, rn, cb, nb_gu,
                       nb_dn, g1, g2, g3);
  else
    hipLaunchKernelGGL(gemm_wide_pipe_kernel<false>, grid, dim3(256), 0, s, gu, dn, rn, cb, nb_gu,
                       nb_dn, g1, g2, g3);
  return hipGetLastError();
}

hipError_t launch_gemm_wide(int epi, const GemmParams &p, int tiles, int nblocks, hipStream_t s) {
  if (tiles <= 0 || nblocks <= 0) return hipSuccess;
  const bool multi = p.proj[0].num_stages > 1 || (epi == EPI_GATEUP && p.proj[1].num_stages > 1);
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

}  // namespace exl3
