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
// and output scaling; per-stage tables in which a stage may be absent).
//
// Arithmetic contract (makes a row's bytes independent of the other rows,
// the tile it lands in, the capacity and the chunking):
//   P_t[row][n] = v_mfma_f32_16x16x32_f16 chain over ascending 32-input
//                 k-steps (each two whole trellis tiles along k), from 0
//   acc         = fmaf(s_t, P_t, acc) over stages in order, from acc = 0,
//                 stages with s_t == 0 skipped
//   epilogue    = fixed-order fp32 FWHT per 128-block, then per-element
//                 scalings, identical code for every tile shape.

#include <atomic>
#include <algorithm>
#include <utility>

#include "gemm_shared.hpp"

namespace exl3 {

// Narrow tiles (decode-size work): a work item is a tile of at most 16 rows
// of one expert times 64 output columns of one projection, one workgroup of
// 4 waves. Wave w streams strip 4 cg + w (16 columns) over the whole input.
// Waves never wait for each other until the end, so there is one 64-column
// work item per few CUs' worth of waves even at one routed row.
//
// Trellis: each wave copies its strip global->LDS by DMA in blocks of 128
// inputs (8 tiles, 256K bytes) into a ring of kNRing slots of its own, three
// blocks ahead of the one it decodes. A (rotated rows, L2-resident) goes
// straight to registers two blocks ahead: vector loads complete in order, so
// the wait for A[b] also waits for every trellis block issued before it, and
// A's lead bounds the trellis lead. (Deeper rings measured slower: the
// kernel is bound by issue and VALU more than by memory latency, and four
// waves per SIMD beat a deeper ring per wave.) Every wave issues the same loads every
// block (past the end it re-reads the last block), so each wait is an exact
// vmcnt.
//
// MFMA k-step s of block b covers inputs 128 b + 32 s .. +31, i.e. trellis
// tiles 8 b + 2 s and 8 b + 2 s + 1 along k. Lane (g, n) supplies states
// 8 (g & 1) .. +7 of column n of tile 8 b + 2 s + (g >> 1) (a half column)
// and the matching 8 rotated inputs. The 128-row kernel uses the same
// k-steps, so both run one MFMA chain per output.
//
// The pre-rotation fp32 sums go to workspace scratch; the last of the work
// items of a 128-column block (an atomic count: 2, or 4 for gate + up) runs
// the shared epilogue on the whole block.
constexpr int kNRing = 4;
constexpr int kNSlot = 2048;  // bytes: one block at K <= 8
// LDS offset of the staged epilogue vectors (after the 2 x 16 x 132 fp32
// accumulator tile of the epilogue; the ring is free by then)
constexpr int kEpiVecOff = 2 * 16 * 132 * 4;

template <int K>
struct StreamGeom {
  static constexpr int kBlk = 256 * K;                        // bytes per block
  static constexpr int kDma = (kBlk + 1023) / 1024;           // 1 or 2
  static constexpr int kLanes1 = (kBlk > 1024) ? (kBlk - 1024) / 16 : 0;
  static constexpr uint64_t kMask0 = (kBlk >= 1024) ? ~0ull : ((1ull << (kBlk / 16)) - 1);
  static constexpr uint64_t kMask1 = (kLanes1 >= 64) ? ~0ull : ((1ull << kLanes1) - 1);
};

// Every asm block below that reads an SGPR operand (a base address) in a
// vector memory instruction first spends five wait states (its own SALU
// instructions plus s_nop): the compiler may write that SGPR with a VALU
// instruction (v_readfirstlane, or v_readlane reloading a spilled SGPR) just
// before the block, CDNA requires five wait states between such a write and
// a vector memory read of the SGPR, and the compiler's hazard check does not
// look inside inline asm. Without them the load can use the register's
// previous contents as its address.

// 16-byte-per-lane global->LDS copy (lanes in `lanes`): lane L reads
// sbase + voff and writes LDS byte m0 + 16 L.
__device__ __forceinline__ void sdma16(uint32_t voff, const void *sbase, uint32_t lds_base,
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

template <int N>
__device__ __forceinline__ void swait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// The 4 A fragments of one block (16 bytes each, 64 bytes apart) into
// registers, on the lanes in `lanes` only (rows past the tile's end are never
// loaded: their MFMA output rows are discarded). Invisible to the compiler's
// wait counting: the chain's own vmcnt waits cover it (see a_wait). COH:
// device-coherent loads (sc1), for rows another workgroup of the same launch
// wrote.
template <bool COH>
__device__ __forceinline__ void aload_block(u32x4 &a0, u32x4 &a1, u32x4 &a2, u32x4 &a3,
                                            uint32_t voff, const char *sbase, uint64_t lanes) {
  uint64_t saved;
  if constexpr (COH) {
    asm volatile(
        "s_mov_b64 %4, exec\n\t"
        "s_and_b64 exec, exec, %7\n\t"
        "s_nop 2\n\t"
        "global_load_dwordx4 %0, %5, %6 offset:0 sc1\n\t"
        "global_load_dwordx4 %1, %5, %6 offset:64 sc1\n\t"
        "global_load_dwordx4 %2, %5, %6 offset:128 sc1\n\t"
        "global_load_dwordx4 %3, %5, %6 offset:192 sc1\n\t"
        "s_mov_b64 exec, %4"
        : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3), "=&s"(saved)
        : "v"(voff), "s"(sbase), "s"(lanes)
        : "memory", "scc");
  } else {
    asm volatile(
        "s_mov_b64 %4, exec\n\t"
        "s_and_b64 exec, exec, %7\n\t"
        "s_nop 2\n\t"
        "global_load_dwordx4 %0, %5, %6 offset:0\n\t"
        "global_load_dwordx4 %1, %5, %6 offset:64\n\t"
        "global_load_dwordx4 %2, %5, %6 offset:128\n\t"
        "global_load_dwordx4 %3, %5, %6 offset:192\n\t"
        "s_mov_b64 exec, %4"
        : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3), "=&s"(saved)
        : "v"(voff), "s"(sbase), "s"(lanes)
        : "memory", "scc");
  }
}

// Wait until at most N vector loads are outstanding; the A registers of the
// block about to be used are tied to the wait so no use moves above it.
template <int N>
__device__ __forceinline__ void a_wait(u32x4 &a0, u32x4 &a1, u32x4 &a2, u32x4 &a3) {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%4)" : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3) : "n"(N) : "memory");
}

// One device-coherent dword load (sc1), invisible to the compiler's wait
// counting like aload_block: a readiness count another workgroup of the same
// launch writes. Every lane loads the same (uniform) address.
__device__ __forceinline__ void flag_load(uint32_t &v, const char *sbase) {
  asm volatile("s_nop 4\n\tglobal_load_dword %0, %1, %2 sc1"
               : "=&v"(v)
               : "v"(0u), "s"(sbase)
               : "memory");
}

// a_wait that also holds the block's readiness count.
template <int N>
__device__ __forceinline__ void a_wait_f(u32x4 &a0, u32x4 &a1, u32x4 &a2, u32x4 &a3,
                                         uint32_t &f) {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%5)"
               : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(f)
               : "n"(N)
               : "memory");
}

__device__ __forceinline__ const char *sgpr_ptr(const void *ptr) {
  const uint64_t b = (uint64_t)(uintptr_t)ptr;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  return (const char *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Wait until the n counts in `flags` are set: lane j of the wave reads
// count j (64 at a time, one load for all of them) and the wave votes;
// bounded, a give-up counted in ctrl[2].
__device__ __forceinline__ void wait_all_set(const int32_t *flags, int n, int32_t *ctrl) {
  const int lane = threadIdx.x & 63;
  int spins = 0;
  for (int j0 = 0; j0 < n; j0 += 64) {
    const int j = j0 + lane;
    for (;;) {
      const int v =
          j < n ? __hip_atomic_load(flags + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 1;
      if (__all(v >= 1)) break;
      if (++spins > (1 << 22)) {
        if (lane == 0) atomicAdd(ctrl + 2, 1);
        return;
      }
      __builtin_amdgcn_s_sleep(8);
    }
  }
}

// P = MFMA chain of one stage over all inputs for this wave's strip.
constexpr int kNADist = kNRing - 2;  // A blocks in flight ahead of the one in use

// WA (the single-pass launch's down items): A block b is the a~ block b of
// the tile, written by a gate/up item of the same launch, and is read only
// once aflags[b] is set. The count of block b + kNADist is loaded together
// with A[b] (kNADist blocks before its A is issued) and checked when A[b]
// has arrived, so the chain starts as soon as its first blocks are ready
// and meets the later ones as they come.
template <int K, bool COH, bool WA>
struct StreamChain {
  using G = StreamGeom<K>;
  static constexpr int ND = HalfGeom<K>::kLoadDw, NN = HalfGeom<K>::kNormDw;
  static constexpr int TD = Geom<K>::kTileDw;
  static constexpr int kF = WA ? 1 : 0;          // readiness loads per block
  static constexpr int kIssue = kF + 4 + G::kDma;  // loads per block: flag, A, then T
  // outstanding loads issued after A[b] when A[b] is needed
  static constexpr int kAWait = G::kDma + (kNADist - 1) * kIssue;
  static_assert(kNADist + 1 == kNRing - 1, "the A lead equals the trellis lead");

  const char *strip;  // uniform: the strip's trellis
  const char *ring;   // this wave's LDS ring
  uint32_t ring_lds;  // its LDS address (uniform)
  const char *abase;  // uniform: A rows of the tile
  uint32_t avoff;     // lane's A byte offset (row, k-group)
  uint64_t alanes;    // lanes whose A row is inside the tile
  uint32_t tvoff;     // lane's byte offset inside a block
  uint32_t traddr[ND];
  uint32_t shift, mask;
  int nblk;
  u32x4 a[kNADist + 1][4];  // A of blocks b .. b + kNADist (ring by b % (kNADist + 1))
  const int32_t *aflags;    // WA: readiness counts of the tile's A blocks
  int32_t *ctrl;            // WA: [2] counts a wait that gave up
  uint32_t fl[kNADist + 1]; // WA: count of A block b + kNADist, with A[b]

  __device__ __forceinline__ void load_a(int ba, int aslot) {
    const char *src = sgpr_ptr(abase + (size_t)ba * 256);
    aload_block<COH>(a[aslot][0], a[aslot][1], a[aslot][2], a[aslot][3], avoff, src, alanes);
  }
  __device__ __forceinline__ void load_flag(int bf, int fslot) {
    if constexpr (WA) flag_load(fl[fslot], sgpr_ptr(aflags + bf));
  }
  __device__ __forceinline__ void issue(int b, int aslot) {
    const int last = nblk - 1;
    load_flag(min(b + 2 * kNADist, last), aslot);
    load_a(min(b + kNADist, last), aslot);
    issue_t(min(b + kNRing - 1, last));
  }
  // WA: spin until A block ba is ready (all loads drained first, so the
  // exact counts of later waits still hold); bounded, a give-up counted.
  __device__ __forceinline__ void wait_ready(int ba) {
    swait_vmcnt<0>();
    int spins = 0;
    while (__builtin_amdgcn_readfirstlane(
               (int)__hip_atomic_load(aflags + ba, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) < 1) {
      if (++spins > (1 << 22)) {
        if ((threadIdx.x & 63) == 0) atomicAdd(ctrl + 2, 1);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __device__ __forceinline__ void issue_t(int bt) {
    const char *src = sgpr_ptr(strip + (size_t)bt * G::kBlk);
    const uint32_t dst = (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)(ring_lds + (uint32_t)((bt % kNRing) * kNSlot)));
    sdma16(tvoff, src, dst, G::kMask0);
    if constexpr (G::kDma > 1) sdma16(tvoff + 1024, src, dst + 1024, G::kMask1);
  }

  __device__ __forceinline__ void compute(int b, int aslot, f32x4 &acc) {
    const uint32_t base = (uint32_t)((b % kNRing) * kNSlot);
    // the block's trellis words first (one LDS wait), then decode + MFMA
    uint32_t raw[4][ND];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int j = 0; j < ND; ++j)
        raw[s][j] = *(const uint32_t *)(ring + base + traddr[j] + s * 2 * TD * 4);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 w = decode_half<K>(raw[s], shift, mask);
      acc = mfma16x16x32(__builtin_bit_cast(f16x8, a[aslot][s]), __builtin_bit_cast(f16x8, w), acc);
    }
  }

  // Block b: wait for A[b] (issued kNADist blocks earlier after its group's
  // readiness load; T[b] was issued before it), check that the next A block
  // is ready (WA), issue A[b + kNADist] and T[b + kNRing - 1], compute.
  template <int AS>
  __device__ __forceinline__ void block(int b, f32x4 &acc) {
    if constexpr (WA) {
      a_wait_f<kAWait>(a[AS][0], a[AS][1], a[AS][2], a[AS][3], fl[AS]);
      const int nb = min(b + kNADist, nblk - 1);
      if (__builtin_amdgcn_readfirstlane((int)fl[AS]) < 1) wait_ready(nb);
    } else {
      a_wait<kAWait>(a[AS][0], a[AS][1], a[AS][2], a[AS][3]);
    }
    issue(b, (AS + kNADist) % (kNADist + 1));
    compute(b, AS, acc);
  }

  // blocks b .. b + kNADist (A ring slots 0 .. kNADist), those < nblk
  template <int... Is>
  __device__ __forceinline__ void blocks(int b, f32x4 &acc, std::integer_sequence<int, Is...>) {
    ((b + Is < nblk ? block<Is>(b + Is, acc) : void()), ...);
  }

  __device__ __forceinline__ f32x4 run() {
    const int last = nblk - 1;
    if constexpr (WA) {  // the first blocks' A must be ready before it is loaded
      swait_vmcnt<0>();
      wait_all_set(aflags, min(kNADist, nblk), ctrl);
    }
    // prologue in steady-state order: T[0], then (count of A[j + kNADist])
    // A[j] T[j + 1] for j = 0 .. kNADist - 1
    issue_t(0);
#pragma unroll
    for (int j = 0; j < kNADist; ++j) {
      load_flag(min(j + kNADist, last), j);
      load_a(min(j, last), j);
      issue_t(min(j + 1, last));
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int b = 0; b < nblk; b += kNADist + 1)
      blocks(b, acc, std::make_integer_sequence<int, kNADist + 1>{});
    // no DMA may land after the ring is reused, and no load after its
    // register is given to something else
    static_assert(kNADist == 2, "the drain below names every A and count register");
    if constexpr (WA)
      asm volatile("s_waitcnt vmcnt(0)"
                   : "+v"(a[0][0]), "+v"(a[0][1]), "+v"(a[0][2]), "+v"(a[0][3]), "+v"(a[1][0]),
                     "+v"(a[1][1]), "+v"(a[1][2]), "+v"(a[1][3]), "+v"(a[2][0]), "+v"(a[2][1]),
                     "+v"(a[2][2]), "+v"(a[2][3]), "+v"(fl[0]), "+v"(fl[1]), "+v"(fl[2])
                   :
                   : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)"
                   : "+v"(a[0][0]), "+v"(a[0][1]), "+v"(a[0][2]), "+v"(a[0][3]), "+v"(a[1][0]),
                     "+v"(a[1][1]), "+v"(a[1][2]), "+v"(a[1][3]), "+v"(a[2][0]), "+v"(a[2][1]),
                     "+v"(a[2][2]), "+v"(a[2][3])
                   :
                   : "memory");
    return acc;
  }
};

template <int K, bool COH, bool WA>
__device__ __forceinline__ f32x4 stream_chain(const char *strip, int in_f, const char *ring,
                                              const char *abase, uint32_t avoff, uint64_t alanes,
                                              int lane, const int32_t *aflags, int32_t *ctrl) {
  StreamChain<K, COH, WA> c;
  c.alanes = alanes;
  c.aflags = aflags;
  c.ctrl = ctrl;
  const int g = lane >> 4;
  c.strip = sgpr_ptr(strip);
  c.ring = ring;
  c.ring_lds = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)ring);
  c.abase = sgpr_ptr(abase);
  c.avoff = avoff + 16u * g;  // 8 halves per k-group
  c.tvoff = 16u * (uint32_t)lane;
  c.nblk = in_f >> 7;
  const HalfWindow<K> hw(lane);
  c.shift = hw.shift;
#pragma unroll
  for (int j = 0; j < StreamChain<K, COH, WA>::ND; ++j) c.traddr[j] = hw.off[j];
  c.mask = codebook_mask();
  return c.run();
}

// Stage loop of one projection for one wave: acc = sum fmaf(s_t, P_t, acc).
// aflags (WA): readiness counts of the tile's A blocks.
template <bool COH, bool WA = false>
__device__ __forceinline__ f32x4 stream_strip(const ProjDev &pd, int E, int e, int in_f, int nt,
                                              const char *ring, const char *abase,
                                              uint32_t avoff, uint64_t alanes, int lane,
                                              int32_t *ctrl, bool report,
                                              const int32_t *aflags = nullptr) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int t = 0; t < pd.num_stages; ++t) {
    const float s = uload_f32(pd.scale + t * E + e);
    if (s == 0.0f) continue;  // zero scale: the stage is skipped entirely
    const char *tens = (const char *)uload_ptr(pd.trellis + t * E + e);
    const int K = uload_i32(pd.bits + t * E + e);
    if (tens == nullptr || K < 2 || K > 8) {
      if (report && lane == 0) atomicAdd(ctrl + 1, 1);
      continue;
    }
    const char *strip = tens + (size_t)nt * (in_f / 16) * 32 * K;
    f32x4 q;
    switch (K) {
      case 2: q = stream_chain<2, COH, WA>(strip, in_f, ring, abase, avoff, alanes, lane, aflags, ctrl); break;
      case 3: q = stream_chain<3, COH, WA>(strip, in_f, ring, abase, avoff, alanes, lane, aflags, ctrl); break;
      case 4: q = stream_chain<4, COH, WA>(strip, in_f, ring, abase, avoff, alanes, lane, aflags, ctrl); break;
      case 5: q = stream_chain<5, COH, WA>(strip, in_f, ring, abase, avoff, alanes, lane, aflags, ctrl); break;
      case 6: q = stream_chain<6, COH, WA>(strip, in_f, ring, abase, avoff, alanes, lane, aflags, ctrl); break;
      case 7: q = stream_chain<7, COH, WA>(strip, in_f, ring, abase, avoff, alanes, lane, aflags, ctrl); break;
      default: q = stream_chain<8, COH, WA>(strip, in_f, ring, abase, avoff, alanes, lane, aflags, ctrl); break;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = fmaf(s, q[r], acc[r]);
  }
  return acc;
}

// DMA every block of this wave's strip, for every live stage, into its ring
// slots without waiting: the data is not used from LDS (the chain copies
// each block again) but is then held in the caches, so a work item that must
// wait for its inputs streams its trellis from HBM while it waits. The caller
// waits for these copies (vmcnt 0) before the chain reuses the ring.
__device__ __forceinline__ void prefetch_strip(const ProjDev &pd, int E, int e, int in_f, int nt,
                                               const char *ring, int lane) {
  const uint32_t ring_lds = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)ring);
  for (int t = 0; t < pd.num_stages; ++t) {
    const float sc = uload_f32(pd.scale + t * E + e);
    const char *tens = (const char *)uload_ptr(pd.trellis + t * E + e);
    const int K = uload_i32(pd.bits + t * E + e);
    if (sc == 0.0f || tens == nullptr || K < 2 || K > 8) continue;
    const int blk = 256 * K;  // bytes per 128-input block of the strip
    const char *strip = tens + (size_t)nt * (in_f / 16) * 32 * K;
    const int nblk = in_f >> 7;
    for (int b = 0; b < nblk; ++b) {
      const uint32_t dst = (uint32_t)__builtin_amdgcn_readfirstlane(
          (int)(ring_lds + (uint32_t)((b % kNRing) * kNSlot)));
      const char *src = sgpr_ptr(strip + (size_t)b * blk);
      // lanes past the block's end re-read its last 16 bytes (in bounds)
      for (int off = 0; off < blk; off += 1024)
        sdma16((uint32_t)min(16 * lane, blk - off - 16), src + off, dst + off, ~0ull);
    }
  }
}

// Ordered combine at the end of a fused down item (single pass, 16-row
// tiles). After its d block (128 columns `blk` of every row of the tile) is
// written and its stores are complete, the item counts that block once for
// the output row of each of its tile rows; the count that completes a
// (row, block) (one per kept pair of the row) makes this item sum d over the
// row's positions in ascending order, from 0 in fp32, and write that output
// block. The additions are those of the combine kernels, in the same order.
// s_tmp: 2 * kMaxTopk ints of free LDS; s_rows: kBM ints.
__device__ __forceinline__ void narrow_combine(const GemmParams &p, const NarrowFusedParams &f,
                                               int row0, int nrows, int blk, int *s_rows,
                                               int *s_tmp) {
  const int nhb = p.out_f >> 7;
  const int end = min(*f.total_valid, f.pairs);
  if ((int)threadIdx.x < nrows) {
    const int q = f.pair_of_pos[p.pass_base + row0 + threadIdx.x];
    int r = -1;
    if (q >= 0 && q < f.pairs) {
      r = q / f.topk;
      int kept = 0;
      for (int j = 0; j < f.topk; ++j) {
        const int pp = f.pos_of_pair[r * f.topk + j];
        kept += (pp >= 0 && pp < end) ? 1 : 0;
      }
      const int c = __hip_atomic_fetch_add(f.row_cnt + (int64_t)r * nhb + blk, 1,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (c != kept - 1) r = -1;
    }
    s_rows[threadIdx.x] = r;
  }
  __syncthreads();
  int *s_pp = s_tmp, *s_sorted = s_tmp + kMaxTopk;
  for (int t = 0; t < nrows; ++t) {
    const int r = s_rows[t];  // uniform
    if (r < 0) continue;
    if ((int)threadIdx.x < f.topk) s_pp[threadIdx.x] = f.pos_of_pair[r * f.topk + threadIdx.x];
    __syncthreads();
    // the row's kept positions in ascending order: each pair writes its
    // position at its rank (ties, possible only in inconsistent caller
    // metadata, ranked by pair index)
    int n = 0;
    for (int j = 0; j < f.topk; ++j) {
      const int v = s_pp[j];
      n += (v >= 0 && v < end) ? 1 : 0;
    }
    if ((int)threadIdx.x < f.topk) {
      const int pp = s_pp[threadIdx.x];
      if (pp >= 0 && pp < end) {
        int rank = 0;
        for (int j = 0; j < f.topk; ++j) {
          const int v = s_pp[j];
          rank += (v >= 0 && v < end && (v < pp || (v == pp && j < (int)threadIdx.x))) ? 1 : 0;
        }
        s_sorted[rank] = pp;
      }
    }
    __syncthreads();
    if (threadIdx.x < 128) {
      const int col = blk * 128 + threadIdx.x;
      float v[kMaxTopk];
#pragma unroll
      for (int k = 0; k < kMaxTopk; ++k)
        if (k < n)  // every load in flight together
          v[k] = __hip_atomic_load(p.out_f32 + (int64_t)s_sorted[k] * p.ldo + col,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      float y = 0.0f;
#pragma unroll
      for (int k = 0; k < kMaxTopk; ++k)
        if (k < n) y += v[k];
      const int64_t o = (int64_t)r * p.out_f + col;
      if (f.out_f32) ((float *)f.out)[o] = y;
      else ((uint16_t *)f.out)[o] = f32_to_out16(y, f.out_bf16);
    }
    __syncthreads();  // s_pp / s_sorted reused for the next row
  }
}

// One work item of the 16-row kernels: rows of plan tile `bx` times the
// 64-column group `by` (for gate/up, by < out_f / 64 is gate, the rest up).
// FUSED (every kernel of a single pass in one launch, experts_narrow_kernel):
//  - gate/up: the last item of a 128-column block writes its a~ block with
//    device-coherent stores, waits for them, then sets the block's count in
//    f.blk_ready[bx][blk];
//  - down: the item first prefetches its trellis (prefetch_strip), then
//    reads a~ with device-coherent loads: WA, its chain reads each a~ block
//    once that block's count is set (the chain starts on the first blocks);
//    otherwise it first waits until every a~ block of its tile is set. The
//    last item of a 128-column block writes d
//    with device-coherent stores and counts the block for each row of the
//    tile in f.row_cnt; the count that completes a row's block (one per kept
//    pair of the row) makes this item sum the row's d in ascending position
//    for that block and write the output (the ordered combine).
// Every wait is on items of lower id (gate/up before down), which were
// dispatched earlier on their XCD and never wait themselves, so it ends; it
// is also bounded, a give-up counted in ctrl[2].

template <int EPI, bool FUSED, bool WA = false>
__device__ __forceinline__ void narrow_item(const GemmParams &p, char *smem, int *s_flag, int bx,
                                            int by, const NarrowFusedParams *f) {
  constexpr int NPROJ = (EPI == EPI_GATEUP) ? 2 : 1;
  constexpr bool kCohA = FUSED && EPI == EPI_DOWN;
  int e, row0, nrows;
  if (!tile_of_block(p, kBM, bx, e, row0, nrows)) return;
  const int ncg = p.out_f >> 6;
  const int pj = (EPI == EPI_GATEUP) ? by / ncg : 0;
  const int cg = by - pj * ncg;
  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const int nt = cg * 4 + w;
  char *ring = smem + w * kNRing * kNSlot;

  // Lanes of rows past the tile's end read the last valid row (same cache
  // lines, no extra traffic); their results are never stored.
  const int arow = min(lane & 15, nrows - 1);
  const uint16_t *a_tile = p.A + (int64_t)row0 * p.lda + pj * p.a_proj_stride;
  const uint32_t avoff = (uint32_t)(arow * p.lda * 2);

  // lanes n < nrows of every 16-lane group carry rows of the tile
  const uint64_t rows16 = (nrows >= 16) ? 0xFFFFull : ((1ull << nrows) - 1);
  const uint64_t alanes = rows16 | (rows16 << 16) | (rows16 << 32) | (rows16 << 48);
  const ProjDev pd = (pj == 0) ? p.proj[0] : p.proj[1];

  // The epilogue's per-column vectors of this item's 128-column block (and
  // the route weights of the tile's rows), loaded now so their latency hides
  // under the chain; staged in LDS if this item runs the epilogue.
  const int blk = cg >> 1;
  const int tc = threadIdx.x & 127;
  const size_t vb = (size_t)e * p.out_f + blk * 128 + tc;
  uint16_t v_svh0 = 0, v_cs0 = 0, v_svh1 = 0, v_cs1 = 0, v_suh = 0;
  float v_wt = 0.0f;
  if (threadIdx.x < 128) {
    v_svh0 = p.proj[0].svh[vb];
    v_cs0 = p.proj[0].cs[vb];
    if constexpr (EPI == EPI_GATEUP) {
      v_svh1 = p.proj[1].svh[vb];
      v_cs1 = p.proj[1].cs[vb];
      v_suh = p.suh_down[vb];
    }
  } else if constexpr (EPI == EPI_DOWN) {
    if ((int)threadIdx.x - 128 < nrows) v_wt = p.weight_of_pos[p.pass_base + row0 + threadIdx.x - 128];
  }

  const int32_t *aflags = nullptr;
  if constexpr (FUSED && EPI == EPI_DOWN) {
    prefetch_strip(pd, p.E, e, p.in_f, nt, ring, lane);
    aflags = f->blk_ready + (int64_t)bx * (p.in_f >> 7);
    if constexpr (!WA) wait_all_set(aflags, p.in_f >> 7, p.ctrl);
    swait_vmcnt<0>();  // the prefetch copies have landed before the ring is reused
  }

  const f32x4 acc =
      stream_strip<kCohA, kCohA && WA>(pd, p.E, e, p.in_f, nt, ring, (const char *)a_tile, avoff,
                                       alanes, lane, p.ctrl, cg == 0 && w == 0, aflags);

  // Pre-rotation sums of this work item -> scratch [row][NPROJ][out_f].
  // Hand-off to the last work item of the 128-column block without cache
  // maintenance: the sums are written and read with device-coherent
  // (agent-scope) relaxed atomic accesses, every store has completed
  // (vmcnt 0) before the count is incremented, and the reads start only
  // after the increment that saw every other count.
  const int64_t ldn = (int64_t)NPROJ * p.out_f;
  const int col = nt * 16 + (lane & 15);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * (lane >> 4) + r;
    if (row < nrows)
      __hip_atomic_store(p.nacc + (int64_t)(row0 + row) * ldn + pj * p.out_f + col, acc[r],
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  int32_t *cnt = p.ncnt + (int64_t)bx * (p.out_f >> 7) + blk;
  if (threadIdx.x == 0)
    *s_flag = (__hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               2 * NPROJ - 1)
                  ? 1
                  : 0;
  __syncthreads();
  if (!*s_flag) return;
  if (threadIdx.x == 0)  // ready for the next launch
    __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  float *T = (float *)smem;  // [NPROJ][16][kLdsStride]
  // every item's sums of the block, all loads in flight together
  constexpr int kPer = NPROJ * kBM * 128 / 256;
  float sums[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int i = threadIdx.x + 256 * k;
    const int q = i / (kBM * 128), rem = i - q * (kBM * 128);
    const int row = rem >> 7, c = rem & 127;
    sums[k] = row < nrows ? __hip_atomic_load(p.nacc + (int64_t)(row0 + row) * ldn +
                                                  q * p.out_f + blk * 128 + c,
                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                          : 0.0f;
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int i = threadIdx.x + 256 * k;
    const int q = i / (kBM * 128), rem = i - q * (kBM * 128);
    T[(q * kBM + (rem >> 7)) * kLdsStride + (rem & 127)] = sums[k];
  }
  // staged vectors, past the accumulator tile
  uint16_t *lv = (uint16_t *)(smem + kEpiVecOff);
  float *lwt = (float *)(smem + kEpiVecOff + 5 * 128 * 2);
  if (threadIdx.x < 128) {
    lv[tc] = v_svh0;
    lv[128 + tc] = v_cs0;
    lv[256 + tc] = v_svh1;
    lv[384 + tc] = v_cs1;
    lv[512 + tc] = v_suh;
  } else if ((int)threadIdx.x - 128 < kBM) {
    lwt[threadIdx.x - 128] = v_wt;
  }
  __syncthreads();
  EpiVec ev;
  ev.v = lv;
  ev.wt = lwt;
  epilogue<EPI, FUSED, true>(p, T, kLdsStride, kBM * kLdsStride, e, row0, nrows, blk * 128, 1,
                             ev);
  if constexpr (FUSED) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's a~ / d stores
    __syncthreads();                                     // ... and every wave's
    if constexpr (EPI == EPI_GATEUP) {
      if (threadIdx.x == 0)
        __hip_atomic_store(f->blk_ready + (int64_t)bx * (p.out_f >> 7) + blk, 1,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      narrow_combine(p, *f, row0, nrows, blk, s_flag + 1, (int *)smem);
    }
  }
}

// grid: x = tile, y = NPROJ * (out_f / 64) column groups (projection major).
template <int EPI>
__global__ void __launch_bounds__(256, 4) gemm_narrow_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) char smem[4 * kNRing * kNSlot];
  __shared__ int s_flag[1];
  narrow_item<EPI, false>(p, smem, s_flag, blockIdx.x, blockIdx.y, nullptr);
}

// A single pass of the routed experts on 16-row tiles in one launch: gate/up
// work items (tile-major: tile x (2 x I/64) column groups), then down items
// (tile x H/64 groups), each waiting only on gate/up items of its own tile;
// the combine runs at the end of the down items (see narrow_item). The pack,
// plan, rotation and the zeroing of every count come before, in stream order.
// WA: down items wait per a~ block inside their chain (see StreamChain).
template <bool WA>
__global__ void __launch_bounds__(256, 4) experts_narrow_kernel(NarrowFusedParams f) {
  __shared__ __attribute__((aligned(16))) char smem[4 * kNRing * kNSlot];
  __shared__ int s_flag[1 + kBM];
  int id = blockIdx.x;
  if (id < f.g1) {
    const int per = 2 * (f.gu.out_f >> 6);
    narrow_item<EPI_GATEUP, true>(f.gu, smem, s_flag, id / per, id % per, &f);
    return;
  }
  id -= f.g1;
  const int per = f.dn.out_f >> 6;
  narrow_item<EPI_DOWN, true, WA>(f.dn, smem, s_flag, id / per, id % per, &f);
}

// Work items of experts_narrow_kernel the current device holds at once
// (cached per device).
static int64_t narrow_resident_items() {
  static std::atomic<int64_t> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int64_t v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, experts_narrow_kernel<true>, 256, 0) !=
          hipSuccess)
    return 0;
  v = (int64_t)cus * per_cu;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

// Per-block waits pay when every work item is resident at once (the down
// items then sit on CUs while gate/up finishes: starting on the first a~
// blocks shortens the critical path); with more items the launch runs in
// waves, down items of early tiles overlap gate/up of later ones anyway and
// the per-block readiness loads only cost issue slots.
hipError_t launch_experts_narrow(const NarrowFusedParams &f, hipStream_t s) {
  if (f.tiles <= 0) return hipSuccess;
  const int64_t g1 = (int64_t)f.tiles * 2 * (f.gu.out_f >> 6);
  const int64_t g2 = (int64_t)f.tiles * (f.dn.out_f >> 6);
  if (g1 != f.g1) return hipErrorInvalidValue;
  if (g1 + g2 <= narrow_resident_items())
    hipLaunchKernelGGL(experts_narrow_kernel<true>, dim3((unsigned)(g1 + g2)), dim3(256), 0, s, f);
  else
    hipLaunchKernelGGL(experts_narrow_kernel<false>, dim3((unsigned)(g1 + g2)), dim3(256), 0, s, f);
  return hipGetLastError();
}

hipError_t launch_gemm(int epi, const GemmParams &p, int tiles, int nblocks, hipStream_t s,
                       bool wide) {
  if (tiles <= 0 || nblocks <= 0) return hipSuccess;
  if (wide) return launch_gemm_wide(epi, p, tiles, nblocks, s);
  // nblocks: 128-column blocks per projection
  const int nproj = (epi == EPI_GATEUP) ? 2 : 1;
  const dim3 grid(tiles, nproj * 2 * nblocks);
  switch (epi) {
    case EPI_GATEUP:
      hipLaunchKernelGGL(gemm_narrow_kernel<EPI_GATEUP>, grid, dim3(256), 0, s, p);
      break;
    case EPI_DOWN:
      hipLaunchKernelGGL(gemm_narrow_kernel<EPI_DOWN>, grid, dim3(256), 0, s, p);
      break;
    default:
      hipLaunchKernelGGL(gemm_narrow_kernel<EPI_LINEAR>, grid, dim3(256), 0, s, p);
      break;
  }
  return hipGetLastError();
}

// Diagnostic decode with the GEMMs' own decode path: one wave per pair of
// consecutive tiles (taken as the two tiles of one 32-input k-step), each
// lane decoding the half column HalfWindow assigns it with decode_half, from
// the same window byte offsets and shift the GEMM kernels use (the GEMMs read
// those dwords from their LDS rings, this kernel from global memory). Output
// [tile][k][n] fp16 in natural k order: register r of lane (g, n) holds
// states (r, r + 4) of its half, i.e. k = 8 (g & 1) + r and k + 4.
template <int K>
__device__ void decode_pair_wave(const uint16_t *words, int ntiles, int pair, uint16_t *out,
                                 int lane) {
  const int g = lane >> 4, n = lane & 15;
  const int tile = 2 * pair + (g >> 1);
  if (tile >= ntiles) return;
  const uint32_t *base = (const uint32_t *)(words + (size_t)(2 * pair) * 16 * K);
  const HalfWindow<K> hw(lane);
  uint32_t raw[HalfGeom<K>::kLoadDw];
#pragma unroll
  for (int j = 0; j < HalfGeom<K>::kLoadDw; ++j) raw[j] = base[hw.off[j] >> 2];
  const u32x4 b = decode_half<K>(raw, hw.shift, codebook_mask());
  uint16_t *o = out + (size_t)tile * 256;
  const int k0 = 8 * (g & 1);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    o[(k0 + r) * 16 + n] = (uint16_t)(b[r] & 0xFFFFu);
    o[(k0 + r + 4) * 16 + n] = (uint16_t)(b[r] >> 16);
  }
}

__global__ void decode_tiles_kernel(const uint16_t *words, int ntiles, int K,
                                    uint16_t *out) {
  const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (2 * pair >= ntiles) return;
  const int lane = threadIdx.x & 63;
  switch (K) {
    case 2: decode_pair_wave<2>(words, ntiles, pair, out, lane); break;
    case 3: decode_pair_wave<3>(words, ntiles, pair, out, lane); break;
    case 4: decode_pair_wave<4>(words, ntiles, pair, out, lane); break;
    case 5: decode_pair_wave<5>(words, ntiles, pair, out, lane); break;
    case 6: decode_pair_wave<6>(words, ntiles, pair, out, lane); break;
    case 7: decode_pair_wave<7>(words, ntiles, pair, out, lane); break;
    default: decode_pair_wave<8>(words, ntiles, pair, out, lane); break;
  }
}

hipError_t launch_decode_tiles(const uint16_t *words, int ntiles, int K,
                               uint16_t *out, hipStream_t s) {
  if (ntiles <= 0) return hipSuccess;
  const int pairs = (ntiles + 1) / 2;
  hipLaunchKernelGGL(decode_tiles_kernel, dim3((pairs + 3) / 4), dim3(256), 0, s,
                     words, ntiles, K, out);
  return hipGetLastError();
}

}  // namespace exl3
