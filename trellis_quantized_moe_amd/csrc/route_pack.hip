// Route histogram -> exclusive scan -> stable pack of (row, expert) pairs, and
// the per-pass work plan over the fixed-capacity workspace.
// exllamav3 PR #284 "MoE: Add fused additive EXL3 kernels" (Summary: stable
// route packing; oversized expert spans tiled within the fixed scratch;
// API contract: num_active counts non-empty experts and is only a hint;
// Relationship to #246: route histogram, scan and stable packing).
//
// One workgroup of 1024 threads (16 waves). Wave w owns one contiguous
// segment of the pairs and walks it twice, 64 pairs per round in pair order:
// first it counts its pairs per expert into an LDS row of its own, then (once
// the counts are scanned over experts and over the waves before it) it gives
// each pair the next position of its expert. Inside a round, the lanes that
// hold the same expert find each other with bitwise ballots, so positions
// follow pair order exactly without atomics on the positions.
#include "common.hpp"
#include "kernels.hpp"
#include "rotate_dev.hpp"

namespace exl3 {

constexpr int kPackThreads = 1024;
constexpr int kPackWaves = kPackThreads / 64;
constexpr int kMaxE = 1024;

// Exclusive scan over the block (1024 threads); returns the prefix and the
// block total. `tmp` holds kPackWaves ints.
__device__ int block_exclusive_scan(int v, int *tmp, int &total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) tmp[w] = x;
  __syncthreads();
  int before = 0, all = 0;
  for (int k = 0; k < kPackWaves; ++k) {
    const int t = tmp[k];
    before += (k < w) ? t : 0;
    all += t;
  }
  __syncthreads();
  total = all;
  return before + x - v;
}

// Inclusive prefix maximum over the block (1024 threads); `tmp` holds
// kPackWaves ints. Returns the prefix and sets `all` to the block maximum.
__device__ int block_inclusive_max(int v, int *tmp, int &all) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x = max(x, y);
  }
  if (lane == 63) tmp[w] = x;
  __syncthreads();
  int before = x, m = INT_MIN;
  for (int k = 0; k < kPackWaves; ++k) {
    const int t = tmp[k];
    if (k < w) before = max(before, t);
    m = max(m, t);
  }
  __syncthreads();
  all = m;
  return before;
}

// Last expert whose span starts at or before `pos` (offsets nondecreasing).
__device__ __forceinline__ int expert_at(const int *off, int E, int pos) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= pos) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ float load_weight(const void *w, int dtype, int q) {
  if (dtype == 3) return ((const float *)w)[q];
  const uint16_t b = ((const uint16_t *)w)[q];
  if (dtype == 2) return __builtin_bit_cast(float, (uint32_t)b << 16);  // bf16
  return f16_bits_to_f32(b);
}

__device__ __forceinline__ int load_expert(const void *ids, int i64, int q, int E) {
  if (i64) {
    const int64_t v = ((const int64_t *)ids)[q];
    return (v >= 0 && v < E) ? (int)v : -1;
  }
  const int32_t v = ((const int32_t *)ids)[q];
  return (v >= 0 && v < E) ? v : -1;
}

// Lanes of the wave holding the same key as this lane (among `live`), using
// the low `nb` bits of the key.
__device__ __forceinline__ uint64_t match_key(int key, uint64_t live, int nb) {
  uint64_t m = live;
  for (int b = 0; b < nb; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t bal = __ballot(bit);
    m &= bit ? bal : ~bal;
  }
  return m;
}

constexpr int kPackBatch = 8;  // rounds whose loads are issued together

// a4 for one position range [pb, pe) (a pass, or a launch unit of several
// passes), by one wave: the row tiles of every expert's sub-span inside the
// range; only the experts overlapping the range are visited.
// Order: full tiles (bm rows) first, in expert order, then the partial
// tiles (at most one per expert: the end of its span); for 128-row tiles
// and at most 128 experts in the range those go by rows descending, ties in
// expert order, otherwise in expert order. Heavy tiles so come first in
// dispatch order, where each gets a CU of its own before the light ones
// fill the second slots; the order never changes a result. s_off: the
// expert offsets (E + 1, nondecreasing), kept = s_off[E].
// Tiles of the range go to `plan` (after its count word), their first rows
// relative to pb. Returns the range's tile count; the caller writes it.
__device__ int plan_range(const PackParams &p, const int *s_off, int E, int pb, int pe, int lane,
                          int32_t *plan) {
  int total = 0;
  if (pb < pe) {
    const int e_lo = expert_at(s_off, E, pb), e_hi = expert_at(s_off, E, pe - 1);
    const int bm = p.bm;
    auto span = [&](int e, int &lo, int &hi) {
      lo = max(s_off[e], pb);
      hi = min(s_off[e + 1], pe);
    };
    for (int eb = e_lo; eb <= e_hi; eb += 64) {  // full tiles
      const int e = eb + lane;
      int lo = 0, hi = 0, nf = 0;
      if (e <= e_hi) {
        span(e, lo, hi);
        nf = hi > lo ? (hi - lo) / bm : 0;
      }
      int x = nf;  // inclusive scan over the wave
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
      }
      const int slot0 = total + x - nf;
      for (int t = 0; t < nf; ++t) {
        int32_t *d = plan + 1 + 3 * (slot0 + t);
        d[0] = e;
        d[1] = lo - pb + t * bm;
        d[2] = bm;
      }
      total += __shfl(x, 63, 64);
    }
    // partial rows of the experts e_lo + lane and e_lo + 64 + lane
    int prow[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int e = e_lo + 64 * c + lane;
      int lo = 0, hi = 0;
      if (e <= e_hi) span(e, lo, hi);
      prow[c] = hi > lo ? (hi - lo) % bm : 0;
    }
    const bool sort = bm == kBMWide && e_hi - e_lo < 128;
    const int nfull = total;
    int npart = 0;
    for (int eb = e_lo; eb <= e_hi; eb += 64) {  // partial tiles
      const int e = eb + lane, c = (eb - e_lo) >> 6;
      int lo = 0, hi = 0;
      if (e <= e_hi) span(e, lo, hi);
      const int rows = (c < 2) ? prow[c & 1] : (hi > lo ? (hi - lo) % bm : 0);
      const uint64_t has = __ballot(rows > 0);
      int rank = npart + __popcll(has & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
      if (sort) {  // rows descending, then expert order, over both chunks
        rank = 0;
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
          for (int l = 0; l < 64; ++l) {
            const int r2 = __shfl(prow[c2], l, 64);
            const int e2 = e_lo + 64 * c2 + l;
            rank += (r2 > rows || (r2 == rows && e2 < e)) ? 1 : 0;
          }
      }
      if (rows > 0) {
        int32_t *d = plan + 1 + 3 * (nfull + rank);
        d[0] = e;
        d[1] = lo - pb + (hi - lo) / bm * bm;
        d[2] = rows;
      }
      npart += __popcll(has);
    }
    total = nfull + npart;
  }
  return total;
}

// Plans of every launch unit (p.group consecutive passes), one wave per unit.
// A unit's passes are consecutive position ranges, and every pass but the
// last holds exactly `capacity` positions, so the unit's rows are one
// contiguous range of its buffers: its tiles are planned over the whole
// range, and an expert span that a pass boundary cuts inside the unit still
// gives one run of tiles (each row's result does not depend on its tile).
__device__ void plan_units(const PackParams &p, const int *s_off, int E, int kept, int w,
                           int nw, int lane) {
  const int G = max(p.group, 1);
  const int units = (p.passes + G - 1) / G;
  for (int u = w; u < units; u += nw) {
    int32_t *plan = p.plan + (int64_t)u * (1 + 3 * (int64_t)G * p.slots);
    const int64_t ub = (int64_t)u * G * p.capacity;
    const int ue = (int)min(ub + (int64_t)G * p.capacity, (int64_t)kept);
    const int n = plan_range(p, s_off, E, (int)ub, ue, lane, plan);
    if (lane == 0) plan[0] = n;
  }
}

// ---------------------------------------------------- phases of the pack
// Shared by the one-workgroup kernel and the three-launch form for many
// pairs. A wave's segment of pairs [q0, q1) is walked in rounds of 64 pairs
// in pair order.

// a1: the segment's pairs counted per expert into wc (this wave's LDS row);
// returns the number of pairs with an ID outside [0, E).
__device__ __forceinline__ int count_segment(const PackParams &p, int q0, int q1, int *wc,
                                             int lane) {
  int drop = 0;
  for (int qb = q0; qb < q1; qb += 64 * kPackBatch) {
    int eb[kPackBatch];
#pragma unroll
    for (int i = 0; i < kPackBatch; ++i) {
      const int q = qb + 64 * i + lane;
      eb[i] = (q < q1) ? load_expert(p.ids, p.ids_i64, q, p.E) : -2;
    }
#pragma unroll
    for (int i = 0; i < kPackBatch; ++i) {
      const int e = eb[i];
      if (e >= 0) atomicAdd(&wc[e], 1);  // counts are order-free
      drop += (e == -1) ? 1 : 0;
    }
  }
  return drop;
}

// a3: stable scatter of the segment; wc[e] holds the next position of expert
// e for this wave. Inside a round, the lanes holding the same expert find
// each other with ballots, so positions follow pair order without atomics.
__device__ __forceinline__ void scatter_segment(const PackParams &p, int q0, int q1, int *wc,
                                                int lane) {
  const int E = p.E;
  const int nb = 32 - __clz(E);  // bits of the keys 0 .. E
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int qb = q0; qb < q1; qb += 64 * kPackBatch) {
    int eb[kPackBatch];
    float wb[kPackBatch];
#pragma unroll
    for (int i = 0; i < kPackBatch; ++i) {
      const int q = qb + 64 * i + lane;
      const bool in = q < q1;
      eb[i] = in ? load_expert(p.ids, p.ids_i64, q, E) : -2;
      wb[i] = in ? load_weight(p.w, p.w_dtype, q) : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < kPackBatch; ++i) {
      if (qb + 64 * i >= q1) break;  // uniform
      const int q = qb + 64 * i + lane;
      const int e = eb[i];
      const bool valid = e >= 0;
      const uint64_t m = match_key(valid ? e : E, __ballot(valid), nb);
      if (valid) {
        const int rank = __popcll(m & lt_mask);
        const int base = wc[e];
        const int pos = base + rank;
        if (rank == 0) wc[e] = base + __popcll(m);
        p.pair_of_pos[pos] = q;
        p.weight_of_pos[pos] = wb[i];
        p.pos_of_pair[q] = pos;
      } else if (e == -1) {
        p.pos_of_pair[q] = -1;
      }
    }
  }
}

// The positions [a, b) of the metadata after the pack: empty ones past the
// kept pairs cleared, kept ones given their expert (positions before the
// first span, possible only with caller-supplied offsets, get expert 0).
// s_off: the expert offsets (E + 1). Threads t of nt.
__device__ __forceinline__ void finish_positions(const PackParams &p, const int *s_off, int a,
                                                 int b, int t, int nt, bool clear_tail) {
  const int E = p.E, kept = s_off[E];
  for (int pos = a + t; pos < b; pos += nt) {
    if (pos >= kept) {
      if (clear_tail) {
        p.pair_of_pos[pos] = -1;
        p.weight_of_pos[pos] = 0.0f;
      }
      continue;
    }
    if (p.do_plan) p.expert_of_pos[pos] = (pos < s_off[0]) ? 0 : expert_at(s_off, E, pos);
  }
}

// Zero output rows r in [r0, r1) none of whose pairs is kept.
__device__ __forceinline__ void zero_unrouted_rows(const PackParams &p, int r0, int r1, int t,
                                                   int nt) {
  for (int r = r0 + t; r < r1; r += nt) {
    bool any = false;
    for (int j = 0; j < p.topk; ++j) any |= p.pos_of_pair[r * p.topk + j] >= 0;
    if (!any) {
      for (int c = 0; c < p.H; ++c) {
        if (p.out_f32) ((float *)p.out)[(int64_t)r * p.H + c] = 0.0f;
        else ((uint16_t *)p.out)[(int64_t)r * p.H + c] = 0;
      }
    }
  }
}

// a4 and the clears of the call: the plan of every launch unit, ctrl[1..2]
// and the completion counts. One workgroup of kPackThreads.
__device__ __forceinline__ void plan_and_clear(const PackParams &p, const int *s_off, int tid) {
  const int E = p.E, w = tid >> 6, lane = tid & 63;
  if (tid == 0 && p.ctrl) {
    p.ctrl[1] = 0;  // bad stage entries
    p.ctrl[2] = 0;  // waits that gave up
  }
  for (int i = tid; i < p.nzero; i += kPackThreads) p.zero[i] = 0;
  const int kept = s_off[E];
  plan_units(p, s_off, E, kept, w, kPackWaves, lane);
}

__global__ void __launch_bounds__(kPackThreads) pack_plan_kernel(PackParams p) {
  __shared__ int s_wc[kPackWaves][kMaxE];  // per wave: count, then next position
  __shared__ int s_off[kMaxE + 1];
  __shared__ int s_tmp[kPackWaves];
  __shared__ int s_dropped;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int E = p.E;
  const int pairs = p.rows * p.topk;
  if (tid == 0) s_dropped = 0;

  if (p.do_pack) {
    // the wave's segment: whole rounds of 64 pairs
    const int seg = (((pairs + kPackWaves - 1) / kPackWaves) + 63) & ~63;
    const int q0 = w * seg;
    const int q1 = min(q0 + seg, pairs);
    int *wc = s_wc[w];
    for (int e = lane; e < E; e += 64) wc[e] = 0;
    __syncthreads();

    // a1: this wave's histogram (only this wave touches its row)
    const int drop = count_segment(p, q0, q1, wc, lane);
    if (drop) atomicAdd(&s_dropped, drop);
    __syncthreads();

    // a2: counts over the waves, exclusive scan over experts, then each
    // wave's first position per expert
    {
      int c = 0;
      if (tid < E)
        for (int k = 0; k < kPackWaves; ++k) c += s_wc[k][tid];
      int total;
      const int ex = block_exclusive_scan(c, s_tmp, total);
      int nact;
      block_exclusive_scan((tid < E && c > 0) ? 1 : 0, s_tmp, nact);
      if (tid < E) {
        int run = ex;
        for (int k = 0; k < kPackWaves; ++k) {
          const int t = s_wc[k][tid];
          s_wc[k][tid] = run;
          run += t;
        }
        s_off[tid] = ex;
        p.count[tid] = c;
        p.offset[tid] = ex;
      }
      if (tid == 0) {
        s_off[E] = total;
        p.offset[E] = total;
        *p.num_active = nact;
        *p.status = s_dropped;
        if (p.ctrl) p.ctrl[0] = s_dropped;
      }
      __syncthreads();
    }

    // a3: stable scatter, the same walk again
    scatter_segment(p, q0, q1, wc, lane);
    finish_positions(p, s_off, 0, pairs, tid, kPackThreads, true);
  } else {
    // caller-supplied offsets, clamped into the pairs and made nondecreasing
    // (a prefix maximum leaves consistent offsets unchanged), so every index
    // derived from them stays inside the pairs and the experts
    const int v = (tid < E) ? min(max(p.offset[tid], 0), pairs) : 0;
    int vmax;
    const int m = block_inclusive_max(v, s_tmp, vmax);
    if (tid < E) s_off[tid] = m;
    if (tid == 0) s_off[E] = max(min(max(p.offset[E], 0), pairs), vmax);
    // dropped pairs of the caller's pack (no position): reported in ctrl[0]
    int drop = 0;
    for (int q = tid; q < pairs; q += kPackThreads) drop += (p.pos_of_pair[q] < 0) ? 1 : 0;
    if (drop) atomicAdd(&s_dropped, drop);
    __syncthreads();
    if (tid == 0 && p.ctrl) p.ctrl[0] = s_dropped;
    if (p.do_plan) finish_positions(p, s_off, 0, pairs, tid, kPackThreads, false);
  }

  if (!p.do_plan) return;
  plan_and_clear(p, s_off, tid);

  // rows whose pairs were all dropped produce zeros (rare). A pack that
  // dropped nothing has no such row.
  __syncthreads();
  if (p.out && (!p.do_pack || s_dropped > 0)) zero_unrouted_rows(p, 0, p.rows, tid, kPackThreads);
}

// ------------------------------------------- the pack over many workgroups
// For many pairs the walk above is split over nblk workgroups of kPackThreads
// in three launches (stream order carries every dependency): block b owns
// pairs [b S, (b + 1) S), S = kPairsPerPackBlock, and its wave w the w-th
// sixteenth of them.
//   pack_count_kernel: every wave counts its pairs per expert into gwc[b][w][e];
//   pack_scan_kernel (one workgroup): expert totals, the exclusive scan over
//     experts and over (b, w) in that order, written back into gwc as each
//     wave's first position per expert; counts, offsets and status words;
//   pack_scatter_kernel: every wave scatters its pairs from those positions
//     (the same positions as one walk over all pairs), then clears and labels
//     its block's share of the positions; one extra workgroup plans.
constexpr int kPairsPerPackBlock = 4096;

int pack_blocks(int64_t pairs) { return (int)((pairs + kPairsPerPackBlock - 1) / kPairsPerPackBlock); }

__device__ __forceinline__ void pack_block_segment(const PackParams &p, int b, int w, int &q0,
                                                   int &q1) {
  const int pairs = p.rows * p.topk;
  const int seg = kPairsPerPackBlock / kPackWaves;  // whole rounds of 64
  q0 = min(b * kPairsPerPackBlock + w * seg, pairs);
  q1 = min(q0 + seg, pairs);
}

__global__ void __launch_bounds__(kPackThreads) pack_count_kernel(PackParams p) {
  __shared__ int s_wc[kPackWaves][kMaxE];
  __shared__ int s_dropped;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, b = blockIdx.x, E = p.E;
  if (tid == 0) s_dropped = 0;
  int *wc = s_wc[w];
  for (int e = lane; e < E; e += 64) wc[e] = 0;
  __syncthreads();
  int q0, q1;
  pack_block_segment(p, b, w, q0, q1);
  const int drop = count_segment(p, q0, q1, wc, lane);
  if (drop) atomicAdd(&s_dropped, drop);
  int32_t *g = p.gwc + ((int64_t)b * kPackWaves + w) * E;
  for (int e = lane; e < E; e += 64) g[e] = wc[e];
  __syncthreads();
  if (tid == 0) p.gwc[(int64_t)p.nblk * kPackWaves * E + b] = s_dropped;
}

__global__ void __launch_bounds__(kPackThreads) pack_scan_kernel(PackParams p) {
  __shared__ int s_tmp[kPackWaves];
  const int tid = threadIdx.x, E = p.E, nw = p.nblk * kPackWaves;
  // one block's 16 wave counts per step, loaded together
  int c = 0;
  if (tid < E)
    for (int b = 0; b < p.nblk; ++b) {
      int v[kPackWaves];
#pragma unroll
      for (int w = 0; w < kPackWaves; ++w) v[w] = p.gwc[(int64_t)(b * kPackWaves + w) * E + tid];
#pragma unroll
      for (int w = 0; w < kPackWaves; ++w) c += v[w];
    }
  int total;
  const int ex = block_exclusive_scan(c, s_tmp, total);
  int nact;
  block_exclusive_scan((tid < E && c > 0) ? 1 : 0, s_tmp, nact);
  if (tid < E) {
    int run = ex;
    for (int b = 0; b < p.nblk; ++b) {
      int32_t *g = p.gwc + (int64_t)b * kPackWaves * E + tid;
      int v[kPackWaves];
#pragma unroll
      for (int w = 0; w < kPackWaves; ++w) v[w] = g[(int64_t)w * E];
#pragma unroll
      for (int w = 0; w < kPackWaves; ++w) {
        g[(int64_t)w * E] = run;
        run += v[w];
      }
    }
    p.count[tid] = c;
    p.offset[tid] = ex;
  }
  if (tid == 0) {
    int dropped = 0;
    for (int b = 0; b < p.nblk; ++b) dropped += p.gwc[(int64_t)nw * E + b];
    p.offset[E] = total;
    *p.num_active = nact;
    *p.status = dropped;
    if (p.ctrl) p.ctrl[0] = dropped;
  }
}

__global__ void __launch_bounds__(kPackThreads) pack_scatter_kernel(PackParams p) {
  __shared__ int s_wc[kPackWaves][kMaxE];
  __shared__ int s_off[kMaxE + 1];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, b = blockIdx.x, E = p.E;
  for (int e = tid; e <= E; e += kPackThreads) s_off[e] = p.offset[e];
  if (b == p.nblk) {  // the planner
    __syncthreads();
    if (p.do_plan) plan_and_clear(p, s_off, tid);
    return;
  }
  int *wc = s_wc[w];
  const int32_t *g = p.gwc + ((int64_t)b * kPackWaves + w) * E;
  for (int e = lane; e < E; e += 64) wc[e] = g[e];
  __syncthreads();
  int q0, q1;
  pack_block_segment(p, b, w, q0, q1);
  scatter_segment(p, q0, q1, wc, lane);
  const int pairs = p.rows * p.topk;
  const int a = min(b * kPairsPerPackBlock, pairs), z = min(a + kPairsPerPackBlock, pairs);
  finish_positions(p, s_off, a, z, tid, kPackThreads, true);
  // rows with no kept pair (IDs all outside [0, E)) produce zeros: the rows
  // whose first pair is in this block, found from their IDs
  if (p.out && p.do_plan && *p.status > 0) {
    const int r0 = (a + p.topk - 1) / p.topk, r1 = (z + p.topk - 1) / p.topk;
    for (int r = r0 + tid; r < r1; r += kPackThreads) {
      bool any = false;
      for (int j = 0; j < p.topk; ++j) any |= load_expert(p.ids, p.ids_i64, r * p.topk + j, E) >= 0;
      if (!any) {
        for (int c = 0; c < p.H; ++c) {
          if (p.out_f32) ((float *)p.out)[(int64_t)r * p.H + c] = 0.0f;
          else ((uint16_t *)p.out)[(int64_t)r * p.H + c] = 0;
        }
      }
    }
  }
}

// The same pack and one-pass plan for at most kSmallPairs pairs, by a single
// wave and without barriers (decode-size calls, where the big kernel's
// barriers and phases are most of its time). Lane l holds pairs l, l + 64,
// l + 128 and l + 192 (rounds 0..3); the pairs are counted per expert with
// LDS atomics, the counts scanned over the experts by the wave, and the
// rounds walked in pair order, each pair's rank among the earlier pairs of
// its expert in its round found with ballots: the same positions as the big
// kernel.
constexpr int kSmallRounds = 4;
constexpr int kSmallPairs = 64 * kSmallRounds;

struct SmallPairs {
  int e[kSmallRounds];      // expert of the lane's pair; -1 dropped, -2 no pair
  float w[kSmallRounds];    // its route weight (when loaded)
  int pos[kSmallRounds];    // its position, -1 if none
  int kept, dropped, nact;
};

// Positions of the (at most kSmallPairs) pairs by one wave. s_cur and s_off
// hold E and E + 1 ints of LDS; s_off ends as the expert offsets. With
// `meta` the weights are loaded and the counts and offsets written.
__device__ SmallPairs small_positions(const PackParams &p, int *s_cur, int *s_off, bool meta) {
  const int lane = threadIdx.x & 63;
  const int E = p.E;
  const int pairs = p.rows * p.topk;
  SmallPairs r;
  for (int e = lane; e < E; e += 64) s_cur[e] = 0;
  int dropped = 0;
#pragma unroll
  for (int i = 0; i < kSmallRounds; ++i) {
    const int q = 64 * i + lane;
    const bool in = q < pairs;
    r.e[i] = in ? load_expert(p.ids, p.ids_i64, q, E) : -2;
    r.w[i] = (in && meta) ? load_weight(p.w, p.w_dtype, q) : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < kSmallRounds; ++i) {
    if (r.e[i] >= 0) atomicAdd(&s_cur[r.e[i]], 1);  // counts are order-free
    dropped += __popcll(__ballot(r.e[i] == -1));
  }
  r.dropped = dropped;
  int run = 0, nact = 0;
  for (int eb = 0; eb < E; eb += 64) {  // exclusive scan over the experts
    const int e = eb + lane;
    const int c = (e < E) ? s_cur[e] : 0;
    int x = c;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(x, d, 64);
      if (lane >= d) x += y;
    }
    const int ex = run + x - c;
    if (e < E) {
      s_off[e] = ex;
      s_cur[e] = ex;
      if (meta) {
        p.count[e] = c;
        p.offset[e] = ex;
      }
    }
    nact += __popcll(__ballot(e < E && c > 0));
    run += __shfl(x, 63, 64);
  }
  r.kept = run;
  r.nact = nact;
  if (lane == 0) s_off[E] = run;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int nb = 32 - __clz(E);
#pragma unroll
  for (int i = 0; i < kSmallRounds; ++i) {  // rounds in pair order
    if (64 * i >= pairs) {
      r.pos[i] = -1;
      continue;
    }
    const bool valid = r.e[i] >= 0;
    const uint64_t m = match_key(valid ? r.e[i] : E, __ballot(valid), nb);
    const int rank = __popcll(m & lt_mask);
    int base = 0;
    if (valid) base = s_cur[r.e[i]];
    r.pos[i] = valid ? base + rank : -1;
    // the round's lowest lane of each expert moves that expert's cursor on;
    // every lane read the cursor first (LDS ops of one wave complete in order)
    if (valid && rank == 0) s_cur[r.e[i]] = base + __popcll(m);
  }
  return r;
}

// Pack (and with do_plan the one-pass plan) of at most kSmallPairs pairs by
// the first wave of the block; the other waves return. With `zero` the wave
// also clears the counts p.zero (else the caller's other waves do).
__device__ void pack_small(const PackParams &p, bool zero) {
  __shared__ int s_cur[kMaxE];
  __shared__ int s_off[kMaxE + 1];
  __shared__ int s_rowhit[kSmallPairs];
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  const int pairs = p.rows * p.topk;
  const SmallPairs r = small_positions(p, s_cur, s_off, true);
  if (lane == 0) {
    p.offset[p.E] = r.kept;
    *p.num_active = r.nact;
    *p.status = r.dropped;
    if (p.ctrl) p.ctrl[0] = r.dropped;
  }
  if (p.do_plan)
    for (int row = lane; row < p.rows; row += 64) s_rowhit[row] = 0;
#pragma unroll
  for (int i = 0; i < kSmallRounds; ++i) {
    const int q = 64 * i + lane;
    if (r.e[i] >= 0) {
      p.pair_of_pos[r.pos[i]] = q;
      p.weight_of_pos[r.pos[i]] = r.w[i];
      p.pos_of_pair[q] = r.pos[i];
      if (p.do_plan) {
        p.expert_of_pos[r.pos[i]] = r.e[i];
        s_rowhit[q / p.topk] = 1;
      }
    } else if (r.e[i] == -1) {
      p.pos_of_pair[q] = -1;
    }
  }
  for (int pos = r.kept + lane; pos < pairs; pos += 64) {
    p.pair_of_pos[pos] = -1;
    p.weight_of_pos[pos] = 0.0f;
  }
  if (!p.do_plan) return;
  if (lane == 0 && p.ctrl) {
    p.ctrl[1] = 0;  // bad stage entries
    p.ctrl[2] = 0;  // waits that gave up
  }
  if (zero)
    for (int i = lane; i < p.nzero; i += 64) p.zero[i] = 0;
  plan_units(p, s_off, p.E, r.kept, 0, 1, lane);  // one pass: capacity >= pairs
  // rows whose pairs were all dropped produce zeros
  if (p.out && r.dropped > 0) {
    for (int row = 0; row < p.rows; ++row) {
      if (s_rowhit[row]) continue;  // uniform
      for (int c = lane; c < p.H; c += 64) {
        if (p.out_f32) ((float *)p.out)[(int64_t)row * p.H + c] = 0.0f;
        else ((uint16_t *)p.out)[(int64_t)row * p.H + c] = 0;
      }
    }
  }
}

__global__ void __launch_bounds__(64) pack_small_kernel(PackParams p) { pack_small(p, true); }

// Pack, plan and the rotation of the one pass in a single launch (at most
// kSmallPairs pairs): block 0 packs, plans and clears the counts; every other
// block rotates 16 (pair, 128-block) units, one per 16-lane group, finding
// each pair's position itself: pos(q) = #{kept pairs of a lower expert} +
// #{earlier pairs of the same expert}, counted over the route IDs (loaded
// into LDS once per block). That is the stable pack's position by
// definition, so no block waits for another.
__global__ void __launch_bounds__(256) pack_rotate_small_kernel(PackParams p, RotParams rp) {
  if (blockIdx.x == 0) {
    // waves 1-3 clear the counts of the launches that follow while wave 0
    // packs and plans
    if (threadIdx.x >= 64)
      for (int i = threadIdx.x - 64; i < p.nzero; i += blockDim.x - 64) p.zero[i] = 0;
    pack_small(p, false);
    return;
  }
  __shared__ int s_ids[kSmallPairs];
  const int pairs = p.rows * p.topk;
  for (int q = threadIdx.x; q < pairs; q += blockDim.x)
    s_ids[q] = load_expert(p.ids, p.ids_i64, q, p.E);
  __syncthreads();
  const int nblk = rp.H >> 7;
  const int gid = (blockIdx.x - 1) * 16 + (threadIdx.x >> 4);
  const int q = gid / nblk, blk = gid - q * nblk;
  if (q >= pairs) return;  // uniform per group
  const int e = s_ids[q];
  if (e < 0) return;  // dropped pair
  const int i = threadIdx.x & 15;
  int before = 0;
  for (int q2 = i; q2 < pairs; q2 += 16) {
    const int e2 = s_ids[q2];
    before += (e2 >= 0 && (e2 < e || (e2 == e && q2 < q))) ? 1 : 0;
  }
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) before += __shfl_xor(before, d, 64);
  rotate_block16(rp, before, blk, q / p.topk, e, i);
}

hipError_t launch_pack_rotate(const PackParams &p, const RotParams &rp, hipStream_t s) {
  const int64_t pairs = (int64_t)p.rows * p.topk;
  if (!p.do_pack || !p.do_plan || p.passes != 1 || pairs > kSmallPairs || rp.nproj < 1 ||
      rp.nproj > 2 || rp.pass_base != 0 || rp.nitems < pairs)
    return hipErrorInvalidValue;
  const int64_t units = pairs * (rp.H >> 7);
  hipLaunchKernelGGL(pack_rotate_small_kernel, dim3((unsigned)(1 + (units + 15) / 16)), dim3(256),
                     0, s, p, rp);
  return hipGetLastError();
}

bool pack_rotate_fits(int64_t pairs, int passes) { return pairs <= kSmallPairs && passes == 1; }

// A pack launched alone takes the single wave up to 64 pairs (one round);
// with more pairs the 16-wave kernel measured faster there.
constexpr int kSmallPackAlone = 64;

// From this many pairs the pack runs over several workgroups (three
// launches, pack_count/scan/scatter): on the 24576-pair prefill layer the one
// workgroup took 80 us, 45 of them in the scatter.
constexpr int64_t kMultiPackPairs = 2 * kPairsPerPackBlock;

hipError_t launch_pack(const PackParams &p, hipStream_t s) {
  const int64_t pairs = (int64_t)p.rows * p.topk;
  if (p.do_pack && pairs <= kSmallPackAlone && (!p.do_plan || p.passes == 1)) {
    hipLaunchKernelGGL(pack_small_kernel, dim3(1), dim3(64), 0, s, p);
  } else if (p.do_pack && pairs >= kMultiPackPairs && p.gwc) {
    // (exl3_route_pack has no workspace: it keeps the one-workgroup kernel)
    if (p.nblk != pack_blocks(pairs) || p.E > kMaxE) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pack_count_kernel, dim3(p.nblk), dim3(kPackThreads), 0, s, p);
    hipLaunchKernelGGL(pack_scan_kernel, dim3(1), dim3(kPackThreads), 0, s, p);
    hipLaunchKernelGGL(pack_scatter_kernel, dim3(p.nblk + 1), dim3(kPackThreads), 0, s, p);
  } else {
    hipLaunchKernelGGL(pack_plan_kernel, dim3(1), dim3(kPackThreads), 0, s, p);
  }
  return hipGetLastError();
}

size_t pack_scratch_ints(int64_t pairs, int E) {
  if (pairs < kMultiPackPairs) return 0;
  const int64_t nb = pack_blocks(pairs);
  return (size_t)(nb * kPackWaves * (int64_t)E + nb);
}

}  // namespace exl3
