// Route histogram -> exclusive scan -> stable pack of (row, expert) pairs, and
// the per-pass work plan over the fixed-capacity workspace.
// exllamav3 PR #284 "MoE: Add fused additive EXL3 kernels" (Summary: stable
// route packing; oversized expert spans tiled within the fixed scratch;
// API contract: num_active counts non-empty experts and is only a hint;
// Relationship to #246: route histogram, scan and stable packing).
//
// One workgroup of 1024 threads (16 waves). Pairs are visited in chunks of
// 1024 in pair order; inside a chunk each lane finds the lanes of its wave
// holding the same expert with a bitwise ballot match, and earlier waves'
// counts come from an LDS table, so positions follow pair order exactly.
#include "common.hpp"
#include "kernels.hpp"

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

__global__ void __launch_bounds__(kPackThreads) pack_plan_kernel(PackParams p) {
  __shared__ int s_cnt[kMaxE];
  __shared__ int s_off[kMaxE + 1];
  __shared__ int s_cur[kMaxE];
  __shared__ uint8_t s_wcnt[kPackWaves][kMaxE];
  __shared__ int s_tmp[kPackWaves];
  __shared__ int s_dropped;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int E = p.E;
  const int pairs = p.rows * p.topk;

  if (p.do_pack) {
    for (int e = tid; e < E; e += kPackThreads) s_cnt[e] = 0;
    for (int k = tid; k < kPackWaves * kMaxE; k += kPackThreads) (&s_wcnt[0][0])[k] = 0;
    if (tid == 0) s_dropped = 0;
    __syncthreads();
    // a1: histogram (integer LDS atomics: the counts are order-free)
    int drop = 0;
    for (int q = tid; q < pairs; q += kPackThreads) {
      const int e = load_expert(p.ids, p.ids_i64, q, E);
      if (e >= 0) atomicAdd(&s_cnt[e], 1);
      else ++drop;
    }
    if (drop) atomicAdd(&s_dropped, drop);
    __syncthreads();
  } else {
    // caller-supplied offsets, clamped so every index stays inside the pairs
    for (int e = tid; e <= E; e += kPackThreads) s_off[e] = min(max(p.offset[e], 0), pairs);
    __syncthreads();
    for (int e = tid; e < E; e += kPackThreads) s_cnt[e] = max(s_off[e + 1] - s_off[e], 0);
    __syncthreads();
  }

  // a2: exclusive scan (E <= 1024: one expert per thread)
  {
    const int c = (tid < E) ? s_cnt[tid] : 0;
    int total;
    const int ex = block_exclusive_scan(c, s_tmp, total);
    int nact;
    const int act = block_exclusive_scan((tid < E && c > 0) ? 1 : 0, s_tmp, nact);
    (void)act;
    if (p.do_pack) {
      if (tid < E) {
        s_off[tid] = ex;
        s_cur[tid] = ex;
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
    }
    __syncthreads();
  }

  if (p.do_pack) {
    // a3: stable scatter, 1024 pairs per round in pair order
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base = 0; base < pairs; base += kPackThreads) {
      const int q = base + tid;
      const bool in = q < pairs;
      const int e = in ? load_expert(p.ids, p.ids_i64, q, E) : -1;
      const bool valid = e >= 0;
      // lanes of this wave with the same key (key = E for invalid lanes)
      const int key = valid ? e : E;
      uint64_t m = __ballot(in);
#pragma unroll
      for (int b = 0; b < 11; ++b) {
        const bool bit = (key >> b) & 1;
        const uint64_t bal = __ballot(bit);
        m &= bit ? bal : ~bal;
      }
      const int rank = __popcll(m & lt_mask);
      if (in && valid && rank == 0) s_wcnt[w][e] = (uint8_t)__popcll(m);
      __syncthreads();
      if (in) {
        if (valid) {
          int pos = s_cur[e] + rank;
          for (int k = 0; k < w; ++k) pos += s_wcnt[k][e];
          p.pair_of_pos[pos] = q;
          p.weight_of_pos[pos] = load_weight(p.w, p.w_dtype, q);
          p.pos_of_pair[q] = pos;
        } else {
          p.pos_of_pair[q] = -1;
        }
      }
      __syncthreads();
      for (int x = tid; x < E; x += kPackThreads) {
        int add = 0;
        for (int k = 0; k < kPackWaves; ++k) {
          add += s_wcnt[k][x];
          s_wcnt[k][x] = 0;
        }
        s_cur[x] += add;
      }
      __syncthreads();
    }
    for (int pos = s_off[E] + tid; pos < pairs; pos += kPackThreads) {
      p.pair_of_pos[pos] = -1;
      p.weight_of_pos[pos] = 0.0f;
    }
  }

  if (!p.do_plan) return;
  if (tid == 0 && p.ctrl) {
    p.ctrl[1] = 0;  // bad stage entries
  }
  for (int i = tid; i < p.nzero; i += kPackThreads) p.zero[i] = 0;

  // expert of every kept position (binary search over the offsets)
  const int kept = s_off[E];
  for (int pos = tid; pos < kept; pos += kPackThreads) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {  // last e with s_off[e] <= pos
      const int mid = (lo + hi + 1) >> 1;
      if (s_off[mid] <= pos) lo = mid; else hi = mid - 1;
    }
    p.expert_of_pos[pos] = lo;
  }

  // a4: per pass, the row tiles of every expert's sub-span
  for (int pass = 0; pass < p.passes; ++pass) {
    const int pb = pass * p.capacity, pe = pb + p.capacity;
    int lo = 0, hi = 0, nt = 0;
    if (tid < E) {
      lo = max(s_off[tid], pb);
      hi = min(s_off[tid + 1], pe);
      nt = hi > lo ? (hi - lo + p.bm - 1) / p.bm : 0;
    }
    int total;
    const int slot0 = block_exclusive_scan(nt, s_tmp, total);
    int32_t *plan = p.plan + (int64_t)pass * (1 + 3 * p.slots);
    for (int t = 0; t < nt; ++t) {
      int32_t *d = plan + 1 + 3 * (slot0 + t);
      d[0] = tid;
      d[1] = lo - pb + t * p.bm;
      d[2] = min(p.bm, hi - lo - t * p.bm);
    }
    if (tid == 0) plan[0] = total;
  }

  // rows whose pairs were all dropped produce zeros: one row per thread to
  // find them (rare), then the row is cleared by that thread. A pack that
  // dropped nothing has no such row.
  __syncthreads();
  if (p.out && (!p.do_pack || s_dropped > 0)) {
    for (int r = tid; r < p.rows; r += kPackThreads) {
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
}

hipError_t launch_pack(const PackParams &p, hipStream_t s) {
  hipLaunchKernelGGL(pack_plan_kernel, dim3(1), dim3(kPackThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace exl3
