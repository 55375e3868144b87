// Internal launch interface between the C ABI (host.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace exl3 {

enum Epilogue { EPI_LINEAR = 0, EPI_GATEUP = 1, EPI_DOWN = 2 };

struct ProjDev {
  const int64_t *trellis;  // [S][E] device addresses
  const float *scale;      // [S][E]
  const int32_t *bits;     // [S][E]
  const uint16_t *svh;     // [E][out]
  const uint16_t *cs;      // [E][out]
  int num_stages;
};

struct GemmParams {
  ProjDev proj[2];  // GATEUP: gate, up; otherwise proj[0]
  int E, in_f, out_f;
  // A operand: rotated fp16 rows in kSigma order; row r of projection pj at
  // A + r * lda + pj * a_proj_stride (elements).
  const uint16_t *A;
  int64_t lda, a_proj_stride;
  // Work tiles. Implicit (linear): tile t = rows [t*BM, min(rows, t*BM+BM)),
  // expert 0. Plan (MoE): plan_tiles[3*t] = {expert, first row, rows}.
  int rows;
  const int32_t *plan_ntiles;
  const int32_t *plan_tiles;
  // Epilogue.
  const uint16_t *suh_down;  // GATEUP: [E][I] (down input signs)
  uint16_t *out_h;           // GATEUP: a~ [C][I]; LINEAR 16-bit output
  int out_bf16;              // LINEAR: out_h holds bf16 (else fp16)
  float *out_f32;            // DOWN: d [C][H]; LINEAR fp32 output
  int64_t ldo;
  const float *weight_of_pos;  // DOWN
  int pass_base;               // DOWN: packed position of tile row 0
  int32_t *ctrl;               // [1] bad stage entries, [2] waits that gave up
  // narrow tiles: pre-rotation sums [rows][NPROJ][out_f] and per (tile,
  // 128-column block) completion counts, zero between launches
  float *nacc;
  int32_t *ncnt;
};

// One launch for a single pass on 16-row tiles (experts_narrow_kernel):
// gate/up and down work items plus the ordered combine. gu and dn each have
// their own pre-rotation sums (nacc) and completion counts (ncnt).
struct NarrowFusedParams {
  GemmParams gu, dn;
  int32_t *blk_ready;   // [tiles][I / 128]: a~ block finished (zero at launch)
  int32_t *row_cnt;     // [rows][H / 128]: d blocks finished per output row (zero)
  const int32_t *pair_of_pos, *pos_of_pair, *total_valid;
  int rows, topk, pairs;
  void *out;            // [rows][H]
  int out_f32, out_bf16;
  int tiles;            // plan tile bound (surplus items exit)
  int g1;               // gate/up work items: tiles * 2 * (I / 64)
};

struct RotParams {
  const uint16_t *x;  // [rows][H] fp16, or bf16 if x_bf16
  int x_bf16;
  int H, topk;
  const uint16_t *suh[2];  // [E][H] per projection (suh[1] may be null)
  int nproj;
  // MoE mode: item position -> pair/expert via the pack; linear: row = item.
  const int32_t *pair_of_pos;
  const int32_t *expert_of_pos;
  const int32_t *total_valid;  // device: kept pairs
  int pass_base;
  int pairs;   // rows * topk (bound for caller-supplied metadata)
  int nitems;  // positions of this pass (upper bound) or rows
  uint16_t *xt;  // [nitems][nproj][H]
  int32_t *ctrl_clear;  // if set, block 0 zeroes ctrl[0..2] (linear calls)
  int32_t *zero;        // if set, zeroed (nzero ints) before the GEMMs run
  int nzero;
};

struct CombineParams {
  int rows, topk, H, pairs;
  const int32_t *pair_of_pos, *pos_of_pair, *total_valid;
  int pass_base, pass_end;
  const float *d;  // [C][H]
  float *yacc;     // [rows][H]
  void *out;
  int out_f32;     // 1: fp32 out, 0: 16-bit out
  int out_bf16;    // 16-bit out is bf16 (else fp16)
};

struct PackParams {
  // pack inputs (do_pack)
  const void *ids;
  int ids_i64;
  const void *w;
  int w_dtype;  // 1 f16, 2 bf16, 3 f32
  int rows, topk, E;
  // meta (written when do_pack, read otherwise)
  int32_t *count, *offset, *pair_of_pos, *pos_of_pair, *num_active, *status;
  float *weight_of_pos;
  int do_pack, do_plan;
  // plan outputs
  int32_t *expert_of_pos;
  int32_t *plan;  // per unit of `group` passes: [1 + 3 * group * slots]
  int passes, capacity, slots, bm;
  int group;      // passes per plan (tiles of pass j of a unit start j * capacity rows in)
  // unrouted rows get zero output
  void *out;
  int out_f32, H;
  int32_t *ctrl;  // [0] dropped pairs (written), [1] bad stage entries and
                  // [2] waits that gave up (both zeroed)
  int32_t *zero;  // narrow-tile completion counts, zeroed (nzero ints)
  int nzero;
  // the pack over several workgroups (many pairs): per-wave counts and
  // positions [nblk][16][E] plus nblk dropped counts (pack_scratch_ints)
  int32_t *gwc;
  int nblk;
};

hipError_t launch_gemm(int epi, const GemmParams &p, int tiles, int nblocks,
                       hipStream_t s, bool wide);
// 128-row tiles (gemm_wide.hip); called by launch_gemm.
hipError_t launch_gemm_wide(int epi, const GemmParams &p, int tiles, int nblocks,
                            hipStream_t s);
hipError_t launch_experts_narrow(const NarrowFusedParams &f, hipStream_t s);
// One pass of 128-row routed experts: gate/up and down in one launch, a
// tile's down work starting once its own gate/up items are done. `q` holds
// `slots` ints, zero at launch (slots >= plan tiles of the pass).
hipError_t launch_gemm_wide_pass(const GemmParams &gu, const GemmParams &dn, int tiles,
                                 int slots, int nb_gu, int nb_dn, int32_t *q, hipStream_t s);
// Several passes of 128-row routed experts, pipelined across launches: one
// launch runs gate/up of pass k (gu, tiles_gu), down of pass k - 1 (dn,
// tiles_dn), the rotation of pass k + 1 (rn) and the combine of pass k - 2
// (cb, one item for each of rows_cb rows); an absent part has 0 tiles /
// items. The caller
// gives each pass's x~, a~ and d the buffer of its parity.
hipError_t launch_gemm_wide_pipe(const GemmParams &gu, int tiles_gu, const GemmParams &dn,
                                 int tiles_dn, const RotParams &rn, const CombineParams &cb,
                                 int rows_cb, int nb_gu, int nb_dn, hipStream_t s);
hipError_t launch_rotate(const RotParams &p, hipStream_t s);
hipError_t launch_combine(const CombineParams &p, int npos, hipStream_t s);
hipError_t launch_combine_rows(const CombineParams &p, hipStream_t s);
hipError_t launch_pack(const PackParams &p, hipStream_t s);
// Scratch ints launch_pack needs in PackParams::gwc for a pack of `pairs`
// pairs (0: none), and its workgroup count PackParams::nblk.
size_t pack_scratch_ints(int64_t pairs, int E);
int pack_blocks(int64_t pairs);
// Pack, one-pass plan and the rotation of that pass in one launch, for calls
// where pack_rotate_fits (few pairs, one pass). rp: the pass's rotation.
bool pack_rotate_fits(int64_t pairs, int passes);
hipError_t launch_pack_rotate(const PackParams &p, const RotParams &rp, hipStream_t s);
hipError_t launch_decode_tiles(const uint16_t *words, int ntiles, int K,
                               uint16_t *out, hipStream_t s);

constexpr int kBM = 16;       // rows per narrow GEMM work tile
constexpr int kMaxTopk = 32;  // EXL3_MAX_TOPK
constexpr int kBMWide = 128;  // rows per wide GEMM work tile

}  // namespace exl3
