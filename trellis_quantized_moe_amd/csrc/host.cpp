// C ABI of the fused EXL3 routed-experts layer: host-side validation,
// workspace layout and stream-ordered launch orchestration. No call
// synchronises, allocates or frees; every argument is checked before the
// first launch (exllamav3 PR #284 "MoE: Add fused additive EXL3 kernels",
// Summary: all argument checks precede any device work; API contract: an
// exact ABI version number).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/exl3moe.h"
#include "kernels.hpp"

using namespace exl3;

namespace {

// ------------------------------------------------------------- profiling
// Optional per-launch timing into the caller's exl3_profile record (null: no
// timing): the kernel launch in the scope is bracketed by the record's next
// event pair on its stream. The library keeps no state of its own for it.
struct ProfScope {
  exl3_profile *p;
  hipStream_t s;
  int slot = -1;
  ProfScope(exl3_profile *prof, hipStream_t st, int32_t kernel_id) : p(prof), s(st) {
    if (p && p->events && p->n >= 0 && p->n < p->cap) {
      slot = p->n++;
      if (p->kernel_ids) p->kernel_ids[slot] = kernel_id;
      (void)hipEventRecord((hipEvent_t)p->events[2 * slot], s);
    }
  }
  ~ProfScope() {
    if (slot >= 0) (void)hipEventRecord((hipEvent_t)p->events[2 * slot + 1], s);
  }
};

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned_to(const void *p, unsigned a) { return ((uintptr_t)p & (a - 1)) == 0; }
// ids / route weights / metadata arrays are read element by element: their
// natural alignment is enough.
unsigned ids_align(int32_t t) { return t == EXL3_I64 ? 8u : 4u; }
unsigned w_align(int32_t t) { return t == EXL3_F32 ? 4u : 2u; }

// Device residency: the pointer must be device (or managed) memory of the
// current device. Called only after every host-side check passed.
int32_t check_device(const void *p) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return EXL3_E_DEVICE;
  hipPointerAttribute_t a;
  std::memset(&a, 0, sizeof(a));
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();
    return EXL3_E_DEVICE;
  }
  if (a.type != hipMemoryTypeDevice && a.type != hipMemoryTypeManaged) return EXL3_E_DEVICE;
  if (a.device != dev) return EXL3_E_DEVICE;
  return EXL3_OK;
}

int32_t check_features(int32_t f) {
  return (f > 0 && f <= EXL3_MAX_FEATURES && f % 128 == 0) ? EXL3_OK : EXL3_E_SHAPE;
}

int32_t check_proj_host(const exl3_proj *p) {
  if (!p) return EXL3_E_NULL;
  if (!p->trellis || !p->scale || !p->bits || !p->suh || !p->svh || !p->chscale)
    return EXL3_E_NULL;
  if (check_features(p->in_features) || check_features(p->out_features)) return EXL3_E_SHAPE;
  if (p->num_experts < 1 || p->num_experts > EXL3_MAX_EXPERTS) return EXL3_E_ARG;
  if (p->num_stages < 1 || p->num_stages > EXL3_MAX_STAGES) return EXL3_E_ARG;
  const void *ptrs[] = {p->trellis, p->scale, p->bits, p->suh, p->svh, p->chscale};
  for (const void *q : ptrs)
    if (!aligned16(q)) return EXL3_E_ALIGN;
  return EXL3_OK;
}

int32_t check_proj_device(const exl3_proj *p) {
  const void *ptrs[] = {p->trellis, p->scale, p->bits, p->suh, p->svh, p->chscale};
  for (const void *q : ptrs)
    if (int32_t s = check_device(q)) return s;
  return EXL3_OK;
}

ProjDev to_dev(const exl3_proj *p) {
  ProjDev d;
  d.trellis = p->trellis;
  d.scale = p->scale;
  d.bits = p->bits;
  d.svh = p->svh;
  d.cs = p->chscale;
  d.num_stages = p->num_stages;
  return d;
}

bool out_dtype_ok(int32_t t) { return t == EXL3_F16 || t == EXL3_BF16 || t == EXL3_F32; }
bool x_dtype_ok(int32_t t) { return t == EXL3_F16 || t == EXL3_BF16; }

// Tile shape choice (never changes results: both tile shapes run the same
// per-element MFMA chain and the same epilogue code). Wide 128-row tiles pay
// off once expert spans average 64+ rows; otherwise 16-row tiles keep the
// machine full at decode sizes.
bool moe_wide(int64_t pairs, int E) { return pairs >= 64 * (int64_t)E; }
bool linear_wide(int rows, int out) {
  return (int64_t)((rows + kBMWide - 1) / kBMWide) * ((out + 255) / 256) >= 256;
}

struct MoeLayout {
  size_t ctrl, count, offset, pair_of_pos, weight_of_pos, pos_of_pair, num_active, status;
  size_t expert_of_pos, plan, xt, at, d, yacc, nacc, ncnt, pack, total;
  int passes, slots, cap, ncnt_ints;
  // A launch unit is `group` consecutive passes (on the pipelined path
  // about half the passes, at most 8; else 1): one plan, one buffer set of
  // gcap = group * cap rows, planned as one position range.
  int group, units, gcap;
  // fused: a single pass on 16-row tiles runs its GEMMs and combine in one
  // launch (experts_narrow_kernel), with separate sums and counts for the
  // concurrent gate/up and down items
  bool wide, pipe, fused;
  size_t xt_bytes, at_bytes, d_bytes;  // one buffer each (pipe: two of each)
};

MoeLayout moe_layout(int32_t rows, int32_t topk, int32_t E, int32_t H, int32_t I,
                     int32_t capacity) {
  MoeLayout L{};
  const int64_t P = (int64_t)rows * topk;
  const int64_t C = std::max<int64_t>(1, std::min<int64_t>(capacity, std::max<int64_t>(P, 1)));
  L.cap = (int)C;
  L.passes = P > 0 ? (int)((P + C - 1) / C) : 0;
  L.slots = (int)(std::min<int64_t>(E, C) + (C + kBM - 1) / kBM);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  L.ctrl = take(256);
  L.count = take(4 * (size_t)E);
  L.offset = take(4 * (size_t)(E + 1));
  L.pair_of_pos = take(4 * (size_t)P);
  L.weight_of_pos = take(4 * (size_t)P);
  L.pos_of_pair = take(4 * (size_t)P);
  L.num_active = take(4);
  L.status = take(4);
  L.expert_of_pos = take(4 * (size_t)P);
  L.wide = P > 0 && moe_wide(P, E);
  // 128-row tiles over several passes run pipelined across launches, with
  // two buffers (by unit parity) of x~, a~ and d. A launch unit holds about
  // half the passes (two units), at most 8: more work per launch to spread
  // over the CUs and fewer launch tails, for buffers of group * capacity
  // rows (on the 3072-row prefill at capacity 2048, 12 passes: 4.37 / 4.20
  // / 4.05 ms per layer with 1 / 2 / 4 passes per unit, and 6 passes per
  // unit faster again; 1.3 GB of buffers at 6)
  L.pipe = L.wide && L.passes >= 2;
  L.group = !L.pipe ? 1 : std::min(8, (L.passes + 1) / 2);
  L.units = (L.passes + L.group - 1) / L.group;
  L.gcap = L.group * L.cap;
  L.plan = take(4 * (size_t)L.units * (1 + 3 * (size_t)L.group * L.slots));
  const size_t nbuf = L.pipe ? 2 : 1;
  const size_t G = (size_t)L.gcap;
  L.xt_bytes = align_up(2 * G * 2 * H);
  L.at_bytes = align_up(2 * G * I);
  L.d_bytes = align_up(4 * G * H);
  L.xt = take(nbuf * L.xt_bytes);
  L.at = take(nbuf * L.at_bytes);
  L.d = take(nbuf * L.d_bytes);
  L.yacc = take(4 * (size_t)rows * H);
  // 16-row tiles: per (tile, 128-column block) completion counts; 128-row
  // tiles in one pass: per tile, the finished gate/up items. Fused: gate/up
  // counts [slots][I/128], down counts [slots][H/128], finished a~ blocks
  // [slots][I/128], d blocks per output row [rows][H/128], and the
  // pre-rotation sums of gate/up [C][2I] and of down [C][H] side by side.
  L.fused = P > 0 && !L.wide && L.passes == 1;
  L.ncnt_ints = L.fused  ? L.slots * (2 * (I / 128) + H / 128) + rows * (H / 128)
                : L.pipe ? 0
                : L.wide ? L.slots
                         : L.slots * (std::max(I, H) / 128);
  L.nacc = take(L.wide     ? 0
                : L.fused ? 4 * (size_t)C * (2 * I + H)
                          : 4 * (size_t)C * std::max(2 * I, H));
  L.ncnt = take(4 * (size_t)L.ncnt_ints);
  L.pack = take(4 * pack_scratch_ints(P, E));
  L.total = o;
  return L;
}


template <typename T>
T *at(void *ws, size_t off) {
  return (T *)((char *)ws + off);
}

int32_t validate_moe_common(const uint16_t *x, int32_t x_dtype, int32_t rows, int32_t topk,
                            const exl3_proj *gate, const exl3_proj *up,
                            const exl3_proj *down, void *out, int32_t out_dtype,
                            int32_t capacity, void *ws) {
  if (rows < 0) return EXL3_E_ARG;
  if (!x || !out || !ws) return EXL3_E_NULL;
  for (const exl3_proj *p : {gate, up, down})
    if (int32_t s = check_proj_host(p)) return s;
  if (!x_dtype_ok(x_dtype) || !out_dtype_ok(out_dtype)) return EXL3_E_DTYPE;
  if (topk < 1 || topk > EXL3_MAX_TOPK) return EXL3_E_ARG;
  if (capacity < 1) return EXL3_E_ARG;
  const int H = gate->in_features, I = gate->out_features, E = gate->num_experts;
  if (up->in_features != H || up->out_features != I || down->in_features != I ||
      down->out_features != H)
    return EXL3_E_SHAPE;
  if (up->num_experts != E || down->num_experts != E) return EXL3_E_SHAPE;
  if ((int64_t)rows * topk > (int64_t)1 << 30) return EXL3_E_ARG;
  if (!aligned16(x) || !aligned16(out) || !aligned16(ws)) return EXL3_E_ALIGN;
  return EXL3_OK;
}

int32_t validate_moe_device(const uint16_t *x, const exl3_proj *gate,
                            const exl3_proj *up, const exl3_proj *down, void *out,
                            void *ws) {
  for (const void *q : {(const void *)x, (const void *)out, (const void *)ws})
    if (q && check_device(q)) return EXL3_E_DEVICE;
  for (const exl3_proj *p : {gate, up, down})
    if (int32_t s = check_proj_device(p)) return s;
  return EXL3_OK;
}

// Passes over the packed positions: rotate, gate/up, down, combine.
int32_t run_experts(const uint16_t *x, int32_t x_dtype, int32_t rows, int32_t topk,
                    const exl3_proj *gate, const exl3_proj *up,
                    const exl3_proj *down, void *out, int32_t out_dtype,
                    const MoeLayout &L, void *ws, const int32_t *pair_of_pos,
                    const int32_t *pos_of_pair, const float *weight_of_pos,
                    const int32_t *offset, hipStream_t st, exl3_profile *prof,
                    const PackParams *fused_pack = nullptr) {
  const int H = gate->in_features, I = gate->out_features, E = gate->num_experts;
  const int64_t P = (int64_t)rows * topk;
  const int32_t *total_valid = offset + E;
  int32_t *ctrl = at<int32_t>(ws, L.ctrl);
  const bool wide = L.wide;
  const int bm = wide ? kBMWide : kBM;
  // Launch units of L.group passes (see MoeLayout): u covers packed
  // positions [u * gcap, (u + 1) * gcap), planned as one range.
  auto npos_of = [&](int u) {
    return (int)std::min<int64_t>(L.gcap, P - (int64_t)u * L.gcap);
  };
  auto tiles_of = [&](int u) {  // bound on the unit's plan tiles
    // the unit's positions are planned as one range: full tiles, plus at
    // most one partial tile per expert present
    const int64_t first = (int64_t)u * L.group * L.cap;
    const int np = (int)std::min<int64_t>((int64_t)L.group * L.cap, P - first);
    return std::min(E, np) + (np + bm - 1) / bm;
  };
  auto plan_of = [&](int u) {
    return at<int32_t>(ws, L.plan) + (size_t)u * (1 + 3 * (size_t)L.group * L.slots);
  };
  uint16_t *xt0 = at<uint16_t>(ws, L.xt), *at0 = at<uint16_t>(ws, L.at);
  float *d0 = at<float>(ws, L.d);
  auto xt_buf = [&](int b) { return (uint16_t *)((char *)xt0 + (size_t)b * L.xt_bytes); };
  auto at_buf = [&](int b) { return (uint16_t *)((char *)at0 + (size_t)b * L.at_bytes); };
  auto d_buf = [&](int b) { return (float *)((char *)d0 + (size_t)b * L.d_bytes); };
  // rotation of the inputs of one pass into x~ buffer b
  auto rot_params = [&](int pass, int b) {
    RotParams rp{};
    rp.x = x;
    rp.x_bf16 = x_dtype == EXL3_BF16;
    rp.H = H;
    rp.topk = topk;
    rp.suh[0] = gate->suh;
    rp.suh[1] = up->suh;
    rp.nproj = 2;
    rp.pair_of_pos = pair_of_pos;
    rp.expert_of_pos = at<int32_t>(ws, L.expert_of_pos);
    rp.total_valid = total_valid;
    rp.pass_base = pass * L.gcap;
    rp.pairs = (int)P;
    rp.nitems = npos_of(pass);
    rp.xt = xt_buf(b);
    rp.ctrl_clear = nullptr;
    return rp;
  };
  // gate/up of one pass: x~ buffer b in, a~ buffer b out
  auto gu_params = [&](int pass, int b) {
    const int32_t *plan = plan_of(pass);
    GemmParams g{};
    g.proj[0] = to_dev(gate);
    g.proj[1] = to_dev(up);
    g.E = E;
    g.in_f = H;
    g.out_f = I;
    g.A = xt_buf(b);
    g.lda = 2 * (int64_t)H;
    g.a_proj_stride = H;
    g.plan_ntiles = plan;
    g.plan_tiles = plan + 1;
    g.suh_down = down->suh;
    g.out_h = at_buf(b);
    g.ldo = I;
    g.ctrl = ctrl;
    g.nacc = at<float>(ws, L.nacc);
    g.ncnt = at<int32_t>(ws, L.ncnt);
    return g;
  };
  // down of one pass: a~ buffer b in, d buffer b out
  auto dn_params = [&](int pass, int b) {
    const int32_t *plan = plan_of(pass);
    GemmParams dn{};
    dn.proj[0] = to_dev(down);
    dn.E = E;
    dn.in_f = I;
    dn.out_f = H;
    dn.A = at_buf(b);
    dn.lda = I;
    dn.plan_ntiles = plan;
    dn.plan_tiles = plan + 1;
    dn.out_f32 = d_buf(b);
    dn.ldo = H;
    dn.weight_of_pos = weight_of_pos;
    dn.pass_base = pass * L.gcap;
    dn.ctrl = ctrl;
    dn.nacc = at<float>(ws, L.nacc);
    dn.ncnt = at<int32_t>(ws, L.ncnt);
    return dn;
  };
  // combine of one pass: d buffer b in
  auto cb_params = [&](int pass, int b) {
    CombineParams cp{};
    cp.rows = rows;
    cp.topk = topk;
    cp.H = H;
    cp.pairs = (int)P;
    cp.pair_of_pos = pair_of_pos;
    cp.pos_of_pair = pos_of_pair;
    cp.total_valid = total_valid;
    cp.pass_base = pass * L.gcap;
    cp.pass_end = pass * L.gcap + L.gcap;
    cp.d = d_buf(b);
    cp.yacc = at<float>(ws, L.yacc);
    cp.out = out;
    cp.out_f32 = out_dtype == EXL3_F32;
    cp.out_bf16 = out_dtype == EXL3_BF16;
    return cp;
  };

  if (L.pipe) {
    // launch k: gate/up of unit k, down of k - 1, rotation of k + 1, combine
    // of k - 2; unit q uses the buffers of parity q & 1
    {
      ProfScope ps(prof, st, EXL3_K_ROTATE);
      if (launch_rotate(rot_params(0, 0), st) != hipSuccess) return EXL3_E_LAUNCH;
    }
    for (int k = 0; k <= L.units + 1; ++k) {
      const bool has_gu = k < L.units, has_dn = k >= 1 && k <= L.units;
      const bool has_rn = k + 1 < L.units, has_cb = k >= 2;
      const GemmParams g = has_gu ? gu_params(k, k & 1) : GemmParams{};
      const GemmParams dn = has_dn ? dn_params(k - 1, (k - 1) & 1) : GemmParams{};
      const RotParams rn = has_rn ? rot_params(k + 1, (k + 1) & 1) : RotParams{};
      const CombineParams cp = has_cb ? cb_params(k - 2, k & 1) : CombineParams{};
      ProfScope ps(prof, st, EXL3_K_EXPERTS);
      if (launch_gemm_wide_pipe(g, has_gu ? tiles_of(k) : 0, dn, has_dn ? tiles_of(k - 1) : 0, rn,
                                cp, has_cb ? rows : 0, I / 128, (H + 255) / 256,
                                st) != hipSuccess)
        return EXL3_E_LAUNCH;
    }
    return EXL3_OK;
  }

  if (L.fused) {
    // launch 1: pack, plan and rotation in one launch (few pairs) or the
    // rotation after the pack already enqueued; it also zeroes the counts.
    // launch 2: gate/up, down and combine.
    if (fused_pack) {
      ProfScope ps(prof, st, EXL3_K_PACK);
      if (launch_pack_rotate(*fused_pack, rot_params(0, 0), st) != hipSuccess)
        return EXL3_E_LAUNCH;
    } else {
      ProfScope ps(prof, st, EXL3_K_ROTATE);
      if (launch_rotate(rot_params(0, 0), st) != hipSuccess) return EXL3_E_LAUNCH;
    }
    NarrowFusedParams f{};
    f.gu = gu_params(0, 0);
    f.dn = dn_params(0, 0);
    const int slots = L.slots;
    int32_t *cnt = at<int32_t>(ws, L.ncnt);
    float *nacc = at<float>(ws, L.nacc);
    f.gu.nacc = nacc;
    f.dn.nacc = nacc + (size_t)L.cap * 2 * I;
    f.gu.ncnt = cnt;
    f.dn.ncnt = cnt + (size_t)slots * (I / 128);
    f.blk_ready = f.dn.ncnt + (size_t)slots * (H / 128);
    f.row_cnt = f.blk_ready + (size_t)slots * (I / 128);
    f.pair_of_pos = pair_of_pos;
    f.pos_of_pair = pos_of_pair;
    f.total_valid = total_valid;
    f.rows = rows;
    f.topk = topk;
    f.pairs = (int)P;
    f.out = out;
    f.out_f32 = out_dtype == EXL3_F32;
    f.out_bf16 = out_dtype == EXL3_BF16;
    f.tiles = tiles_of(0);
    f.g1 = f.tiles * 2 * (I / 64);
    ProfScope ps(prof, st, EXL3_K_EXPERTS);
    return launch_experts_narrow(f, st) == hipSuccess ? EXL3_OK : EXL3_E_LAUNCH;
  }

  // otherwise: pass by pass, one pass per unit (128-row tiles: a single pass)
  for (int pass = 0; pass < L.units; ++pass) {
    const int npos = npos_of(pass);
    const int tiles = tiles_of(pass);
    if (fused_pack && pass == 0) {  // pack, plan and this rotation in one launch
      ProfScope ps(prof, st, EXL3_K_PACK);
      if (launch_pack_rotate(*fused_pack, rot_params(0, 0), st) != hipSuccess)
        return EXL3_E_LAUNCH;
    } else {
      RotParams rp = rot_params(pass, 0);
      if (wide) {  // the pass kernel's per-tile counts start at zero
        rp.zero = at<int32_t>(ws, L.ncnt);
        rp.nzero = L.ncnt_ints;
      }
      ProfScope ps(prof, st, EXL3_K_ROTATE);
      if (launch_rotate(rp, st) != hipSuccess) return EXL3_E_LAUNCH;
    }
    const GemmParams g = gu_params(pass, 0);
    if (!wide) {
      ProfScope ps(prof, st, EXL3_K_GATEUP);
      if (launch_gemm(EPI_GATEUP, g, tiles, I / 128, st, wide) != hipSuccess) return EXL3_E_LAUNCH;
    }
    const GemmParams dn = dn_params(pass, 0);
    if (wide) {
      ProfScope ps(prof, st, EXL3_K_EXPERTS);
      if (launch_gemm_wide_pass(g, dn, tiles, L.slots, I / 128, (H + 255) / 256,
                                at<int32_t>(ws, L.ncnt), st) != hipSuccess)
        return EXL3_E_LAUNCH;
    } else {
      ProfScope ps(prof, st, EXL3_K_DOWN);
      if (launch_gemm(EPI_DOWN, dn, tiles, H / 128, st, wide) != hipSuccess) return EXL3_E_LAUNCH;
    }
    const CombineParams cp = cb_params(pass, 0);
    {
      ProfScope ps(prof, st, EXL3_K_COMBINE);
      const hipError_t err =
          (L.passes == 1) ? launch_combine_rows(cp, st) : launch_combine(cp, npos, st);
      if (err != hipSuccess) return EXL3_E_LAUNCH;
    }
  }
  return EXL3_OK;
}

// Linear workspace: 256 B control word block, the rotated rows, and for
// 16-row tiles the pre-rotation sums and completion counts.
struct LinLayout {
  size_t xt, nacc, ncnt, total;
  int ncnt_ints;
  bool wide;
};
LinLayout lin_layout(int32_t rows, int32_t in_features, int32_t out_features) {
  LinLayout L{};
  L.wide = linear_wide(rows, out_features);
  L.xt = 256;
  L.nacc = L.xt + align_up(2 * (size_t)rows * in_features);
  const size_t nacc_bytes = L.wide ? 0 : 4 * (size_t)rows * out_features;
  L.ncnt = L.nacc + align_up(nacc_bytes);
  L.ncnt_ints = L.wide ? 0 : ((rows + kBM - 1) / kBM) * (out_features / 128);
  L.total = L.ncnt + align_up(4 * (size_t)L.ncnt_ints);
  return L;
}

}  // namespace

extern "C" {

int32_t exl3_abi_version(void) { return EXL3_ABI_VERSION; }

const char *exl3_status_string(int32_t s) {
  switch (s) {
    case EXL3_OK: return "ok";
    case EXL3_E_NULL: return "null pointer";
    case EXL3_E_DTYPE: return "unsupported dtype";
    case EXL3_E_SHAPE: return "bad or inconsistent shape (features must be positive multiples of 128)";
    case EXL3_E_ALIGN: return "pointer not 16-byte aligned";
    case EXL3_E_DEVICE: return "pointer not on the current HIP device (or no device)";
    case EXL3_E_WORKSPACE: return "workspace missing or too small";
    case EXL3_E_ARG: return "argument out of range";
    case EXL3_E_LAUNCH: return "kernel launch failed";
    case EXL3_E_SCRATCH:
      return "call needs a larger workspace than the static scratch of exl3_moe_forward_static "
             "(EXL3_STATIC_SCRATCH_BYTES = 32 MiB); use exl3_moe_forward with a workspace";
    default: return "unknown status";
  }
}

size_t exl3_linear_workspace_size(int32_t rows, int32_t in_features, int32_t out_features) {
  if (rows < 0 || in_features < 0 || out_features < 0) return 0;
  return lin_layout(rows, in_features, out_features).total;
}

int32_t exl3_linear(const uint16_t *x, int32_t x_dtype, int32_t rows, const exl3_proj *proj,
                    void *out, int32_t out_dtype, void *ws, size_t ws_bytes, void *stream,
                    exl3_profile *prof) {
  if (rows < 0) return EXL3_E_ARG;
  if (rows == 0) return EXL3_OK;
  if (!x || !out || !ws) return EXL3_E_NULL;
  if (int32_t s = check_proj_host(proj)) return s;
  if (proj->num_experts != 1) return EXL3_E_ARG;
  if (!x_dtype_ok(x_dtype) || !out_dtype_ok(out_dtype)) return EXL3_E_DTYPE;
  if (!aligned16(x) || !aligned16(out) || !aligned16(ws)) return EXL3_E_ALIGN;
  if (ws_bytes < exl3_linear_workspace_size(rows, proj->in_features, proj->out_features))
    return EXL3_E_WORKSPACE;
  for (const void *q : {(const void *)x, (const void *)out, (const void *)ws})
    if (int32_t s = check_device(q)) return s;
  if (int32_t s = check_proj_device(proj)) return s;

  hipStream_t st = (hipStream_t)stream;
  const LinLayout LL = lin_layout(rows, proj->in_features, proj->out_features);
  int32_t *ctrl = (int32_t *)ws;
  uint16_t *xt = at<uint16_t>(ws, LL.xt);
  RotParams rp{};
  rp.x = x;
  rp.x_bf16 = x_dtype == EXL3_BF16;
  rp.H = proj->in_features;
  rp.suh[0] = proj->suh;
  rp.nproj = 1;
  rp.nitems = rows;
  rp.xt = xt;
  rp.ctrl_clear = ctrl;
  rp.zero = LL.ncnt_ints ? at<int32_t>(ws, LL.ncnt) : nullptr;
  rp.nzero = LL.ncnt_ints;
  {
    ProfScope ps(prof, st, EXL3_K_ROTATE);
    if (launch_rotate(rp, st) != hipSuccess) return EXL3_E_LAUNCH;
  }

  GemmParams g{};
  g.proj[0] = to_dev(proj);
  g.E = 1;
  g.in_f = proj->in_features;
  g.out_f = proj->out_features;
  g.A = xt;
  g.lda = proj->in_features;
  g.rows = rows;
  g.ldo = proj->out_features;
  if (out_dtype == EXL3_F32) g.out_f32 = (float *)out;
  else g.out_h = (uint16_t *)out;
  g.out_bf16 = out_dtype == EXL3_BF16;
  g.ctrl = ctrl;
  g.nacc = at<float>(ws, LL.nacc);
  g.ncnt = at<int32_t>(ws, LL.ncnt);
  ProfScope ps(prof, st, EXL3_K_LINEAR);
  const int fo = proj->out_features;
  const bool wide = LL.wide;
  const hipError_t le =
      wide ? launch_gemm(EPI_LINEAR, g, (rows + kBMWide - 1) / kBMWide, (fo + 255) / 256, st, true)
           : launch_gemm(EPI_LINEAR, g, (rows + kBM - 1) / kBM, fo / 128, st, false);
  if (le != hipSuccess) return EXL3_E_LAUNCH;
  return EXL3_OK;
}

int32_t exl3_moe_layout(int32_t rows, int32_t topk, int32_t num_experts, int32_t hidden,
                        int32_t intermediate, int32_t capacity, exl3_moe_layout_t *out) {
  if (!out) return EXL3_E_NULL;
  if (rows < 0 || topk < 1 || topk > EXL3_MAX_TOPK || capacity < 1 || num_experts < 1 ||
      num_experts > EXL3_MAX_EXPERTS)
    return EXL3_E_ARG;
  if (check_features(hidden) || check_features(intermediate)) return EXL3_E_SHAPE;
  const MoeLayout L = moe_layout(rows, topk, num_experts, hidden, intermediate, capacity);
  out->ctrl = L.ctrl;
  out->meta = L.count;
  out->expert_of_pos = L.expert_of_pos;
  out->plan = L.plan;
  out->xt = L.xt;
  out->at = L.at;
  out->d = L.d;
  out->yacc = L.yacc;
  out->total = L.total;
  out->passes = L.passes;
  out->plan_slots = L.slots;
  out->plan_group = L.group;
  return EXL3_OK;
}

size_t exl3_moe_workspace_size(int32_t rows, int32_t topk, int32_t num_experts, int32_t hidden,
                               int32_t intermediate, int32_t capacity) {
  exl3_moe_layout_t l;
  if (exl3_moe_layout(rows, topk, num_experts, hidden, intermediate, capacity, &l) != EXL3_OK)
    return 0;
  return l.total;
}

int32_t exl3_route_pack(const void *ids, int32_t ids_dtype, const void *w, int32_t w_dtype,
                        int32_t rows, int32_t topk, int32_t num_experts,
                        const exl3_route_meta *meta, void *stream, exl3_profile *prof) {
  if (rows < 0) return EXL3_E_ARG;
  if (!meta) return EXL3_E_NULL;
  if (topk < 1 || topk > EXL3_MAX_TOPK || num_experts < 1 || num_experts > EXL3_MAX_EXPERTS)
    return EXL3_E_ARG;
  if ((int64_t)rows * topk > (int64_t)1 << 30) return EXL3_E_ARG;
  if (rows == 0) return EXL3_OK;
  if (!ids || !w) return EXL3_E_NULL;
  if (ids_dtype != EXL3_I32 && ids_dtype != EXL3_I64) return EXL3_E_DTYPE;
  if (w_dtype != EXL3_F16 && w_dtype != EXL3_BF16 && w_dtype != EXL3_F32) return EXL3_E_DTYPE;
  void *mp[] = {meta->expert_count, meta->expert_offset, meta->pair_of_pos,
                meta->weight_of_pos, meta->pos_of_pair, meta->num_active, meta->status};
  for (void *q : mp)
    if (!q) return EXL3_E_NULL;
  if (!aligned_to(ids, ids_align(ids_dtype)) || !aligned_to(w, w_align(w_dtype)))
    return EXL3_E_ALIGN;
  for (void *q : mp)
    if (!aligned_to(q, 4)) return EXL3_E_ALIGN;
  for (const void *q : {ids, w})
    if (int32_t s = check_device(q)) return s;
  for (void *q : mp)
    if (int32_t s = check_device(q)) return s;

  PackParams p{};
  p.ids = ids;
  p.ids_i64 = ids_dtype == EXL3_I64;
  p.w = w;
  p.w_dtype = w_dtype == EXL3_F16 ? 1 : w_dtype == EXL3_BF16 ? 2 : 3;
  p.rows = rows;
  p.topk = topk;
  p.E = num_experts;
  p.count = meta->expert_count;
  p.offset = meta->expert_offset;
  p.pair_of_pos = meta->pair_of_pos;
  p.weight_of_pos = meta->weight_of_pos;
  p.pos_of_pair = meta->pos_of_pair;
  p.num_active = meta->num_active;
  p.status = meta->status;
  p.do_pack = 1;
  p.do_plan = 0;
  ProfScope ps(prof, (hipStream_t)stream, EXL3_K_PACK);
  return launch_pack(p, (hipStream_t)stream) == hipSuccess ? EXL3_OK : EXL3_E_LAUNCH;
}

}  // extern "C"

namespace {

// exl3_moe_forward with the workspace either the caller's (checked like any
// other argument) or the library's own static scratch (ws_is_scratch: its
// address comes from hipGetSymbolAddress, not from an allocation, so it is
// not given to hipPointerGetAttributes). ws_bytes of 0 with ws_is_scratch
// means "the call does not fit the scratch".
int32_t moe_forward_impl(const uint16_t *x, int32_t x_dtype, int32_t rows, const void *ids,
                         int32_t ids_dtype, const void *w, int32_t w_dtype, int32_t topk,
                         const exl3_proj *gate, const exl3_proj *up, const exl3_proj *down,
                         void *out, int32_t out_dtype, int32_t capacity, void *ws,
                         size_t ws_bytes, void *stream, bool ws_is_scratch,
                         exl3_profile *prof) {
  if (rows < 0) return EXL3_E_ARG;
  if (rows == 0) return EXL3_OK;
  if (int32_t s = validate_moe_common(x, x_dtype, rows, topk, gate, up, down, out, out_dtype,
                                      capacity, ws))
    return s;
  if (!ids || !w) return EXL3_E_NULL;
  if (ids_dtype != EXL3_I32 && ids_dtype != EXL3_I64) return EXL3_E_DTYPE;
  if (w_dtype != EXL3_F16 && w_dtype != EXL3_BF16 && w_dtype != EXL3_F32) return EXL3_E_DTYPE;
  if (!aligned_to(ids, ids_align(ids_dtype)) || !aligned_to(w, w_align(w_dtype)))
    return EXL3_E_ALIGN;
  const int H = gate->in_features, I = gate->out_features, E = gate->num_experts;
  const MoeLayout L = moe_layout(rows, topk, E, H, I, capacity);
  if (ws_bytes < L.total) return ws_is_scratch ? EXL3_E_SCRATCH : EXL3_E_WORKSPACE;
  if (int32_t s = validate_moe_device(x, gate, up, down, out, ws_is_scratch ? nullptr : ws))
    return s;
  for (const void *q : {ids, w})
    if (int32_t s = check_device(q)) return s;

  hipStream_t st = (hipStream_t)stream;
  PackParams p{};
  p.ids = ids;
  p.ids_i64 = ids_dtype == EXL3_I64;
  p.w = w;
  p.w_dtype = w_dtype == EXL3_F16 ? 1 : w_dtype == EXL3_BF16 ? 2 : 3;
  p.rows = rows;
  p.topk = topk;
  p.E = E;
  p.count = at<int32_t>(ws, L.count);
  p.offset = at<int32_t>(ws, L.offset);
  p.pair_of_pos = at<int32_t>(ws, L.pair_of_pos);
  p.weight_of_pos = at<float>(ws, L.weight_of_pos);
  p.pos_of_pair = at<int32_t>(ws, L.pos_of_pair);
  p.num_active = at<int32_t>(ws, L.num_active);
  p.status = at<int32_t>(ws, L.status);
  p.do_pack = 1;
  p.do_plan = 1;
  p.expert_of_pos = at<int32_t>(ws, L.expert_of_pos);
  p.plan = at<int32_t>(ws, L.plan);
  p.passes = L.passes;
  p.capacity = L.cap;
  p.slots = L.slots;
  p.group = L.group;
  p.bm = moe_wide((int64_t)rows * topk, E) ? kBMWide : kBM;
  p.out = out;
  p.out_f32 = out_dtype == EXL3_F32;
  p.H = H;
  p.ctrl = at<int32_t>(ws, L.ctrl);
  p.zero = L.ncnt_ints ? at<int32_t>(ws, L.ncnt) : nullptr;
  p.nzero = L.ncnt_ints;
  p.gwc = at<int32_t>(ws, L.pack);
  p.nblk = pack_blocks((int64_t)rows * topk);
  // few pairs in one pass: the pack runs inside the first rotation's launch
  const bool fuse = !L.pipe && pack_rotate_fits((int64_t)rows * topk, L.passes);
  if (!fuse) {
    ProfScope ps(prof, st, EXL3_K_PACK);
    if (launch_pack(p, st) != hipSuccess) return EXL3_E_LAUNCH;
  }
  return run_experts(x, x_dtype, rows, topk, gate, up, down, out, out_dtype, L, ws, p.pair_of_pos,
                     p.pos_of_pair, p.weight_of_pos, p.offset, st, prof, fuse ? &p : nullptr);
}

// ------------------------------------------------ static scratch workspace
// The workspace of exl3_moe_forward_static: a file-scope device array, so
// calls through that entry point allocate nothing. The runtime gives every
// device that loads this library its own copy. In host code `scratch` names
// a host-side stand-in, not device memory: its device address is taken once
// per device with hipGetSymbolAddress (on that device's first call, with the
// device current) and only that address is passed on.
static __device__ __align__(256) char scratch[EXL3_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void *g_scratch_ptr[kMaxDevices];

// Device address of this device's scratch array, nullptr on failure.
void *scratch_ptr(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_scratch_once[dev], [dev] {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();
      ptr = nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  });
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int32_t exl3_moe_forward(const uint16_t *x, int32_t x_dtype, int32_t rows, const void *ids,
                         int32_t ids_dtype,
                         const void *w, int32_t w_dtype, int32_t topk, const exl3_proj *gate,
                         const exl3_proj *up, const exl3_proj *down, void *out,
                         int32_t out_dtype, int32_t capacity, int32_t num_active_hint,
                         void *ws, size_t ws_bytes, void *stream, exl3_profile *prof) {
  (void)num_active_hint;
  return moe_forward_impl(x, x_dtype, rows, ids, ids_dtype, w, w_dtype, topk, gate, up, down,
                          out, out_dtype, capacity, ws, ws_bytes, stream, false, prof);
}

int32_t exl3_moe_forward_static(const uint16_t *x, int32_t x_dtype, int32_t rows,
                                const void *ids, int32_t ids_dtype, const void *w,
                                int32_t w_dtype, int32_t topk, const exl3_proj *gate,
                                const exl3_proj *up, const exl3_proj *down, void *out,
                                int32_t out_dtype, int32_t capacity, int32_t num_active_hint,
                                void *stream, exl3_profile *prof) {
  (void)num_active_hint;
  if (rows < 0) return EXL3_E_ARG;
  if (rows == 0) return EXL3_OK;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return EXL3_E_DEVICE;
  void *ws = scratch_ptr(dev);
  if (!ws) return EXL3_E_DEVICE;
  return moe_forward_impl(x, x_dtype, rows, ids, ids_dtype, w, w_dtype, topk, gate, up, down,
                          out, out_dtype, capacity, ws, EXL3_STATIC_SCRATCH_BYTES, stream,
                          true, prof);
}

int32_t exl3_moe_additive(const uint16_t *x, int32_t x_dtype, int32_t rows, int32_t topk,
                          const exl3_route_meta *meta, const exl3_proj *gate,
                          const exl3_proj *up, const exl3_proj *down, void *out,
                          int32_t out_dtype, int32_t capacity, int32_t num_active_hint,
                          void *ws, size_t ws_bytes, void *stream, exl3_profile *prof) {
  (void)num_active_hint;
  if (rows < 0) return EXL3_E_ARG;
  if (rows == 0) return EXL3_OK;
  if (int32_t s = validate_moe_common(x, x_dtype, rows, topk, gate, up, down, out, out_dtype,
                                      capacity, ws))
    return s;
  if (!meta) return EXL3_E_NULL;
  void *mp[] = {meta->expert_offset, meta->pair_of_pos, meta->weight_of_pos, meta->pos_of_pair};
  for (void *q : mp)
    if (!q) return EXL3_E_NULL;
  for (void *q : mp)
    if (!aligned_to(q, 4)) return EXL3_E_ALIGN;
  const int H = gate->in_features, I = gate->out_features, E = gate->num_experts;
  const MoeLayout L = moe_layout(rows, topk, E, H, I, capacity);
  if (ws_bytes < L.total) return EXL3_E_WORKSPACE;
  if (int32_t s = validate_moe_device(x, gate, up, down, out, ws)) return s;
  for (void *q : mp)
    if (int32_t s = check_device(q)) return s;

  hipStream_t st = (hipStream_t)stream;
  PackParams p{};
  p.rows = rows;
  p.topk = topk;
  p.E = E;
  p.offset = meta->expert_offset;
  p.pos_of_pair = meta->pos_of_pair;
  p.do_pack = 0;
  p.do_plan = 1;
  p.expert_of_pos = at<int32_t>(ws, L.expert_of_pos);
  p.plan = at<int32_t>(ws, L.plan);
  p.passes = L.passes;
  p.capacity = L.cap;
  p.slots = L.slots;
  p.group = L.group;
  p.bm = moe_wide((int64_t)rows * topk, E) ? kBMWide : kBM;
  p.out = out;
  p.out_f32 = out_dtype == EXL3_F32;
  p.H = H;
  p.ctrl = at<int32_t>(ws, L.ctrl);
  p.zero = L.ncnt_ints ? at<int32_t>(ws, L.ncnt) : nullptr;
  p.nzero = L.ncnt_ints;
  {
    ProfScope ps(prof, st, EXL3_K_PACK);
    if (launch_pack(p, st) != hipSuccess) return EXL3_E_LAUNCH;
  }
  return run_experts(x, x_dtype, rows, topk, gate, up, down, out, out_dtype, L, ws,
                     meta->pair_of_pos,
                     meta->pos_of_pair, meta->weight_of_pos, meta->expert_offset, st, prof);
}

int32_t exl3_decode_tiles(const uint16_t *words, int32_t ntiles, int32_t K, uint16_t *out,
                          void *stream, exl3_profile *prof) {
  if (ntiles < 0 || K < 2 || K > 8) return EXL3_E_ARG;
  if (ntiles == 0) return EXL3_OK;
  if (!words || !out) return EXL3_E_NULL;
  if (!aligned16(words) || !aligned16(out)) return EXL3_E_ALIGN;
  for (const void *q : {(const void *)words, (const void *)out})
    if (int32_t s = check_device(q)) return s;
  ProfScope ps(prof, (hipStream_t)stream, EXL3_K_DECODE);
  return launch_decode_tiles(words, ntiles, K, out, (hipStream_t)stream) == hipSuccess
             ? EXL3_OK
             : EXL3_E_LAUNCH;
}

int32_t exl3_events_create(int32_t count, void **events) {
  if (count < 0) return EXL3_E_ARG;
  if (count > 0 && !events) return EXL3_E_NULL;
  for (int i = 0; i < count; ++i) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) {
      for (int j = 0; j < i; ++j) (void)hipEventDestroy((hipEvent_t)events[j]);
      for (int j = 0; j < i; ++j) events[j] = nullptr;
      return EXL3_E_DEVICE;
    }
    events[i] = (void *)e;
  }
  return EXL3_OK;
}

int32_t exl3_events_destroy(int32_t count, void **events) {
  if (count < 0) return EXL3_E_ARG;
  if (count > 0 && !events) return EXL3_E_NULL;
  int32_t status = EXL3_OK;
  for (int i = 0; i < count; ++i) {
    if (events[i] && hipEventDestroy((hipEvent_t)events[i]) != hipSuccess) status = EXL3_E_DEVICE;
    events[i] = nullptr;
  }
  return status;
}

int32_t exl3_profile_read(const exl3_profile *prof, float *ms) {
  if (!prof) return EXL3_E_NULL;
  if (prof->n < 0 || prof->n > prof->cap) return EXL3_E_ARG;
  if (prof->n > 0 && (!prof->events || !ms)) return EXL3_E_NULL;
  int32_t status = EXL3_OK;
  for (int i = 0; i < prof->n; ++i) {
    float t = -1.0f;
    if (hipEventSynchronize((hipEvent_t)prof->events[2 * i + 1]) != hipSuccess ||
        hipEventElapsedTime(&t, (hipEvent_t)prof->events[2 * i],
                            (hipEvent_t)prof->events[2 * i + 1]) != hipSuccess)
      status = EXL3_E_DEVICE;
    ms[i] = t;
  }
  return status;
}

}  // extern "C"
