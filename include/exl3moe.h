/*
 * exl3moe.h — C ABI of the MI355X (gfx950) fused EXL3 routed-experts layer.
 *
 * Sources for the contracts below:
 *   [p1] exllamav3 PR #284 "MoE: Add fused additive EXL3 kernels"
 *        (Summary; API contract; Validation)
 *   [p2] TensorFold PR #837 "cuda: EXL3 linear and grouped routed experts,
 *        every codebook and width, a width per expert" (What this changes)
 *   [p4] exllamav3 PR #246 "Persistent route-packed (route_block x n_tile)
 *        schedule for exl3 fused MoE (sm120)" (The change)
 *
 * General rules (every entry point):
 *   - All data pointers are DEVICE pointers on the current HIP device unless
 *     a comment says "host". Structs are passed by host pointer and read on
 *     the host before the call returns; the device arrays they point to are
 *     read on the device, in stream order.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream). All work
 *     is enqueued on it; no call synchronises, allocates, frees or retains
 *     memory, so every call can be captured into a hipGraph. Table contents
 *     may change between graph replays; their addresses may not.
 *   - Every argument is validated on the host BEFORE any device work is
 *     enqueued [p1 Summary: the device, layout, dtypes, shapes, workspace and
 *     routing are all checked first]. On error
 *     the call returns a negative EXL3_E_* code and enqueues nothing.
 *     rows == 0 is a successful no-op.
 *   - Problems only the device can see (route ID outside [0, E), a stage
 *     with a nonzero scale but a null trellis or a width outside 2..8) drop
 *     the pair / skip the stage and are counted in device status words; the
 *     host never waits for them.
 *   - The caller owns every buffer. Pointer tables do not retain their
 *     pointees: referenced trellis and rotation buffers must stay alive,
 *     unmoved and on the same device until the enqueued work completes, and
 *     for the lifetime of any captured graph that uses them [p1 API
 *     contract].
 *   - Calls that share a workspace on one stream are ordered; calls that
 *     share a workspace on different streams race.
 */
#ifndef EXL3MOE_H
#define EXL3MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Exact-match compatibility contract [p1 API contract]: bumped on any
 * incompatible signature, pointer-layout, workspace, residual-encoding or
 * overflow-semantics change. Consumers must require an exact value. */
#define EXL3_ABI_VERSION 4

enum exl3_dtype {
  EXL3_F16 = 1, EXL3_BF16 = 2, EXL3_F32 = 3, EXL3_I32 = 4, EXL3_I64 = 5
};

enum exl3_status {
  EXL3_OK = 0,
  EXL3_E_NULL = -1,      /* a required pointer is NULL */
  EXL3_E_DTYPE = -2,     /* unsupported dtype enum for that argument */
  EXL3_E_SHAPE = -3,     /* dimension not a positive multiple of 128, or
                            gate/up/down shapes inconsistent */
  EXL3_E_ALIGN = -4,     /* x, out, ws, trellis tensors and projection
                            tables must be 16-byte aligned; ids, route
                            weights and route metadata need the natural
                            alignment of their element type */
  EXL3_E_DEVICE = -5,    /* a pointer is not device memory of the current
                            device, or no HIP device is usable */
  EXL3_E_WORKSPACE = -6, /* workspace NULL or smaller than *_workspace_size */
  EXL3_E_ARG = -7,       /* scalar argument out of range (topk, stages,
                            capacity, experts, rows) */
  EXL3_E_LAUNCH = -8,    /* a kernel launch failed */
  EXL3_E_SCRATCH = -9    /* exl3_moe_forward_static: the call needs more
                            workspace than EXL3_STATIC_SCRATCH_BYTES */
};

/* Limits checked by validation. */
#define EXL3_MAX_EXPERTS 1024
#define EXL3_MAX_TOPK 32
#define EXL3_MAX_STAGES 8
#define EXL3_MAX_FEATURES 65536

int32_t exl3_abi_version(void);
/* Static string for a status code (host; never NULL). */
const char *exl3_status_string(int32_t status);

/*
 * One projection (gate, up or down) of all experts; num_experts == 1 for a
 * plain linear. Stage 0 is the base; stages 1.. are additive residual
 * ("cartridge") stages [p1 Summary: per-stage tables of trellis addresses,
 * scales and widths, any entry of which may be empty]. Tables are laid out
 * [num_stages][num_experts]:
 *   trellis  int64 device addresses of uint16 trellis tensors, each
 *            [out/16][in/16][16*K] words (16x16 tiles of 256*K bits,
 *            16-bit tail-biting window state, MCG16 codebook); 16-byte
 *            aligned; 0 allowed only where scale == 0.
 *   scale    fp32; 0.0f skips that stage's GEMM, bit-identical to leaving
 *            the stage out [p1 API contract].
 *   bits     int32 K in 2..8, validated by the CALLER before capture
 *            [p1 API contract]; the device skips and counts bad entries.
 *   suh      fp16 [E][in]   input signs; residual stages reuse the base
 *   svh      fp16 [E][out]  output signs  rotations [p1 API contract]
 *   chscale  fp16 [E][out]  per-output-channel scale
 * The layer computes, per expert e and row x (fp16):
 *   x~  = fp16_rne(Hhat(x * suh_e))            Hhat: 128-point Sylvester
 *   acc = sum_{t: scale!=0} scale_t (x~ W_t)    fp32 accumulation
 *   y   = Hhat(acc) * svh_e * chscale_e        [p2 What this changes]
 */
typedef struct exl3_proj {
  int32_t in_features;   /* multiple of 128 */
  int32_t out_features;  /* multiple of 128 */
  int32_t num_experts;   /* 1 .. EXL3_MAX_EXPERTS */
  int32_t num_stages;    /* 1 .. EXL3_MAX_STAGES */
  const int64_t *trellis;
  const float *scale;
  const int32_t *bits;
  const uint16_t *suh;
  const uint16_t *svh;
  const uint16_t *chscale;
} exl3_proj;

/*
 * Route metadata: written by exl3_route_pack, read by exl3_moe_additive.
 * pairs = rows * topk; pair q = r * topk + j. All device int32 / fp32:
 *   expert_count  [E]       kept pairs per expert
 *   expert_offset [E+1]     exclusive scan; expert_offset[E] = kept pairs
 *   pair_of_pos   [pairs]   pair at each packed position, ascending pair
 *                           index within an expert (stable); -1 past the end
 *   weight_of_pos [pairs]   route weight of that pair, widened exactly to
 *                           fp32; 0 past the end
 *   pos_of_pair   [pairs]   packed position of each pair; -1 if dropped
 *   num_active    [1]       experts with count > 0 (launch hint only)
 *   status        [1]       number of dropped pairs (ID outside [0, E))
 * [p1 Summary; Relationship to #246: route histogram, scan, stable pack]
 */
typedef struct exl3_route_meta {
  int32_t *expert_count;
  int32_t *expert_offset;
  int32_t *pair_of_pos;
  float *weight_of_pos;
  int32_t *pos_of_pair;
  int32_t *num_active;
  int32_t *status;
} exl3_route_meta;

/*
 * Optional per-launch timing, owned by the caller (a diagnostic, not part of
 * the layer). The caller creates 2 * cap events with exl3_events_create
 * (which allocates them: call it outside timed or captured regions), fills
 * the record and passes it to any call through that call's last argument
 * `prof` (NULL: no timing). While n < cap, each kernel the call launches is
 * bracketed by events[2 n] and events[2 n + 1], recorded on the call's
 * stream; kernel_ids[n] (if kernel_ids is not NULL) is set to its
 * exl3_kernel_id and n is incremented. The library keeps no state of its own
 * between calls and allocates nothing for it. exl3_profile_read waits for the
 * first n event pairs and writes each launch's milliseconds to ms[0 .. n-1].
 * Event recording is not allowed during graph capture: pass NULL there.
 * A record is not thread-safe; calls on different threads use different
 * records.
 */
enum exl3_kernel_id {
  EXL3_K_PACK = 1, EXL3_K_ROTATE = 2, EXL3_K_GATEUP = 3, EXL3_K_DOWN = 4,
  EXL3_K_COMBINE = 5, EXL3_K_LINEAR = 6, EXL3_K_DECODE = 7,
  EXL3_K_EXPERTS = 8 /* 128-row tiles: gate/up and down of a single pass in one launch, or one
                        launch of the passes pipelined across launches */
};
typedef struct exl3_profile {
  void **events;        /* host: 2 * cap event handles (hipEvent_t) */
  int32_t *kernel_ids;  /* host: cap entries, or NULL */
  int32_t cap;
  int32_t n;            /* launches recorded so far; the library appends */
} exl3_profile;
/*
 * Route histogram -> exclusive scan -> stable pack of (row, expert) pairs.
 * ids: [rows][topk] int32 or int64 (EXL3_I32 / EXL3_I64); w: [rows][topk]
 * fp16, bf16 or fp32 [p1 Validation]. Bit-exact and deterministic.
 */
int32_t exl3_route_pack(const void *ids, int32_t ids_dtype, const void *w,
                        int32_t w_dtype, int32_t rows, int32_t topk,
                        int32_t num_experts, const exl3_route_meta *meta,
                        void *stream, exl3_profile *prof);

/*
 * Plain EXL3 linear [p2 What this changes: row-invariant linear; prompt rows
 * in blocks]. x: [rows][in], x_dtype EXL3_F16 or EXL3_BF16 (read exactly; the
 * rotated rows are rounded to fp16 either way); out: [rows][out], out_dtype
 * EXL3_F16 or EXL3_BF16 (round to nearest even of the fp32 result) or
 * EXL3_F32.
 * A row's output bytes do not depend on rows or on how rows are chunked.
 * ws: device workspace of at least exl3_linear_workspace_size() bytes (the
 * rotated rows, plus pre-rotation sums and completion counts for small row
 * counts); calls that share it must be ordered on one stream.
 */
size_t exl3_linear_workspace_size(int32_t rows, int32_t in_features,
                                  int32_t out_features);
int32_t exl3_linear(const uint16_t *x, int32_t x_dtype, int32_t rows,
                    const exl3_proj *proj, void *out, int32_t out_dtype, void *ws,
                    size_t ws_bytes, void *stream, exl3_profile *prof);

/*
 * Routed-experts layer. Per kept pair (r, j), e = ids[r][j], w = weight:
 *   g, u = gate_e(x_r), up_e(x_r)   (fp32, no output rounding)
 *   a~   = fp16_rne(Hhat(silu(g) * u * suh_down_e))
 *   d    = down_e applied to a~ (stages, output rotation, chscale)
 *   y_r  = sum_j w * d, summed in fp32 in ascending packed position
 * [p2 What this changes: member lists, each expert's rotation, gate and up,
 * SwiGLU, down, weighted combine; a width per expert].
 * capacity: scratch rows counted in pairs, >= 1. Packed positions are
 * processed in passes of `capacity`; expert spans longer than it are cut
 * across passes, so rows * topk scratch is not required and the result is
 * bit-identical for every capacity [p1 Summary, API contract].
 * num_active_hint: launch-size hint only; never changes results (pass <= 0
 * for "unknown") [p1 API contract].
 * x: [rows][hidden], x_dtype EXL3_F16 or EXL3_BF16 (read exactly; the rotated
 * inputs x~ are rounded to fp16 either way, since the decoded weights are
 * fp16 values); out: [rows][hidden], out_dtype EXL3_F16 or EXL3_BF16 (round
 * to nearest even of the fp32 result) or EXL3_F32.
 */
size_t exl3_moe_workspace_size(int32_t rows, int32_t topk, int32_t num_experts,
                               int32_t hidden, int32_t intermediate,
                               int32_t capacity);

/* Stable route pack + experts in one call [p1 Summary: fused variant]. */
int32_t exl3_moe_forward(const uint16_t *x, int32_t x_dtype, int32_t rows,
                         const void *ids, int32_t ids_dtype, const void *w, int32_t w_dtype,
                         int32_t topk, const exl3_proj *gate,
                         const exl3_proj *up, const exl3_proj *down, void *out,
                         int32_t out_dtype, int32_t capacity,
                         int32_t num_active_hint, void *ws, size_t ws_bytes,
                         void *stream, exl3_profile *prof);

/*
 * exl3_moe_forward for callers that cannot allocate device memory (code under
 * hipGraph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments without ws / ws_bytes. The workspace is the library's
 * own static device array of EXL3_STATIC_SCRATCH_BYTES (32 MiB), which every
 * GPU the library runs on holds until the process ends; this call allocates
 * and frees nothing. A call whose exl3_moe_workspace_size() exceeds it
 * returns EXL3_E_SCRATCH and enqueues nothing (32 MiB holds, for example,
 * 64 rows x top-8 at hidden 4096 / intermediate 1536 with capacity = pairs).
 * Every call on one GPU uses that GPU's one array: calls that can overlap on
 * a GPU (different streams, or different host threads without ordering)
 * race and give wrong results; order them on one stream. The array keeps the
 * last call's contents; each call clears what it needs cleared. The status
 * words are not readable through this entry point.
 */
#define EXL3_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
int32_t exl3_moe_forward_static(const uint16_t *x, int32_t x_dtype, int32_t rows,
                                const void *ids, int32_t ids_dtype, const void *w,
                                int32_t w_dtype, int32_t topk, const exl3_proj *gate,
                                const exl3_proj *up, const exl3_proj *down, void *out,
                                int32_t out_dtype, int32_t capacity,
                                int32_t num_active_hint, void *stream,
                                exl3_profile *prof);

/* Experts only, for callers that already hold route metadata (from
 * exl3_route_pack or equivalent) [p1 Summary: exl3_moe_additive]. */
int32_t exl3_moe_additive(const uint16_t *x, int32_t x_dtype, int32_t rows, int32_t topk,
                          const exl3_route_meta *meta, const exl3_proj *gate,
                          const exl3_proj *up, const exl3_proj *down,
                          void *out, int32_t out_dtype, int32_t capacity,
                          int32_t num_active_hint, void *ws, size_t ws_bytes,
                          void *stream, exl3_profile *prof);

/*
 * Workspace layout of exl3_moe_forward / exl3_moe_additive (byte offsets
 * from ws, each region 256-byte aligned, in this order):
 *   ctrl        256 B   int32[64], status words of the last call, written
 *               or zeroed at its start by its first launch:
 *               [0] pairs left out: IDs outside [0, E) (exl3_moe_forward) or
 *                   pairs whose pos_of_pair is negative (exl3_moe_additive);
 *               [1] stage entries skipped because a nonzero scale came with a
 *                   null trellis or a width outside 2..8;
 *               [2] device-side waits between work items that gave up (never
 *                   expected; the output of that call is then invalid).
 *               A caller reads them after the call's stream work completes;
 *               the library itself never waits for them.
 *   meta        forward only: count[E], offset[E+1], pair_of_pos[P],
 *               weight_of_pos[P], pos_of_pair[P], num_active[1] (P = pairs;
 *               each array starts 256-byte aligned)
 *   expert_of_pos int32[P]
 *   Passes are grouped into launch units of G = plan_group passes when the
 *   call runs several passes on 128-row tiles (rows * topk >= 64 *
 *   num_experts): G = min(8, ceil(passes / 2)), else 1. A unit covers
 *   packed positions [u G C, (u + 1) G C) and is planned as one range, so
 *   an expert span that a pass boundary cuts inside a unit is tiled as one
 *   run. The scratch for such calls is therefore 2 G C rows of xt, at and d
 *   (1.38 GB in all for 3072 rows x top-8, hidden 6144, intermediate 2048
 *   at C = 2048, where G = 6).
 *   plan        per unit: int32 ntiles + tiles of {expert, start, len}
 *               (start relative to the unit; slots: G * plan_slots)
 *   xt          fp16 [G C][2][hidden]  rotated gate/up inputs of the unit
 *   at          fp16 [G C][intermediate] rotated down inputs a~ of the unit
 *   d           fp32 [G C][hidden]     weighted per-pair down outputs
 *               (xt, at and d each hold two such buffers, the second one
 *               256-byte aligned after the first, when the call runs several
 *               passes on 128-row tiles (rows * topk >= 64 * num_experts and
 *               capacity < rows * topk): unit u uses buffer u % 2)
 *   yacc        fp32 [rows][hidden]  running row sums across passes
 *   (then private scratch of the 16-row tile path, used when rows * topk <
 *   64 * num_experts: pre-rotation fp32 sums [C][max(2 intermediate,
 *   hidden)] and int32 completion counts; not part of the layout struct)
 * Rotated vectors (xt, at) are stored with the 16 entries of each aligned
 * group of 16 permuted as k = {0,4,1,5,2,6,3,7,8,12,9,13,10,14,11,15}[p]
 * (stored slot p holds entry k). exl3_moe_layout() returns the offsets.
 */
typedef struct exl3_moe_layout_t {
  size_t ctrl, meta, expert_of_pos, plan, xt, at, d, yacc, total;
  int32_t passes, plan_slots, plan_group;
} exl3_moe_layout_t;
int32_t exl3_moe_layout(int32_t rows, int32_t topk, int32_t num_experts,
                        int32_t hidden, int32_t intermediate, int32_t capacity,
                        exl3_moe_layout_t *layout /* host */);

/*
 * Diagnostic: decode `ntiles` consecutive trellis tiles of width K with the
 * GEMM kernels' own decode path: consecutive tile pairs are taken as the two
 * tiles of one 32-input MFMA k-step, and each lane decodes the half column
 * those kernels give it, from the same in-tile window offsets and shift,
 * with the same register decode. words: [ntiles][16K] uint16;
 * out: [ntiles][16 (k)][16 (n)] fp16. For bit-exact decode tests.
 */
int32_t exl3_decode_tiles(const uint16_t *words, int32_t ntiles, int32_t K,
                          uint16_t *out, void *stream, exl3_profile *prof);

/* Create / destroy `count` events into / from the host array `events`
 * (destroy sets each entry to NULL). */
int32_t exl3_events_create(int32_t count, void **events /* host */);
int32_t exl3_events_destroy(int32_t count, void **events /* host */);
int32_t exl3_profile_read(const exl3_profile *prof /* host */, float *ms /* host */);

#ifdef __cplusplus
}
#endif
#endif /* EXL3MOE_H */
