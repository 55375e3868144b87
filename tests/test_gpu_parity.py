"""GPU parity of the HIP path against the float64 oracle (MI355X only).

Bars: bit-exact for the route pack and decoded weights; floating-point
outputs within max|gpu - oracle_R| <= 2e-3 * RMS(oracle_R) (fp32 output);
fp16 output equal to RNE of the fp32 output; invariances bit-exact.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import linear as olinear  # noqa: E402
from oracle import moe as omoe  # noqa: E402
from oracle import route as oroute  # noqa: E402
from oracle import trellis as otrellis  # noqa: E402
from trellis_quantized_moe_amd import exl3, synth  # noqa: E402

pytestmark = pytest.mark.gpu
TOL = 2e-3
DEV = "cuda"


def _say(*a):
    print(*a, flush=True)


def _rel_err(got, ref):
    rms = float(np.sqrt(np.mean(np.square(ref))))
    return float(np.max(np.abs(got - ref))) / rms


def _fp16_of(t):
    return t.float().cpu().numpy().astype(np.float16)


# ------------------------------------------------------- status-word checks
# Every call below goes through these wrappers: they pass an explicit
# workspace and, once the call's work is done, read the status words at its
# start (exl3moe.h: ctrl[0] pairs left out, ctrl[1] skipped stage entries,
# ctrl[2] waits that gave up) and assert them.
def _ctrl(ws):
    torch.cuda.synchronize()
    return [int(v) for v in ws[:12].view(torch.int32).cpu()]


def _ids_dropped(ids, E):
    a = ids.cpu().numpy() if hasattr(ids, "cpu") else np.asarray(ids)
    return int(np.sum((a < 0) | (a >= E)))


def moe_forward(x, ids, w, gate, up, down, capacity, out_dtype=torch.float32, out=None,
                ws=None, num_active_hint=-1, bad_stages=0):
    rows, topk = ids.shape
    if ws is None:
        need = exl3.moe_workspace_size(rows, topk, gate.num_experts, gate.in_features,
                                       gate.out_features, capacity)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    y = exl3.exl3_moe_forward(x, ids, w, gate, up, down, capacity, out_dtype, out=out, ws=ws,
                              num_active_hint=num_active_hint)
    assert _ctrl(ws)[:3] == [_ids_dropped(ids, gate.num_experts), bad_stages, 0]
    return y


def moe_additive(x, topk, meta, gate, up, down, capacity, out_dtype=torch.float32, out=None,
                 ws=None, num_active_hint=-1):
    rows = x.shape[0]
    if ws is None:
        need = exl3.moe_workspace_size(rows, topk, gate.num_experts, gate.in_features,
                                       gate.out_features, capacity)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    y = exl3.exl3_moe_additive(x, topk, meta, gate, up, down, capacity, out_dtype, out=out,
                               ws=ws, num_active_hint=num_active_hint)
    left_out = int((meta["pos_of_pair"][:rows * topk] < 0).sum())
    assert _ctrl(ws)[:3] == [left_out, 0, 0]
    return y


def linear(x, proj, out_dtype=torch.float32):
    rows = x.shape[0]
    ws = torch.empty(max(256, exl3.linear_workspace_size(rows, proj.in_features,
                                                         proj.out_features)),
                     dtype=torch.uint8, device=x.device)
    y = exl3.exl3_linear(x, proj, out_dtype, ws=ws)
    assert _ctrl(ws)[:3] == [0, 0, 0]
    return y


# ------------------------------------------------------------------ decode
@pytest.mark.parametrize("K", range(2, 9))
def test_decode_tiles_bit_exact(K):
    _say("decode K=%d" % K)
    rng = np.random.default_rng(100 + K)
    ntiles = 4097  # odd: the last k-step pair holds one tile
    words = rng.integers(0, 65536, size=(ntiles, 16 * K), dtype=np.uint16)
    words[0] = 0
    words[1] = 0xFFFF
    d = torch.from_numpy(words.reshape(-1).view(np.int16)).to(DEV)
    got = exl3.exl3_decode_tiles(d, K).cpu().numpy()
    ref = otrellis.decode_tiles_shift(words, K).astype(np.float16)
    assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))


# ------------------------------------------------------------------- route
@pytest.mark.parametrize("rows,topk,E,idt,wdt,seed", [
    (16, 2, 8, "i32", "f32", 0), (32, 8, 128, "i64", "bf16", 1),
    (1, 8, 128, "i64", "f16", 2), (3072, 8, 192, "i32", "f16", 3),
    (700, 6, 1024, "i64", "f32", 4), (5, 32, 3, "i32", "bf16", 5)])
def test_route_pack_bit_exact(rows, topk, E, idt, wdt, seed):
    _say("route", rows, topk, E, idt, wdt)
    rng = np.random.default_rng(seed)
    ids = rng.integers(-2, E + 2, size=(rows, topk))  # some dropped
    w = rng.random((rows, topk)).astype(np.float32)
    if wdt == "bf16":
        wb = synth.f32_to_bf16_bits(w)
        wt = torch.from_numpy(wb.view(np.int16)).view(torch.bfloat16)
        wexact = synth.bf16_bits_to_f64(wb)
    elif wdt == "f16":
        wt = torch.from_numpy(w.astype(np.float16))
        wexact = w.astype(np.float16).astype(np.float64)
    else:
        wt = torch.from_numpy(w)
        wexact = w.astype(np.float64)
    it = torch.from_numpy(ids.astype(np.int64 if idt == "i64" else np.int32))
    meta = exl3.exl3_route_pack(it.to(DEV), wt.to(DEV), E)
    torch.cuda.synchronize()
    ref = oroute.route_pack(ids, wexact, E)
    P = rows * topk
    assert np.array_equal(meta["expert_count"].cpu().numpy(), ref["count"])
    assert np.array_equal(meta["expert_offset"].cpu().numpy(), ref["offset"])
    assert np.array_equal(meta["pair_of_pos"].cpu().numpy()[:P], ref["pair_of_pos"])
    assert np.array_equal(meta["pos_of_pair"].cpu().numpy()[:P], ref["pos_of_pair"])
    assert np.array_equal(meta["weight_of_pos"].cpu().numpy()[:P].astype(np.float64),
                          ref["weight_of_pos"])
    assert int(meta["num_active"][0]) == ref["num_active"]
    assert int(meta["status"][0]) == ref["dropped"]


# ------------------------------------------------------------------ linear
def _linear_case(fin, fout, stages, rows, seed):
    bits = np.array([[k] for k, _ in stages], dtype=np.int32)
    scale = np.array([[s] for _, s in stages], dtype=np.float32)
    p = synth.make_proj(seed, "linear", 1, fin, fout, bits, scale)
    x = np.random.default_rng(seed).standard_normal((rows, fin)).astype(np.float16)
    return p, x


@pytest.mark.parametrize("fin,fout,stages,rows", [
    (256, 384, ((4, 1.0),), 1), (256, 384, ((3, 1.0), (2, 0.37)), 33),
    (512, 256, ((8, 1.0), (5, -0.25)), 7), (384, 128, ((2, 1.0), (7, 0.5), (6, 0.0)), 17),
    (128, 256, ((6, 1.0),), 40)])
def test_linear_parity(fin, fout, stages, rows):
    _say("linear", fin, fout, stages, rows)
    p, x = _linear_case(fin, fout, stages, rows, seed=fin + fout + rows)
    dp = exl3.DeviceProj(p, DEV)
    xd = exl3.f16_tensor(x)
    y32 = linear(xd, dp, torch.float32)
    y16 = linear(xd, dp, torch.float16)
    torch.cuda.synchronize()
    ref = olinear.linear(x, p, "R")
    got = y32.cpu().double().numpy()
    assert _rel_err(got, ref) <= TOL
    assert np.array_equal(_fp16_of(y32).view(np.uint16),
                          y16.cpu().numpy().view(np.uint16))


@pytest.mark.parametrize("K", [2, 3, 4, 8])
def test_linear_4096_parity_and_row_invariance(K):
    """The linear workload: rows 1/7/32/128 and 2048 (also as 16 chunks of
    128); a row's output bytes are identical in every call."""
    _say("linear4096 K=%d" % K)
    p, x = synth.linear_workload(K, 2048)
    dp = exl3.DeviceProj(p, DEV)
    xd = exl3.f16_tensor(x)
    full = linear(xd, dp, torch.float16)
    chunks = torch.cat([linear(xd[i:i + 128], dp, torch.float16)
                        for i in range(0, 2048, 128)])
    torch.cuda.synchronize()
    fb = full.cpu().numpy().view(np.uint16)
    assert np.array_equal(chunks.cpu().numpy().view(np.uint16), fb)
    for rows in (1, 7, 32, 128):
        y = linear(xd[:rows], dp, torch.float16)
        assert np.array_equal(y.cpu().numpy().view(np.uint16), fb[:rows]), rows
    # parity on sampled rows (fp32 output)
    sample = [0, 1, 777, 2047]
    y32 = linear(xd, dp, torch.float32).cpu().double().numpy()
    ref = olinear.linear(x[sample], p, "R")
    assert _rel_err(y32[sample], ref) <= TOL


# --------------------------------------------------------------------- moe
def _moe_inputs(wl):
    gate, up, down = (exl3.DeviceProj(p, DEV) for p in (wl.gate, wl.up, wl.down))
    x, ids, w = exl3.device_inputs(wl, DEV)
    return gate, up, down, x, ids, w


def _tiny(**over):
    return synth.moe_workload("tiny", **over)


@pytest.mark.parametrize("over", [
    {}, dict(K=(2, 3, 5, 8)), dict(rows=37, topk=3, E=5, K=(4, 6)),
    dict(rows=1, topk=8, E=16, K=(3, 4))])
def test_moe_tiny_parity(over):
    _say("moe tiny", over)
    wl = _tiny(**over)
    gate, up, down, x, ids, w = _moe_inputs(wl)
    y32 = moe_forward(x, ids, w, gate, up, down, wl.capacity, torch.float32)
    y16 = moe_forward(x, ids, w, gate, up, down, wl.capacity, torch.float16)
    torch.cuda.synchronize()
    ref = omoe.moe_forward(wl.x, wl.ids, wl.weights_f64, wl.gate, wl.up, wl.down, "R")
    assert _rel_err(y32.cpu().double().numpy(), ref) <= TOL
    assert np.array_equal(_fp16_of(y32).view(np.uint16), y16.cpu().numpy().view(np.uint16))


def test_moe_capacity_invariance():
    """capacity in {1, 7, span, span+1, 32, inf}: identical bytes."""
    wl = _tiny()
    gate, up, down, x, ids, w = _moe_inputs(wl)
    span = int(np.bincount(wl.ids.reshape(-1), minlength=8).max())
    base = moe_forward(x, ids, w, gate, up, down, 10 ** 6, torch.float32)
    for cap in (1, 7, span, span + 1, 32):
        _say("capacity", cap)
        y = moe_forward(x, ids, w, gate, up, down, cap, torch.float32)
        assert torch.equal(y.view(torch.int32), base.view(torch.int32)), cap


def test_moe_additive_equals_forward_and_ignores_hint():
    wl = _tiny(rows=29)
    gate, up, down, x, ids, w = _moe_inputs(wl)
    fwd = moe_forward(x, ids, w, gate, up, down, 16, torch.float32)
    meta = exl3.exl3_route_pack(ids, w, wl.num_experts)
    for hint in (-1, 0, 3, 1000):
        add = moe_additive(x, wl.topk, meta, gate, up, down, 16, torch.float32,
                                     num_active_hint=hint)
        assert torch.equal(add.view(torch.int32), fwd.view(torch.int32)), hint


def test_moe_row_invariance_member_counts():
    """A row's bytes do not change with the other rows (member counts)."""
    wl = _tiny(rows=64)
    gate, up, down, x, ids, w = _moe_inputs(wl)
    full = moe_forward(x, ids, w, gate, up, down, 10 ** 6, torch.float32)
    for r0, r1 in ((0, 1), (5, 6), (0, 17), (40, 64)):
        part = moe_forward(x[r0:r1], ids[r0:r1], w[r0:r1], gate, up, down,
                                     10 ** 6, torch.float32)
        assert torch.equal(part.view(torch.int32), full[r0:r1].view(torch.int32)), (r0, r1)


def test_zero_scale_equals_absent_stage():
    wl = _tiny(rows=16)
    gate, up, down, x, ids, w = _moe_inputs(wl)
    base = moe_forward(x, ids, w, gate, up, down, 64, torch.float32)

    def with_zero_stage(p, null):
        n3 = synth.words_per_tensor(p.in_features, p.out_features, 3)
        words = p.words + [[None if null else np.full(n3, 0x1234, np.uint16)
                            for e in range(p.num_experts)]]
        return synth.Proj(p.in_features, p.out_features, p.num_experts, words,
                          np.concatenate([p.scale, np.zeros((1, p.num_experts), np.float32)]),
                          np.concatenate([p.bits, np.full((1, p.num_experts), 3, np.int32)]),
                          p.suh, p.svh, p.chscale)

    for null in (False, True):
        g2, u2, d2 = (exl3.DeviceProj(with_zero_stage(p, null), DEV)
                      for p in (wl.gate, wl.up, wl.down))
        y = moe_forward(x, ids, w, g2, u2, d2, 64, torch.float32)
        assert torch.equal(y.view(torch.int32), base.view(torch.int32)), null


def test_dropped_ids_and_unrouted_rows():
    wl = _tiny(rows=8)
    ids_np = wl.ids.copy()
    ids_np[3, :] = [99, -1]        # row 3 fully dropped -> zeros
    ids_np[5, 1] = 8               # one dropped pair
    wl.ids = ids_np
    gate, up, down, x, ids, w = _moe_inputs(wl)
    ref = omoe.moe_forward(wl.x, ids_np, wl.weights_f64, wl.gate, wl.up, wl.down, "R")
    # capacity 5: several passes; 10**6: one pass (pack, plan and rotation in
    # one launch for so few pairs)
    for cap in (5, 10 ** 6):
        for dt in (torch.float32, torch.float16):
            out = torch.full((8, wl.hidden), 7.0, dtype=dt, device=DEV)
            y = moe_forward(x, ids, w, gate, up, down, cap, dt, out=out)
            torch.cuda.synchronize()
            assert torch.all(y[3] == 0), (cap, dt)
            assert _rel_err(y.cpu().double().numpy(), ref) <= (TOL if dt == torch.float32 else 5e-3)


def _ws_meta(ws, rows, topk, E, H, I, cap):
    """The pack metadata a forward call left in its workspace (the layout of
    exl3moe.h: count, offset, pair_of_pos, weight_of_pos, pos_of_pair, each
    256-byte aligned, then expert_of_pos)."""
    lay = exl3.moe_layout(rows, topk, E, H, I, cap)
    P = rows * topk
    b = ws.cpu().numpy()
    al = lambda v: (v + 255) // 256 * 256
    o = lay.meta
    out = {}
    for name, n, dt in (("count", E, np.int32), ("offset", E + 1, np.int32),
                        ("pair_of_pos", P, np.int32), ("weight_of_pos", P, np.float32),
                        ("pos_of_pair", P, np.int32)):
        out[name] = b[o:o + 4 * n].view(dt)
        o = al(o + 4 * n)
    out["expert_of_pos"] = b[lay.expert_of_pos:lay.expert_of_pos + 4 * P].view(np.int32)
    return out


@pytest.mark.parametrize("rows,topk,E,idt,seed", [(1200, 8, 64, "i32", 11),
                                                   (3072, 8, 192, "i64", 12)])
def test_forward_pack_many_pairs_bit_exact(rows, topk, E, idt, seed):
    """Calls with 8192 pairs or more pack over several workgroups (three
    launches): the metadata they leave in the workspace must be the oracle's
    stable pack bit for bit (dropped IDs, fully dropped rows, skewed counts),
    expert_of_pos must label every kept position with its expert, and rows
    with no kept pair must come out as zeros."""
    _say("forward pack", rows, topk, E, idt)
    wl = synth.moe_workload("tiny", rows=rows, topk=topk, E=E)
    rng = np.random.default_rng(seed)
    pop = rng.zipf(1.3, size=(rows, topk)) % E  # skewed expert popularity
    ids_np = np.where(rng.random((rows, topk)) < 0.03, rng.integers(-3, 0, (rows, topk)),
                      pop).astype(np.int64)
    ids_np[7, :] = E + 1               # a fully dropped row
    ids_np[rows - 2, :] = -1           # another, near the end
    wl.ids = ids_np.astype(np.int64 if idt == "i64" else np.int32)
    gate, up, down, x, ids, w = _moe_inputs(wl)
    cap = rows * topk
    need = exl3.moe_workspace_size(rows, topk, E, wl.hidden, wl.intermediate, cap)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    out = torch.full((rows, wl.hidden), 7.0, dtype=torch.float32, device=DEV)
    y = moe_forward(x, ids, w, gate, up, down, cap, torch.float32, out=out, ws=ws)
    torch.cuda.synchronize()
    got = _ws_meta(ws, rows, topk, E, wl.hidden, wl.intermediate, cap)
    ref = oroute.route_pack(ids_np, wl.weights_f64, E)
    kept = int(ref["offset"][E])
    assert np.array_equal(got["count"], ref["count"])
    assert np.array_equal(got["offset"], ref["offset"])
    assert np.array_equal(got["pair_of_pos"][:kept], ref["pair_of_pos"][:kept])
    assert np.all(got["pair_of_pos"][kept:] == -1)
    assert np.array_equal(got["pos_of_pair"], ref["pos_of_pair"])
    assert np.array_equal(got["weight_of_pos"][:kept].astype(np.float64),
                          ref["weight_of_pos"][:kept])
    lab = np.repeat(np.arange(E), ref["count"])
    assert np.array_equal(got["expert_of_pos"][:kept], lab)
    yc = y.cpu().numpy()
    assert np.all(yc[7] == 0) and np.all(yc[rows - 2] == 0)
    rs = [0, 1, rows // 2, rows - 1]
    refy = omoe.moe_forward(wl.x, wl.ids, wl.weights_f64, wl.gate, wl.up, wl.down, "R", rows=rs)
    assert _rel_err(yc[rs].astype(np.float64), refy) <= TOL


# ---------------------------------------------------- full-size workloads
def _sampled_parity(wl, rows_sample, capacity):
    gate, up, down, x, ids, w = _moe_inputs(wl)
    y = moe_forward(x, ids, w, gate, up, down, capacity, torch.float32)
    torch.cuda.synchronize()
    got = y.cpu().double().numpy()[rows_sample]
    ref = omoe.moe_forward(wl.x, wl.ids, wl.weights_f64, wl.gate, wl.up, wl.down, "R",
                           rows=rows_sample)
    err = _rel_err(got, ref)
    _say("  sampled rows", rows_sample, "err %.3e" % err)
    return err


@pytest.mark.parametrize("M", [1, 8, 32])
def test_decode_workload_sampled(M):
    """The decode layer at 1, 8 and 32 rows: every row up to 8 rows; at 32
    rows the first and the last row plus 6 more chosen to share experts."""
    _say("decode workload M=%d" % M)
    wl = synth.moe_workload("decode", rows=M)
    rows = list(range(M)) if M <= 8 else _greedy_rows(wl.ids, [[0], [M - 1]], 8)
    assert _sampled_parity(wl, sorted(rows), M * 8) <= TOL


def test_decode_rows_same_bytes_in_both_wait_modes():
    """Each decode row alone (every work item of the single-pass launch
    resident at once: down items wait per a~ block inside their chains) and
    inside an 8-row batch (the launch runs in waves: down items wait for
    their whole tile first) gives the same bytes."""
    _say("decode rows alone vs in an 8-row batch")
    wl = synth.moe_workload("decode", rows=8)
    gate, up, down, x, ids, w = _moe_inputs(wl)
    full = moe_forward(x, ids, w, gate, up, down, 8 * 8, torch.float32)
    for r in range(8):
        one = moe_forward(x[r:r + 1], ids[r:r + 1], w[r:r + 1], gate, up, down, 8,
                          torch.float32)
        assert torch.equal(one.view(torch.int32), full[r:r + 1].view(torch.int32)), r


def test_additive_workload_sampled():
    """The additive layer (base K=3 + residual K=2, 30% zero residual
    scales, half of those with a null trellis). Rows by rule: for each of
    gate, up and down, a pair whose residual stage has a zero scale with a
    trellis, one with a zero scale and a null trellis, and one with a
    nonzero scale; at least 4 rows."""
    _say("additive workload")
    wl = synth.moe_workload("additive")
    needs = []
    for p in (wl.gate, wl.up, wl.down):
        zero_ptr = {e for e in range(wl.num_experts) if p.scale[1][e] == 0 and p.words[1][e] is not None}
        zero_null = {e for e in range(wl.num_experts) if p.words[1][e] is None}
        live = {e for e in range(wl.num_experts) if p.scale[1][e] != 0}
        assert zero_ptr and zero_null and live
        for group in (zero_ptr, zero_null, live):
            needs.append([r for r in range(wl.rows) if set(map(int, wl.ids[r])) & group])
    rows = _greedy_rows(wl.ids, needs, 4)
    assert _sampled_parity(wl, sorted(rows), 1024) <= TOL


# ------------------------------------------------ wide (128-row) MoE tiles
def _wide_wl(rows=300):
    # pairs >= 64 * experts selects 128-row tiles
    return synth.moe_workload("tiny", rows=rows, topk=2, E=4, H=256, I=384, K=(3, 5, 8))


def test_moe_wide_tiles_parity():
    wl = _wide_wl()
    gate, up, down, x, ids, w = _moe_inputs(wl)
    y = moe_forward(x, ids, w, gate, up, down, 10 ** 6, torch.float32)
    torch.cuda.synchronize()
    ref = omoe.moe_forward(wl.x, wl.ids, wl.weights_f64, wl.gate, wl.up, wl.down, "R")
    assert _rel_err(y.cpu().double().numpy(), ref) <= TOL


def test_moe_wide_equals_narrow_rows():
    """The same rows through 128-row tiles (many rows) and 16-row tiles (few
    rows): identical bytes."""
    wl = _wide_wl()
    gate, up, down, x, ids, w = _moe_inputs(wl)
    full = moe_forward(x, ids, w, gate, up, down, 10 ** 6, torch.float32)
    for r0, r1 in ((0, 3), (100, 117), (290, 300)):
        part = moe_forward(x[r0:r1], ids[r0:r1], w[r0:r1], gate, up, down,
                                     10 ** 6, torch.float32)
        assert torch.equal(part.view(torch.int32), full[r0:r1].view(torch.int32)), (r0, r1)


def test_moe_wide_capacity_invariance():
    wl = _wide_wl()
    gate, up, down, x, ids, w = _moe_inputs(wl)
    base = moe_forward(x, ids, w, gate, up, down, 10 ** 6, torch.float32)
    for cap in (1, 100, 128, 129, 257, 599):
        _say("wide capacity", cap)
        y = moe_forward(x, ids, w, gate, up, down, cap, torch.float32)
        assert torch.equal(y.view(torch.int32), base.view(torch.int32)), cap


def test_moe_wide_pipelined_edge_cases():
    """Several passes on 128-row tiles (capacity 100 of 600 pairs: 6 passes,
    pipelined across launches) with dropped IDs and a fully dropped row,
    fp16 output equal to RNE(fp32), and an extra zero-scale stage (with and
    without a trellis pointer) equal to no stage."""
    wl = _wide_wl()
    ids_np = wl.ids.copy()
    ids_np[7, :] = [-3, 4]        # row 7 fully dropped -> zeros
    ids_np[150, 0] = 99           # one dropped pair
    wl.ids = ids_np
    gate, up, down, x, ids, w = _moe_inputs(wl)
    lay = exl3.moe_layout(wl.rows, wl.topk, wl.num_experts, wl.hidden, wl.intermediate, 100)
    assert lay.passes == 6
    out = torch.full((wl.rows, wl.hidden), 7.0, dtype=torch.float32, device=DEV)
    y = moe_forward(x, ids, w, gate, up, down, 100, torch.float32, out=out)
    y16 = moe_forward(x, ids, w, gate, up, down, 100, torch.float16)
    y1 = moe_forward(x, ids, w, gate, up, down, 10 ** 6, torch.float32)
    torch.cuda.synchronize()
    assert torch.all(y[7] == 0)
    assert torch.equal(y.view(torch.int32), y1.view(torch.int32))
    assert np.array_equal(_fp16_of(y).view(np.uint16), y16.cpu().numpy().view(np.uint16))
    ref = omoe.moe_forward(wl.x, ids_np, wl.weights_f64, wl.gate, wl.up, wl.down, "R")
    assert _rel_err(y.cpu().double().numpy(), ref) <= TOL

    def with_zero_stage(pr, null):
        n3 = synth.words_per_tensor(pr.in_features, pr.out_features, 3)
        words = pr.words + [[None if null else np.full(n3, 0x1234, np.uint16)
                             for e in range(pr.num_experts)]]
        return synth.Proj(pr.in_features, pr.out_features, pr.num_experts, words,
                          np.concatenate([pr.scale, np.zeros((1, pr.num_experts), np.float32)]),
                          np.concatenate([pr.bits, np.full((1, pr.num_experts), 3, np.int32)]),
                          pr.suh, pr.svh, pr.chscale)

    for null in (False, True):
        g2, u2, d2 = (exl3.DeviceProj(with_zero_stage(pr, null), DEV)
                      for pr in (wl.gate, wl.up, wl.down))
        y2 = moe_forward(x, ids, w, g2, u2, d2, 100, torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(y2.view(torch.int32), y.view(torch.int32)), null


@pytest.mark.parametrize("cap,group", [(100, 3), (50, 6), (7, 8)])
def test_moe_wide_grouped_passes_additive_equals_forward(cap, group):
    """128-row tiles over several passes grouped into launch units (3, 6 or
    8 passes per plan and buffer set: 6, 12 and 86 passes):
    exl3_moe_additive on the route pack equals exl3_moe_forward, and both
    equal the one-pass result."""
    wl = _wide_wl()
    lay = exl3.moe_layout(wl.rows, wl.topk, wl.num_experts, wl.hidden, wl.intermediate, cap)
    assert lay.plan_group == group, (lay.passes, lay.plan_group)
    _say("wide grouped", cap, lay.passes, group)
    gate, up, down, x, ids, w = _moe_inputs(wl)
    one = moe_forward(x, ids, w, gate, up, down, 10 ** 6, torch.float32)
    fwd = moe_forward(x, ids, w, gate, up, down, cap, torch.float32)
    meta = exl3.exl3_route_pack(ids, w, wl.num_experts)
    add = moe_additive(x, wl.topk, meta, gate, up, down, cap, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(fwd.view(torch.int32), one.view(torch.int32))
    assert torch.equal(add.view(torch.int32), one.view(torch.int32))


@pytest.mark.parametrize("E,rows,cap", [(4, 300, 100), (4, 300, 7), (16, 1024, 100),
                                        (300, 9600, 2400)])
def test_unit_plan_tiles_each_span_once(E, rows, cap):
    """The plan of every launch unit, read back from the workspace, tiles the
    unit's packed positions exactly once: tiles are disjoint and cover
    [unit start, unit end); each lies inside its expert's span; all are 128
    rows but the last of an expert's run inside the unit, so a span that a
    pass boundary cuts inside the unit is still one run; the count stays
    within the launch bound min(E, positions) + positions / 128. With 300
    experts a unit spans more than 128 of them (the planner's unsorted
    order for partial tiles). The output equals the one-pass output bit for
    bit."""
    wl = synth.moe_workload("tiny", rows=rows, topk=2, E=E, H=256, I=384, K=(3, 5, 8))
    P = rows * wl.topk
    assert P >= 64 * E
    lay = exl3.moe_layout(rows, wl.topk, E, wl.hidden, wl.intermediate, cap)
    G, C = lay.plan_group, min(cap, P)
    assert G > 1, lay.plan_group
    gate, up, down, x, ids, w = _moe_inputs(wl)
    ws = torch.empty(lay.total, dtype=torch.uint8, device=DEV)
    y = moe_forward(x, ids, w, gate, up, down, cap, torch.float32, ws=ws)
    one = moe_forward(x, ids, w, gate, up, down, 10 ** 6, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), one.view(torch.int32))
    raw = ws.cpu().numpy()
    o0 = lay.meta + (4 * E + 255) // 256 * 256  # offset[E + 1] follows count[E], 256-B aligned
    offset = raw[o0:o0 + 4 * (E + 1)].view(np.int32)
    kept = int(offset[E])
    assert kept == P
    units = (lay.passes + G - 1) // G
    per_unit = 1 + 3 * G * lay.plan_slots
    plan = raw[lay.plan:lay.plan + 4 * units * per_unit].view(np.int32).reshape(units, per_unit)
    for u in range(units):
        ub, ue = u * G * C, min((u + 1) * G * C, kept)
        n = int(plan[u, 0])
        t = plan[u, 1:1 + 3 * n].reshape(n, 3)
        assert n <= min(E, ue - ub) + -(-(ue - ub) // 128), (u, n)
        order = np.argsort(t[:, 1], kind="stable")
        starts, lens = t[order, 1], t[order, 2]
        assert starts[0] == 0 and np.all(lens > 0) and np.all(lens <= 128), u
        assert np.array_equal(starts[1:], (starts + lens)[:-1]), u  # disjoint, no gaps
        assert starts[-1] + lens[-1] == ue - ub, u
        for e, st, ln in t[order]:
            lo, hi = ub + st, ub + st + ln
            assert offset[e] <= lo and hi <= offset[e + 1], (u, e, st, ln)
        for e in np.unique(t[:, 0]):
            et = t[t[:, 0] == e]
            et = et[np.argsort(et[:, 1])]
            assert np.all(et[:-1, 2] == 128), (u, e)  # one run: only the last is partial
            lo, hi = max(offset[e], ub), min(offset[e + 1], ue)
            assert et[0, 1] == lo - ub and et[-1, 1] + et[-1, 2] == hi - ub, (u, e)


def test_linear_wide_multistage_parity():
    # 1024 rows x 8192 out selects 128-row tiles; three stages, one zero
    p, x = _linear_case(256, 8192, ((3, 1.0), (2, 0.25), (4, 0.0)), 1024, seed=9)
    dp = exl3.DeviceProj(p, DEV)
    xd = exl3.f16_tensor(x)
    y = linear(xd, dp, torch.float32)
    y_small = linear(xd[:5], dp, torch.float32)
    torch.cuda.synchronize()
    ref = olinear.linear(x[[0, 4, 1023]], p, "R")
    assert _rel_err(y.cpu().double().numpy()[[0, 4, 1023]], ref) <= TOL
    assert torch.equal(y_small.view(torch.int32), y[:5].view(torch.int32))


# ------------------------------- active residual stages on 128-row tiles
def _wide_residual_wl(rows=300):
    """pairs >= 64 * experts (128-row tiles) with a K=2 residual stage on
    gate, up and down (scales N(0, 0.1^2), one expert per projection with a
    zero scale)."""
    return synth.moe_workload("additive", rows=rows, topk=2, E=4, H=256, I=384, K=3)


def test_moe_wide_active_residual_stage():
    """128-row tiles with a live residual stage (the multi-stage variants of
    the single-pass and the pipelined kernels): one pass, capacity 100 (6
    passes, units of 2) and capacity 7 (86 passes, units of 4) give the same
    bytes; the result meets the oracle bar; rows computed alone (16-row
    tiles) give the same bytes as in the full call."""
    wl = _wide_residual_wl()
    assert wl.rows * wl.topk >= 64 * wl.num_experts
    for p in (wl.gate, wl.up, wl.down):
        assert np.sum(p.scale[1] != 0) >= 3
    gate, up, down, x, ids, w = _moe_inputs(wl)
    one = moe_forward(x, ids, w, gate, up, down, 10 ** 6, torch.float32)
    for cap, group in ((100, 3), (7, 8)):
        lay = exl3.moe_layout(wl.rows, wl.topk, wl.num_experts, wl.hidden, wl.intermediate, cap)
        assert lay.plan_group == group
        _say("wide residual capacity", cap, lay.passes)
        y = moe_forward(x, ids, w, gate, up, down, cap, torch.float32)
        assert torch.equal(y.view(torch.int32), one.view(torch.int32)), cap
    ref = omoe.moe_forward(wl.x, wl.ids, wl.weights_f64, wl.gate, wl.up, wl.down, "R")
    assert _rel_err(one.cpu().double().numpy(), ref) <= TOL
    for r0, r1 in ((0, 3), (150, 161), (297, 300)):
        part = moe_forward(x[r0:r1], ids[r0:r1], w[r0:r1], gate, up, down, 10 ** 6, torch.float32)
        assert torch.equal(part.view(torch.int32), one[r0:r1].view(torch.int32)), (r0, r1)


# ---------------------------------------------- capacity cases of the pages
@pytest.mark.parametrize("rows", [40, 300])
def test_topk2_capacity_equal_to_rows(rows):
    """topk = 2 with capacity = rows (pairs = 2 x capacity: two passes, the
    downstream case exllamav3 PR #284 lists under Validation), on 16-row
    tiles (40 rows) and on 128-row tiles (300 rows): equal to one pass bit
    for bit and within the oracle bar."""
    wl = synth.moe_workload("tiny", rows=rows, topk=2, E=4, H=256, I=384, K=(3, 5, 8))
    gate, up, down, x, ids, w = _moe_inputs(wl)
    assert exl3.moe_layout(rows, 2, 4, 256, 384, rows).passes == 2
    y = moe_forward(x, ids, w, gate, up, down, rows, torch.float32)
    one = moe_forward(x, ids, w, gate, up, down, 10 ** 6, torch.float32)
    assert torch.equal(y.view(torch.int32), one.view(torch.int32))
    ref = omoe.moe_forward(wl.x, wl.ids, wl.weights_f64, wl.gate, wl.up, wl.down, "R")
    assert _rel_err(y.cpu().double().numpy(), ref) <= TOL


@pytest.mark.parametrize("rows,E", [(20, 8), (300, 4)])
def test_pairs_exactly_capacity_plus_one(rows, E):
    """rows x topk == capacity + 1: a second pass holding one pair (exllamav3
    PR #284, Validation: exactly capacity + 1), on 16-row and 128-row tiles;
    also a capacity that cuts every span several times (multi-tile
    overflow). Both equal one pass bit for bit."""
    wl = synth.moe_workload("tiny", rows=rows, topk=2, E=E, H=256, I=384, K=(4, 6))
    gate, up, down, x, ids, w = _moe_inputs(wl)
    P = rows * 2
    one = moe_forward(x, ids, w, gate, up, down, 10 ** 6, torch.float32)
    for cap in (P - 1, max(1, P // (3 * E))):
        lay = exl3.moe_layout(rows, 2, E, 256, 384, cap)
        _say("capacity", cap, "passes", lay.passes)
        y = moe_forward(x, ids, w, gate, up, down, cap, torch.float32)
        assert torch.equal(y.view(torch.int32), one.view(torch.int32)), cap
    ref = omoe.moe_forward(wl.x, wl.ids, wl.weights_f64, wl.gate, wl.up, wl.down, "R")
    assert _rel_err(one.cpu().double().numpy(), ref) <= TOL


# -------------------------------- bf16 inputs outside the fp16 range at R2
def _bf16_range_rows(n, seed):
    """bf16 rows: 0 normal; 1 a single input of 2e6 (its rotated block
    overflows fp16: |x~| = 2e6 / sqrt(128) > 65504); 2 all inputs ~1e-6
    (x~ in the fp16 subnormal range); 3 inputs ~1000 (bf16-only precision,
    x~ normal); 4 normal plus a few inputs of 4e4; 5 normal."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((6, n)).astype(np.float32)
    v[1, 7] = 2.0e6
    v[2] *= 1e-6
    v[3] *= 1000.0
    v[4, ::37] = 4.0e4
    bits = synth.f32_to_bf16_bits(v)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    return t, synth.bf16_bits_to_f64(bits)


def _check_range_rows(got, ref, expect_bad):
    """Rows whose oracle output is not finite (a rounding point overflowed
    to inf) are exactly the GPU's non-finite rows, and exactly
    ``expect_bad``; every finite row is within the bar relative to its own
    RMS (the tiny row included)."""
    bad_ref = ~np.all(np.isfinite(ref), axis=1)
    bad_gpu = ~np.all(np.isfinite(got), axis=1)
    assert np.array_equal(bad_ref, bad_gpu), (bad_ref, bad_gpu)
    assert sorted(np.nonzero(bad_ref)[0].tolist()) == sorted(expect_bad), bad_ref
    for r in np.nonzero(~bad_ref)[0]:
        if not np.any(ref[r]):  # every a~ of the row underflowed to 0 at R3
            assert not np.any(got[r]), r
        else:
            assert _rel_err(got[r], ref[r]) <= TOL, r


def test_linear_bf16_out_of_fp16_range():
    """x~ = fp16_rne(Hhat(x * suh)) for bf16 x beyond the fp16 range: an
    overflowing rotated input becomes inf (IEEE round to nearest), so that
    row's output is not finite, as in the oracle; subnormal x~ values are
    kept, not flushed."""
    p, _ = _linear_case(256, 384, ((4, 1.0),), 6, seed=11)
    xd, xv = _bf16_range_rows(256, 12)
    dp = exl3.DeviceProj(p, DEV)
    with np.errstate(all="ignore"):
        ref = olinear.linear(xv, p, "R")
    got = linear(xd, dp, torch.float32).cpu().double().numpy()
    _check_range_rows(got, ref, [1])


def test_linear_fp16_subnormal_inputs():
    """fp16 x holding subnormal values is read exactly: the rotation widens
    each fp16 input inside its product with the sign, and a flushed
    subnormal would zero rows 0 and 2 here. Rows: 0 only subnormals; 1
    normal values with every 5th input subnormal; 2 zeros and a few
    subnormals; 3 normal."""
    p, x = _linear_case(256, 384, ((4, 1.0),), 4, seed=21)
    rng = np.random.default_rng(22)
    sub = (rng.integers(-1023, 1024, size=(4, 256)) * 2.0 ** -24).astype(np.float16)
    x[0] = sub[0]
    x[1, ::5] = sub[1, ::5]
    x[2] = 0
    x[2, ::17] = sub[2, ::17]
    assert np.all(np.abs(x[0][x[0] != 0]) < 2.0 ** -14)
    dp = exl3.DeviceProj(p, DEV)
    ref = olinear.linear(x, p, "R")
    got = linear(torch.from_numpy(x).to(DEV), dp, torch.float32).cpu().double().numpy()
    _check_range_rows(got, ref, [])
    assert np.any(got[0]) and np.any(got[2])


def test_moe_bf16_out_of_fp16_range():
    """The same rows through the routed-experts layer (16-row tiles). Row 1
    overflows at R2; rows 3 and 4 overflow at R3 instead: SwiGLU multiplies
    two projections of x, so inputs of 1000 (row 3) and 4e4 (row 4) give
    |Hhat(a * suh_down)| far above 65504, and a~ is inf there, in the oracle
    and on the GPU alike. Row 2 (inputs ~1e-6) gives |a~| ~ 1e-11, which
    rounds to 0 at R3, so its output is exactly zero on both sides."""
    wl = _tiny(rows=6, K=(3, 4, 6, 8))
    gate, up, down, _, ids, w = _moe_inputs(wl)
    xd, xv = _bf16_range_rows(wl.hidden, 13)
    with np.errstate(all="ignore"):
        ref = omoe.moe_forward(xv, wl.ids, wl.weights_f64, wl.gate, wl.up, wl.down, "R")
    got = moe_forward(xd, ids, w, gate, up, down, wl.capacity, torch.float32)
    _check_range_rows(got.cpu().double().numpy(), ref, [1, 3, 4])


# ------------------------------------------- bf16 activations and outputs
def _bf16_x(shape, seed):
    """Seeded bf16 activations: device tensor and the exact values (float64)."""
    v = np.random.default_rng(seed).standard_normal(shape).astype(np.float32)
    v[np.abs(v) < 2.0 ** -14] = 0.0  # every value then also exact in fp16
    bits = synth.f32_to_bf16_bits(v)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    return t, synth.bf16_bits_to_f64(bits)


def _check_out16(y32, y16, dtype):
    """A 16-bit output equals torch's CPU round-to-nearest-even of the fp32 one."""
    want = y32.cpu().to(dtype).view(torch.int16).numpy()
    assert np.array_equal(y16.cpu().view(torch.int16).numpy(), want), dtype


@pytest.mark.parametrize("fin,fout,stages,rows", [
    (256, 384, ((3, 1.0), (2, 0.37)), 33), (256, 8192, ((4, 1.0),), 1024)])
def test_linear_bf16_activations_and_outputs(fin, fout, stages, rows):
    """bf16 x is read exactly (the rotated rows still round to fp16); bf16
    and fp16 outputs are the fp32 output rounded to nearest even."""
    _say("linear bf16", fin, fout, rows)
    p, _ = _linear_case(fin, fout, stages, rows, seed=fin + fout + rows)
    xd, xv = _bf16_x((rows, fin), seed=rows)
    dp = exl3.DeviceProj(p, DEV)
    y32 = linear(xd, dp, torch.float32)
    yb = linear(xd, dp, torch.bfloat16)
    yh = linear(xd, dp, torch.float16)
    torch.cuda.synchronize()
    sample = list(range(rows)) if rows <= 64 else [0, 5, rows - 1]
    ref = olinear.linear(xv[sample], p, "R")
    assert _rel_err(y32.cpu().double().numpy()[sample], ref) <= TOL
    _check_out16(y32, yb, torch.bfloat16)
    _check_out16(y32, yh, torch.float16)
    # an fp16 x holding the same values gives the same bytes
    xh = torch.from_numpy(xv.astype(np.float16)).to(DEV)
    assert np.array_equal(xh.cpu().double().numpy(), xv)
    assert torch.equal(linear(xh, dp, torch.float32).view(torch.int32),
                       y32.view(torch.int32))


@pytest.mark.parametrize("case", ["tiny", "one_row", "wide", "wide_pipelined"])
def test_moe_bf16_activations_and_outputs(case):
    """bf16 x through every launch form (16-row tiles, the one-launch decode
    pack + rotation, 128-row tiles in one pass and pipelined over 6 passes);
    bf16 output equal to RNE of the fp32 output."""
    _say("moe bf16", case)
    if case == "tiny":
        wl, cap = _tiny(K=(2, 3, 5, 8)), None
    elif case == "one_row":
        wl, cap = _tiny(rows=1, topk=8, E=16, K=(3, 4)), None
    else:
        wl, cap = _wide_wl(), (100 if case == "wide_pipelined" else 10 ** 6)
    cap = wl.capacity if cap is None else cap
    gate, up, down, _, ids, w = _moe_inputs(wl)
    xd, xv = _bf16_x((wl.rows, wl.hidden), seed=len(case))
    y32 = moe_forward(xd, ids, w, gate, up, down, cap, torch.float32)
    yb = moe_forward(xd, ids, w, gate, up, down, cap, torch.bfloat16)
    torch.cuda.synchronize()
    ref = omoe.moe_forward(xv, wl.ids, wl.weights_f64, wl.gate, wl.up, wl.down, "R")
    assert _rel_err(y32.cpu().double().numpy(), ref) <= TOL
    _check_out16(y32, yb, torch.bfloat16)
    if case == "wide_pipelined":
        y1 = moe_forward(xd, ids, w, gate, up, down, 10 ** 6, torch.float32)
        assert torch.equal(y1.view(torch.int32), y32.view(torch.int32))
        meta = exl3.exl3_route_pack(ids, w, wl.num_experts)
        ya = moe_additive(xd, wl.topk, meta, gate, up, down, cap, torch.bfloat16)
        assert torch.equal(ya.view(torch.int16), yb.view(torch.int16))


# ------------------------------------------ prefill workload at full scale
def _ulp_dist(a16, b16):
    """Distance in fp16 ulps between two fp16 arrays (ordered bit patterns)."""
    def ordered(v):
        i = v.view(np.uint16).astype(np.int32)
        return np.where(i & 0x8000, 0x8000 - (i & 0x7FFF), 0x8000 + i)
    return np.abs(ordered(a16) - ordered(b16))


def _greedy_rows(ids, needs, min_rows, exclude=()):
    """Rows chosen by rule: for every need (a set of candidate rows), the
    candidate that adds the fewest experts not yet covered; then rows adding
    the fewest new experts until ``min_rows`` rows are chosen."""
    chosen, experts = [], set()

    def take(cands):
        cands = [r for r in cands if r not in chosen and r not in exclude]
        if not cands:
            return
        r = min(cands, key=lambda r: (len(set(map(int, ids[r])) - experts), r))
        chosen.append(r)
        experts.update(map(int, ids[r]))

    for cands in needs:
        if not any(r in chosen for r in cands):
            take(cands)
    while len(chosen) < min_rows:
        take(range(ids.shape[0]))
    return chosen


def _prefill_rows(wl, pack):
    """Sampled rows of the prefill workload, by rule: a pair routed to an
    expert of every width K; both sides of two expert spans that a pass
    boundary cuts (the rows of the positions just before and at the cut; of
    all such cuts, the two whose rows bring the fewest experts); the last
    row of the first and of the last partial 128-row tile (spans of a pass
    whose length is not a multiple of 128); at least 8 rows, sharing experts
    where possible."""
    ids, topk, cap = wl.ids, wl.topk, wl.capacity
    K = wl.extra["K_per_expert"]
    off, pop = pack["offset"], pack["pair_of_pos"]
    needs = []
    for k in sorted(set(int(v) for v in K)):
        needs.append([r for r in range(wl.rows) if any(K[int(e)] == k for e in ids[r])])
    kept = int(off[-1])
    cuts = [b for b in range(cap, kept, cap)
            if any(off[e] < b < off[e + 1] for e in range(wl.num_experts))]
    sides = [(int(pop[b - 1]) // topk, int(pop[b]) // topk) for b in cuts]
    sides.sort(key=lambda rr: (len(set(map(int, ids[rr[0]])) | set(map(int, ids[rr[1]]))), rr))
    for r0, r1 in sides[:2]:
        needs.append([r0])
        needs.append([r1])
    partial = []
    for p in range((kept + cap - 1) // cap):
        for e in range(wl.num_experts):
            lo, hi = max(off[e], p * cap), min(off[e + 1], (p + 1) * cap)
            if hi > lo and (hi - lo) % 128:
                partial.append(int(pop[hi - 1]) // topk)
    needs.append(partial[:1])
    needs.append(partial[-1:])
    return _greedy_rows(ids, needs, 8), len(cuts)


_U = 2.0 ** -24          # fp32 unit roundoff
_R128 = 1.0 / np.sqrt(128.0)


def _gamma(n, u):
    return n * u / (1.0 - n * u)


def _bsum(v):
    """Sum over each contiguous 128-block, broadcast back to the block."""
    b = v.reshape(*v.shape[:-1], -1, 128)
    return np.broadcast_to(b.sum(-1, keepdims=True), b.shape).reshape(v.shape)


def _at_error_model(xr, e, gate, up, down, cache):
    """Oracle-side error analysis of the rotated down input a~ of one pair.

    The GPU's x~ equals the oracle's (checked bit for bit), so a~ differs
    only by fp32 rounding inside the GPU's gate/up projection, its output
    rotation, SwiGLU and the down-input rotation, then the fp16 rounding R3.
    Returns (a~ exact before R3, deterministic bound, sigma), per element:
      deterministic  every dot product of in_f exact products summed with at
                     most in_f roundings of relative size <= 2u (Higham's
                     gamma_n; 2u also covers truncating hardware), each
                     128-point FWHT with 7 levels of rounded adds, every
                     multiply rounded, silu within 5u (expf within 2 ulp,
                     a correctly rounded divide) and |silu'| <= 1.1;
      sigma          the same steps with independent mean-zero roundings
                     (|delta| <= u) whose effects add in quadrature, the dot
                     product taken as rounding after every one of its in_f
                     terms (partial sums S_i: var = u^2/3 sum S_i^2)."""
    outs = {}
    for name, P in (("g", gate), ("u", up)):
        xt = olinear.rotate_input(xr, P, e, "R")[0]
        W = cache.get(P, 0, e)
        acc = xt @ W
        dacc = _gamma(W.shape[0], 2 * _U) * (np.abs(xt) @ np.abs(W))
        sacc = _U * np.sqrt((np.cumsum(xt[:, None] * W, axis=0) ** 2).sum(0) / 3.0)
        cs = np.abs(np.asarray(P.chscale[e], np.float64))
        y = olinear.rotate_output(acc[None], P, e)[0]
        dv = _bsum(dacc) + _gamma(7, _U) * (_bsum(np.abs(acc)) + _bsum(dacc))
        dy = cs * _R128 * dv * (1 + 4 * _U) + 4.1 * _U * np.abs(y)
        sy = cs * _R128 * np.sqrt(_bsum(sacc ** 2) + 7.0 / 3.0 * _U ** 2 * _bsum(acc ** 2)) \
            + _U * np.abs(y)
        outs[name] = (y, dy, sy)
    (g, dg, sg), (u, du, su) = outs["g"], outs["u"]
    sig = 1.0 / (1.0 + np.exp(-g))
    sil = g * sig
    dsil = np.abs(sig * (1.0 + g * (1.0 - sig)))
    a = sil * u
    ds = 1.1 * dg + 5 * _U * np.abs(sil)
    da = ds * np.abs(u) + np.abs(sil) * du + ds * du
    da = da + _U * (np.abs(a) + da)
    ss = dsil * sg + 2 * _U * np.abs(sil)
    sa = np.sqrt((ss * u) ** 2 + (sil * su) ** 2) + _U * np.abs(a)
    suh = np.asarray(down.suh[e], np.float64)
    from oracle.hadamard import rotate_blocks
    at = rotate_blocks(a * suh)
    dv2 = _bsum(da) + _gamma(7, _U) * (_bsum(np.abs(a)) + _bsum(da))
    bound = dv2 * _R128 * (1 + 2 * _U) + 2.1 * _U * np.abs(at)
    sigma = _R128 * np.sqrt(_bsum(sa ** 2) + 7.0 / 3.0 * _U ** 2 * _bsum(a ** 2))
    return at, bound, sigma


def _spacing16(v):
    """fp16 ulp at |v| (the spacing above the fp16 value nearest |v|)."""
    return np.spacing(np.float16(np.minimum(np.abs(v), 65504.0))).astype(np.float64)


def test_prefill_workload_full_scale():
    """The mixed-width prefill layer at its full size: 192 experts, top-8,
    hidden 6144, intermediate 2048, K per expert in {3,4,5,6,8}, 3072 rows,
    Zipf(1.2) routing, capacity 2048 pairs (12 passes, expert spans cut across
    passes), in the launch configuration the benchmark times. Rows are
    sampled by rule (_prefill_rows). Checks:
      - 12 passes equal one pass bit for bit;
      - R2: the rotated gate/up inputs x~ of every sampled pair, read from the
        one-pass workspace, equal the oracle's bit for bit;
      - R3: the rotated down input a~ against the oracle's, per element,
        within the deterministic worst-case bound plus one fp16 ulp, and
        within 8 sigma of the rounding-error model plus one ulp (a rounding
        model failure probability of about 1e-14 per element); the number
        of elements a whole ulp or more apart is at most 1.5x the model's
        expectation (+ 3 sqrt + 5);
      - the down projection + combine teacher-forced with the GPU's a~, and
        the rows end to end, within the 2e-3 RMS-relative bar."""
    from oracle import route as oroute
    from oracle.linear import WeightCache
    _say("prefill workload: drawing inputs")
    wl = synth.moe_workload("prefill", materialize=False)
    P = wl.rows * wl.topk
    counts = np.bincount(wl.ids.reshape(-1), minlength=wl.num_experts)
    assert int(np.sum(counts > wl.capacity)) >= 2
    pack = oroute.route_pack(wl.ids, wl.weights_f64, wl.num_experts)
    sample, ncuts = _prefill_rows(wl, pack)
    experts = sorted({int(wl.ids[r, j]) for r in sample for j in range(wl.topk)})
    _say("  sampled rows %s (%d experts, K %s, %d cut spans)" % (
        sample, len(experts), sorted({int(wl.extra["K_per_expert"][e]) for e in experts}), ncuts))
    assert ncuts >= 2 and len(sample) >= 8
    gate, up, down = (exl3.DeviceProj(p, DEV, words_fn=synth.realize_words)
                      for p in (wl.gate, wl.up, wl.down))
    x, ids, w = exl3.device_inputs(wl, DEV)
    _say("prefill workload: 12-pass forward")
    y = moe_forward(x, ids, w, gate, up, down, wl.capacity, torch.float32)
    _say("prefill workload: one-pass forward")
    lay = exl3.moe_layout(wl.rows, wl.topk, wl.num_experts, wl.hidden, wl.intermediate, P)
    assert lay.passes == 1
    ws = torch.empty(lay.total, dtype=torch.uint8, device=DEV)
    y1 = moe_forward(x, ids, w, gate, up, down, P, torch.float32, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), y1.view(torch.int32))

    H, I = wl.hidden, wl.intermediate
    xt_all = ws[lay.xt:lay.xt + P * 2 * H * 2].view(torch.float16).view(P, 2, H)
    at_all = ws[lay.at:lay.at + P * I * 2].view(torch.float16).view(P, I)
    views = [synth.materialized_view(p, set(experts)) for p in (wl.gate, wl.up, wl.down)]
    cache = WeightCache()
    y_tf = np.zeros((len(sample), H))
    y_e2e = np.zeros((len(sample), H))
    n_el = flips = 0
    expect = 0.0
    worst_det = worst_sig = 0.0
    ulps = []
    for li, r in enumerate(sample):
        _say("  oracle row %d (%d of %d)" % (r, li + 1, len(sample)))
        xr = wl.x[r:r + 1].astype(np.float64)
        for j in range(wl.topk):
            e = int(wl.ids[r, j])
            pos = int(pack["pos_of_pair"][r * wl.topk + j])
            xt_gpu = exl3.unpermute_rotated(xt_all[pos]).cpu().numpy()
            for pj, proj in enumerate(views[:2]):
                xt_ref = olinear.rotate_input(xr, proj, e, "R")[0].astype(np.float16)
                assert np.array_equal(xt_gpu[pj].view(np.uint16), xt_ref.view(np.uint16)), (r, j, pj)
            at_exact, det, sig = _at_error_model(xr, e, *views, cache)
            at_ref = at_exact.astype(np.float16).astype(np.float64)  # oracle R3
            at_gpu = exl3.unpermute_rotated(at_all[pos]).cpu().numpy()
            diff = np.abs(at_gpu.astype(np.float64) - at_ref)
            ulp = _spacing16(np.abs(at_exact) + det)
            worst_det = max(worst_det, float(np.max(diff / (det + ulp))))
            ulp_s = _spacing16(np.abs(at_exact) + 8 * sig)
            worst_sig = max(worst_sig, float(np.max(diff / (8 * sig + ulp_s))))
            u_el = _ulp_dist(at_gpu, at_exact.astype(np.float16))
            ulps.append(u_el.max())
            flips += int(np.sum(u_el > 0))
            n_el += at_exact.size
            expect += float(np.sum(np.minimum(1.0, sig * np.sqrt(2 / np.pi) / _spacing16(at_exact))))
            wt = wl.weights_f64[r, j]
            y_tf[li] += wt * omoe.down_output(at_gpu.astype(np.float64)[None], e, views[2], cache)[0]
            y_e2e[li] += wt * omoe.down_output(at_ref[None], e, views[2], cache)[0]
    got = y.cpu().double().numpy()[sample]
    e_tf, e_e2e = _rel_err(got, y_tf), _rel_err(got, y_e2e)
    _say("  x~ bit-exact; a~: %d of %d elements off by >= 1 ulp (%.3f%%; model expects %.1f = "
         "%.3f%%), max %d ulp; max |diff| / (det bound + ulp) %.3g, / (8 sigma + ulp) %.3f; "
         "teacher-forced err %.3e; end-to-end err %.3e"
         % (flips, n_el, 100.0 * flips / n_el, expect, 100.0 * expect / n_el, max(ulps),
            worst_det, worst_sig, e_tf, e_e2e))
    assert worst_det <= 1.0
    assert worst_sig <= 1.0
    assert flips <= 1.5 * expect + 3 * np.sqrt(expect) + 5
    assert e_tf <= TOL
    assert e_e2e <= TOL


# ------------------------------------------- tensor-parallel shard shapes
# One GPU's share of the layer under 4-way tensor parallelism: the
# intermediate size split into 128-aligned quarters (decode 1536 / 4 = 384,
# prefill 2048 / 4 = 512), hidden size and routing unchanged.
def test_tp4_shard_decode_sampled():
    _say("tp4 shard decode M=32, I=384")
    wl = synth.moe_workload("decode", rows=32, I=384)
    assert _sampled_parity(wl, [0, 31], 32 * 8) <= TOL


def test_tp4_shard_prefill_sampled():
    """1536 rows of the prefill layer at I = 512: 12288 pairs = 64 per expert,
    so 128-row tiles, and capacity 2048 makes 6 passes. Checks 6 passes
    against one pass bit for bit, and sampled rows end to end against the
    oracle."""
    _say("tp4 shard prefill: drawing inputs")
    wl = synth.moe_workload("prefill", rows=1536, I=512, materialize=False)
    P = wl.rows * wl.topk
    lay = exl3.moe_layout(wl.rows, wl.topk, wl.num_experts, wl.hidden, wl.intermediate,
                          wl.capacity)
    assert lay.passes == 6
    gate, up, down = (exl3.DeviceProj(p, DEV, words_fn=synth.realize_words)
                      for p in (wl.gate, wl.up, wl.down))
    x, ids, w = exl3.device_inputs(wl, DEV)
    _say("tp4 shard prefill: 6-pass and one-pass forwards")
    y = moe_forward(x, ids, w, gate, up, down, wl.capacity, torch.float32)
    y1 = moe_forward(x, ids, w, gate, up, down, P, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), y1.view(torch.int32))
    sample = [0, wl.rows - 1]
    experts = {int(wl.ids[r, j]) for r in sample for j in range(wl.topk)}
    views = [synth.materialized_view(p, experts) for p in (wl.gate, wl.up, wl.down)]
    ref = np.zeros((len(sample), wl.hidden))
    for li, r in enumerate(sample):
        for j in range(wl.topk):
            e = int(wl.ids[r, j])
            at_ref = omoe.stage1(wl.x[r:r + 1].astype(np.float64), e, *views, "R")
            ref[li] += wl.weights_f64[r, j] * omoe.down_output(at_ref, e, views[2])[0]
    err = _rel_err(y.cpu().double().numpy()[sample], ref)
    _say("  sampled rows", sample, "err %.3e" % err)
    assert err <= TOL


# ------------------------------------- graph capture and cartridge swapping
def test_additive_graph_capture_cartridge_swap():
    """exl3_moe_additive captured once in a graph; between replays only the
    contents of the residual-stage tables change (pointer and scale rows of
    stage 1: cartridge A -> cartridge B -> no residual -> A). Every replay
    equals an eager call with the same tables bit for bit, and restoring the
    tables restores the output bytes (exllamav3 PR #284 "MoE: Add fused
    additive EXL3 kernels", Summary and API contract: graph-safe additive
    stages; table contents may change between replays)."""
    small = dict(rows=24, E=16, topk=4, H=256, I=512)
    wa = synth.moe_workload("additive", **small)
    wb = synth.moe_workload("additive", seed=77, **small)

    def with_residual(p, q):
        return synth.Proj(p.in_features, p.out_features, p.num_experts,
                          [p.words[0], q.words[1]], np.stack([p.scale[0], q.scale[1]]),
                          np.stack([p.bits[0], q.bits[1]]), p.suh, p.svh, p.chscale)

    projs_a = [exl3.DeviceProj(p, DEV) for p in (wa.gate, wa.up, wa.down)]
    projs_b = [exl3.DeviceProj(with_residual(p, q), DEV)
               for p, q in zip((wa.gate, wa.up, wa.down), (wb.gate, wb.up, wb.down))]
    x, ids, w = exl3.device_inputs(wa, DEV)
    meta = exl3.exl3_route_pack(ids, w, wa.num_experts)
    cap = wa.rows * wa.topk
    need = exl3.moe_workspace_size(wa.rows, wa.topk, wa.num_experts, wa.hidden,
                                   wa.intermediate, cap)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    out = torch.empty(wa.rows, wa.hidden, dtype=torch.float32, device=DEV)
    saved = [(p.trellis.clone(), p.scale.clone()) for p in projs_a]

    def set_cartridge(src):
        for p, s in zip(projs_a, src):
            p.trellis[1].copy_(s[0][1])
            p.scale[1].copy_(s[1][1])

    def eager():
        y = moe_additive(x, wa.topk, meta, *projs_a, cap, torch.float32)
        torch.cuda.synchronize()
        return y.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moe_additive(x, wa.topk, meta, *projs_a, cap, torch.float32, out=out, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        exl3.exl3_moe_additive(x, wa.topk, meta, *projs_a, cap, torch.float32, out=out, ws=ws)
    torch.cuda.synchronize()

    def replay():
        out.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _ctrl(ws)[:3] == [0, 0, 0]
        return out.clone()

    bits = lambda t: t.view(torch.int32)
    ya = replay()
    assert torch.equal(bits(ya), bits(eager()))
    set_cartridge([(p.trellis, p.scale) for p in projs_b])
    yb = replay()
    assert torch.equal(bits(yb), bits(eager()))
    assert not torch.equal(bits(yb), bits(ya))
    for p in projs_a:
        p.scale[1].zero_()
    y0 = replay()
    assert torch.equal(bits(y0), bits(eager()))
    set_cartridge(saved)
    assert torch.equal(bits(replay()), bits(ya))
    # the replayed outputs also meet the oracle bar (cartridge A)
    ref = omoe.moe_forward(wa.x, wa.ids, wa.weights_f64, wa.gate, wa.up, wa.down, "R")
    assert _rel_err(ya.cpu().double().numpy(), ref) <= TOL
