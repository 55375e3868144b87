"""Pins of the oracle's projection and MoE layer (CPU only)."""

import numpy as np
import pytest

from oracle import brute, hadamard, linear, moe, trellis
from trellis_quantized_moe_amd import synth


def _small_proj(seed, E=1, fin=256, fout=384, stages=((4, 1.0),), null=None):
    bits = np.array([[k] * E for k, _ in stages])
    scale = np.array([[s] * E for _, s in stages], dtype=np.float32)
    return synth.make_proj(seed, "linear", E, fin, fout, bits, scale, null)


def _rel(a, b):
    return np.max(np.abs(a - b)) / np.max(np.abs(b))


def test_linear_pure_equals_dense_brute_force():
    p = _small_proj(3, stages=((3, 1.0), (2, 0.37)))
    x = np.random.default_rng(0).standard_normal((5, 256)).astype(np.float16)
    assert _rel(linear.linear(x, p, "pure"), brute.linear_pure(x, p)) < 1e-12


def test_linear_r_equals_dense_brute_force():
    p = _small_proj(4, stages=((5, 1.0), (2, -0.2)))
    x = np.random.default_rng(1).standard_normal((7, 256)).astype(np.float16)
    assert _rel(linear.linear(x, p, "R"), brute.linear_r(x, p)) < 1e-12


def test_r_mode_is_fp16_rounding_of_rotated_input():
    # R differs from pure only by rounding x~ once (half an fp16 ulp per
    # element); through W and the orthonormal output rotation that moves each
    # output by at most sqrt(128) * max_n (|dx| @ |W|)_n * max|svh * cs|
    p = _small_proj(5)
    x = np.random.default_rng(2).standard_normal((3, 256)).astype(np.float16)
    pure = linear.linear(x, p, "pure")
    r = linear.linear(x, p, "R")
    xt = hadamard.rotate_blocks(x.astype(np.float64) * p.suh[0])
    dx = np.abs(linear.to_f16_rne(xt) - xt)
    assert np.all(dx <= np.abs(xt) * 2.0 ** -11 + 2.0 ** -25)
    W = trellis.dequantize(p.words[0][0], 256, 384, 4)
    bound = np.sqrt(128) * (dx @ np.abs(W)).max(axis=1, keepdims=True)
    assert np.all(np.abs(r - pure) <= bound * np.abs(p.chscale[0]).max() + 1e-12)
    assert np.max(np.abs(r - pure)) > 0      # the rounding is really applied


def test_zero_scale_equals_absent_stage():
    x = np.random.default_rng(3).standard_normal((4, 256)).astype(np.float16)
    with_zero = _small_proj(6, stages=((4, 1.0), (2, 0.0)))
    without = synth.Proj(256, 384, 1, with_zero.words[:1], with_zero.scale[:1],
                         with_zero.bits[:1], with_zero.suh, with_zero.svh,
                         with_zero.chscale)
    nulled = synth.Proj(256, 384, 1, [with_zero.words[0], [None]],
                        with_zero.scale, with_zero.bits, with_zero.suh,
                        with_zero.svh, with_zero.chscale)
    a = linear.linear(x, with_zero, "R")
    assert np.array_equal(a, linear.linear(x, without, "R"))
    assert np.array_equal(a, linear.linear(x, nulled, "R"))


def test_all_zero_and_all_ones_streams_closed_form():
    p = _small_proj(7)
    x = np.random.default_rng(4).standard_normal((2, 256)).astype(np.float16)
    xt = linear.rotate_input(x, p, 0, "R")
    S = xt.sum(axis=1, keepdims=True)
    svh = p.svh[0].astype(np.float64)
    cs = p.chscale[0].astype(np.float64)
    # all-zero stream: every state 0 -> W == 1/8; all-ones: W == 1481/8192.
    # A constant W == c gives acc[n] = c * sum_k x~_k for every n, so the
    # output rotation puts sqrt(128) * c * S at n = 0 mod 128 and 0 elsewhere
    for fill, c in ((0x0000, 0.125), (0xFFFF, 1481 / 8192)):
        p.words[0][0] = np.full_like(p.words[0][0], fill)
        y = linear.linear(x, p, "R")
        expect = np.zeros_like(y)
        expect[:, ::128] = np.sqrt(128) * c * S * svh[::128] * cs[::128]
        assert np.allclose(y, expect, rtol=1e-12, atol=1e-12)


def _tiny_moe(E=8, topk=2, H=256, I=384, rows=6, seed=11, bad=True):
    wl = synth.moe_workload("tiny", rows=rows, seed=seed, E=E, topk=topk, H=H,
                            I=I, K=(2, 3, 4, 8))
    ids = wl.ids.astype(np.int64)
    if bad:
        ids[0, 0] = E + 3       # dropped
        ids[1, 1] = ids[1, 0]   # duplicate expert in one row
    return wl, ids


def test_moe_pure_equals_row_by_row_brute_force():
    wl, ids = _tiny_moe()
    w = wl.weights_f64
    y = moe.moe_forward(wl.x, ids, w, wl.gate, wl.up, wl.down, "pure")
    yb = brute.moe_pure(wl.x, ids, w, wl.gate, wl.up, wl.down)
    assert _rel(y, yb) < 1e-12


def test_moe_r_equals_dense_rounded_path():
    # the R-mode layer rebuilt with dense scipy Hadamard blocks and explicit
    # fp16 roundings at R2 and R3
    wl, ids = _tiny_moe(seed=12)
    w = wl.weights_f64
    y = moe.moe_forward(wl.x, ids, w, wl.gate, wl.up, wl.down, "R")
    hb = {n: brute.block_hadamard(n) for n in (wl.hidden, wl.intermediate)}
    f16 = lambda v: v.astype(np.float16).astype(np.float64)
    x = wl.x.astype(np.float64)
    yb = np.zeros_like(y)
    for r in range(wl.rows):
        for j in range(wl.topk):
            e = int(ids[r, j])
            if not 0 <= e < wl.num_experts:
                continue
            outs = []
            for p in (wl.gate, wl.up):
                xt = f16((x[r] * p.suh[e]) @ hb[p.in_features])
                acc = xt @ brute.stage_sum(p, e)
                outs.append((acc @ hb[p.out_features]) * p.svh[e] * p.chscale[e])
            g, u = outs
            a = g / (1 + np.exp(-g)) * u
            at = f16((a * wl.down.suh[e]) @ hb[wl.intermediate])
            d = (at @ brute.stage_sum(wl.down, e) @ hb[wl.hidden])
            yb[r] += w[r, j] * d * wl.down.svh[e] * wl.down.chscale[e]
    assert _rel(y, yb) < 1e-12


def test_moe_rows_subset_and_stage_split_agree():
    wl, ids = _tiny_moe(seed=13, bad=False)
    w = wl.weights_f64
    full = moe.moe_forward(wl.x, ids, w, wl.gate, wl.up, wl.down, "R")
    sub = moe.moe_forward(wl.x, ids, w, wl.gate, wl.up, wl.down, "R",
                          rows=[4, 1])
    assert np.array_equal(sub, full[[4, 1]])
    # stage1 + down_output reproduce one pair's contribution
    r, j = 2, 1
    e = int(ids[r, j])
    at = moe.stage1(wl.x[r:r + 1].astype(np.float64), e, wl.gate, wl.up,
                    wl.down, "R")
    d = moe.down_output(at, e, wl.down)
    assert np.all(at == at.astype(np.float16).astype(np.float64))
    other = moe.moe_forward(wl.x, ids, w, wl.gate, wl.up, wl.down, "R",
                            rows=[r])
    e2 = int(ids[r, 1 - j])
    at2 = moe.stage1(wl.x[r:r + 1].astype(np.float64), e2, wl.gate, wl.up,
                     wl.down, "R")
    d2 = moe.down_output(at2, e2, wl.down)
    assert _rel(w[r, j] * d + w[r, 1 - j] * d2, other) < 1e-13
