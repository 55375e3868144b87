"""Routed-experts layer: gate/up, SwiGLU, down, top-k combine (oracle side).

TensorFold #837 (What this changes) lists the grouped-experts pipeline:
member lists, each expert's rotation, gate and up, SwiGLU, down and the
weighted combine, with a width per expert. exllamav3 #284 (Summary, API
contract) adds additive residual stages sharing the base rotations.

Per kept pair (r, j) with expert e = ids[r][j] and weight w = weights[r][j]:
  g   = gate_e(x_r),  u = up_e(x_r)       projections, no output rounding
  a   = silu(g) * u,   silu(z) = z / (1 + exp(-z))
  a~  = Hhat(a * suh_down_e)              rounded to fp16 in mode R (R3)
  d   = Hhat(sum_t s_t a~ W_down_t) * svh_down_e * chscale_down_e
  y_r = sum_j w * d
The pages leave "GLM's SwiGLU roundings" undefined; this library reads them
as SwiGLU in full precision with a single rounding of the rotated down-
projection input (R3), plus the gate/up input rounding R2. IDs outside
[0, E) contribute nothing. Route weights are used as given.
"""

import numpy as np

from .hadamard import rotate_blocks
from .linear import (MODES, WeightCache, project, rotate_output,
                     stage_accumulate, to_f16_rne)


def silu(z):
    return z / (1.0 + np.exp(-z))


def down_input(g, u, down, e, mode):
    """a~ = Hhat(silu(g) * u * suh_down_e), fp16-rounded in mode R."""
    a = silu(g) * u
    at = rotate_blocks(a * np.asarray(down.suh[e], dtype=np.float64))
    return to_f16_rne(at) if mode == "R" else at


def stage1(x_rows, e, gate, up, down, mode="R", cache=None):
    """Rotated, rounded down-projection input a~ for rows routed to e."""
    cache = cache or WeightCache()
    g = project(x_rows, gate, e, mode, cache)
    u = project(x_rows, up, e, mode, cache)
    return down_input(g, u, down, e, mode)


def down_output(at, e, down, cache=None):
    """Unweighted per-pair down-projection output d from a given a~."""
    cache = cache or WeightCache()
    return rotate_output(stage_accumulate(np.asarray(at, np.float64), down, e,
                                          cache), down, e)


def moe_forward(x, ids, weights, gate, up, down, mode="R", rows=None,
                cache=None):
    """Layer output y (float64) for ``rows`` (default: every row)."""
    if mode not in MODES:
        raise ValueError(mode)
    x = np.asarray(x, dtype=np.float64)
    ids = np.asarray(ids)
    w = np.asarray(weights, dtype=np.float64)
    E = gate.num_experts
    rows = list(range(x.shape[0])) if rows is None else list(rows)
    cache = cache or WeightCache()
    y = np.zeros((len(rows), down.out_features))

    members = {}
    for li, r in enumerate(rows):
        for j in range(ids.shape[1]):
            e = int(ids[r, j])
            if 0 <= e < E:
                members.setdefault(e, []).append((li, r, j))

    for e in sorted(members):
        mem = members[e]
        xr = x[[r for (_, r, _) in mem]]
        at = stage1(xr, e, gate, up, down, mode, cache)
        d = down_output(at, e, down, cache)
        for k, (li, r, j) in enumerate(mem):
            y[li] += w[r, j] * d[k]
    return y
