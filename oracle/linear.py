"""One EXL3 projection with additive trellis stages (oracle side).

What is computed, following the pages:
  * TensorFold #837 (What this changes): the input rotation, then the trellis
    decode feeding the matrix product; a row's result does not depend on the
    other rows.
  * exllamav3 #284 (Summary, API contract): FP32 accumulation and output
    scaling in the inner GEMM; stage-major trellis/scale/bitrate tables with
    entries that may be empty; residual stages reuse the base suh/svh; a zero
    scale skips that stage's GEMM.

Reading used where the pages are silent (the library's format definition):
  x~  = Hhat(x * suh)                       (128-blocks)
  acc = sum over stages t with scale_t != 0 of scale_t * (x~ @ W_t)
  y   = Hhat(acc) * svh * chscale           (128-blocks, output side)
Mode "pure" is exact float64. Mode "R" rounds x~ to fp16 (round-to-nearest-
even) once, the rounding point R2 of the kernels; nothing else is rounded.

A projection object is duck-typed: it needs ``in_features``,
``out_features``, ``num_experts``, ``words[t][e]`` (flat uint16 trellis or
None), ``scale[t][e]`` (fp32), ``bits[t][e]``, ``suh[e]``, ``svh[e]``,
``chscale[e]`` (fp16 arrays). Nothing is imported from the generator.
"""

import numpy as np

from .hadamard import rotate_blocks
from .trellis import dequantize

MODES = ("pure", "R")


def to_f16_rne(v):
    """Round float64 values to the nearest fp16 (ties to even), as float64."""
    return np.asarray(v, dtype=np.float64).astype(np.float16).astype(np.float64)


class WeightCache:
    """Memoises dequantised stage tensors by (projection, stage, expert)."""

    def __init__(self):
        self._d = {}

    def get(self, proj, t, e):
        key = (id(proj), t, e)
        if key not in self._d:
            self._d[key] = dequantize(proj.words[t][e], proj.in_features,
                                      proj.out_features, int(proj.bits[t][e]))
        return self._d[key]


def rotate_input(x_rows, proj, e, mode):
    """x~ = Hhat(x * suh_e), rounded to fp16 in mode R (rounding point R2)."""
    suh = np.asarray(proj.suh[e], dtype=np.float64)
    xt = rotate_blocks(np.asarray(x_rows, dtype=np.float64) * suh)
    return to_f16_rne(xt) if mode == "R" else xt


def stage_accumulate(xt, proj, e, cache):
    """acc = sum_{t: scale != 0} scale_t * (x~ @ W_t) in float64."""
    acc = np.zeros((xt.shape[0], proj.out_features))
    for t in range(len(proj.words)):
        s = float(np.float32(proj.scale[t][e]))
        if s == 0.0:
            continue  # a zero scale skips the stage entirely
        acc += s * (xt @ cache.get(proj, t, e))
    return acc


def rotate_output(acc, proj, e):
    """y = Hhat(acc) * svh_e * chscale_e (no rounding)."""
    svh = np.asarray(proj.svh[e], dtype=np.float64)
    cs = np.asarray(proj.chscale[e], dtype=np.float64)
    return rotate_blocks(acc) * svh * cs


def project(x_rows, proj, e, mode="R", cache=None):
    """Rows of x through expert e of ``proj``; float64 [rows][out]."""
    if mode not in MODES:
        raise ValueError(mode)
    cache = cache or WeightCache()
    xt = rotate_input(x_rows, proj, e, mode)
    return rotate_output(stage_accumulate(xt, proj, e, cache), proj, e)


def linear(x, proj, mode="R", cache=None):
    """exl3_linear: a plain (num_experts == 1) projection of every row."""
    return project(x, proj, 0, mode, cache)
