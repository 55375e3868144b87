"""Dense dequantise-then-matmul brute force for tiny shapes (oracle side).

Independent of ``oracle.hadamard``: the rotation is a dense block-diagonal
matrix built from ``scipy.linalg.hadamard``. Used to pin the blockwise
oracle (``linear``, ``moe``) on tiny inputs: with every rounding removed the
layer is x @ W_eff with
  W_eff = D(suh) Hb (sum_t s_t W_t) Hb D(svh) D(chscale),
Hb = I (x) H128 / sqrt(128), which is the format definition written as one
matrix (exllamav3 #284, API contract: residual stages reuse the base
rotations; TensorFold #837, What this changes: input rotation, decode,
product).
"""

import numpy as np
import scipy.linalg

from .trellis import dequantize


def block_hadamard(n, block=128):
    h = scipy.linalg.hadamard(block).astype(np.float64) / np.sqrt(block)
    return np.kron(np.eye(n // block), h)


def stage_sum(proj, e):
    W = np.zeros((proj.in_features, proj.out_features))
    for t in range(len(proj.words)):
        s = float(np.float32(proj.scale[t][e]))
        if s != 0.0:
            W += s * dequantize(proj.words[t][e], proj.in_features,
                                proj.out_features, int(proj.bits[t][e]),
                                decoder="window")
    return W


def dense_weight(proj, e):
    """W_eff of expert e as one dense float64 matrix."""
    hi = block_hadamard(proj.in_features)
    ho = block_hadamard(proj.out_features)
    suh = np.asarray(proj.suh[e], dtype=np.float64)
    svh = np.asarray(proj.svh[e], dtype=np.float64)
    cs = np.asarray(proj.chscale[e], dtype=np.float64)
    return (suh[:, None] * hi) @ stage_sum(proj, e) @ (ho * (svh * cs)[None, :])


def linear_pure(x, proj, e=0):
    return np.asarray(x, dtype=np.float64) @ dense_weight(proj, e)


def linear_r(x, proj, e=0):
    """Brute force with the R2 rounding made explicit on dense matrices."""
    hi = block_hadamard(proj.in_features)
    ho = block_hadamard(proj.out_features)
    suh = np.asarray(proj.suh[e], dtype=np.float64)
    xt = (np.asarray(x, dtype=np.float64) * suh) @ hi
    xt = xt.astype(np.float16).astype(np.float64)
    svh = np.asarray(proj.svh[e], dtype=np.float64)
    cs = np.asarray(proj.chscale[e], dtype=np.float64)
    return (xt @ stage_sum(proj, e) @ ho) * svh * cs


def moe_pure(x, ids, weights, gate, up, down):
    """Row-by-row dense MoE, no packing, no rounding."""
    x = np.asarray(x, dtype=np.float64)
    ids = np.asarray(ids)
    w = np.asarray(weights, dtype=np.float64)
    E = gate.num_experts
    dense = {}
    y = np.zeros((x.shape[0], down.out_features))
    for r in range(x.shape[0]):
        for j in range(ids.shape[1]):
            e = int(ids[r, j])
            if not (0 <= e < E):
                continue
            if e not in dense:
                dense[e] = (dense_weight(gate, e), dense_weight(up, e),
                            dense_weight(down, e))
            wg, wu, wd = dense[e]
            g = x[r] @ wg
            u = x[r] @ wu
            a = g / (1.0 + np.exp(-g)) * u
            y[r] += w[r, j] * (a @ wd)
    return y
