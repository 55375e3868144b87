"""Seeded synthetic inputs shared by the tests and the benchmark.

This module only draws random inputs: it holds none of the layer's
arithmetic (no decode, no rotation, no routing pack, no GEMM). Both the HIP
library and the float64 oracle consume the arrays it returns.

Every array is a pure function of (workload seed, role, stage, expert), so a
sampled expert can be regenerated alone without drawing the whole layer.

Workloads (sizes and distributions of the EXL3 MoE shapes being modelled):
  tiny     8 experts, top-2, 16 rows, hidden 256, intermediate 512, K=4;
           router logits N(0,1), top-k by logit, softmax of the selected
           logits in fp32; int32 IDs
  linear   one 4096->4096 projection, K in {2,3,4,8}, rows 1/7/32/128/2048
  decode   128 experts, top-8, hidden 4096, intermediate 1536, K=4,
           rows 1/8/32; uniform routing; bf16 weights; int64 IDs
  prefill  192 experts, top-8, hidden 6144, intermediate 2048, K per expert
           from {3,4,5,6,8}, 3072 rows; Zipf(1.2) popularity; fp16 weights;
           int32 IDs
  additive 256 experts, top-8, hidden 4096, intermediate 2048, 128 rows;
           base K=3 plus one K=2 residual stage per projection with scales
           N(0, 0.1^2), exactly 77 of 256 scales per projection set to 0.0
           (half of those with a null trellis); fp32 weights; int64 IDs
Common: activations fp16 N(0,1); trellis words uniform random bits;
suh/svh uniform +-1; per-output-channel scales fp16(|N(0,1)| * 0.05).
"""

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

ROLE_IDS = {"gate": 1, "up": 2, "down": 3, "linear": 4}


def _rng(*key):
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def words_per_tensor(in_features, out_features, K):
    return (in_features // 16) * (out_features // 16) * 16 * K


def random_words(n, *key):
    """n uniform random uint16 trellis words for the given key."""
    return np.frombuffer(_rng(*key).bytes(2 * n), dtype=np.uint16).copy()


def f32_to_bf16_bits(v):
    """Round fp32 values to bf16 (nearest-even); returns uint16 bit patterns."""
    b = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(
        np.float32).astype(np.float64)


@dataclass
class Proj:
    """One projection (gate, up, down or a plain linear) of all experts.

    ``words[t][e]`` is the flat uint16 trellis of stage t of expert e in the
    tensor order [out/16][in/16][16*K], or None for a sparse zero-scale entry.
    """
    in_features: int
    out_features: int
    num_experts: int
    words: List[List[Optional[np.ndarray]]]
    scale: np.ndarray          # float32 [T][E]
    bits: np.ndarray           # int32 [T][E]
    suh: np.ndarray            # float16 [E][in]
    svh: np.ndarray            # float16 [E][out]
    chscale: np.ndarray        # float16 [E][out]

    @property
    def num_stages(self):
        return len(self.words)


def make_proj(seed, role, E, in_f, out_f, bits, scale, null_mask=None,
              materialize=True):
    """Draw one projection. ``bits``/``scale``: [T][E] arrays; entries with
    ``null_mask`` set get no trellis (their scale must be 0)."""
    rid = ROLE_IDS[role]
    bits = np.asarray(bits, dtype=np.int32)
    scale = np.asarray(scale, dtype=np.float32)
    T = bits.shape[0]
    words = []
    for t in range(T):
        row = []
        for e in range(E):
            if null_mask is not None and null_mask[t][e]:
                row.append(None)
            elif materialize:
                n = words_per_tensor(in_f, out_f, int(bits[t][e]))
                row.append(random_words(n, seed, rid, 100 + t, e))
            else:
                row.append(("lazy", seed, rid, 100 + t, e))
        words.append(row)
    r = _rng(seed, rid, 1)
    suh = np.where(r.random((E, in_f)) < 0.5, -1.0, 1.0).astype(np.float16)
    svh = np.where(r.random((E, out_f)) < 0.5, -1.0, 1.0).astype(np.float16)
    cs = (np.abs(r.standard_normal((E, out_f))) * 0.05).astype(np.float16)
    return Proj(in_f, out_f, E, words, scale, bits, suh, svh, cs)


def realize_words(proj, t, e):
    """Materialise lazily described trellis words of (stage t, expert e)."""
    w = proj.words[t][e]
    if isinstance(w, tuple):
        _, seed, rid, tt, ee = w
        n = words_per_tensor(proj.in_features, proj.out_features,
                             int(proj.bits[t][e]))
        w = random_words(n, seed, rid, tt, ee)
    return w


def materialized_view(proj, experts):
    """A copy of ``proj`` whose words are real arrays for ``experts`` only."""
    words = [[realize_words(proj, t, e) if e in experts else None
              for e in range(proj.num_experts)] for t in range(proj.num_stages)]
    return Proj(proj.in_features, proj.out_features, proj.num_experts, words,
                proj.scale, proj.bits, proj.suh, proj.svh, proj.chscale)


@dataclass
class MoEWorkload:
    name: str
    rows: int
    topk: int
    num_experts: int
    hidden: int
    intermediate: int
    x: np.ndarray              # float16 [rows][hidden]
    ids: np.ndarray            # int32 or int64 [rows][topk]
    weights_bits: np.ndarray   # raw route weights (fp16/fp32 values or bf16 bits)
    weights_dtype: str         # "f16" | "bf16" | "f32"
    gate: Proj
    up: Proj
    down: Proj
    capacity: int
    extra: dict = field(default_factory=dict)

    @property
    def weights_f64(self):
        """Exact float64 values of the route weights."""
        if self.weights_dtype == "bf16":
            return bf16_bits_to_f64(self.weights_bits)
        return np.asarray(self.weights_bits).astype(np.float64)


def _activations(seed, rows, hidden):
    return _rng(seed, 7).standard_normal((rows, hidden)).astype(np.float16)


def _uniform_routes(seed, rows, E, topk):
    r = _rng(seed, 8)
    ids = np.argsort(r.random((rows, E)), axis=1)[:, :topk]
    logits = r.standard_normal((rows, topk))
    w = np.exp(logits - logits.max(axis=1, keepdims=True))
    return ids, (w / w.sum(axis=1, keepdims=True)).astype(np.float32)


def _logit_routes(seed, rows, E, topk):
    """Router logits N(0,1); top-k by logit (ties to the lower ID); softmax
    of the selected logits in fp32."""
    logits = _rng(seed, 8).standard_normal((rows, E)).astype(np.float32)
    ids = np.argsort(-logits, axis=1, kind="stable")[:, :topk]
    sel = np.take_along_axis(logits, ids, axis=1)
    w = np.exp(sel - sel.max(axis=1, keepdims=True))
    return ids, (w / w.sum(axis=1, keepdims=True)).astype(np.float32)


def _zipf_routes(seed, rows, E, topk, s=1.2):
    """Zipf(s) expert popularity over a seeded rank->id permutation; top-k
    without replacement by Gumbel-top-k; softmax of N(0,1) logits."""
    r = _rng(seed, 8)
    perm = r.permutation(E)
    p = np.empty(E)
    p[perm] = np.arange(1, E + 1, dtype=np.float64) ** (-s)
    p /= p.sum()
    g = -np.log(-np.log(r.random((rows, E))))
    ids = np.argsort(-(np.log(p)[None, :] + g), axis=1, kind="stable")[:, :topk]
    logits = r.standard_normal((rows, topk))
    w = np.exp(logits - logits.max(axis=1, keepdims=True))
    return ids, (w / w.sum(axis=1, keepdims=True)).astype(np.float32)


def _cast_weights(w, dtype):
    if dtype == "f16":
        return w.astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(w)
    return w.astype(np.float32)


def routes(kind, seed, rows, E, topk, wdtype, idtype=np.int64):
    """Only the routing of a workload: (ids, raw weights) for a fresh seed."""
    router = {"uniform": _uniform_routes, "logit": _logit_routes,
              "zipf": _zipf_routes}[kind]
    ids, w = router(seed, rows, E, topk)
    return ids.astype(idtype), _cast_weights(w, wdtype)


def moe_workload(name, rows=None, seed=None, capacity=None, materialize=True,
                 **over):
    """Build one of the MoE workloads (tiny, decode, prefill, additive),
    optionally with overridden sizes (for small parity variants)."""
    base = {
        "tiny": dict(seed=1, E=8, topk=2, H=256, I=512, rows=16, K=4,
                     route="logit", wdtype="f32", idtype=np.int32),
        "decode": dict(seed=3, E=128, topk=8, H=4096, I=1536, rows=1, K=4,
                       route="uniform", wdtype="bf16", idtype=np.int64),
        "prefill": dict(seed=4, E=192, topk=8, H=6144, I=2048, rows=3072,
                        K=(3, 4, 5, 6, 8), route="zipf", wdtype="f16",
                        idtype=np.int32, capacity=2048),
        "additive": dict(seed=5, E=256, topk=8, H=4096, I=2048, rows=128,
                         K=3, K_res=2, route="uniform", wdtype="f32",
                         idtype=np.int64),
    }[name]
    cfg = dict(base)
    cfg.update(over)
    if rows is not None:
        cfg["rows"] = rows
    if seed is not None:
        cfg["seed"] = seed
    sd, E, k, H, I, M = (cfg["seed"], cfg["E"], cfg["topk"], cfg["H"],
                         cfg["I"], cfg["rows"])

    r = _rng(sd, 2)
    if isinstance(cfg["K"], tuple):
        kexp = r.choice(np.array(cfg["K"]), size=E)
    else:
        kexp = np.full(E, cfg["K"])
    projs = {}
    for role, (fi, fo) in (("gate", (H, I)), ("up", (H, I)), ("down", (I, H))):
        if "K_res" in cfg:
            rr = _rng(sd, 3, ROLE_IDS[role])
            s1 = (rr.standard_normal(E) * 0.1).astype(np.float32)
            nz = int(round(0.3 * E))
            zero = rr.permutation(E)[:nz]
            s1[zero] = 0.0
            null = np.zeros((2, E), dtype=bool)
            null[1, zero[: nz // 2]] = True
            bits = np.stack([kexp, np.full(E, cfg["K_res"])])
            scale = np.stack([np.ones(E, np.float32), s1])
            projs[role] = make_proj(sd, role, E, fi, fo, bits, scale, null,
                                    materialize)
        else:
            projs[role] = make_proj(sd, role, E, fi, fo, kexp[None, :],
                                    np.ones((1, E), np.float32), None,
                                    materialize)

    x = _activations(sd, M, H)
    router = {"uniform": _uniform_routes, "logit": _logit_routes,
              "zipf": _zipf_routes}[cfg["route"]]
    ids, w = router(sd, M, E, k)
    ids = ids.astype(cfg["idtype"])
    cap = capacity if capacity is not None else cfg.get("capacity", M * k)
    return MoEWorkload(name, M, k, E, H, I, x, ids,
                       _cast_weights(w, cfg["wdtype"]), cfg["wdtype"],
                       projs["gate"], projs["up"], projs["down"], cap,
                       {"K_per_expert": kexp})


def linear_workload(K, rows, in_f=4096, out_f=4096, seed=2, stages=1,
                    res_K=2, res_scale=0.1):
    """The plain-linear workload: one (in -> out) projection and rows x.

    ``stages`` > 1 adds residual stages at ``res_K`` bits with fixed scales."""
    bits = np.array([[K]] + [[res_K]] * (stages - 1), dtype=np.int32)
    scale = np.array([[1.0]] + [[res_scale * (t + 1)] for t in range(stages - 1)],
                     dtype=np.float32)
    proj = make_proj(seed * 1000 + K, "linear", 1, in_f, out_f, bits, scale)
    x = _activations(seed * 1000 + K, rows, in_f)
    return proj, x
