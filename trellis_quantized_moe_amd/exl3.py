"""ctypes binding of libexl3moe.so (C ABI in include/exl3moe.h).

Argument marshalling only: every step of the layer runs in the HIP library.
torch provides device memory and the current stream. If the library is not
built, every call raises; there is no fallback path.
"""

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libexl3moe.so")

F16, BF16, F32, I32, I64 = 1, 2, 3, 4, 5
_DT = {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32,
       torch.int32: I32, torch.int64: I64}
_OUT = {F16: torch.float16, BF16: torch.bfloat16, F32: torch.float32}


def _dt(t):
    """Library dtype code of a tensor; 0 (rejected by the library) if it has none."""
    return _DT.get(t.dtype, 0)


class Exl3Error(RuntimeError):
    pass


class ProjC(ctypes.Structure):
    _fields_ = [("in_features", ctypes.c_int32), ("out_features", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("num_stages", ctypes.c_int32),
                ("trellis", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("bits", ctypes.c_void_p), ("suh", ctypes.c_void_p),
                ("svh", ctypes.c_void_p), ("chscale", ctypes.c_void_p)]


class MetaC(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("expert_count", "expert_offset", "pair_of_pos", "weight_of_pos",
                 "pos_of_pair", "num_active", "status")]


class ProfileC(ctypes.Structure):
    _fields_ = [("events", ctypes.POINTER(ctypes.c_void_p)),
                ("kernel_ids", ctypes.POINTER(ctypes.c_int32)),
                ("cap", ctypes.c_int32), ("n", ctypes.c_int32)]


class LayoutC(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("ctrl", "meta", "expert_of_pos", "plan", "xt", "at", "d", "yacc",
                 "total")] + [("passes", ctypes.c_int32), ("plan_slots", ctypes.c_int32),
                              ("plan_group", ctypes.c_int32)]


_lib = None
_i32, _sz, _vp = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
_PP = ctypes.POINTER(ProfileC)
_SIGS = {
    "exl3_abi_version": (_i32, []),
    "exl3_status_string": (ctypes.c_char_p, [_i32]),
    "exl3_route_pack": (_i32, [_vp, _i32, _vp, _i32, _i32, _i32, _i32,
                               ctypes.POINTER(MetaC), _vp, _PP]),
    "exl3_linear_workspace_size": (_sz, [_i32, _i32, _i32]),
    "exl3_linear": (_i32, [_vp, _i32, _i32, ctypes.POINTER(ProjC), _vp, _i32, _vp, _sz,
                           _vp, _PP]),
    "exl3_moe_workspace_size": (_sz, [_i32] * 6),
    "exl3_moe_forward": (_i32, [_vp, _i32, _i32, _vp, _i32, _vp, _i32, _i32,
                                ctypes.POINTER(ProjC), ctypes.POINTER(ProjC),
                                ctypes.POINTER(ProjC), _vp, _i32, _i32, _i32, _vp, _sz,
                                _vp, _PP]),
    "exl3_moe_forward_static": (_i32, [_vp, _i32, _i32, _vp, _i32, _vp, _i32, _i32,
                                       ctypes.POINTER(ProjC), ctypes.POINTER(ProjC),
                                       ctypes.POINTER(ProjC), _vp, _i32, _i32, _i32, _vp,
                                       _PP]),
    "exl3_moe_additive": (_i32, [_vp, _i32, _i32, _i32, ctypes.POINTER(MetaC),
                                 ctypes.POINTER(ProjC), ctypes.POINTER(ProjC),
                                 ctypes.POINTER(ProjC), _vp, _i32, _i32, _i32, _vp, _sz,
                                 _vp, _PP]),
    "exl3_moe_layout": (_i32, [_i32] * 6 + [ctypes.POINTER(LayoutC)]),
    "exl3_decode_tiles": (_i32, [_vp, _i32, _i32, _vp, _vp, _PP]),
    "exl3_events_create": (_i32, [_i32, ctypes.POINTER(ctypes.c_void_p)]),
    "exl3_events_destroy": (_i32, [_i32, ctypes.POINTER(ctypes.c_void_p)]),
    "exl3_profile_read": (_i32, [_PP, ctypes.POINTER(ctypes.c_float)]),
}
KERNEL_NAMES = {1: "route_pack", 2: "rotate", 3: "gemm_gateup", 4: "gemm_down",
                5: "combine", 6: "gemm_linear", 7: "decode_tiles", 8: "gemm_experts"}


def lib():
    """Load libexl3moe.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise Exl3Error("%s is missing: build it with __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        raise Exl3Error("exl3 status %d: %s" % (status, lib().exl3_status_string(status).decode()))


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _p(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def abi_version():
    return lib().exl3_abi_version()


class DeviceProj:
    """A projection's tables and tensors resident on the GPU.

    ``proj`` is any object with in_features, out_features, num_experts,
    words[t][e] (flat uint16 numpy or None), scale, bits, suh, svh, chscale
    (e.g. ``synth.Proj``). All trellis tensors live in one device buffer,
    each 256-byte aligned; the int64 pointer table addresses into it.
    """

    def __init__(self, proj, device="cuda", words_fn=None):
        S = len(proj.words)
        E = proj.num_experts
        self.in_features, self.out_features = proj.in_features, proj.out_features
        self.num_experts, self.num_stages = E, S
        offs = np.zeros((S, E), dtype=np.int64)
        total = 0
        sizes = {}
        for t in range(S):
            for e in range(E):
                w = proj.words[t][e]
                if w is None:
                    offs[t, e] = -1
                    continue
                n = (proj.in_features // 16) * (proj.out_features // 16) * 16 * int(proj.bits[t][e])
                sizes[(t, e)] = n
                offs[t, e] = total
                total += (2 * n + 255) // 256 * 256
        self.buffer = torch.empty(max(total, 256), dtype=torch.uint8, device=device)
        base = self.buffer.data_ptr()
        for (t, e), n in sizes.items():
            w = proj.words[t][e]
            if words_fn is not None and not isinstance(w, np.ndarray):
                w = words_fn(proj, t, e)
            arr = torch.from_numpy(np.ascontiguousarray(w).view(np.uint8))
            o = int(offs[t, e])
            self.buffer[o:o + 2 * n].copy_(arr, non_blocking=False)
        ptrs = np.where(offs >= 0, offs + base, 0).astype(np.int64)
        self.trellis = torch.from_numpy(ptrs).to(device)
        self.scale = torch.from_numpy(np.asarray(proj.scale, np.float32).copy()).to(device)
        self.bits = torch.from_numpy(np.asarray(proj.bits, np.int32).copy()).to(device)
        self.suh = torch.from_numpy(np.asarray(proj.suh, np.float16).copy()).to(device)
        self.svh = torch.from_numpy(np.asarray(proj.svh, np.float16).copy()).to(device)
        self.chscale = torch.from_numpy(np.asarray(proj.chscale, np.float16).copy()).to(device)
        self.offsets = offs

    def cstruct(self):
        return ProjC(self.in_features, self.out_features, self.num_experts,
                     self.num_stages, self.trellis.data_ptr(), self.scale.data_ptr(),
                     self.bits.data_ptr(), self.suh.data_ptr(), self.svh.data_ptr(),
                     self.chscale.data_ptr())

    def trellis_bytes(self, t, e):
        """Bytes of the (stage, expert) trellis, 0 if absent."""
        if self.offsets[t, e] < 0:
            return 0
        return (self.in_features // 16) * (self.out_features // 16) * 32 * int(
            self.bits[t, e].item())


def alloc_meta(rows, topk, num_experts, device="cuda"):
    P = rows * topk
    i32 = dict(dtype=torch.int32, device=device)
    return {
        "expert_count": torch.empty(num_experts, **i32),
        "expert_offset": torch.empty(num_experts + 1, **i32),
        "pair_of_pos": torch.empty(max(P, 1), **i32),
        "weight_of_pos": torch.empty(max(P, 1), dtype=torch.float32, device=device),
        "pos_of_pair": torch.empty(max(P, 1), **i32),
        "num_active": torch.empty(4, **i32),
        "status": torch.empty(4, **i32),
    }


def _meta_c(m):
    return MetaC(*[m[n].data_ptr() for n in
                   ("expert_count", "expert_offset", "pair_of_pos", "weight_of_pos",
                    "pos_of_pair", "num_active", "status")])


def exl3_route_pack(ids, w, num_experts, meta=None):
    rows, topk = ids.shape
    meta = meta or alloc_meta(rows, topk, num_experts, ids.device)
    mc = _meta_c(meta)
    _check(lib().exl3_route_pack(_p(ids), _DT[ids.dtype], _p(w), _DT[w.dtype], rows, topk,
                                 num_experts, ctypes.byref(mc), _stream(), _prof()))
    return meta


def linear_workspace_size(rows, in_f, out_f):
    return lib().exl3_linear_workspace_size(rows, in_f, out_f)


def exl3_linear(x, proj, out_dtype=torch.float32, out=None, ws=None):
    rows = x.shape[0]
    out = out if out is not None else torch.empty(rows, proj.out_features, dtype=out_dtype,
                                                  device=x.device)
    need = linear_workspace_size(rows, proj.in_features, proj.out_features)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    pc = proj.cstruct()
    _check(lib().exl3_linear(_p(x), _dt(x), rows, ctypes.byref(pc), _p(out), _DT[out.dtype],
                             _p(ws), ws.numel(), _stream(), _prof()))
    return out


def moe_layout(rows, topk, num_experts, hidden, intermediate, capacity):
    lay = LayoutC()
    _check(lib().exl3_moe_layout(rows, topk, num_experts, hidden, intermediate, capacity,
                                 ctypes.byref(lay)))
    return lay


def moe_workspace_size(rows, topk, num_experts, hidden, intermediate, capacity):
    return lib().exl3_moe_workspace_size(rows, topk, num_experts, hidden, intermediate,
                                         capacity)


def exl3_moe_forward(x, ids, w, gate, up, down, capacity, out_dtype=torch.float32,
                     out=None, ws=None, num_active_hint=-1):
    rows, topk = ids.shape
    out = out if out is not None else torch.empty(rows, down.out_features, dtype=out_dtype,
                                                  device=x.device)
    need = moe_workspace_size(rows, topk, gate.num_experts, gate.in_features,
                              gate.out_features, capacity)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    g, u, d = gate.cstruct(), up.cstruct(), down.cstruct()
    _check(lib().exl3_moe_forward(_p(x), _dt(x), rows, _p(ids), _DT[ids.dtype], _p(w),
                                  _DT[w.dtype], topk, ctypes.byref(g), ctypes.byref(u),
                                  ctypes.byref(d), _p(out), _DT[out.dtype], capacity,
                                  num_active_hint,
                                  _p(ws), ws.numel(), _stream(), _prof()))
    return out


def exl3_moe_forward_static(x, ids, w, gate, up, down, capacity, out_dtype=torch.float32,
                            out=None, num_active_hint=-1):
    """exl3_moe_forward on the library's static scratch (no workspace)."""
    rows, topk = ids.shape
    out = out if out is not None else torch.empty(rows, down.out_features, dtype=out_dtype,
                                                  device=x.device)
    g, u, d = gate.cstruct(), up.cstruct(), down.cstruct()
    _check(lib().exl3_moe_forward_static(_p(x), _dt(x), rows, _p(ids), _DT[ids.dtype], _p(w),
                                         _DT[w.dtype], topk, ctypes.byref(g), ctypes.byref(u),
                                         ctypes.byref(d), _p(out), _DT[out.dtype], capacity,
                                         num_active_hint, _stream(), _prof()))
    return out


STATIC_SCRATCH_BYTES = 32 << 20


def exl3_moe_additive(x, topk, meta, gate, up, down, capacity, out_dtype=torch.float32,
                      out=None, ws=None, num_active_hint=-1):
    rows = x.shape[0]
    out = out if out is not None else torch.empty(rows, down.out_features, dtype=out_dtype,
                                                  device=x.device)
    need = moe_workspace_size(rows, topk, gate.num_experts, gate.in_features,
                              gate.out_features, capacity)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    g, u, d = gate.cstruct(), up.cstruct(), down.cstruct()
    mc = _meta_c(meta)
    _check(lib().exl3_moe_additive(_p(x), _dt(x), rows, topk, ctypes.byref(mc),
                                   ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), _p(out),
                                   _DT[out.dtype], capacity, num_active_hint, _p(ws), ws.numel(), _stream(),
                                   _prof()))
    return out


def exl3_decode_tiles(words, K):
    """words: uint16-bit tensor (int16 view) [ntiles * 16K] -> fp16 [ntiles][16][16]."""
    ntiles = words.numel() // (16 * K)
    out = torch.empty(ntiles, 16, 16, dtype=torch.float16, device=words.device)
    _check(lib().exl3_decode_tiles(_p(words), ntiles, K, _p(out), _stream(), _prof()))
    return out


def unpermute_rotated(t):
    """Undo the in-group storage order of rotated vectors read from the
    workspace (slot p of each 16-group holds entry kSigma[p])."""
    sigma = torch.tensor([0, 4, 1, 5, 2, 6, 3, 7, 8, 12, 9, 13, 10, 14, 11, 15],
                         device=t.device)
    shape = t.shape
    g = t.reshape(*shape[:-1], shape[-1] // 16, 16)
    out = torch.empty_like(g)
    out[..., sigma] = g
    return out.reshape(shape)


_active_profile = None


def _prof():
    """The caller-owned timing record of the enclosing ``Profile`` block, or None."""
    return ctypes.byref(_active_profile.c) if _active_profile is not None else None


class Profile:
    """Per-launch kernel timing: ``with Profile(n) as p: ...`` then
    ``p.records`` = [(name, ms), ...]. The events are created on entry and
    destroyed on exit (outside the calls being timed); inside the block every
    call of this module passes the record to the library, which brackets each
    of its launches with the next event pair."""

    def __init__(self, max_launches=4096):
        self.max = max_launches
        self.records = []

    def __enter__(self):
        global _active_profile
        if _active_profile is not None:
            raise Exl3Error("Profile blocks do not nest")
        self._events = (ctypes.c_void_p * (2 * self.max))()
        self._ids = (ctypes.c_int32 * self.max)()
        _check(lib().exl3_events_create(2 * self.max, self._events))
        self.c = ProfileC(self._events, self._ids, self.max, 0)
        _active_profile = self
        return self

    def __exit__(self, *exc):
        global _active_profile
        _active_profile = None
        ms = (ctypes.c_float * self.max)()
        try:
            _check(lib().exl3_profile_read(ctypes.byref(self.c), ms))
            self.records = [(KERNEL_NAMES.get(self._ids[i], str(self._ids[i])), float(ms[i]))
                            for i in range(self.c.n)]
        finally:
            lib().exl3_events_destroy(2 * self.max, self._events)
        return False


def device_inputs(wl, device="cuda"):
    """x, ids and route weights of a synth MoE workload as device tensors."""
    x = torch.from_numpy(np.ascontiguousarray(wl.x).view(np.int16)).view(torch.float16)
    ids = torch.from_numpy(np.ascontiguousarray(wl.ids))
    wb = np.ascontiguousarray(wl.weights_bits)
    if wl.weights_dtype == "bf16":
        w = torch.from_numpy(wb.view(np.int16)).view(torch.bfloat16)
    elif wl.weights_dtype == "f16":
        w = torch.from_numpy(wb.view(np.int16)).view(torch.float16)
    else:
        w = torch.from_numpy(wb.astype(np.float32))
    return x.to(device), ids.to(device), w.to(device)


def f16_tensor(a, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16).view(np.int16)).view(
        torch.float16).to(device)
