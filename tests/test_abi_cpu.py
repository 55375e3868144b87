"""C ABI checks that need no GPU: the library loads, exports every function
the header declares, reports its ABI version, and rejects bad arguments on
the host before any device work."""

import ctypes
import os
import re

import pytest

from trellis_quantized_moe_amd import exl3

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "exl3moe.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(exl3_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = exl3.lib()
    names = _declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_status_strings():
    assert exl3.abi_version() == 4
    L = exl3.lib()
    for s in range(0, -10, -1):
        msg = L.exl3_status_string(s).decode()
        assert msg and msg != "unknown status"
    assert L.exl3_status_string(123).decode() == "unknown status"


def test_workspace_sizes():
    L = exl3.lib()
    a = L.exl3_moe_workspace_size(3072, 8, 192, 6144, 2048, 2048)
    b = L.exl3_moe_workspace_size(3072, 8, 192, 6144, 2048, 4096)
    c = L.exl3_moe_workspace_size(3072, 8, 192, 6144, 2048, 10 ** 6)
    assert 0 < a and 0 < b and 0 < c
    # capacity beyond rows*topk does not grow the workspace
    assert c == L.exl3_moe_workspace_size(3072, 8, 192, 6144, 2048, 24576)
    assert L.exl3_moe_workspace_size(4, 2, 8, 200, 512, 8) == 0  # not a multiple of 128
    lay = exl3.moe_layout(3072, 8, 192, 6144, 2048, 2048)
    assert lay.passes == 12 and lay.plan_group == 6
    offs = [lay.ctrl, lay.meta, lay.expert_of_pos, lay.plan, lay.xt, lay.at, lay.d, lay.yacc]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert lay.total == a
    # two buffers (by unit parity) of group * capacity rows each
    rows = lay.plan_group * 2048
    assert lay.at - lay.xt >= 2 * rows * 2 * 6144 * 2
    assert lay.d - lay.at >= 2 * rows * 2048 * 2
    assert lay.yacc - lay.d >= 2 * rows * 6144 * 4
    # a single pass needs a single buffer of every pair
    one = exl3.moe_layout(3072, 8, 192, 6144, 2048, 10 ** 6)
    assert (one.passes, one.plan_group) == (1, 1)
    assert one.at - one.xt >= 24576 * 2 * 6144 * 2
    assert L.exl3_linear_workspace_size(7, 4096, 4096) >= 7 * 4096 * 2


def _proj(**kw):
    d = dict(in_features=256, out_features=512, num_experts=8, num_stages=1,
             trellis=256, scale=512, bits=768, suh=1024, svh=1280, chscale=1536)
    d.update(kw)
    return exl3.ProjC(**d)


def _fwd(gate=None, up=None, down=None, rows=4, topk=2, capacity=8, out_dtype=exl3.F32,
         x_dtype=exl3.F16, ids=4096, ids_dtype=exl3.I32, w=8192, w_dtype=exl3.F32, x=16384, out=32768,
         ws=65536, ws_bytes=1 << 40):
    gate = gate or _proj()
    up = up or _proj()
    down = down or _proj(in_features=512, out_features=256)
    return exl3.lib().exl3_moe_forward(
        ctypes.c_void_p(x), x_dtype, rows, ctypes.c_void_p(ids), ids_dtype, ctypes.c_void_p(w),
        w_dtype, topk, ctypes.byref(gate), ctypes.byref(up), ctypes.byref(down),
        ctypes.c_void_p(out), out_dtype, capacity, -1, ctypes.c_void_p(ws), ws_bytes, None,
        None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=0), -1), (dict(ids=0), -1), (dict(ws=0), -1),
    (dict(ids_dtype=exl3.F16), -2), (dict(w_dtype=exl3.I32), -2), (dict(out_dtype=exl3.I32), -2),
    (dict(x_dtype=exl3.F32), -2), (dict(x_dtype=0), -2),
    (dict(gate=_proj(in_features=200)), -3), (dict(up=_proj(out_features=384)), -3),
    (dict(down=_proj(in_features=512, out_features=128)), -3),
    (dict(up=_proj(num_experts=7)), -3),
    (dict(x=16385), -4), (dict(out=32770), -4),
    (dict(topk=0), -7), (dict(topk=33), -7), (dict(capacity=0), -7), (dict(rows=-1), -7),
    (dict(gate=_proj(num_stages=9)), -7), (dict(gate=_proj(num_experts=2000)), -7),
    (dict(ws_bytes=10), -6),
])
def test_forward_rejects_bad_arguments_before_device_work(kw, code):
    assert _fwd(**kw) == code


def test_rows_zero_is_a_noop():
    assert _fwd(rows=0, x=0, ws=0) == 0


@pytest.mark.parametrize("xdt,odt", [(exl3.BF16, exl3.F32), (exl3.F16, exl3.BF16),
                                     (exl3.BF16, exl3.BF16)])
def test_bf16_activations_and_outputs_pass_validation(xdt, odt):
    # accepted dtypes get as far as the device-pointer check (-5)
    assert _fwd(x_dtype=xdt, out_dtype=odt) == -5


def test_host_pointers_are_rejected_as_not_device():
    # everything valid on the host side; the device check must fail (no GPU
    # here, or host memory on a GPU machine) without launching anything
    assert _fwd() == -5


def _lin(x_dtype=exl3.F16, out_dtype=exl3.F32, proj=None, rows=3, x=16384, out=32768,
         ws=65536, ws_bytes=1 << 40):
    proj = proj or _proj(num_experts=1)
    return exl3.lib().exl3_linear(ctypes.c_void_p(x), x_dtype, rows, ctypes.byref(proj),
                                  ctypes.c_void_p(out), out_dtype, ctypes.c_void_p(ws),
                                  ws_bytes, None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(x_dtype=exl3.F32), -2), (dict(x_dtype=exl3.I64), -2), (dict(out_dtype=exl3.I32), -2),
    (dict(x=0), -1), (dict(proj=_proj(num_experts=2)), -7), (dict(x=16386), -4),
    (dict(ws_bytes=1), -6), (dict(rows=-2), -7),
    # accepted dtypes reach the device check (host pointers here)
    (dict(x_dtype=exl3.BF16, out_dtype=exl3.BF16), -5), (dict(out_dtype=exl3.F16), -5),
])
def test_linear_validates_dtypes_and_arguments_on_the_host(kw, code):
    assert _lin(**kw) == code


def _add(x_dtype=exl3.F16, out_dtype=exl3.F32, meta_ptr=8192):
    g, u, d = _proj(), _proj(), _proj(in_features=512, out_features=256)
    mc = exl3.MetaC(*([ctypes.c_void_p(meta_ptr)] * len(exl3.MetaC._fields_)))
    return exl3.lib().exl3_moe_additive(
        ctypes.c_void_p(16384), x_dtype, 4, 2, ctypes.byref(mc), ctypes.byref(g),
        ctypes.byref(u), ctypes.byref(d), ctypes.c_void_p(32768), out_dtype, 8, -1,
        ctypes.c_void_p(65536), 1 << 40, None, None)


@pytest.mark.parametrize("xdt,odt,code", [
    (exl3.F32, exl3.F32, -2), (0, exl3.F32, -2), (exl3.F16, exl3.I64, -2),
    (exl3.BF16, exl3.F32, -5), (exl3.BF16, exl3.BF16, -5), (exl3.F16, exl3.F16, -5)])
def test_additive_validates_dtypes_on_the_host(xdt, odt, code):
    assert _add(xdt, odt) == code


@pytest.mark.parametrize("rows,cap,passes,group", [
    (3072, 2048, 12, 6), (3072, 10 ** 6, 1, 1), (3072, 12288, 2, 1), (3072, 8192, 3, 2),
    (3072, 6144, 4, 2), (3072, 4916, 5, 3), (3072, 3511, 7, 4), (3072, 3072, 8, 4),
    (3072, 1024, 24, 8)])
def test_pipelined_passes_are_grouped_per_launch_unit(rows, cap, passes, group):
    # 128-row tiles (rows * topk >= 64 * experts), several passes: a launch
    # unit holds half the passes, rounded up, at most 8 (one plan, buffers
    # of group * capacity)
    lay = exl3.moe_layout(rows, 8, 192, 6144, 2048, cap)
    assert (lay.passes, lay.plan_group) == (passes, group)
    one = exl3.moe_layout(rows, 8, 192, 6144, 2048, cap if group == 1 else 10 ** 6)
    assert lay.total > 0 and one.total > 0


def test_small_tiles_never_group_passes():
    lay = exl3.moe_layout(64, 8, 128, 4096, 1536, 16)  # 16-row tiles, 32 passes
    assert lay.passes == 32 and lay.plan_group == 1


def test_profile_record_checks_on_the_host():
    # the timing record is the caller's: the library validates it and, with
    # nothing recorded, touches no device
    L = exl3.lib()
    ms = (ctypes.c_float * 4)()
    ev = (ctypes.c_void_p * 8)()
    ids = (ctypes.c_int32 * 4)()
    assert L.exl3_profile_read(None, ms) == -1
    assert L.exl3_profile_read(ctypes.byref(exl3.ProfileC(ev, ids, 4, 5)), ms) == -7
    assert L.exl3_profile_read(ctypes.byref(exl3.ProfileC(ev, ids, 4, -1)), ms) == -7
    assert L.exl3_profile_read(ctypes.byref(exl3.ProfileC(ev, ids, 4, 0)), ms) == 0
    assert L.exl3_profile_read(ctypes.byref(exl3.ProfileC(None, ids, 4, 2)), ms) == -1
    assert L.exl3_events_create(-1, ev) == -7
    assert L.exl3_events_create(2, None) == -1
    assert L.exl3_events_create(0, None) == 0
    assert L.exl3_events_destroy(-1, ev) == -7
    assert L.exl3_events_destroy(0, None) == 0
