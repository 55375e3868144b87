"""GPU: exl3_moe_forward_static, the allocation-free variant of
exl3_moe_forward (its workspace is the library's static device array),
against exl3_moe_forward with a caller workspace."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import moe as omoe  # noqa: E402
from trellis_quantized_moe_amd import exl3, synth  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_static_scratch_forward_equals_forward():
    """The decode layer (128 experts, top-8, 4096/1536, K=4): two calls in a
    row through the static entry point, 16 rows and then 3 rows (the second
    call finds the first call's contents in the scratch), each equal bit for
    bit to exl3_moe_forward with its own workspace; the 3-row output also
    meets the oracle bar on its first row. A call that needs more than the
    32 MiB scratch is refused on the host with EXL3_E_SCRATCH."""
    wl = synth.moe_workload("decode", rows=16)
    gate, up, down = (exl3.DeviceProj(p, DEV) for p in (wl.gate, wl.up, wl.down))
    x, ids, w = exl3.device_inputs(wl, DEV)
    for M in (16, 3):
        print("static scratch forward, %d rows" % M, flush=True)
        cap = M * wl.topk
        need = exl3.moe_workspace_size(M, wl.topk, wl.num_experts, wl.hidden,
                                       wl.intermediate, cap)
        assert need <= exl3.STATIC_SCRATCH_BYTES
        ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        ref = exl3.exl3_moe_forward(x[:M], ids[:M], w[:M], gate, up, down, cap,
                                    torch.float32, ws=ws)
        got = exl3.exl3_moe_forward_static(x[:M], ids[:M], w[:M], gate, up, down, cap,
                                           torch.float32)
        got16 = exl3.exl3_moe_forward_static(x[:M], ids[:M], w[:M], gate, up, down, cap,
                                             torch.float16)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), M
        assert torch.equal(got16.view(torch.int16), ref.to(torch.float16).view(torch.int16)), M
    orc = omoe.moe_forward(wl.x, wl.ids, wl.weights_f64, wl.gate, wl.up, wl.down, "R", rows=[0])
    err = float(np.max(np.abs(got.cpu().double().numpy()[0] - orc[0]))) / float(
        np.sqrt(np.mean(orc[0] ** 2)))
    print("  row 0 against the oracle: %.3e" % err, flush=True)
    assert err <= 2e-3
    big = 4096
    assert exl3.moe_workspace_size(big, 8, 128, 4096, 1536, big * 8) > exl3.STATIC_SCRATCH_BYTES
    xb = torch.zeros(big, 4096, dtype=torch.float16, device=DEV)
    ib = torch.zeros(big, 8, dtype=torch.int64, device=DEV)
    wb = torch.zeros(big, 8, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(exl3.Exl3Error, match="status -9"):
        exl3.exl3_moe_forward_static(xb, ib, wb, gate, up, down, big * 8)
