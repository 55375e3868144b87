"""Float64 CPU oracle for the fused EXL3 routed-experts layer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
library (``trellis_quantized_moe_amd``) and imports nothing from it.

Sources. The method is described by four pull-request pages:
  * exllamav3 PR #284 "MoE: Add fused additive EXL3 kernels" (Summary,
    API contract, Validation);
  * TensorFold PR #837 "cuda: EXL3 linear and grouped routed experts, every
    codebook and width, a width per expert" (What this changes, Receipt);
  * sparkinfer PR #99 "moe: add isolated mixed K3/K4 Trellis comparison path"
    (closing review);
  * exllamav3 PR #246 "Persistent route-packed (route_block x n_tile) schedule
    for exl3 fused MoE (sm120)" (Motivation, The change).
The pages name the trellis codebooks but define none of them, nor the tile
bit layout or the rotation size. Those are fixed by this library's own format
definition (MCG16 codebook, 16x16 tail-biting tiles, 128-point Sylvester
Hadamard), restated in each module's docstring.

Modules:
  trellis   codebook + two independent tile decoders + tensor dequantisation
  hadamard  orthonormal 128-point Sylvester Hadamard on contiguous blocks
  linear    one EXL3 projection with additive stages (pure / R modes)
  route     route histogram, exclusive scan, stable pack
  moe       routed-experts layer (gate/up, SwiGLU, down, top-k combine)
  brute     dense dequantise-then-matmul brute force for tiny shapes

Every function here is pinned by ``tests/test_oracle_*.py`` (``-m "not gpu"``)
against closed forms, library routines, brute force or the format's printed
test vectors; none is "parity unpinned".
"""

from . import trellis, hadamard, linear, route, moe, brute  # noqa: F401
