"""CPU oracle for ROCmFPX block-quantized MoE layers — TEST INFRASTRUCTURE.

This package is the slow, plain, obviously-correct reference that the HIP
library is checked against. It is not part of the product: only the tests,
the smoke check and the CPU-baseline leg of the benchmark may import it. It
shares no code with the HIP library (``bit_block_quantized_rocmfp2_amd``), and
neither imports the other; the seeded input generators live in ``synth``.

Page citations used in this package:

* [Strix-284B] lucebox.com, "DeepSeek V4 Flash: 284B model, up to 32 tok/s on
  AMD Ryzen AI MAX+ 395" — section "ROCmFPX: fitting 284B weights into 128 GB"
  (32-weight blocks of low-bit codes plus a small scale; FP2 = 10 bytes =
  2.50 bpw, FP3 3.50 bpw, FP4 4.25 bpw; codebooks expanded in registers and fed
  to integer dot products), section "Decode: up to 32 tok/s" (q = 4 columns).
* [0731-Strix] lucebox.com, "Lucebox × Geometric: DeepSeek V4 Flash 0731
  reaches 32.7 tok/s on AMD Strix Halo" — section "How the model fits on AMD
  Strix Halo" (per-expert codebooks; gate/up 2.5 bpw, down 3.5 bpw) and
  "Run with Lucebox Engine" (256 experts, 6 routed).
* [evox3] soothill.io, "DeepSeek V4 Flash 0731 on evox3" — introduction and
  table "The optimization ladder" (H32 rotations on the 3.5-bit experts;
  shared / fused H32 input; layer-major prefill).

Everything the pages leave open (bit positions, scale encodings, activation
quantization, the H32 convention, router precision and order, SwiGLU) follows
the readings written down with the format specification of this repository;
each function's docstring restates the reading it implements.

Parity pins: every function here is checked by ``tests/test_oracle_*.py``
against hand-worked values, closed forms, exact rational arithmetic, brute
force on tiny inputs or a public specification (OCP MX FP4). No function is
"parity unpinned".
"""
from . import formats, quant, hadamard, dots, router, moe, quantize  # noqa: F401
