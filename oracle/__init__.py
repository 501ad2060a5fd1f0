"""CPU oracle for the GPTQ weight-only quantized linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its
Python binding) imports, links or calls this package.  Only the test-suite, the
package smoke check and the CPU-baseline leg of the benchmark may use it.

It is a plain, slow, obviously-correct definition of what the GPU path computes:
unpack the int32 words, dequantise in float64 with W[n, k] = (code - zero) * scale,
and multiply in float64.  See ``gptq_oracle`` for the per-function citations.
``gptq_quant_oracle`` (``oracle.quant``) is the GPTQ quantizer, the step before the path, in the
page's float32 steps; its pins are in ``tests/test_quant_oracle_pins.py``.

Parity status: every function in ``gptq_oracle`` is pinned by the not-gpu tests in
``tests/test_oracle_pins.py``.  One reading is pinned only against itself and the
pages' prose, not against upstream bytes: the continuous 3-bit "10 / split / 10"
word layout (no 3-bit bytes are printed on the pages) -- its *upstream byte parity
is unpinned*.
"""
from .gptq_oracle import *  # noqa: F401,F403
from . import gptq_quant_oracle as quant  # noqa: E402,F401  (the GPTQ quantizer: oracle.quant)
