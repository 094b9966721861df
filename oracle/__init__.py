"""CPU oracle for weight-only group-quantized matrix multiplication.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, obviously correct
statement of what the GPU library computes. Only the test-suite, the smoke
check and the CPU-baseline leg of the benchmark may import it; the product
path (the HIP library and its Python binding) never does, and the two share
no code.

Contents
  numerics  bit-level bf16 / fp16 encode and decode (round-to-nearest-even)
  quant     RTN scale choice and the fixed-grid quantizer Q_s
  layout    the packed-weight tile layout, written out index by index
  gemm      exact dequantization and the reference product, plus the
            acceptance test used for floating-point parity
  attention the drafter's symmetric sliding-window attention over a full
            KV cache (window rule, grouped-query heads, softmax)

Sources: "Quantize the Target, Quantize the Drafter" (arXiv 2607.04244, HTML
text: the QAD method paragraph, the drafter-PTQ calibration paragraph and
the Drafter SWA paragraph) and
the Qwen3.5-4B-DFlash-W8A16 model card ("What changed vs upstream" table).

Every function here is pinned by a CPU test against something other than
itself (closed forms, brute force, library routines, values printed on the
pages). None is "parity unpinned".
"""

from . import numerics, quant, layout, gemm, attention  # noqa: F401
