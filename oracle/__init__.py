"""CPU oracle for the dual-mode shared-weight INT4 linear layer and the
draft/verify acceptance step of quantization-based self-speculative decoding.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
numpy implementation (fp64 where the method leaves the precision free) that
the GPU path is checked against.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  The product path
(``quantization_self_speculation_amd``) never imports, calls or links it, and
this package never imports the product path: they share no code.

Pages cited (titles as printed; section names in brackets):

* [QSpec]  "QSpec: Speculative Decoding with Complementary Quantization
  Schemes" (arXiv 2410.11305 index page) -- [Abstract (arXiv)].
* [QSpec-blog]  "QSpec の論文要点整理" (tech-dashboard summary of QSpec),
  cited by paragraph number (1 = the opening paragraph).
* [SpecMQuant]  "Speculative Decoding Meets Quantization: Compatibility
  Evaluation and Hierarchical Framework Design" -- [Abstract (arXiv)].
* [SpecQuant]  "SpecQuant: Speculative Decoding with Multi-Parent Quantization
  for Adaptive LLM Inference" -- [Abstract (arXiv)].
* [SpecQuant-review]  the agihunt.info review of SpecQuant, cited by its
  method paragraph ("Verification ...") and its results table.

Where the pages are silent (they print no formula, layout or precision for
any step) the module docstrings state the reading taken.

Parity status per function is listed in each module's header.

``oracle.model`` (imported on demand: ``import oracle.model``) holds the
decoder used by the end-to-end self-speculative loop.
"""

from .quant import (  # noqa: F401
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    pack_nibbles,
    unpack_nibbles,
    pack_w4,
    tile_w4,
    untile_w4,
    tile_scales,
    untile_scales,
    dequant_w4,
    quant_act,
    quant_act_values,
    w4a4_partials,
    gemm_w4a4,
    gemm_w4a16,
)
from .w4a8 import gemm_w4a8, quant_act8, w4a8_partials  # noqa: F401
from .rotate import (  # noqa: F401
    fwht128_f32,
    rotate_x,
    rotate_x_bf16,
    rotate_w,
    quant_act_rot,
)
from .verify import (  # noqa: F401
    softmax64,
    verify_greedy,
    verify_sample,
)
