"""Plain float64 CPU oracle of the GPTQ layer-wise solver.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package.  The HIP library never calls it and shares no code with it; the only
module both sides use is ``synth`` (seeded inputs, no method arithmetic).

Sources (web pages about GPTQ, cited by title and section):
  [skillmd]   skillmd.com "Gptq" skill page
  [polydesk]  polydesk.ai glossary "GPTQ (Generative Pre-trained Transformer Quantization)"
  [wikiprompt] wikiprompt.org "GPTQ"
  [ayinedjimi] ayinedjimi-consultants "Quantization : GPTQ, GGUF, AWQ - Quel Format Choisir"

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
something other than itself (closed forms, textbook special cases, brute force,
values the pages print).  Nothing is "parity unpinned" except the absolute
loss/code statistics of the synthetic workloads, which the pages do not print.
"""
from .gptq import (  # noqa: F401
    QuantConfig, NotPositiveDefinite,
    hessian, hessian_entries, prepare, grid_params, quantize_column, sweep,
    quantize_layer, gptq_layer, rtn, obs_bruteforce, pack, unpack,
    dequantize, dequant_matmul, grouped_order, rel_loss, to_fp16,
)
from . import block  # noqa: F401  (block-sequential calibration: forward of one decoder block)
