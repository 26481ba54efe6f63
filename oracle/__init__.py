"""CPU oracle for NVFP4-compressed sparse-MLA decode.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or link anything in this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
use it. It shares no code, table or constant generator with the HIP library.

Sources followed (cited by page title and section, as printed on the page):

* [PI] "Prime Inference: Fast, Reliable Serving for Frontier Open Models" (Prime Intellect blog,
  read through its traeai.com Chinese translation).
  - section "Making room for low-latency decode": the 512-value MLA latent is stored as 4-bit
    values with one FP8 scale per 16 values, the 64-value rope part stays FP8, and a row shrinks
    from 576 to 352 bytes.
  - section "Native NVFP4 sparse MLA decode kernel": attention reads the rows chosen by the sparse
    indexer, NVFP4 is only the storage format, the arithmetic uses FP16 operands with FP32
    accumulation; rows of one query token are split across cooperating blocks whose partial
    results are merged; empty (-1) slots of the 2048-entry list are not loaded.
* OCP 8-bit Floating Point Specification (OFP8), E4M3 encoding (bias 7, no infinities, the all-ones
  code is NaN, max 448).
* OCP Microscaling Formats (MX) v1.0, FP4 E2M1 element encoding (bias 1, values 0, 0.5, 1, 1.5,
  2, 3, 4, 6).

Modules: ``nvfp4`` (element and row codec), ``fp8`` (the 576-byte FP8 baseline row and the staged
NVFP4 -> FP8 conversion), ``cache`` (paged row addressing), ``attention`` (fp64 sparse / dense
absorbed-MLA decode and the split log-sum-exp merge), ``layout`` (block-major and layer-major
multi-layer page layouts, transfer regions, block copy), ``topk`` (top-k selection of positions
from per-position scores), ``indexer`` (the FP8 indexer scores top-k selects from).

Parity pins live in ``tests/test_oracle_*.py`` (run with ``-m "not gpu"``).
"""

from . import nvfp4, fp8, cache, attention, layout, topk, indexer  # noqa: F401
