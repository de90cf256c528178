"""Oracle: a plain, slow CPU statement of what the persistent GEMM and the
persistent add compute, plus a model of each tile scheduler.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke entry point and the
CPU-baseline leg of the benchmark may import anything from this package.  It
shares no code, header, table or helper with the HIP library: it decodes the
stored bits itself, accumulates in fp64 itself and derives every schedule
from the formulas on the pages itself.

Sources (cited by page title and section):
* "Implement persistent kernels" (Helion PR #238), example output: the
  PERSISTENT BLOCKED / PERSISTENT INTERLEAVED / PERSISTENT BLOCKED WITH L2
  GROUPING listings give the blocked ranges, the stride-by-grid loop, the
  plain tile decode, the grouped decode and the masked element-wise add.
* "Work Stealing Scheduler Kernel" (tritonBLAS PR #65), Copilot overview and
  the review comments on the matmul wrapper and the work-stealing kernel:
  per-XCD atomic tile counters keyed by program id modulo the XCD count,
  counters reset before every launch, masked (never wrapped) edge tiles.
* "[Feature] Introduce tile scheduler" (TileLang PR #2441), the MXFP8
  block-scaled example header and producer loop: block-scale shape
  (1, 1, 128) with scale arrays laid out K-group-major.

Every function here is pinned by tests that do not re-derive it (closed forms,
format-definition tables checked against library casts, brute force, hand
derived schedule fixtures); none is marked "parity unpinned".
"""
