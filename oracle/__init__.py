"""CPU oracle for one transformer layer of RAG KV-cache fusion.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, float64 numpy
statement of what the fused-layer path computes, written from the pages'
equations.  Only the test suite, the smoke check of the package entry point
and the CPU-baseline leg of the benchmark may import it.  It shares no code
with the HIP library (`rag_kv_cache_kvf_amd`) and imports nothing from it;
inputs reach it as plain numpy arrays.

Sources (cited by page title and section / equation):
  [QCF] "QCFuse: Query-Aware Cache Fusion via Compressed View for Efficient
        RAG Serving" - sections 2.1.1-2.1.3 (Eq. 1-7), 2.2 (2.2.1), 3.2.1
        (Eq. 9-11), 3.3.1 (Eq. 14), 3.4.2 (Eq. 20).
  [KVB] "KVBoost: Chunk-Level Key-Value Cache Reuse with Deviation-Guided
        Recomputation for Efficient Large Language Model Inference" -
        section 3.1 (Eq. 1-2), 3.2 (Eq. 3), 4.1, 4.5 (Eq. 7), 4.6.1
        (Algorithm 1), 4.6.2 (Algorithm 2), 7.3 (memory budget).

Pins: every function here is checked by `tests/test_oracle_*.py` against
closed forms, invariants, brute force on tiny inputs or special cases
(see the docstring of each function for its pin).  No function in this
package is "parity unpinned"; the quality of the selected set on real text
(which needs trained weights and datasets) is not claimed anywhere.
"""
from . import storage, rope, kivi, fusion, selectors, multilayer, q8cache  # noqa: F401
