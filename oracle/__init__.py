"""fp64 CPU oracle for quantized-KV decode attention.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check of the package
entry module and the CPU-baseline leg of the benchmark may import, call or
run anything in this package.  The product (the HIP library and its Python
binding) never does: it shares no code, header, table or constant with this
package and fails loudly when its native library is missing.

What it is: a plain, slow, obviously correct restatement of what the two
pages define, written with numpy in float64 (the KIVI quantiser follows the
pages' fp16 storage and takes its code decisions with IEEE binary32 steps,
see `kivi.py`).  Each function cites the passage it follows.  Pages:

* "LoopVQ: Sub 1-bit KV Cache Quantization for Looped Transformers"
  (Cheong & Yoo), called the LoopVQ page below.
* "KIVI 完全拆解：非对称 2-bit KV Cache 量化", called the KIVI page below.

Every function here is pinned by tests in `tests/test_oracle_*.py` against
closed forms, invariants, brute force on tiny inputs, or figures the pages
print; none is marked "parity unpinned".
"""

from . import loopvq, kivi  # noqa: F401
