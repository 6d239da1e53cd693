"""fp64 CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library, its
Python binding, the timed part of the benchmark) may import, call or link
anything in this package; only the tests, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code with the GPU path.

Modules
-------
exact       the definition written out: materialised score matrix, softmax,
            weighted sum of values (prefill, packed variable-length prefill
            with bottom-right causal alignment and a left window, KV-cache
            decode contiguous or paged) and its gradients, plus the
            tile-by-tile running-softmax form and the log-sum-exp merge of
            partial results that the exactness claim rests on.
traffic     the page-1 tiled-GEMM load-count model.

Every function is pinned by tests/test_oracle.py against closed forms,
invariants, brute force in 50-digit arithmetic and PyTorch's CPU float64
scaled_dot_product_attention.
"""

from .exact import (  # noqa: F401
    attention,
    attention_backward,
    attention_rows,
    attention_varlen,
    varlen_visible,
    decode,
    decode_paged,
    score_matrix,
    tiled_attention,
    merge_partials,
)
from .traffic import tiled_gemm_reads  # noqa: F401
