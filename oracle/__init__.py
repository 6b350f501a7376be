"""fp64 CPU oracle for tree verification -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this package.  The product path (the HIP library and its Python binding)
never imports it.
"""

from .tree_verify import (  # noqa: F401
    OracleInputError,
    ancestors,
    argmax_lowest,
    bf16_to_f64,
    build_mask,
    commit_kv,
    greedy_accept,
    pack_accepted_tokens,
    tree_attention,
)
