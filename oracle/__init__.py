"""fp64 CPU oracle for tree verification (greedy and stochastic), SpecPV block
selection and SpecPV's buffer policy -- test infrastructure only.

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
from .block_select import (  # noqa: F401
    REDUCTIONS,
    block_scores,
    block_summaries,
    num_blocks,
    select_blocks,
    specpv_select,
    ub_score,
)
from .stochastic import (  # noqa: F401
    philox4x64_10,
    stochastic_accept,
    target_probs,
)
