"""fp64 CPU oracle for drafter block attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import, call or run anything in this package.  The product path (the
HIP library and its Python binding) never does; it shares no code, header,
table or constant with this package.
"""
from .drafter_attn_oracle import (  # noqa: F401
    rms_norm,
    rope_neox,
    rope_inv_freq,
    yarn_inv_freq,
    yarn_mscale,
    yarn_pair_at_turns,
    YARN_RAMPS,
    gather_context,
    drafter_attn,
    drafter_attn_qknorm,
    drafter_attn_split_merge,
    qk_norm_rope,
    kv_append,
    paged_attn,
    OracleContractError,
)
