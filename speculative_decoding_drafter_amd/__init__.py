"""MI355X-native (gfx950) DFlash drafter block attention.

The compute path is the HIP library ``libdrafter_attn.so`` (C ABI in
``include/drafter_attn.h``); this package is a thin torch binding over it.
Importing the package does not load the library; the first call does, and
fails loudly if it has not been built.
"""
from .ops import (  # noqa: F401
    DrafterAttnError,
    drafter_attn,
    drafter_attn_qknorm,
    drafter_attn_qknorm_noalloc,
    kv_append,
    make_workspace,
    paged_attn,
    plan,
    qk_norm_rope,
    workspace_bytes,
)
