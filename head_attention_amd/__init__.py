"""MI355X-native scaled dot-product attention (gfx950 HIP kernels behind a C ABI).

    from head_attention_amd import forward, decode, cache_append
    O = forward(Q, K, V, mask_kind=ATTN_MASK_CAUSAL, scale=0.125)
    cache_append(k_new, v_new, Kcache, Vcache, kv_lens)   # then decode(...)

The C ABI is include/headattn.h; libheadattn.so is built in-tree with
`python -m head_attention_amd.build`.
"""
from ._binding import (  # noqa: F401
    ATTN_BF16,
    ATTN_F32,
    ATTN_MASK_CAUSAL,
    ATTN_MASK_KEY_PADDING,
    ATTN_MASK_NONE,
    ATTN_MASK_RESTRICTED,
    DECODE_NOALLOC_MAX_BYTES,
    LIB_PATH,
    AttnError,
    attn_layout,
    backward,
    backward_workspace_bytes,
    cache_append,
    decode,
    decode_noalloc,
    decode_workspace_bytes,
    forward,
    forward_restricted,
    head_projection,
    lib,
    output_projection,
    status_string,
)
