"""RadixAttention's hot path on MI355X (gfx950): host radix tree + HIP kernels behind
the C ABI of librax (include/rax.h), with a thin ctypes binding (_lib) and the
request-lifecycle driver that calls it (runtime)."""
from ._lib import (  # noqa: F401
    Tree, RaxError, kv_scatter, req_to_token_write, extend_attention, decode_attention,
    attention_workspace_bytes, device_errors, lib, EXPORTS,
)
