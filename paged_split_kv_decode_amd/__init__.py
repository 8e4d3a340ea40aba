"""Paged split-KV decode attention for AMD MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of
``include/paged_decode.h`` (``libpaged_decode.so`` in this directory); this
package is the thin torch binding of that ABI.  Importing it fails loudly if
the library has not been built: there is no CPU fallback.
"""

from .api import (  # noqa: F401
    PD_KV_BF16,
    PD_KV_FP8_E4M3FN,
    alloc_workspace,
    gqa_split_cap,
    merge_splits,
    mla_split_cap,
    num_kv_splits_cap,
    paged_decode_gqa,
    paged_decode_gqa_partials,
    paged_kv_append,
    paged_verify_gqa,
    paged_verify_gqa_append,
    paged_verify_gqa_partials,
    paged_verify_gqa_varlen,
    paged_verify_mla,
    paged_verify_mla_partials,
    split_rule,
    stream_read_probe,
    workspace_bytes,
)
from ._native import LIB_PATH, PagedDecodeError  # noqa: F401
