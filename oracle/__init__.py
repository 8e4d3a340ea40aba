"""fp64 CPU oracle for paged split-KV decode attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(the HIP library and its Python binding) never imports, calls or links it, and
it shares no code with that path: it decodes raw bf16 / fp8 bit patterns
itself, gathers pages through the block table itself and computes the plain
softmax-attention definition in float64 with NumPy.

Every function cites the passage of the source pages it follows, by page title
and section.  The pages are:

* "vllm.v1.attention.ops.triton_decode_attention" (API page of the MLA causal
  verify op: ``decode_attention_fwd_verify``, ``verify_num_kv_splits``);
* "vllm.models.flint.ops.decode_attention" (GQA split-KV decode with sinks and
  sliding window: module docstring, ``_FlintDecodeAttention`` methods,
  ``flint_decode_attention``);
* "Atención paginada" (Hugging Face transformers paged-attention docs: the
  decode path and its worked block-table example).

Parity status of each function is listed in ``oracle.attention.__doc__``.
"""

from .attention import (  # noqa: F401
    LN2,
    LOG2E,
    attend,
    bf16_bits_to_f64,
    fp8_e4m3fn_table,
    fp8_bits_to_f64,
    gqa_decode,
    gqa_partials,
    gqa_verify,
    gqa_verify_varlen,
    kv_append,
    merge_partials,
    mla_verify,
    row_key_range,
    varlen_row_requests,
    verify_num_kv_splits,
)
