"""CPU oracle for batched paged MLA decode in absorbed form (float64, NumPy).

TEST INFRASTRUCTURE ONLY.  This package is the slow, obviously-correct
definition the GPU path is checked against.  Only the test suite, the
package's smoke check and the CPU-baseline leg of the benchmark may import it;
the library and its Python binding never do, and the oracle imports nothing
from them.  Its inputs are raw storage bits (bf16 / fp8 e4m3fn codes as
integers) plus int32 metadata, exactly as the generator hands them out.

Sources (web pages on the method; cited by title and section):
  * FlashInfer docs, "flashinfer.attention.prims_ts.prims_ts_batch_decode_with_kv_cache_mla"
    -- signature, layout/mask paragraph, contract paragraph.
  * FlashInfer issue #3131, "Support cum_seq_lens_q in
    trtllm_batch_decode_with_kv_cache_mla trtllm-gen backend" -- the launcher
    excerpt passes one cache tensor as both K and V; cum_seq_lens_q is the
    ragged query-offset array.
  * FlashInfer PR #1248, "update cubins for dynamic scale factor interface and
    one-copy kvcache on trtllm-gen mla" -- bmm1/bmm2 scale derivation.
  * FlashInfer issue #3131 -- the trtllm_batch_decode_with_kv_cache_mla and
    trtllm_paged_attention_decode signatures carry sparse_mla_top_k (the
    sparse top-k reading is in oracle/sparse.py).
  * vLLM docs, "FlashInferMLAImpl" -- forward_mqa (scale folding for
    quantized KV, natural-log LSE, ragged/uniform query branches) and
    _flattened_decode_metadata.

Every function here is pinned by tests that do not re-type its formula:
closed forms, invariants, brute force and a library attention routine (see
tests/test_oracle_pins.py, tests/test_oracle_sparse.py).  No function is parity-unpinned.
"""

from .formats import bf16_bits_to_f64, e4m3fn_bits_to_f64, e4m3fn_table
from .mla import (
    MlaProblem,
    visible_count,
    gather_request_rows,
    reference_decode,
    reference_partial,
    reference_dcp_partial,
    merge_partials,
)
from .sparse import reference_sparse_decode

__all__ = [
    "bf16_bits_to_f64",
    "e4m3fn_bits_to_f64",
    "e4m3fn_table",
    "MlaProblem",
    "visible_count",
    "gather_request_rows",
    "reference_decode",
    "reference_partial",
    "reference_dcp_partial",
    "merge_partials",
    "reference_sparse_decode",
]
