"""CPU oracle for varlen attention over a paged KV cache (test infrastructure).

This package is the checker, not the product. Only the tests, the smoke check
and the bench's CPU-baseline leg may import it; the library's own path never
does, and it never imports anything from the library.

It computes, plainly and slowly, in float64 (numpy):
  * the in-place append of new K/V into the paged cache, bit-exact on the
    stored bytes (bf16 copy, or OCP e4m3fn quantisation with a per-tensor
    scale) -- ``append``;
  * de-paging of a sequence's keys/values through its block-table row --
    ``depage``;
  * softmax(scale * Q K^T + mask) V and the natural-log LSE per sequence and
    query head, with grouped-query heads and bottom-right causal masking --
    ``attend`` / ``attend_rows``;
  * the associative LSE merge of partial results over a split of the key
    range -- ``merge_partials``;
  * rotary position embedding of the query rows and the new key rows before
    the append (optional) -- ``rope.positions`` / ``rope.rotate_bf16`` and
    ``run_call(rope=...)``;
  * fp8 "QKV-Prob" attention: fp8 query codes, and the softmax quantised to
    fp8 before the second product -- ``prob8.attend`` and
    ``run_call(prob8=...)``.

Pages this follows (cited by title and section):
  * "Add flash_attn_varlen_func_with_kvcache" (flash-attention PR), sections
    Usage and Minor Changes: packed varlen q with cumulative offsets, optional
    new k/v with their own cumulative offsets, an in-place cache update, and a
    per-sequence cache length attribute.
  * "Add KV cache for paged/non-paged attention" (TransformerEngine PR),
    Description: the unfused backend converts the paged cache to a contiguous
    one through the page table and then runs matmul -> softmax -> matmul; K and
    V share one page table; batches may mix context and generation phases.
  * "[Kernel][Triton][FP8] Adding fp8 and variable length sequence support to
    Triton FAv2 kernel" (vLLM PR), feature list: 8-bit KV cache, causal
    masking, grouped-query attention, variable sequence lengths.
  * "Extend FlashAttention Prefill with KV cache" (cutlass-sycl PR),
    description: prefill over cached KV plus the current KV, causal or not.

Every function is pinned in tests/test_oracle_*.py against facts fixed by the
mathematics or by library routines (see each function's docstring).
"""
from .formats import (  # noqa: F401
    bf16_bits_to_f64, e4m3fn_decode, e4m3fn_encode, e4m3fn_encode_f64, e4m3fn_value_table,
)
from . import prob8, rope  # noqa: F401
from .attention import (  # noqa: F401
    append, attend, attend_rows, depage, merge_partials, run_call, run_workload, sequence_kv,
)
