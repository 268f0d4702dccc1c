"""fp64 CPU oracle for split-KV single-query decode attention, for the step
before it (rotary embedding of the new tokens and their K/V-cache write), for
the weight products of a decode step (bf16 and INT8 weight-only GEMV), and for
the accept/reject step of speculative decoding with its rollback of the cache
lengths.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or link
this package: only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` use it. It shares no code with the HIP library; both sides
consume the same seeded bf16 bytes from ``workloads``.

Every function is plain NumPy in float64, written from the definition the pages
give (tinydecode README, "how the decode step is put together" and
"speculative decoding"; llm-decode-cuda, attention section and design notes;
the FlashSpec page's correctness paragraph). Where the pages leave a step open the
reading taken is stated in the function's docstring.
"""
from .attention import (  # noqa: F401
    bf16_bits_to_f64,
    decode_attention,
    decode_attention_f64,
    chunk_attention,
    chunk_attention_f64,
    split_kv_attention_f64,
    kv_head_of,
)
from .bf16 import bf16_bracket, f64_to_bf16_bits_rne  # noqa: F401
from .rope import (  # noqa: F401
    llama3_scale_frequencies,
    model_frequencies,
    rope_frequencies,
    rope_kv_write,
    rope_kv_write_f64,
    rotate_f64,
    token_positions,
)
from .gemv import (  # noqa: F401
    gemv,
    gemv_f64,
    gemv_int8,
    gemv_int8_f64,
    quantize_rows_int8,
)
from .speculative import (  # noqa: F401
    accept_reject,
    accept_reject_row,
    argmax_first,
    log_target_probs,
    new_length,
    sample_index,
    target_probs,
)
