"""Page-printed roofline figures reproduced by the byte-count arithmetic bench.py uses."""
import json
import os

from stream_decode_attention_amd import roofline

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "llm_decode_cuda_roofline.json")


def test_kv_bytes_per_token_is_40_kb():
    g = json.load(open(GOLDEN))
    per_tok = roofline.kv_bytes_per_token(g["layers"], g["kv_heads"], g["head_dim"], g["bytes_per_element"])
    assert per_tok == g["kv_bytes_per_token_printed_KB"] * 1024


def test_roofline_rates_match_the_page():
    g = json.load(open(GOLDEN))
    bw = g["measured_stream_read_GBps"] * 1e9
    w = g["weight_bytes_MB"] * 1e6
    per_tok = roofline.kv_bytes_per_token(g["layers"], g["kv_heads"], g["head_dim"], g["bytes_per_element"])
    assert round(roofline.roofline_tokens_per_s(bw, w, 0, per_tok)) == g["roofline_tok_s_short_context_printed"]
    assert round(roofline.roofline_tokens_per_s(bw, w, g["context_tokens"], per_tok)) == \
        g["roofline_tok_s_at_context_printed"]


def test_decode_and_chunk_byte_counts():
    # one 4k-context SmolLM2 layer call reads 1280 bytes per key
    assert roofline.kv_bytes_decode([4096], 5, 64, 4096) == 4096 * 1280
    # lengths clamp to [0, S_max]
    assert roofline.kv_bytes_decode([-3, 10**6], 8, 128, 32768) == 32768 * 4096
    # verify chunk: ctx + T keys read once
    assert roofline.kv_bytes_chunk([8192], 6, 8, 128, 16384) == 33579008
