"""The byte model against the closed form printed on the pages."""
from importance_aware_kv_amd import bytes_model as BM


def test_kv_cache_closed_form_70b_128k():
    # "KV Cache Compression and Dynamic Pruning in Production Serving", Sec. 1:
    # a 70B-class GQA model (80 layers, 8 KV heads, D = 128, 2-byte elements)
    # needs about 41.9 GB for one 128,000-token sequence.
    m = BM.kv_cache_bytes(1, 128000, 80, 8, 128, 2)
    assert round(m / 1e9, 1) == 41.9
    # and "over 167 GB" for a batch of 4 of them
    assert BM.kv_cache_bytes(4, 128000, 80, 8, 128, 2) > 167e9


def test_step_bytes_components():
    # one unit, one live token, G = 1, D = 64, fp32: 2*256 + 12 for the token,
    # 256 (q) + 512 (k, v new) + 256 (out); one move adds 2*(512 + 8)
    assert BM.decode_step_bytes(1, 1, 1, 64, 4, [1], 0) == 524 + 256 + 512 + 256
    assert BM.decode_step_bytes(1, 1, 1, 64, 4, [1], 1) == 524 + 256 + 512 + 256 + 1040
