"""Closed-form pins of the cache layout against the figures the pages print
(tests/golden/pages_numbers.json, each value with its page and section)."""
import json
import os

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))
GIB = float(1 << 30)


def g(k):
    return GOLD[k]["value"]


def test_entries_per_block(orc):
    blk = g("block_native_positions")
    assert orc.HostPool(4, 2, 64, 0, 1e4, orc.BF16, 1).rows_per_page == g("c4a_entries_per_block")
    assert orc.HostPool(128, 1, 64, 0, 1e4, orc.BF16, 1).rows_per_page == g("c128a_entries_per_block")
    assert blk == orc.BLOCK


def test_entries_at_1m():
    n = 1 << 20
    assert abs(n // 4 - g("c4a_entries_at_1m_approx")) / g("c4a_entries_at_1m_approx") < 0.05
    assert abs(n // 128 - g("c128a_entries_at_1m_approx")) / g("c128a_entries_at_1m_approx") < 0.05


def test_kv_bytes_per_1m_sequence(orc):
    """bf16 rows: shared K=V latent of 512, indexer key of 128 (c4a layers only).
    The V3.2-style stack stores per token a 576-wide MLA latent and a 128-wide
    indexer key in every one of 61 layers."""
    n = 1 << 20
    main = orc.row_bytes(512, orc.BF16)
    idx = orc.row_bytes(128, orc.BF16)
    v4 = g("c4a_layers") * (n // 4) * (main + idx) + g("c128a_layers") * (n // 128) * main
    v32 = g("v32_layers") * n * (orc.row_bytes(576, orc.BF16) + idx)
    assert round(v4 / GIB, 2) == g("v4_kv_gib_per_1m_seq_bf16")
    assert round(v32 / GIB, 1) == g("v32_kv_gib_per_1m_seq_bf16")
    assert round(v32 / v4, 1) == g("ratio_v32_over_v4")


def test_fp8_row_is_about_half(orc):
    # fp8 rows with one fp32 scale per 64 elements: 544 B vs 1024 B
    assert orc.row_bytes(512, orc.FP8) == 544
