"""The byte/flop accounting the roofline is priced on, pinned to the pages' figures."""

import json
import os

from decode_attention_kv_amd import accounting as acc


def test_llama7b_decode_read_per_layer_and_token(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "kv_bytes.json")))["decode_read"]
    per_layer = acc.kv_layer_bytes(g["heads"], g["head_dim"], g["context"], g["elem_bytes"])
    assert per_layer == g["bytes_per_layer"] == 64 * 2 ** 20
    assert g["layers"] * per_layer == g["bytes_per_token"]
    # one decode call over the full 4096 rows reads exactly that many K/V bytes
    total = acc.decode_static_bytes(1, 32, 128, [4096], with_mask=False)
    assert total - per_layer == 32 * 128 * 4 * 2 + 4


def test_copy_kvcache_volume(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "kv_bytes.json")))["copy_kvcache"]
    assert acc.copy_kvcache_bytes(g["layers"], g["heads"], g["seq_len"], g["head_dim"],
                                  g["elem_bytes"]) == g["bytes"] == 512 * 2 ** 20


def test_hbm_time_estimate_is_bytes_over_bandwidth(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "kv_bytes.json")))["hbm_read_time_estimate"]
    assert round(g["bytes_decimal_mb"] / g["bandwidth_bytes_per_s"] * 1e6) == g["microseconds"]


def test_sparse_mac_count_matches_the_cube_cycle_table(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "mla_cycle_table.json")))
    d = g["d"]
    l2_bw = g["l2_total_bw"] / g["num_cores"] / g["freq_hz"]
    for row in g["rows"]:
        macs = acc.sparse_macs(1, row["h_q"], d, d, row["topk"])
        assert macs // g["macs_per_clock"] == row["cube_cycles"]
        assert acc.sparse_flops(1, row["h_q"], d, d, row["topk"]) == 2 * macs
        # Q + O at 2 bytes each plus the gathered KV rows, as the table prices memory
        mem = row["h_q"] * d * 2 * 2 + row["topk"] * d * 2
        assert round(mem / l2_bw) == row["mem_cycles"]


def test_sparse_config_bytes_and_flops():
    # batch 16, 128 heads, d_qk 576, d_v 512, top-2048: 9.13 GFLOP, 44.4 MB
    assert acc.sparse_flops(16, 128, 576, 512, 2048) == 9_126_805_504
    b = acc.sparse_bytes(16, 128, 576, 512, 2048)
    assert b == 16 * 2048 * 576 * 2 + 16 * 128 * 576 * 2 + 16 * 128 * 512 * 4 + 16 * 2048 * 4
    assert 44.0e6 < b < 44.5e6


def test_gather_bytes_count_read_and_write_of_valid_rows():
    b = acc.gather_bytes([3, 0, 130], 8, 128, 8, 128, 128, with_offset=True)
    rows = 133 * 2 * 8 * 128 * 2
    assert b == 2 * rows + (1 + 0 + 2) * 4 + 4 * 4 + 3 * 4


def test_sparse_fp8_bytes_halve_the_gathered_rows():
    # one byte per latent value plus a 4-byte scale per gathered row
    b = acc.sparse_fp8_bytes(16, 128, 576, 512, 2048)
    assert b == 16 * 2048 * (576 + 4) + 16 * 128 * 576 * 2 + 16 * 128 * 512 * 4 + 16 * 2048 * 4
    full = acc.sparse_bytes(16, 128, 576, 512, 2048)
    assert full - b == 16 * 2048 * (576 * 2 - 576 - 4)


def test_sparse_fp4_bytes_are_half_a_byte_per_value():
    b4 = acc.sparse_fp4_bytes(16, 128, 576, 512, 2048)
    b8 = acc.sparse_fp8_bytes(16, 128, 576, 512, 2048)
    assert b8 - b4 == 16 * 2048 * 576 // 2
    assert b4 == 16 * 2048 * (288 + 4) + 16 * 128 * 576 * 2 + 16 * 128 * 512 * 4 + 16 * 2048 * 4


def test_paged_fp4_bytes_are_half_a_byte_per_value():
    lengths = [5, 300, 17]
    b4 = acc.decode_paged_fp4_bytes(lengths, 32, 8, 128, 16)
    b8 = acc.decode_paged_fp8_bytes(lengths, 32, 8, 128, 16)
    assert b8 - b4 == sum(lengths) * 8 * 64 * 2
