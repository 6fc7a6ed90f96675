"""The oracle's formats against figures printed on the pages (tests/golden/page_facts.json)."""
import json
import os

import numpy as np

import oracle

FACTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))


def test_q4_row_and_position_sizes():
    assert oracle.q4_row_bytes(256) == FACTS["q4_row_bytes_head_dim_256"]["value"]
    # 16 layers x 4 KV heads x (K, V) rows per position
    per_pos = 16 * 4 * 2 * oracle.q4_row_bytes(256)
    assert per_pos == FACTS["q4_kib_per_position_16_layers"]["value"] * 1024
    assert 16 * 4 * 2 * 256 * 2 == FACTS["q4_kib_per_position_16_layers"]["bf16_value"] * 1024
    assert oracle.q4_row_bytes(256) / 256 == FACTS["bytes_per_element"]["q4"]


def test_q4_exact_scale_example():
    f = FACTS["q4_exact_scale_example"]
    # a group whose rotated values are integers with amax 8 (present as -8)
    import scipy.linalg
    H = scipy.linalg.hadamard(32) / np.sqrt(32.0)
    c = np.arange(32) % 16 - 8.0
    x = (c @ H.T).astype(np.float32)
    rows = oracle.q4_encode_rows(x[None])
    scale = oracle.f16_bits_to_f32(rows[0, 16:18].view(np.uint16))[0]
    assert abs(c).max() == f["amax"] and scale == f["scale"]


def test_fp8_position_bytes_and_ratio():
    f = FACTS["fp8_bytes_per_position"]
    codes, scale = oracle.fp8_encode_part(np.ones(f["kv_lora"], np.float32))
    assert codes.nbytes + f["rope"] + 2 * np.float32(scale).nbytes == f["value"]
    ratio = (f["kv_lora"] + f["rope"]) * 4 / f["value"]
    assert abs(ratio - FACTS["fp8_f32_row_ratio"]["value"]) < 0.05


def test_e4m3_max():
    assert oracle.e4m3_decode(np.array([0x7E], np.uint8))[0] == FACTS["e4m3_max"]["value"]
    assert oracle.e4m3_encode(np.array([1e9], np.float32))[0] == 0x7E
