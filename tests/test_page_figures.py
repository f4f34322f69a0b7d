"""Host-side arithmetic pinned to figures the pages print
(tests/golden/page_figures.json)."""
import json
import os

import bench

GOLD = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def fig():
    with open(GOLD) as f:
        return json.load(f)


def test_table_size_figures():
    g = fig()
    R, d, K = g["table_rows"]["value"], g["row_dim"]["value"], g["rows_per_token"]["value"]
    assert (R, d, K) == (20_000_000, 2560, bench.K_ROWS)
    assert round(R * d / 1e9, 1) == g["table_params_billion"]["value"]
    assert round(bench.table_bytes(R, d, "bf16") / 2**30, 1) == g["table_gib_bf16"]["value"]
    assert abs(bench.table_bytes(R, d, "bf16") / 1e9 - g["table_gb_bf16_approx"]["value"]) < 1
    assert abs(R * d / 1e9 - g["table_gb_int8_approx"]["value"]) < 1


def test_dma_estimate_reproduces_the_page():
    e = fig()["dma_estimate"]
    t = bench.dma_time_estimate_us(e["K"], e["d"], e["bytes_per_elem"], e["bandwidth_GBps"])
    assert round(t, 3) == e["microseconds"]


def test_nominal_bytes_per_token():
    # 16 rows of 5120 B + e1 row + residual read + output write + token id
    assert bench.nominal_bytes_per_token(2560, "bf16", True, True) == 16 * 5120 + 3 * 5120 + 4
    assert bench.nominal_bytes_per_token(2560, "bf16", True, False) == 16 * 5120 + 2 * 5120 + 4
    assert bench.nominal_bytes_per_token(2560, "int8", True, True) == 16 * 2564 + 3 * 5120 + 4
