"""Host-side work/traffic model checked against numbers the pages print."""
import json
import math
import os

from causal_gqa_prefill_amd import roofline
from causal_gqa_prefill_amd.configs import CONFIGS

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                     "page_numbers.json")))


def test_ridges_match_pages():
    for name, r in GOLDEN["ridges"].items():
        if name.startswith("_"):
            continue
        assert round(roofline.ridge(r["tflops"], r["gbps"]), 1) == r["ridge"], name


def test_l_ridge_matches_pages():
    ridges = GOLDEN["ridges"]
    for c in GOLDEN["l_ridge"]["cases"]:
        r = ridges[c["device"]]
        lr = roofline.l_ridge(roofline.ridge(r["tflops"], r["gbps"]), c["g"])
        assert round(lr) == c["tokens"], c


def test_intensity_example():
    ex = GOLDEN["intensity_example"]
    ai = roofline.intensity_kv(ex["L"], ex["g"])
    assert ai == ex["ai"]
    h = GOLDEN["ridges"]["H100 SXM"]
    assert int(ai / roofline.ridge(h["tflops"], h["gbps"])) == ex["times_h100_ridge"]
    # AI = flops / K+V bytes for any shape with g = n_q / n_kv
    f = roofline.attn_flops(1, ex["L"], 32, 128)
    b = roofline.kv_bytes(1, ex["L"], 8, 128)
    assert f / b == ai


def test_kv_bytes_per_token():
    ex = GOLDEN["kv_bytes_per_token"]
    per_layer = roofline.kv_bytes(1, 1, ex["n_kv"], ex["d_h"])
    assert per_layer * ex["layers"] == ex["bytes"]


def test_score_table_bytes():
    for c in GOLDEN["score_table_bytes"]["cases"]:
        gb = c["L"] * c["L"] * c["heads"] * 2 / 1e9
        assert abs(gb - c["gb"]) / c["gb"] < 0.005, c


def test_causal_halves_flops_not_bytes():
    # "Scales with": the causal mask halves flops and leaves bytes alone;
    # batch leaves AI unchanged; g multiplies AI
    assert roofline.attn_flops(2, 100, 8, 64, False) == 2 * roofline.attn_flops(2, 100, 8, 64)
    for B in (1, 4):
        ai = roofline.attn_flops(B, 1024, 32, 128) / roofline.kv_bytes(B, 1024, 8, 128)
        assert ai == roofline.intensity_kv(1024, 4)


def test_mi355x_numbers():
    assert abs(roofline.MI355X_BF16_DENSE_TFLOPS - 256 * 4096 * 2.4e9 / 1e12) < 0.1
    r = roofline.ridge(roofline.MI355X_BF16_DENSE_TFLOPS, roofline.MI355X_HBM_GBPS)
    assert abs(r - 314.6) < 0.1
    assert round(roofline.l_ridge(r, 1)) == 629


def test_config_flops():
    want = {1: 8388608, 2: 137438953472, 3: 549755813888,
            4: 17592186044416, 5: 158329674399744}
    for c in CONFIGS:
        assert roofline.attn_flops(c.B, c.L, c.n_q, c.d_h) == want[c.index]
    assert roofline.attainable(64, 2516.6e12, 8e12) == 64 * 8e12
    assert math.isclose(roofline.attainable(1e6, 2516.6e12, 8e12), 2516.6e12)
