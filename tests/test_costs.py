"""The cost model behind the benchmark's roofline reproduces the worked
arithmetic the pages print (tests/golden/cost_examples.json, each entry cited
there), and the path's own counts follow from it."""
import json
import os

import pytest

from paged_mla_decode_amd import costs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "cost_examples.json")
ENTRIES = json.load(open(GOLDEN))["entries"]


@pytest.mark.parametrize("e", ENTRIES, ids=[e["id"] for e in ENTRIES])
def test_printed_worked_examples(e):
    got = getattr(costs, e["fn"])(**e["args"])
    assert abs(got - e["printed"]) <= e["tol"], (e["id"], got, e["printed"], e["cite"])


def test_exact_mac_counts_and_ratio():
    a = costs.absorb_macs_per_query(128, 128, 512)
    d = costs.decompress_macs_per_query(4096, 512, 128, 128)
    assert a == 8_388_608 and d == 34_359_738_368
    assert d // a == 4096  # the ratio is the history length: four orders of magnitude here


def test_path_counts():
    # One MLA cache row: 576 values, shared by all heads.
    assert costs.mla_bytes_per_token(2) == 1152 and costs.mla_bytes_per_token(1) == 576
    assert costs.mla_decode_latent_bytes(10, 2) == 11520
    # 2 flops per MAC, 576-wide score plus 512-wide value product per head and token.
    assert costs.mla_decode_flops(1, 128) == 278_528
    # At H = 128 in bf16 the decode sits at 241.8 flop/B, below MI355X's ridge.
    intensity = costs.mla_decode_flops(1, 128) / costs.mla_decode_latent_bytes(1, 2)
    assert abs(intensity - 241.78) < 0.01
    assert intensity < costs.ridge_flop_per_byte(2.5e15, 8e12)
    # The two projections move the same bytes at this shape: weight, 128-wide side, 512-wide side.
    assert costs.absorb_bytes(128, 128) == 2 * (512 * 128 * 128 + 128 * 128 * 128 + 128 * 128 * 512)
    assert costs.project_bytes(128, 128) == costs.absorb_bytes(128, 128)
