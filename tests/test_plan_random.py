"""Planner invariants on random batches (no GPU): request lengths from empty
to long, page sizes from 1 to 1024 (powers of two and not), 1 to 9 query rows
per request, every head count and the flags that change the plan, several CU
counts and split caps. The invariants are those of tests/test_plan.py."""
import numpy as np
import pytest

import paged_mla_decode_amd as m
import workloads
from test_plan import build, check_invariants


def random_case(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    B = int(rng.integers(1, 12))
    kind = rng.integers(0, 3, size=B)
    lens = np.where(kind == 0, rng.integers(0, 40, size=B),
                    np.where(kind == 1, rng.integers(40, 3000, size=B), rng.integers(3000, 40000, size=B)))
    ps = int(rng.choice([1, 3, 16, 48, 64, 128, 1024]))
    H = int(rng.choice([16, 32, 64, 128]))
    rows = rng.integers(0, 10, size=B) if rng.random() < 0.5 else 1
    flags = 0
    if rng.random() < 0.5:
        flags |= m.MLA_DECODE_SHARED_ROWS
    graph = rng.random() < 0.3
    cus = int(rng.choice([1, 7, 64, 80, 256]))
    splits = int(rng.choice([0, 0, 1, 3]))
    return lens, ps, H, rows, flags, graph, cus, splits


@pytest.mark.parametrize("seed", range(40))
def test_random_plans_keep_the_invariants(seed):
    lens, ps, H, rows, flags, graph, cus, splits = random_case(seed)
    batch = workloads.random_decode_batch(seed, lens, num_heads=H, page_size=ps, rows_per_request=rows,
                                          layout_only=True)
    max_rows = max(1, batch.num_rows + 3) if graph else 0
    p = m.make_params(H, ps, num_cus=cus, max_splits=splits,
                      flags=flags | (m.MLA_DECODE_GRAPH_SAFE if graph else 0), max_rows=max_rows)
    h, items, merges, workers = build(p, batch)
    check_invariants(p, batch, h, items, merges, workers)
