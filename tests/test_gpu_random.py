"""Seeded random small batches through the whole decode path against the
oracle: head counts, page sizes (powers of two and not), bf16 and fp8 caches,
bf16 and fp32 outputs, several query rows per request with and without shared
rows, CU counts and split caps drawn per case."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import compare, require_gpu, run_decode, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.mark.parametrize("seed", range(48))
def test_random_batch_against_the_oracle(dev, seed):
    rng = np.random.Generator(np.random.PCG64(1000 + seed))
    B = int(rng.integers(1, 7))
    lens = [int(x) for x in rng.choice([0, 1, 5, 31, 32, 33, 200, 777, 1500, 3000], size=B)]
    ps = int(rng.choice([1, 3, 16, 64, 128]))
    H = int(rng.choice([16, 32, 64, 128]))
    kv = str(rng.choice(["bf16", "fp8_e4m3fn"]))
    out_dtype = str(rng.choice(["bf16", "fp32"]))
    rows = [int(x) for x in rng.integers(0, 5, size=B)] if rng.random() < 0.5 else 1
    shared = bool(rng.random() < 0.5)
    cus = int(rng.choice([1, 7, 32, 256]))
    splits = int(rng.choice([0, 0, 1, 3]))
    batch = workloads.random_decode_batch(2000 + seed, lens, num_heads=H, page_size=ps, cache_dtype=kv,
                                          rows_per_request=rows)
    what = (f"seed={seed} B={B} lens={lens} ps={ps} H={H} kv={kv} out={out_dtype} rows={rows} "
            f"shared={shared} cus={cus} splits={splits}")
    say(what)
    ref_out, ref_lse = oracle.decode_batch(batch)
    out, lse, dec = run_decode(batch, dev, out_dtype, max_splits=splits, num_cus=cus, shared_rows=shared)
    compare(out, lse, ref_out, ref_lse, out_dtype == "fp32", what)
