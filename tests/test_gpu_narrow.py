"""GPU parity of the narrow (at most 16 packed rows a tile) kernels on rows with many keys.

A pass runs on the narrow instantiation only when every tile in it is narrow, so these batches
hold nothing but short extends and one-token rows: 1-4 tokens at a GQA group of 4 (16 rows),
1-2 at a group of 6 (12 rows), behind prefixes of 300-9,000 tokens, among them rows on both
sides of the 4,096-token split boundary. They cover every narrow instantiation that ships:
fp8 E4M3 at head_dim 128, 256 and 512, bf16 at 64, 128, 256 and 512, with per-lane power-of-two page
addressing (page 16) and general addressing (pages 12 and 1,024), and at head_dim 128 both
the head_dim-split launch (few units) and the one-workgroup-per-unit launch (many units).

Every row is compared with the oracle, and bit for bit with the same row of its prompt's full
prefill, which runs on the wide kernels (sglang PR #46351 page, "Validation": short tails must
match the full prefill; the model-serving-minefield issue #73 report, "What were you serving":
the fp8 E4M3 KV cache at 24/4/256).
"""
import numpy as np
import pytest

import workloads as wl
from dpp_header import parse
from gpu_helpers import Device, assert_bits_equal, assert_close_to_oracle, oracle_rows, say

pytestmark = pytest.mark.gpu

SHAPES = {  # name: (hq, hkv, d, kv_dtype)
    "fp8_d128": (32, 8, 128, "fp8_e4m3"),
    "fp8_d256": (24, 4, 256, "fp8_e4m3"),
    "bf16_d64": (16, 4, 64, "bf16"),
    "bf16_d128": (32, 8, 128, "bf16"),
    "bf16_d256": (24, 4, 256, "bf16"),
    "bf16_d512": (16, 4, 512, "bf16"),
    "fp8_d512": (16, 4, 512, "fp8_e4m3"),
}


def _narrow_specs(g: int, seed: int):
    """(prompt_len, qo_len) pairs: every request's tile holds at most 16 packed rows."""
    tmax = 16 // g
    rng = np.random.default_rng(seed)
    t = lambda: int(rng.integers(1, tmax + 1))  # noqa: E731
    return [(300, t()), (1000, tmax), (4097, min(2, tmax)), (4096, 1), (4100, t()),
            (8193, 1), (9000, t()), (2049, tmax)]


@pytest.fixture(scope="module")
def oracle():
    import oracle as o
    o.build(force=False)
    return o


def _run_case(oracle, seed, shape, page, specs):
    hq, hkv, d, kv_dtype = SHAPES[shape]
    g = hq // hkv
    work = wl.random_workload(seed, hq=hq, hkv=hkv, d=d, page_size=page, kv_dtype=kv_dtype,
                              specs=specs, pool_factor=2)
    dev = Device(work)
    batch, full = work.batches["batch"], work.batches["full"]
    p = dev.plan(batch)
    parsed = parse(p.header())
    bm = p.info.block_m
    for it in parsed.items:
        qo_len = int(parsed.requests[int(it[0])][1])
        assert min(bm, qo_len * g - int(it[1])) <= 16, "every tile is narrow"
    say(f"narrow {shape} page {page}: {len(specs)} requests, {len(parsed.items)} items x {hkv} kv heads")
    o, l = dev.run(batch, plan=p)
    ro, rl = oracle_rows(oracle, work, batch)
    assert_close_to_oracle(o, l, ro, rl, what=f"narrow {shape} page {page}")
    o_f, l_f = dev.run(full)
    for i in range(len(specs)):
        ia, ib = wl.matching_rows(batch, i, full, i)
        assert_bits_equal(o[ia], o_f[ib], f"narrow {shape} page {page} request {i} o vs full prefill")
        assert_bits_equal(l[ia], l_f[ib], f"narrow {shape} page {page} request {i} lse vs full prefill")


CASES = [(shape, page) for shape in SHAPES for page in (16, 12, 1024)]


@pytest.mark.parametrize("shape,page", CASES, ids=[f"{s}-page{p}" for s, p in CASES])
def test_narrow_multi_key_rows(oracle, shape, page):
    hq, hkv = SHAPES[shape][:2]
    seed = 70 + list(SHAPES).index(shape) * 7 + {16: 0, 12: 1, 1024: 2}[page]
    _run_case(oracle, seed, shape, page, _narrow_specs(hq // hkv, seed))


@pytest.mark.parametrize("page", [16, 12])
def test_narrow_many_units_one_workgroup_each(oracle, page):
    """More than one unit per two compute units: the head_dim-128 narrow launch runs every
    unit on one workgroup instead of splitting head_dim over two."""
    rng = np.random.default_rng(90 + page)
    specs = [(int(rng.integers(200, 3000)), int(rng.integers(1, 5))) for _ in range(34)]
    specs += [(4097, 2), (5000, 4)]
    _run_case(oracle, 90 + page, "bf16_d128", page, specs)
