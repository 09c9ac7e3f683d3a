"""GPU tests of persistent launches (chains of units per workgroup).

A wide bf16 launch of the eight-wave kernel (head_dim 128: 256-row tiles of two 16-row blocks
a wave; head_dim 256: 128-row tiles of one block a wave) runs as 256 workgroups, each over a
chain of units (q tile, KV split, kv head) that the planner fixes; between units a workgroup
swaps page-id tables, reloads Q and its first K/V tiles while writing the previous unit's
rows. These cases have more than 256 units (chains longer than one), a request crossing the
4096-token split (partials inside chains), ragged last tiles and every page-addressing mode of
the wide kernel: scalar descriptors (page size a power of two holding at least one wave-wide
load's key rows: 4 at head_dim 128, 2 at 256), per-lane power-of-two (2 at head_dim 128) and
general (12); page size 1 does not fit two page tables and runs one unit per workgroup. Each
case is checked against the oracle on sampled rows, and requests run alone (chains of their
own units only) must give the same bits as inside the batch.
"""
import numpy as np
import pytest

import workloads as wl
from gpu_helpers import Device, assert_bits_equal, assert_close_to_oracle, oracle_rows, sample_rows, say

pytestmark = pytest.mark.gpu

SPECS = [(1500, 1500), (1200, 700), (4300, 300), (900, 900), (77, 77), (260, 33)]
SHAPES = {"d128": (32, 8, 128), "d256": (24, 4, 256)}  # hq, hkv, head_dim


@pytest.fixture(scope="module")
def oracle():
    import oracle as o
    o.build(force=False)
    return o


@pytest.mark.parametrize("shape", list(SHAPES))
@pytest.mark.parametrize("page", [16, 4, 2, 12, 1])
def test_chains_against_oracle_and_alone(oracle, page, shape):
    hq, hkv, d = SHAPES[shape]
    work = wl.random_workload(700 + page + d, hq=hq, hkv=hkv, d=d, page_size=page, kv_dtype="bf16",
                              specs=SPECS)
    dev = Device(work)
    batch = work.batches["batch"]
    plan = dev.plan(batch)
    units = len(__import__("dpp_header").parse(plan.header()).units)
    say(f"{shape} page {page}: {plan.info.num_prefill_items} items, {units} unit records")
    if page > 1:
        assert units > 256, "chains longer than one unit"
    else:
        assert units == 0, "page size 1: one unit per workgroup"
    o, l = dev.run(batch, plan=plan)
    rows = sample_rows(batch, 24, seed=page)
    ro, rl = oracle_rows(oracle, work, batch, rows=rows)
    assert_close_to_oracle(o, l, ro, rl, rows=rows, what=f"chains {shape} page {page}")
    for i in (0, 2, 4):
        alone = wl.sub_batch(batch, work.prompts, page, [i])
        o_1, l_1 = dev.run(alone)
        a, b = int(batch.qo_indptr[i]), int(batch.qo_indptr[i + 1])
        assert_bits_equal(o_1, o[a:b], f"{shape} page {page}: request {i} alone vs in the batch")
        assert_bits_equal(l_1, l[a:b], f"{shape} page {page}: request {i} alone vs in the batch (lse)")


@pytest.mark.parametrize("shape", list(SHAPES))
def test_chained_and_unchained_launches_agree(shape):
    """One set of prompts placed with page size 16 (persistent launch, scalar descriptors),
    12 (persistent, per-lane general addressing) and 1 (one unit per workgroup): the outputs
    are bit-identical -- neither the chain a unit lands in nor the page layout enters a
    row's arithmetic."""
    hq, hkv, d = SHAPES[shape]
    outs = {}
    for page in (16, 12, 1):
        work = wl.random_workload(790, hq=hq, hkv=hkv, d=d, page_size=page, kv_dtype="bf16", specs=SPECS)
        outs[page] = Device(work).run(work.batches["batch"])
    for page in (12, 1):
        assert_bits_equal(outs[page][0], outs[16][0], f"page {page} vs page 16")
        assert_bits_equal(outs[page][1], outs[16][1], f"page {page} vs page 16 (lse)")
    assert np.isfinite(outs[16][0].float().numpy()).all()


@pytest.mark.parametrize("shape", list(SHAPES))
def test_chained_passes_under_a_workspace_cap(shape):
    """A cap small enough to cut the partial-holding tiles of a 9000-token prompt into several
    passes: every pass is its own persistent launch over its own unit records (plus a merge);
    the rows are bit-identical to the uncapped single pass."""
    specs = [(9000, 900), (1300, 1300), (600, 200)]
    hq, hkv, d = SHAPES[shape]
    work = wl.random_workload(795, hq=hq, hkv=hkv, d=d, page_size=16, kv_dtype="bf16", specs=specs)
    dev = Device(work)
    batch = work.batches["batch"]
    free = dev.plan(batch)
    capped = dev.plan(batch, cap=6 << 20)
    say(f"passes: uncapped {free.info.num_passes}, capped {capped.info.num_passes}")
    assert free.info.num_passes == 1 and capped.info.num_passes > 1
    header = __import__("dpp_header").parse(capped.header())
    assert len(set(int(x) for x in header.units[:, 14])) == capped.info.num_passes
    o1, l1 = dev.run(batch, plan=free)
    o2, l2 = dev.run(batch, plan=capped)
    assert_bits_equal(o2, o1, "capped vs uncapped")
    assert_bits_equal(l2, l1, "capped vs uncapped (lse)")
