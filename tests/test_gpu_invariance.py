"""GPU batch-invariance: the bits of a row do not depend on its batch-mates, its page
placement, the order requests are listed in, repeated runs, or the workspace cap.

The batch-mate case mirrors the measurement on the sglang PR #46351 page (kahyunnam's
status comment): a 512-token request alone versus beside 63 one-row batch-mates, which
FlashInfer's eager plan changed by 3.9e-3; here it must not change at all.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_helpers import Device, assert_bits_equal, assert_close_to_oracle, oracle_rows, say

pytestmark = pytest.mark.gpu

SHAPES = dict(hq=32, hkv=8, d=128)


@pytest.fixture(scope="module")
def oracle():
    import oracle as o
    o.build(force=False)
    return o


def test_batch_mates_do_not_change_a_request():
    specs = [(512, 512)] + [(int(L), 1) for L in np.random.default_rng(0).integers(1, 2000, 63)]
    work = wl.random_workload(40, **SHAPES, page_size=16, kv_dtype="bf16", specs=specs)
    dev = Device(work)
    batch = work.batches["batch"]
    o_all, l_all = dev.run(batch)
    alone = wl.sub_batch(batch, work.prompts, 16, [0])
    o_1, l_1 = dev.run(alone)
    assert_bits_equal(o_1, o_all[:512], "512-token request alone vs + 63 one-row mates")
    assert_bits_equal(l_1, l_all[:512], "lse")
    # and each one-row mate alone
    for i in (1, 30, 63):
        one = wl.sub_batch(batch, work.prompts, 16, [i])
        o_i, l_i = dev.run(one)
        r = int(batch.qo_indptr[i])
        assert_bits_equal(o_i, o_all[r:r + 1], f"mate {i}")
        assert_bits_equal(l_i, l_all[r:r + 1], f"mate {i} lse")


@pytest.mark.parametrize("tail", list(range(1, 17)) + [31, 32, 33, 37, 64, 127, 128, 129])
def test_every_short_tail_matches_full_prefill(tail):
    """Tails of 1..16 tokens are where FlashInfer's tile choice flipped (the page measured
    8 of 12 such cases differing); every tail must equal the full prefill's rows."""
    L = 700 + tail
    work = wl.random_workload(100 + tail, **SHAPES, page_size=16, kv_dtype="bf16",
                              specs=[(L, tail)])
    dev = Device(work)
    o_c, l_c = dev.run(work.batches["batch"])
    o_f, l_f = dev.run(work.batches["full"])
    ia, ib = wl.matching_rows(work.batches["batch"], 0, work.batches["full"], 0)
    assert_bits_equal(o_c[ia], o_f[ib], f"tail {tail}")
    assert_bits_equal(l_c[ia], l_f[ib], f"tail {tail} lse")


def test_page_placement_and_request_order():
    specs = [(300, 300), (301, 7), (90, 90), (1200, 33)]
    work = wl.random_workload(41, **SHAPES, page_size=16, kv_dtype="bf16", specs=specs)
    dev = Device(work)
    b = work.batches["batch"]
    o, l = dev.run(b)
    # reversed request order -> different item order, same rows
    rev = wl.sub_batch(b, work.prompts, 16, [3, 2, 1, 0])
    o_r, l_r = dev.run(rev)
    for i_new, i_old in enumerate([3, 2, 1, 0]):
        a0, a1 = int(b.qo_indptr[i_old]), int(b.qo_indptr[i_old + 1])
        b0 = int(rev.qo_indptr[i_new])
        assert_bits_equal(o_r[b0:b0 + a1 - a0], o[a0:a1], f"order: request {i_old}")
        assert_bits_equal(l_r[b0:b0 + a1 - a0], l[a0:a1], f"order: request {i_old} lse")
    # the same prompts copied into other (shuffled) pages
    pool = wl.PagePool(work.num_pages * 2, 16, 8, 128, "bf16", seed=999)
    moved = [wl.Request(r.prompt, r.kv_len, r.qo_len, pool.place(work.prompts[r.prompt], r.kv_len))
             for r in b.requests]
    mb = wl.make_batch(moved, work.prompts, 16)
    work2 = wl.Workload(**{**work.__dict__, "k_pool": pool.k, "v_pool": pool.v})
    o_m, l_m = Device(work2).run(mb)
    assert_bits_equal(o_m, o, "page placement")
    assert_bits_equal(l_m, l, "page placement lse")


def test_repeated_runs_are_identical():
    work = wl.random_workload(42, **SHAPES, page_size=16, kv_dtype="bf16",
                              specs=[(1028, 1028)] * 4 + [(1030, 3)])
    dev = Device(work)
    b = work.batches["batch"]
    p = dev.plan(b)
    o0, l0 = dev.run(b, plan=p)
    for i in range(10):
        o, l = dev.run(b, plan=p)
        assert_bits_equal(o, o0, f"repeat {i}")
        assert_bits_equal(l, l0, f"repeat {i} lse")


def test_empty_and_degenerate_batches(oracle):
    work = wl.random_workload(43, **SHAPES, page_size=16, kv_dtype="bf16",
                              specs=[(5, 0), (1, 1), (16, 16), (17, 1)])
    dev = Device(work)
    b = work.batches["batch"]
    o, l = dev.run(b)
    ro, rl = oracle_rows(oracle, work, b)
    assert_close_to_oracle(o, l, ro, rl, what="degenerate batch")
    # a batch with no query rows at all runs nothing and returns empty outputs
    empty = wl.sub_batch(b, work.prompts, 16, [0])
    o_e, l_e = dev.run(empty)
    assert o_e.shape[0] == 0 and l_e.shape[0] == 0


PERMUTE_CASES = [
    # (name, workload builder, batch, cap): a persistent mixed batch, narrow extends, fp8 with
    # merges over several passes, the long-KV decode rows
    ("mixed", lambda: wl.mixed_batch(), "mixed", None),
    ("extend", lambda: wl.extend_batch(layout="distinct"), "cached", None),
    ("fp8_split", lambda: wl.random_workload(10, hq=24, hkv=4, d=256, page_size=16, kv_dtype="fp8_e4m3",
                                              specs=[(4100, 30), (8193, 1), (9000, 40), (300, 300)]),
     "batch", 4 << 20),
]


@pytest.mark.parametrize("case", PERMUTE_CASES, ids=[c[0] for c in PERMUTE_CASES])
def test_permuted_work_order_gives_the_same_bits(case):
    """The test-only work permutation (items, merges, and so the workgroup, XCD and persistent
    chain of every unit) changes no bit: the reduction order of a row is fixed by its own
    position and the constants (sglang PR #46351 page, "Root cause")."""
    name, build, which, cap = case
    work = build()
    dev = Device(work)
    batch = work.batches[which]
    o_ref, l_ref = dev.run(batch, cap=cap)
    for seed in (1, 2, 3):
        w = work
        kw = dict(kv_dtype=w.kv_dtype, k_scale=w.k_scale, v_scale=w.v_scale, permute_seed=seed)
        if cap is not None:
            kw["workspace_cap"] = cap
        p = dev.dpp.plan(w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size,
                         batch.qo_indptr, batch.kv_indptr, batch.kv_last_page_len, **kw)
        o, l = dev.run(batch, plan=p)
        assert_bits_equal(o, o_ref, f"{name} permutation {seed} o")
        assert_bits_equal(l, l_ref, f"{name} permutation {seed} lse")
