"""GPU parity: libdpp against the fp64 oracle on every configuration, plus cached-vs-full
bit-exactness on the configurations that define it.

Tolerances: max |o - oracle| <= 1e-2 on bf16 outputs, max |lse - oracle| <= 2e-3 on fp32 lse.
Bit-exactness: the cached tail's rows equal the full prefill's rows bit for bit (o and lse).
"""
import numpy as np
import pytest
import torch

import workloads as wl
from dpp_header import parse
from gpu_helpers import (Device, assert_bits_equal, assert_close_to_oracle, oracle_rows,
                         sample_rows, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def oracle():
    import oracle as o
    o.build(force=False)
    return o


def _check_pairs(cached_batch, o_c, l_c, full_batch, o_f, l_f, pairs, what):
    for rc, rf in pairs:
        assert cached_batch.requests[rc].qo_len < cached_batch.requests[rc].kv_len, "the hit is real"
        ia, ib = wl.matching_rows(cached_batch, rc, full_batch, rf)
        assert len(ia) == cached_batch.requests[rc].qo_len
        assert_bits_equal(o_c[ia], o_f[ib], f"{what} o req {rc}")
        assert_bits_equal(l_c[ia], l_f[ib], f"{what} lse req {rc}")


def test_single_extend(oracle):
    work = wl.single_extend()
    dev = Device(work)
    full, cached = work.batches["full"], work.batches["cached"]
    o_f, l_f = dev.run(full)
    o_c, l_c = dev.run(cached)
    for b, o, l, name in ((full, o_f, l_f, "full"), (cached, o_c, l_c, "cached")):
        ro, rl = oracle_rows(oracle, work, b)
        assert_close_to_oracle(o, l, ro, rl, what=f"single extend {name}")
    _check_pairs(cached, o_c, l_c, full, o_f, l_f, [(0, 0)], "single extend")


RANDOM_CASES = [
    # (seed, hq, hkv, d, page, kv_dtype, specs [(prompt_len, qo_len)])
    (1, 32, 8, 128, 16, "bf16", [(1, 1), (2, 2), (63, 63), (64, 64), (65, 65), (67, 3), (300, 0), (129, 1)]),
    (2, 32, 8, 128, 1, "bf16", [(200, 17), (97, 97), (33, 32)]),
    (3, 32, 8, 128, 5, "bf16", [(150, 150), (151, 2), (40, 39)]),
    (4, 8, 8, 128, 64, "bf16", [(180, 180), (181, 35), (7, 7)]),
    (5, 16, 2, 128, 16, "bf16", [(130, 130), (257, 16)]),
    (6, 24, 4, 256, 16, "bf16", [(160, 160), (161, 5), (70, 1)]),
    (7, 24, 4, 256, 16, "fp8_e4m3", [(160, 160), (161, 5), (70, 1)]),
    (8, 32, 8, 128, 16, "fp8_e4m3", [(140, 140), (141, 9)]),
    (9, 32, 8, 128, 16, "bf16", [(4100, 12), (4096, 3), (4097, 1), (8200, 2)]),
    (10, 24, 4, 256, 16, "fp8_e4m3", [(4100, 30), (8193, 1)]),
    # head_dim 64: persistent wide (scalar page addressing) + narrow, per-lane pow2 pages,
    # general pages, fp8 with a split row, narrow rows spanning splits
    (11, 16, 4, 64, 16, "bf16", [(300, 300), (301, 3), (70, 1), (129, 16), (64, 64)]),
    (12, 16, 2, 64, 4, "bf16", [(200, 200), (201, 7), (33, 33)]),
    (13, 16, 4, 64, 5, "bf16", [(150, 150), (151, 2)]),
    (14, 16, 4, 64, 16, "fp8_e4m3", [(160, 160), (161, 5), (4100, 30)]),
    (15, 32, 8, 64, 16, "bf16", [(4100, 12), (8200, 2), (4097, 1)]),
    # the largest page size (one page holds a whole short prompt) and a 32-wide GQA group
    (16, 32, 8, 128, 1024, "bf16", [(3000, 3000), (3001, 5), (1025, 1), (1024, 2)]),
    (17, 64, 2, 128, 16, "bf16", [(200, 200), (201, 3), (33, 1)]),
    # head_dim 512 (64-row x 32-key tiles, a two-deep LDS ring): wide and narrow tiles, rows
    # across the 4096 split, per-lane power-of-two pages (16, 1) and general addressing (12, 64)
    (18, 16, 4, 512, 16, "bf16", [(300, 300), (301, 3), (70, 1), (129, 16), (64, 64), (4100, 12)]),
    (19, 16, 4, 512, 16, "fp8_e4m3", [(200, 200), (201, 2), (4100, 8), (33, 33)]),
    (20, 8, 2, 512, 1, "bf16", [(150, 150), (151, 4)]),
    (21, 8, 2, 512, 12, "fp8_e4m3", [(130, 130), (131, 1), (4097, 2)]),
    (22, 8, 8, 512, 64, "bf16", [(180, 180), (181, 35), (7, 7)]),
    # a 96-wide group: a wave's 32 packed rows span two tokens' heads (the kernels split packed
    # rows into token and q head by a multiply-shift)
    (23, 96, 1, 128, 16, "bf16", [(90, 90), (91, 3), (33, 1)]),
]


@pytest.mark.parametrize("case", RANDOM_CASES, ids=[f"seed{c[0]}" for c in RANDOM_CASES])
def test_random_against_oracle(oracle, case):
    seed, hq, hkv, d, page, kv_dtype, specs = case
    work = wl.random_workload(seed, hq=hq, hkv=hkv, d=d, page_size=page, kv_dtype=kv_dtype,
                              specs=specs)
    dev = Device(work)
    batch = work.batches["batch"]
    o, l = dev.run(batch)
    ro, rl = oracle_rows(oracle, work, batch)
    assert_close_to_oracle(o, l, ro, rl, what=f"random seed {seed}")
    # the same rows inside full prefills, placed in other pages, are bit-identical
    full = work.batches["full"]
    o_f, l_f = dev.run(full)
    pairs = [(i, i) for i in range(len(specs)) if 0 < batch.requests[i].qo_len < batch.requests[i].kv_len]
    _check_pairs(batch, o, l, full, o_f, l_f, pairs, f"random seed {seed}")


@pytest.mark.parametrize("layout", ["radix", "distinct"])
def test_extend_batch(oracle, layout):
    work = wl.extend_batch(layout=layout)
    dev = Device(work)
    cached, full = work.batches["cached"], work.batches["full"]
    o_c, l_c = dev.run(cached)
    ro, rl = oracle_rows(oracle, work, cached)
    assert_close_to_oracle(o_c, l_c, ro, rl, what=f"extend batch {layout}")
    o_f, l_f = dev.run(full)
    _check_pairs(cached, o_c, l_c, full, o_f, l_f, [(i, i) for i in range(16)], f"extend batch {layout}")
    # each extend alone gives the same bits as inside the batch
    for i in (0, 7, 15):
        one = wl.sub_batch(cached, work.prompts, work.page_size, [i])
        o1, l1 = dev.run(one)
        a, b = int(cached.qo_indptr[i]), int(cached.qo_indptr[i + 1])
        assert_bits_equal(o1, o_c[a:b], f"extend batch request {i} alone vs batched")
        assert_bits_equal(l1, l_c[a:b], f"extend batch request {i} alone vs batched (lse)")


def test_cold_prefill(oracle):
    work = wl.cold_prefill()
    dev = Device(work)
    full = work.batches["full"]
    o, l = dev.run(full)
    rows = sample_rows(full, 24, seed=3)
    ro, rl = oracle_rows(oracle, work, full, rows)
    assert_close_to_oracle(o, l, ro, rl, rows=rows, what="cold prefill sampled rows")
    for i in (0, 9):
        one = wl.sub_batch(full, work.prompts, work.page_size, [i])
        o1, l1 = dev.run(one)
        a, b = int(full.qo_indptr[i]), int(full.qo_indptr[i + 1])
        assert_bits_equal(o1, o[a:b], f"cold prefill request {i} alone vs batch of 16")
        assert_bits_equal(l1, l[a:b], f"cold prefill request {i} alone vs batch of 16 (lse)")


def test_mixed_batch(oracle):
    work = wl.mixed_batch()
    dev = Device(work)
    mixed, full = work.batches["mixed"], work.batches["full"]
    o_m, l_m = dev.run(mixed)
    rows = np.concatenate([sample_rows(wl.sub_batch(mixed, work.prompts, 16, [0]), 40, seed=4),
                           np.arange(3700, mixed.num_q_tokens)])
    ro, rl = oracle_rows(oracle, work, mixed, rows)
    assert_close_to_oracle(o_m, l_m, ro, rl, rows=rows, what="mixed batch")
    o_f, l_f = dev.run(full)
    _check_pairs(mixed, o_m, l_m, full, o_f, l_f, [(i + 1, i) for i in range(7)], "mixed batch")
    # the full 3700-token request in the mixed batch equals itself alone
    one = wl.sub_batch(mixed, work.prompts, 16, [0])
    o1, l1 = dev.run(one)
    assert_bits_equal(o1, o_m[:3700], "mixed batch: full request alone vs mixed")
    assert_bits_equal(l1, l_m[:3700], "mixed batch: full request alone vs mixed (lse)")


@pytest.fixture(scope="module")
def long_fp8_work():
    return wl.long_fp8()


def pass_spread_rows(plan, batch, group: int, n_rows: int, seed: int) -> np.ndarray:
    """About n_rows global q tokens spread over every pass of the plan and every split count:
    the first and last token of each pass's tiles, the tokens on both sides of every
    4096-token split boundary, and random tokens drawn pass by pass."""
    parsed = parse(plan.header())
    bm = plan.info.block_m
    tiles = {}
    for it in parsed.items:
        r, rs, ps = int(it[0]), int(it[1]), int(it[7])
        q_start, qo_len = int(parsed.requests[r][0]), int(parsed.requests[r][1])
        rows = min(bm, qo_len * group - rs)
        tiles[(r, rs)] = (ps, q_start + rs // group, q_start + (rs + rows - 1) // group)
    passes = sorted({t[0] for t in tiles.values()})
    rng = np.random.default_rng(seed)
    pick = set()
    per_pass = max(2, n_rows // len(passes))
    for ps in passes:
        spans = [(a, b) for (p_, a, b) in tiles.values() if p_ == ps]
        lo, hi = min(a for a, _ in spans), max(b for _, b in spans)
        pick |= {lo, hi}
        toks = np.concatenate([np.arange(a, b + 1) for a, b in spans])
        pick |= set(int(x) for x in rng.choice(toks, size=min(per_pass, toks.size), replace=False))
    for r, req in enumerate(batch.requests):
        a = int(batch.qo_indptr[r])
        ctx = req.kv_len - req.qo_len
        for boundary in range(4096, req.kv_len, 4096):
            for pos in (boundary - 1, boundary):
                if ctx <= pos < req.kv_len:
                    pick.add(a + pos - ctx)
    return np.array(sorted(pick), dtype=np.int64)


@pytest.mark.parametrize("name", ["prefill_8192", "prefill_32768", "extend"])
def test_long_fp8_parity(oracle, long_fp8_work, name):
    """Hundreds of rows of each long fp8 batch against the oracle, spread over every pass of
    the 256 MiB-capped plan and every split count (1-8 at 32,768 tokens)."""
    work = long_fp8_work
    dev = Device(work)
    b = work.batches[name]
    p = dev.plan(b, cap=256 << 20)
    o, l = dev.run(b, plan=p)
    g = work.num_qo_heads // work.num_kv_heads
    rows = pass_spread_rows(p, b, g, 280, seed=5)
    splits = {(b.requests[0].kv_len - b.requests[0].qo_len + int(t)) // 4096 + 1 for t in rows}
    say(f"long fp8 {name}: {p.info.num_passes} passes, {len(rows)} oracle rows, split counts {sorted(splits)}")
    assert len(rows) >= 256
    if name == "prefill_32768":
        assert p.info.num_passes >= 10 and splits == set(range(1, 9))
    ro, rl = oracle_rows(oracle, work, b, rows)
    assert_close_to_oracle(o, l, ro, rl, rows=rows, what=f"long fp8 {name}")


def test_long_fp8_extend_matches_32k_prefill(long_fp8_work):
    work = long_fp8_work
    dev = Device(work)
    ext, full = work.batches["extend"], work.batches["prefill_32768"]
    o_e, l_e = dev.run(ext, cap=256 << 20)
    o_f, l_f = dev.run(full, cap=256 << 20)
    _check_pairs(ext, o_e, l_e, full, o_f, l_f, [(0, 0)], "long fp8 extend vs 32k prefill")


def test_long_fp8_workspace_cap_does_not_change_bits(long_fp8_work):
    work = long_fp8_work
    dev = Device(work)
    b = work.batches["prefill_8192"]
    p_small = dev.plan(b, cap=32 << 20)
    p_big = dev.plan(b, cap=0)
    say(f"passes: cap 32 MiB -> {p_small.info.num_passes}, no cap -> {p_big.info.num_passes}")
    assert p_small.info.num_passes > p_big.info.num_passes == 1
    assert p_small.workspace_bytes <= 32 << 20
    o1, l1 = dev.run(b, plan=p_small)
    o2, l2 = dev.run(b, plan=p_big)
    assert_bits_equal(o1, o2, "long fp8 8k: cap 32 MiB vs unbounded")
    assert_bits_equal(l1, l2, "long fp8 8k: cap 32 MiB vs unbounded (lse)")
