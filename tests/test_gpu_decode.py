"""GPU parity on a long-KV decode batch: one new token per request over 8k-128k cached keys,
so each row spans 2 to 32 fixed 4096-token KV splits whose partial (o, lse) states are merged
in ascending split order.

Checks: every row against the fp64 oracle (max |o - oracle| <= 1e-2, max |lse - oracle| <=
2e-3); each decode row bit-identical to the last row of its prompt's full prefill; the batch's
bits unchanged by running each request alone, by reversing the batch and by a workspace cap
that cuts the batch into several passes. A one-token row's partials take 16 slot rows per
(kv head, split), not a full tile's 256: the whole batch plans into 5.6 MB.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_helpers import Device, assert_bits_equal, assert_close_to_oracle, oracle_rows, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def oracle():
    import oracle as o
    o.build(force=False)
    return o


@pytest.fixture(scope="module")
def work():
    return wl.decode_batch()


@pytest.fixture(scope="module")
def dev(work):
    return Device(work)


@pytest.fixture(scope="module")
def decoded(dev, work):
    return dev.run(work.batches["decode"])


def test_decode_parity(oracle, work, decoded):
    b = work.batches["decode"]
    assert [r.kv_len for r in b.requests] == list(wl.DECODE_KV_LENS)
    ro, rl = oracle_rows(oracle, work, b)
    assert_close_to_oracle(*decoded, ro, rl, what="decode batch")


def test_decode_rows_match_full_prefill(work, dev, decoded):
    dec, full = work.batches["decode"], work.batches["full"]
    o_f, l_f = dev.run(full)
    for r in range(full.batch_size):
        ia, ib = wl.matching_rows(dec, r, full, r)
        assert list(ib) == [int(full.qo_indptr[r + 1]) - 1]
        assert_bits_equal(decoded[0][ia], o_f[ib], f"decode vs full o, kv_len {dec.requests[r].kv_len}")
        assert_bits_equal(decoded[1][ia], l_f[ib], f"decode vs full lse, kv_len {dec.requests[r].kv_len}")


def test_decode_alone_and_reversed(work, dev, decoded):
    dec = work.batches["decode"]
    n = dec.batch_size
    for r in range(n):
        one = wl.sub_batch(dec, work.prompts, work.page_size, [r])
        o, l = dev.run(one)
        assert_bits_equal(o[0], decoded[0][r], f"alone o {r}")
        assert_bits_equal(l[0], decoded[1][r], f"alone lse {r}")
    rev = wl.sub_batch(dec, work.prompts, work.page_size, list(range(n))[::-1])
    o, l = dev.run(rev)
    assert_bits_equal(o.flip(0), decoded[0], "reversed o")
    assert_bits_equal(l.flip(0), decoded[1], "reversed lse")


def test_decode_workspace_cap_passes(work, dev, decoded):
    dec = work.batches["decode"]
    assert dev.plan(dec).info.workspace_bytes < 6 << 20
    plan = dev.plan(dec, cap=3 << 20)
    say(f"decode batch under a 3 MiB cap: {plan.info.num_passes} passes, "
        f"workspace {plan.info.workspace_bytes} B")
    assert plan.info.num_passes > 1
    assert plan.info.workspace_bytes <= 3 << 20
    o, l = dev.run(dec, plan=plan)
    assert_bits_equal(o, decoded[0], "capped o")
    assert_bits_equal(l, decoded[1], "capped lse")
