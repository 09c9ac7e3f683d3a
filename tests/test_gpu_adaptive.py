"""GPU negative control: the adaptive-tile comparison mode (dpp_plan_create_ex with
DPP_PLAN_ADAPTIVE_KV_TILE) picks the KV tile from the batch the way FlashInfer picks its q tile
(average packed query length <= 16 -> the other tile), and so loses what the default plans
keep: the cached tails of the extend batch (32-key tiles) no longer reproduce their full
prefills (64-key tiles) bit for bit, while both stay within the oracle tolerance. The default
plans of the same batches stay bit-exact.
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


def _run(dev, batch, adaptive):
    w = dev.work
    p = dev.dpp.plan(w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size, batch.qo_indptr,
                     batch.kv_indptr, batch.kv_last_page_len, adaptive_kv_tile=adaptive)
    return p.info.block_n, dev.run(batch, plan=p)


def test_adaptive_tile_breaks_cached_vs_full_and_default_does_not(oracle):
    work = wl.extend_batch(layout="radix")
    dev = Device(work)
    cached, full = work.batches["cached"], work.batches["full"]
    bn_c, (o_c, l_c) = _run(dev, cached, True)
    bn_f, (o_f, l_f) = _run(dev, full, True)
    assert (bn_c, bn_f) == (32, 64)
    ro, rl = oracle_rows(oracle, work, cached)
    assert_close_to_oracle(o_c, l_c, ro, rl, what="adaptive-tile extend batch")
    ia = np.concatenate([wl.matching_rows(cached, r, full, r)[0] for r in range(cached.batch_size)])
    ib = np.concatenate([wl.matching_rows(cached, r, full, r)[1] for r in range(cached.batch_size)])
    do = float((o_c[ia].float() - o_f[ib].float()).abs().max())
    dl = float((l_c[ia] - l_f[ib]).abs().max())
    n_lse = int((l_c[ia].view(torch.int32) != l_f[ib].view(torch.int32)).sum())
    say(f"adaptive tile: cached vs full max|diff| o = {do:.3e}, lse = {dl:.3e}, "
        f"{n_lse} of {l_c[ia].numel()} lse values differ")
    assert n_lse > 0, "the comparison mode should move the reduction split"
    assert do <= 1e-2 and dl <= 2e-3
    # default plans of the same batches: bit-exact
    _, (o_c0, l_c0) = _run(dev, cached, False)
    _, (o_f0, l_f0) = _run(dev, full, False)
    assert_bits_equal(o_c0[ia], o_f0[ib], "default cached vs full o")
    assert_bits_equal(l_c0[ia], l_f0[ib], "default cached vs full lse")
    # the full prefill's plan is the same in both modes (its tiles are wide)
    assert_bits_equal(o_f, o_f0, "full prefill, adaptive vs default plan")
