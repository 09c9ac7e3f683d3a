"""GPU parity of ragged (contiguous, non-paged) KV: page_size 0, K/V as [tokens, Hkv, D] with
kv_indptr counting tokens.

Each batch runs twice, over its paged layout (shuffled, NaN-poisoned pages) and over a ragged
copy of the same keys (requests' keys back to back in request order); the two outputs must be
identical bit for bit, and both within tolerance of the fp64 oracle. The cases cover the
narrow launch (head_dim split), the persistent wide launch, rows spanning several 4096-token
splits (partials + merge), fp8 E4M3 and head_dim 256.
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


def ragged_kv(work, batch):
    """K, V [sum kv_len, Hkv, D] (storage dtype) and the token kv_indptr of a batch."""
    ks, vs, ind = [], [], [0]
    for r in batch.requests:
        p = work.prompts[r.prompt]
        ks.append(p.k[:r.kv_len])
        vs.append(p.v[:r.kv_len])
        ind.append(ind[-1] + r.kv_len)
    k = torch.cat(ks) if ks else work.prompts[0].k[:0]
    v = torch.cat(vs) if vs else work.prompts[0].v[:0]
    if k.shape[0] == 0:  # at least one row so the device tensors are real
        k, v = work.prompts[0].k[:1], work.prompts[0].v[:1]
    return k.contiguous(), v.contiguous(), np.asarray(ind, np.int32)


def run_ragged(work, batch, cap=None):
    import deterministic_paged_prefill_amd as dpp
    k, v, kvp = ragged_kv(work, batch)
    kw = dict(kv_dtype=work.kv_dtype, k_scale=work.k_scale, v_scale=work.v_scale)
    if cap is not None:
        kw["workspace_cap"] = cap
    say(f"ragged {work.name}: B={batch.batch_size} rows={batch.num_q_tokens} tokens={int(kvp[-1])}")
    p = dpp.plan(work.num_qo_heads, work.num_kv_heads, work.head_dim, 0, batch.qo_indptr, kvp, **kw)
    kd, vd = k.cuda(), v.cuda()
    o, lse = p.run(batch.q.cuda(), kd, vd)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


CASES = {
    "extend_batch": lambda: (wl.extend_batch(layout="distinct"), "cached"),
    "cold_prefill_4x1028": lambda: (wl.cold_prefill(batch=4), "full"),
    "mixed_3700": lambda: (wl.mixed_batch(), "mixed"),
    "split_rows": lambda: (wl.random_workload(9, hq=32, hkv=8, d=128, page_size=16, kv_dtype="bf16",
                                              specs=[(4100, 12), (4096, 3), (4097, 1), (8200, 2), (70, 70)]), "batch"),
    "fp8_d256": lambda: (wl.random_workload(7, hq=24, hkv=4, d=256, page_size=16, kv_dtype="fp8_e4m3",
                                            specs=[(160, 160), (161, 5), (70, 1), (4100, 30)]), "batch"),
    "bf16_d256": lambda: (wl.random_workload(6, hq=24, hkv=4, d=256, page_size=16, kv_dtype="bf16",
                                             specs=[(160, 160), (161, 5), (70, 1)]), "batch"),
    "bf16_d64": lambda: (wl.random_workload(11, hq=16, hkv=4, d=64, page_size=16, kv_dtype="bf16",
                                            specs=[(300, 300), (301, 3), (70, 1), (4100, 12)]), "batch"),
    "bf16_d512": lambda: (wl.random_workload(18, hq=16, hkv=4, d=512, page_size=16, kv_dtype="bf16",
                                             specs=[(300, 300), (301, 3), (70, 1), (4100, 12)]), "batch"),
    "fp8_d512": lambda: (wl.random_workload(19, hq=16, hkv=4, d=512, page_size=16, kv_dtype="fp8_e4m3",
                                            specs=[(200, 200), (201, 2), (4100, 8)]), "batch"),
}


@pytest.mark.parametrize("case", list(CASES))
def test_ragged_equals_paged_and_oracle(oracle, case):
    work, name = CASES[case]()
    batch = work.batches[name]
    o_p, l_p = Device(work).run(batch)
    o_r, l_r = run_ragged(work, batch)
    assert_bits_equal(o_r, o_p, f"{case}: ragged vs paged o")
    assert_bits_equal(l_r, l_p, f"{case}: ragged vs paged lse")
    rows = None
    if batch.num_q_tokens > 512:
        rng = np.random.default_rng(11)
        rows = np.unique(np.concatenate([[0, batch.num_q_tokens - 1],
                                         rng.integers(0, batch.num_q_tokens, 96)])).astype(np.int64)
    ro, rl = oracle_rows(oracle, work, batch, rows)
    assert_close_to_oracle(o_r, l_r, ro, rl, rows=rows, what=f"{case} ragged")


def test_ragged_cached_tail_matches_full_prefill():
    work = wl.extend_batch(layout="radix")
    cached, full = work.batches["cached"], work.batches["full"]
    o_c, l_c = run_ragged(work, cached)
    o_f, l_f = run_ragged(work, full)
    for r in range(cached.batch_size):
        ia, ib = wl.matching_rows(cached, r, full, r)
        assert_bits_equal(o_c[ia], o_f[ib], f"ragged cached vs full o {r}")
        assert_bits_equal(l_c[ia], l_f[ib], f"ragged cached vs full lse {r}")
