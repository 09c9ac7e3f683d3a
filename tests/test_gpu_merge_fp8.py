"""GPU: the standalone merge-states entry point against the oracle's merge, and an exhaustive
check of the in-kernel E4M3 decode (every code, through single-key attention rows)."""
import math

import numpy as np
import pytest
import torch

import workloads as wl
from gpu_helpers import Device, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def oracle():
    import oracle as o
    o.build(force=False)
    return o


@pytest.mark.parametrize("R,S,H,D", [(7, 1, 3, 128), (33, 2, 4, 128), (5, 8, 6, 256), (3, 3, 2, 12)])
def test_merge_states_against_oracle(oracle, R, S, H, D):
    import deterministic_paged_prefill_amd as dpp
    g = torch.Generator().manual_seed(R * 1000 + S)
    o_part = torch.randn(R, S, H, D, generator=g)
    lse = torch.randn(R, S, H, generator=g) * 4
    if S > 1:
        lse[0, 1:, 0] = -math.inf     # empty partials carry no weight
        o_part[0, 1:, 0] = 0.0
        lse[1 % R, :, 1 % H] = -math.inf  # an all-empty row
        o_part[1 % R, :, 1 % H] = 0.0
    say(f"merge_states R={R} S={S} H={H} D={D}")
    o_gpu, lse_gpu = dpp.merge_states(o_part.cuda(), lse.cuda())
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.merge_states(o_part.double().numpy(), lse.double().numpy())
    og = o_gpu.cpu().float().numpy()
    lg = lse_gpu.cpu().numpy()
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isneginf(lg), ~fin)
    # bf16 output: round-to-nearest costs at most 2^-8 |o| (half an ulp), fp32 math ~1e-6
    bound = 2.0 ** -8 * np.abs(o_ref) + 1e-5
    assert (np.abs(og - o_ref) <= bound).all(), float((np.abs(og - o_ref) - bound).max())
    assert np.abs(lg[fin] - lse_ref[fin]).max() <= 2e-5 * max(1.0, np.abs(lse_ref[fin]).max())


@pytest.mark.parametrize("v_scale", [None, 2.0 ** -60, 3.0])
def test_e4m3_decode_every_code(oracle, v_scale):
    """Single-key rows return their value row exactly: o = bf16(decode(code) * v_scale).

    Two 128-wide value rows hold all 256 codes; keys hold small finite codes. Scales: the
    workload's (a power of two: the kernels decode with the scaled conversion instruction), a
    power of two near the end of that instruction's range, and 3 (the multiply path)."""
    hq, hkv, d, page = 1, 1, 128, 16
    work = wl.random_workload(77, hq=hq, hkv=hkv, d=d, page_size=page, kv_dtype="fp8_e4m3",
                              specs=[(1, 1), (1, 1)])
    if v_scale is not None:
        work.v_scale = v_scale
    b = work.batches["batch"]
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).reshape(2, 128)
    for r, req in enumerate(b.requests):
        pg = req.pages[0]
        work.v_pool[pg, 0, 0] = codes[r]
        work.k_pool[pg, 0, 0] = torch.full((128,), 0x30, dtype=torch.uint8)  # 0.5 each
    dev = Device(work)
    o, lse = dev.run(b)
    table = oracle.e4m3_decode_table() * work.v_scale
    expect = torch.from_numpy(table.reshape(2, 128)).to(torch.bfloat16)
    got = o[:, 0, :]
    nan_e = torch.isnan(expect)
    assert torch.equal(torch.isnan(got), nan_e)
    # values compared as numbers: the +-0 codes both come out as +0 (the MFMA sums onto +0)
    assert torch.equal(got[~nan_e].float(), expect[~nan_e].float())
