"""GPU checks of the C ABI's run-time contract: a reused upload must name its workspace, a
short page list is refused before any launch, and a run on another stream without a
workspace gives the same bits as one on the current stream."""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_helpers import Device, assert_bits_equal, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def work():
    return wl.single_extend()


def test_reuse_upload_needs_the_same_workspace(work):
    import deterministic_paged_prefill_amd as dpp
    dev = Device(work)
    b = work.batches["cached"]
    p = dev.plan(b)
    q = b.q.cuda()
    kvi = torch.from_numpy(b.kv_indices).cuda()
    ws1, ws2 = p.new_workspace(), p.new_workspace()
    say("upload to workspace 1, reuse with workspace 1, then with workspace 2")
    p.upload(ws1)
    o1, l1 = p.run(q, dev.k_pool, dev.v_pool, kvi, workspace=ws1, reuse_upload=True)
    torch.cuda.synchronize()
    with pytest.raises(dpp.DppValueError, match="another workspace"):
        p.run(q, dev.k_pool, dev.v_pool, kvi, workspace=ws2, reuse_upload=True)
    # a plain run uploads to ws2; reusing ws2 is then fine and ws1 no longer is
    o2, l2 = p.run(q, dev.k_pool, dev.v_pool, kvi, workspace=ws2)
    o3, l3 = p.run(q, dev.k_pool, dev.v_pool, kvi, workspace=ws2, reuse_upload=True)
    torch.cuda.synchronize()
    with pytest.raises(dpp.DppValueError, match="another workspace"):
        p.run(q, dev.k_pool, dev.v_pool, kvi, workspace=ws1, reuse_upload=True)
    for o, l, what in ((o2, l2, "fresh upload"), (o3, l3, "reused upload")):
        assert_bits_equal(o.cpu(), o1.cpu(), what)
        assert_bits_equal(l.cpu(), l1.cpu(), what)


def test_short_page_list_is_refused(work):
    import deterministic_paged_prefill_amd as dpp
    dev = Device(work)
    b = work.batches["full"]
    p = dev.plan(b)
    kvi = torch.from_numpy(b.kv_indices[:-1].copy()).cuda()
    with pytest.raises(dpp.DppValueError, match="kv_indices holds"):
        p.run(b.q.cuda(), dev.k_pool, dev.v_pool, kvi)
    with pytest.raises(dpp.DppValueError, match="outside"):
        p.check_page_table(b.kv_indices, num_pages=int(b.kv_indices.max()))


def test_side_stream_without_workspace(work):
    dev = Device(work)
    b = work.batches["full"]
    p = dev.plan(b)
    q, kvi = b.q.cuda(), torch.from_numpy(b.kv_indices).cuda()
    o_ref, l_ref = p.run(q, dev.k_pool, dev.v_pool, kvi)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    say("run on a side stream, workspace allocated by the binding")
    outs = []
    for _ in range(4):
        o, l = p.run(q, dev.k_pool, dev.v_pool, kvi, stream=side)
        outs.append((o, l))
        junk = torch.empty(p.workspace_bytes, dtype=torch.uint8, device="cuda").fill_(0xFF)  # reuse bait
        del junk
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for i, (o, l) in enumerate(outs):
        assert_bits_equal(o.cpu(), o_ref.cpu(), f"side-stream run {i} o")
        assert_bits_equal(l.cpu(), l_ref.cpu(), f"side-stream run {i} lse")


def test_stream_reference_runs_every_mode():
    """The read-only streaming reference (a measurement tool) runs by keys (1, 2 and 4
    workgroups per unit) and by head_dim halves, at every load depth, over a narrow extend plan
    with the head_dim-split launch's grid and a wide prefill plan, and leaves the workspace
    beyond the work list untouched."""
    import deterministic_paged_prefill_amd as dpp
    ext = wl.extend_batch(layout="distinct")
    long = wl.random_workload(97, hq=32, hkv=8, d=128, page_size=16, kv_dtype="bf16", specs=[(9000, 900)])
    lib = dpp.library()
    for work, name in ((ext, "cached"), (ext, "full"), (long, "batch")):
        dev = Device(work)
        b = work.batches[name]
        p = dev.plan(b)
        assert name != "batch" or p.info.workspace_bytes > p.info.header_bytes, "a plan with partials"
        kvi = torch.from_numpy(b.kv_indices).cuda()
        ws = p.new_workspace()
        ws.fill_(0x5A)
        p.upload(ws)
        head = p.info.header_bytes
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream().cuda_stream
        for split, flags in ((1, 0), (2, 0), (4, 0), (2, dpp.STREAM_HEAD_SPLIT)):
            for depth in (4, 8, 16, 32):
                say(f"stream reference {name}: split {split} flags {flags} depth {depth}")
                st = lib.dpp_stream_kv(p._h, dev.k_pool.data_ptr(), dev.v_pool.data_ptr(), dev.k_pool.shape[0],
                                       kvi.data_ptr(), kvi.numel(), ws.data_ptr(), ws.numel(), split, depth,
                                       dpp.RUN_REUSE_UPLOAD | flags, stream)
                assert st == 0, lib.dpp_last_error()
        torch.cuda.synchronize()
        rest = ws[head:].cpu().numpy()
        assert (rest == 0x5A).all(), "the reference writes nothing past the work list"
