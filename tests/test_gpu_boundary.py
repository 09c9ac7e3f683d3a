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
