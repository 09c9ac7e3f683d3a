"""HIP graph capture and replay of the attention path (torch.cuda.graph over dpp_run).

A captured launch reads the work list uploaded beforehand (reuse_upload), static q/o/lse and
workspace buffers. Each replay, with eager work and synchronisations between replays, must
match the oracle and give the eager run's bits. The extend batch is padded with zero-length requests to several
capture sizes ("buckets"); in every bucket the real requests' rows must equal their full
prefill's rows bit for bit -- nothing about the padded batch shape reaches a row.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_helpers import Device, assert_bits_equal, assert_close_to_oracle, oracle_rows, sample_rows, say

pytestmark = pytest.mark.gpu


def _pad(batch, prompts, page_size, size):
    """The batch followed by zero-length requests (no query rows, no pages) up to ``size``."""
    pad = [wl.Request(0, 0, 0, []) for _ in range(size - batch.batch_size)]
    return wl.make_batch(list(batch.requests) + pad, prompts, page_size)


class Captured:
    def __init__(self, dev, batch):
        self.plan = dev.plan(batch)
        self.q = batch.q.cuda()
        self.kvi = torch.from_numpy(batch.kv_indices).cuda() if batch.kv_indices.size else \
            torch.zeros(1, dtype=torch.int32, device="cuda")
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((self.q.shape[0], dev.work.num_qo_heads), dtype=torch.float32, device="cuda")
        self.ws = self.plan.new_workspace("cuda")
        self.dev = dev
        # eager run first (also the reference bits), then the capture
        say(f"eager run before capture: B={batch.batch_size} rows={batch.num_q_tokens}")
        self.plan.run(self.q, dev.k_pool, dev.v_pool, self.kvi, out=self.o, lse=self.lse, workspace=self.ws)
        torch.cuda.synchronize()
        self.ref = (self.o.cpu().clone(), self.lse.cpu().clone())
        say("capture")
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.plan.run(self.q, dev.k_pool, dev.v_pool, self.kvi, out=self.o, lse=self.lse,
                          workspace=self.ws, reuse_upload=True)
        torch.cuda.synchronize()

    def replay(self):
        self.o.fill_(0)
        self.lse.fill_(0)
        torch.cuda.synchronize()
        self.graph.replay()
        torch.cuda.synchronize()
        return self.o.cpu(), self.lse.cpu()


@pytest.fixture(scope="module")
def oracle():
    import oracle as o
    o.build(force=False)
    return o


@pytest.fixture(scope="module")
def extend_work():
    return wl.extend_batch(layout="radix")


def test_graph_replays_match_eager(oracle, extend_work):
    dev = Device(extend_work)
    batch = extend_work.batches["cached"]
    cap = Captured(dev, batch)
    other = extend_work.batches["full"]
    ro, rl = oracle_rows(oracle, extend_work, batch)
    for i in range(4):
        say(f"replay {i}")
        o, l = cap.replay()
        assert_close_to_oracle(o, l, ro, rl, what=f"extend replay {i} vs oracle")
        assert_bits_equal(o, cap.ref[0], f"replay {i} o")
        assert_bits_equal(l, cap.ref[1], f"replay {i} lse")
        dev.run(other)  # eager work between replays


def test_graph_of_persistent_prefill(oracle):
    work = wl.cold_prefill(batch=4, length=1028)
    dev = Device(work)
    batch = work.batches["full"]
    cap = Captured(dev, batch)
    assert cap.plan.info.num_prefill_items > 0
    rows = sample_rows(batch, 40, seed=8)
    ro, rl = oracle_rows(oracle, work, batch, rows)
    for i in range(3):
        say(f"prefill replay {i}")
        o, l = cap.replay()
        assert_close_to_oracle(o, l, ro, rl, rows=rows, what=f"prefill replay {i} vs oracle")
        assert_bits_equal(o, cap.ref[0], f"prefill replay {i} o")
        assert_bits_equal(l, cap.ref[1], f"prefill replay {i} lse")


@pytest.mark.parametrize("bucket", [16, 24, 32, 64])
def test_graph_buckets_match_full_prefill(oracle, extend_work, bucket):
    dev = Device(extend_work)
    cached, full = extend_work.batches["cached"], extend_work.batches["full"]
    o_f, l_f = dev.run(full)
    padded = _pad(cached, extend_work.prompts, extend_work.page_size, bucket)
    cap = Captured(dev, padded)
    ro, rl = oracle_rows(oracle, extend_work, padded)
    for i in range(2):
        say(f"bucket {bucket} replay {i}")
        o, l = cap.replay()
        assert_close_to_oracle(o, l, ro, rl, what=f"bucket {bucket} replay {i} vs oracle")
        assert_bits_equal(o, cap.ref[0], f"bucket {bucket} replay {i} o")
        for r in range(cached.batch_size):
            ia, ib = wl.matching_rows(padded, r, full, r)
            assert_bits_equal(o[ia], o_f[ib], f"bucket {bucket} req {r} o")
            assert_bits_equal(l[ia], l_f[ib], f"bucket {bucket} req {r} lse")
