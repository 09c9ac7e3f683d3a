"""The allocation-free entry point, dpp_run_static, against dpp_run through the C ABI.

dpp_run_static runs the same kernels over a scratch array the library owns instead of a
caller workspace. Two calls in a row on one device -- the first with split partials and merges
(long-KV decode rows), the second smaller (the short-extend batch), whose run finds the first
one's partials still in the scratch -- must each give dpp_run's bits; so must a plan that needs
several passes to stay under the scratch size. A reused upload is accepted only while the
scratch still holds that plan's work list.
"""
import ctypes

import numpy as np
import pytest
import torch

import workloads as wl
from gpu_helpers import assert_bits_equal, say

pytestmark = pytest.mark.gpu


class Buffers:
    """Device inputs and outputs of one batch (allocated here, by the caller)."""

    def __init__(self, work, batch, cap):
        import deterministic_paged_prefill_amd as dpp
        self.dpp = dpp
        self.plan = dpp.plan(work.num_qo_heads, work.num_kv_heads, work.head_dim, work.page_size,
                             batch.qo_indptr, batch.kv_indptr, batch.kv_last_page_len,
                             kv_dtype=work.kv_dtype, k_scale=work.k_scale, v_scale=work.v_scale,
                             workspace_cap=cap)
        self.k = work.k_pool.cuda()
        self.v = work.v_pool.cuda()
        self.q = batch.q.cuda()
        self.kvi = torch.from_numpy(batch.kv_indices).cuda()
        self.rows = self.q.shape[0]
        self.hq = work.num_qo_heads

    def outputs(self):
        o = torch.full_like(self.q, float("nan"))
        lse = torch.full((self.rows, self.hq), float("nan"), dtype=torch.float32, device="cuda")
        return o, lse

    def args(self, o, lse):
        return (self.plan._h, self.q.data_ptr(), self.rows, self.k.data_ptr(), self.v.data_ptr(),
                self.k.shape[0], self.kvi.data_ptr(), self.kvi.numel(), o.data_ptr(), lse.data_ptr())

    def run(self):
        """dpp_run with a caller workspace: the reference bits."""
        o, lse = self.outputs()
        ws = self.plan.new_workspace()
        st = self.dpp.library().dpp_run(*self.args(o, lse), ws.data_ptr(), ws.numel(), 0,
                                        torch.cuda.current_stream().cuda_stream)
        self.dpp._check(st)
        torch.cuda.synchronize()
        return o.cpu(), lse.cpu()

    def run_static(self, flags=0):
        o, lse = self.outputs()
        st = self.dpp.library().dpp_run_static(*self.args(o, lse), flags,
                                               torch.cuda.current_stream().cuda_stream)
        if st != 0:
            return st, None, None
        torch.cuda.synchronize()
        return st, o.cpu(), lse.cpu()


def _same(got, ref, what):
    st, o, lse = got
    assert st == 0, what
    assert_bits_equal(o, ref[0], f"{what} o")
    assert_bits_equal(lse, ref[1], f"{what} lse")


def test_static_entry_matches_dpp_run():
    import deterministic_paged_prefill_amd as dpp
    cap = dpp.STATIC_SCRATCH_BYTES
    dec_work = wl.decode_batch()
    dec = Buffers(dec_work, dec_work.batches["decode"], cap)
    assert dec.plan.info.num_merge_items > 0, "the first call leaves partials in the scratch"
    ext_work = wl.extend_batch(layout="radix")
    ext = Buffers(ext_work, ext_work.batches["cached"], cap)
    assert ext.plan.workspace_bytes < dec.plan.workspace_bytes and ext.rows < 64
    say("reference runs through dpp_run")
    ref_dec, ref_ext = dec.run(), ext.run()

    say("dpp_run_static: decode batch (merges), then the smaller extend batch")
    _same(dec.run_static(), ref_dec, "static decode")
    _same(ext.run_static(), ref_ext, "static extend after decode")
    # the scratch now holds the extend plan's work list: reusing it is fine, the decode's not
    _same(ext.run_static(dpp.RUN_REUSE_UPLOAD), ref_ext, "static extend, reused upload")
    st, _, _ = dec.run_static(dpp.RUN_REUSE_UPLOAD)
    assert st == dpp.DPP_ERR_INVALID
    _same(dec.run_static(), ref_dec, "static decode again")

    say("a plan cut into passes to fit the scratch: fp8 8k prefill")
    fp8 = wl.long_fp8(lengths=(8192,), extend=1024)
    big = Buffers(fp8, fp8.batches["prefill_8192"], cap)
    assert big.plan.info.num_passes > 1 and big.plan.workspace_bytes <= cap
    _same(big.run_static(), big.run(), "static fp8 8k prefill in passes")
    # and the small extend once more, after the largest run
    _same(ext.run_static(), ref_ext, "static extend after the fp8 prefill")
