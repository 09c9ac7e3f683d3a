"""Helpers for GPU tests: run a workload batch through libdpp, compare with the oracle."""
import sys

import numpy as np
import torch

O_TOL = 1e-2     # max |o_gpu - o_oracle| on bf16 outputs
LSE_TOL = 2e-3   # max |lse_gpu - lse_oracle| on fp32 lse


def say(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a failing run says where it was."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


class Device:
    """Device copies of a workload's pools (made once) and batch runner."""

    def __init__(self, work):
        import deterministic_paged_prefill_amd as dpp
        self.dpp = dpp
        self.work = work
        self.k_pool = work.k_pool.cuda()
        self.v_pool = work.v_pool.cuda()

    def plan(self, batch, cap=None):
        w = self.work
        kw = dict(kv_dtype=w.kv_dtype, k_scale=w.k_scale, v_scale=w.v_scale)
        if cap is not None:
            kw["workspace_cap"] = cap
        return self.dpp.plan(w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size,
                             batch.qo_indptr, batch.kv_indptr, batch.kv_last_page_len, **kw)

    def run(self, batch, cap=None, plan=None, q=None):
        say(f"run {self.work.name}: B={batch.batch_size} rows={batch.num_q_tokens} "
            f"cap={cap} block_n={plan.info.block_n if plan else 'default'}")
        p = plan or self.plan(batch, cap)
        qd = (batch.q if q is None else q).cuda()
        kvi = torch.from_numpy(batch.kv_indices).cuda()
        o, lse = p.run(qd, self.k_pool, self.v_pool, kvi)
        torch.cuda.synchronize()
        return o.cpu(), lse.cpu()


def oracle_rows(oracle, work, batch, rows=None):
    return oracle.paged_prefill(**work.oracle_kwargs(batch), rows=rows)


def assert_close_to_oracle(o_gpu, lse_gpu, o_ref, lse_ref, rows=None, what=""):
    og = o_gpu.float().numpy().astype(np.float64)
    lg = lse_gpu.numpy().astype(np.float64)
    if rows is not None:
        og, lg = og[rows], lg[rows]
    assert np.isfinite(og).all(), f"{what}: non-finite outputs"
    assert np.isfinite(lg).all(), f"{what}: non-finite lse"
    eo = np.abs(og - o_ref).max() if og.size else 0.0
    el = np.abs(lg - lse_ref).max() if lg.size else 0.0
    ulps, n_far = bf16_ulps(og, o_ref)
    say(f"{what}: max|o-oracle| = {eo:.3e} ({ulps:.2f} bf16 ulps of the oracle rounded to bf16, "
        f"{n_far} values beyond 2 ulps), max|lse-oracle| = {el:.3e}")
    assert eo <= O_TOL, f"{what}: max |o - oracle| = {eo}"
    assert el <= LSE_TOL, f"{what}: max |lse - oracle| = {el}"


def bf16_ulps(o_gpu: np.ndarray, o_ref: np.ndarray):
    """Error of bf16 outputs against the oracle rounded to bf16 (round to nearest even), in
    units of that value's bf16 ulp, over values of magnitude >= 2^-6 (smaller ones are judged
    by the absolute bound). Returns (max ulps, number of values beyond 2 ulps)."""
    if o_gpu.size == 0:
        return 0.0, 0
    rne = torch.from_numpy(np.ascontiguousarray(o_ref, dtype=np.float32)).to(torch.bfloat16).double().numpy()
    big = np.abs(rne) >= 2.0 ** -6
    if not big.any():
        return 0.0, 0
    ulp = np.exp2(np.floor(np.log2(np.abs(rne[big]))) - 7)
    u = np.abs(o_gpu[big] - rne[big]) / ulp
    return float(u.max()), int((u > 2).sum())


def assert_bits_equal(a: torch.Tensor, b: torch.Tensor, what=""):
    """Bit-for-bit equality (also catches -0 vs +0 and NaN payloads)."""
    ia = a.contiguous().view(torch.int16 if a.element_size() == 2 else torch.int32)
    ib = b.contiguous().view(torch.int16 if b.element_size() == 2 else torch.int32)
    if not torch.equal(ia, ib):
        diff = (a.float() - b.float()).abs()
        diff = torch.nan_to_num(diff, nan=float("inf"))
        n = int((ia != ib).sum())
        raise AssertionError(f"{what}: {n} elements differ, max|diff| = {float(diff.max())}")


def sample_rows(batch, per_request: int, seed: int) -> np.ndarray:
    """Global q-token rows: each request's first/last rows, tile edges and a random sample."""
    rng = np.random.default_rng(seed)
    rows = []
    for r in range(batch.batch_size):
        a, b = int(batch.qo_indptr[r]), int(batch.qo_indptr[r + 1])
        if b == a:
            continue
        n = b - a
        pick = {0, n - 1, min(n - 1, 31), min(n - 1, 32), n // 2}
        pick |= set(int(x) for x in rng.integers(0, n, size=min(per_request, n)))
        rows.extend(a + i for i in sorted(pick))
    return np.array(sorted(set(rows)), dtype=np.int64)
