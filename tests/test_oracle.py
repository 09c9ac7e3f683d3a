"""Pins for the CPU oracle, checked against things other than itself.

* brute force: a numpy fp64 dense masked softmax on tiny inputs;
* a library routine: torch's scaled_dot_product_attention in fp64 (causal flag when
  qo_len == kv_len, explicit boolean mask otherwise);
* closed forms: zero queries give the mean of the visible values and lse = ln(p + 1); a
  single key returns its value; a one-hot score picks one value;
* invariants: cached-tail rows equal full-prefill rows bit for bit, page placement and page
  size do not matter, keys past a row's position do not matter, replicated kv heads equal
  grouped heads;
* KV splits: partial states over disjoint key ranges combine into the unsplit result.
"""
import math

import numpy as np
import pytest
import torch

import workloads as wl


def _dense_inputs(prompt, L):
    q = prompt.q.float().numpy().astype(np.float64)
    k = prompt.k.float().numpy().astype(np.float64)[:L]
    v = prompt.v.float().numpy().astype(np.float64)[:L]
    return q, k, v


def _brute_force_rows(work, batch):
    """numpy dense attention for every request of a batch, rows in batch order."""
    outs, lses = [], []
    d = work.head_dim
    for r in batch.requests:
        if r.qo_len == 0:
            continue  # no rows
        q, k, v = _dense_inputs(work.prompts[r.prompt], r.kv_len)
        pos = np.arange(r.kv_len - r.qo_len, r.kv_len)
        o, lse = wl_dense(q[pos], k, v, pos, 1.0 / math.sqrt(d))
        outs.append(o)
        lses.append(lse)
    return np.concatenate(outs), np.concatenate(lses)


def wl_dense(q, k, v, pos, scale):
    import oracle
    return oracle.dense_attention_np(q, k, v, pos, scale)


@pytest.mark.parametrize("hq,hkv,d,page", [(4, 4, 8, 3), (8, 2, 8, 1), (12, 2, 16, 16),
                                           (6, 1, 128, 5), (32, 8, 128, 16), (8, 2, 512, 4)])
def test_oracle_matches_numpy_brute_force(oracle_lib, hq, hkv, d, page):
    specs = [(1, 1), (9, 4), (23, 23), (40, 17), (37, 1), (16, 0)]
    work = wl.random_workload(7 + hq + page, hq=hq, hkv=hkv, d=d, page_size=page,
                              kv_dtype="bf16", specs=specs)
    batch = work.batches["batch"]
    o, lse = oracle_lib.paged_prefill(**work.oracle_kwargs(batch))
    o_ref, lse_ref = _brute_force_rows(work, batch)
    assert o.shape == o_ref.shape
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def _sdpa_fp64(q, k, v, pos, g):
    # library routine: torch SDPA in fp64 on CPU; [n, Hq, d] -> [Hq, n, d]
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(k).repeat_interleave(g, dim=1).permute(1, 0, 2)
    vt = torch.from_numpy(v).repeat_interleave(g, dim=1).permute(1, 0, 2)
    L = k.shape[0]
    if len(pos) == L:
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    else:
        mask = torch.arange(L)[None, :] <= torch.from_numpy(pos)[:, None]
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
def test_oracle_matches_torch_sdpa(oracle_lib, kv_dtype):
    hq, hkv, d, page = 8, 2, 32, 16
    specs = [(50, 50), (50, 7), (33, 1)]
    work = wl.random_workload(3, hq=hq, hkv=hkv, d=d, page_size=page, kv_dtype=kv_dtype,
                              specs=specs)
    batch = work.batches["batch"]
    o, _ = oracle_lib.paged_prefill(**work.oracle_kwargs(batch))
    table = oracle_lib.e4m3_decode_table()
    row = 0
    for r in batch.requests:
        p = work.prompts[r.prompt]
        q = p.q.float().numpy().astype(np.float64)
        if kv_dtype == "bf16":
            k = p.k.float().numpy().astype(np.float64)
            v = p.v.float().numpy().astype(np.float64)
        else:
            k = p.k.view(torch.float8_e4m3fn).to(torch.float64).numpy() * work.k_scale
            v = p.v.view(torch.float8_e4m3fn).to(torch.float64).numpy() * work.v_scale
            np.testing.assert_array_equal(k, table[p.k.numpy()] * work.k_scale)
        k, v = k[:r.kv_len], v[:r.kv_len]
        pos = np.arange(r.kv_len - r.qo_len, r.kv_len)
        ref = _sdpa_fp64(q[pos], k, v, pos, hq // hkv)
        np.testing.assert_allclose(o[row:row + r.qo_len], ref, rtol=0, atol=1e-12)
        row += r.qo_len


def test_closed_form_zero_queries(oracle_lib):
    """q == 0: every score is 0, so o = mean(V[0..p]) and lse = ln(p + 1)."""
    work = wl.random_workload(11, hq=8, hkv=2, d=16, page_size=4, kv_dtype="bf16",
                              specs=[(30, 30), (21, 5)])
    batch = work.batches["batch"]
    batch.q = torch.zeros_like(batch.q)
    o, lse = oracle_lib.paged_prefill(**work.oracle_kwargs(batch))
    row = 0
    for r in batch.requests:
        v = work.prompts[r.prompt].v.float().numpy().astype(np.float64)
        for i in range(r.qo_len):
            p = r.kv_len - r.qo_len + i
            for h in range(8):
                np.testing.assert_allclose(o[row, h], v[:p + 1, h // 4].mean(axis=0), atol=1e-13)
                assert lse[row, h] == pytest.approx(math.log(p + 1), abs=1e-14)
            row += 1


def test_closed_form_single_key(oracle_lib):
    """kv_len == 1: o is that key's value exactly, lse is its score."""
    work = wl.random_workload(12, hq=4, hkv=1, d=64, page_size=16, kv_dtype="bf16",
                              specs=[(1, 1), (1, 1)])
    batch = work.batches["batch"]
    o, lse = oracle_lib.paged_prefill(**work.oracle_kwargs(batch))
    for r, req in enumerate(batch.requests):
        p = work.prompts[req.prompt]
        v0 = p.v.float().numpy().astype(np.float64)[0, 0]
        k0 = p.k.float().numpy().astype(np.float64)[0, 0]
        q = p.q.float().numpy().astype(np.float64)[0]
        for h in range(4):
            np.testing.assert_array_equal(o[r, h], v0)
            assert lse[r, h] == pytest.approx(float(q[h] @ k0) / 8.0, abs=1e-13)


def test_closed_form_one_hot(oracle_lib):
    """One key aligned with the query dominates: o = V_t up to exp(-score gap)."""
    d, L, t = 16, 12, 5
    work = wl.random_workload(13, hq=1, hkv=1, d=d, page_size=4, kv_dtype="bf16",
                              specs=[(L, 1)])
    batch = work.batches["batch"]
    e = torch.zeros(d)
    e[3] = 1.0
    batch.q = (e * 8.0).to(torch.bfloat16).reshape(1, 1, d)
    # keys: orthogonal to e except key t, which scores 8 * 30 / sqrt(16) = 60
    req = batch.requests[0]
    pages = req.pages
    kp = work.k_pool
    for j in range(L):
        row = torch.zeros(d)
        row[(j % (d - 1)) + (1 if (j % (d - 1)) >= 3 else 0)] = 1.0
        if j == t:
            row = e * 30.0
        kp[pages[j // 4], j % 4, 0] = row.to(torch.bfloat16)
    o, lse = oracle_lib.paged_prefill(**work.oracle_kwargs(batch))
    v = np.zeros((L, d))
    for j in range(L):
        v[j] = work.v_pool[pages[j // 4], j % 4, 0].float().numpy()
    np.testing.assert_allclose(o[0, 0], v[t], rtol=0, atol=1e-20)
    assert lse[0, 0] == pytest.approx(60.0 + math.log1p((L - 1) * math.exp(-60)), abs=1e-12)


def test_invariant_cached_tail_equals_full_rows(oracle_lib):
    work = wl.single_extend()
    full, cached = work.batches["full"], work.batches["cached"]
    o_f, l_f = oracle_lib.paged_prefill(**work.oracle_kwargs(full))
    o_c, l_c = oracle_lib.paged_prefill(**work.oracle_kwargs(cached))
    ia, ib = wl.matching_rows(cached, 0, full, 0)
    assert list(ib) == [64, 65, 66]
    assert cached.requests[0].qo_len < cached.requests[0].kv_len  # the hit is real
    np.testing.assert_array_equal(o_c[ia], o_f[ib])
    np.testing.assert_array_equal(l_c[ia], l_f[ib])


def test_invariant_page_size_and_placement(oracle_lib):
    """The same prompts laid out with page sizes 1, 16 and >= kv_len give the same rows."""
    specs = [(45, 45), (45, 10), (20, 3)]
    res = []
    for page in (1, 16, 64):
        work = wl.random_workload(21, hq=8, hkv=4, d=32, page_size=page, kv_dtype="bf16",
                                  specs=specs)
        res.append(oracle_lib.paged_prefill(**work.oracle_kwargs(work.batches["batch"])))
    for o, lse in res[1:]:
        np.testing.assert_array_equal(o, res[0][0])
        np.testing.assert_array_equal(lse, res[0][1])


def test_invariant_future_keys_do_not_matter(oracle_lib):
    """Changing K/V at positions > p leaves row p unchanged (causality)."""
    work = wl.random_workload(22, hq=4, hkv=2, d=16, page_size=4, kv_dtype="bf16",
                              specs=[(20, 20)])
    batch = work.batches["batch"]
    o1, l1 = oracle_lib.paged_prefill(**work.oracle_kwargs(batch))
    pages = batch.requests[0].pages
    for j in range(10, 20):
        work.k_pool[pages[j // 4], j % 4] = 7.0
        work.v_pool[pages[j // 4], j % 4] = -3.0
    o2, l2 = oracle_lib.paged_prefill(**work.oracle_kwargs(batch))
    np.testing.assert_array_equal(o1[:10], o2[:10])
    np.testing.assert_array_equal(l1[:10], l2[:10])
    assert not np.array_equal(o1[10:], o2[10:])


def test_invariant_gqa_equals_replicated_mha(oracle_lib):
    work = wl.random_workload(23, hq=8, hkv=2, d=16, page_size=4, kv_dtype="bf16",
                              specs=[(19, 19), (19, 6)])
    batch = work.batches["batch"]
    o_g, l_g = oracle_lib.paged_prefill(**work.oracle_kwargs(batch))
    kw = work.oracle_kwargs(batch)
    kw["k_pool"] = work.k_pool.repeat_interleave(4, dim=2).contiguous()
    kw["v_pool"] = work.v_pool.repeat_interleave(4, dim=2).contiguous()
    kw["num_kv_heads"] = 8
    o_m, l_m = oracle_lib.paged_prefill(**kw)
    np.testing.assert_array_equal(o_g, o_m)
    np.testing.assert_array_equal(l_g, l_m)


def test_never_reads_unused_slots(oracle_lib):
    """Pools are NaN outside the used slots; outputs stay finite."""
    work = wl.mixed_batch(tails=(1, 5))
    o, lse = oracle_lib.paged_prefill(**work.oracle_kwargs(work.batches["mixed"]),
                                      rows=[0, 1000, 3699, 3700, 3701, 3705])
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    assert torch.isnan(work.k_pool.float()).any()


@pytest.mark.parametrize("boundaries", [[0, 8, 40], [0, 16, 17, 32, 40], [0, 1, 40]])
def test_split_partials_merge_to_unsplit(oracle_lib, boundaries):
    """Partial softmax states over consecutive key ranges combine into the full row."""
    work = wl.random_workload(31, hq=6, hkv=3, d=24, page_size=4, kv_dtype="bf16",
                              specs=[(40, 40)])
    batch = work.batches["batch"]
    kw = work.oracle_kwargs(batch)
    o_full, l_full = oracle_lib.paged_prefill(**kw)
    parts = [oracle_lib.paged_prefill(**kw, key_range=(a, b))
             for a, b in zip(boundaries[:-1], boundaries[1:])]
    o_part = np.stack([p[0] for p in parts], axis=1)  # [R, S, H, d]
    l_part = np.stack([p[1] for p in parts], axis=1)  # [R, S, H]
    assert np.isneginf(l_part).any()  # early rows have empty later splits
    o, lse = oracle_lib.merge_states(o_part, l_part)
    np.testing.assert_allclose(o, o_full, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, l_full, rtol=0, atol=1e-13)


def test_merge_two_partials_hand_formula(oracle_lib):
    o1, o2 = np.array([1.0, -2.0]), np.array([3.0, 5.0])
    l1, l2 = 0.5, -1.25
    o, lse = oracle_lib.merge_states(np.stack([o1, o2])[None, :, None, :],
                                     np.array([[[l1], [l2]]]))
    w1, w2 = math.exp(l1), math.exp(l2)
    np.testing.assert_allclose(o[0, 0], (w1 * o1 + w2 * o2) / (w1 + w2), atol=1e-15)
    assert lse[0, 0] == pytest.approx(math.log(w1 + w2), abs=1e-15)


def test_e4m3_decode_all_codes(oracle_lib):
    """All 256 E4M3 codes against torch's float8_e4m3fn (OCP E4M3) and the format's fixed points."""
    table = oracle_lib.e4m3_decode_table()
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn) \
        .to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    np.testing.assert_array_equal(np.isnan(table), nan)
    np.testing.assert_array_equal(table[~nan], ref[~nan])
    assert table[0x7E] == 448.0 and table[0xFE] == -448.0       # largest finite
    assert table[0x01] == 2.0 ** -9 and table[0x08] == 2.0 ** -6  # min subnormal / normal
    assert table[0x38] == 1.0 and table[0x80] == 0.0 and math.copysign(1, table[0x80]) < 0


@pytest.mark.parametrize("page", [1, 4, 16])
def test_row_subset_equals_brute_force_rows(oracle_lib, page):
    """The rows= path (what every large GPU check uses): any selection of global query tokens,
    unsorted and with repeats, around zero-length requests, gives exactly the rows of the full
    run and matches the numpy brute force row by row."""
    specs = [(5, 0), (9, 4), (0, 0), (23, 23), (16, 0), (40, 17), (1, 1), (0, 0), (12, 3)]
    work = wl.random_workload(41 + page, hq=6, hkv=2, d=16, page_size=page, kv_dtype="bf16",
                              specs=specs)
    batch = work.batches["batch"]
    kw = work.oracle_kwargs(batch)
    o_all, l_all = oracle_lib.paged_prefill(**kw)
    o_bf, l_bf = _brute_force_rows(work, batch)
    nq = batch.num_q_tokens
    rng = np.random.default_rng(page)
    # every request's first and last row (their starts coincide with empty requests' starts)
    edges = []
    for r in range(batch.batch_size):
        a, b = int(batch.qo_indptr[r]), int(batch.qo_indptr[r + 1])
        if b > a:
            edges += [a, b - 1]
    rows = np.concatenate([rng.permutation(nq), np.array(edges[::-1]), rng.integers(0, nq, 7)])
    o, lse = oracle_lib.paged_prefill(**kw, rows=rows)
    assert o.shape == (len(rows), 6, 16)
    np.testing.assert_array_equal(o, o_all[rows])
    np.testing.assert_array_equal(lse, l_all[rows])
    np.testing.assert_allclose(o, o_bf[rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, l_bf[rows], rtol=0, atol=1e-12)
    # an empty selection and a selection outside the batch
    o0, l0 = oracle_lib.paged_prefill(**kw, rows=[])
    assert o0.shape == (0, 6, 16) and l0.shape == (0, 6)
    with pytest.raises(ValueError):
        oracle_lib.paged_prefill(**kw, rows=[nq])
