"""CPU tests of the host planner and the C ABI's argument checks (no GPU, no kernel launch).

Like the pages' host-plan test suite (sglang PR #46351, "Tests"), these check the work list
itself: every (row, head, key <= p) is covered exactly once per split, each row's split count
is a function of its position only, the workspace has a closed form and stays under the cap,
and malformed input is rejected with a status before anything is launched.
"""
import ctypes
import json
import os
import re
import subprocess

import numpy as np
import pytest

import workloads as wl
from dpp_header import parse

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def dpp():
    import deterministic_paged_prefill_amd as dpp
    if not os.path.exists(dpp.LIB_PATH):
        from deterministic_paged_prefill_amd import build
        build.build()
    dpp.library()
    return dpp


def _align(x, a=256):
    return (x + a - 1) // a * a


def test_library_exports_every_declared_symbol(dpp):
    header = open(os.path.join(ROOT, "include", "dpp.h")).read()
    declared = set(re.findall(r"\b(dpp_[a-z_]+)\s*\(", header))
    out = subprocess.run(["nm", "-D", "--defined-only", dpp.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert declared, "no declarations parsed"
    assert declared <= exported, declared - exported
    assert declared == set(dpp.EXPORTS)
    assert dpp.library().dpp_abi_version() == 3


def _plan(dpp, batch, hq=32, hkv=8, d=128, page=16, cap=0, **kw):
    return dpp.plan(hq, hkv, d, page, batch.qo_indptr, batch.kv_indptr,
                    batch.kv_last_page_len, workspace_cap=cap, **kw)


def _specs_batch(specs, page=16, g=4):
    """A batch from (kv_len, qo_len) pairs without drawing data (page ids are arbitrary)."""
    qo, kvp, last = [0], [0], []
    for kv, qlen in specs:
        npg = -(-kv // page)
        qo.append(qo[-1] + qlen)
        kvp.append(kvp[-1] + npg)
        last.append(kv - (npg - 1) * page if npg else 0)

    class B:
        pass
    b = B()
    b.qo_indptr = np.array(qo, np.int32)
    b.kv_indptr = np.array(kvp, np.int32)
    b.kv_last_page_len = np.array(last, np.int32)
    return b


def _coverage(parsed, g, bm):
    """Map (request, packed row, split) -> KV tile range visited; check exactly-once."""
    seen = {}
    for it in parsed.items:
        r, rs, s, S, kb, ke, slot = (int(x) for x in it[:7])
        q_start, qo_len, page_start, kv_len = parsed.requests[r]
        # the item carries a copy of its request's descriptor
        assert [int(x) for x in it[8:12]] == [int(q_start), int(qo_len), int(page_start), int(kv_len)]
        rows = min(bm, qo_len * g - rs)
        for lr in range(rows):
            key = (r, rs + lr, s)
            assert key not in seen, f"row {key} covered twice"
            seen[key] = (kb, ke)
    return seen


@pytest.mark.parametrize("specs", [
    [(67, 67)], [(67, 3)], [(1028, 1028)] * 3, [(1025, 1), (1028, 4), (1026, 2)],
    [(3700, 3700), (3701, 1), (3702, 2), (3704, 4), (3706, 6), (3737, 37), (3764, 64), (4000, 300)],
    [(9000, 9000)], [(8192, 100), (5000, 0), (4097, 4097)], [(1, 1), (0, 0), (2, 1)]])
def test_every_key_covered_once_per_split(dpp, specs):
    g = 4
    b = _specs_batch(specs)
    p = _plan(dpp, b)
    bm, bn = p.info.block_m, p.info.block_n
    assert (bm, bn) == dpp.tile_shape(128)
    tps = 4096 // bn
    parsed = parse(p.header())
    cov = _coverage(parsed, g, bm)
    expected = set()
    for r, (kv, qlen) in enumerate(specs):
        for R in range(qlen * g):
            pos = kv - qlen + R // g
            n_splits = pos // 4096 + 1
            for s in range(n_splits):
                expected.add((r, R, s))
                kb, ke = cov[(r, R, s)]
                # the item visits every tile holding keys s*4096 .. min(p, split end)
                assert kb == s * tps
                assert ke * bn > min(pos, (s + 1) * 4096 - 1)
                assert ke <= (s + 1) * tps
    # rows may ride along in items of splits they do not need (tile-mates' splits); the
    # kernel skips their writes. Every needed (row, split) is present:
    assert expected <= set(cov)


def test_row_split_count_depends_only_on_position(dpp):
    """A request's items (tile geometry, KV ranges) are identical alone and in any batch."""
    alone = _specs_batch([(5000, 300)])
    mixed = _specs_batch([(100, 100), (5000, 300), (9000, 1), (4096, 4096)])
    a = parse(_plan(dpp, alone).header())
    m = parse(_plan(dpp, mixed).header())
    key = lambda it: (int(it[1]), int(it[2]), int(it[3]), int(it[4]), int(it[5]))
    ia = sorted(key(it) for it in a.items if it[0] == 0)
    im = sorted(key(it) for it in m.items if it[0] == 1)
    assert ia == im


def test_workspace_closed_form_single_pass(dpp):
    specs = [(9000, 9000), (5000, 40), (100, 100)]
    b = _specs_batch(specs)
    p = _plan(dpp, b)
    bm = p.info.block_m
    parsed = parse(p.header())
    slots = 0
    ntile = 0
    for kv, qlen in specs:
        for rs in range(0, qlen * 4, bm):
            rows = min(bm, qlen * 4 - rs)
            pmax = kv - qlen + (rs + rows - 1) // 4
            S = pmax // 4096 + 1
            ntile += 1
            if S > 1:
                slots += S * 8 * (-(-rows // 16) * 16)  # the tile's rows, rounded up to 16
    # every tile is wide: each (item, kv head) also has a unit record of the persistent launch
    assert len(parsed.units) == 8 * len(parsed.items)
    words = 16 + 4 * len(specs) + 16 * len(parsed.items) + 4 * len(parsed.merges) + 16 * len(parsed.units)
    hdr = _align(words * 4)
    assert p.info.header_bytes == hdr
    assert p.info.max_partial_slots == slots
    assert p.workspace_bytes == hdr + _align(slots * 128 * 4) + _align(slots * 4)
    assert p.info.num_passes == 1


@pytest.mark.parametrize("cap_mib", [8, 16, 64])
def test_cap_bounds_workspace_and_adds_passes(dpp, cap_mib):
    b = _specs_batch([(32768, 32768)])
    cap = cap_mib << 20
    unbounded = dpp.plan(24, 4, 256, 16, b.qo_indptr, b.kv_indptr, b.kv_last_page_len,
                         kv_dtype="fp8_e4m3", k_scale=1 / 32, v_scale=1 / 32, workspace_cap=0)
    p = dpp.plan(24, 4, 256, 16, b.qo_indptr, b.kv_indptr, b.kv_last_page_len,
                 kv_dtype="fp8_e4m3", k_scale=1 / 32, v_scale=1 / 32, workspace_cap=cap)
    assert p.workspace_bytes <= cap
    assert p.info.num_passes > 1
    assert unbounded.info.num_passes == 1
    assert unbounded.workspace_bytes > 3 << 30  # ~3.5 GB of partials without a cap
    # same work, only cut into passes
    key = lambda it: tuple(int(x) for x in it[:6])
    assert sorted(map(key, parse(p.header()).items)) == sorted(map(key, parse(unbounded.header()).items))


def _xcd_group(hkv, xcds=8):
    """Neighbouring XCDs that share one run of the plain launch order: as many as share one kv
    head's units (8 / kv heads rounded down to a power of two, at least 1)."""
    xg = 1
    while xg * 2 <= xcds and xg * 2 * hkv <= xcds:
        xg *= 2
    return xg


def _group_of(b, hkv, xcds=8):
    return (b % xcds) // _xcd_group(hkv, xcds)


def _check_chains(parsed, items, units, hkv, blocks=256, xcds=8):
    """The unit records of one persistent launch over `items` (its pass's items, launch order)."""
    n = len(items)
    n_units = n * hkv
    assert len(units) == n_units
    nb = min(n_units, blocks)
    index = {tuple(int(x) for x in it[:3]): i for i, it in enumerate(items)}
    cost = lambda rec: int(rec[5] - rec[4]) + 2
    seen = np.zeros(n_units, dtype=bool)
    covered = set()
    load = {}
    group_units = {}
    for b in range(nb):
        assert units[b][13] == b, "workgroup b starts at record b"
        k, costs = b, []
        while k >= 0:
            assert not seen[k], "a record reached twice"
            seen[k] = True
            rec = units[k]
            assert rec[13] == b
            i = index[tuple(int(x) for x in rec[:3])]
            assert (rec[:7] == items[i][:7]).all() and (rec[8:12] == items[i][8:12]).all()
            h = int(rec[12])
            group_units.setdefault(_group_of(b, hkv, xcds), []).append(h * n + i)  # plain launch order
            covered.add((i, h))
            c = cost(rec)
            costs.append(c)
            load[b] = load.get(b, 0) + c
            k = int(rec[7])
        # a chain is its units longest first, rotated: at most one cyclic ascent
        ascents = sum(costs[j] < costs[(j + 1) % len(costs)] for j in range(len(costs)))
        assert ascents <= 1, costs
    assert seen.all(), "every record is on a chain"
    assert covered == {(i, h) for i in range(n) for h in range(hkv)}
    biggest = max(cost(u) for u in units)
    groups = xcds // _xcd_group(hkv, xcds)
    members = {g: [b for b in range(nb) if _group_of(b, hkv, xcds) == g] for g in range(groups)}
    for g in range(groups):
        loads = [load[b] for b in members[g]]
        if loads:
            assert max(loads) - min(loads) <= biggest
    # group g holds a contiguous run of the plain order, the runs in group order, and its share
    # of the cost in proportion to its workgroups (within the largest units, unless its run is
    # pinned at one unit per workgroup)
    total = sum(load.values())
    start = 0
    for g in range(groups):
        run = sorted(group_units.get(g, []))
        assert run == list(range(start, start + len(run))), "contiguous runs in group order"
        start += len(run)
        bg = len(members[g])
        assert len(run) >= bg, "a unit for every workgroup"
        share = total * bg / nb
        got = sum(load[b] for b in members[g])
        assert abs(got - share) <= 2 * biggest or len(run) == bg, (g, got, share)
    assert start == n_units


def _check_table(table, items, hkv, xcds=8):
    """The block table of a wide launch that is not persistent over `items`."""
    n = len(items)
    n_units = n * hkv
    t = np.asarray(table)
    assert len(t) % xcds == 0 and len(t) >= n_units
    used = t[t >= 0]
    assert sorted(used.tolist()) == list(range(n_units)), "every unit once"
    cost = np.array([int(items[u % n][5] - items[u % n][4]) + 2 for u in range(n_units)])
    xg = _xcd_group(hkv, xcds)
    groups = xcds // xg
    start = 0
    per_xcd = np.zeros(xcds)
    for g in range(groups):
        blocks = [b for b in range(len(t)) if _group_of(b, hkv, xcds) == g and t[b] >= 0]
        run = sorted(int(t[b]) for b in blocks)
        assert run == list(range(start, start + len(run))), "contiguous runs in group order"
        start += len(run)
        for x in range(g * xg, (g + 1) * xg):
            mine = [int(t[b]) for b in range(x, len(t), xcds)]
            live = [w for w in mine if w >= 0]
            assert mine[:len(live)] == live, "an XCD's blocks without a unit come last"
            assert all(cost[a] >= cost[b] for a, b in zip(live, live[1:])), "longest first"
            per_xcd[x] = cost[live].sum() if live else 0
    assert start == n_units
    if n_units >= 8 * xcds:
        biggest = cost.max()
        assert per_xcd.max() - per_xcd.mean() <= 2 * biggest + 0.05 * per_xcd.mean(), per_xcd


@pytest.mark.parametrize("specs", [[(1028, 1028)] * 16, [(67, 67)], [(1028, 1028)] * 2,
                                   [(3700, 3700), (3701, 1), (4000, 300)], [(9000, 9000)],
                                   [(1024 + t, t) for t in (1, 2, 3, 4)] * 4 + [(500, 500)]])
def test_persistent_chains_cover_every_unit_once(dpp, specs):
    parsed = parse(_plan(dpp, _specs_batch(specs)).header())
    assert (parsed.units[:, 14] == 0).all()
    _check_chains(parsed, parsed.items, parsed.units, 8)


def test_persistent_chains_balance_xcds_at_four_kv_heads(dpp):
    # 4 kv heads on 8 XCDs: equal-count runs of the plain order would give one XCD of each pair
    # the long tiles of its head and the other the short ones (1.42 : 0.58 at 8,192 tokens)
    for specs in ([(8192, 8192)], [(32768, 32768)], [(3000, 3000), (200, 200)] * 3):
        p = _plan(dpp, _specs_batch(specs, g=6), hq=24, hkv=4, d=256, cap=256 << 20)
        parsed = parse(p.header())
        for ps in range(p.info.num_passes):
            units = parsed.units[parsed.units[:, 14] == ps]
            items = parsed.items[parsed.items[:, 7] == ps]
            _check_chains(parsed, items, units, 4)
            cost = (units[:, 5] - units[:, 4]) + 2
            per_xcd = np.bincount(units[:, 13] % 8, weights=cost, minlength=8)
            assert per_xcd.max() <= 1.05 * per_xcd.mean(), per_xcd


@pytest.mark.parametrize("kind", ["fp8_d256", "fp8_d128", "bf16_d512", "bf16_d128_page1"])
def test_block_tables_of_wide_launches(dpp, kind):
    # wide launches that are not persistent (fp8, head_dim 512, page size 1 where two page
    # tables do not fit) run a block table: every unit once, contiguous cost-balanced runs per
    # pair of XCDs, each XCD's units longest first; persistent and narrow launches have none
    fp8 = dict(kv_dtype="fp8_e4m3", k_scale=1.0, v_scale=1.0)
    hq, hkv, d, page, kw = {"fp8_d256": (24, 4, 256, 16, fp8), "fp8_d128": (32, 8, 128, 16, fp8),
                            "bf16_d512": (16, 4, 512, 16, {}), "bf16_d128_page1": (32, 8, 128, 1, {})}[kind]
    for specs in ([(8192, 8192)], [(2048, 2048)] * 4, [(9000, 900), (1300, 1300), (600, 200)], [(67, 67)],
                  [(32768, 32768)]):
        if page == 1 and specs[0][0] > 9000:
            continue
        p = _plan(dpp, _specs_batch(specs, page=page, g=hq // hkv), hq=hq, hkv=hkv, d=d, page=page,
                  cap=64 << 20, **kw)
        parsed = parse(p.header())
        if kind != "bf16_d128_page1":
            assert len(parsed.units) == 0
        for ps in range(p.info.num_passes):
            items = parsed.items[parsed.items[:, 7] == ps]
            if ps in parsed.tables:
                assert not (parsed.units[:, 14] == ps).any()
                _check_table(parsed.tables[ps], items, hkv)
            else:  # page size 1 with units short enough for two page tables: persistent
                _check_chains(parsed, items, parsed.units[parsed.units[:, 14] == ps], hkv)
        if kind == "bf16_d128_page1" and specs[0][0] > 4200:
            assert parsed.tables, "a unit spanning 4096 one-token pages needs the one-table launch"
    ext = _specs_batch([(1024 + t, t) for t in range(1, 16 // (hq // hkv) + 1)] * 4, page=page, g=hq // hkv)
    assert parse(_plan(dpp, ext, hq=hq, hkv=hkv, d=d, page=page, **kw).header()).tables == {}


def test_block_tables_balance_xcds(dpp):
    # the fp8 24/4/256 prefill of 8,192 tokens: equal-count XCD runs put 1.42x the mean cost on
    # half the XCDs; the table's per-XCD costs are within 2 % of the mean
    p = _plan(dpp, _specs_batch([(8192, 8192)], g=6), hq=24, hkv=4, d=256, kv_dtype="fp8_e4m3", k_scale=1.0,
              v_scale=1.0)
    parsed = parse(p.header())
    t = parsed.tables[0]
    cost = (parsed.items[:, 5] - parsed.items[:, 4]) + 2
    n = len(parsed.items)
    per_xcd = np.zeros(8)
    for b, w in enumerate(t):
        if w >= 0:
            per_xcd[b % 8] += cost[w % n]
    assert per_xcd.max() <= 1.02 * per_xcd.mean(), per_xcd


def test_persistent_chains_per_pass(dpp):
    b = _specs_batch([(9000, 9000), (6000, 6000)])
    p = _plan(dpp, b, cap=24 << 20)
    assert p.info.num_passes > 1
    parsed = parse(p.header())
    # items of a pass are contiguous in the header and, with wide tiles only, all chained
    seen = 0
    for ps in range(p.info.num_passes):
        units = parsed.units[parsed.units[:, 14] == ps]
        n = len(units) // 8
        _check_chains(parsed, parsed.items[seen:seen + n], units, 8)
        seen += n
    assert seen == len(parsed.items)


def test_no_chains_where_not_persistent(dpp):
    # narrow passes (extends), head_dim 512 (four waves) and fp8 launches are not persistent;
    # wide bf16 passes at head_dim 256 (eight waves) are
    ext = _specs_batch([(1024 + t, t) for t in (1, 2, 3, 4)] * 4)
    assert len(parse(_plan(dpp, ext).header()).units) == 0
    big = _specs_batch([(1028, 1028)] * 2)
    assert len(parse(_plan(dpp, big, hq=16, hkv=4, d=512).header()).units) == 0
    assert len(parse(_plan(dpp, big, kv_dtype="fp8_e4m3", k_scale=1.0, v_scale=1.0).header()).units) == 0
    assert len(parse(_plan(dpp, big, hq=16, hkv=4, d=256, kv_dtype="fp8_e4m3", k_scale=1.0,
                           v_scale=1.0).header()).units) == 0
    p256 = _plan(dpp, big, hq=16, hkv=4, d=256)
    parsed = parse(p256.header())
    _check_chains(parsed, parsed.items, parsed.units, 4)
    # page size 1: two page tables of a 4096-key split do not fit beside the ring
    assert len(parse(_plan(dpp, _specs_batch([(5000, 5000)], page=1), page=1).header()).units) == 0


def test_zero_length_request_gets_no_rows(dpp):
    b = _specs_batch([(50, 0), (50, 5), (0, 0)])
    parsed = parse(_plan(dpp, b).header())
    assert set(int(r) for r in parsed.items[:, 0]) == {1}
    assert parsed.requests[0][1] == 0 and parsed.requests[2][3] == 0


def test_p2_split_workspace_figures():
    """The pages' split-buffer numbers follow from q tiles x fixed 4096-token splits.

    Pinned against the figures the page prints: 1,536 work items and 2,415,919,104 bytes for
    an 8,192-token prefill at 24/4/256 with cta_tile_q 64, and the ~7,275-token prompt at
    which a fixed 2 GiB buffer first overflows. Our planner uses the same item structure
    (one item per q tile per split), but bounds the partials by passes.
    """
    with open(os.path.join(ROOT, "tests", "golden", "split_workspace_p2.json")) as f:
        gold = json.load(f)
    s = gold["shape"]
    g = s["num_qo_heads"] // s["num_kv_heads"]

    def items(n):
        return -(-n * g // s["cta_tile_q"]) * -(-n // s["split_tokens"])

    def buffer_bytes(n):
        return s["num_qo_heads"] * items(n) * s["cta_tile_q"] * s["head_dim"] * 4

    assert items(gold["prefill_tokens"]) == gold["work_items"]
    assert buffer_bytes(gold["prefill_tokens"]) == gold["buffer_bytes"]
    first = next(n for n in range(1, 10000) if buffer_bytes(n) > gold["fixed_workspace_bytes"])
    assert first == gold["first_overflowing_prompt_tokens_approx"]


@pytest.mark.parametrize("mutate,status", [
    (lambda q, k, l: q.__setitem__(1, q[2] + 1), "DPP_ERR_INVALID"),    # non-monotone qo_indptr
    (lambda q, k, l: q.__setitem__(0, 1), "DPP_ERR_INVALID"),            # qo_indptr[0] != 0
    (lambda q, k, l: k.__setitem__(1, -1), "DPP_ERR_INVALID"),           # negative page count
    (lambda q, k, l: l.__setitem__(0, 0), "DPP_ERR_SHAPE"),              # last page length 0
    (lambda q, k, l: l.__setitem__(0, 17), "DPP_ERR_SHAPE"),             # last page length > page
    (lambda q, k, l: q.__setitem__(slice(1, None), q[1:] + 100), "DPP_ERR_SHAPE"),  # qo_len > kv_len
])
def test_malformed_batches_are_rejected(dpp, mutate, status):
    b = _specs_batch([(67, 3), (40, 40)])
    q, k, l = b.qo_indptr.copy(), b.kv_indptr.copy(), b.kv_last_page_len.copy()
    mutate(q, k, l)
    with pytest.raises(dpp.DppValueError, match=status):
        dpp.plan(32, 8, 128, 16, q, k, l)


@pytest.mark.parametrize("args,status", [
    (dict(num_qo_heads=32, num_kv_heads=8, head_dim=96), "DPP_ERR_UNSUPPORTED"),
    (dict(num_qo_heads=32, num_kv_heads=8, head_dim=1024), "DPP_ERR_UNSUPPORTED"),
    (dict(num_qo_heads=30, num_kv_heads=8, head_dim=128), "DPP_ERR_UNSUPPORTED"),
    (dict(num_qo_heads=2050, num_kv_heads=2, head_dim=128), "DPP_ERR_UNSUPPORTED"),
    (dict(num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=-1), "DPP_ERR_UNSUPPORTED"),
    (dict(num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=1025), "DPP_ERR_UNSUPPORTED"),
])
def test_unsupported_configs(dpp, args, status):
    b = _specs_batch([(67, 3)])
    kw = dict(num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=16)
    kw.update(args)
    with pytest.raises(dpp.DppValueError, match=status):
        dpp.plan(kw["num_qo_heads"], kw["num_kv_heads"], kw["head_dim"], kw["page_size"],
                 b.qo_indptr, b.kv_indptr, b.kv_last_page_len)


def test_cap_below_one_tile_is_rejected(dpp):
    b = _specs_batch([(9000, 9000)])
    with pytest.raises(dpp.DppValueError, match="DPP_ERR_WORKSPACE"):
        _plan(dpp, b, cap=1 << 20)


def test_run_rejects_bad_shapes_before_any_launch(dpp):
    """dpp_run's checks happen on the host before any HIP call (exercised here without a GPU)."""
    lib = dpp.library()
    b = _specs_batch([(67, 3)])
    p = _plan(dpp, b)
    fake = 1 << 20  # never dereferenced: every call below fails its host-side checks
    ws = p.workspace_bytes
    st = lib.dpp_run(p._h, fake, 4, fake, fake, 64, fake, 5, fake, fake, fake, ws, 0, None)
    assert st == dpp.DPP_ERR_SHAPE and b"q has 4 rows" in lib.dpp_last_error()
    st = lib.dpp_run(p._h, fake, 3, fake, fake, 64, fake, 5, fake, fake, fake, ws - 1, 0, None)
    assert st == dpp.DPP_ERR_WORKSPACE
    st = lib.dpp_run(p._h, fake, 3, fake, fake, 64, fake, 5, fake, fake, fake + 16, ws, 0, None)
    assert st == dpp.DPP_ERR_WORKSPACE  # misaligned workspace
    st = lib.dpp_run(p._h, fake, 3, fake, fake, 64, fake, 5, fake, fake, None, ws, 0, None)
    assert st == dpp.DPP_ERR_WORKSPACE
    st = lib.dpp_run(p._h, fake, 3, fake, fake, 64, fake, 5, fake, fake, fake, ws, 4, None)
    assert st == dpp.DPP_ERR_INVALID  # unknown flag
    st = lib.dpp_plan_upload(p._h, fake + 16, ws, None)
    assert st == dpp.DPP_ERR_WORKSPACE
    # a page list shorter than kv_indptr[-1] (5 pages) would be read past its end on the device
    st = lib.dpp_run(p._h, fake, 3, fake, fake, 64, fake, 4, fake, fake, fake, ws, 0, None)
    assert st == dpp.DPP_ERR_SHAPE and b"kv_indices holds 4" in lib.dpp_last_error()
    # reusing an upload that never happened: the kernels would find no work list
    st = lib.dpp_run(p._h, fake, 3, fake, fake, 64, fake, 5, fake, fake, fake, ws, 1, None)
    assert st == dpp.DPP_ERR_INVALID and b"never uploaded" in lib.dpp_last_error()
    st = lib.dpp_merge_states(fake, fake, 1, 0, 1, 128, fake, fake, None)
    assert st == dpp.DPP_ERR_INVALID
    st = lib.dpp_merge_states(fake, fake, 1, 2, 1, 130, fake, fake, None)
    assert st == dpp.DPP_ERR_UNSUPPORTED


def test_stream_reference_rejects_bad_arguments(dpp):
    """dpp_stream_kv's checks happen on the host before any HIP call (no GPU needed)."""
    lib = dpp.library()
    b = _specs_batch([(1028, 3)])
    p = _plan(dpp, b)
    fake = 1 << 20
    ws = p.workspace_bytes
    n = int(b.kv_indptr[-1])

    def call(split=2, depth=4, flags=1, workspace=fake, kv=n):
        return lib.dpp_stream_kv(p._h, fake, fake, 4096, fake, kv, workspace, ws, split, depth, flags, None)

    assert call(split=0) == dpp.DPP_ERR_INVALID and b"split" in lib.dpp_last_error()
    assert call(split=9) == dpp.DPP_ERR_INVALID
    assert call(depth=5) == dpp.DPP_ERR_INVALID and b"depth" in lib.dpp_last_error()
    assert call(split=1, flags=1 | dpp.STREAM_HEAD_SPLIT) == dpp.DPP_ERR_INVALID
    assert b"split 2" in lib.dpp_last_error()
    assert call(flags=4) == dpp.DPP_ERR_INVALID and b"unknown flags" in lib.dpp_last_error()
    assert call(kv=n - 1) == dpp.DPP_ERR_SHAPE
    assert call(workspace=fake + 16) == dpp.DPP_ERR_WORKSPACE
    assert call(workspace=None) == dpp.DPP_ERR_INVALID


def test_null_arguments(dpp):
    lib = dpp.library()
    assert lib.dpp_plan_create(None, 0, None, None, None, 0, None) == dpp.DPP_ERR_INVALID
    assert lib.dpp_plan_workspace_bytes(None) == 0
    lib.dpp_plan_destroy(None)


def test_workload_batches_plan(dpp):
    """Every configuration's batches plan without error (shapes only; no data drawn here)."""
    for specs in ([(1028, 1028)] * 16, [(1024 + t, t) for t in (1, 2, 3, 4)] * 4):
        p = _plan(dpp, _specs_batch(specs))
        assert p.info.num_prefill_items > 0
    work = wl.single_extend()
    p = _plan(dpp, work.batches["cached"])
    assert p.info.total_q_rows == 3


# ---- ragged (contiguous) KV: page_size 0, kv_indptr in tokens

def _ragged_indptr(specs):
    kv_len = [kv for kv, _ in specs]
    return np.concatenate([[0], np.cumsum(kv_len)]).astype(np.int32), kv_len


@pytest.mark.parametrize("specs", [[(67, 3), (40, 40), (300, 0), (1, 1)], [(4100, 12), (8200, 2), (129, 129)]])
def test_ragged_plan_has_the_paged_plans_work(dpp, specs):
    """The same tiles, splits and items as the paged plan; each request's page_start is its
    first token and its kv_len is its token count."""
    b = _specs_batch(specs)
    paged = parse(_plan(dpp, b).header())
    kvp, kv_len = _ragged_indptr(specs)
    rp = dpp.plan(32, 8, 128, 0, b.qo_indptr, kvp)  # no kv_last_page_len
    ragged = parse(rp.header())
    assert rp.info.workspace_bytes == _plan(dpp, b).info.workspace_bytes
    assert list(ragged.requests[:, 3]) == kv_len
    assert list(ragged.requests[:, 2]) == list(kvp[:-1])
    assert (ragged.requests[:, [0, 1, 3]] == paged.requests[:, [0, 1, 3]]).all()
    cols = [0, 1, 2, 3, 4, 5, 6, 8, 9, 11]  # everything but the page list offset
    assert (ragged.items[:, cols] == paged.items[:, cols]).all()
    assert (ragged.merges == paged.merges).all()


def test_ragged_plan_ignores_last_page_len_and_checks_request_bytes(dpp):
    qo = np.array([0, 2], dtype=np.int32)
    a = dpp.plan(32, 8, 128, 0, qo, np.array([0, 100], dtype=np.int32), np.array([7], dtype=np.int32))
    b = dpp.plan(32, 8, 128, 0, qo, np.array([0, 100], dtype=np.int32))
    assert (a.header()[16:] == b.header()[16:]).all()
    # 8 kv heads x 128 x 2 B = 2 KiB a token: a request's K plus one tile's worth of keys
    # past its end must stay below 2 GiB
    dpp.plan(32, 8, 128, 0, qo, np.array([0, (1 << 20) - 257], dtype=np.int32), workspace_cap=0)
    with pytest.raises(dpp.DppValueError, match="DPP_ERR_UNSUPPORTED"):
        dpp.plan(32, 8, 128, 0, qo, np.array([0, 1 << 20], dtype=np.int32), workspace_cap=0)
    with pytest.raises(ValueError):
        dpp.plan(32, 8, 128, 16, qo, np.array([0, 7], dtype=np.int32))  # paged needs last_page_len


def test_ragged_run_rejects_kv_beyond_the_tokens_passed(dpp):
    """Ragged KV: kv_indptr[-1] above the token rows the caller passes fails on the host."""
    lib = dpp.library()
    p = dpp.plan(32, 8, 128, 0, np.array([0, 3, 5], np.int32), np.array([0, 67, 107], np.int32))
    fake = 1 << 20
    ws = p.workspace_bytes
    st = lib.dpp_run(p._h, fake, 5, fake, fake, 106, None, 0, fake, fake, fake, ws, 0, None)
    assert st == dpp.DPP_ERR_SHAPE and b"107 tokens" in lib.dpp_last_error()


# ---- adaptive-tile comparison mode (not batch invariant)

def test_adaptive_tile_mode_picks_the_kv_tile_from_the_batch(dpp):
    """FlashInfer's rule: an average packed query length of at most 16 over a batch of narrow
    tiles gets 32-key KV tiles at head_dim 128; anything else, and the default mode, 64."""
    extend = _specs_batch([(1025, 1), (1026, 2), (1028, 4), (1027, 3)])  # avg packed 10
    longer = _specs_batch([(1025, 4), (1026, 4), (1028, 4), (1027, 5)])  # avg packed 17
    prefill = _specs_batch([(1028, 1028)])
    ad = lambda b: _plan(dpp, b, adaptive_kv_tile=True)
    assert _plan(dpp, extend).info.block_n == 64
    p = ad(extend)
    assert p.info.block_n == 32
    items = parse(p.header()).items
    fixed = parse(_plan(dpp, extend).header()).items
    # the same items, their KV tiles counted in 32-key units: 1028 keys -> 33 tiles, not 17
    assert (items[:, 5] == [-(-(kv) // 32) for kv in (1025, 1026, 1028, 1027)]).all()
    assert (fixed[:, 5] == [-(-(kv) // 64) for kv in (1025, 1026, 1028, 1027)]).all()
    assert ad(longer).info.block_n == 64 and ad(prefill).info.block_n == 64
    # head_dim 256 keeps its 32-key tile, fp8 its own
    assert _plan(dpp, extend, hq=24, hkv=4, d=256, adaptive_kv_tile=True).info.block_n == 32
    assert _plan(dpp, extend, kv_dtype="fp8_e4m3", adaptive_kv_tile=True).info.block_n == 64


def test_plan_create_ex_rejects_unknown_flags(dpp):
    lib = dpp.library()
    b = _specs_batch([(67, 3)])
    cfg = dpp._Config(32, 8, 128, 16, 0, 0.0, 1.0, 1.0)
    h = ctypes.c_void_p()
    st = lib.dpp_plan_create_ex(ctypes.byref(cfg), 1, b.qo_indptr.ctypes.data, b.kv_indptr.ctypes.data,
                                b.kv_last_page_len.ctypes.data, 0, 4, ctypes.byref(h))
    assert st == dpp.DPP_ERR_INVALID and h.value is None
    # a permutation seed without the permutation flag
    st = lib.dpp_plan_create_ex(ctypes.byref(cfg), 1, b.qo_indptr.ctypes.data, b.kv_indptr.ctypes.data,
                                b.kv_last_page_len.ctypes.data, 0, 5 << 16, ctypes.byref(h))
    assert st == dpp.DPP_ERR_INVALID and h.value is None


@pytest.mark.parametrize("specs", [[(1028, 1028)] * 2, [(1025, 1), (4100, 12), (8200, 2)]])
def test_head_dim_64_plans_like_128(dpp, specs):
    """head_dim 64 uses the tile of head_dim <= 128 (256 packed rows x 64 keys): the same
    items as a head_dim 128 plan of the batch, every needed (row, split) covered, a persistent
    unit record per (item, kv head) for wide passes, partial slots of (64 + 1) floats."""
    b = _specs_batch(specs)
    p64, p128 = _plan(dpp, b, d=64), _plan(dpp, b, d=128)
    assert (p64.info.block_m, p64.info.block_n) == (256, 64) == dpp.tile_shape(64)
    a, c = parse(p64.header()), parse(p128.header())
    assert (a.items[:, :7] == c.items[:, :7]).all() and (a.merges == c.merges).all()
    assert len(a.units) == len(c.units)
    cov = _coverage(a, 4, 256)
    for r, (kv, qlen) in enumerate(specs):
        for R in range(qlen * 4):
            pos = kv - qlen + R // 4
            for s in range(pos // 4096 + 1):
                assert (r, R, s) in cov
    slots = p64.info.max_partial_slots
    assert slots == p128.info.max_partial_slots
    if slots:
        assert p64.workspace_bytes - p64.info.header_bytes == _align(slots * 64 * 4) + _align(slots * 4)


@pytest.mark.parametrize("specs", [[(1028, 1028)], [(1025, 1), (4100, 12), (8200, 2), (300, 0)],
                                   [(9000, 9000), (67, 3)]])
def test_head_dim_512_tiles(dpp, specs):
    """head_dim 512: 64 packed rows x 32 keys a tile (4 waves of one 16-row block), every needed
    (row, split) covered, no persistent chains, partial slots of (512 + 1) floats."""
    g = 4
    b = _specs_batch(specs, g=g)
    p = _plan(dpp, b, hq=32, hkv=8, d=512)
    assert (p.info.block_m, p.info.block_n) == (64, 32) == dpp.tile_shape(512)
    a = parse(p.header())
    assert len(a.units) == 0
    cov = _coverage(a, g, 64)
    for r, (kv, qlen) in enumerate(specs):
        for R in range(qlen * g):
            pos = kv - qlen + R // g
            for s in range(pos // 4096 + 1):
                kb, ke = cov[(r, R, s)]
                assert kb == s * 128 and ke * 32 > min(pos, (s + 1) * 4096 - 1) and ke <= (s + 1) * 128
    slots = p.info.max_partial_slots
    if slots:
        assert p.workspace_bytes - p.info.header_bytes == _align(slots * 512 * 4) + _align(slots * 4)


# ---- page-table contract (host check)

def test_check_page_table(dpp):
    """Every page id a request reads must lie in [0, num_pages); the host check names the first
    one that does not, and a page list shorter than kv_indptr[-1] is a shape error."""
    b = _specs_batch([(67, 3), (0, 0), (20, 20)])  # 5 + 0 + 2 pages
    p = _plan(dpp, b)
    ids = np.arange(7, dtype=np.int32) * 3
    p.check_page_table(ids, num_pages=19)          # largest id 18
    with pytest.raises(dpp.DppValueError, match="request 2, page 1: id 18"):
        p.check_page_table(ids, num_pages=18)
    bad = ids.copy()
    bad[3] = -1
    with pytest.raises(dpp.DppValueError, match="request 0, page 3: id -1"):
        p.check_page_table(bad, num_pages=64)
    with pytest.raises(dpp.DppValueError, match="kv_indices holds 6"):
        p.check_page_table(ids[:6], num_pages=64)
    # entries past kv_indptr[-1] are never read
    p.check_page_table(np.concatenate([ids, [-5, 10**6]]).astype(np.int32), num_pages=19)
    # ragged KV has no page table
    pr = dpp.plan(32, 8, 128, 0, np.array([0, 3], np.int32), np.array([0, 67], np.int32))
    pr.check_page_table(np.zeros(0, np.int32), num_pages=67)


# ---- partial-slot invariant: the split-partial writes and the merge's reads stay inside the
# pass's slot region, and only multi-split tiles own slots

def _check_slot_invariant(parsed, hkv, g, bm, max_slots):
    S_of_tile = {}
    blocks = {}
    for it in parsed.items:
        r, rs, s, S, kb, ke, slot = (int(x) for x in it[:7])
        q_start, qo_len, page_start, kv_len = (int(x) for x in parsed.requests[r])
        rows = min(bm, qo_len * g - rs)
        p_max = kv_len - qo_len + (rs + rows - 1) // g
        assert S == p_max // 4096 + 1, "tile split count is its last row's"
        S_of_tile.setdefault((r, rs), (S, slot))
        assert S_of_tile[(r, rs)] == (S, slot), "every item of a tile carries the same slot block"
        if S == 1:
            assert slot == -1, f"single-split tile {(r, rs)} owns slot base {slot}"
        else:
            assert slot >= 0, f"multi-split tile {(r, rs)} has no slot block"
            size = S * hkv * ((rows + 15) // 16 * 16)
            assert slot + size <= max_slots, f"tile {(r, rs)} block [{slot}, {slot + size}) past {max_slots}"
            blocks[(r, rs)] = (slot, slot + size)
    merged = {(int(m[0]), int(m[1])): (int(m[2]), int(m[3])) for m in parsed.merges}
    for key, (S, slot) in S_of_tile.items():
        if S == 1:
            assert key not in merged, f"single-split tile {key} has a merge item"
        else:
            assert merged[key] == (S, slot), f"merge item of {key} disagrees with its prefill items"
    return blocks


@pytest.mark.parametrize("seed", range(12))
def test_partial_slots_stay_inside_each_pass(dpp, seed):
    rng = np.random.default_rng(seed)
    d = int(rng.choice([64, 128, 256]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 3, 4, 6]))
    specs = []
    for _ in range(int(rng.integers(1, 9))):
        kv = int(rng.choice([rng.integers(0, 300), rng.integers(3000, 13000), rng.integers(4090, 4100)]))
        ql = int(rng.choice([kv, min(kv, int(rng.integers(0, 40))), min(kv, 1)]))
        specs.append((kv, ql))
    b = _specs_batch(specs)
    bm = dpp.tile_shape(d)[0]
    # the largest single tile's partials decide the smallest cap that plans
    need = 0
    for kv, ql in specs:
        for rs in range(0, ql * g, bm):
            rows = min(bm, ql * g - rs)
            S = (kv - ql + (rs + rows - 1) // g) // 4096 + 1
            if S > 1:
                need = max(need, S * hkv * ((rows + 15) // 16 * 16))
    caps = [0, 256 << 20] + ([int(need * (d + 1) * 4 * f) + (4 << 20) for f in (1.0, 1.7, 3.1)] if need else [])
    for cap in caps:
        p = _plan(dpp, b, hq=hkv * g, hkv=hkv, d=d, cap=cap)
        parsed = parse(p.header())
        blocks = _check_slot_invariant(parsed, hkv, g, bm, p.info.max_partial_slots)
        # unit records of persistent launches carry their tile's (tile_splits, slot_base)
        for u in parsed.units:
            r, rs, S, slot = int(u[0]), int(u[1]), int(u[3]), int(u[6])
            assert slot == (-1 if S == 1 else blocks[(r, rs)][0])
        if cap:
            assert p.workspace_bytes <= cap
        _check_disjoint_per_pass(p, parsed, blocks)


def _check_disjoint_per_pass(p, parsed, blocks):
    """Slot blocks of the tiles of one pass never overlap (each item records its pass)."""
    by_pass = {}
    for it in parsed.items:
        key, ps = (int(it[0]), int(it[1])), int(it[7])
        assert 0 <= ps < p.info.num_passes
        if key in blocks:
            by_pass.setdefault(ps, set()).add(blocks[key])
    for ps, spans in by_pass.items():
        spans = sorted(spans)
        for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
            assert a1 <= b0, f"pass {ps}: slot blocks [{a0}, {a1}) and [{b0}, {b1}) overlap"


@pytest.mark.parametrize("seed", [1, 2, 77])
def test_permuted_plan_has_the_same_work(dpp, seed):
    """The test-only permutation reorders items and merges inside each pass and nothing else."""
    b = _specs_batch([(3700, 3700), (3701, 1), (3737, 37), (9000, 300), (1028, 1028), (5000, 4)])
    base = _plan(dpp, b, cap=64 << 20)
    perm = _plan(dpp, b, cap=64 << 20, permute_seed=seed)
    pa, pb = parse(base.header()), parse(perm.header())
    assert base.info == perm.info
    key = lambda rows: sorted(tuple(int(x) for x in r) for r in rows)  # noqa: E731
    assert key(pa.items) == key(pb.items)
    assert key(pa.merges) == key(pb.merges)
    assert [tuple(map(int, r)) for r in pa.items] != [tuple(map(int, r)) for r in pb.items]
    # items stay in their pass
    ps_a = [int(it[7]) for it in pa.items]
    assert ps_a == sorted(ps_a) and [int(it[7]) for it in pb.items] == ps_a


def test_run_static_refuses_plans_above_its_scratch(dpp):
    """dpp_run_static checks the plan against its fixed scratch before any HIP call."""
    lib = dpp.library()
    b = _specs_batch([(8192, 8192)])
    big = _plan(dpp, b, hq=24, hkv=4, d=256, cap=0)
    assert big.workspace_bytes > dpp.STATIC_SCRATCH_BYTES
    fake = 1 << 20
    st = lib.dpp_run_static(big._h, fake, 8192, fake, fake, 600, fake, 512, fake, fake, 0, None)
    assert st == dpp.DPP_ERR_WORKSPACE and b"static scratch" in lib.dpp_last_error()
    # the same batch planned under the scratch's size fits, in more passes
    small = _plan(dpp, b, hq=24, hkv=4, d=256, cap=dpp.STATIC_SCRATCH_BYTES)
    assert small.workspace_bytes <= dpp.STATIC_SCRATCH_BYTES and small.info.num_passes > 1
    st = lib.dpp_run_static(small._h, fake, 8191, fake, fake, 600, fake, 512, fake, fake, 0, None)
    assert st == dpp.DPP_ERR_SHAPE  # dpp_run's argument checks come first
    st = lib.dpp_run_static(small._h, fake, 8192, fake, fake, 600, fake, 512, fake, fake, 2, None)
    assert st == dpp.DPP_ERR_INVALID


def test_row_split_multiply_shift_is_exact():
    """The kernels split packed row R0 + off of a wave into (token, q head) with
    (h0 + off) * ceil(2^24 / g) >> 24 in place of (h0 + off) / g, for h0 < g, off < 32 and
    g up to the planner's limit of 1024; that quotient must be exact and the product must fit
    in 32 bits."""
    for g in range(1, 1025):
        m = ((1 << 24) + g - 1) // g
        x = np.arange(0, g + 32, dtype=np.uint64)
        assert (x * m < 2**32).all()
        assert ((x * m) >> 24 == x // g).all()
