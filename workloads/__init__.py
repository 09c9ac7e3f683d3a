"""Seeded synthetic workloads for paged-KV causal GQA prefill attention.

Shared by the test suite, the benchmark and the smoke check. This module holds no attention
arithmetic: it draws N(0,1) tensors, encodes them to the storage dtype (bf16, or OCP E4M3 via
torch's own cast), lays prompts out in a shuffled, NaN-poisoned page pool and writes page
tables. Everything is CPU-side and deterministic in its seed.

Vocabulary
----------
* A *prompt* is a sequence of tokens, each with a q row per q head and a k/v row per kv head.
* A *request* in a batch is (prompt, kv_len, qo_len): its KV is the prompt's first kv_len
  tokens, its queries are the prompt's tokens kv_len-qo_len .. kv_len-1 (the uncached tail).
  A full prefill has qo_len == kv_len; a prefix-cache hit has qo_len < kv_len.
* Two rows are *the same computation* when they belong to the same prompt, sit at the same
  absolute position and see the same kv_len-independent key prefix; their outputs must be
  bit-identical (see :func:`matching_rows`).

Shapes follow the pages' workloads: Qwen3-8B / Qwen3-4B attention (32 q heads, 8 kv heads,
head_dim 128) and a 24/4/256 model with an fp8 E4M3 KV cache, page size 16.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

BF16_NAN_BITS = 0x7FC0  # poison for unused bf16 pool slots
E4M3_NAN_CODE = 0x7F    # poison for unused fp8 pool slots (S.1111.111)
FP8_DATA_SCALE = 32.0   # N(0,1) values are multiplied by this before E4M3 encoding


@dataclass
class Prompt:
    q: torch.Tensor  # bf16 [L - q_from, Hq, d]: queries of tokens q_from .. L-1
    k: torch.Tensor  # storage dtype [L, Hkv, d] (bf16, or uint8 E4M3 codes)
    v: torch.Tensor
    q_from: int = 0  # first token with a query (long decode prompts keep only their last ones)

    @property
    def length(self) -> int:
        return int(self.k.shape[0])


@dataclass
class Request:
    prompt: int
    kv_len: int
    qo_len: int
    pages: list  # physical page ids, ceil(kv_len / page_size) of them


@dataclass
class PagedBatch:
    requests: list
    qo_indptr: np.ndarray = field(default=None)
    kv_indptr: np.ndarray = field(default=None)
    kv_indices: np.ndarray = field(default=None)
    kv_last_page_len: np.ndarray = field(default=None)
    q: torch.Tensor = field(default=None)  # bf16 [qo_indptr[-1], Hq, d]

    @property
    def batch_size(self) -> int:
        return len(self.requests)

    @property
    def num_q_tokens(self) -> int:
        return int(self.qo_indptr[-1])


@dataclass
class Workload:
    name: str
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    kv_dtype: str  # "bf16" | "fp8_e4m3"
    k_scale: float
    v_scale: float
    k_pool: torch.Tensor  # [num_pages, page_size, Hkv, d] bf16 or uint8
    v_pool: torch.Tensor
    prompts: list
    batches: dict
    description: str = ""

    @property
    def num_pages(self) -> int:
        return int(self.k_pool.shape[0])

    def oracle_kwargs(self, batch: PagedBatch) -> dict:
        return dict(q=batch.q, k_pool=self.k_pool, v_pool=self.v_pool,
                    qo_indptr=batch.qo_indptr, kv_indptr=batch.kv_indptr,
                    kv_indices=batch.kv_indices, kv_last_page_len=batch.kv_last_page_len,
                    num_qo_heads=self.num_qo_heads, num_kv_heads=self.num_kv_heads,
                    head_dim=self.head_dim, page_size=self.page_size, kv_dtype=self.kv_dtype,
                    k_scale=self.k_scale, v_scale=self.v_scale)


# --------------------------------------------------------------------------- drawing

def _randn(shape, seed: int) -> torch.Tensor:
    g = torch.Generator().manual_seed(int(seed))
    return torch.randn(*shape, generator=g, dtype=torch.float32)


def _to_storage(x: torch.Tensor, kv_dtype: str) -> torch.Tensor:
    if kv_dtype == "bf16":
        return x.to(torch.bfloat16)
    if kv_dtype == "fp8_e4m3":
        return (x * FP8_DATA_SCALE).to(torch.float8_e4m3fn).view(torch.uint8)
    raise ValueError(kv_dtype)


def draw_prompt(length: int, hq: int, hkv: int, d: int, kv_dtype: str, seed: int,
                q_from: int = 0) -> Prompt:
    """q, k, v ~ N(0, 1) (k, v scaled by 32 before E4M3 encoding when kv_dtype is fp8).

    Queries are drawn for tokens q_from .. length-1 only."""
    q = _randn((length - q_from, hq, d), seed * 7 + 1).to(torch.bfloat16)
    k = _to_storage(_randn((length, hkv, d), seed * 7 + 2), kv_dtype)
    v = _to_storage(_randn((length, hkv, d), seed * 7 + 3), kv_dtype)
    return Prompt(q, k, v, q_from)


def extend_prompt(base: Prompt, extra: int, hq: int, hkv: int, d: int, kv_dtype: str,
                  seed: int) -> Prompt:
    """A prompt whose first tokens are ``base`` (a shared prefix) followed by fresh tokens."""
    assert base.q_from == 0
    tail = draw_prompt(extra, hq, hkv, d, kv_dtype, seed)
    return Prompt(torch.cat([base.q, tail.q]), torch.cat([base.k, tail.k]),
                  torch.cat([base.v, tail.v]))


# --------------------------------------------------------------------------- page pool

class PagePool:
    """A KV page pool whose pages are handed out in a seed-shuffled order.

    Every slot starts as NaN, so a kernel that reads an unused slot (past a request's last
    valid token, or a page no request owns) poisons its output.
    """

    def __init__(self, num_pages: int, page_size: int, hkv: int, d: int, kv_dtype: str,
                 seed: int):
        self.page_size = page_size
        self.kv_dtype = kv_dtype
        shape = (num_pages, page_size, hkv, d)
        if kv_dtype == "bf16":
            self.k = torch.full(shape, BF16_NAN_BITS, dtype=torch.int16).view(torch.bfloat16)
            self.v = torch.full(shape, BF16_NAN_BITS, dtype=torch.int16).view(torch.bfloat16)
        else:
            self.k = torch.full(shape, E4M3_NAN_CODE, dtype=torch.uint8)
            self.v = torch.full(shape, E4M3_NAN_CODE, dtype=torch.uint8)
        rng = np.random.default_rng(seed)
        self._free = list(rng.permutation(num_pages))

    def alloc(self) -> int:
        if not self._free:
            raise RuntimeError("page pool exhausted")
        return int(self._free.pop())

    def write_tokens(self, prompt: Prompt, start: int, stop: int, pages: list) -> None:
        """Write prompt tokens [start, stop) into ``pages`` (token t -> pages[t // P])."""
        P = self.page_size
        for t0 in range(start - start % P, stop, P):
            page = pages[t0 // P]
            a, b = max(t0, start), min(t0 + P, stop)
            self.k[page, a - t0:b - t0] = prompt.k[a:b]
            self.v[page, a - t0:b - t0] = prompt.v[a:b]

    def place(self, prompt: Prompt, kv_len: int, shared_pages: list | None = None) -> list:
        """Page list for the prompt's first kv_len tokens.

        ``shared_pages`` are existing full pages holding the prompt's leading tokens (a
        radix-cache prefix); they are reused as-is and fresh pages hold the rest.
        """
        P = self.page_size
        n_pages = -(-kv_len // P)
        pages = list(shared_pages or [])
        assert len(pages) * P <= kv_len
        first_new = len(pages) * P
        while len(pages) < n_pages:
            pages.append(self.alloc())
        self.write_tokens(prompt, first_new, kv_len, pages)
        return pages


def make_batch(requests: list, prompts: list, page_size: int) -> PagedBatch:
    qo, kvp, idx, last, qs = [0], [0], [], [], []
    for r in requests:
        assert 0 <= r.qo_len <= r.kv_len <= prompts[r.prompt].length
        assert len(r.pages) == -(-r.kv_len // page_size)
        qo.append(qo[-1] + r.qo_len)
        kvp.append(kvp[-1] + len(r.pages))
        idx.extend(r.pages)
        last.append(r.kv_len - (len(r.pages) - 1) * page_size if r.pages else 0)
        p = prompts[r.prompt]
        assert r.kv_len - r.qo_len >= p.q_from, "a query row the prompt does not hold"
        qs.append(p.q[r.kv_len - r.qo_len - p.q_from:r.kv_len - p.q_from])
    hq, d = prompts[0].q.shape[1:]
    q = torch.cat(qs) if qs else torch.zeros((0, hq, d), dtype=torch.bfloat16)
    return PagedBatch(requests=list(requests),
                      qo_indptr=np.asarray(qo, dtype=np.int32),
                      kv_indptr=np.asarray(kvp, dtype=np.int32),
                      kv_indices=np.asarray(idx, dtype=np.int32),
                      kv_last_page_len=np.asarray(last, dtype=np.int32),
                      q=q.contiguous())


def sub_batch(batch: PagedBatch, prompts: list, page_size: int, which: list) -> PagedBatch:
    return make_batch([batch.requests[i] for i in which], prompts, page_size)


def concat_batches(batches: list, prompts: list, page_size: int) -> PagedBatch:
    return make_batch([r for b in batches for r in b.requests], prompts, page_size)


def matching_rows(a: PagedBatch, ra: int, b: PagedBatch, rb: int):
    """Global q-token indices (in a, in b) of rows that are the same computation.

    Requests ra of ``a`` and rb of ``b`` must be the same prompt. Returns two equal-length
    int64 arrays; the rows are the positions both requests query.
    """
    A, B = a.requests[ra], b.requests[rb]
    assert A.prompt == B.prompt
    a0, b0 = A.kv_len - A.qo_len, B.kv_len - B.qo_len
    lo, hi = max(a0, b0), min(A.kv_len, B.kv_len)
    # a row at position p sees keys 0..p only, so it is the same computation in both
    pos = np.arange(lo, hi, dtype=np.int64)
    return (a.qo_indptr[ra] + pos - a0).astype(np.int64), (b.qo_indptr[rb] + pos - b0).astype(np.int64)


def _pool_pages(token_counts, page_size: int, factor: int = 2) -> int:
    need = sum(-(-t // page_size) for t in token_counts)
    return max(64, factor * need)


# --------------------------------------------------------------------------- the five workloads

QWEN3_8B = dict(hq=32, hkv=8, d=128)
QWEN3_4B = dict(hq=32, hkv=8, d=128)
LONG_FP8 = dict(hq=24, hkv=4, d=256)


def _new(name, shapes, page_size, kv_dtype, pool, prompts, batches, desc):
    scale = 1.0 / FP8_DATA_SCALE if kv_dtype == "fp8_e4m3" else 1.0
    return Workload(name=name, num_qo_heads=shapes["hq"], num_kv_heads=shapes["hkv"],
                    head_dim=shapes["d"], page_size=page_size, kv_dtype=kv_dtype,
                    k_scale=scale, v_scale=scale, k_pool=pool.k, v_pool=pool.v,
                    prompts=prompts, batches=batches, description=desc)


def single_extend(seed_base: int = 1000, page_size: int = 16) -> Workload:
    """One 67-token prompt: full prefill vs 64-token cached prefix + 3-token extend.

    The two batches place the prompt's KV in different, seed-shuffled pages.
    """
    s = dict(QWEN3_8B)
    L = 67
    prompts = [draw_prompt(L, s["hq"], s["hkv"], s["d"], "bf16", seed_base + 1)]
    pool = PagePool(64, page_size, s["hkv"], s["d"], "bf16", seed_base + 4)
    full = Request(0, L, L, pool.place(prompts[0], L))
    cached = Request(0, L, 3, pool.place(prompts[0], L))
    batches = {"full": make_batch([full], prompts, page_size),
               "cached": make_batch([cached], prompts, page_size)}
    return _new("single_extend_67", s, page_size, "bf16", pool, prompts, batches,
                "32/8/128 bf16, one 67-token prompt: full prefill vs 3-token extend behind a "
                "64-token cached prefix")


def extend_batch(seed_base: int = 2000, page_size: int = 16, batch: int = 16,
                         prefix: int = 1024, layout: str = "radix") -> Workload:
    """16 requests behind one shared 1024-token prefix, each extending 1-4 tokens (uniform).

    layout "radix": the prefix pages are physically shared by every request (what a prefix
    cache holds); "distinct": every request owns a private copy of the prefix pages.
    Batches: "cached" (the extends), "full" (each prompt's full 1025-1028-token prefill).
    """
    s = dict(QWEN3_8B)
    rng = np.random.default_rng(seed_base + 5)
    tails = [int(t) for t in rng.integers(1, 5, size=batch)]
    base = draw_prompt(prefix, s["hq"], s["hkv"], s["d"], "bf16", seed_base + 1)
    prompts = [extend_prompt(base, t, s["hq"], s["hkv"], s["d"], "bf16", seed_base + 10 + i)
               for i, t in enumerate(tails)]
    lens = [prefix + t for t in tails]
    pool = PagePool(_pool_pages(lens * 2 + [prefix], page_size), page_size, s["hkv"], s["d"],
                    "bf16", seed_base + 4)
    assert prefix % page_size == 0
    if layout == "radix":
        shared = pool.place(base, prefix)
        cached = [Request(i, L, t, pool.place(prompts[i], L, shared))
                  for i, (L, t) in enumerate(zip(lens, tails))]
    elif layout == "distinct":
        cached = [Request(i, L, t, pool.place(prompts[i], L)) for i, (L, t) in enumerate(zip(lens, tails))]
    else:
        raise ValueError(layout)
    full = [Request(i, L, L, pool.place(prompts[i], L)) for i, L in enumerate(lens)]
    batches = {"cached": make_batch(cached, prompts, page_size),
               "full": make_batch(full, prompts, page_size)}
    return _new(f"extend_16x1-4_behind_1024_{layout}", s, page_size, "bf16", pool, prompts,
                batches, f"32/8/128 bf16, {batch} extends of 1-4 tokens behind a shared "
                f"{prefix}-token prefix ({layout} page layout)")


def cold_prefill(seed_base: int = 3000, page_size: int = 16, batch: int = 16,
                         length: int = 1028) -> Workload:
    """16 distinct prompts x 1028 tokens, full causal prefill, no cache hits."""
    s = dict(QWEN3_8B)
    prompts = [draw_prompt(length, s["hq"], s["hkv"], s["d"], "bf16", seed_base + 1 + 10 * i)
               for i in range(batch)]
    pool = PagePool(_pool_pages([length] * batch, page_size), page_size, s["hkv"], s["d"],
                    "bf16", seed_base + 4)
    reqs = [Request(i, length, length, pool.place(prompts[i], length)) for i in range(batch)]
    return _new("cold_prefill_16x1028", s, page_size, "bf16", pool, prompts,
                {"full": make_batch(reqs, prompts, page_size)},
                f"32/8/128 bf16, cold causal prefill of {batch} x {length} tokens")


def mixed_batch(seed_base: int = 4000, page_size: int = 16, prefix: int = 3700,
                  tails=(1, 2, 4, 6, 37, 64, 300)) -> Workload:
    """One 3700-token full prefill plus 7 cached-prefix requests with uncached tails.

    The 231 full pages of the 3700-token prefix are shared; each cached request owns a
    copy of the partial page holding tokens 3696.. (copy-on-write). Batches: "mixed"
    (the full 3700 prefill first, then the 7 tails) and "full" (the 7 full prompts).
    """
    s = dict(QWEN3_4B)
    base = draw_prompt(prefix, s["hq"], s["hkv"], s["d"], "bf16", seed_base + 1)
    prompts = [base] + [extend_prompt(base, t, s["hq"], s["hkv"], s["d"], "bf16",
                                      seed_base + 10 + i) for i, t in enumerate(tails)]
    lens = [prefix] + [prefix + t for t in tails]
    pool = PagePool(_pool_pages(lens * 2, page_size), page_size, s["hkv"], s["d"], "bf16",
                    seed_base + 4)
    base_pages = pool.place(base, prefix)
    n_shared = prefix // page_size
    mixed = [Request(0, prefix, prefix, base_pages)]
    for i, t in enumerate(tails):
        mixed.append(Request(i + 1, prefix + t, t,
                             pool.place(prompts[i + 1], prefix + t, base_pages[:n_shared])))
    full = [Request(i + 1, prefix + t, prefix + t, pool.place(prompts[i + 1], prefix + t))
            for i, t in enumerate(tails)]
    return _new("mixed_3700_plus_7_tails", s, page_size, "bf16", pool, prompts,
                {"mixed": make_batch(mixed, prompts, page_size),
                 "full": make_batch(full, prompts, page_size)},
                "32/8/128 bf16: one 3700-token prefill + 7 cached requests with tails "
                + ", ".join(map(str, tails)))


def long_fp8(seed_base: int = 5000, page_size: int = 16, lengths=(8192, 32768),
                     extend: int = 1024) -> Workload:
    """24/4/256 with an fp8 E4M3 KV cache (N(0,1) x 32, dequant scale 1/32).

    Batches: "prefill_<n>" for each length (single full prefills) and "extend": the last
    ``extend`` tokens of the longest prompt behind its cached prefix, whose page list shares
    the prefix pages of that prompt's own full prefill.
    """
    s = dict(LONG_FP8)
    prompts = [draw_prompt(n, s["hq"], s["hkv"], s["d"], "fp8_e4m3", seed_base + 1 + 10 * i)
               for i, n in enumerate(lengths)]
    pool = PagePool(_pool_pages(list(lengths) + [extend], page_size), page_size, s["hkv"],
                    s["d"], "fp8_e4m3", seed_base + 4)
    batches = {}
    longest = len(lengths) - 1
    pages_of = {}
    for i, n in enumerate(lengths):
        pages_of[i] = pool.place(prompts[i], n)
        batches[f"prefill_{n}"] = make_batch([Request(i, n, n, pages_of[i])], prompts, page_size)
    n = lengths[longest]
    prefix = n - extend
    assert prefix % page_size == 0
    ext_pages = pool.place(prompts[longest], n, pages_of[longest][:prefix // page_size])
    batches["extend"] = make_batch([Request(longest, n, extend, ext_pages)], prompts, page_size)
    return _new("long_fp8_24x4x256", s, page_size, "fp8_e4m3", pool, prompts, batches,
                "24/4/256, fp8 E4M3 KV: prefills of " + ", ".join(map(str, lengths))
                + f" tokens and a {extend}-token extend behind a {prefix}-token prefix")


DECODE_KV_LENS = (8192, 8999, 16384, 24001, 32768, 50000, 65536, 131072)


def decode_batch(seed_base: int = 6000, page_size: int = 16, kv_lens=DECODE_KV_LENS,
                 full_prompts: int = 2) -> Workload:
    """Long-KV decode: one new token per request over 8k-128k cached tokens (32/8/128 bf16).

    Every request owns its pages (distinct prompts). The lengths sit on and between the
    4096-token split boundaries, so rows span 2 to 32 splits. Batches: "decode" (the one-row
    requests) and "full" (the full prefill of the first ``full_prompts`` prompts, placed in
    other pages, whose last rows are the same computations as those decode rows). Only those
    prompts carry queries for every token; the others hold their last token's only.
    """
    s = dict(QWEN3_8B)
    prompts = [draw_prompt(L, s["hq"], s["hkv"], s["d"], "bf16", seed_base + 1 + 10 * i,
                           q_from=0 if i < full_prompts else L - 1)
               for i, L in enumerate(kv_lens)]
    lens = list(kv_lens)
    pool = PagePool(_pool_pages(lens + lens[:full_prompts], page_size), page_size, s["hkv"],
                    s["d"], "bf16", seed_base + 4)
    dec = [Request(i, L, 1, pool.place(prompts[i], L)) for i, L in enumerate(lens)]
    full = [Request(i, L, L, pool.place(prompts[i], L)) for i, L in enumerate(lens[:full_prompts])]
    return _new("decode_8x1_over_8k-128k", s, page_size, "bf16", pool, prompts,
                {"decode": make_batch(dec, prompts, page_size),
                 "full": make_batch(full, prompts, page_size)},
                "32/8/128 bf16: 8 one-token decodes over " + ", ".join(map(str, lens)) + " keys")


def random_workload(seed: int, *, hq: int, hkv: int, d: int, page_size: int, kv_dtype: str,
                    specs, pool_factor: int = 3) -> Workload:
    """Small randomised workload for parity sweeps.

    ``specs`` is a list of (prompt_len, qo_len) pairs, one request each, in one batch
    "batch"; a second batch "full" holds the full prefill of every prompt, placed in other
    pages.
    """
    prompts = [draw_prompt(L, hq, hkv, d, kv_dtype, seed * 101 + i) for i, (L, _) in enumerate(specs)]
    lens = [L for L, _ in specs]
    pool = PagePool(_pool_pages(lens * 2, page_size, pool_factor), page_size, hkv, d, kv_dtype,
                    seed * 101 + 99)
    reqs = [Request(i, L, t, pool.place(prompts[i], L)) for i, (L, t) in enumerate(specs)]
    full = [Request(i, L, L, pool.place(prompts[i], L)) for i, (L, _) in enumerate(specs)]
    return _new(f"random_{seed}", dict(hq=hq, hkv=hkv, d=d), page_size, kv_dtype, pool, prompts,
                {"batch": make_batch(reqs, prompts, page_size),
                 "full": make_batch(full, prompts, page_size)}, "randomised parity workload")
