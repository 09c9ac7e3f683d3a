"""Batch-invariant causal GQA prefill attention over a paged KV cache, for MI355X (gfx950).

Thin Python binding of ``libdpp.so`` (C ABI in ``include/dpp.h``). It only marshals
arguments: every step of the attention runs in the library's HIP kernels. PyTorch provides
device memory and the current stream.

    import deterministic_paged_prefill_amd as dpp
    p = dpp.plan(32, 8, 128, 16, qo_indptr, kv_indptr, kv_last_page_len)   # host int32 arrays
    o, lse = p.run(q, k_pool, v_pool, kv_indices)                           # device tensors

Ragged (contiguous) KV: ``page_size=0``, ``kv_indptr`` in tokens, no ``kv_last_page_len``;
``run(q, k, v)`` with k, v ``[tokens, Hkv, D]`` and no page list.

Importing the package does not load the library; the first call does, and raises
:class:`LibraryNotBuilt` if ``libdpp.so`` is missing (build it with
``python -m deterministic_paged_prefill_amd.build``). There is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

__all__ = ["plan", "Plan", "PlanInfo", "merge_states", "library", "LibraryNotBuilt",
           "DppError", "DppValueError", "DEFAULT_WORKSPACE_CAP", "SPLIT_TOKENS", "tile_shape"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdpp.so")
DEFAULT_WORKSPACE_CAP = 256 << 20
STATIC_SCRATCH_BYTES = 32 << 20  # DPP_STATIC_SCRATCH_BYTES: plans for run_static stay under it
SPLIT_TOKENS = 4096


def tile_shape(head_dim: int) -> tuple:
    """(packed query rows, keys) of one tile: constants of head_dim (see dpp_internal.h)."""
    return {64: (256, 64), 128: (256, 64), 256: (128, 32), 512: (64, 32)}[head_dim]

DPP_OK, DPP_ERR_INVALID, DPP_ERR_SHAPE, DPP_ERR_UNSUPPORTED, DPP_ERR_WORKSPACE, DPP_ERR_HIP = range(6)
RUN_REUSE_UPLOAD = 1
STREAM_HEAD_SPLIT = 2  # dpp_stream_kv: two workgroups per unit split V's head_dim, as the narrow launch does
PLAN_ADAPTIVE_KV_TILE = 1  # comparison mode: NOT batch invariant (see include/dpp.h)
PLAN_PERMUTE_WORK = 2      # test mode: work order shuffled with the seed in bits 16..31
KV_DTYPES = {"bf16": 0, "fp8_e4m3": 1}


class LibraryNotBuilt(ImportError):
    pass


class DppError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class DppValueError(DppError, ValueError):
    """Invalid arguments, shapes, unsupported configs or an undersized workspace."""


class _Config(ctypes.Structure):
    _fields_ = [("num_qo_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("sm_scale", ctypes.c_float),
                ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float)]


class _PlanInfo(ctypes.Structure):
    _fields_ = [("block_m", ctypes.c_int32), ("block_n", ctypes.c_int32),
                ("split_tokens", ctypes.c_int32), ("num_passes", ctypes.c_int32),
                ("num_prefill_items", ctypes.c_int64), ("num_merge_items", ctypes.c_int64),
                ("max_partial_slots", ctypes.c_int64), ("header_bytes", ctypes.c_size_t),
                ("workspace_bytes", ctypes.c_size_t), ("total_q_rows", ctypes.c_int64)]


@dataclass(frozen=True)
class PlanInfo:
    block_m: int
    block_n: int
    split_tokens: int
    num_passes: int
    num_prefill_items: int
    num_merge_items: int
    max_partial_slots: int
    header_bytes: int
    workspace_bytes: int
    total_q_rows: int


_lib = None
EXPORTS = ("dpp_plan_create", "dpp_plan_create_ex", "dpp_plan_workspace_bytes", "dpp_plan_get_info", "dpp_plan_header",
           "dpp_plan_upload", "dpp_plan_destroy", "dpp_run", "dpp_run_static", "dpp_stream_kv",
           "dpp_check_page_table",
           "dpp_merge_states",
           "dpp_last_error", "dpp_status_string", "dpp_abi_version")


def library():
    """Load libdpp.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LibraryNotBuilt(f"{LIB_PATH} is missing; build it with "
                              "`python -m deterministic_paged_prefill_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.dpp_plan_create.restype = ctypes.c_int
    lib.dpp_plan_create.argtypes = [ctypes.POINTER(_Config), i32, vp, vp, vp, sz, ctypes.POINTER(vp)]
    lib.dpp_plan_create_ex.restype = ctypes.c_int
    lib.dpp_plan_create_ex.argtypes = [ctypes.POINTER(_Config), i32, vp, vp, vp, sz, ctypes.c_uint32,
                                       ctypes.POINTER(vp)]
    lib.dpp_plan_workspace_bytes.restype = sz
    lib.dpp_plan_workspace_bytes.argtypes = [vp]
    lib.dpp_plan_get_info.restype = ctypes.c_int
    lib.dpp_plan_get_info.argtypes = [vp, ctypes.POINTER(_PlanInfo)]
    lib.dpp_plan_header.restype = ctypes.c_int
    lib.dpp_plan_header.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(sz)]
    lib.dpp_plan_upload.restype = ctypes.c_int
    lib.dpp_plan_upload.argtypes = [vp, vp, sz, vp]
    lib.dpp_plan_destroy.restype = None
    lib.dpp_plan_destroy.argtypes = [vp]
    lib.dpp_run.restype = ctypes.c_int
    lib.dpp_run.argtypes = [vp, vp, i64, vp, vp, i64, vp, i64, vp, vp, vp, sz, ctypes.c_uint32, vp]
    lib.dpp_run_static.restype = ctypes.c_int
    lib.dpp_run_static.argtypes = [vp, vp, i64, vp, vp, i64, vp, i64, vp, vp, ctypes.c_uint32, vp]
    lib.dpp_stream_kv.restype = ctypes.c_int
    lib.dpp_stream_kv.argtypes = [vp, vp, vp, i64, vp, i64, vp, sz, i32, i32, ctypes.c_uint32, vp]
    lib.dpp_check_page_table.restype = ctypes.c_int
    lib.dpp_check_page_table.argtypes = [vp, vp, i64, i64]
    lib.dpp_merge_states.restype = ctypes.c_int
    lib.dpp_merge_states.argtypes = [vp, vp, i64, i32, i32, i32, vp, vp, vp]
    lib.dpp_last_error.restype = ctypes.c_char_p
    lib.dpp_last_error.argtypes = []
    lib.dpp_status_string.restype = ctypes.c_char_p
    lib.dpp_status_string.argtypes = [ctypes.c_int]
    lib.dpp_abi_version.restype = i32
    lib.dpp_abi_version.argtypes = []
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status == DPP_OK:
        return
    lib = library()
    msg = f"{lib.dpp_status_string(status).decode()}: {lib.dpp_last_error().decode()}"
    if status == DPP_ERR_HIP:
        raise DppError(status, msg)
    raise DppValueError(status, msg)


def _i32(a) -> np.ndarray:
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(a), dtype=np.int32)


def _stream_handle(stream) -> int | None:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


class Plan:
    """Work list of one batch shape; reusable across layers and runs."""

    def __init__(self, handle, cfg: _Config, batch_size: int):
        self._h = handle
        self.cfg = cfg
        self.batch_size = batch_size
        self._ran = False
        info = _PlanInfo()
        _check(library().dpp_plan_get_info(self._h, ctypes.byref(info)))
        self.info = PlanInfo(**{f: getattr(info, f) for f, _ in _PlanInfo._fields_})

    @property
    def workspace_bytes(self) -> int:
        return self.info.workspace_bytes

    def header(self) -> np.ndarray:
        """The int32 work list exactly as run() uploads it."""
        data, nbytes = ctypes.c_void_p(), ctypes.c_size_t()
        _check(library().dpp_plan_header(self._h, ctypes.byref(data), ctypes.byref(nbytes)))
        buf = (ctypes.c_char * nbytes.value).from_address(data.value)
        return np.frombuffer(bytes(buf), dtype=np.int32).copy()

    def new_workspace(self, device="cuda"):
        import torch
        return torch.empty(max(self.workspace_bytes, 256), dtype=torch.uint8, device=device)

    def upload(self, workspace, stream=None) -> None:
        """Copy the work list into ``workspace`` once; later run(..., reuse_upload=True) skip it."""
        _check(library().dpp_plan_upload(self._h, workspace.data_ptr(),
                                         workspace.numel() * workspace.element_size(),
                                         _stream_handle(stream)))
        self._ran = True

    def run(self, q, k_pool, v_pool, kv_indices=None, out=None, lse=None, workspace=None,
            stream=None, reuse_upload: bool = False):
        """Attention of the planned batch. Returns (o bf16 [rows, Hq, D], lse fp32 [rows, Hq]).

        ``reuse_upload=True`` requires an earlier upload()/run() of this plan into the same
        ``workspace`` (nothing else written to its head since)."""
        import torch
        c = self.cfg
        rows = q.shape[0]
        if q.dtype != torch.bfloat16 or q.dim() != 3 or tuple(q.shape[1:]) != (c.num_qo_heads, c.head_dim):
            raise ValueError(f"q must be bf16 [rows, {c.num_qo_heads}, {c.head_dim}], got "
                             f"{q.dtype} {tuple(q.shape)}")
        ragged = c.page_size == 0
        want = (c.num_kv_heads, c.head_dim) if ragged else (c.page_size, c.num_kv_heads, c.head_dim)
        for name, pool in (("k_pool", k_pool), ("v_pool", v_pool)):
            if pool.dim() != len(want) + 1 or tuple(pool.shape[1:]) != want:
                lead = "tokens" if ragged else "num_pages"
                raise ValueError(f"{name} must be [{lead}, {', '.join(map(str, want))}], "
                                 f"got {tuple(pool.shape)}")
            ok = (pool.dtype == torch.bfloat16) if c.kv_dtype == 0 else \
                (pool.dtype in (torch.uint8, torch.float8_e4m3fn))
            if not ok:
                raise ValueError(f"{name} dtype {pool.dtype} does not match the plan's kv dtype")
            if not pool.is_contiguous() or not pool.is_cuda:
                raise ValueError(f"{name} must be a contiguous device tensor")
        if k_pool.shape[0] != v_pool.shape[0]:
            raise ValueError("k_pool and v_pool must have the same number of pages")
        if ragged:
            if kv_indices is not None:
                raise ValueError("ragged KV takes no kv_indices")
        elif kv_indices is None or kv_indices.dtype != torch.int32 or not kv_indices.is_cuda or \
                not kv_indices.is_contiguous():
            raise ValueError("kv_indices must be a contiguous int32 device tensor")
        if not q.is_cuda or not q.is_contiguous():
            raise ValueError("q must be a contiguous device tensor")
        if out is None:
            out = torch.empty_like(q)
        if lse is None:
            lse = torch.empty((rows, c.num_qo_heads), dtype=torch.float32, device=q.device)
        if tuple(out.shape) != tuple(q.shape) or out.dtype != torch.bfloat16 or not out.is_contiguous():
            raise ValueError("out must be a contiguous bf16 tensor shaped like q")
        if tuple(lse.shape) != (rows, c.num_qo_heads) or lse.dtype != torch.float32 or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous fp32 tensor [rows, num_qo_heads]")
        if workspace is None:
            if reuse_upload:
                raise ValueError("reuse_upload needs the workspace the plan was uploaded to")
            workspace = self.new_workspace(q.device)
            if stream is not None and _stream_handle(stream) != torch.cuda.current_stream(q.device).cuda_stream:
                # allocated on the current stream, used on `stream`: keep the caching
                # allocator from handing it out again before that stream's kernels are done
                workspace.record_stream(stream if isinstance(stream, torch.cuda.Stream)
                                        else torch.cuda.ExternalStream(_stream_handle(stream)))
        status = library().dpp_run(self._h, q.data_ptr(), rows, k_pool.data_ptr(), v_pool.data_ptr(),
                                   k_pool.shape[0], None if ragged else kv_indices.data_ptr(),
                                   0 if ragged else kv_indices.numel(), out.data_ptr(),
                                   lse.data_ptr(), workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(),
                                   RUN_REUSE_UPLOAD if reuse_upload else 0,
                                   _stream_handle(stream))
        _check(status)
        self._ran = True
        return out, lse

    def check_page_table(self, kv_indices, num_pages: int) -> None:
        """Host check that every page id the plan's requests read lies in [0, num_pages)
        (dpp_check_page_table); raises DppValueError naming the first bad (request, page)."""
        kvi = _i32(kv_indices)
        _check(library().dpp_check_page_table(self._h, kvi.ctypes.data if kvi.size else None,
                                              kvi.size, int(num_pages)))

    def close(self) -> None:
        if self._h is not None:
            if self._ran:
                import torch
                torch.cuda.synchronize()  # the upload reads the plan's pinned buffer
            library().dpp_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def plan(num_qo_heads: int, num_kv_heads: int, head_dim: int, page_size: int, qo_indptr,
         kv_indptr, kv_last_page_len=None, *, kv_dtype: str = "bf16", sm_scale: float | None = None,
         k_scale: float = 1.0, v_scale: float = 1.0,
         workspace_cap: int = DEFAULT_WORKSPACE_CAP, adaptive_kv_tile: bool = False,
         permute_seed: int | None = None) -> Plan:
    """Plan one batch from host copies of its index arrays (no GPU work).

    ``adaptive_kv_tile=True`` is the comparison mode that picks the KV tile from the batch
    (dpp_plan_create_ex with DPP_PLAN_ADAPTIVE_KV_TILE): NOT batch invariant.
    ``permute_seed`` (test mode, DPP_PLAN_PERMUTE_WORK) shuffles the order of the work in every
    pass; the results stay bit-identical."""
    if kv_dtype not in KV_DTYPES:
        raise ValueError(f"kv_dtype must be one of {sorted(KV_DTYPES)}")
    qo, kvp = _i32(qo_indptr), _i32(kv_indptr)
    batch = len(qo) - 1
    if kv_last_page_len is None:
        if page_size != 0:
            raise ValueError("a paged layout needs kv_last_page_len")
        kv_last_page_len = np.zeros(max(batch, 0), dtype=np.int32)  # ignored for ragged KV
    last = _i32(kv_last_page_len)
    if batch < 0 or len(kvp) != batch + 1 or len(last) != batch:
        raise ValueError("need qo_indptr[B+1], kv_indptr[B+1], kv_last_page_len[B]")
    cfg = _Config(num_qo_heads, num_kv_heads, head_dim, page_size, KV_DTYPES[kv_dtype],
                  0.0 if sm_scale is None else float(sm_scale), float(k_scale), float(v_scale))
    h = ctypes.c_void_p()
    last_ptr = last.ctypes.data if batch > 0 else None
    _check(library().dpp_plan_create_ex(ctypes.byref(cfg), batch, qo.ctypes.data, kvp.ctypes.data,
                                        last_ptr, int(workspace_cap),
                                        (PLAN_ADAPTIVE_KV_TILE if adaptive_kv_tile else 0) |
                                        (0 if permute_seed is None else
                                         PLAN_PERMUTE_WORK | ((int(permute_seed) & 0xFFFF) << 16)),
                                        ctypes.byref(h)))
    return Plan(h, cfg, batch)


def merge_states(o_partial, lse_partial, out=None, lse=None, stream=None):
    """Combine partial states o_partial [R, S, H, D] fp32, lse_partial [R, S, H] fp32 (natural
    log) into (o bf16 [R, H, D], lse fp32 [R, H]) on the GPU."""
    import torch
    if o_partial.dtype != torch.float32 or lse_partial.dtype != torch.float32:
        raise ValueError("o_partial and lse_partial must be float32")
    if o_partial.dim() != 4 or tuple(lse_partial.shape) != tuple(o_partial.shape[:3]):
        raise ValueError("o_partial must be [R, S, H, D] and lse_partial [R, S, H]")
    if not (o_partial.is_cuda and lse_partial.is_cuda and o_partial.is_contiguous() and lse_partial.is_contiguous()):
        raise ValueError("partials must be contiguous device tensors")
    R, S, H, D = o_partial.shape
    if out is None:
        out = torch.empty((R, H, D), dtype=torch.bfloat16, device=o_partial.device)
    if lse is None:
        lse = torch.empty((R, H), dtype=torch.float32, device=o_partial.device)
    _check(library().dpp_merge_states(o_partial.data_ptr(), lse_partial.data_ptr(), R, S, H, D,
                                      out.data_ptr(), lse.data_ptr(), _stream_handle(stream)))
    return out, lse

