"""Thin ctypes binding of the LOCKS C ABI (include/locks.h).

Argument marshalling only: tensors are passed as device pointers plus sizes,
the current torch stream is passed as the HIP stream, and every computation
runs in the HIP library. Importing this module raises if the library has not
been built (python -m kv_cache_page_amd.build_lib).
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblocks_hip.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(
        f"LOCKS HIP library not found at {_LIB_PATH}; build it with "
        "`python -m kv_cache_page_amd.build_lib` (hipcc, gfx950)")
_lib = ctypes.CDLL(_LIB_PATH)

OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED = -2
ERR_WORKSPACE = -3
ERR_HIP = -4
STEP_DEFER_BUILD = 1      # LOCKS_STEP_DEFER_BUILD

ENTRY_POINTS = (
    "locks_status_string", "locks_summary_slot_bytes", "locks_summary_slot_stride",
    "locks_workspace_bytes", "locks_build", "locks_build_filled", "locks_append_kv",
    "locks_score_select", "locks_score_pages", "locks_select_pages", "locks_sparse_attn",
    "locks_decode_step", "locks_decode_step_noalloc", "locks_host_pool_alloc",
    "locks_host_pool_free",
)
NOALLOC_SCRATCH_BYTES = 16 << 20   # LOCKS_NOALLOC_SCRATCH_BYTES


MERGE_SHARE, MERGE_MAX, MERGE_MASS, MERGE_PER_HEAD = 0, 1, 2, 3   # LOCKS_MERGE_*
MERGE_RULES = {"share": MERGE_SHARE, "max": MERGE_MAX, "mass": MERGE_MASS,
               "per_head": MERGE_PER_HEAD}


class Dims(ctypes.Structure):
    """locks_dims: head_dim, page_size, rank, num_kv_heads, group_size,
    basis_bits (0 = 4), merge_rule (LOCKS_MERGE_*; a name of MERGE_RULES is
    accepted too)."""
    _fields_ = [("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("rank", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("basis_bits", ctypes.c_int32),
                ("merge_rule", ctypes.c_int32)]

    def __init__(self, num_kv_heads, group_size, rank=8, head_dim=128, page_size=16,
                 basis_bits=0, merge_rule=MERGE_SHARE):
        if isinstance(merge_rule, str):
            merge_rule = MERGE_RULES[merge_rule]
        super().__init__(head_dim, page_size, rank, num_kv_heads, group_size, basis_bits,
                         merge_rule)


class LocksError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_pd = ctypes.POINTER(Dims)


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_status_string = _sig("locks_status_string", ctypes.c_char_p, [ctypes.c_int])
_slot_bytes = _sig("locks_summary_slot_bytes", _sz, [_pd])
_slot_stride = _sig("locks_summary_slot_stride", _sz, [_pd])
_ws_bytes = _sig("locks_workspace_bytes", _sz, [_pd, _i32, _i32, _i32])
_build = _sig("locks_build", ctypes.c_int, [_pd, _vp, _i64, _vp, _i32, _vp, _vp])
_build_filled = _sig("locks_build_filled", ctypes.c_int,
                     [_pd, _vp, _i64, _vp, _vp, _i32, _i32, _vp, _vp])
_append = _sig("locks_append_kv", ctypes.c_int,
               [_pd, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _i32, _i32, _vp])
_score_select = _sig("locks_score_select", ctypes.c_int,
                     [_pd, _vp, _vp, _i64, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp,
                      _vp, _sz, _vp])
_score_pages = _sig("locks_score_pages", ctypes.c_int,
                    [_pd, _vp, _vp, _i64, _vp, _vp, _i32, _i32, _vp, _vp])
_select_pages = _sig("locks_select_pages", ctypes.c_int,
                     [_pd, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _sz, _vp])
_sparse_attn = _sig("locks_sparse_attn", ctypes.c_int,
                    [_pd, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp,
                     _vp, _sz, _vp])
_u32 = ctypes.c_uint32
_decode_step = _sig("locks_decode_step", ctypes.c_int,
                    [_pd, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _i32, _i32,
                     _i32, _vp, _vp, _vp, _vp, _u32, _vp, _sz, _vp])

_decode_step_noalloc = _sig("locks_decode_step_noalloc", ctypes.c_int,
                            [_pd, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _i32,
                             _i32, _i32, _vp, _vp, _vp, _vp, _u32, _vp])


_host_alloc = _sig("locks_host_pool_alloc", ctypes.c_int,
                   [_sz, ctypes.POINTER(_vp), ctypes.POINTER(_vp)])
_host_free = _sig("locks_host_pool_free", ctypes.c_int, [_vp])


def status_string(status):
    return _status_string(int(status)).decode()


def slot_bytes(dims):
    return int(_slot_bytes(ctypes.byref(dims)))


def slot_stride(dims):
    return int(_slot_stride(ctypes.byref(dims)))


def workspace_bytes(dims, num_seqs, max_pages, max_budget):
    return int(_ws_bytes(ctypes.byref(dims), num_seqs, max_pages, max_budget))


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

class HostPool:
    """A K or V pool in pinned, device-mapped host memory (locks_host_pool_alloc):
    `host` is a CPU tensor of the given shape over that memory, and entry
    points given the HostPool pass its device address to the kernels."""

    def __init__(self, shape, dtype=torch.bfloat16):
        self.shape = torch.Size(shape)
        self.dtype = dtype
        nbytes = self.shape.numel() * torch.tensor([], dtype=dtype).element_size()
        hp, dp = _vp(), _vp()
        _check(_host_alloc(nbytes, ctypes.byref(hp), ctypes.byref(dp)), "locks_host_pool_alloc")
        self._host_ptr, self.device_ptr = hp.value, dp.value
        buf = (ctypes.c_uint8 * nbytes).from_address(self._host_ptr)
        self.host = torch.frombuffer(buf, dtype=torch.uint8).view(dtype).view(self.shape)

    def is_contiguous(self):
        return True

    def free(self):
        """Release the memory (no enqueued work may still use it)."""
        if self._host_ptr:
            self.host = None
            _check(_host_free(self._host_ptr), "locks_host_pool_free")
            self._host_ptr = self.device_ptr = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if isinstance(t, HostPool):
        if dtype is not None and t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        if t.device_ptr is None:
            raise ValueError(f"{name}: host pool already freed")
        return t.device_ptr
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if isinstance(stream, torch.cuda.Stream) else int(stream)


def _check(status, where):
    if status != OK:
        raise LocksError(status, where)


def alloc_summaries(dims, num_blocks, device):
    """Zeroed summary pool uint8 [num_blocks][H][slot_stride]."""
    return torch.zeros(num_blocks, dims.num_kv_heads, slot_stride(dims), dtype=torch.uint8,
                       device=device)


def alloc_workspace(dims, num_seqs, max_pages, max_budget, device):
    """Workspace of locks_workspace_bytes bytes (no initialisation needed)."""
    return torch.empty(max(workspace_bytes(dims, num_seqs, max_pages, max_budget), 1),
                       dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------
# entry points (names follow include/locks.h)
# ---------------------------------------------------------------------------

def build(dims, k_pool, block_ids, summaries, stream=None):
    """locks_build over the int32 block ids in `block_ids` (device)."""
    st = _build(ctypes.byref(dims), _ptr(k_pool, torch.bfloat16, "k_pool"), k_pool.shape[0],
                _ptr(block_ids, torch.int32, "block_ids"), block_ids.numel(),
                _ptr(summaries, torch.uint8, "summaries"), _stream(stream))
    _check(st, "locks_build")


def build_filled(dims, k_pool, block_table, seq_lens, summaries, stream=None):
    st = _build_filled(ctypes.byref(dims), _ptr(k_pool, torch.bfloat16, "k_pool"),
                       k_pool.shape[0], _ptr(block_table, torch.int32, "block_table"),
                       _ptr(seq_lens, torch.int32, "seq_lens"), seq_lens.numel(),
                       block_table.shape[1], _ptr(summaries, torch.uint8, "summaries"),
                       _stream(stream))
    _check(st, "locks_build_filled")


def append_kv(dims, k_new, v_new, k_pool, v_pool, block_table, seq_lens, stream=None):
    st = _append(ctypes.byref(dims), _ptr(k_new, torch.bfloat16, "k_new"),
                 _ptr(v_new, torch.bfloat16, "v_new"), _ptr(k_pool, torch.bfloat16, "k_pool"),
                 _ptr(v_pool, torch.bfloat16, "v_pool"), k_pool.shape[0],
                 _ptr(block_table, torch.int32, "block_table"),
                 _ptr(seq_lens, torch.int32, "seq_lens"), seq_lens.numel(),
                 block_table.shape[1], _stream(stream))
    _check(st, "locks_append_kv")


def score_select(dims, q, summaries, block_table, seq_lens, budgets, max_budget, sel_pages,
                 sel_count, workspace, scores_out=None, num_blocks=None, stream=None):
    nb = summaries.shape[0] if num_blocks is None else num_blocks
    st = _score_select(ctypes.byref(dims), _ptr(q, torch.bfloat16, "q"),
                       _ptr(summaries, torch.uint8, "summaries"), nb,
                       _ptr(block_table, torch.int32, "block_table"),
                       _ptr(seq_lens, torch.int32, "seq_lens"), _ptr(budgets, torch.int32, "budgets"),
                       seq_lens.numel(), block_table.shape[1], max_budget,
                       _ptr(sel_pages, torch.int32, "sel_pages"),
                       _ptr(sel_count, torch.int32, "sel_count"),
                       _ptr(scores_out, torch.float32, "scores_out"),
                       _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                       _stream(stream))
    _check(st, "locks_score_select")


def score_pages(dims, q, summaries, block_table, seq_lens, scores, num_blocks=None, stream=None):
    nb = summaries.shape[0] if num_blocks is None else num_blocks
    st = _score_pages(ctypes.byref(dims), _ptr(q, torch.bfloat16, "q"),
                      _ptr(summaries, torch.uint8, "summaries"), nb,
                      _ptr(block_table, torch.int32, "block_table"),
                      _ptr(seq_lens, torch.int32, "seq_lens"), seq_lens.numel(),
                      block_table.shape[1], _ptr(scores, torch.float32, "scores"), _stream(stream))
    _check(st, "locks_score_pages")


def select_pages(dims, scores, seq_lens, budgets, max_pages, max_budget, sel_pages, sel_count,
                 workspace, stream=None):
    st = _select_pages(ctypes.byref(dims), _ptr(scores, torch.float32, "scores"),
                       _ptr(seq_lens, torch.int32, "seq_lens"), _ptr(budgets, torch.int32, "budgets"),
                       seq_lens.numel(), max_pages, max_budget,
                       _ptr(sel_pages, torch.int32, "sel_pages"),
                       _ptr(sel_count, torch.int32, "sel_count"),
                       _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream))
    _check(st, "locks_select_pages")


def sparse_attn(dims, q, k_pool, v_pool, block_table, seq_lens, sel_pages, sel_count, max_budget,
                out, workspace, lse_out=None, stream=None):
    st = _sparse_attn(ctypes.byref(dims), _ptr(q, torch.bfloat16, "q"),
                      _ptr(k_pool, torch.bfloat16, "k_pool"), _ptr(v_pool, torch.bfloat16, "v_pool"),
                      k_pool.shape[0], _ptr(block_table, torch.int32, "block_table"),
                      _ptr(seq_lens, torch.int32, "seq_lens"),
                      _ptr(sel_pages, torch.int32, "sel_pages"),
                      _ptr(sel_count, torch.int32, "sel_count"), seq_lens.numel(),
                      block_table.shape[1], max_budget, _ptr(out, torch.float32, "out"),
                      _ptr(lse_out, torch.float32, "lse_out"),
                      _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                      _stream(stream))
    _check(st, "locks_sparse_attn")


def decode_step(dims, q, k_new, v_new, k_pool, v_pool, summaries, block_table, seq_lens, budgets,
                max_budget, out, workspace, lse_out=None, sel_pages=None, sel_count=None,
                seq_lens_host=None, defer_build=False, stream=None):
    """locks_decode_step. seq_lens_host: optional CPU int32 tensor equal to
    seq_lens (lets the call skip the page-build launch when no page fills).
    defer_build: LOCKS_STEP_DEFER_BUILD (the caller then runs build_filled)."""
    if seq_lens_host is not None:
        if seq_lens_host.device.type != "cpu":
            raise ValueError("seq_lens_host must be a CPU tensor")
        if seq_lens_host.numel() != seq_lens.numel():
            raise ValueError("seq_lens_host must have one entry per sequence")
    st = _decode_step(ctypes.byref(dims), _ptr(q, torch.bfloat16, "q"),
                      _ptr(k_new, torch.bfloat16, "k_new"), _ptr(v_new, torch.bfloat16, "v_new"),
                      _ptr(k_pool, torch.bfloat16, "k_pool"), _ptr(v_pool, torch.bfloat16, "v_pool"),
                      _ptr(summaries, torch.uint8, "summaries"), k_pool.shape[0],
                      _ptr(block_table, torch.int32, "block_table"),
                      _ptr(seq_lens, torch.int32, "seq_lens"),
                      _ptr(seq_lens_host, torch.int32, "seq_lens_host"),
                      _ptr(budgets, torch.int32, "budgets"), seq_lens.numel(),
                      block_table.shape[1], max_budget, _ptr(out, torch.float32, "out"),
                      _ptr(lse_out, torch.float32, "lse_out"),
                      _ptr(sel_pages, torch.int32, "sel_pages"),
                      _ptr(sel_count, torch.int32, "sel_count"),
                      STEP_DEFER_BUILD if defer_build else 0,
                      _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                      _stream(stream))
    _check(st, "locks_decode_step")


def decode_step_noalloc(dims, q, k_new, v_new, k_pool, v_pool, summaries, block_table, seq_lens,
                        budgets, max_budget, out, lse_out=None, sel_pages=None, sel_count=None,
                        seq_lens_host=None, defer_build=False, stream=None):
    """locks_decode_step_noalloc: decode_step on the library's built-in
    per-device scratch (no workspace argument, nothing allocated)."""
    if seq_lens_host is not None:
        if seq_lens_host.device.type != "cpu":
            raise ValueError("seq_lens_host must be a CPU tensor")
        if seq_lens_host.numel() != seq_lens.numel():
            raise ValueError("seq_lens_host must have one entry per sequence")
    st = _decode_step_noalloc(
        ctypes.byref(dims), _ptr(q, torch.bfloat16, "q"), _ptr(k_new, torch.bfloat16, "k_new"),
        _ptr(v_new, torch.bfloat16, "v_new"), _ptr(k_pool, torch.bfloat16, "k_pool"),
        _ptr(v_pool, torch.bfloat16, "v_pool"), _ptr(summaries, torch.uint8, "summaries"),
        k_pool.shape[0], _ptr(block_table, torch.int32, "block_table"),
        _ptr(seq_lens, torch.int32, "seq_lens"), _ptr(seq_lens_host, torch.int32, "seq_lens_host"),
        _ptr(budgets, torch.int32, "budgets"), seq_lens.numel(), block_table.shape[1], max_budget,
        _ptr(out, torch.float32, "out"), _ptr(lse_out, torch.float32, "lse_out"),
        _ptr(sel_pages, torch.int32, "sel_pages"), _ptr(sel_count, torch.int32, "sel_count"),
        STEP_DEFER_BUILD if defer_build else 0, _stream(stream))
    _check(st, "locks_decode_step_noalloc")


def selection_heads(dims):
    """Rows of the per-head arrays (sel_pages, sel_count, page scores): the KV
    heads, or every query head under LOCKS_MERGE_PER_HEAD."""
    if dims.merge_rule == MERGE_PER_HEAD:
        return dims.num_kv_heads * dims.group_size
    return dims.num_kv_heads


class Decoder:
    """Holds the per-layer output buffers and workspace of one decode step and
    calls score_select then sparse_attn on the current stream."""

    def __init__(self, dims, num_seqs, max_pages, max_budget, device):
        self.dims, self.max_budget = dims, max_budget
        H, G = dims.num_kv_heads, dims.group_size
        self.sel = torch.empty(num_seqs, selection_heads(dims), max_budget, dtype=torch.int32,
                               device=device)
        self.cnt = torch.empty(num_seqs, selection_heads(dims), dtype=torch.int32, device=device)
        self.out = torch.empty(num_seqs, H * G, dims.head_dim, dtype=torch.float32, device=device)
        self.lse = torch.empty(num_seqs, H * G, dtype=torch.float32, device=device)
        self.ws = alloc_workspace(dims, num_seqs, max_pages, max_budget, device)

    def step(self, q, summaries, k_pool, v_pool, block_table, seq_lens, budgets, stream=None,
             scores_out=None):
        score_select(self.dims, q, summaries, block_table, seq_lens, budgets, self.max_budget,
                     self.sel, self.cnt, self.ws, scores_out=scores_out, stream=stream)
        sparse_attn(self.dims, q, k_pool, v_pool, block_table, seq_lens, self.sel, self.cnt,
                    self.max_budget, self.out, self.ws, lse_out=self.lse, stream=stream)
        return self.out

    def decode(self, q, k_new, v_new, summaries, k_pool, v_pool, block_table, seq_lens, budgets,
               seq_lens_host=None, stream=None):
        """One fused decode step (append, build of filled pages, score,
        select, attend) through locks_decode_step."""
        decode_step(self.dims, q, k_new, v_new, k_pool, v_pool, summaries, block_table, seq_lens,
                    budgets, self.max_budget, self.out, self.ws, lse_out=self.lse,
                    sel_pages=self.sel, sel_count=self.cnt, seq_lens_host=seq_lens_host,
                    stream=stream)
        return self.out
