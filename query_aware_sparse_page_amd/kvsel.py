"""ctypes binding of libkvsel.so (the C ABI in include/kvsel.h).

Argument marshalling only: these wrappers check devices / dtypes / contiguity, allocate outputs
and workspaces with torch when the caller does not pass them, and hand raw device pointers plus
torch's current HIP stream to the library. Every step of the computation runs in the library's
HIP kernels; there is no fallback path. A missing library raises ``KvselError``.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvsel.so")

KVSEL_F32 = 0
KVSEL_BF16 = 1
KVSEL_FP8_E4M3 = 2
KVSEL_OP_SCORE_TOPK = 1
KVSEL_OP_ATTENTION = 2
KVSEL_OP_SELECT_ATTEND = 3
KVSEL_OP_SPECULATIVE_STEP = 4
KVSEL_SCORE_REFRESH_TAIL = 1
KVSEL_CHECK_SEQ_LEN = 1
KVSEL_CHECK_PAGE_ID = 2
KVSEL_CHECK_SELECTION = 4
KVSEL_CHECK_NO_FREE_PAGE = 8
KVSEL_CHECK_PAGE_FILL = 16
KVSEL_ERR_SCRATCH = 6
KVSEL_STATIC_SCRATCH_BYTES = 8 << 20  # the library's per-GPU scratch (kvsel_select_attend_static)

c_i32 = ctypes.c_int32
c_vp = ctypes.c_void_p


class KvselError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class PagedKVDesc(ctypes.Structure):
    _fields_ = [
        ("dtype", c_i32), ("batch", c_i32), ("num_q_heads", c_i32), ("num_kv_heads", c_i32),
        ("head_dim", c_i32), ("page_size", c_i32), ("num_phys_pages", c_i32),
        ("max_pages_per_seq", c_i32), ("k_pool", c_vp), ("v_pool", c_vp), ("page_table", c_vp),
        ("seq_lens", c_vp), ("max_seq_len", c_i32), ("k_scale", c_vp), ("v_scale", c_vp),
        ("page_fill", c_vp),
    ]


class FreePagesDesc(ctypes.Structure):
    _fields_ = [("ids", c_vp), ("count", c_vp), ("capacity", c_i32)]


class RopeDesc(ctypes.Structure):
    _fields_ = [("cos", c_vp), ("sin", c_vp), ("page_row", c_vp), ("n_rows", c_i32),
                ("row_step", c_i32), ("per_sequence", c_i32)]


class ReuseDesc(ctypes.Structure):
    _fields_ = [
        ("q_prev", c_vp), ("prev_idx", c_vp), ("prev_cnt", c_vp), ("tau", ctypes.c_double),
        ("first_step", c_i32), ("used_idx", c_vp), ("used_cnt", c_vp), ("corrected", c_vp),
        ("similarity", c_vp),
    ]


EXPORTS = {
    "kvsel_abi_version": (c_i32, []),
    "kvsel_status_str": (ctypes.c_char_p, [c_i32]),
    "kvsel_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(PagedKVDesc), c_i32, c_i32, c_i32]),
    "kvsel_step_pages_per_split": (c_i32, [ctypes.POINTER(PagedKVDesc), c_i32]),
    "kvsel_build_summaries": (c_i32, [ctypes.POINTER(PagedKVDesc), ctypes.POINTER(RopeDesc), c_i32,
                                      c_vp, c_vp]),
    "kvsel_score_topk": (c_i32, [ctypes.POINTER(PagedKVDesc), ctypes.POINTER(RopeDesc), c_vp, c_vp,
                                 c_i32, c_i32, c_vp, c_vp, c_vp, ctypes.POINTER(ReuseDesc), c_vp,
                                 ctypes.c_size_t, c_vp]),
    "kvsel_sparse_decode_attn": (c_i32, [ctypes.POINTER(PagedKVDesc), ctypes.POINTER(RopeDesc), c_vp,
                                         c_vp, c_vp, c_i32, ctypes.c_float, c_i32, c_vp, c_vp, c_vp,
                                         ctypes.c_size_t, c_vp]),
    "kvsel_select_attend": (c_i32, [ctypes.POINTER(PagedKVDesc), ctypes.POINTER(RopeDesc), c_vp, c_vp,
                                    c_i32, c_i32, ctypes.c_float, c_vp, c_vp, c_vp, c_vp, c_vp,
                                    ctypes.c_size_t, c_vp]),
    "kvsel_select_attend_static": (c_i32, [ctypes.POINTER(PagedKVDesc), ctypes.POINTER(RopeDesc),
                                           c_vp, c_vp, c_i32, c_i32, ctypes.c_float, c_vp, c_vp,
                                           c_vp, c_vp, c_vp]),
    "kvsel_speculative_step": (c_i32, [ctypes.POINTER(PagedKVDesc), ctypes.POINTER(RopeDesc), c_vp,
                                       c_vp, c_i32, c_i32, ctypes.c_float,
                                       ctypes.POINTER(ReuseDesc), c_vp, c_vp, c_vp, c_vp, c_vp,
                                       ctypes.c_size_t, c_vp]),
    "kvsel_quantize_pages": (c_i32, [ctypes.POINTER(PagedKVDesc), c_vp, c_vp, c_vp, c_vp, c_vp]),
    "kvsel_append_kv": (c_i32, [ctypes.POINTER(PagedKVDesc), c_vp, c_vp, c_vp, c_vp,
                                ctypes.POINTER(FreePagesDesc), c_vp, c_vp]),
    "kvsel_check_inputs": (c_i32, [ctypes.POINTER(PagedKVDesc), c_vp, c_vp, c_i32, c_vp, c_vp]),
    "kvsel_gather_probe": (c_i32, [c_vp, c_i32, c_i32, c_vp, c_vp]),
    "kvsel_rope_table": (c_i32, [ctypes.c_double, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp]),
    "kvsel_rope_shift": (c_i32, [ctypes.POINTER(PagedKVDesc), ctypes.POINTER(RopeDesc), c_vp, c_vp]),
}

_lib = None


ABI_VERSION = 7  # KVSEL_ABI_VERSION of include/kvsel.h


def lib() -> ctypes.CDLL:
    """Load libkvsel.so (once) and declare its signatures."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise KvselError(-1, f"{LIB_PATH} is not built; run "
                                 "`python -m query_aware_sparse_page_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        if handle.kvsel_abi_version() != ABI_VERSION:  # the descriptor layouts above
            raise KvselError(-1, f"{LIB_PATH} has ABI {handle.kvsel_abi_version()}, this binding "
                                 f"{ABI_VERSION}; rebuild it")
        _lib = handle
    return _lib


def status_str(status: int) -> str:
    return lib().kvsel_status_str(status).decode()


def _check(status: int) -> None:
    if status != 0:
        raise KvselError(status, status_str(status))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _check_summ(kv: "PagedKV", summ: torch.Tensor) -> None:
    _dev(summ, "summ", kv.act_dtype)
    shape = (kv.batch, kv.num_kv_heads, int(kv.page_table.shape[1]), 2, kv.head_dim)
    if tuple(summ.shape) != shape:
        raise ValueError(f"summ must be {shape} (sequence-major), got {tuple(summ.shape)}")


def _elem_code(dtype: torch.dtype) -> int:
    if dtype == torch.float32:
        return KVSEL_F32
    if dtype == torch.bfloat16:
        return KVSEL_BF16
    if dtype == torch.uint8:
        return KVSEL_FP8_E4M3
    raise ValueError(f"unsupported element type {dtype}")


def device_v_layout(v_pool: torch.Tensor) -> torch.Tensor:
    """Values in the library's page layout: [Npp][Hkv][P][D] (token-major) -> [Npp][Hkv][D][P]
    (channel-major pages)."""
    return v_pool.transpose(-1, -2).contiguous()


@dataclass
class PagedKV:
    """Device tensors of one paged KV cache: k_pool [Npp][Hkv][P][D] (token-major pages),
    v_pool [Npp][Hkv][D][P] (channel-major pages, see ``device_v_layout``), page_table int32
    [B][max_pages], seq_lens int32 [B]. ``max_seq_len`` (host int, 0 = the table width) bounds every
    length so that launches follow the live pages rather than the table width."""

    k_pool: torch.Tensor
    v_pool: Optional[torch.Tensor]
    page_table: torch.Tensor
    seq_lens: torch.Tensor
    num_q_heads: int
    max_seq_len: int = 0
    k_scale: Optional[torch.Tensor] = None  # fp8 pools (uint8 codes): [Npp][Hkv] fp32
    v_scale: Optional[torch.Tensor] = None
    page_fill: Optional[torch.Tensor] = None  # int32 [Npp] valid slots per page (composition)

    @property
    def is_fp8(self) -> bool:
        return self.k_pool.dtype == torch.uint8

    @property
    def act_dtype(self) -> torch.dtype:
        """Element type of queries, summaries and outputs (bf16 for an fp8 cache)."""
        return torch.bfloat16 if self.is_fp8 else self.k_pool.dtype

    def desc(self) -> PagedKVDesc:
        _dev(self.k_pool, "k_pool")
        if self.v_pool is not None:
            _dev(self.v_pool, "v_pool", self.k_pool.dtype)
            if self.is_fp8 and self.v_scale is None:
                raise ValueError("an fp8 value pool needs v_scale")
            Npp, Hkv, P, D = self.k_pool.shape
            if tuple(self.v_pool.shape) != (Npp, Hkv, D, P):
                raise ValueError(f"v_pool must be [Npp][Hkv][D][P] = {(Npp, Hkv, D, P)}, got "
                                 f"{tuple(self.v_pool.shape)}")
        _dev(self.page_table, "page_table", torch.int32)
        _dev(self.seq_lens, "seq_lens", torch.int32)
        Npp, Hkv, P, D = self.k_pool.shape
        scales = [None, None]
        if self.is_fp8:
            for i, (t, name) in enumerate(((self.k_scale, "k_scale"), (self.v_scale, "v_scale"))):
                if t is None:
                    continue
                _dev(t, name, torch.float32)
                if tuple(t.shape) != (Npp, Hkv):
                    raise ValueError(f"{name} must be [Npp][Hkv] = {(Npp, Hkv)}")
                scales[i] = t.data_ptr()
            if scales[0] is None:
                raise ValueError("an fp8 key pool needs k_scale")
        fill = None
        if self.page_fill is not None:
            _dev(self.page_fill, "page_fill", torch.int32)
            if tuple(self.page_fill.shape) != (Npp,):
                raise ValueError(f"page_fill must be int32 [Npp] = [{Npp}]")
            fill = self.page_fill.data_ptr()
        B, maxp = self.page_table.shape
        return PagedKVDesc(_elem_code(self.k_pool.dtype), B, self.num_q_heads, Hkv, D, P, Npp, maxp,
                           self.k_pool.data_ptr(),
                           self.v_pool.data_ptr() if self.v_pool is not None else None,
                           self.page_table.data_ptr(), self.seq_lens.data_ptr(),
                           int(self.max_seq_len), scales[0], scales[1], fill)

    @property
    def batch(self) -> int:
        return int(self.page_table.shape[0])

    @property
    def num_kv_heads(self) -> int:
        return int(self.k_pool.shape[1])

    @property
    def head_dim(self) -> int:
        return int(self.k_pool.shape[3])

    @property
    def device(self) -> torch.device:
        return self.k_pool.device


@dataclass
class Rope:
    """Rotary table (fp32 [n_rows][D/2] cos and sin) and the first table row of each page: int32
    [Npp] by physical page, or, with ``per_sequence``, int32 [B][max_pages] by (sequence, logical
    page), so that sequences sharing pages can place them at different positions."""

    cos: torch.Tensor
    sin: torch.Tensor
    page_row: torch.Tensor
    row_step: int = 0
    per_sequence: bool = False

    def desc(self) -> RopeDesc:
        _dev(self.cos, "cos", torch.float32)
        _dev(self.sin, "sin", torch.float32)
        _dev(self.page_row, "page_row", torch.int32)
        return RopeDesc(self.cos.data_ptr(), self.sin.data_ptr(), self.page_row.data_ptr(),
                        int(self.cos.shape[0]), int(self.row_step), int(bool(self.per_sequence)))


def _rope_ptr(rope: Optional[Rope]):
    return None if rope is None else ctypes.byref(rope.desc())


def workspace_bytes(kv: PagedKV, k: int, op: int, pages_per_split: int = 0) -> int:
    return int(lib().kvsel_workspace_bytes(ctypes.byref(kv.desc()), k, op, pages_per_split))


def step_pages_per_split(kv: PagedKV, k: int) -> int:
    """Pages per split at which select_attend, select_attend_static and speculative_step run their
    attention (they equal sparse_decode_attn at this pages_per_split, bit for bit)."""
    d = kv.desc()
    n = lib().kvsel_step_pages_per_split(ctypes.byref(d), int(k))
    if n <= 0:
        raise KvselError(-1, "no attention split for this descriptor and k")
    return int(n)


def new_workspace(kv: PagedKV, k: int, op: int, pages_per_split: int = 0) -> torch.Tensor:
    """A zero-filled workspace for ``op`` (the library leaves its counters zero after each
    call, so the buffer can be reused by later calls on the same stream)."""
    need = workspace_bytes(kv, k, op, pages_per_split)
    return torch.zeros(max(need, 1), dtype=torch.uint8, device=kv.device)


def _workspace(kv: PagedKV, k: int, op: int, pps: int, ws: Optional[torch.Tensor]):
    if ws is None:
        ws = new_workspace(kv, k, op, pps)
    return ws, ws.numel() * ws.element_size()


def build_summaries(kv: PagedKV, rope: Optional[Rope] = None, tail_only: bool = False,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-page channel-wise key min/max, sequence-major: returns summ [B][Hkv][max_pages][2][D]
    (pool element type); summ[b][j][n] summarizes logical page n of sequence b."""
    d = kv.desc()
    _, Hkv, _, D = kv.k_pool.shape
    shape = (kv.batch, Hkv, int(kv.page_table.shape[1]), 2, D)
    if out is None:
        out = torch.empty(shape, dtype=kv.act_dtype, device=kv.device)
    _dev(out, "summ", kv.act_dtype)
    if tuple(out.shape) != shape:
        raise ValueError(f"summ must be {shape}, got {tuple(out.shape)}")
    _check(lib().kvsel_build_summaries(ctypes.byref(d), _rope_ptr(rope), int(bool(tail_only)),
                                       _ptr(out), _stream(kv.device)))
    return out


@dataclass
class FreePages:
    """Device-side free-page list of append_kv: ids int32 [capacity]; ids[:count] are free and the
    top one is taken first; count int32 [1]."""

    ids: torch.Tensor
    count: torch.Tensor


@dataclass
class Reuse:
    """Inputs of the speculative-reuse decision (previous query and previous fresh selection)."""

    q_prev: torch.Tensor
    prev_idx: torch.Tensor
    prev_cnt: torch.Tensor
    tau: float
    first_step: bool = False


def score_topk(kv: PagedKV, summ: torch.Tensor, q: torch.Tensor, k: int, *,
               refresh_tail: bool = False, rope: Optional[Rope] = None,
               scores: Optional[torch.Tensor] = None, reuse: Optional[Reuse] = None,
               sel_idx: Optional[torch.Tensor] = None, sel_cnt: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None):
    """Page scores + top-k. Returns (sel_idx [B][Hkv][k], sel_cnt [B][Hkv]) and,
    with ``reuse``, additionally (used_idx, used_cnt, corrected uint8, similarity fp64).
    ``refresh_tail`` first rebuilds each sequence's last-page summary in ``summ``."""
    d = kv.desc()
    B, Hkv = kv.batch, kv.num_kv_heads
    dev = kv.device
    _check_summ(kv, summ)
    _dev(q, "q", kv.act_dtype)
    if sel_idx is None:
        sel_idx = torch.empty((B, Hkv, k), dtype=torch.int32, device=dev)
    if sel_cnt is None:
        sel_cnt = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    if scores is not None:
        _dev(scores, "scores", torch.float32)
    rd = None
    extra = ()
    if reuse is not None:
        used_idx = torch.empty((B, Hkv, k), dtype=torch.int32, device=dev)
        used_cnt = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
        corrected = torch.empty((B, Hkv), dtype=torch.uint8, device=dev)
        sim = torch.empty((B, Hkv), dtype=torch.float64, device=dev)
        _dev(reuse.q_prev, "q_prev", kv.act_dtype)
        _dev(reuse.prev_idx, "prev_idx", torch.int32)
        _dev(reuse.prev_cnt, "prev_cnt", torch.int32)
        rd = ReuseDesc(reuse.q_prev.data_ptr(), reuse.prev_idx.data_ptr(), reuse.prev_cnt.data_ptr(),
                       float(reuse.tau), int(bool(reuse.first_step)), used_idx.data_ptr(),
                       used_cnt.data_ptr(), corrected.data_ptr(), sim.data_ptr())
        extra = (used_idx, used_cnt, corrected, sim)
    ws, ws_bytes = _workspace(kv, k, KVSEL_OP_SCORE_TOPK, 0, workspace)
    flags = KVSEL_SCORE_REFRESH_TAIL if refresh_tail else 0
    _check(lib().kvsel_score_topk(ctypes.byref(d), _rope_ptr(rope), _ptr(summ), _ptr(q), k, flags,
                                  _ptr(sel_idx), _ptr(sel_cnt), _ptr(scores),
                                  None if rd is None else ctypes.byref(rd), _ptr(ws), ws_bytes,
                                  _stream(dev)))
    return (sel_idx, sel_cnt) + extra


def default_scale(head_dim: int) -> float:
    """1/sqrt(D) rounded to fp32 (the softmax scale both the library and its callers use)."""
    return float(torch.tensor(1.0 / math.sqrt(head_dim), dtype=torch.float32))


def sparse_decode_attn(kv: PagedKV, q: torch.Tensor, sel_idx: torch.Tensor, sel_cnt: torch.Tensor,
                       k: Optional[int] = None, *, scale: Optional[float] = None,
                       pages_per_split: int = 0, rope: Optional[Rope] = None,
                       out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                       want_lse: bool = True, workspace: Optional[torch.Tensor] = None
                       ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Decode attention over the selected pages. Returns (out [B][Hq][D], lse fp32 [B][Hq])."""
    d = kv.desc()
    dev = kv.device
    _dev(q, "q", kv.act_dtype)
    _dev(sel_idx, "sel_idx", torch.int32)
    _dev(sel_cnt, "sel_cnt", torch.int32)
    k = int(sel_idx.shape[-1]) if k is None else k
    if scale is None:
        scale = default_scale(kv.head_dim)
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=dev)
    if lse is None and want_lse:
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    ws, ws_bytes = _workspace(kv, k, KVSEL_OP_ATTENTION, pages_per_split, workspace)
    _check(lib().kvsel_sparse_decode_attn(ctypes.byref(d), _rope_ptr(rope), _ptr(q), _ptr(sel_idx),
                                          _ptr(sel_cnt), k, scale, pages_per_split, _ptr(out),
                                          _ptr(lse), _ptr(ws), ws_bytes, _stream(dev)))
    return out, lse



def select_attend(kv: PagedKV, summ: torch.Tensor, q: torch.Tensor, k: int, *,
                  refresh_tail: bool = False, rope: Optional[Rope] = None,
                  scale: Optional[float] = None, sel_idx: Optional[torch.Tensor] = None,
                  sel_cnt: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                  lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                  workspace: Optional[torch.Tensor] = None):
    """score_topk + sparse_decode_attn (at step_pages_per_split) in one call, with the top-k fused into the
    attention launch. Returns (sel_idx, sel_cnt, out, lse)."""
    d = kv.desc()
    B, Hkv = kv.batch, kv.num_kv_heads
    dev = kv.device
    _check_summ(kv, summ)
    _dev(q, "q", kv.act_dtype)
    if sel_idx is None:
        sel_idx = torch.empty((B, Hkv, k), dtype=torch.int32, device=dev)
    if sel_cnt is None:
        sel_cnt = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    if scale is None:
        scale = default_scale(kv.head_dim)
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=dev)
    if lse is None and want_lse:
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    ws, ws_bytes = _workspace(kv, k, KVSEL_OP_SELECT_ATTEND, 0, workspace)
    flags = KVSEL_SCORE_REFRESH_TAIL if refresh_tail else 0
    _check(lib().kvsel_select_attend(ctypes.byref(d), _rope_ptr(rope), _ptr(summ), _ptr(q), k, flags,
                                     scale, _ptr(sel_idx), _ptr(sel_cnt), _ptr(out), _ptr(lse),
                                     _ptr(ws), ws_bytes, _stream(dev)))
    return sel_idx, sel_cnt, out, lse


def select_attend_static(kv: PagedKV, summ: torch.Tensor, q: torch.Tensor, k: int, *,
                         sel_idx: torch.Tensor, sel_cnt: torch.Tensor, out: torch.Tensor,
                         lse: Optional[torch.Tensor] = None, refresh_tail: bool = False,
                         rope: Optional[Rope] = None, scale: Optional[float] = None):
    """kvsel_select_attend_static: select_attend with its scores and split partials in the
    library's per-GPU device array instead of a workspace. Every output is the caller's (this
    wrapper allocates nothing either). Returns (sel_idx, sel_cnt, out, lse)."""
    d = kv.desc()
    dev = kv.device
    _check_summ(kv, summ)
    _dev(q, "q", kv.act_dtype)
    _dev(sel_idx, "sel_idx", torch.int32)
    _dev(sel_cnt, "sel_cnt", torch.int32)
    _dev(out, "out", q.dtype)
    if lse is not None:
        _dev(lse, "lse", torch.float32)
    if scale is None:
        scale = default_scale(kv.head_dim)
    flags = KVSEL_SCORE_REFRESH_TAIL if refresh_tail else 0
    _check(lib().kvsel_select_attend_static(ctypes.byref(d), _rope_ptr(rope), _ptr(summ), _ptr(q),
                                            k, flags, scale, _ptr(sel_idx), _ptr(sel_cnt),
                                            _ptr(out), _ptr(lse), _stream(dev)))
    return sel_idx, sel_cnt, out, lse


def rope_table(theta: float, head_dim: int, first_position: int, n_rows: int,
               device: torch.device) -> Tuple[torch.Tensor, torch.Tensor]:
    """cos/sin fp32 [n_rows][D/2] of (first_position + r) * theta^(-2i/D), built on the device."""
    cos = torch.empty((n_rows, head_dim // 2), dtype=torch.float32, device=device)
    sin = torch.empty_like(cos)
    _check(lib().kvsel_rope_table(float(theta), head_dim, first_position, n_rows, _ptr(cos),
                                  _ptr(sin), _stream(torch.device(device))))
    return cos, sin


def rope_shift(kv: PagedKV, rope: Rope, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Materialized rotation of the key pool (out may be kv.k_pool for in place)."""
    d = kv.desc()
    if out is None:
        out = torch.empty_like(kv.k_pool)
    _dev(out, "k_out", kv.k_pool.dtype)
    _check(lib().kvsel_rope_shift(ctypes.byref(d), ctypes.byref(rope.desc()), _ptr(out),
                                  _stream(kv.device)))
    return out


def gather_probe(chunk_addr: torch.Tensor, chunk_bytes: int, sink: Optional[torch.Tensor] = None):
    """Read-bandwidth probe over device chunks (``chunk_addr``: int64 device addresses)."""
    _dev(chunk_addr, "chunk_addr", torch.int64)
    dev = chunk_addr.device
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
    _check(lib().kvsel_gather_probe(_ptr(chunk_addr), int(chunk_addr.numel()), int(chunk_bytes),
                                    _ptr(sink), _stream(dev)))
    return sink


def tile_addresses(kv: PagedKV, sel_idx: torch.Tensor, sel_cnt: torch.Tensor,
                   page_table: torch.Tensor) -> torch.Tensor:
    """Device addresses of the K and V (page, KV head) tiles the selection names (host-side
    bookkeeping for gather_probe; ``page_table`` on the host)."""
    sel = sel_idx.cpu()
    cnt = sel_cnt.cpu()
    esize = kv.k_pool.element_size()
    tile = kv.k_pool.shape[2] * kv.head_dim * esize  # P * D elements
    kb, vb = kv.k_pool.data_ptr(), kv.v_pool.data_ptr()
    addrs = []
    for b in range(sel.shape[0]):
        for j in range(sel.shape[1]):
            for n in sel[b, j, :int(cnt[b, j])].tolist():
                p = int(page_table[b, n])
                off = (p * kv.num_kv_heads + j) * tile
                addrs.append(kb + off)
                addrs.append(vb + off)
    return torch.tensor(addrs, dtype=torch.int64).to(kv.device)


def append_kv(kv: PagedKV, k_new: torch.Tensor, v_new: torch.Tensor,
              summ: Optional[torch.Tensor] = None, seq_lens_out: Optional[torch.Tensor] = None,
              flags: Optional[torch.Tensor] = None,
              free_pages: Optional["FreePages"] = None) -> torch.Tensor:
    """Decode-time append of one token per sequence (k_new, v_new [B][Hkv][D]) into the pools,
    with the tail page's summary kept current when ``summ`` is given. Writes the new lengths to
    ``seq_lens_out`` (default: kv.seq_lens, in place) and returns it. The page a token opens is
    taken from ``free_pages`` (and written into the page table) when given; otherwise its
    page-table entry must be set by the caller first."""
    d = kv.desc()
    dev = kv.device
    if kv.v_pool is None:
        raise ValueError("append_kv needs the value pool")
    for t, name in ((k_new, "k_new"), (v_new, "v_new")):
        _dev(t, name, kv.k_pool.dtype)
        if tuple(t.shape) != (kv.batch, kv.num_kv_heads, kv.head_dim):
            raise ValueError(f"{name} must be [B][Hkv][D]")
    if summ is not None:
        _check_summ(kv, summ)
    if seq_lens_out is None:
        seq_lens_out = kv.seq_lens
    _dev(seq_lens_out, "seq_lens_out", torch.int32)
    if flags is not None:
        _dev(flags, "flags", torch.int32)
    fp = None
    if free_pages is not None:
        _dev(free_pages.ids, "free_pages.ids", torch.int32)
        _dev(free_pages.count, "free_pages.count", torch.int32)
        if free_pages.ids.dim() != 1 or free_pages.count.numel() != 1:
            raise ValueError("free_pages: ids [capacity], count [1]")
        fp = ctypes.byref(FreePagesDesc(free_pages.ids.data_ptr(), free_pages.count.data_ptr(),
                                        int(free_pages.ids.numel())))
    _check(lib().kvsel_append_kv(ctypes.byref(d), _ptr(k_new), _ptr(v_new), _ptr(summ),
                                 _ptr(seq_lens_out), fp, _ptr(flags), _stream(dev)))
    return seq_lens_out


def quantize_pages(kv: PagedKV, values: bool = True) -> PagedKV:
    """The cache with its pages quantized to fp8 (uint8 E4M3 codes, one fp32 scale per (physical
    page, KV head) tile of K and of V), sharing kv's page table and lengths."""
    d = kv.desc()
    if kv.is_fp8:
        raise ValueError("the cache is already fp8")
    dev = kv.device
    Npp, Hkv = kv.k_pool.shape[:2]
    k_codes = torch.empty(kv.k_pool.shape, dtype=torch.uint8, device=dev)
    k_scale = torch.empty((Npp, Hkv), dtype=torch.float32, device=dev)
    v_codes = v_scale = None
    if values and kv.v_pool is not None:
        v_codes = torch.empty(kv.v_pool.shape, dtype=torch.uint8, device=dev)
        v_scale = torch.empty((Npp, Hkv), dtype=torch.float32, device=dev)
    _check(lib().kvsel_quantize_pages(ctypes.byref(d), _ptr(k_codes), _ptr(k_scale), _ptr(v_codes),
                                      _ptr(v_scale), _stream(dev)))
    return PagedKV(k_codes, v_codes, kv.page_table, kv.seq_lens, kv.num_q_heads, kv.max_seq_len,
                   k_scale, v_scale, kv.page_fill)


def check_inputs(kv: PagedKV, sel_idx: Optional[torch.Tensor] = None,
                 sel_cnt: Optional[torch.Tensor] = None, k: Optional[int] = None,
                 flags: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Device-side contract check; returns the (sticky) int32 flag word (KVSEL_CHECK_* bits)."""
    d = kv.desc()
    dev = kv.device
    if flags is None:
        flags = torch.zeros(1, dtype=torch.int32, device=dev)
    if sel_idx is not None:
        _dev(sel_idx, "sel_idx", torch.int32)
        _dev(sel_cnt, "sel_cnt", torch.int32)
        k = int(sel_idx.shape[-1]) if k is None else k
    _check(lib().kvsel_check_inputs(ctypes.byref(d), _ptr(sel_idx), _ptr(sel_cnt),
                                    0 if k is None else int(k), _ptr(flags), _stream(dev)))
    return flags



def speculative_step(kv: PagedKV, summ: torch.Tensor, q: torch.Tensor, k: int, reuse: Reuse, *,
                     refresh_tail: bool = False, rope: Optional[Rope] = None,
                     scale: Optional[float] = None, sel_idx: Optional[torch.Tensor] = None,
                     sel_cnt: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                     lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                     workspace: Optional[torch.Tensor] = None):
    """score_topk with reuse + sparse_decode_attn over the used pages in one call, the attention
    over the previous step's pages sharing a launch with the scoring. Returns (sel_idx, sel_cnt,
    used_idx, used_cnt, corrected, similarity, out, lse)."""
    d = kv.desc()
    B, Hkv = kv.batch, kv.num_kv_heads
    dev = kv.device
    _check_summ(kv, summ)
    _dev(q, "q", kv.act_dtype)
    _dev(reuse.q_prev, "q_prev", kv.act_dtype)
    _dev(reuse.prev_idx, "prev_idx", torch.int32)
    _dev(reuse.prev_cnt, "prev_cnt", torch.int32)
    if sel_idx is None:
        sel_idx = torch.empty((B, Hkv, k), dtype=torch.int32, device=dev)
    if sel_cnt is None:
        sel_cnt = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    if scale is None:
        scale = default_scale(kv.head_dim)
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=dev)
    if lse is None and want_lse:
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    used_idx = torch.empty((B, Hkv, k), dtype=torch.int32, device=dev)
    used_cnt = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    corrected = torch.empty((B, Hkv), dtype=torch.uint8, device=dev)
    sim = torch.empty((B, Hkv), dtype=torch.float64, device=dev)
    rd = ReuseDesc(reuse.q_prev.data_ptr(), reuse.prev_idx.data_ptr(), reuse.prev_cnt.data_ptr(),
                   float(reuse.tau), int(bool(reuse.first_step)), used_idx.data_ptr(),
                   used_cnt.data_ptr(), corrected.data_ptr(), sim.data_ptr())
    ws, ws_bytes = _workspace(kv, k, KVSEL_OP_SPECULATIVE_STEP, 0, workspace)
    flags = KVSEL_SCORE_REFRESH_TAIL if refresh_tail else 0
    _check(lib().kvsel_speculative_step(ctypes.byref(d), _rope_ptr(rope), _ptr(summ), _ptr(q), k,
                                        flags, scale, ctypes.byref(rd), _ptr(sel_idx),
                                        _ptr(sel_cnt), _ptr(out), _ptr(lse), _ptr(ws), ws_bytes,
                                        _stream(dev)))
    return sel_idx, sel_cnt, used_idx, used_cnt, corrected, sim, out, lse

