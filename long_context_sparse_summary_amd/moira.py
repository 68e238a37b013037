"""Thin ctypes binding of libmoira.so (argument marshalling only).

Every function mirrors one ``extern "C"`` entry point of include/moira.h, takes
torch tensors that already live on the GPU, passes their device pointers and
torch's current HIP stream, and raises MoiraError on a non-zero return code.
No computation happens here: every step of the decode path runs in the HIP
kernels of libmoira.so. If the library is missing the binding raises; there is
no fallback.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MOIRA_LIB", os.path.join(_HERE, "libmoira.so"))

MOIRA_BF16 = 1
MOIRA_F32 = 2
MOIRA_FP8_E4M3 = 3   # page summaries only (torch.float8_e4m3fn)
SUM_ALL = 0
SUM_TAIL = 1

ST_CAPACITY = 1
ST_BAD_LEN = 2
ST_BAD_PAGE = 4
ST_BAD_LIST = 8
ST_MASS_RANGE = 16

E_CODES = {
    0: "MOIRA_OK", -1: "MOIRA_E_NULL", -2: "MOIRA_E_SHAPE", -3: "MOIRA_E_DTYPE",
    -4: "MOIRA_E_GAMMA", -5: "MOIRA_E_UNSUPPORTED", -6: "MOIRA_E_LAUNCH", -7: "MOIRA_E_ARG",
    -8: "MOIRA_E_SCRATCH",
}


class MoiraError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {E_CODES.get(code, code)} ({strerror(code)})")


class Shape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages", ctypes.c_int32),
        ("num_phys_pages", ctypes.c_int64),
        ("kv_dtype", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32),
        ("sum_dtype", ctypes.c_int32),
    ]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_SIGS = {
    "moira_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "moira_abi_version": (ctypes.c_int, []),
    "moira_advance_seq_lens": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P]),
    "moira_append_kv": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moira_page_summaries": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, _I32, _P, _P]),
    "moira_select_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(Shape)]),
    "moira_select_pages": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, ctypes.c_double,
                                          ctypes.c_float, _P, _P, _P, _P, _P]),
    "moira_select_pages_rule": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, _I32,
                                               ctypes.c_double, ctypes.c_float, _P, _P, _P, _P,
                                               _P]),
    "moira_select_pages_noalloc": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P,
                                                  ctypes.c_double, ctypes.c_float, _P, _P, _P,
                                                  _P]),
    "moira_append_select": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, _P, _P, _P, _P,
                                           ctypes.c_double, ctypes.c_float, _P, _P, _P, _P, _P]),
    "moira_partials_slots": (ctypes.c_size_t, [ctypes.POINTER(Shape), _I32]),
    "moira_partials_bytes": (ctypes.c_size_t, [ctypes.POINTER(Shape), _I32]),
    "moira_ragged_decode_attn": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, _P, _P, _P,
                                                ctypes.c_float, _I32, _P, _P, _P, _P]),
    "moira_combine": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _I32, _P, _P, _P, _P]),
    "moira_ragged_decode_attn_combine": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, _P,
                                                        _P, _P, ctypes.c_float, _I32, _P, _P, _P,
                                                        _P, _P, _P]),
    "moira_stream_read_sink_words": (ctypes.c_size_t, []),
    "moira_stream_read": (ctypes.c_int, [_P, ctypes.c_size_t, _P, _P]),
}

_lib = None


ABI_VERSION = 5   # MOIRA_ABI_VERSION of include/moira.h


def load(path: Optional[str] = None):
    """Load libmoira.so (once). Raises OSError/RuntimeError if it is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libmoira.so not built at {p}; run `python -m long_context_sparse_summary_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.moira_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{p} has ABI version {lib.moira_abi_version()}, this binding expects "
                           f"{ABI_VERSION}: rebuild it")
    if path is None:
        _lib = lib
    return lib


def strerror(code: int) -> str:
    return load().moira_strerror(int(code)).decode()


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return MOIRA_BF16
    if dt == torch.float32:
        return MOIRA_F32
    if dt == torch.float8_e4m3fn:
        return MOIRA_FP8_E4M3
    raise ValueError(f"unsupported dtype {dt}")


def make_shape(batch: int, num_kv_heads: int, group: int, head_dim: int, max_pages: int,
               num_phys_pages: int, kv_dtype: torch.dtype = torch.bfloat16,
               q_dtype: torch.dtype = torch.bfloat16, page_size: int = 16,
               sum_dtype: torch.dtype = torch.float32) -> Shape:
    return Shape(batch, num_kv_heads, group, head_dim, page_size, max_pages, num_phys_pages,
                 _dtype_code(kv_dtype), _dtype_code(q_dtype), _dtype_code(sum_dtype))


def summary_dtype(shape: Shape) -> torch.dtype:
    """Element type of the page summaries for this shape."""
    return {MOIRA_BF16: torch.bfloat16, MOIRA_FP8_E4M3: torch.float8_e4m3fn}.get(shape.sum_dtype,
                                                                             torch.float32)


def _ptr(t: Optional[torch.Tensor], what: str, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{what} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{what} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(rc: int, where: str):
    if rc != 0:
        raise MoiraError(rc, where)


def advance_seq_lens(shape: Shape, seq_lens, status=None):
    _check(load().moira_advance_seq_lens(ctypes.byref(shape), _ptr(seq_lens, "seq_lens", torch.int32),
                                         _ptr(status, "status", torch.int32), _stream()),
           "moira_advance_seq_lens")


def append_kv(shape: Shape, k_new, v_new, k_pool, v_pool, summaries, block_table, seq_lens,
              status=None):
    _check(load().moira_append_kv(ctypes.byref(shape), _ptr(k_new, "k_new"), _ptr(v_new, "v_new"),
                                  _ptr(k_pool, "k_pool"), _ptr(v_pool, "v_pool"),
                                  _ptr(summaries, "summaries", summary_dtype(shape)),
                                  _ptr(block_table, "block_table", torch.int32),
                                  _ptr(seq_lens, "seq_lens", torch.int32),
                                  _ptr(status, "status", torch.int32), _stream()),
           "moira_append_kv")


def page_summaries(shape: Shape, k_pool, block_table, seq_lens, summaries, mode: int = SUM_ALL,
                   status=None):
    _check(load().moira_page_summaries(ctypes.byref(shape), _ptr(k_pool, "k_pool"),
                                       _ptr(block_table, "block_table", torch.int32),
                                       _ptr(seq_lens, "seq_lens", torch.int32),
                                       _ptr(summaries, "summaries", summary_dtype(shape)), int(mode),
                                       _ptr(status, "status", torch.int32), _stream()),
           "moira_page_summaries")


def select_workspace_bytes(shape: Shape) -> int:
    return int(load().moira_select_workspace_bytes(ctypes.byref(shape)))


def select_pages(shape: Shape, q, summaries, block_table, seq_lens, gamma: float, scale: float,
                 workspace, page_lists, list_lens, status=None):
    _check(load().moira_select_pages(ctypes.byref(shape), _ptr(q, "q"),
                                     _ptr(summaries, "summaries", summary_dtype(shape)),
                                     _ptr(block_table, "block_table", torch.int32),
                                     _ptr(seq_lens, "seq_lens", torch.int32), float(gamma),
                                     float(scale), _ptr(workspace, "workspace"),
                                     _ptr(page_lists, "page_lists", torch.int32),
                                     _ptr(list_lens, "list_lens", torch.int32),
                                     _ptr(status, "status", torch.int32), _stream()),
           "moira_select_pages")


def select_pages_noalloc(shape: Shape, q, summaries, block_table, seq_lens, gamma: float,
                         scale: float, page_lists, list_lens, status=None):
    """select_pages without a workspace argument (the library's static scratch)."""
    _check(load().moira_select_pages_noalloc(ctypes.byref(shape), _ptr(q, "q"),
                                             _ptr(summaries, "summaries", summary_dtype(shape)),
                                             _ptr(block_table, "block_table", torch.int32),
                                             _ptr(seq_lens, "seq_lens", torch.int32), float(gamma),
                                             float(scale),
                                             _ptr(page_lists, "page_lists", torch.int32),
                                             _ptr(list_lens, "list_lens", torch.int32),
                                             _ptr(status, "status", torch.int32), _stream()),
           "moira_select_pages_noalloc")


RULES = {"coverage": 0, "topk": 1, "topdelta": 2}


def select_pages_rule(shape: Shape, q, summaries, block_table, seq_lens, rule: str, param: float,
                      scale: float, workspace, page_lists, list_lens, status=None):
    """Selection under a rule: "coverage" (param = gamma), "topk" (param =
    k) or "topdelta" (param = delta), over the same masses as select_pages."""
    _check(load().moira_select_pages_rule(ctypes.byref(shape), _ptr(q, "q"),
                                          _ptr(summaries, "summaries", summary_dtype(shape)),
                                          _ptr(block_table, "block_table", torch.int32),
                                          _ptr(seq_lens, "seq_lens", torch.int32),
                                          int(RULES[rule]), float(param), float(scale),
                                          _ptr(workspace, "workspace"),
                                          _ptr(page_lists, "page_lists", torch.int32),
                                          _ptr(list_lens, "list_lens", torch.int32),
                                          _ptr(status, "status", torch.int32), _stream()),
           "moira_select_pages_rule")


def append_select(shape: Shape, q, k_new, v_new, k_pool, v_pool, summaries, block_table, seq_lens,
                  gamma: float, scale: float, workspace, page_lists, list_lens, status=None):
    _check(load().moira_append_select(ctypes.byref(shape), _ptr(q, "q"), _ptr(k_new, "k_new"),
                                      _ptr(v_new, "v_new"), _ptr(k_pool, "k_pool"),
                                      _ptr(v_pool, "v_pool"),
                                      _ptr(summaries, "summaries", summary_dtype(shape)),
                                      _ptr(block_table, "block_table", torch.int32),
                                      _ptr(seq_lens, "seq_lens", torch.int32), float(gamma),
                                      float(scale), _ptr(workspace, "workspace"),
                                      _ptr(page_lists, "page_lists", torch.int32),
                                      _ptr(list_lens, "list_lens", torch.int32),
                                      _ptr(status, "status", torch.int32), _stream()),
           "moira_append_select")


def partials_slots(shape: Shape, num_workgroups: int) -> int:
    return int(load().moira_partials_slots(ctypes.byref(shape), int(num_workgroups)))


def partials_bytes(shape: Shape, num_workgroups: int) -> int:
    return int(load().moira_partials_bytes(ctypes.byref(shape), int(num_workgroups)))


def ragged_decode_attn(shape: Shape, q, k_pool, v_pool, block_table, seq_lens, page_lists,
                       list_lens, scale: float, num_workgroups: int, partial_o, partial_ml,
                       status=None):
    _check(load().moira_ragged_decode_attn(ctypes.byref(shape), _ptr(q, "q"), _ptr(k_pool, "k_pool"),
                                           _ptr(v_pool, "v_pool"),
                                           _ptr(block_table, "block_table", torch.int32),
                                           _ptr(seq_lens, "seq_lens", torch.int32),
                                           _ptr(page_lists, "page_lists", torch.int32),
                                           _ptr(list_lens, "list_lens", torch.int32), float(scale),
                                           int(num_workgroups),
                                           _ptr(partial_o, "partial_o", torch.float32),
                                           _ptr(partial_ml, "partial_ml", torch.float32),
                                           _ptr(status, "status", torch.int32), _stream()),
           "moira_ragged_decode_attn")


def ragged_decode_attn_combine(shape: Shape, q, k_pool, v_pool, block_table, seq_lens, page_lists,
                               list_lens, scale: float, num_workgroups: int, partial_o, partial_ml,
                               counters, out, status=None):
    """Attention and the merge of its partial states, in one launch where it can."""
    _check(load().moira_ragged_decode_attn_combine(
        ctypes.byref(shape), _ptr(q, "q"), _ptr(k_pool, "k_pool"), _ptr(v_pool, "v_pool"),
        _ptr(block_table, "block_table", torch.int32), _ptr(seq_lens, "seq_lens", torch.int32),
        _ptr(page_lists, "page_lists", torch.int32), _ptr(list_lens, "list_lens", torch.int32),
        float(scale), int(num_workgroups), _ptr(partial_o, "partial_o", torch.float32),
        _ptr(partial_ml, "partial_ml", torch.float32), _ptr(counters, "counters", torch.int32),
        _ptr(out, "out", torch.float32), _ptr(status, "status", torch.int32), _stream()),
        "moira_ragged_decode_attn_combine")


def combine(shape: Shape, list_lens, num_workgroups: int, partial_o, partial_ml, out):
    _check(load().moira_combine(ctypes.byref(shape), _ptr(list_lens, "list_lens", torch.int32),
                                int(num_workgroups), _ptr(partial_o, "partial_o", torch.float32),
                                _ptr(partial_ml, "partial_ml", torch.float32),
                                _ptr(out, "out", torch.float32), _stream()),
           "moira_combine")


def stream_read_sink_words() -> int:
    return int(load().moira_stream_read_sink_words())


def stream_read(src, sink):
    """Measurement aid: read every byte of src once (the HBM read ceiling)."""
    _check(load().moira_stream_read(_ptr(src, "src"), src.numel() * src.element_size(),
                                    _ptr(sink, "sink", torch.int32), _stream()),
           "moira_stream_read")


@dataclass
class StepBuffers:
    """Device buffers one decode step needs besides the KV pool (allocated with
    torch; the library itself never allocates)."""
    shape: Shape
    num_workgroups: int
    workspace: torch.Tensor
    page_lists: torch.Tensor
    list_lens: torch.Tensor
    partial_o: torch.Tensor
    partial_ml: torch.Tensor
    out: torch.Tensor
    status: torch.Tensor
    counters: torch.Tensor      # per (request, KV head) arrival counters of the fused merge

    @classmethod
    def allocate(cls, shape: Shape, num_workgroups: int, device="cuda") -> "StepBuffers":
        S = shape.batch * shape.num_kv_heads
        slots = partials_slots(shape, num_workgroups)
        ws = select_workspace_bytes(shape)
        if slots == 0 or ws == 0:
            raise MoiraError(-2, "StepBuffers.allocate")
        G, D = shape.group, shape.head_dim
        return cls(
            shape, int(num_workgroups),
            torch.zeros(ws, dtype=torch.uint8, device=device),
            torch.empty((S, shape.max_pages), dtype=torch.int32, device=device),
            torch.empty(S, dtype=torch.int32, device=device),
            torch.empty((slots, G, D), dtype=torch.float32, device=device),
            torch.empty((slots, G, 2), dtype=torch.float32, device=device),
            torch.empty((shape.batch, shape.num_kv_heads * G, D), dtype=torch.float32, device=device),
            torch.zeros(1, dtype=torch.int32, device=device),
            torch.zeros(S, dtype=torch.int32, device=device),
        )


def layer_step(buf: StepBuffers, q, k_new, v_new, k_pool, v_pool, summaries, block_table, seq_lens,
               gamma: float, scale: float, fused_append: bool = True, fused_combine: bool = False):
    """One layer of a decode step: append, select, attend, combine (seq_lens
    must already count the new token; see advance_seq_lens). fused_append
    uses moira_append_select; otherwise append and select are separate calls.
    fused_combine uses moira_ragged_decode_attn_combine; otherwise attention
    and the combine are separate calls."""
    sh = buf.shape
    if fused_append:
        append_select(sh, q, k_new, v_new, k_pool, v_pool, summaries, block_table, seq_lens, gamma,
                      scale, buf.workspace, buf.page_lists, buf.list_lens, buf.status)
    else:
        append_kv(sh, k_new, v_new, k_pool, v_pool, summaries, block_table, seq_lens, buf.status)
        select_pages(sh, q, summaries, block_table, seq_lens, gamma, scale, buf.workspace,
                     buf.page_lists, buf.list_lens, buf.status)
    if fused_combine:
        ragged_decode_attn_combine(sh, q, k_pool, v_pool, block_table, seq_lens, buf.page_lists,
                                   buf.list_lens, scale, buf.num_workgroups, buf.partial_o,
                                   buf.partial_ml, buf.counters, buf.out, buf.status)
        return buf.out
    ragged_decode_attn(sh, q, k_pool, v_pool, block_table, seq_lens, buf.page_lists, buf.list_lens,
                       scale, buf.num_workgroups, buf.partial_o, buf.partial_ml, buf.status)
    combine(sh, buf.list_lens, buf.num_workgroups, buf.partial_o, buf.partial_ml, buf.out)
    return buf.out
