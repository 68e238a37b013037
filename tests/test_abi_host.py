"""Host-side checks of the C ABI: the library loads, exports every entry point
include/moira.h declares, and rejects bad arguments with the documented codes
before anything is enqueued (no GPU is touched by these calls)."""

import ctypes
import os
import re

import pytest

from long_context_sparse_summary_amd import moira as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moira.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moira_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return M.load()


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ["moira_append_kv", "moira_page_summaries", "moira_select_pages",
              "moira_ragged_decode_attn", "moira_combine"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in M._SIGS, f"binding lacks a signature for {name}"


def test_abi_version(lib):
    assert lib.moira_abi_version() == 5


def test_strerror_messages(lib):
    for code in [0, -1, -2, -3, -4, -5, -6, -7, -8, 99]:
        assert isinstance(M.strerror(code), str) and M.strerror(code)


def shape(**kw):
    base = dict(batch=2, num_kv_heads=4, group=4, head_dim=128, max_pages=64, num_phys_pages=128)
    base.update(kw)
    return M.make_shape(**base)


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation


def call_select(lib, sh, gamma=0.9, scale=0.1, null_at=None):
    args = [FAKE] * 7
    if null_at is not None:
        args[null_at] = None
    return lib.moira_select_pages(ctypes.byref(sh), args[0], args[1], args[2], args[3], gamma, scale,
                                  args[4], args[5], args[6], None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), -2), (dict(num_kv_heads=-1), -2), (dict(group=0), -2), (dict(max_pages=0), -2),
    (dict(num_phys_pages=0), -2), (dict(num_phys_pages=1 << 40), -2),
    (dict(head_dim=96), -5), (dict(head_dim=256), -5), (dict(group=17), -5),
    (dict(max_pages=16385), -5), (dict(batch=1025), -5), (dict(page_size=32), -5),
])
def test_shape_errors(lib, kw, code):
    ps = kw.pop("page_size", 16)
    sh = shape(**kw)
    sh.page_size = ps
    assert call_select(lib, sh) == code
    assert lib.moira_select_workspace_bytes(ctypes.byref(sh)) == 0
    assert lib.moira_partials_slots(ctypes.byref(sh), 8) == 0


def test_dtype_errors(lib):
    sh = shape()
    sh.kv_dtype = 7
    assert call_select(lib, sh) == -3
    sh = shape()
    sh.q_dtype = 0
    assert call_select(lib, sh) == -3
    sh = shape()
    sh.sum_dtype = 4
    assert call_select(lib, sh) == -3
    # E4M3 is a summary type only
    for field in ("kv_dtype", "q_dtype"):
        sh = shape()
        setattr(sh, field, M.MOIRA_FP8_E4M3)
        assert call_select(lib, sh) == -3


def test_summary_dtype_field(lib):
    """0 and MOIRA_F32 both mean fp32 summaries; the workspace does not depend on it."""
    import torch
    sizes = set()
    for code in (0, M.MOIRA_F32, M.MOIRA_BF16, M.MOIRA_FP8_E4M3):
        sh = shape()
        sh.sum_dtype = code
        sizes.add(lib.moira_select_workspace_bytes(ctypes.byref(sh)))
    assert len(sizes) == 1 and sizes.pop() > 0
    assert M.summary_dtype(shape()) == torch.float32
    assert M.summary_dtype(shape(sum_dtype=torch.bfloat16)) == torch.bfloat16
    assert M.summary_dtype(shape(sum_dtype=torch.float8_e4m3fn)) == torch.float8_e4m3fn


def test_null_shape(lib):
    assert lib.moira_combine(None, FAKE, 4, FAKE, FAKE, FAKE, None) == -1


@pytest.mark.parametrize("i", range(7))
def test_select_null_pointers(lib, i):
    assert call_select(lib, shape(), null_at=i) == -1


@pytest.mark.parametrize("gamma", [0.0, -0.5, 1.0000001, 2.0, float("nan"), float("inf")])
def test_gamma_errors(lib, gamma):
    assert call_select(lib, shape(), gamma=gamma) == -4


def test_scale_error(lib):
    assert call_select(lib, shape(), scale=float("inf")) == -7
    assert call_select(lib, shape(), scale=float("nan")) == -7


def test_attn_and_combine_argument_errors(lib):
    sh = shape()
    args = [FAKE] * 7
    for n in [0, -3, 65537]:
        assert lib.moira_ragged_decode_attn(ctypes.byref(sh), *args, 0.1, n, FAKE, FAKE, None, None) == -7
        assert lib.moira_combine(ctypes.byref(sh), FAKE, n, FAKE, FAKE, FAKE, None) == -7
    assert lib.moira_ragged_decode_attn(ctypes.byref(sh), *args, float("nan"), 8, FAKE, FAKE, None, None) == -7
    assert lib.moira_ragged_decode_attn(ctypes.byref(sh), None, *args[1:], 0.1, 8, FAKE, FAKE, None, None) == -1
    assert lib.moira_combine(ctypes.byref(sh), FAKE, 8, FAKE, FAKE, None, None) == -1


def test_append_select_argument_errors(lib):
    sh = shape()
    args = [FAKE] * 8     # q, k_new, v_new, k_pool, v_pool, summaries, block_table, seq_lens
    tail = [FAKE] * 3     # workspace, page_lists, list_lens
    for i in range(8):
        a = list(args)
        a[i] = None
        assert lib.moira_append_select(ctypes.byref(sh), *a, 0.9, 0.1, *tail, None, None) == -1
    for i in range(3):
        t = list(tail)
        t[i] = None
        assert lib.moira_append_select(ctypes.byref(sh), *args, 0.9, 0.1, *t, None, None) == -1
    for g in [0.0, 1.5, float("nan")]:
        assert lib.moira_append_select(ctypes.byref(sh), *args, g, 0.1, *tail, None, None) == -4
    assert lib.moira_append_select(ctypes.byref(sh), *args, 0.9, float("inf"), *tail, None, None) == -7
    bad = shape(group=17)
    assert lib.moira_append_select(ctypes.byref(bad), *args, 0.9, 0.1, *tail, None, None) == -5


def test_summaries_mode_error(lib):
    sh = shape()
    assert lib.moira_page_summaries(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, 2, None, None) == -7
    assert lib.moira_page_summaries(ctypes.byref(sh), None, FAKE, FAKE, FAKE, 0, None, None) == -1


def test_append_and_advance_null_errors(lib):
    sh = shape()
    assert lib.moira_append_kv(ctypes.byref(sh), FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None) == -1
    assert lib.moira_advance_seq_lens(ctypes.byref(sh), None, None, None) == -1


def test_sizes(lib):
    sh = shape()
    # per segment: two 2048-band histograms (u64 mass + u32 count each), a key
    # per page, a maximum per 64-page chunk, and 48 bytes of per-segment words
    assert lib.moira_select_workspace_bytes(ctypes.byref(sh)) == 2 * 4 * (2048 * 24 + 64 * 8 + 8 + 48)
    assert lib.moira_partials_slots(ctypes.byref(sh), 100) == 100 + 8 - 1
    assert lib.moira_partials_slots(ctypes.byref(sh), 0) == 0
    # partial_o then partial_ml: slots * group * (head_dim + 2) floats
    assert lib.moira_partials_bytes(ctypes.byref(sh), 100) == (100 + 8 - 1) * 4 * (128 + 2) * 4
    assert lib.moira_partials_bytes(ctypes.byref(sh), 0) == 0
    assert lib.moira_partials_bytes(None, 100) == 0


def test_select_workspace_alignment_error(lib):
    """A workspace that is not 16-byte aligned is refused before any launch."""
    sh = shape()
    odd = ctypes.c_void_p(0x1008)
    args = [FAKE] * 4     # q, summaries, block_table, seq_lens
    assert lib.moira_select_pages(ctypes.byref(sh), *args, 0.9, 0.1, odd, FAKE, FAKE, None, None) == -7
    args = [FAKE] * 8     # q, k_new, v_new, k_pool, v_pool, summaries, block_table, seq_lens
    assert lib.moira_append_select(ctypes.byref(sh), *args, 0.9, 0.1, odd, FAKE, FAKE, None, None) == -7


def test_select_rule_argument_errors(lib):
    """Rules and their parameters are checked before any launch."""
    sh = shape()
    args = [FAKE] * 4     # q, summaries, block_table, seq_lens
    tail = [FAKE] * 3     # workspace, page_lists, list_lens

    def call(rule, param, scale=0.1):
        return lib.moira_select_pages_rule(ctypes.byref(sh), *args, rule, param, scale, *tail,
                                           None, None)
    for rule, param in [(7, 0.5), (-1, 0.5), (1, 0.0), (1, 2.5), (1, -3.0), (1, float("nan")),
                        (2, -0.1), (2, 1.5), (2, float("inf"))]:
        assert call(rule, param) == -7, (rule, param)
    for g in (0.0, 1.5):
        assert call(0, g) == -4
    assert call(1, 8.0, scale=float("nan")) == -7
    assert lib.moira_select_pages_rule(ctypes.byref(sh), None, *args[1:], 1, 8.0, 0.1, *tail,
                                       None, None) == -1


def test_noalloc_select_argument_errors(lib):
    """moira_select_pages_noalloc checks its arguments, and the static scratch
    limit, before anything is enqueued."""
    sh = shape()
    args = [FAKE] * 4     # q, summaries, block_table, seq_lens
    assert lib.moira_select_pages_noalloc(ctypes.byref(sh), None, *args[1:], 0.9, 0.1, FAKE, FAKE,
                                          None, None) == -1
    assert lib.moira_select_pages_noalloc(ctypes.byref(sh), *args, 1.5, 0.1, FAKE, FAKE, None, None) == -4
    assert lib.moira_select_pages_noalloc(ctypes.byref(sh), *args, 0.9, float("nan"), FAKE, FAKE,
                                          None, None) == -7
    huge = shape(batch=4096, num_kv_heads=1, max_pages=16384, num_phys_pages=1 << 20)
    assert lib.moira_select_pages_noalloc(ctypes.byref(huge), *args, 0.9, 0.1, FAKE, FAKE,
                                          None, None) == -8
