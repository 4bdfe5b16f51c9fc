"""C-ABI checks that need no GPU: the library loads, exports every function
include/lce.h declares, and rejects bad arguments on the host before any
launch (so these calls never touch a device)."""
import ctypes
import os
import re

import pytest
import torch

import chunked_lm_head_lce_amd as lce
from chunked_lm_head_lce_amd import _lib
from lce_inputs import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # never dereferenced: every call below fails validation first


def header_functions():
    text = open(os.path.join(ROOT, "include", "lce.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lce_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def prob(n=512, h=256, v=4096, **kw):
    p = _lib.LceProblem()
    p.n_rows, p.hidden, p.vocab = n, h, v
    p.ld_hidden = kw.get("ld_hidden", h)
    p.ld_weight = kw.get("ld_weight", h)
    p.ignore_index = -100
    p.chunk_rows = kw.get("chunk_rows", 256)
    p.rows_in_flight = kw.get("rows_in_flight", 0)
    p.reduction = kw.get("reduction", 1)
    p.dtype = kw.get("dtype", 0)
    return p


def test_exports_every_declared_function(lib):
    names = header_functions()
    assert set(names) == set(_lib.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_strings(lib):
    assert lib.lce_abi_version() == 103
    for code in range(6):
        assert _lib.status_string(code) != "unknown status"
    assert _lib.status_string(99) == "unknown status"


def ws(lib, p, kind):
    return lib.lce_workspace_bytes(ctypes.byref(p), kind)


def test_workspace_sizes(lib):
    f = ws(lib, prob(), 0)
    b = ws(lib, prob(), 1)
    e = ws(lib, prob(), 2)
    assert 0 < f < e < b
    assert b - e >= 4096 * 256 * 4          # the FP32 grad_weight accumulator
    assert ws(lib, prob(n=1024), 0) > f      # grows with N
    assert ws(lib, prob(n=0), 0) > 0
    assert ws(lib, prob(chunk_rows=0), 0) == 0
    assert ws(lib, prob(), 7) == 0


@pytest.mark.parametrize("name", ["qwen3_0p6b_head", "qwen3_4b_32k", "qwen3_4b_160k", "qwen3_8b_1m_shard"])
def test_no_full_logits_buffer(lib, name):
    """No [N, V] logits: the whole backward workspace stays below the fp32
    [N, V] logits an eager loss holds, its dlogits buffers are sized by
    rows_in_flight rather than N, and once N is many row groups it is below
    even a bf16 [N, V]."""
    w = WORKLOADS[name]
    b = ws(lib, prob(w.n_rows, w.hidden, w.vocab), 1)
    if w.n_rows >= 8 * w.hidden:   # below that the V x H grad buffers alone exceed it
        assert b < w.n_rows * w.vocab * 4, (b, w.n_rows * w.vocab * 4)
    b_small = ws(lib, prob(w.n_rows, w.hidden, w.vocab, rows_in_flight=4096), 1)
    if w.n_rows > 4096:
        assert b - b_small >= 2 * (16384 - 4096) * w.vocab   # the bf16 p~ / G buffer of a row group
    if w.n_rows >= 8 * 16384:
        assert b < w.n_rows * w.vocab * 2, (b, w.n_rows * w.vocab * 2)


def fwd(lib, p, hidden=FAKE, weight=FAKE, labels=FAKE, loss=FAKE, wsp=FAKE, wsb=1 << 40):
    return lib.lce_forward(ctypes.byref(p) if p is not None else None, hidden, weight, None, labels, loss, None,
                           None, None, None, wsp, wsb, None)


@pytest.mark.parametrize("bad,code", [
    (dict(chunk_rows=0), 1), (dict(chunk_rows=-3), 1), (dict(ld_hidden=128), 1), (dict(ld_weight=8), 1),
    (dict(reduction=3), 1), (dict(dtype=1), 2), (dict(h=96, ld_hidden=96, ld_weight=96), 2),
    (dict(ld_hidden=260), 2), (dict(rows_in_flight=-1), 1), (dict(ld_hidden=(1 << 22) + 8), 2),
    (dict(ld_weight=(1 << 22) + 8), 2), (dict(v=(1 << 22) + 1), 2),
])
def test_forward_rejects_bad_problem(lib, bad, code):
    kw = dict(bad)
    n = kw.pop("n", 512)
    h = kw.pop("h", 256)
    v = kw.pop("v", 4096)
    assert fwd(lib, prob(n, h, v, **kw)) == code


def test_forward_rejects_bad_pointers(lib):
    assert fwd(lib, None) == 1
    assert fwd(lib, prob(), loss=None) == 1
    assert fwd(lib, prob(), hidden=None) == 1
    assert fwd(lib, prob(), weight=None) == 1
    assert fwd(lib, prob(), labels=None) == 1
    assert fwd(lib, prob(), hidden=FAKE + 2) == 2           # not 16-byte aligned
    assert fwd(lib, prob(), wsp=None) == 3
    assert fwd(lib, prob(), wsb=100) == 3
    assert fwd(lib, prob(), wsp=FAKE + 8) == 3


def test_forward_backward_rejects(lib):
    p = prob(reduction=0)
    code = lib.lce_forward_backward(ctypes.byref(p), FAKE, FAKE, None, FAKE, 1.0, FAKE, None, None, None, FAKE,
                                    FAKE, None, None, None, None, FAKE, 1 << 40, None)
    assert code == 2  # reduction NONE has no backward here
    p = prob()
    code = lib.lce_forward_backward(ctypes.byref(p), FAKE, FAKE, None, FAKE, 1.0, FAKE, None, None, None, FAKE,
                                    FAKE, FAKE, None, None, None, FAKE, 1 << 40, None)
    assert code == 1  # grad_bias without bias
    code = lib.lce_forward_backward(ctypes.byref(p), FAKE, FAKE, None, FAKE, 1.0, FAKE, None, None, None, FAKE,
                                    FAKE, None, None, None, None, FAKE, 64, None)
    assert code == 3  # workspace too small


def test_python_layer_mirrors_page_rules():
    h = torch.zeros(4, 64, dtype=torch.bfloat16)
    w = torch.zeros(8, 64, dtype=torch.bfloat16)
    y = torch.zeros(4, dtype=torch.int64)
    for bad in (0, -1):
        with pytest.raises(ValueError, match="must be positive"):
            lce._problem(h, w, y, -100, bad, "sum", None)
    p = lce._problem(h, w, y, -100, None, "sum", None)
    assert p.chunk_rows == 4            # None: one chunk of all rows
    with pytest.raises(ValueError):
        lce._problem(h.float(), w, y, -100, 256, "sum", None)
    with pytest.raises(ValueError):
        lce._problem(h, w, y, -100, 256, "avg", None)
    with pytest.raises(ValueError):
        lce.lce_forward(h, w, None, y)  # CPU tensors are refused, nothing is launched


def _opts(row_scale=None, accumulate=0, reserved=0):
    o = _lib.LceBackwardOptions()
    o.row_scale = row_scale
    o.accumulate = accumulate
    o.reserved = reserved
    return o


def _fbx(lib, p, opts, gw=None, gw32=None):
    return lib.lce_forward_backward_ex(ctypes.byref(p), FAKE, FAKE, None, FAKE, 1.0, FAKE, None, None, None,
                                       None, gw, None, gw32, None, None, FAKE, 1 << 40, None,
                                       None if opts is None else ctypes.byref(opts), None)


def test_forward_backward_ex_host_errors(lib):
    """Rejected on the host, before anything is enqueued."""
    assert _fbx(lib, prob(reduction=0), None) == 2                  # NONE needs per-row scales
    assert _fbx(lib, prob(reduction=0), _opts()) == 2
    assert _fbx(lib, prob(), _opts(reserved=1)) == 1
    assert _fbx(lib, prob(), _opts(accumulate=1), gw=FAKE) == 1     # accumulate without FP32 totals
    assert _fbx(lib, prob(), _opts(row_scale=FAKE + 2)) == 2        # misaligned row_scale
    assert _fbx(lib, prob(chunk_rows=0), _opts()) == 1


def test_scale_host_errors(lib):
    assert lib.lce_scale(FAKE, 0, -1, FAKE, None) == 1
    assert lib.lce_scale(None, 0, 10, FAKE, None) == 1
    assert lib.lce_scale(FAKE, 0, 10, None, None) == 1
    assert lib.lce_scale(FAKE, 7, 10, FAKE, None) == 1
    assert lib.lce_scale(None, 0, 0, None, None) == 0                # nothing to do
