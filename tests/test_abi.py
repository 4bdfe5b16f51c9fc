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
    assert lib.lce_abi_version() == 105
    for code in range(7):
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


def _up(x, m):
    return (x + m - 1) // m * m


def group_rows(n, rows_in_flight=0):
    """The backward row group the library uses (rounded to 256-row tiles):
    the caller's rows_in_flight, else 16384 rows but at most a quarter of
    the rows (at least one tile)."""
    np_ = _up(n, 256)
    if rows_in_flight > 0:
        g = _up(min(rows_in_flight, 1 << 20), 256)
    else:
        g = min(16384, max(256, np_ // 4 // 256 * 256))
    return min(g, np_)


def layout(n, h, v, kind, rows_in_flight=0, chunk_rows=256):
    """The workspace regions, in order, as the library carves them (each
    start 256-byte aligned). kind 0 forward, 1 backward with the FP32
    grad_weight inside, 2 backward with caller FP32 buffers."""
    np_, vp = _up(n, 256), _up(v, 256)
    n_vt = vp // 256
    bwd = kind in (1, 2)
    g = group_rows(n, rows_in_flight)
    part_rows = g if bwd else np_
    regions = [("label32", np_ * 4), ("n_valid", 8), ("status", 4), ("zy2", np_ * 4), ("lse", np_ * 4),
               ("part_m", 4 * n_vt * part_rows * 4), ("part_s", 4 * n_vt * part_rows * 4),
               ("chunk_acc", -(-n // chunk_rows) * 8), ("tile_ctr", 32)]
    if bwd:
        split_max = min(8, g // 256)
        n_tiles = n_vt * -(-h // 256)
        items = min(256, n_tiles * split_max) if split_max >= 2 else 0
        regions += [("zlab", np_ * 4), ("block_cnt", np_ // 256 * 4), ("block_off", np_ // 256 * 4),
                    ("perm", np_ * 4), ("labp", np_ * 4), ("hperm", np_ * h * 2),
                    ("wT", h * vp * 2), ("hT", h * g * 2), ("gw_part", items * 256 * 256 * 4),
                    ("dlog", g * vp * 2), ("gb_f32", vp * 4), ("rref", g * 4), ("rowc", g * 4), ("ovf", 4)]
        if kind == 1:
            regions.append(("gw_f32", v * h * 4))
    off = 0
    for _, b in regions:   # regions of 1 MiB or more start on 2 MiB boundaries
        if b >= 1 << 20:
            off = _up(off, 2 << 20)
        off = _up(off + b, 256)
    return dict(regions), off


@pytest.mark.parametrize("name", ["tiny", "qwen3_0p6b_head", "qwen3_4b_32k", "qwen3_4b_160k", "qwen3_8b_1m_shard"])
@pytest.mark.parametrize("rif", [0, 4096])
def test_workspace_layout(lib, name, rif):
    """lce_workspace_bytes is exactly the documented regions."""
    w = WORKLOADS[name]
    for kind in (0, 1, 2):
        _, total = layout(w.n_rows, w.hidden, w.vocab, kind, rif, w.chunk_rows)
        assert ws(lib, prob(w.n_rows, w.hidden, w.vocab, rows_in_flight=rif, chunk_rows=w.chunk_rows), kind) \
            == total, (name, kind)


@pytest.mark.parametrize("name", ["tiny", "qwen3_0p6b_head", "qwen3_4b_32k", "qwen3_4b_160k", "qwen3_8b_1m_shard"])
def test_no_full_logits_buffer(lib, name):
    """No [N, V] logits at any size: with the default row group every
    logits-shaped region (the group's bf16 softmax numerators, the per-tile
    max / sum-exp partials) is below half a bf16 [N, V], and the whole
    backward workspace beside the FP32 grad_weight the method keeps is below
    FP32 [N, V] logits for every workload but the tiny one (whose [N, V] is
    smaller than its [V, H] head)."""
    w = WORKLOADS[name]
    n, h, v = w.n_rows, w.hidden, w.vocab
    nv2 = n * v * 2
    for kind in (0, 1, 2):
        regions, total = layout(n, h, v, kind, 0, w.chunk_rows)
        assert ws(lib, prob(n, h, v, chunk_rows=w.chunk_rows), kind) == total
        for r in ("dlog", "part_m", "part_s"):
            if r in regions:
                assert regions[r] <= nv2 // 2, (name, kind, r, regions[r], nv2)
        if name != "tiny":
            assert total < 2 * nv2, (name, kind, total, 2 * nv2)
    # a caller may trade memory for speed explicitly (rows_in_flight), up to all rows at once
    regions, _ = layout(n, h, v, 1, n, w.chunk_rows)
    assert regions["dlog"] == _up(n, 256) * _up(v, 256) * 2


def test_group_rows_default():
    assert [group_rows(n) for n in (1, 256, 257, 1000, 1024, 2048, 32768, 65536, 131072, 163840)] == \
        [256, 256, 256, 256, 256, 512, 8192, 16384, 16384, 16384]
    assert group_rows(1000, 512) == 512 and group_rows(300, 4096) == 512 and group_rows(10, 1) == 256


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


def test_python_layer_rejects_bad_bias_labels_and_outputs():
    """The binding checks what the C ABI cannot see through raw pointers:
    bias dtype / shape / layout, label layout and caller-given outputs."""
    n, h, v = 6, 64, 10
    hid = torch.zeros(n, h, dtype=torch.bfloat16)
    w = torch.zeros(v, h, dtype=torch.bfloat16)
    y = torch.zeros(n, dtype=torch.int64)
    lce._problem(hid, w, y, -100, 256, "sum", None, torch.zeros(v, dtype=torch.bfloat16))   # accepted
    for bad in (torch.zeros(v, dtype=torch.float32),                # an FP32 master bias
                torch.zeros(v - 1, dtype=torch.bfloat16),           # shorter than V
                torch.zeros(v + 1, dtype=torch.bfloat16),
                torch.zeros(v, 2, dtype=torch.bfloat16)[:, 0],      # strided
                torch.zeros(1, v, dtype=torch.bfloat16)):           # not 1-D
        with pytest.raises(ValueError, match="bias"):
            lce._problem(hid, w, y, -100, 256, "sum", None, bad)
    with pytest.raises(ValueError, match="labels"):
        lce._problem(hid, w, torch.zeros(2 * n, dtype=torch.int64)[::2], -100, 256, "sum", None)
    with pytest.raises(ValueError, match="labels"):
        lce._problem(hid, w, torch.zeros(n, dtype=torch.int32), -100, 256, "sum", None)

    def good_out():
        return lce.LceOutput(torch.empty(()), torch.empty(n), torch.empty(1), torch.empty((), dtype=torch.int64),
                             torch.empty((), dtype=torch.int32), torch.empty(n, h, dtype=torch.bfloat16),
                             torch.empty(v, h, dtype=torch.bfloat16), torch.empty(v, dtype=torch.bfloat16),
                             torch.empty(v, h), torch.empty(v))
    dev = hid.device
    lce._check_out(good_out(), n, h, v, "sum", 256, dev)
    for field, bad in (("loss", torch.empty(n)), ("lse", torch.empty(n + 1)), ("chunk_loss", torch.empty(2)),
                       ("n_valid", torch.empty((), dtype=torch.int32)), ("status", None),
                       ("grad_hidden", torch.empty(n, h)), ("grad_weight", torch.empty(h, v, dtype=torch.bfloat16)),
                       ("grad_bias", torch.empty(v - 1, dtype=torch.bfloat16)),
                       ("grad_weight_f32", torch.empty(v, h, dtype=torch.bfloat16)),
                       ("grad_bias_f32", torch.empty(2 * v)[::2])):
        o = good_out()
        setattr(o, field, bad)
        with pytest.raises(ValueError, match=field):
            lce._check_out(o, n, h, v, "sum", 256, dev)
    o = good_out()
    o.loss = torch.empty(n)
    lce._check_out(o, n, h, v, "none", 256, dev)   # per-row loss for reduction none
    with pytest.raises(ValueError, match="workspace"):
        lce._check_workspace(torch.empty(16, dtype=torch.float32), dev)


def test_noalloc_rejects_on_the_host(lib):
    """The allocation-free forward refuses, before touching any device, a
    problem whose workspace cannot fit its fixed scratch even 256 rows at a
    time (12 bytes per row alone pass 64 MiB near 5.6M rows), and reports
    argument errors like lce_forward."""
    def call(p):
        return lib.lce_forward_noalloc(ctypes.byref(p), FAKE, FAKE, None, FAKE, FAKE, None, None, None, None, None)
    assert call(prob(n=6_000_000, h=64, v=4096)) == _lib.LCE_ERR_TOO_LARGE
    assert call(prob(n=512, h=64, v=1 << 22)) == _lib.LCE_ERR_TOO_LARGE     # 256 rows of partials alone: 128 MiB
    assert call(prob(chunk_rows=0)) == _lib.LCE_ERR_INVALID_ARG
    assert call(prob(dtype=1)) == _lib.LCE_ERR_UNSUPPORTED
    assert lib.lce_forward_noalloc(None, FAKE, FAKE, None, FAKE, FAKE, None, None, None, None, None) == 1
    assert _lib.LCE_NOALLOC_SCRATCH_BYTES == 64 << 20
