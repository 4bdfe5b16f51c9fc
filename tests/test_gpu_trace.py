"""GPU checks of the traced entry points: per-launch events recorded on the
caller's stream, one (before, after) pair per kernel launch, and results
identical to the untraced calls."""
import ctypes

import pytest
import torch

import chunked_lm_head_lce_amd as lce
from chunked_lm_head_lce_amd import _lib
from gpu_helpers import say, to_device
from lce_inputs import make_case

pytestmark = pytest.mark.gpu


class _Events:
    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(ev)) == 0
            self.arr[i] = ev

    def ms(self, a, b):
        out = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), self.arr[a], self.arr[b]) == 0
        return float(out.value)

    def close(self):
        for ev in self.arr:
            self.hip.hipEventDestroy(ev)


def _trace(events, cap):
    t = _lib.LceTrace()
    kinds = (ctypes.c_int32 * cap)()
    dims = (ctypes.c_int64 * (3 * cap))()
    t.events = ctypes.cast(events.arr, ctypes.POINTER(ctypes.c_void_p))
    t.kinds = ctypes.cast(kinds, ctypes.POINTER(ctypes.c_int32))
    t.dims = ctypes.cast(dims, ctypes.POINTER(ctypes.c_int64))
    t.capacity = cap
    t.count = 0
    return t, kinds, dims


def test_traced_forward_backward_matches_untraced(cuda):
    n, h, v, g = 1100, 256, 3000, 512          # three row groups
    inp = make_case(n, h, v, seed=31, bias_std=0.05, ignore_frac=0.1)
    hd, wd, bd, yd = to_device(inp, cuda)
    cap = 64
    ev = _Events(2 * cap)
    try:
        t, kinds, dims = _trace(ev, cap)
        say("[gpu] traced forward+backward, 3 row groups")
        a = lce.lce_forward_backward(hd, wd, bd, yd, rows_in_flight=g, trace=t)
        b = lce.lce_forward_backward(hd, wd, bd, yd, rows_in_flight=g)
        torch.cuda.synchronize()
        assert torch.equal(a.grad_hidden, b.grad_hidden) and torch.equal(a.grad_weight, b.grad_weight)
        assert torch.equal(a.lse, b.lse)
        assert int(a.n_valid.item()) == int(b.n_valid.item())
        names = [_lib.KERNEL_KINDS[kinds[i]] for i in range(t.count)]
        groups = 3
        # per row group: the forward tiles, their retry (a no-op here), the
        # row scales (and their retry), both row-reference steps and the two
        # gradient products; grad_weight adds the grad_bias sums itself
        for k, per_group in (("fwd_lse", 1), ("fwd_retry", 1), ("bwd_dlogits", 2), ("row_ref", 2),
                             ("grad_hidden", 1), ("grad_weight", 1), ("finalize_rows", 1), ("bias_sums", 0)):
            assert names.count(k) == per_group * groups, (k, names)
        assert names.count("label_logit") == 1 and names.count("finalize_loss") == 1
        assert names.count("partition") == 1 and names.count("gather_rows") == 1   # valid rows first
        # product dims: grad_hidden rows x H x V, grad_weight V x H x the group's valid rows
        valid_rows = [g, g, n - 2 * g]
        gh = [i for i, k in enumerate(names) if k == "grad_hidden"]
        gw = [i for i, k in enumerate(names) if k == "grad_weight"]
        for j, i in enumerate(gh):
            assert (dims[3 * i], dims[3 * i + 1], dims[3 * i + 2]) == (valid_rows[j], h, v)
        for j, i in enumerate(gw):
            assert (dims[3 * i], dims[3 * i + 1], dims[3 * i + 2]) == (v, h, valid_rows[j])
        # every recorded pair has a non-negative duration, and launches are recorded in stream order
        for i in range(t.count):
            assert ev.ms(2 * i, 2 * i + 1) >= 0.0
            if i:
                assert ev.ms(2 * (i - 1) + 1, 2 * i) >= 0.0
    finally:
        ev.close()


# one hidden tile (16 rows per wave and stage), 3 tiles (8, some rows past
# the stage), 4 (4), 10 (2), 15 (2, some rows past) and 16 (1); then
# grad_bias without grad_weight, which takes the column-sum pass
@pytest.mark.parametrize("h,want_gw", [(256, True), (768, True), (1024, True), (2560, True), (3840, True),
                                       (4096, True), (768, False)])
def test_grad_bias_inside_grad_weight_trace(cuda, h, want_gw):
    """When grad_weight runs, its kernel adds the grad_bias column sums
    itself at every hidden size; without it, a column-sum pass per row group
    does. Same results as untraced either way."""
    n, v, g = 600, 700, 256                   # three row groups
    inp = make_case(n, h, v, seed=33, bias_std=0.05, ignore_frac=0.1, weight_std=0.02)
    hd, wd, bd, yd = to_device(inp, cuda)
    cap = 64
    ev = _Events(2 * cap)
    try:
        t, kinds, _ = _trace(ev, cap)
        say(f"[gpu] traced forward+backward at H={h}, grad_weight {want_gw}, 3 row groups")
        a = lce.lce_forward_backward(hd, wd, bd, yd, rows_in_flight=g, trace=t, want_grad_weight=want_gw,
                                     want_f32=True)
        b = lce.lce_forward_backward(hd, wd, bd, yd, rows_in_flight=g, want_grad_weight=want_gw, want_f32=True)
        torch.cuda.synchronize()
        names = [_lib.KERNEL_KINDS[kinds[i]] for i in range(t.count)]
        groups = 3
        assert names.count("grad_weight") == (groups if want_gw else 0), names
        assert names.count("bias_sums") == (0 if want_gw else groups), names
        if want_gw:
            assert torch.equal(a.grad_weight, b.grad_weight)
        assert torch.equal(a.grad_hidden, b.grad_hidden)
        # FP32 atomics: equal up to their order
        torch.testing.assert_close(a.grad_bias_f32, b.grad_bias_f32, rtol=1e-5, atol=1e-6)
    finally:
        ev.close()


def test_trace_capacity_limit(cuda):
    inp = make_case(600, 128, 1000, seed=32, bias_std=0.05)
    hd, wd, bd, yd = to_device(inp, cuda)
    ev = _Events(2 * 3)
    try:
        t, kinds, _ = _trace(ev, 3)
        say("[gpu] traced forward with a 3-launch capacity")
        a = lce.lce_forward(hd, wd, bd, yd, trace=t)
        b = lce.lce_forward(hd, wd, bd, yd)
        torch.cuda.synchronize()
        assert t.count == 3                        # stops recording silently at capacity
        assert abs(float(a.loss.item()) - float(b.loss.item())) <= 1e-6 * abs(float(b.loss.item()))
        assert torch.equal(a.lse, b.lse)
    finally:
        ev.close()
