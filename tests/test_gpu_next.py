"""GPU parity of the caller-side rows above the fused call: per-row upstream
gradients (reduction "none" backward), FP32 gradient accumulation across
micro-batches, the device-scalar scaling kernel, and the autograd wrapper,
all against the float64 oracle."""
import numpy as np
import pytest
import torch

import chunked_lm_head_lce_amd as lce
from gpu_helpers import assert_grad_close, assert_loss_close, assert_rows_close, np32, say, to_device
from lce_inputs import make_case
from oracle import lce_oracle as O

pytestmark = pytest.mark.gpu


def _case(seed=3, n=700, h=192, v=3000, bias=0.05, ignore=0.2):
    return make_case(n, h, v, seed=seed, bias_std=bias, ignore_frac=ignore, weight_std=0.05)


def _row_scale(n, seed):
    # per-token upstream gradients, some negative and some zero
    r = np.random.default_rng(seed).normal(size=n).astype(np.float32)
    r[::17] = 0.0
    return r


def _oracle(inp, reduction, grad_scale):
    return O.forward_backward(inp.hidden_f32(), inp.weight_f32(), inp.bias_f32(), inp.labels,
                              reduction=reduction, grad_scale=grad_scale, chunk_rows=256)


def _check_grads(gh, gw, gb, ref, inp):
    assert_grad_close(np32(gh), ref.grad_hidden, "grad_hidden")
    assert_grad_close(np32(gw), ref.grad_weight, "grad_weight")
    if inp.bias_bits is not None:
        assert_grad_close(np32(gb), ref.grad_bias, "grad_bias")


def test_row_scale_reduction_none(cuda):
    say("[gpu] row_scale with reduction none")
    inp = _case()
    hd, wd, bd, yd = to_device(inp, cuda)
    r = _row_scale(len(inp.labels), 11)
    out = lce.lce_forward_backward(hd, wd, bd, yd, reduction="none", row_scale=torch.from_numpy(r).to(cuda))
    torch.cuda.synchronize()
    ref = _oracle(inp, "none", r.astype(np.float64))
    assert int(out.n_valid.item()) == ref.n_valid
    assert_rows_close(np32(out.loss), ref.row_loss, "row loss")
    _check_grads(out.grad_hidden, out.grad_weight, out.grad_bias, ref, inp)


@pytest.mark.parametrize("reduction", ["sum", "mean"])
def test_row_scale_with_reduction(cuda, reduction):
    say(f"[gpu] row_scale with reduction {reduction}")
    inp = _case(seed=4)
    hd, wd, bd, yd = to_device(inp, cuda)
    n = len(inp.labels)
    r = _row_scale(n, 12)
    out = lce.lce_forward_backward(hd, wd, bd, yd, reduction=reduction, grad_scale=0.5,
                                   row_scale=torch.from_numpy(r).to(cuda))
    torch.cuda.synchronize()
    nv = int((inp.labels != -100).sum())
    s = 0.5 / max(nv, 1) if reduction == "mean" else 0.5
    # G_i = s * r_i * valid_i * (softmax - onehot): the oracle's per-row form
    ref = _oracle(inp, "none", s * r.astype(np.float64))
    assert_loss_close(float(out.loss.item()), _oracle(inp, reduction, 1.0).loss)
    _check_grads(out.grad_hidden, out.grad_weight, out.grad_bias, ref, inp)


def test_none_without_row_scale_is_unsupported(cuda):
    inp = _case(n=64, v=300)
    hd, wd, bd, yd = to_device(inp, cuda)
    with pytest.raises(lce.LceError):
        lce.lce_forward_backward(hd, wd, bd, yd, reduction="none")


def test_accumulate_two_micro_batches(cuda):
    say("[gpu] accumulate grad_weight / grad_bias over two micro-batches")
    a = _case(seed=5, n=600)
    b = _case(seed=6, n=333)
    # the same head for both micro-batches
    b.weight_bits = a.weight_bits
    b.bias_bits = a.bias_bits
    ha, wd, bd, ya = to_device(a, cuda)
    hb, _, _, yb = to_device(b, cuda)
    out = lce.lce_forward_backward(ha, wd, bd, ya, reduction="sum", accumulate=True)
    out2 = lce.lce_forward_backward(hb, wd, bd, yb, reduction="sum", accumulate=True,
                                    out=lce.LceOutput(out.loss.clone(), None, None, out.n_valid.clone(),
                                                      out.status.clone(), grad_hidden=torch.empty_like(hb),
                                                      grad_weight=out.grad_weight, grad_bias=out.grad_bias,
                                                      grad_weight_f32=out.grad_weight_f32,
                                                      grad_bias_f32=out.grad_bias_f32))
    torch.cuda.synchronize()
    ra, rb = _oracle(a, "sum", 1.0), _oracle(b, "sum", 1.0)
    assert_grad_close(np32(out2.grad_weight_f32), ra.grad_weight + rb.grad_weight, "accumulated grad_weight f32")
    assert_grad_close(np32(out2.grad_weight), ra.grad_weight + rb.grad_weight, "accumulated grad_weight")
    assert_grad_close(np32(out2.grad_bias_f32), ra.grad_bias + rb.grad_bias, "accumulated grad_bias")
    assert_grad_close(np32(out2.grad_hidden), rb.grad_hidden, "grad_hidden of the second micro-batch")


def test_accumulate_requires_f32_buffers(cuda):
    inp = _case(n=64, v=300)
    hd, wd, bd, yd = to_device(inp, cuda)
    o = lce.lce_forward_backward(hd, wd, bd, yd)
    with pytest.raises(ValueError):
        lce.lce_forward_backward(hd, wd, bd, yd, accumulate=True, out=o)   # no FP32 totals in `out`


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_scale_kernel(cuda, dtype):
    say(f"[gpu] lce_scale {dtype}")
    g = torch.Generator().manual_seed(7)
    x = torch.randn(100003, generator=g).to(dtype)
    s = torch.tensor([-0.37], dtype=torch.float32)
    want = (x.float() * s).to(dtype)          # fp32 product, one rounding to the storage type
    xd = x.to(cuda)
    lce.lce_scale(xd, s.to(cuda))
    torch.cuda.synchronize()
    assert torch.equal(xd.cpu(), want)


@pytest.mark.parametrize("reduction", ["sum", "mean", "none"])
def test_autograd_function(cuda, reduction):
    say(f"[gpu] autograd linear_cross_entropy reduction={reduction}")
    inp = _case(seed=8)
    hd, wd, bd, yd = to_device(inp, cuda)
    h = hd.clone().requires_grad_(True)
    w = wd.clone().requires_grad_(True)
    b = bd.clone().requires_grad_(True)
    loss = lce.linear_cross_entropy(h, w, yd, b, reduction=reduction)
    n = len(inp.labels)
    if reduction == "none":
        r = _row_scale(n, 13)
        loss.backward(torch.from_numpy(r).to(cuda))
        ref = _oracle(inp, "none", r.astype(np.float64))
        assert_rows_close(np32(loss), ref.row_loss, "row loss")
    else:
        (loss * 1.7).backward()
        ref = _oracle(inp, reduction, 1.7)
        assert_loss_close(float(loss.item()), _oracle(inp, reduction, 1.0).loss)
    torch.cuda.synchronize()
    _check_grads(h.grad, w.grad, b.grad, ref, inp)


def test_autograd_frozen_head(cuda):
    say("[gpu] autograd with a frozen head (no weight / bias gradient)")
    inp = _case(seed=9)
    hd, wd, bd, yd = to_device(inp, cuda)
    h = hd.clone().requires_grad_(True)
    loss = lce.linear_cross_entropy(h, wd, yd, bd, reduction="sum")
    loss.backward()
    torch.cuda.synchronize()
    ref = _oracle(inp, "sum", 1.0)
    assert_grad_close(np32(h.grad), ref.grad_hidden, "grad_hidden")
