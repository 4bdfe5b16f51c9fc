"""GPU parity: the HIP path through the C ABI against the float64 oracle, on
seeded inputs that span several 256 x 256 tiles with ragged row and
vocabulary tails, plus the edge cases of the method."""
import math

import numpy as np
import pytest
import torch

import chunked_lm_head_lce_amd as lce
from gpu_helpers import (assert_grad_close, assert_loss_close, assert_rows_close, np32, say, to_device)
from lce_inputs import IGNORE_INDEX, make_case
from oracle import lce_oracle as O

pytestmark = pytest.mark.gpu


def oracle_of(inp, reduction="sum", grad_scale=1.0, chunk_rows=256):
    b = inp.bias_f32()
    return O.forward_backward(inp.hidden_f32(), inp.weight_f32(), b, inp.labels, reduction=reduction,
                              grad_scale=grad_scale, chunk_rows=chunk_rows)


def check_all(out, ref, inp, reduction, grads=True):
    assert int(out.n_valid.item()) == ref.n_valid
    assert int(out.status.item()) == 0
    if reduction == "none":
        assert_rows_close(np32(out.loss), ref.row_loss, "row loss")
    else:
        assert_loss_close(float(out.loss.item()), ref.loss)
    assert_rows_close(np32(out.lse), ref.lse, "lse")
    if grads:
        assert_grad_close(np32(out.grad_hidden), ref.grad_hidden, "grad_hidden")
        assert_grad_close(np32(out.grad_weight), ref.grad_weight, "grad_weight")
        if inp.bias_bits is not None:
            assert_grad_close(np32(out.grad_bias), ref.grad_bias, "grad_bias")


# (N, H, V): several tiles, ragged tails in rows and vocabulary, H not a
# multiple of the 256 tile
SHAPES = [(600, 256, 5000), (300, 128, 1000), (257, 64, 300), (512, 320, 4096), (40, 192, 130)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("bias", [False, True])
def test_forward_backward_sum(cuda, shape, bias):
    n, h, v = shape
    say(f"[gpu] forward_backward sum shape={shape} bias={bias}")
    inp = make_case(n, h, v, seed=n + v, bias_std=(0.05 if bias else None), ignore_frac=0.1, weight_std=0.05)
    hd, wd, bd, yd = to_device(inp, cuda)
    out = lce.lce_forward_backward(hd, wd, bd, yd, reduction="sum")
    torch.cuda.synchronize()
    check_all(out, oracle_of(inp, "sum"), inp, "sum")


@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_grad_scale_and_mean(cuda, reduction):
    say(f"[gpu] grad_scale reduction={reduction}")
    inp = make_case(700, 128, 2100, seed=5, bias_std=0.1, ignore_frac=0.3, weight_std=0.1)
    hd, wd, bd, yd = to_device(inp, cuda)
    out = lce.lce_forward_backward(hd, wd, bd, yd, reduction=reduction, grad_scale=0.37)
    torch.cuda.synchronize()
    check_all(out, oracle_of(inp, reduction, grad_scale=0.37), inp, reduction)


def test_forward_only_all_reductions(cuda):
    inp = make_case(520, 192, 3000, seed=9, bias_std=0.02, ignore_frac=0.15)
    hd, wd, bd, yd = to_device(inp, cuda)
    for reduction in ("none", "sum", "mean"):
        say(f"[gpu] forward reduction={reduction}")
        ref = O.forward(inp.hidden_f32(), inp.weight_f32(), inp.bias_f32(), inp.labels, reduction=reduction,
                        chunk_rows=100)
        out = lce.lce_forward(hd, wd, bd, yd, reduction=reduction, chunk_rows=100, want_chunk_loss=True)
        torch.cuda.synchronize()
        check_all(out, ref, inp, reduction, grads=False)
        assert_rows_close(np32(out.chunk_loss), ref.chunk_loss, "chunk sums")
        assert out.chunk_loss.numel() == math.ceil(520 / 100)


def test_chunk_rows_invariance(cuda):
    """Rows split cleanly: the chunk size only changes the chunk sums."""
    inp = make_case(900, 128, 1500, seed=11, bias_std=0.05)
    hd, wd, bd, yd = to_device(inp, cuda)
    outs = {}
    for c in (1, 100, 256, 900, 4096):
        say(f"[gpu] chunk_rows={c}")
        o = lce.lce_forward_backward(hd, wd, bd, yd, chunk_rows=c, want_chunk_loss=True)
        torch.cuda.synchronize()
        outs[c] = o
        assert o.chunk_loss.numel() == math.ceil(900 / c)
        assert abs(float(o.chunk_loss.double().sum()) - float(o.loss.item())) <= 1e-5 * abs(float(o.loss.item()))
    ref = outs[256]
    for c, o in outs.items():
        assert int(o.n_valid.item()) == int(ref.n_valid.item())
        assert_loss_close(float(o.loss.item()), float(ref.loss.item()))
        assert torch.equal(o.grad_hidden, ref.grad_hidden)   # same kernels, same order: identical
        assert_grad_close(np32(o.grad_weight), np32(ref.grad_weight), f"grad_weight c={c}")


def test_row_groups_match(cuda):
    """rows_in_flight only changes how many rows' dlogits are alive at once."""
    inp = make_case(1100, 128, 1300, seed=12, bias_std=0.05, ignore_frac=0.05)
    hd, wd, bd, yd = to_device(inp, cuda)
    ref = oracle_of(inp)
    for g in (256, 512, 0):
        say(f"[gpu] rows_in_flight={g}")
        out = lce.lce_forward_backward(hd, wd, bd, yd, rows_in_flight=g)
        torch.cuda.synchronize()
        check_all(out, ref, inp, "sum")


@pytest.mark.parametrize("reduction,want_lse", [("sum", True), ("sum", False), ("mean", False)])
def test_mostly_ignored_rows(cuda, reduction, want_lse):
    """A masked prompt plus scattered ignored rows (70% in all) over six row
    groups: the backward works on the labelled rows only (valid rows first,
    stopping at the device-side count), so whole groups and tiles have no
    work; every output must still match the oracle, ignored rows' grad_hidden
    must be exactly zero and, when asked for, their lse must be right too."""
    import dataclasses
    inp = make_case(1500, 128, 3000, seed=44, bias_std=0.05, ignore_frac=0.1, weight_std=0.05)
    y = inp.labels.copy()
    y[:900] = IGNORE_INDEX                                   # the prompt
    inp = dataclasses.replace(inp, labels=y)
    hd, wd, bd, yd = to_device(inp, cuda)
    say(f"[gpu] mostly ignored rows reduction={reduction} lse={want_lse}")
    out = lce.lce_forward_backward(hd, wd, bd, yd, reduction=reduction, rows_in_flight=256, want_lse=want_lse,
                                   want_chunk_loss=True)
    torch.cuda.synchronize()
    ref = oracle_of(inp, reduction)
    assert int(out.n_valid.item()) == ref.n_valid == int((y >= 0).sum())
    assert_loss_close(float(out.loss.item()), ref.loss)
    assert_rows_close(np32(out.chunk_loss), ref.chunk_loss, "chunk sums")
    if want_lse:
        assert_rows_close(np32(out.lse), ref.lse, "lse, every row")
    assert_grad_close(np32(out.grad_hidden), ref.grad_hidden, "grad_hidden")
    assert_grad_close(np32(out.grad_weight), ref.grad_weight, "grad_weight")
    assert_grad_close(np32(out.grad_bias), ref.grad_bias, "grad_bias")
    ign = torch.from_numpy(y == IGNORE_INDEX).to(cuda)
    assert torch.count_nonzero(out.grad_hidden[ign]) == 0


def test_no_valid_rows_backward(cuda):
    """Every row ignored: zero loss and zero gradients from a backward that
    has no row to work on."""
    inp = make_case(700, 128, 900, seed=45, bias_std=0.05, ignore_frac=0.0)
    hd, wd, bd, _ = to_device(inp, cuda)
    yd = torch.full((700,), IGNORE_INDEX, dtype=torch.int64, device=cuda)
    for reduction in ("sum", "mean"):
        say(f"[gpu] no valid rows, {reduction}")
        out = lce.lce_forward_backward(hd, wd, bd, yd, reduction=reduction, rows_in_flight=256, want_f32=True)
        torch.cuda.synchronize()
        assert int(out.n_valid.item()) == 0 and float(out.loss.item()) == 0.0
        for t in (out.grad_hidden, out.grad_weight, out.grad_bias, out.grad_weight_f32, out.grad_bias_f32):
            assert torch.count_nonzero(t) == 0


def test_confident_rows_have_nonnegative_loss(cuda):
    """Rows whose label logit exceeds every other logit by ~30 have a loss of
    ~1e-9. The label logit is taken from the same FP32 accumulators that
    give the row's maximum and sum, so l_i = lse_i - z_{i,y_i} can round to
    0 but never below it; it must also match the oracle to ~1e-6."""
    import dataclasses
    from lce_inputs import bf16_bits
    inp = make_case(600, 256, 5000, seed=41, bias_std=0.05, ignore_frac=0.1, weight_std=0.05)
    h = inp.hidden_f32().copy()
    w = inp.weight_f32()
    conf = np.flatnonzero(inp.labels >= 0)[::3]                 # a third of the valid rows
    h[conf] = 50.0 * w[inp.labels[conf]]
    inp = dataclasses.replace(inp, hidden_bits=bf16_bits(h))
    ref = oracle_of(inp)
    assert ref.row_loss[conf].max() < 1e-6
    hd, wd, bd, yd = to_device(inp, cuda)
    say("[gpu] confident rows: forward, reduction none")
    f = lce.lce_forward(hd, wd, bd, yd, reduction="none")
    say("[gpu] confident rows: forward_backward")
    out = lce.lce_forward_backward(hd, wd, bd, yd)
    torch.cuda.synchronize()
    rl = np32(f.loss)
    assert rl.min() >= 0.0, rl.min()
    np.testing.assert_allclose(rl[conf], ref.row_loss[conf], rtol=0, atol=2e-6)
    assert_rows_close(rl, ref.row_loss, "row loss")
    check_all(out, ref, inp, "sum")


def test_split_last_group_without_f32_outputs(cuda):
    """The path the benchmark times, at a small size: several row groups,
    grad_weight's last round split along K (274 vocabulary tiles on 256
    CUs leave 18, each split 2 ways: 8 K stages of 64 rows in each group),
    the second group adding into the FP32 accumulator (first = 0) and, with
    no FP32 output requested, writing only the bf16 result (keep32 = 0)."""
    inp = make_case(1000, 256, 70000, seed=31, bias_std=0.05, ignore_frac=0.1, weight_std=0.05)
    hd, wd, bd, yd = to_device(inp, cuda)
    say("[gpu] split last group: bf16 outputs only")
    out = lce.lce_forward_backward(hd, wd, bd, yd, rows_in_flight=512, want_f32=False)
    say("[gpu] split last group: with FP32 outputs")
    o32 = lce.lce_forward_backward(hd, wd, bd, yd, rows_in_flight=512, want_f32=True)
    torch.cuda.synchronize()
    assert out.grad_weight_f32 is None and o32.grad_weight_f32 is not None
    check_all(out, oracle_of(inp), inp, "sum")
    assert torch.equal(out.grad_hidden, o32.grad_hidden)
    assert torch.equal(out.grad_weight, o32.grad_weight_f32.to(torch.bfloat16))
    assert torch.equal(o32.grad_weight, o32.grad_weight_f32.to(torch.bfloat16))


@pytest.mark.parametrize("g,reduction", [(256, "sum"), (0, "sum"), (256, "mean")])
def test_far_label_logit_retry(cuda, g, reduction):
    """Rows whose largest logit lies far above their label logit (over 60):
    the stored softmax numerators would leave their range, so the group is
    recomputed against the row's lse. The results must not notice."""
    import dataclasses
    from lce_inputs import bf16_bits
    inp = make_case(700, 128, 1500, seed=23, bias_std=0.05, ignore_frac=0.1)
    h = inp.hidden_f32().copy()
    w = inp.weight_f32().copy()
    y = inp.labels.copy()
    # rows 5 and 600 (different row groups at 256 rows per group): logit of
    # id 7 is 128 * 1.0 = 128, label id 9 has logit 0
    for r in (5, 600):
        h[r, :] = 1.0
        y[r] = 9
    w[7, :] = 1.0
    w[9, :] = 0.0
    inp = dataclasses.replace(inp, hidden_bits=bf16_bits(h), weight_bits=bf16_bits(w), labels=y)
    hd, wd, bd, yd = to_device(inp, cuda)
    say(f"[gpu] far label logit, rows_in_flight={g}, {reduction}")
    out = lce.lce_forward_backward(hd, wd, bd, yd, rows_in_flight=g, reduction=reduction)
    torch.cuda.synchronize()
    ref = oracle_of(inp, reduction=reduction)
    # without the retry these rows' stored values would be capped at e^60
    # and their gradients off by a factor of about e^-68
    assert ref.row_loss[5] > 100 and ref.row_loss[600] > 100
    check_all(out, ref, inp, reduction)


@pytest.mark.parametrize("g", [256, 0])
def test_reference_sum_fallback(cuda, g):
    """Rows whose label logit lies 59 below 100 other logits: no value is
    more than 60 above the reference (no retry), but their sums against it
    exceed e^60, so those row blocks take their sums against the maximum
    instead. The results must not notice."""
    import dataclasses
    from lce_inputs import bf16_bits
    inp = make_case(700, 128, 1500, seed=27, bias_std=None, ignore_frac=0.1)
    h = inp.hidden_f32().copy()
    w = inp.weight_f32().copy()
    y = inp.labels.copy()
    for r in (3, 300, 650):
        h[r, :] = 1.0
        y[r] = 9
    w[100:200, :] = 59.0 / 128.0      # 0.4609375 in bf16: 128 * it = 59
    w[9, :] = 0.0
    inp = dataclasses.replace(inp, hidden_bits=bf16_bits(h), weight_bits=bf16_bits(w), labels=y)
    hd, wd, bd, yd = to_device(inp, cuda)
    say(f"[gpu] reference-sum fallback, rows_in_flight={g}")
    out = lce.lce_forward_backward(hd, wd, bd, yd, rows_in_flight=g)
    torch.cuda.synchronize()
    ref = oracle_of(inp)
    assert all(55 < ref.row_loss[r] < 60 + math.log(100) + 1 for r in (3, 300, 650))
    check_all(out, ref, inp, "sum")


def test_strided_hidden_and_weight(cuda):
    inp = make_case(300, 128, 700, seed=13, bias_std=0.05)
    hd, wd, bd, yd = to_device(inp, cuda)
    hw = torch.zeros(300, 200, dtype=torch.bfloat16, device=cuda)
    hw[:, :128] = hd
    ww = torch.zeros(700, 136, dtype=torch.bfloat16, device=cuda)
    ww[:, :128] = wd
    say("[gpu] strided operands")
    out = lce.lce_forward_backward(hw[:, :128], ww[:, :128], bd, yd)
    torch.cuda.synchronize()
    check_all(out, oracle_of(inp), inp, "sum")


def test_optional_outputs_and_f32(cuda):
    inp = make_case(400, 128, 900, seed=14, bias_std=0.05)
    hd, wd, bd, yd = to_device(inp, cuda)
    ref = oracle_of(inp)
    say("[gpu] only grad_hidden")
    o = lce.lce_forward_backward(hd, wd, bd, yd, want_grad_weight=False, want_grad_bias=False)
    torch.cuda.synchronize()
    assert o.grad_weight is None and o.grad_bias is None
    assert_grad_close(np32(o.grad_hidden), ref.grad_hidden, "grad_hidden")
    say("[gpu] grad_bias without grad_weight (its own column-sum pass)")
    o = lce.lce_forward_backward(hd, wd, bd, yd, want_grad_hidden=False, want_grad_weight=False,
                                 want_grad_bias=True, rows_in_flight=256)
    torch.cuda.synchronize()
    assert o.grad_weight is None and o.grad_hidden is None
    assert_grad_close(np32(o.grad_bias), ref.grad_bias, "grad_bias alone")
    say("[gpu] only weight grads, fp32 exposed")
    o = lce.lce_forward_backward(hd, wd, bd, yd, want_grad_hidden=False, want_f32=True)
    torch.cuda.synchronize()
    assert_grad_close(np32(o.grad_weight_f32), ref.grad_weight, "grad_weight_f32")
    assert_grad_close(np32(o.grad_bias_f32), ref.grad_bias, "grad_bias_f32")
    assert torch.equal(o.grad_weight, o.grad_weight_f32.to(torch.bfloat16))   # one RNE cast
    assert torch.equal(o.grad_bias, o.grad_bias_f32.to(torch.bfloat16))
    assert_loss_close(float(o.loss.item()), ref.loss)


def test_zero_weight_closed_form(cuda):
    """W = 0, b = 0: l_i = ln V; grad_hidden = 0; grad_bias_j = n_valid/V - count_j."""
    n, h, v = 300, 64, 1000
    inp = make_case(n, h, v, seed=15, bias_std=0.1, ignore_frac=0.2)
    hd, _, _, yd = to_device(inp, cuda)
    wd = torch.zeros(v, h, dtype=torch.bfloat16, device=cuda)
    bd = torch.zeros(v, dtype=torch.bfloat16, device=cuda)
    say("[gpu] zero weight closed form")
    o = lce.lce_forward_backward(hd, wd, bd, yd, want_f32=True)
    torch.cuda.synchronize()
    nv = int((inp.labels != IGNORE_INDEX).sum())
    assert int(o.n_valid.item()) == nv
    assert abs(float(o.loss.item()) - nv * math.log(v)) <= 1e-6 * nv * math.log(v)
    assert np.allclose(np32(o.lse), math.log(v), rtol=1e-6)
    assert torch.count_nonzero(o.grad_hidden) == 0
    counts = np.bincount(inp.labels[inp.labels >= 0], minlength=v)
    np.testing.assert_allclose(np32(o.grad_bias_f32), nv / v - counts, atol=1e-5)


def test_all_rows_ignored(cuda):
    inp = make_case(300, 64, 500, seed=16, bias_std=0.1, ignore_frac=0.0)
    hd, wd, bd, _ = to_device(inp, cuda)
    yd = torch.full((300,), IGNORE_INDEX, dtype=torch.int64, device=cuda)
    for reduction in ("mean", "sum"):
        say(f"[gpu] all ignored {reduction}")
        o = lce.lce_forward_backward(hd, wd, bd, yd, reduction=reduction)
        torch.cuda.synchronize()
        assert float(o.loss.item()) == 0.0 and int(o.n_valid.item()) == 0
        assert torch.count_nonzero(o.grad_hidden) == 0
        assert torch.count_nonzero(o.grad_weight) == 0 and torch.count_nonzero(o.grad_bias) == 0


def test_custom_ignore_index(cuda):
    inp = make_case(300, 64, 500, seed=17, ignore_frac=0.0)
    y = inp.labels.copy()
    y[::7] = 7          # rows labelled 7 are treated as ignored
    ref = O.forward_backward(inp.hidden_f32(), inp.weight_f32(), None, y, ignore_index=7)
    hd, wd, _, _ = to_device(inp, cuda)
    say("[gpu] ignore_index=7")
    o = lce.lce_forward_backward(hd, wd, None, torch.from_numpy(y).to(cuda), ignore_index=7)
    torch.cuda.synchronize()
    check_all(o, ref, inp, "sum")


def test_label_out_of_range_sets_status(cuda):
    inp = make_case(300, 64, 500, seed=18, ignore_frac=0.1)
    y = inp.labels.copy()
    y[5] = 500
    y[17] = -3
    hd, wd, _, _ = to_device(inp, cuda)
    say("[gpu] label out of range")
    o = lce.lce_forward_backward(hd, wd, None, torch.from_numpy(y).to(cuda))
    torch.cuda.synchronize()
    assert int(o.status.item()) == lce._lib.LCE_ERR_LABEL_RANGE
    assert math.isnan(float(o.loss.item()))
    assert int(o.n_valid.item()) == int(((y >= 0) & (y < 500)).sum())
    with pytest.raises(lce.LceError):
        o.check()
    # the bad rows were treated as ignored: their grad_hidden rows are zero
    assert torch.count_nonzero(o.grad_hidden[5]) == 0 and torch.count_nonzero(o.grad_hidden[17]) == 0
    # and a clean call afterwards reports OK again
    o2 = lce.lce_forward_backward(hd, wd, None, torch.from_numpy(inp.labels).to(cuda))
    torch.cuda.synchronize()
    assert int(o2.status.item()) == 0 and not math.isnan(float(o2.loss.item()))


@pytest.mark.parametrize("shape", [(1, 64, 1), (1, 64, 7), (3, 64, 256), (256, 64, 256), (0, 64, 100)])
def test_degenerate_shapes(cuda, shape):
    n, h, v = shape
    say(f"[gpu] degenerate {shape}")
    inp = make_case(n, h, v, seed=19, bias_std=0.1, ignore_frac=0.0)
    hd, wd, bd, yd = to_device(inp, cuda)
    o = lce.lce_forward_backward(hd, wd, bd, yd)
    torch.cuda.synchronize()
    ref = oracle_of(inp)
    assert int(o.n_valid.item()) == ref.n_valid
    if n == 0:
        assert float(o.loss.item()) == 0.0
        assert torch.count_nonzero(o.grad_weight) == 0 and torch.count_nonzero(o.grad_bias) == 0
        return
    if v == 1:   # one class: lse = z, every loss and gradient is zero
        assert abs(float(o.loss.item())) <= 1e-6
    else:
        assert_loss_close(float(o.loss.item()), ref.loss)
    assert_grad_close(np32(o.grad_hidden), ref.grad_hidden, "grad_hidden")
    assert_grad_close(np32(o.grad_weight), ref.grad_weight, "grad_weight")
    assert_grad_close(np32(o.grad_bias), ref.grad_bias, "grad_bias")


def test_repeatable(cuda):
    inp = make_case(800, 128, 2000, seed=20, bias_std=0.05)
    hd, wd, bd, yd = to_device(inp, cuda)
    say("[gpu] repeatability")
    a = lce.lce_forward_backward(hd, wd, bd, yd)
    b = lce.lce_forward_backward(hd, wd, bd, yd)
    torch.cuda.synchronize()
    assert int(a.n_valid.item()) == int(b.n_valid.item())
    assert torch.equal(a.grad_hidden, b.grad_hidden) and torch.equal(a.grad_weight, b.grad_weight)
    assert torch.equal(a.lse, b.lse)
    assert abs(float(a.loss.item()) - float(b.loss.item())) <= 1e-6 * abs(float(a.loss.item()))
    # grad_bias adds column sums with FP32 atomics: equal up to their order
    torch.testing.assert_close(a.grad_bias.float(), b.grad_bias.float(), rtol=1e-2, atol=1e-6)
    fa = lce.lce_forward(hd, wd, bd, yd, reduction="none")
    fb = lce.lce_forward(hd, wd, bd, yd, reduction="none")
    torch.cuda.synchronize()
    assert torch.equal(fa.loss, fb.loss) and torch.equal(fa.lse, fb.lse)
    # the fused call sums each labelled row against its label logit, the
    # forward alone against the row maximum: the same lse up to rounding
    torch.testing.assert_close(fa.lse, a.lse, rtol=2e-6, atol=2e-6)


# grad_bias summed inside grad_weight's K loop, each wave of a tile on R
# rows of every 64-row stage with R ceil(H / 256) >= 16: one hidden tile of
# 64 or 256 columns (R = 16); 2 and 3 tiles (R = 8, some rows past the stage
# at 3); 4 and 5 tiles (R = 4); 10 tiles (R = 2); 16 tiles, every wave on a
# row; 16 tiles of which the last holds 64 hidden columns (H = 3904); 17
# tiles, the waves of row 3 idle in most tiles; 65 tiles, the last tile has
# no row. Several row groups, a partial last stage and (fewer tiles than
# CUs) tiles split along K.
@pytest.mark.parametrize("shape", [(500, 64, 900), (700, 256, 1000), (300, 512, 800), (300, 768, 700),
                                   (300, 1024, 600), (300, 1280, 650), (300, 2560, 500), (700, 4096, 1000),
                                   (300, 3904, 700), (300, 4160, 600), (257, 16448, 300)])
def test_grad_bias_inside_grad_weight(cuda, shape):
    n, h, v = shape
    say(f"[gpu] grad_bias inside grad_weight shape={shape}")
    inp = make_case(n, h, v, seed=h + v, bias_std=0.05, ignore_frac=0.1, weight_std=0.02)
    hd, wd, bd, yd = to_device(inp, cuda)
    out = lce.lce_forward_backward(hd, wd, bd, yd, reduction="sum", rows_in_flight=256)
    torch.cuda.synchronize()
    check_all(out, oracle_of(inp, "sum"), inp, "sum")


# grad_hidden's tiles of a partial last round split along K (summed by a
# second kernel): 512-row groups of 8 tiles cut into 32 pieces each, with a
# partly labelled third group and an unlabelled fourth; 2 tiles cut into 16
# (the scratch's item count is the limit there).
@pytest.mark.parametrize("shape", [(2048, 1024, 8192), (2300, 256, 4000)])
def test_grad_hidden_split_pieces(cuda, shape):
    n, h, v = shape
    say(f"[gpu] grad_hidden K pieces shape={shape}")
    inp = make_case(n, h, v, seed=n + h, bias_std=0.05, ignore_frac=0.3, weight_std=0.05)
    hd, wd, bd, yd = to_device(inp, cuda)
    out = lce.lce_forward_backward(hd, wd, bd, yd, reduction="sum")
    again = lce.lce_forward_backward(hd, wd, bd, yd, reduction="sum")
    torch.cuda.synchronize()
    check_all(out, oracle_of(inp, "sum"), inp, "sum")
    assert torch.equal(out.grad_hidden, again.grad_hidden)   # fixed order of the pieces


def test_grad_weight_whole_and_split_tiles(cuda):
    """274 grad_weight tiles (V = 70000 over 256-row tiles, one column tile):
    on a GPU with fewer CUs the tiles past the last whole round are split
    along the rows of the group and summed by a second kernel; 700 rows end
    in a partial 64-row stage (zero rows of G and of the transposed h)."""
    n, h, v = 700, 256, 70000
    say(f"[gpu] grad_weight whole + split tiles shape={(n, h, v)}")
    inp = make_case(n, h, v, seed=71, bias_std=0.05, ignore_frac=0.05, weight_std=0.05)
    hd, wd, bd, yd = to_device(inp, cuda)
    out = lce.lce_forward_backward(hd, wd, bd, yd, reduction="sum")
    again = lce.lce_forward_backward(hd, wd, bd, yd, reduction="sum")
    torch.cuda.synchronize()
    check_all(out, oracle_of(inp, "sum"), inp, "sum")
    assert torch.equal(out.grad_weight, again.grad_weight)   # fixed summation order


# The forward tiles' order per XCD: blocks of 64 row tiles, then a remainder
# dealt out per column group (32..63 row tiles) or sliced (below 32). 104
# row tiles = one block + a dealt 40; 73 (ragged) = one block + a sliced 9;
# 54 = dealt only. Forward-only over all rows, and forward+backward with the
# whole input as one row group, compared in full with the oracle.
@pytest.mark.parametrize("n", [104 * 256, 73 * 256 - 100, 54 * 256 - 7])
def test_forward_tile_orders(cuda, n):
    h, v = 64, 1100
    say(f"[gpu] forward tile orders n={n} ({(n + 255) // 256} row tiles)")
    inp = make_case(n, h, v, seed=n, bias_std=0.05, ignore_frac=0.1, weight_std=0.05)
    hd, wd, bd, yd = to_device(inp, cuda)
    ref = oracle_of(inp, "sum")
    f = lce.lce_forward(hd, wd, bd, yd, reduction="sum")
    torch.cuda.synchronize()
    assert int(f.n_valid.item()) == ref.n_valid
    assert_loss_close(float(f.loss.item()), ref.loss)
    assert_rows_close(np32(f.lse), ref.lse, "forward-only lse")
    out = lce.lce_forward_backward(hd, wd, bd, yd, reduction="sum", rows_in_flight=n)
    torch.cuda.synchronize()
    check_all(out, ref, inp, "sum")
