"""GPU parity at the full workload sizes.

The two small workloads are compared with the oracle in full. The three
large ones (32k / 160k rows at H=2560, 131072 rows at H=4096, V=151936) are
compared on seeded subsets: every row's lse and the total loss against the
stored oracle values (tests/golden, written by ``python -m oracle.make_golden``),
grad_hidden on a row subset and grad_weight / grad_bias on a vocabulary
subset recomputed by the oracle on the CPU, plus properties that hold at any
size (sum_j grad_bias_j = 0, sum_j grad_weight[j,:] = 0 for a sum loss).
"""
import json
import os

import numpy as np
import pytest
import torch

import chunked_lm_head_lce_amd as lce
from gpu_helpers import (assert_grad_close, assert_loss_close, assert_rows_close, np32, say, to_device)
from lce_inputs import WORKLOADS, make_inputs, sample_cols, sample_rows
from oracle import lce_oracle as O

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _out_bytes(out) -> int:
    return sum(t.numel() * t.element_size() for t in (out.loss, out.lse, out.chunk_loss, out.n_valid, out.status,
                                                       out.grad_hidden, out.grad_weight, out.grad_bias,
                                                       out.grad_weight_f32, out.grad_bias_f32) if t is not None)


def _timed_call_with_peak(cuda, w, hd, wd, bd, yd, **kw):
    """The benchmark's call (loss and bf16 gradients only: no per-row lse,
    FP32 accumulators in workspace, default row group) with the peak HBM it
    adds beyond inputs and outputs; no [N, V] logits exist, so it stays
    below FP32 [N, V] logits."""
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated(cuda)
    torch.cuda.reset_peak_memory_stats(cuda)
    out = lce.lce_forward_backward(hd, wd, bd, yd, chunk_rows=w.chunk_rows, reduction=w.reduction,
                                   want_f32=False, want_lse=False, **kw)
    torch.cuda.synchronize()
    extra = torch.cuda.max_memory_allocated(cuda) - base - _out_bytes(out)
    logits32 = 4 * w.n_rows * w.vocab
    say(f"[gpu] workload {w.name}: peak extra HBM {extra / 1e9:.3f} GB, FP32 [N,V] logits {logits32 / 1e9:.3f} GB")
    assert extra < logits32, (extra, logits32)
    return out


def _check_row_losses(cuda, w, hd, wd, bd, yd, lse_ref=None):
    """Per-row losses from the forward: l_i >= 0 for every row (and exactly 0
    for ignored rows), and they add up to the loss."""
    say(f"[gpu] workload {w.name}: per-row losses")
    f = lce.lce_forward(hd, wd, bd, yd, chunk_rows=w.chunk_rows, reduction="none")
    torch.cuda.synchronize()
    rl = f.loss.double()
    ign = yd == -100
    if bool(ign.any()):
        assert float(rl[ign].abs().max()) == 0.0
    assert float(rl.min()) >= 0.0, f"negative per-row loss {float(rl.min())!r}"
    if lse_ref is not None:
        assert_rows_close(np32(f.lse), lse_ref, "lse (reduction none)")
    return float(rl.sum())


@pytest.mark.parametrize("name", ["tiny", "qwen3_0p6b_head"])
def test_small_workloads_full(cuda, name):
    w = WORKLOADS[name]
    say(f"[gpu] workload {name}: generating inputs")
    inp = make_inputs(w)
    hd, wd, bd, yd = to_device(inp, cuda)
    say(f"[gpu] workload {name}: running forward_backward")
    out = lce.lce_forward_backward(hd, wd, bd, yd, chunk_rows=w.chunk_rows, reduction=w.reduction,
                                   want_chunk_loss=True)
    torch.cuda.synchronize()
    if name != "tiny":   # the tiny workload's [N, V] is smaller than its [V, H] head
        timed = _timed_call_with_peak(cuda, w, hd, wd, bd, yd)
        assert torch.equal(timed.grad_hidden, out.grad_hidden)
        assert torch.equal(timed.grad_weight, out.grad_weight)
    row_sum = _check_row_losses(cuda, w, hd, wd, bd, yd)
    say(f"[gpu] workload {name}: oracle")
    ref = O.forward_backward(inp.hidden_f32(), inp.weight_f32(), inp.bias_f32(), inp.labels,
                             reduction=w.reduction, chunk_rows=w.chunk_rows)
    assert int(out.n_valid.item()) == ref.n_valid == w.n_rows - w.n_ignored
    assert_loss_close(float(out.loss.item()), ref.loss)
    assert_rows_close(np32(out.lse), ref.lse, "lse")
    assert_rows_close(np32(out.chunk_loss), ref.chunk_loss, "chunk sums")
    assert_grad_close(np32(out.grad_hidden), ref.grad_hidden, "grad_hidden")
    assert_grad_close(np32(out.grad_weight), ref.grad_weight, "grad_weight")
    assert_loss_close(row_sum, ref.loss, "sum of per-row losses")


def _golden(name):
    meta_path = os.path.join(GOLDEN, f"{name}.json")
    if not os.path.exists(meta_path):
        pytest.fail(f"missing stored oracle values for {name}: run python -m oracle.make_golden {name}")
    meta = json.load(open(meta_path))
    lse = np.load(os.path.join(GOLDEN, f"lse_{name}.npy"))
    return meta, lse


def _check_large(cuda, name, chunk_sweep=None):
    w = WORKLOADS[name]
    meta, lse_ref = _golden(name)
    say(f"[gpu] workload {name}: generating inputs")
    inp = make_inputs(w)
    assert inp.digest() == meta["inputs_sha256"], "input generator drifted from the stored oracle values"
    hd, wd, bd, yd = to_device(inp, cuda)
    outs = []
    for c in (chunk_sweep or [w.chunk_rows]):
        say(f"[gpu] workload {name}: forward_backward chunk_rows={c}")
        o = lce.lce_forward_backward(hd, wd, bd, yd, chunk_rows=c, reduction=w.reduction, want_f32=True)
        torch.cuda.synchronize()
        outs.append(o)
        assert int(o.status.item()) == 0
        assert int(o.n_valid.item()) == meta["n_valid"]
        assert_loss_close(float(o.loss.item()), meta["loss_sum"])
        assert_rows_close(np32(o.lse), lse_ref, "lse (all rows)")
    out = outs[0]
    for o in outs[1:]:
        assert torch.equal(o.grad_hidden, out.grad_hidden)
        assert torch.equal(o.grad_weight, out.grad_weight)
    del outs

    # the exact call the benchmark times: bf16 outputs only (FP32 accumulator
    # in workspace, last row group's split tiles writing bf16 without keeping
    # FP32); bit-identical products, grad_bias checked on the vocabulary subset
    say(f"[gpu] workload {name}: the benchmark's call (bf16 outputs only)")
    timed = _timed_call_with_peak(cuda, w, hd, wd, bd, yd)
    assert int(timed.status.item()) == 0
    assert int(timed.n_valid.item()) == meta["n_valid"]
    assert_loss_close(float(timed.loss.item()), meta["loss_sum"])
    assert timed.grad_weight_f32 is None
    assert torch.equal(timed.grad_hidden, out.grad_hidden)
    assert torch.equal(timed.grad_weight, out.grad_weight_f32.to(torch.bfloat16))
    timed_gb = timed.grad_bias
    del timed

    # the forward-only call: every row in one pass, no stored softmax
    say(f"[gpu] workload {name}: forward only")
    f = lce.lce_forward(hd, wd, bd, yd, chunk_rows=w.chunk_rows, reduction=w.reduction, want_chunk_loss=True)
    torch.cuda.synchronize()
    assert int(f.status.item()) == 0
    assert int(f.n_valid.item()) == meta["n_valid"]
    assert_loss_close(float(f.loss.item()), meta["loss_sum"])
    assert_rows_close(np32(f.lse), lse_ref, "forward-only lse (all rows)")
    assert abs(float(f.chunk_loss.double().sum()) - meta["loss_sum"]) <= 2e-3 * abs(meta["loss_sum"])
    del f
    assert_loss_close(_check_row_losses(cuda, w, hd, wd, bd, yd, lse_ref), meta["loss_sum"], "sum of per-row losses")

    h32, w32, b32 = inp.hidden_f32(), inp.weight_f32(), inp.bias_f32()
    rows = sample_rows(w, inp.labels)
    say(f"[gpu] workload {name}: oracle on {len(rows)} rows")
    r_lse, r_loss, r_gh = O.rows_reference(h32, w32, b32, inp.labels, rows, n_valid=meta["n_valid"],
                                           reduction=w.reduction)
    np.testing.assert_allclose(r_lse, lse_ref[rows], rtol=1e-12)   # stored values agree with a fresh oracle
    assert_grad_close(np32(out.grad_hidden[torch.from_numpy(rows).to(cuda)]), r_gh, "grad_hidden rows")

    cols = sample_cols(w, inp.labels)
    say(f"[gpu] workload {name}: oracle on {len(cols)} vocabulary ids")
    c_gw, c_gb = O.cols_reference(h32, w32, b32, inp.labels, lse_ref, cols, n_valid=meta["n_valid"],
                                  reduction=w.reduction)
    ci = torch.from_numpy(cols).to(cuda)
    assert_grad_close(np32(out.grad_weight[ci]), c_gw, "grad_weight cols")
    assert_grad_close(np32(out.grad_weight_f32[ci]), c_gw, "grad_weight_f32 cols")
    cold = np.abs(c_gw).max(axis=1) < 0.01 * np.abs(c_gw).max()
    if cold.any():   # reported, not gated: relative error on rarely-labelled ids
        rel = np.abs(np32(out.grad_weight_f32[ci])[cold] - c_gw[cold]).max() / np.abs(c_gw[cold]).max()
        say(f"[gpu] workload {name}: cold-id grad_weight relative error {rel:.2e}")
    if b32 is not None:
        assert_grad_close(np32(out.grad_bias[ci]), c_gb, "grad_bias cols")
        assert_grad_close(np32(timed_gb[ci]), c_gb, "grad_bias cols (benchmark call)")
        gb = out.grad_bias_f32.double()
        assert abs(float(gb.sum())) <= 1e-3 * float(gb.abs().max()) * np.sqrt(w.vocab)
    gw_colsum = out.grad_weight_f32.double().sum(dim=0)
    assert float(gw_colsum.abs().max()) <= 1e-3 * float(out.grad_weight_f32.abs().max()) * np.sqrt(w.vocab)


@pytest.mark.timeout(900)
def test_qwen3_4b_32k(cuda):
    _check_large(cuda, "qwen3_4b_32k")


@pytest.mark.timeout(900)
def test_qwen3_4b_160k_chunk_sweep(cuda):
    _check_large(cuda, "qwen3_4b_160k", chunk_sweep=[128, 256, 512])


@pytest.mark.timeout(900)
def test_qwen3_8b_1m_shard(cuda):
    _check_large(cuda, "qwen3_8b_1m_shard")
