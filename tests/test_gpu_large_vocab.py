"""A vocabulary above 2^18 ids (262144 + 77: a ragged last tile, past the
largest vocabularies in use) with a full 16384-row group, so that the
group's stored probabilities, K-slabs [V/64][16384][64] of bf16, span more
than 2^32 elements (8.6 GB) and every offset into them must be 64-bit.

Compared with the float64 oracle: every row's lse and the total loss,
grad_hidden on a row subset, grad_weight and grad_bias on a vocabulary
subset (with the full lse), at H = 64 so that the oracle's lse pass over
all 17161 x 262221 logits stays a few seconds."""
import numpy as np
import pytest
import torch

import chunked_lm_head_lce_amd as lce
from gpu_helpers import assert_grad_close, assert_loss_close, assert_rows_close, np32, say, to_device
from lce_inputs import make_case
from oracle import lce_oracle as O

pytestmark = pytest.mark.gpu

N, H, V, GROUP = 16384 + 777, 64, 262144 + 77, 16384


@pytest.mark.timeout(600)
def test_vocab_above_2_18_with_a_full_row_group(cuda):
    say(f"[gpu] large vocabulary: generating {N} x {H} x {V}")
    inp = make_case(N, H, V, seed=2018, bias_std=0.05, ignore_frac=0.05, weight_std=0.05)
    hd, wd, bd, yd = to_device(inp, cuda)
    say("[gpu] large vocabulary: forward_backward, two row groups")
    out = lce.lce_forward_backward(hd, wd, bd, yd, rows_in_flight=GROUP, want_f32=True)
    torch.cuda.synchronize()
    assert int(out.status.item()) == 0
    h32, w32, b32 = inp.hidden_f32(), inp.weight_f32(), inp.bias_f32()
    say("[gpu] large vocabulary: oracle lse over all rows")
    w64 = np.asarray(w32, dtype=np.float64)
    lse = O.lse_rows_blocked(h32, w32, b32, weight64=w64, block_rows=512)
    loss, n_valid = O.loss_sum_from_lse(h32, w32, b32, inp.labels, lse)
    assert int(out.n_valid.item()) == n_valid
    assert_loss_close(float(out.loss.item()), loss)
    assert_rows_close(np32(out.lse), lse, "lse (all rows)")

    g = np.random.Generator(np.random.PCG64(5))
    edges = [0, GROUP - 1, GROUP, N - 1]   # both sides of the group boundary
    ign = np.flatnonzero(inp.labels == -100)[:8]
    rows = np.unique(np.concatenate([g.choice(N, 160, replace=False), edges, ign]))
    say(f"[gpu] large vocabulary: oracle on {len(rows)} rows")
    r_lse, _, r_gh = O.rows_reference(h32, w32, b32, inp.labels, rows, n_valid=n_valid, weight64=w64)
    np.testing.assert_allclose(r_lse, lse[rows], rtol=1e-12)
    assert_grad_close(np32(out.grad_hidden[torch.from_numpy(rows).to(cuda)]), r_gh, "grad_hidden rows")

    valid = inp.labels[inp.labels != -100]
    hot = np.argsort(-np.bincount(valid, minlength=V), kind="stable")[:8]
    cols = np.unique(np.concatenate([g.choice(V, 160, replace=False), hot, np.arange(V - 96, V),
                                     np.arange(2 ** 17 - 4, 2 ** 17 + 4)]))
    say(f"[gpu] large vocabulary: oracle on {len(cols)} vocabulary ids")
    c_gw, c_gb = O.cols_reference(h32, w32, b32, inp.labels, lse, cols, n_valid=n_valid)
    ci = torch.from_numpy(cols).to(cuda)
    assert_grad_close(np32(out.grad_weight[ci]), c_gw, "grad_weight cols")
    assert_grad_close(np32(out.grad_weight_f32[ci]), c_gw, "grad_weight_f32 cols")
    assert_grad_close(np32(out.grad_bias[ci]), c_gb, "grad_bias cols")
    assert torch.equal(out.grad_weight, out.grad_weight_f32.to(torch.bfloat16))
    # a sum loss's gradient has zero column sums over the vocabulary
    gb = out.grad_bias_f32.double()
    assert abs(float(gb.sum())) <= 1e-3 * float(gb.abs().max()) * np.sqrt(V)
