"""GPU parity on a seeded spread of shapes, each compared in full with the
float64 oracle: hidden sizes from 1 to 20 tiles of 256 (every count of rows
per wave that grad_weight's grad_bias sums take), ragged rows and
vocabulary, bias on and off, none / some / most rows ignored, several row
groups and chunk sizes, the three reductions (none with per-token upstream
gradients of 1, which is the sum's gradient), with and without the FP32
accumulators as outputs."""
import numpy as np
import pytest
import torch

import chunked_lm_head_lce_amd as lce
from gpu_helpers import assert_grad_close, assert_loss_close, assert_rows_close, np32, say, to_device
from lce_inputs import make_case
from oracle import lce_oracle as O

pytestmark = pytest.mark.gpu

HIDDEN = [64, 192, 320, 1024, 2560, 3840, 3904, 4096, 4160, 5120]


def _shapes(count: int = 20, seed: int = 2024):
    g = np.random.Generator(np.random.PCG64(seed))
    out = []
    for k in range(count):
        h = HIDDEN[k % len(HIDDEN)]
        v = int(g.integers(130, 4000))
        n_max = int(max(1, min(1500, 6e9 / h // v)))   # keeps the oracle near a second
        n = int(g.integers(min(n_max, 300), n_max + 1))
        out.append(dict(k=k, n=n, h=h, v=v, bias=bool(g.integers(0, 2)), ignore=float(g.choice([0.0, 0.1, 0.6])),
                        rows_in_flight=int(g.choice([0, 256])), chunk=int(g.choice([64, 256, 1000])),
                        reduction=str(g.choice(["sum", "mean", "none"])), f32=bool(g.integers(0, 2))))
    return out


@pytest.mark.parametrize("c", _shapes(), ids=lambda c: f"{c['k']}-{c['n']}x{c['h']}x{c['v']}-{c['reduction']}")
def test_random_shape_against_oracle(cuda, c):
    say(f"[gpu] random shape {c}")
    inp = make_case(c["n"], c["h"], c["v"], seed=1000 + c["k"], bias_std=(0.05 if c["bias"] else None),
                    ignore_frac=c["ignore"], weight_std=0.05)
    hd, wd, bd, yd = to_device(inp, cuda)
    none = c["reduction"] == "none"
    rs = torch.ones(c["n"], dtype=torch.float32, device=cuda) if none else None
    out = lce.lce_forward_backward(hd, wd, bd, yd, reduction=c["reduction"], chunk_rows=c["chunk"],
                                   rows_in_flight=c["rows_in_flight"] or None, want_chunk_loss=True,
                                   want_f32=c["f32"], row_scale=rs)
    torch.cuda.synchronize()
    ref = O.forward_backward(inp.hidden_f32(), inp.weight_f32(), inp.bias_f32(), inp.labels,
                             reduction="sum" if none else c["reduction"], chunk_rows=c["chunk"])
    assert int(out.n_valid.item()) == ref.n_valid
    assert int(out.status.item()) == 0
    if none:
        assert_rows_close(np32(out.loss), ref.row_loss, "row loss")
        assert float(out.loss.min()) >= 0.0
    else:
        assert_loss_close(float(out.loss.item()), float(ref.loss))
    assert out.chunk_loss.numel() == ref.chunk_loss.size
    assert_rows_close(np32(out.chunk_loss), ref.chunk_loss, "chunk sums")
    assert_rows_close(np32(out.lse), ref.lse, "lse")
    assert_grad_close(np32(out.grad_hidden), ref.grad_hidden, "grad_hidden")
    assert_grad_close(np32(out.grad_weight), ref.grad_weight, "grad_weight")
    if c["f32"]:
        assert torch.equal(out.grad_weight, out.grad_weight_f32.to(torch.bfloat16))
    if c["bias"]:
        assert_grad_close(np32(out.grad_bias), ref.grad_bias, "grad_bias")
