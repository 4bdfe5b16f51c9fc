"""The allocation-free forward (lce_forward_noalloc, for callers that cannot
allocate device memory) against lce_forward, through the C ABI, on two calls
in a row: the first large enough that its partials go through the fixed
scratch in row groups, the second smaller and in one pass over stale
scratch contents left by the first."""
import math

import pytest
import torch

import chunked_lm_head_lce_amd as lce
from chunked_lm_head_lce_amd import _lib
from gpu_helpers import say, to_device
from lce_inputs import make_case

pytestmark = pytest.mark.gpu

# (N, H, V, bias, reduction). The first needs 384 MB of partials for all rows
# at once, so it runs in row groups that fit 64 MiB; the second fits whole.
CASES = [(20000, 1024, 151936, True, "sum"), (3000, 512, 50000, False, "mean")]


def test_noalloc_forward_matches_forward(cuda):
    for i, (n, h, v, bias, reduction) in enumerate(CASES):
        say(f"[gpu] noalloc forward call {i}: N={n} H={h} V={v} bias={bias} {reduction}")
        inp = make_case(n, h, v, seed=60 + i, bias_std=(0.02 if bias else None), labels="zipf", ignore_frac=0.05)
        hd, wd, bd, yd = to_device(inp, cuda)
        ref = lce.lce_forward(hd, wd, bd, yd, reduction=reduction, want_chunk_loss=True)
        out = lce.noalloc_outputs(n, cuda, reduction=reduction, want_chunk_loss=True)
        got = lce.lce_forward_noalloc(hd, wd, bd, yd, out=out, reduction=reduction)
        torch.cuda.synchronize()
        assert got is out
        assert int(out.status.item()) == _lib.LCE_OK
        assert int(out.n_valid.item()) == int(ref.n_valid.item()) == n - math.floor(0.05 * n)
        # same tiles, same accumulation and merge order: every row's lse is identical
        assert torch.equal(out.lse, ref.lse)
        # the loss sums rows through float64 atomics, whose order may differ
        a, b = float(out.loss.item()), float(ref.loss.item())
        assert abs(a - b) <= 1e-6 * abs(b), (a, b)
        torch.testing.assert_close(out.chunk_loss, ref.chunk_loss, rtol=1e-5, atol=1e-4)
        del hd, wd, bd, yd, ref, out


def test_noalloc_forward_too_large_is_an_error(cuda):
    """A problem that cannot fit the scratch even 256 rows at a time raises
    before anything is enqueued (partials of 256 rows at V = 2^22 alone take
    128 MiB)."""
    h = torch.zeros(300, 64, dtype=torch.bfloat16, device=cuda)
    w = torch.zeros(1 << 22, 64, dtype=torch.bfloat16, device=cuda)
    y = torch.zeros(300, dtype=torch.int64, device=cuda)
    out = lce.noalloc_outputs(300, cuda)
    with pytest.raises(lce.LceError) as e:
        lce.lce_forward_noalloc(h, w, None, y, out=out)
    assert e.value.code == _lib.LCE_ERR_TOO_LARGE
