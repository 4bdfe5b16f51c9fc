"""Shared helpers for the GPU parity tests: move seeded inputs to the device,
call the library through its C ABI, and compare with the float64 oracle at
the tolerances the benchmark spec states (n_valid bit-exact, loss relative 2e-3,
gradients max-abs-error <= 1e-2 * max|ref| over the compared entries)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import chunked_lm_head_lce_amd as lce
from lce_inputs import Inputs

LOSS_RTOL = 2e-3
GRAD_FRAC = 1e-2
# lse_i / l_i per row: fp32 logits over H <= 4096 bf16 products, fp32 exp and
# log; the loss bound applied row by row (relative to max(1, |value|)).
ROW_RTOL = 2e-3


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def bits_to_device(bits: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def to_device(inp: Inputs, dev):
    h = bits_to_device(inp.hidden_bits, dev)
    w = bits_to_device(inp.weight_bits, dev)
    b = None if inp.bias_bits is None else bits_to_device(inp.bias_bits, dev)
    y = torch.from_numpy(inp.labels).to(dev)
    return h, w, b, y


def np32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_grad_close(got: np.ndarray, ref: np.ndarray, what: str) -> float:
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    assert err <= GRAD_FRAC * scale + 1e-30, f"{what}: max abs err {err:.3e} > 1e-2 * max|ref| ({scale:.3e})"
    return err / scale if scale else 0.0


def assert_loss_close(got: float, ref: float, what: str = "loss") -> None:
    assert abs(got - ref) <= LOSS_RTOL * max(abs(ref), 1e-30), f"{what}: got {got!r}, oracle {ref!r}"


def assert_rows_close(got: np.ndarray, ref: np.ndarray, what: str) -> None:
    bound = ROW_RTOL * np.maximum(1.0, np.abs(ref))
    bad = np.abs(got - ref) > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} rows off, worst {np.max(np.abs(got - ref)):.3e}"
