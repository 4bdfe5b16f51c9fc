"""Chunked linear-cross-entropy on MI355X (gfx950): thin Python binding.

The functions here only marshal arguments to the C ABI of ``liblce.so``
(include/lce.h): they check dtypes and shapes, take device memory and the
current stream from PyTorch, and call the library. Every step of the loss
runs in the library's HIP kernels; there is no fallback implementation.

    lce_forward(hidden, weight, bias, labels, ...)          -> LceOutput
    lce_forward_backward(hidden, weight, bias, labels, ...) -> LceOutput with grads
    lce_scale(tensor, scale)                                -> tensor *= scale (in a library kernel)
    linear_cross_entropy(hidden, weight, labels, bias=...)  -> loss with autograd (torch.autograd.Function)

``chunk_rows`` follows the pages' ``chunk_loss_size`` (LlamaFactory section 2):
positive, ``None`` meaning one chunk of all rows, anything else a ValueError.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import LceProblem

IGNORE_INDEX = -100
DEFAULT_CHUNK_ROWS = 256

__all__ = ["lce_forward", "lce_forward_backward", "lce_forward_noalloc", "noalloc_outputs", "lce_workspace_bytes",
           "lce_scale", "linear_cross_entropy",
           "LinearCrossEntropyFunction", "LceOutput", "LceError", "IGNORE_INDEX", "DEFAULT_CHUNK_ROWS"]


class LceError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {_lib.status_string(code)} (status {code})")
        self.code = code


@dataclass
class LceOutput:
    loss: torch.Tensor                  # [] for sum/mean, [N] for none (float32)
    lse: torch.Tensor | None            # [N] float32
    chunk_loss: torch.Tensor | None     # [T] float32
    n_valid: torch.Tensor               # [] int64
    status: torch.Tensor                # [] int32 (device-side status word)
    grad_hidden: torch.Tensor | None = None
    grad_weight: torch.Tensor | None = None
    grad_bias: torch.Tensor | None = None
    grad_weight_f32: torch.Tensor | None = None
    grad_bias_f32: torch.Tensor | None = None
    workspace_bytes: int = 0

    def check(self) -> "LceOutput":
        """Synchronise and raise if the device reported a label outside [0, V)."""
        code = int(self.status.item())
        if code != _lib.LCE_OK:
            raise LceError(code, "device status")
        return self


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _problem(hidden, weight, labels, ignore_index, chunk_rows, reduction, rows_in_flight,
             bias=None) -> LceProblem:
    if reduction not in _lib.LCE_REDUCTION:
        raise ValueError(f"reduction must be one of {sorted(_lib.LCE_REDUCTION)}, got {reduction!r}")
    if hidden.dim() != 2 or weight.dim() != 2 or labels.dim() != 1:
        raise ValueError("expected hidden [N,H], weight [V,H], labels [N]")
    n, h = hidden.shape
    v, hw = weight.shape
    if hw != h or labels.shape[0] != n:
        raise ValueError(f"shape mismatch: hidden {tuple(hidden.shape)}, weight {tuple(weight.shape)}, "
                         f"labels {tuple(labels.shape)}")
    if hidden.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
        raise ValueError("hidden and weight must be bfloat16")
    if labels.dtype != torch.int64:
        raise ValueError("labels must be int64")
    if not labels.is_contiguous():
        raise ValueError("labels must be contiguous")
    for name, t in (("hidden", hidden), ("weight", weight)):
        if t.numel() > 0 and t.stride(1) != 1:
            raise ValueError(f"{name} rows must be contiguous")
    if bias is not None:
        if bias.dtype != torch.bfloat16 or bias.dim() != 1 or bias.shape[0] != v or not bias.is_contiguous():
            raise ValueError(f"bias must be a contiguous bfloat16 [V={v}] tensor, got {bias.dtype} "
                             f"{tuple(bias.shape)}")
    for name, t in (("weight", weight), ("labels", labels), ("bias", bias)):
        if t is not None and t.device != hidden.device:
            raise ValueError(f"{name} is on {t.device}, hidden on {hidden.device}")
    if chunk_rows is None:
        chunk_rows = max(n, 1)
    if chunk_rows <= 0:
        raise ValueError("`chunk_rows` must be positive.")
    p = LceProblem()
    p.n_rows, p.hidden, p.vocab = n, h, v
    p.ld_hidden = hidden.stride(0) if n > 1 else h
    p.ld_weight = weight.stride(0) if v > 1 else h
    p.ignore_index = ignore_index
    p.chunk_rows = chunk_rows
    p.rows_in_flight = rows_in_flight or 0
    p.reduction = _lib.LCE_REDUCTION[reduction]
    p.dtype = _lib.LCE_DTYPE_BF16
    return p


def _raise(code: int, where: str):
    if code == _lib.LCE_ERR_INVALID_ARG:
        raise ValueError(f"{where}: {_lib.status_string(code)}")
    raise LceError(code, where)


def _check_out(out: "LceOutput", n: int, h: int, v: int, reduction: str, chunk_rows: int, dev) -> None:
    """Caller-given output buffers: shape, dtype, device and contiguity as the
    library writes them (it takes raw pointers and trusts these)."""
    t_chunks = -(-n // chunk_rows) if n else 0
    want = {
        "loss": ((n,) if reduction == "none" else (), torch.float32),
        "lse": ((n,), torch.float32),
        "chunk_loss": ((t_chunks,), torch.float32),
        "n_valid": ((), torch.int64),
        "status": ((), torch.int32),
        "grad_hidden": ((n, h), torch.bfloat16),
        "grad_weight": ((v, h), torch.bfloat16),
        "grad_bias": ((v,), torch.bfloat16),
        "grad_weight_f32": ((v, h), torch.float32),
        "grad_bias_f32": ((v,), torch.float32),
    }
    for name, (shape, dtype) in want.items():
        t = getattr(out, name)
        if t is None:
            if name in ("loss", "n_valid", "status"):
                raise ValueError(f"out.{name} is required")
            continue
        if tuple(t.shape) != shape or t.dtype != dtype or not t.is_contiguous() or t.device != dev:
            raise ValueError(f"out.{name} must be a contiguous {dtype} tensor of shape {shape} on {dev}, got "
                             f"{t.dtype} {tuple(t.shape)} on {t.device}")


def _check_workspace(ws, dev) -> None:
    if ws is not None and (ws.dtype != torch.uint8 or not ws.is_contiguous() or ws.device != dev):
        raise ValueError(f"workspace must be a contiguous uint8 tensor on {dev}")


def lce_workspace_bytes(hidden, weight, labels, *, backward: bool, external_f32: bool = False,
                        ignore_index: int = IGNORE_INDEX, chunk_rows: int | None = DEFAULT_CHUNK_ROWS,
                        reduction: str = "sum", rows_in_flight: int | None = None) -> int:
    lib = _lib.load()
    p = _problem(hidden, weight, labels, ignore_index, chunk_rows, reduction, rows_in_flight)
    kind = (_lib.LCE_WS_BACKWARD_EXTERNAL_F32 if external_f32 else _lib.LCE_WS_BACKWARD) if backward \
        else _lib.LCE_WS_FORWARD
    return int(lib.lce_workspace_bytes(ctypes.byref(p), kind))


def _device_checks(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")


def _common_outputs(n, reduction, chunk_rows, want_lse, want_chunks, dev):
    loss = torch.empty((n,) if reduction == "none" else (), dtype=torch.float32, device=dev)
    lse = torch.empty(n, dtype=torch.float32, device=dev) if want_lse else None
    t = -(-n // chunk_rows) if n else 0
    chunk = torch.empty(t, dtype=torch.float32, device=dev) if want_chunks else None
    n_valid = torch.empty((), dtype=torch.int64, device=dev)
    status = torch.empty((), dtype=torch.int32, device=dev)
    return loss, lse, chunk, n_valid, status


def lce_forward(hidden: torch.Tensor, weight: torch.Tensor, bias: torch.Tensor | None, labels: torch.Tensor,
                *, ignore_index: int = IGNORE_INDEX, chunk_rows: int | None = DEFAULT_CHUNK_ROWS,
                reduction: str = "sum", want_lse: bool = True, want_chunk_loss: bool = False,
                workspace: torch.Tensor | None = None, out: LceOutput | None = None,
                trace: "_lib.LceTrace | None" = None) -> LceOutput:
    """Loss (+ per-row lse, per-chunk sums, valid count) without the [N,V] logits."""
    lib = _lib.load()
    _device_checks(hidden, weight, bias, labels)
    p = _problem(hidden, weight, labels, ignore_index, chunk_rows, reduction, None, bias)
    dev = hidden.device
    if out is None:
        out = LceOutput(*_common_outputs(hidden.shape[0], reduction, p.chunk_rows, want_lse, want_chunk_loss, dev))
    else:
        _check_out(out, hidden.shape[0], hidden.shape[1], weight.shape[0], reduction, p.chunk_rows, dev)
    nbytes = int(lib.lce_workspace_bytes(ctypes.byref(p), _lib.LCE_WS_FORWARD))
    _check_workspace(workspace, dev)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    out.workspace_bytes = nbytes
    stream = torch.cuda.current_stream(dev).cuda_stream
    code = lib.lce_forward_traced(ctypes.byref(p), _ptr(hidden), _ptr(weight), _ptr(bias), _ptr(labels),
                                  _ptr(out.loss), _ptr(out.lse), _ptr(out.chunk_loss), _ptr(out.n_valid),
                                  _ptr(out.status), _ptr(workspace), workspace.numel(), stream,
                                  None if trace is None else ctypes.byref(trace))
    if code != _lib.LCE_OK:
        _raise(code, "lce_forward")
    return out


def lce_forward_noalloc(hidden: torch.Tensor, weight: torch.Tensor, bias: torch.Tensor | None,
                        labels: torch.Tensor, *, out: LceOutput, ignore_index: int = IGNORE_INDEX,
                        chunk_rows: int | None = DEFAULT_CHUNK_ROWS, reduction: str = "sum") -> LceOutput:
    """lce_forward for callers that cannot allocate: the library's fixed
    per-GPU scratch is the workspace, and ``out`` (caller-allocated, e.g. by
    :func:`noalloc_outputs`) receives the results. Calls on one GPU must not
    overlap. Raises LceError with LCE_ERR_TOO_LARGE when the problem does not
    fit the scratch."""
    lib = _lib.load()
    _device_checks(hidden, weight, bias, labels)
    p = _problem(hidden, weight, labels, ignore_index, chunk_rows, reduction, None, bias)
    _check_out(out, hidden.shape[0], hidden.shape[1], weight.shape[0], reduction, p.chunk_rows, hidden.device)
    stream = torch.cuda.current_stream(hidden.device).cuda_stream
    code = lib.lce_forward_noalloc(ctypes.byref(p), _ptr(hidden), _ptr(weight), _ptr(bias), _ptr(labels),
                                   _ptr(out.loss), _ptr(out.lse), _ptr(out.chunk_loss), _ptr(out.n_valid),
                                   _ptr(out.status), stream)
    if code != _lib.LCE_OK:
        _raise(code, "lce_forward_noalloc")
    return out


def noalloc_outputs(n: int, device, *, reduction: str = "sum", chunk_rows: int | None = DEFAULT_CHUNK_ROWS,
                    want_lse: bool = True, want_chunk_loss: bool = False) -> LceOutput:
    """Output buffers for :func:`lce_forward_noalloc`, allocated ahead of time."""
    c = chunk_rows if chunk_rows is not None else max(n, 1)
    return LceOutput(*_common_outputs(n, reduction, c, want_lse, want_chunk_loss, torch.device(device)))


def lce_forward_backward(hidden: torch.Tensor, weight: torch.Tensor, bias: torch.Tensor | None,
                         labels: torch.Tensor, *, grad_scale: float = 1.0, ignore_index: int = IGNORE_INDEX,
                         chunk_rows: int | None = DEFAULT_CHUNK_ROWS, reduction: str = "sum",
                         want_grad_hidden: bool = True, want_grad_weight: bool = True,
                         want_grad_bias: bool | None = None, want_f32: bool = False, want_lse: bool = True,
                         want_chunk_loss: bool = False, rows_in_flight: int | None = None,
                         row_scale: torch.Tensor | None = None, accumulate: bool = False,
                         workspace: torch.Tensor | None = None, out: LceOutput | None = None,
                         trace: "_lib.LceTrace | None" = None) -> LceOutput:
    """Loss and gradients in one call. grad_weight / grad_bias are accumulated
    in FP32 and cast to bf16 at the end; ``want_f32`` also returns the FP32
    accumulators (and makes the call use them instead of workspace).

    ``row_scale`` ([N] float32 on the GPU) multiplies row i's dlogits, e.g. the
    per-token upstream gradient; ``reduction="none"`` requires it.
    ``accumulate=True`` adds into ``out.grad_weight_f32`` / ``out.grad_bias_f32``
    instead of overwriting them (fresh zeroed FP32 buffers when ``out`` is None)."""
    lib = _lib.load()
    _device_checks(hidden, weight, bias, labels)
    if want_grad_bias is None:
        want_grad_bias = bias is not None
    if want_grad_bias and bias is None:
        raise ValueError("grad_bias requested without a bias")
    p = _problem(hidden, weight, labels, ignore_index, chunk_rows, reduction, rows_in_flight, bias)
    dev = hidden.device
    n, h = hidden.shape
    v = weight.shape[0]
    if out is not None:
        _check_out(out, n, h, v, reduction, p.chunk_rows, dev)
        if out.grad_bias is not None or out.grad_bias_f32 is not None:
            if bias is None:
                raise ValueError("out holds grad_bias buffers but there is no bias")
        if accumulate and ((out.grad_weight is not None and out.grad_weight_f32 is None) or
                           (out.grad_bias is not None and out.grad_bias_f32 is None)):
            raise ValueError("accumulate=True needs out.grad_weight_f32 / out.grad_bias_f32")
    if out is None:
        out = LceOutput(*_common_outputs(n, reduction, p.chunk_rows, want_lse, want_chunk_loss, dev))
        if want_grad_hidden:
            out.grad_hidden = torch.empty((n, h), dtype=torch.bfloat16, device=dev)
        if want_grad_weight:
            out.grad_weight = torch.empty((v, h), dtype=torch.bfloat16, device=dev)
            if want_f32 or accumulate:
                out.grad_weight_f32 = (torch.zeros if accumulate else torch.empty)((v, h), dtype=torch.float32,
                                                                                  device=dev)
        if want_grad_bias:
            out.grad_bias = torch.empty(v, dtype=torch.bfloat16, device=dev)
            if want_f32 or accumulate:
                out.grad_bias_f32 = (torch.zeros if accumulate else torch.empty)(v, dtype=torch.float32, device=dev)
    external = out.grad_weight_f32 is not None or out.grad_weight is None
    kind = _lib.LCE_WS_BACKWARD_EXTERNAL_F32 if external else _lib.LCE_WS_BACKWARD
    nbytes = int(lib.lce_workspace_bytes(ctypes.byref(p), kind))
    _check_workspace(workspace, dev)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    out.workspace_bytes = nbytes
    opts = None
    if row_scale is not None or accumulate:
        if row_scale is not None:
            _device_checks(row_scale)
            if row_scale.dtype != torch.float32 or row_scale.shape != (n,) or not row_scale.is_contiguous():
                raise ValueError("row_scale must be a contiguous float32 [N] tensor")
        opts = _lib.LceBackwardOptions()
        opts.row_scale = _ptr(row_scale)
        opts.accumulate = 1 if accumulate else 0
        opts.reserved = 0
    stream = torch.cuda.current_stream(dev).cuda_stream
    code = lib.lce_forward_backward_ex(
        ctypes.byref(p), _ptr(hidden), _ptr(weight), _ptr(bias), _ptr(labels), float(grad_scale), _ptr(out.loss),
        _ptr(out.lse), _ptr(out.chunk_loss), _ptr(out.n_valid), _ptr(out.grad_hidden), _ptr(out.grad_weight),
        _ptr(out.grad_bias), _ptr(out.grad_weight_f32), _ptr(out.grad_bias_f32), _ptr(out.status),
        _ptr(workspace), workspace.numel(), stream, None if opts is None else ctypes.byref(opts),
        None if trace is None else ctypes.byref(trace))
    if code != _lib.LCE_OK:
        _raise(code, "lce_forward_backward")
    return out


def lce_scale(t: torch.Tensor, scale: torch.Tensor) -> torch.Tensor:
    """t *= scale in place, by a library kernel; ``scale`` is a one-element
    float32 tensor on the GPU (read by the kernel, no host synchronisation)."""
    lib = _lib.load()
    _device_checks(t, scale)
    if scale.dtype != torch.float32 or scale.numel() != 1:
        raise ValueError("scale must be a one-element float32 tensor")
    if not t.is_contiguous():
        raise ValueError("t must be contiguous")
    dtype = {torch.bfloat16: _lib.LCE_DTYPE_BF16, torch.float32: _lib.LCE_DTYPE_F32}.get(t.dtype)
    if dtype is None:
        raise ValueError("t must be bfloat16 or float32")
    stream = torch.cuda.current_stream(t.device).cuda_stream
    code = lib.lce_scale(_ptr(t), dtype, t.numel(), _ptr(scale), stream)
    if code != _lib.LCE_OK:
        _raise(code, "lce_scale")
    return t


class LinearCrossEntropyFunction(torch.autograd.Function):
    """Drop-in output head + cross-entropy with the pages' autograd contract
    (LlamaFactory PR #10762 analysis, section 4): for sum / mean the forward
    computes the loss and, for the inputs that need them, the gradients in one
    library call (``needs_input_grad`` plays the pages' needs_weight_grad);
    backward multiplies them by ``grad_output`` in a library kernel. For
    ``reduction="none"`` the per-token gradient is only known in backward, so
    backward runs the fused call with it as the per-row scale."""

    @staticmethod
    def forward(ctx, hidden, weight, bias, labels, ignore_index, chunk_rows, reduction, rows_in_flight):
        need_h, need_w, need_b = ctx.needs_input_grad[:3]
        need_b = need_b and bias is not None
        ctx.reduction = reduction
        ctx.args = (ignore_index, chunk_rows, rows_in_flight)
        ctx.need = (need_h, need_w, need_b)
        if reduction == "none" or not (need_h or need_w or need_b):
            out = lce_forward(hidden, weight, bias, labels, ignore_index=ignore_index, chunk_rows=chunk_rows,
                              reduction=reduction, want_lse=False)
            if reduction == "none":
                ctx.save_for_backward(hidden, weight, bias, labels)
            ctx.grads = None
            return out.loss
        out = lce_forward_backward(hidden, weight, bias, labels, ignore_index=ignore_index, chunk_rows=chunk_rows,
                                   reduction=reduction, want_grad_hidden=need_h, want_grad_weight=need_w,
                                   want_grad_bias=need_b, want_lse=False, rows_in_flight=rows_in_flight)
        ctx.grads = (out.grad_hidden, out.grad_weight, out.grad_bias)
        return out.loss

    @staticmethod
    def backward(ctx, grad_output):
        need_h, need_w, need_b = ctx.need
        if ctx.reduction == "none":
            hidden, weight, bias, labels = ctx.saved_tensors
            ignore_index, chunk_rows, rows_in_flight = ctx.args
            out = lce_forward_backward(hidden, weight, bias, labels, ignore_index=ignore_index,
                                       chunk_rows=chunk_rows, reduction="none", want_grad_hidden=need_h,
                                       want_grad_weight=need_w, want_grad_bias=need_b, want_lse=False,
                                       rows_in_flight=rows_in_flight,
                                       row_scale=grad_output.detach().float().contiguous())
            gh, gw, gb = out.grad_hidden, out.grad_weight, out.grad_bias
        else:
            gh, gw, gb = ctx.grads
            ctx.grads = None
            g = grad_output.detach().float().reshape(1).contiguous()
            for t in (gh, gw, gb):
                if t is not None:
                    lce_scale(t, g)
        return (gh if need_h else None, gw if need_w else None, gb if need_b else None,
                None, None, None, None, None)


def linear_cross_entropy(hidden: torch.Tensor, weight: torch.Tensor, labels: torch.Tensor,
                         bias: torch.Tensor | None = None, *, ignore_index: int = IGNORE_INDEX,
                         chunk_rows: int | None = DEFAULT_CHUNK_ROWS, reduction: str = "mean",
                         rows_in_flight: int | None = None) -> torch.Tensor:
    """Cross-entropy of ``hidden @ weight.T (+ bias)`` against ``labels`` without
    the [N, V] logits, differentiable in hidden, weight and bias. Shapes as
    :func:`lce_forward`; bf16 inputs, float32 loss, bf16 gradients."""
    return LinearCrossEntropyFunction.apply(hidden, weight, bias, labels, ignore_index, chunk_rows, reduction,
                                            rows_in_flight)
