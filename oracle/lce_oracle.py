"""CPU float64 oracle for chunked linear-cross-entropy (test infrastructure).

This module is test infrastructure, not the product. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call it; the GPU library never does, and it shares no code with the
GPU library.

What it computes, and where the pages say so:

* LlamaFactory PR #10762 analysis, section 4 ("Chunk Loss implementation",
  ``_ChunkedLinearCrossEntropy``): rows of the final hidden states go through
  the output head (a plain ``nn.Linear``: logits = h W^T + b) and then through
  per-token cross-entropy with ``reduction="none"`` and ``ignore_index`` (the
  constant -100); chunk losses are summed; gradients for the head weight and
  bias are accumulated across chunks in FP32 and cast once at the end.
* TRL "training on 1M+ tokens", section "chunking": rows split cleanly because
  the loss is a sum over rows and each softmax runs along one row's
  vocabulary, so chunking changes only when rows are computed, not the result.
* LlamaFactory section 2 (``TrainingArguments.chunk_loss_size``): a chunk size
  that is not positive is rejected with ``ValueError``.

Because chunking reaches exactly (up to rounding order) the plain unchunked
cross-entropy of a linear head, the oracle is that definition written out in
float64 on the exact (bfloat16-representable) inputs:

    z      = h W^T + b                                  [N, V]
    lse_i  = m_i + ln sum_j exp(z_ij - m_i),  m_i = max_j z_ij
    l_i    = valid_i * (lse_i - z_{i, y_i})
    loss   = sum_i l_i   (sum)  |  sum_i l_i / max(n_valid, 1)  (mean)  |  l  (none)
    G_ij   = s_i * valid_i * (exp(z_ij - lse_i) - [j == y_i])
    grad_hidden = G W,  grad_weight = G^T h,  grad_bias = sum_i G_i

with ``s_i = grad_scale`` (sum), ``grad_scale / max(n_valid, 1)`` (mean) or
the per-row upstream gradient (none). Every function below is pinned by the
``-m "not gpu"`` tests against an independent library routine (torch's float64
cross-entropy and autograd), central finite differences, closed forms and
invariants; none is "parity unpinned".
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

IGNORE_INDEX = -100
REDUCTIONS = ("none", "sum", "mean")


def check_problem(n_rows: int, hidden: int, vocab: int, chunk_rows: int | None) -> None:
    """Argument rules (LlamaFactory section 2: non-positive chunk size is a
    ValueError; None means one chunk of all rows)."""
    if n_rows < 0 or hidden <= 0 or vocab <= 0:
        raise ValueError(f"bad shape N={n_rows} H={hidden} V={vocab}")
    if chunk_rows is not None and chunk_rows <= 0:
        raise ValueError("`chunk_rows` must be positive.")


def valid_rows(labels: np.ndarray, vocab: int, ignore_index: int = IGNORE_INDEX) -> np.ndarray:
    """valid_i = (y_i != ignore_index); a label outside [0, V) that is not the
    ignore label is an error (torch's cross-entropy refuses it too)."""
    labels = np.asarray(labels, dtype=np.int64)
    valid = labels != ignore_index
    bad = valid & ((labels < 0) | (labels >= vocab))
    if bad.any():
        raise ValueError(f"label out of range at rows {np.flatnonzero(bad)[:8].tolist()}")
    return valid


def logits(hidden: np.ndarray, weight: np.ndarray, bias: np.ndarray | None) -> np.ndarray:
    """z = h W^T (+ b), float64 (the head is an nn.Linear)."""
    z = np.asarray(hidden, dtype=np.float64) @ np.asarray(weight, dtype=np.float64).T
    if bias is not None:
        z += np.asarray(bias, dtype=np.float64)[None, :]
    return z


def row_logsumexp(z: np.ndarray) -> np.ndarray:
    """lse_i = m_i + ln sum_j exp(z_ij - m_i) with m_i the row maximum."""
    m = z.max(axis=1)
    return m + np.log(np.exp(z - m[:, None]).sum(axis=1))


def _label_logits(z: np.ndarray, labels: np.ndarray, valid: np.ndarray) -> np.ndarray:
    safe = np.where(valid, labels, 0)
    return np.where(valid, z[np.arange(z.shape[0]), safe], 0.0)


def row_scale(reduction: str, n_valid: int, grad_scale, n_rows: int) -> np.ndarray:
    """s_i: dLoss/d l_i times the caller's upstream gradient."""
    if reduction not in REDUCTIONS:
        raise ValueError(f"unknown reduction {reduction!r}")
    if reduction == "none":
        g = np.broadcast_to(np.asarray(grad_scale, dtype=np.float64), (n_rows,))
        return np.array(g, dtype=np.float64)
    s = float(grad_scale)
    if reduction == "mean":
        s /= max(n_valid, 1)
    return np.full(n_rows, s, dtype=np.float64)


def reduce_loss(row_loss: np.ndarray, n_valid: int, reduction: str):
    if reduction == "none":
        return row_loss
    total = float(np.sum(row_loss))
    return total / max(n_valid, 1) if reduction == "mean" else total


def chunk_sums(row_loss: np.ndarray, chunk_rows: int) -> np.ndarray:
    """Per-chunk sums of l_i for chunks [k*c, min((k+1)c, N))."""
    n = row_loss.shape[0]
    return np.array([row_loss[s:s + chunk_rows].sum() for s in range(0, n, chunk_rows)],
                    dtype=np.float64)


@dataclass
class Result:
    loss: object                 # float, or [N] for reduction="none"
    lse: np.ndarray              # [N]
    row_loss: np.ndarray         # [N]
    n_valid: int
    chunk_loss: np.ndarray       # [T] sums of row_loss per chunk
    grad_hidden: np.ndarray | None = None   # [N, H]
    grad_weight: np.ndarray | None = None   # [V, H]
    grad_bias: np.ndarray | None = None     # [V]


def forward(hidden, weight, bias, labels, *, ignore_index: int = IGNORE_INDEX,
            reduction: str = "sum", chunk_rows: int | None = None) -> Result:
    """Loss, per-row lse and n_valid from materialised float64 logits."""
    n, h = np.shape(hidden)
    v = np.shape(weight)[0]
    check_problem(n, h, v, chunk_rows)
    if reduction not in REDUCTIONS:
        raise ValueError(f"unknown reduction {reduction!r}")
    labels = np.asarray(labels, dtype=np.int64)
    valid = valid_rows(labels, v, ignore_index)
    n_valid = int(valid.sum())
    z = logits(hidden, weight, bias)
    lse = row_logsumexp(z) if n else np.zeros(0)
    row_loss = np.where(valid, lse - _label_logits(z, labels, valid), 0.0)
    c = chunk_rows if chunk_rows is not None else max(n, 1)
    return Result(reduce_loss(row_loss, n_valid, reduction), lse, row_loss, n_valid,
                  chunk_sums(row_loss, c))


def dlogits(z: np.ndarray, lse: np.ndarray, labels: np.ndarray, valid: np.ndarray,
            scale: np.ndarray) -> np.ndarray:
    """G_ij = s_i * valid_i * (softmax_ij - [j == y_i])."""
    g = np.exp(z - lse[:, None])
    rows = np.flatnonzero(valid)
    g[rows, labels[rows]] -= 1.0
    g *= (scale * valid)[:, None]
    return g


def forward_backward(hidden, weight, bias, labels, *, ignore_index: int = IGNORE_INDEX,
                     reduction: str = "sum", grad_scale=1.0,
                     chunk_rows: int | None = None) -> Result:
    """Forward plus grad_hidden = G W, grad_weight = G^T h, grad_bias = sum_i G_i."""
    res = forward(hidden, weight, bias, labels, ignore_index=ignore_index,
                  reduction=reduction, chunk_rows=chunk_rows)
    h64 = np.asarray(hidden, dtype=np.float64)
    w64 = np.asarray(weight, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    valid = labels != ignore_index
    z = logits(h64, w64, bias)
    g = dlogits(z, res.lse, labels, valid, row_scale(reduction, res.n_valid, grad_scale, len(labels)))
    res.grad_hidden = g @ w64
    res.grad_weight = g.T @ h64
    res.grad_bias = g.sum(axis=0) if bias is not None else None
    return res


def chunked_forward_backward(hidden, weight, bias, labels, chunk_rows: int, *,
                             ignore_index: int = IGNORE_INDEX, reduction: str = "sum",
                             grad_scale=1.0) -> Result:
    """The pages' procedure (LlamaFactory section 4): walk the flattened rows
    in chunks of at most ``chunk_rows``; each chunk makes its own logits, its
    per-token losses and its gradients; chunk losses are summed, grad_hidden
    rows are written per chunk and grad_weight / grad_bias are accumulated
    over chunks. Used to pin chunk-size invariance."""
    n, h = np.shape(hidden)
    v = np.shape(weight)[0]
    check_problem(n, h, v, chunk_rows)
    labels = np.asarray(labels, dtype=np.int64)
    valid = valid_rows(labels, v, ignore_index)
    n_valid = int(valid.sum())
    scale = row_scale(reduction, n_valid, grad_scale, n)
    h64 = np.asarray(hidden, dtype=np.float64)
    w64 = np.asarray(weight, dtype=np.float64)
    lse = np.zeros(n)
    row_loss = np.zeros(n)
    gh = np.zeros((n, h))
    gw = np.zeros((v, h))
    gb = np.zeros(v) if bias is not None else None
    chunk_loss = []
    for s in range(0, n, chunk_rows):
        e = min(n, s + chunk_rows)
        z = logits(h64[s:e], w64, bias)
        lse[s:e] = row_logsumexp(z)
        vk = valid[s:e]
        row_loss[s:e] = np.where(vk, lse[s:e] - _label_logits(z, labels[s:e], vk), 0.0)
        chunk_loss.append(row_loss[s:e].sum())
        g = dlogits(z, lse[s:e], labels[s:e], vk, scale[s:e])
        gh[s:e] = g @ w64
        gw += g.T @ h64[s:e]
        if gb is not None:
            gb += g.sum(axis=0)
    return Result(reduce_loss(row_loss, n_valid, reduction), lse, row_loss, n_valid,
                  np.asarray(chunk_loss), gh, gw, gb)


# ---------------------------------------------------------------------------
# Full-size workloads: the same definitions, evaluated on subsets.
# ---------------------------------------------------------------------------

def lse_rows_blocked(hidden, weight, bias, *, block_rows: int = 1024, rows=None,
                     weight64: np.ndarray | None = None, progress=None) -> np.ndarray:
    """lse_i for every row (or the given rows), one block of rows at a time.

    lse is a per-row quantity, so evaluating it block by block is the same
    definition; only host memory changes (float32 inputs, float64 blocks).
    """
    w64 = np.asarray(weight, dtype=np.float64) if weight64 is None else weight64
    b64 = None if bias is None else np.asarray(bias, dtype=np.float64)
    idx = np.arange(np.shape(hidden)[0]) if rows is None else np.asarray(rows)
    out = np.empty(idx.shape[0])
    for s in range(0, idx.shape[0], block_rows):
        sel = idx[s:s + block_rows]
        z = np.asarray(hidden[sel], dtype=np.float64) @ w64.T
        if b64 is not None:
            z += b64[None, :]
        out[s:s + len(sel)] = row_logsumexp(z)
        if progress is not None:
            progress(s + len(sel), idx.shape[0])
    return out


def rows_reference(hidden, weight, bias, labels, rows, *, n_valid: int,
                   ignore_index: int = IGNORE_INDEX, reduction: str = "sum",
                   grad_scale=1.0, weight64: np.ndarray | None = None):
    """lse, l_i and grad_hidden rows for a subset of rows. A row's lse, loss
    and grad_hidden depend only on that row (and the global n_valid for mean)."""
    rows = np.asarray(rows)
    w64 = np.asarray(weight, dtype=np.float64) if weight64 is None else weight64
    lab = np.asarray(labels, dtype=np.int64)[rows]
    v = w64.shape[0]
    valid = valid_rows(lab, v, ignore_index)
    z = logits(np.asarray(hidden[rows], dtype=np.float64), w64, bias)
    lse = row_logsumexp(z)
    row_loss = np.where(valid, lse - _label_logits(z, lab, valid), 0.0)
    scale = row_scale(reduction, n_valid, grad_scale, len(rows))
    g = dlogits(z, lse, lab, valid, scale)
    return lse, row_loss, g @ w64


def label_logits_rows(hidden, weight, bias, labels, rows) -> np.ndarray:
    """z_{i, y_i} = h_i . W_{y_i} + b_{y_i} (float64) for the given rows, whose
    labels must be valid: the same entry of z = h W^T + b as ``_label_logits``
    picks from materialised logits, without forming the other V - 1."""
    rows = np.asarray(rows)
    lab = np.asarray(labels, dtype=np.int64)[rows]
    h64 = np.asarray(hidden[rows], dtype=np.float64)
    w64 = np.asarray(weight[lab], dtype=np.float64)
    zy = np.einsum("ij,ij->i", h64, w64)
    if bias is not None:
        zy = zy + np.asarray(bias, dtype=np.float64)[lab]
    return zy


def loss_sum_from_lse(hidden, weight, bias, labels, lse_all, *, ignore_index: int = IGNORE_INDEX,
                      block_rows: int = 8192) -> tuple[float, int]:
    """(sum_i l_i, n_valid) from every row's lse (``lse_rows_blocked``): l_i =
    valid_i (lse_i - z_{i, y_i}), the per-token cross-entropy of the pages
    summed over all rows (LlamaFactory section 4, ``reduction="none"`` then a
    sum). Used for the full-size workloads, where [N, V] does not fit; the
    label logits are gathered one block of rows at a time (host memory only).
    ``hidden`` and ``weight`` may be any objects whose row indexing returns
    float arrays and that have a ``shape``."""
    labels = np.asarray(labels, dtype=np.int64)
    valid = valid_rows(labels, np.shape(weight)[0], ignore_index)
    rows = np.flatnonzero(valid)
    lse_all = np.asarray(lse_all, dtype=np.float64)
    row_loss = np.zeros(labels.shape[0])
    for s in range(0, rows.shape[0], block_rows):
        r = rows[s:s + block_rows]
        row_loss[r] = lse_all[r] - label_logits_rows(hidden, weight, bias, labels, r)
    return float(np.sum(row_loss)), int(valid.sum())


def cols_reference(hidden, weight, bias, labels, lse_all, cols, *, n_valid: int,
                   ignore_index: int = IGNORE_INDEX, reduction: str = "sum",
                   grad_scale=1.0, block_rows: int = 8192):
    """grad_weight rows and grad_bias entries for a subset of vocabulary ids:
    grad_weight[j] = sum_i G_ij h_i over ALL rows, which needs every row's lse
    (``lse_all``, from ``lse_rows_blocked``)."""
    cols = np.asarray(cols)
    labels = np.asarray(labels, dtype=np.int64)
    n = labels.shape[0]
    valid = valid_rows(labels, np.shape(weight)[0], ignore_index)
    scale = row_scale(reduction, n_valid, grad_scale, n)
    wc = np.asarray(weight[cols], dtype=np.float64)
    bc = None if bias is None else np.asarray(bias, dtype=np.float64)[cols]
    gw = np.zeros((len(cols), wc.shape[1]))
    gb = np.zeros(len(cols))
    for s in range(0, n, block_rows):
        e = min(n, s + block_rows)
        h64 = np.asarray(hidden[s:e], dtype=np.float64)
        z = h64 @ wc.T
        if bc is not None:
            z += bc[None, :]
        g = np.exp(z - lse_all[s:e, None])
        g -= (labels[s:e, None] == cols[None, :])
        g *= (scale[s:e] * valid[s:e])[:, None]
        gw += g.T @ h64
        gb += g.sum(axis=0)
    return gw, gb
