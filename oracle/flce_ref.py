"""fp64 CPU oracle for fused linear cross-entropy (test infrastructure).

This is the checker, not the product.  Only ``tests/``, the smoke check in
``__graft_entry__.py`` and the ``cpu_baseline`` leg of ``bench.py`` may import
it.  It shares no code with the HIP library and imports nothing from it.

What it computes is the plain definition of the method the Liger Kernel pages
describe:

* The ms-swift blog page (mechanism paragraph, after the RMSNorm+Linear+RoPE
  example) describes fused linear cross entropy as merging the last linear
  layer with the cross-entropy loss, so the quantity is CE(X W^T, y).
* The project overview page ("Implementação Técnica") states the kernels do
  no approximate computation, and ("Computação em Chunk") that chunking only
  splits the work to cut peak memory.  Hence the exact result has a plain
  definition and this oracle is that definition written out, with the full
  N x V logits materialised and no chunking, blocking or fusion.
* The same page ("Método de API de Baixo Nível") calls the loss as
  ``loss_fn(weight, input, target)`` with weight = ``nn.Linear(H, V).weight``
  ([V, H]), input [N, H] and integer targets [N]; only the weight enters (no
  bias).

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):
  * reduction is the mean over tokens whose label is not ``ignore_index``
    (-100); with no valid token the loss and both gradients are 0;
  * a label that is neither ``ignore_index`` nor in [0, V) is an error;
  * ``ignore_index`` is compared for equality, also when it lies in [0, V);
  * no label shift inside the loss: row i of X is scored against target i.

All arithmetic is float64.  Inputs are converted exactly (fp32 and bf16
values are representable in fp64).  Parity status of every function: pinned
by the ``-m "not gpu"`` tests (closed forms, invariants, finite differences,
a pure-Python brute force and torch's float64 cross_entropy).
"""
from __future__ import annotations

import dataclasses

import numpy as np

IGNORE_INDEX = -100


@dataclasses.dataclass
class Result:
    loss: float
    dX: np.ndarray | None      # [N, H] float64
    dW: np.ndarray | None      # [V, H] float64
    lse: np.ndarray            # [N] log-sum-exp of each logits row
    row_loss: np.ndarray       # [N] lse - z_y, 0 on ignored rows
    n_valid: int


# ------------------------------------------------------------------ steps
# Each step is a module-level function so that a test can plant a mistake in
# exactly one of them and check that some pin catches it.

def valid_mask(labels: np.ndarray, V: int, ignore_index: int = IGNORE_INDEX) -> np.ndarray:
    """valid_i = (y_i != ignore_index); raise on a valid label outside [0, V)."""
    labels = np.asarray(labels, dtype=np.int64)
    valid = labels != ignore_index
    bad = valid & ((labels < 0) | (labels >= V))
    if np.any(bad):
        i = int(np.flatnonzero(bad)[0])
        raise ValueError(f"label {int(labels[i])} at row {i} is outside [0, {V})")
    return valid


def logits(X: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Z = X W^T: row i, column v is <x_i, w_v> (the LM-head projection)."""
    return X @ W.T


def row_logsumexp(Z: np.ndarray) -> np.ndarray:
    """lse_i = m_i + log sum_v exp(Z_iv - m_i), m_i = max_v Z_iv (two passes)."""
    m = Z.max(axis=1)
    return m + np.log(np.exp(Z - m[:, None]).sum(axis=1))


def target_logit(Z: np.ndarray, labels: np.ndarray, valid: np.ndarray) -> np.ndarray:
    """z_{i, y_i} on valid rows, 0 elsewhere."""
    out = np.zeros(Z.shape[0])
    idx = np.flatnonzero(valid)
    out[idx] = Z[idx, labels[idx]]
    return out


def row_losses(lse: np.ndarray, zy: np.ndarray, valid: np.ndarray) -> np.ndarray:
    """Per-token cross-entropy -log softmax(z_i)_{y_i} = lse_i - z_{i,y_i}."""
    return np.where(valid, lse - zy, 0.0)


def mean_loss(row_loss: np.ndarray, n_valid: int) -> float:
    """Mean over the valid tokens (0 when there are none)."""
    return float(row_loss.sum() / max(n_valid, 1))


def dlogits(Z: np.ndarray, lse: np.ndarray, labels: np.ndarray, valid: np.ndarray,
            n_valid: int, col_ids: np.ndarray | None = None) -> np.ndarray:
    """dL/dZ = (softmax(Z) - onehot(y)) / N_valid on valid rows, 0 elsewhere.

    ``col_ids`` names the vocabulary ids of Z's columns when Z holds only some
    of them (default: 0..V-1)."""
    if col_ids is None:
        col_ids = np.arange(Z.shape[1])
    P = np.exp(Z - lse[:, None])
    onehot = (labels[:, None] == col_ids[None, :]).astype(np.float64)
    G = (P - onehot) / max(n_valid, 1)
    G[~valid] = 0.0
    return G


def grad_input(G: np.ndarray, W: np.ndarray) -> np.ndarray:
    """dX = G W (chain rule through Z = X W^T)."""
    return G @ W


def grad_weight(G: np.ndarray, X: np.ndarray) -> np.ndarray:
    """dW = G^T X (chain rule through Z = X W^T)."""
    return G.T @ X


# ------------------------------------------------------------------ full definition

def flce(X, W, labels, ignore_index: int = IGNORE_INDEX, grads: bool = True) -> Result:
    """Loss, dX and dW of mean cross-entropy over CE(X W^T, y), all in fp64.

    X [N, H], W [V, H], labels [N] int.  The full logits are materialised."""
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    V = W.shape[0]
    valid = valid_mask(labels, V, ignore_index)
    n_valid = int(valid.sum())
    Z = logits(X, W)
    lse = row_logsumexp(Z)
    rl = row_losses(lse, target_logit(Z, labels, valid), valid)
    loss = mean_loss(rl, n_valid)
    if not grads:
        return Result(loss, None, None, lse, rl, n_valid)
    G = dlogits(Z, lse, labels, valid, n_valid)
    return Result(loss, grad_input(G, W), grad_weight(G, X), lse, rl, n_valid)


# ------------------------------------------------------------------ other reductions
# The loss that chunked post-training losses build on (the project overview
# page, "Exemplo de Uso de Perda de Pós-Treinamento") is a weighted sum of the
# per-token losses: L = sum_i w_i l_i over valid tokens.  The mean above is
# w_i = 1 / N_valid; the sum is w_i = 1; with the per-token loss vector as the
# output ("none"), w_i is the upstream gradient of that vector.

REDUCTIONS = ("mean", "sum", "none")


def token_weights(valid: np.ndarray, n_valid: int, reduction: str,
                  grad_rows=None) -> np.ndarray:
    """w_i of L = sum_i w_i l_i: 1/N_valid (mean), 1 (sum), grad_rows[i] or 1
    (none); 0 on ignored tokens."""
    if reduction == "mean":
        w = np.full(valid.shape, 1.0 / max(n_valid, 1))
    elif reduction == "sum":
        w = np.ones(valid.shape)
    elif reduction == "none":
        w = np.ones(valid.shape) if grad_rows is None else np.asarray(grad_rows, dtype=np.float64)
    else:
        raise ValueError(f"unknown reduction {reduction!r}")
    return np.where(valid, w, 0.0)


def dlogits_weighted(Z: np.ndarray, lse: np.ndarray, labels: np.ndarray, weights: np.ndarray,
                     col_ids: np.ndarray | None = None) -> np.ndarray:
    """dL/dZ for L = sum_i w_i l_i: row i is w_i (softmax(Z_i) - onehot(y_i))."""
    if col_ids is None:
        col_ids = np.arange(Z.shape[1])
    P = np.exp(Z - lse[:, None])
    onehot = (labels[:, None] == col_ids[None, :]).astype(np.float64)
    return weights[:, None] * (P - onehot)


def log_probs(lse: np.ndarray, zy: np.ndarray, valid: np.ndarray) -> np.ndarray:
    """log softmax(z_i)_{y_i} = z_{i,y_i} - lse_i on valid rows, 0 elsewhere."""
    return np.where(valid, zy - lse, 0.0)


@dataclasses.dataclass
class ResultEx:
    loss: float                # mean, or sum of the per-token losses (sum and none)
    row_loss: np.ndarray       # [N] l_i, 0 on ignored rows
    logprob: np.ndarray        # [N] z_{i,y_i} - lse_i, 0 on ignored rows
    lse: np.ndarray
    dX: np.ndarray | None      # dL/dX for L = sum_i w_i l_i
    dW: np.ndarray | None
    n_valid: int


def flce_ex(X, W, labels, ignore_index: int = IGNORE_INDEX, reduction: str = "mean",
            grad_rows=None, grads: bool = True) -> ResultEx:
    """The definition with a choice of reduction; grad_rows is the upstream
    gradient of the per-token loss vector (reduction "none" only)."""
    if grad_rows is not None and reduction != "none":
        raise ValueError("grad_rows goes with reduction 'none'")
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    V = W.shape[0]
    valid = valid_mask(labels, V, ignore_index)
    n_valid = int(valid.sum())
    Z = logits(X, W)
    lse = row_logsumexp(Z)
    zy = target_logit(Z, labels, valid)
    rl = row_losses(lse, zy, valid)
    loss = mean_loss(rl, n_valid) if reduction == "mean" else float(rl.sum())
    w = token_weights(valid, n_valid, reduction, grad_rows)
    if not grads:
        return ResultEx(loss, rl, log_probs(lse, zy, valid), lse, None, None, n_valid)
    G = dlogits_weighted(Z, lse, labels, w)
    return ResultEx(loss, rl, log_probs(lse, zy, valid), lse, grad_input(G, W),
                    grad_weight(G, X), n_valid)


# ------------------------------------------------------------------ cross-entropy on given logits
# The plain cross-entropy loss the pages list beside the fused one (project
# overview page, "Modelos e Operações"): the same steps with the logits given
# instead of computed from X and W.

@dataclasses.dataclass
class CEResult:
    loss: float
    row_loss: np.ndarray
    logprob: np.ndarray
    lse: np.ndarray
    dZ: np.ndarray | None      # dL/dlogits
    n_valid: int


def cross_entropy(Z, labels, ignore_index: int = IGNORE_INDEX, reduction: str = "mean",
                  grad_rows=None, grads: bool = True) -> CEResult:
    """Cross-entropy of logits Z [N, V] against labels, with its gradient."""
    if grad_rows is not None and reduction != "none":
        raise ValueError("grad_rows goes with reduction 'none'")
    Z = np.asarray(Z, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    valid = valid_mask(labels, Z.shape[1], ignore_index)
    n_valid = int(valid.sum())
    lse = row_logsumexp(Z)
    zy = target_logit(Z, labels, valid)
    rl = row_losses(lse, zy, valid)
    loss = mean_loss(rl, n_valid) if reduction == "mean" else float(rl.sum())
    dZ = None
    if grads:
        dZ = dlogits_weighted(Z, lse, labels, token_weights(valid, n_valid, reduction, grad_rows))
    return CEResult(loss, rl, log_probs(lse, zy, valid), lse, dZ, n_valid)


# ------------------------------------------------------------------ the same definition on parts
# For workloads whose N x V logits do not fit in host memory: each function
# below evaluates the definition above for a subset of outputs, still with
# every logits row complete over the whole vocabulary.

def forward_rows(X, W, labels, rows=None, ignore_index: int = IGNORE_INDEX,
                 block: int = 256):
    """lse and per-token loss for ``rows`` (default: all), in row blocks.

    Returns (lse[rows], row_loss[rows], n_valid over all labels)."""
    labels = np.asarray(labels, dtype=np.int64)
    V = W.shape[0]
    valid = valid_mask(labels, V, ignore_index)
    rows = np.arange(X.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    lse = np.empty(rows.size)
    rl = np.empty(rows.size)
    Wd = np.asarray(W, dtype=np.float64)
    for s in range(0, rows.size, block):
        r = rows[s:s + block]
        Z = logits(np.asarray(X[r], dtype=np.float64), Wd)
        l = row_logsumexp(Z)
        lse[s:s + block] = l
        rl[s:s + block] = row_losses(l, target_logit(Z, labels[r], valid[r]), valid[r])
    return lse, rl, int(valid.sum())


def loss_blocked(X, W, labels, ignore_index: int = IGNORE_INDEX, block: int = 256):
    """Mean loss and lse for all rows without materialising N x V at once."""
    lse, rl, nv = forward_rows(X, W, labels, None, ignore_index, block)
    return mean_loss(rl, nv), lse, rl, nv


def dX_rows(X, W, labels, rows, ignore_index: int = IGNORE_INDEX) -> np.ndarray:
    """Rows ``rows`` of dX = G W; each needs only its own logits row."""
    labels = np.asarray(labels, dtype=np.int64)
    Wd = np.asarray(W, dtype=np.float64)
    valid = valid_mask(labels, Wd.shape[0], ignore_index)
    n_valid = int(valid.sum())
    rows = np.asarray(rows, dtype=np.int64)
    Z = logits(np.asarray(X[rows], dtype=np.float64), Wd)
    G = dlogits(Z, row_logsumexp(Z), labels[rows], valid[rows], n_valid)
    return grad_input(G, Wd)


def dW_rows(X, W, labels, lse, vrows, ignore_index: int = IGNORE_INDEX) -> np.ndarray:
    """Rows ``vrows`` of dW = G^T X; needs lse of every token (from forward_rows)."""
    labels = np.asarray(labels, dtype=np.int64)
    Xd = np.asarray(X, dtype=np.float64)
    V = W.shape[0]
    valid = valid_mask(labels, V, ignore_index)
    n_valid = int(valid.sum())
    vrows = np.asarray(vrows, dtype=np.int64)
    Zc = logits(Xd, np.asarray(W[vrows], dtype=np.float64))   # [N, k] columns vrows of Z
    G = dlogits(Zc, np.asarray(lse, dtype=np.float64), labels, valid, n_valid, col_ids=vrows)
    return grad_weight(G, Xd)
