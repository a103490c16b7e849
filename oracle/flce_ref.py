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


# ------------------------------------------------------------------ odds-ratio preference loss
# The project overview page lists fused-linear post-training losses built on
# the same chunked projection ("Kernels de Pós-Treinamento") and calls the
# ORPO one as orpo_loss(lm_head.weight, x, target) ("Exemplo de Uso de Perda
# de Pós-Treinamento").  The pages give no formula; this is the published
# definition of Odds Ratio Preference Optimization (Hong, Lee and Thorne,
# 2024) on top of the per-token log-probabilities above:
#   a_s   = mean over the valid tokens t of sequence s of log p(y_t)
#   odds  = p / (1 - p) with p = exp(a_s), so log odds(a) = a - log(1 - e^a)
#   d_i   = log odds(a_chosen_i) - log odds(a_rejected_i)
#   L_OR  = mean over pairs of -log sigmoid(d_i)
#   L_SFT = mean over the chosen sequences' valid tokens of -log p(y_t)
#   L     = L_SFT + beta L_OR
# Layout (read from the call form): the rows of X are 2B sequences of T
# tokens, the B chosen sequences first, then the B rejected ones, pair i =
# (sequence i, sequence B + i); ignore_index marks the tokens that are not
# scored (prompt, padding).  A pair with an empty sequence adds nothing to
# L_OR (the mean still divides by B).

@dataclasses.dataclass
class ORPOResult:
    loss: float
    nll: float                   # L_SFT
    or_loss: float               # L_OR (before beta)
    chosen_logp: np.ndarray      # [B] a of each chosen sequence (0 if empty)
    rejected_logp: np.ndarray    # [B]
    log_odds_ratio: np.ndarray   # [B] d_i (0 for pairs with an empty sequence)
    dX: np.ndarray | None
    dW: np.ndarray | None


def sequence_logp(lp: np.ndarray, valid: np.ndarray, n_seq: int):
    """Mean log-probability over each sequence's valid tokens and the number
    of valid tokens; lp and valid are [n_seq * T], sequence-major."""
    lp = lp.reshape(n_seq, -1)
    valid = valid.reshape(n_seq, -1)
    n = valid.sum(axis=1)
    a = np.where(n > 0, np.where(valid, lp, 0.0).sum(axis=1) / np.maximum(n, 1), 0.0)
    return a, n


def log_odds(a: np.ndarray) -> np.ndarray:
    """log(p / (1 - p)) for log p = a < 0."""
    return a - np.log(-np.expm1(a))


def odds_ratio_loss(d: np.ndarray, live: np.ndarray) -> np.ndarray:
    """-log sigmoid(d) = log(1 + e^-d) per pair, 0 where the pair is not live."""
    return np.where(live, np.logaddexp(0.0, -d), 0.0)


def orpo_token_weights(a_c, n_c, a_r, n_r, d, live, valid, n_pairs: int, n_chosen_valid: int,
                       beta: float) -> np.ndarray:
    """w_t = -dL/d log p(y_t) for every token (sequence-major [2B * T]): the
    loss above as L = sum_t w_t l_t in the per-token losses l_t = -log p(y_t).

    dL_SFT/d lp_t = -1/N_c on chosen valid tokens; through a_s = mean of lp,
    dL_OR,i/d a_c = -sigmoid(-d_i) / (1 - e^{a_c}) and
    dL_OR,i/d a_r = +sigmoid(-d_i) / (1 - e^{a_r}), each spread as 1/n_s over
    the sequence's valid tokens, and L_OR is their mean over B pairs."""
    s = np.where(live, 1.0 / (1.0 + np.exp(d)), 0.0)                # sigmoid(-d)
    a_c = np.where(live, a_c, -1.0)                                 # pairs not live: s = 0
    a_r = np.where(live, a_r, -1.0)
    gc = -beta / n_pairs * s / (-np.expm1(a_c)) / np.maximum(n_c, 1)
    gr = beta / n_pairs * s / (-np.expm1(a_r)) / np.maximum(n_r, 1)
    T = valid.size // (2 * n_pairs)
    v = valid.reshape(2 * n_pairs, T)
    dlp = np.zeros((2 * n_pairs, T))
    dlp[:n_pairs] = -1.0 / max(n_chosen_valid, 1) + gc[:, None]
    dlp[n_pairs:] = gr[:, None]
    return np.where(v, -dlp, 0.0).reshape(-1)


def orpo_terms(lp: np.ndarray, valid: np.ndarray, n_pairs: int, beta: float):
    """From the per-token log-probabilities (sequence-major, 0 on unscored
    tokens): loss, NLL, L_OR, a_chosen, a_rejected, d and the per-token
    weights of the backward."""
    a, n = sequence_logp(lp, valid, 2 * n_pairs)
    a_c, a_r, n_c, n_r = a[:n_pairs], a[n_pairs:], n[:n_pairs], n[n_pairs:]
    live = (n_c > 0) & (n_r > 0)
    d = np.where(live, log_odds(np.where(live, a_c, -1.0)) - log_odds(np.where(live, a_r, -1.0)),
                 0.0)
    half = lp.size // 2
    n_chosen_valid = int(valid[:half].sum())
    nll = float(-lp[:half].sum() / max(n_chosen_valid, 1))
    or_loss = float(odds_ratio_loss(d, live).sum() / n_pairs)
    w = orpo_token_weights(a_c, n_c, a_r, n_r, d, live, valid, n_pairs, n_chosen_valid, beta)
    return nll + beta * or_loss, nll, or_loss, a_c, a_r, d, w


def _orpo_shape(N: int, n_pairs: int):
    if n_pairs <= 0 or N % (2 * n_pairs) != 0:
        raise ValueError("X must hold 2 * n_pairs sequences of equal length")


def orpo(X, W, labels, n_pairs: int, ignore_index: int = IGNORE_INDEX, beta: float = 0.1,
         grads: bool = True) -> ORPOResult:
    """ORPO loss of 2 * n_pairs sequences (rows of X sequence-major, chosen
    first) and its gradients."""
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    _orpo_shape(X.shape[0], n_pairs)
    valid = valid_mask(labels, W.shape[0], ignore_index)
    Z = logits(X, W)
    lse = row_logsumexp(Z)
    lp = log_probs(lse, target_logit(Z, labels, valid), valid)
    loss, nll, or_loss, a_c, a_r, d, w = orpo_terms(lp, valid, n_pairs, beta)
    if not grads:
        return ORPOResult(loss, nll, or_loss, a_c, a_r, d, None, None)
    G = dlogits_weighted(Z, lse, labels, w)
    return ORPOResult(loss, nll, or_loss, a_c, a_r, d, grad_input(G, W), grad_weight(G, X))


def orpo_rows(X, W, labels, n_pairs: int, rows, vrows, ignore_index: int = IGNORE_INDEX,
              beta: float = 0.1, block: int = 256) -> ORPOResult:
    """The same loss for workloads whose logits do not fit in host memory:
    every token's log-probability from complete logits rows in blocks, and
    dX only for ``rows``, dW only for vocabulary rows ``vrows``."""
    labels = np.asarray(labels, dtype=np.int64)
    Wd = np.asarray(W, dtype=np.float64)
    _orpo_shape(X.shape[0], n_pairs)
    valid = valid_mask(labels, Wd.shape[0], ignore_index)
    lse, rl, _ = forward_rows(X, Wd, labels, None, ignore_index, block)
    lp = np.where(valid, -rl, 0.0)
    loss, nll, or_loss, a_c, a_r, d, w = orpo_terms(lp, valid, n_pairs, beta)
    rows = np.asarray(rows, dtype=np.int64)
    Z = logits(np.asarray(X[rows], dtype=np.float64), Wd)
    dX = grad_input(dlogits_weighted(Z, row_logsumexp(Z), labels[rows], w[rows]), Wd)
    vrows = np.asarray(vrows, dtype=np.int64)
    Xd = np.asarray(X, dtype=np.float64)
    Zc = logits(Xd, Wd[vrows])
    dW = grad_weight(dlogits_weighted(Zc, lse, labels, w, col_ids=vrows), Xd)
    return ORPOResult(loss, nll, or_loss, a_c, a_r, d, dX, dW)


# ------------------------------------------------------------------ other pairwise preference losses
# The same page lists DPO, CPO and SimPO beside ORPO ("Kernels de
# Pós-Treinamento"), again without formulas.  Each is its published pairwise
# form on the same batch layout: with S_s = sum and a_s = S_s / n_s = mean of
# log p(y_t) over sequence s's scored tokens,
#   SimPO (Meng, Xia and Chen, 2024):      z = beta (a_c - a_r) - gamma
#   CPO   (Xu et al., 2024):               z = beta (S_c - S_r)
#   DPO   (Rafailov et al., 2023):         z = beta ((S_c - R_c) - (S_r - R_r)),
#         R_s the reference model's sequence log-probability (an input)
#   L = alpha NLL + mean over pairs of -log sigmoid(z_i)
# with NLL the token-level mean of -log p over the chosen half, as for ORPO.
# ORPO is the same shape with z = log odds(a_c) - log odds(a_r), alpha = 1
# and beta weighting the pair term.  A pair with an empty sequence adds
# nothing to the pair term.

PAIR_KINDS = ("orpo", "simpo", "cpo", "dpo")


@dataclasses.dataclass
class PreferenceResult:
    loss: float
    nll: float                   # token-level mean of -log p over the chosen half
    pair_loss: float             # mean over pairs of -log sigmoid(z_i)
    chosen_logp: np.ndarray      # [B] the sequence log-probability the loss uses (a or S)
    rejected_logp: np.ndarray    # [B]
    pair_logit: np.ndarray       # [B] z_i (0 for pairs with an empty sequence)
    dX: np.ndarray | None
    dW: np.ndarray | None


def sequence_sums(lp: np.ndarray, valid: np.ndarray, n_seq: int):
    """Sum of log p over each sequence's scored tokens, and their number."""
    lp = lp.reshape(n_seq, -1)
    valid = valid.reshape(n_seq, -1)
    return np.where(valid, lp, 0.0).sum(axis=1), valid.sum(axis=1)


def pair_logit(kind: str, S_c, n_c, S_r, n_r, beta: float, gamma: float, ref_c, ref_r):
    """z_i and its derivatives dz/dS_c, dz/dS_r (live pairs: n_c, n_r > 0)."""
    nc, nr = np.maximum(n_c, 1), np.maximum(n_r, 1)
    if kind == "simpo":
        return beta * (S_c / nc - S_r / nr) - gamma, beta / nc, -beta / nr
    if kind == "cpo":
        return beta * (S_c - S_r), np.full(S_c.shape, beta), np.full(S_c.shape, -beta)
    if kind == "dpo":
        return (beta * ((S_c - ref_c) - (S_r - ref_r)), np.full(S_c.shape, beta),
                np.full(S_c.shape, -beta))
    if kind == "orpo":
        a_c, a_r = np.minimum(S_c / nc, -1e-300), np.minimum(S_r / nr, -1e-300)
        return (log_odds(a_c) - log_odds(a_r), 1.0 / (-np.expm1(a_c)) / nc,
                -1.0 / (-np.expm1(a_r)) / nr)
    raise ValueError(f"unknown preference loss {kind!r}")


def preference_token_weights(dz_c, dz_r, z, live, valid, n_pairs: int, n_chosen_valid: int,
                             alpha: float, lam: float) -> np.ndarray:
    """w_t = -dL/d log p(y_t): dL/dz_i = -lam sigmoid(-z_i) / B, reaching each
    token of the pair's sequences through dz/dS; the NLL adds -alpha / N_c on
    chosen scored tokens."""
    g = np.where(live, -lam / n_pairs / (1.0 + np.exp(z)), 0.0)      # dL/dz
    T = valid.size // (2 * n_pairs)
    v = valid.reshape(2 * n_pairs, T)
    dlp = np.zeros((2 * n_pairs, T))
    dlp[:n_pairs] = -alpha / max(n_chosen_valid, 1) + (g * dz_c)[:, None]
    dlp[n_pairs:] = (g * dz_r)[:, None]
    return np.where(v, -dlp, 0.0).reshape(-1)


def preference_terms(kind: str, lp, valid, n_pairs: int, beta: float, gamma: float,
                     alpha: float, ref_c=None, ref_r=None):
    """Loss, NLL, pair loss, sequence scores, z and the backward's per-token
    weights from the per-token log-probabilities."""
    S, n = sequence_sums(lp, valid, 2 * n_pairs)
    S_c, S_r, n_c, n_r = S[:n_pairs], S[n_pairs:], n[:n_pairs], n[n_pairs:]
    live = (n_c > 0) & (n_r > 0)
    if kind == "dpo" and (ref_c is None or ref_r is None):
        raise ValueError("DPO needs the reference sequence log-probabilities")
    ref_c = np.zeros(n_pairs) if ref_c is None else np.asarray(ref_c, dtype=np.float64)
    ref_r = np.zeros(n_pairs) if ref_r is None else np.asarray(ref_r, dtype=np.float64)
    z, dz_c, dz_r = pair_logit(kind, S_c, n_c, S_r, n_r, beta, gamma, ref_c, ref_r)
    z = np.where(live, z, 0.0)
    lam = beta if kind == "orpo" else 1.0
    half = lp.size // 2
    n_chosen_valid = int(valid[:half].sum())
    nll = float(-lp[:half].sum() / max(n_chosen_valid, 1))
    pair_loss = float(np.where(live, np.logaddexp(0.0, -z), 0.0).sum() / n_pairs)
    w = preference_token_weights(dz_c, dz_r, z, live, valid, n_pairs, n_chosen_valid, alpha, lam)
    mean_based = kind in ("orpo", "simpo")
    u_c = np.where(n_c > 0, S_c / np.maximum(n_c, 1), 0.0) if mean_based else S_c
    u_r = np.where(n_r > 0, S_r / np.maximum(n_r, 1), 0.0) if mean_based else S_r
    return alpha * nll + lam * pair_loss, nll, pair_loss, u_c, u_r, z, w


def preference(kind: str, X, W, labels, n_pairs: int, ignore_index: int = IGNORE_INDEX,
               beta: float = 0.1, gamma: float = 0.0, alpha: float = 0.0, ref_chosen=None,
               ref_rejected=None, grads: bool = True) -> PreferenceResult:
    """A pairwise preference loss of 2 * n_pairs sequences (rows of X
    sequence-major, chosen first) and its gradients."""
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    _orpo_shape(X.shape[0], n_pairs)
    valid = valid_mask(labels, W.shape[0], ignore_index)
    Z = logits(X, W)
    lse = row_logsumexp(Z)
    lp = log_probs(lse, target_logit(Z, labels, valid), valid)
    loss, nll, pl, u_c, u_r, z, w = preference_terms(kind, lp, valid, n_pairs, beta, gamma, alpha,
                                                     ref_chosen, ref_rejected)
    if not grads:
        return PreferenceResult(loss, nll, pl, u_c, u_r, z, None, None)
    G = dlogits_weighted(Z, lse, labels, w)
    return PreferenceResult(loss, nll, pl, u_c, u_r, z, grad_input(G, W), grad_weight(G, X))


# ------------------------------------------------------------------ unpaired preference loss (KTO)
# The last of the page's post-training list ("Kernels de Pós-Treinamento"),
# again without a formula: Kahneman-Tversky Optimization (Ethayarajh et al.,
# 2024).  Sequences are unpaired, each marked desirable or undesirable; with
# S the sum of log p(y_t) over a sequence's scored tokens, R the reference
# model's (an input) and r = S - R,
#   desirable:    l = lambda_d (1 - sigmoid(beta (r - z0)))
#   undesirable:  l = lambda_u (1 - sigmoid(beta (z0 - r)))
#   L = mean over sequences of l
# z0 is the reference point (the KL term of the paper), an input through
# which no gradient flows.  Layout: the rows of X are n_seq sequences of T
# tokens; ignore_index marks unscored tokens.

@dataclasses.dataclass
class KTOResult:
    loss: float
    logp: np.ndarray             # [n_seq] S
    reward: np.ndarray           # [n_seq] r = S - R
    dX: np.ndarray | None
    dW: np.ndarray | None


def kto_sequence_terms(r, desirable, beta: float, z0: float, lambda_d: float, lambda_u: float):
    """Per-sequence loss l and dl/dr."""
    u = np.where(desirable, beta * (r - z0), beta * (z0 - r))
    sig = 1.0 / (1.0 + np.exp(-u))
    sig_neg = 1.0 / (1.0 + np.exp(u))                # 1 - sigmoid(u), without cancellation
    lam = np.where(desirable, lambda_d, lambda_u)
    l = lam * sig_neg
    dl_du = -lam * sig * sig_neg
    return l, dl_du * np.where(desirable, beta, -beta)


def kto_token_weights(dl_dr, valid, n_seq: int) -> np.ndarray:
    """w_t = -dL/d log p(y_t) = -(1/n_seq) dl/dr of the token's sequence."""
    T = valid.size // n_seq
    v = valid.reshape(n_seq, T)
    return np.where(v, (-dl_dr / n_seq)[:, None], 0.0).reshape(-1)


def kto_reference_point(X, W, labels, n_seq: int, ref_logp,
                        ignore_index: int = IGNORE_INDEX) -> float:
    """KTO's reference point estimated from a batch (Ethayarajh et al., 2024):
    the rows of X are n_seq completions each scored under a prompt that is
    not its own (mismatched pairs), ref_logp the reference model's sums of
    log p over the same completions; z0 = max(0, mean over sequences of
    S - R), the policy-to-reference KL estimate clamped at zero.  No gradient
    flows through it."""
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    if n_seq <= 0 or X.shape[0] % n_seq != 0:
        raise ValueError("X must hold n_seq sequences of equal length")
    valid = valid_mask(labels, W.shape[0], ignore_index)
    Z = logits(X, W)
    lp = log_probs(row_logsumexp(Z), target_logit(Z, labels, valid), valid)
    S, _ = sequence_sums(lp, valid, n_seq)
    return max(0.0, float(np.mean(S - np.asarray(ref_logp, dtype=np.float64))))


def kto(X, W, labels, n_seq: int, desirable, ref_logp, ignore_index: int = IGNORE_INDEX,
        beta: float = 0.1, z0: float = 0.0, lambda_d: float = 1.0, lambda_u: float = 1.0,
        grads: bool = True) -> KTOResult:
    """KTO loss of n_seq sequences (rows of X sequence-major) and its gradients."""
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    if n_seq <= 0 or X.shape[0] % n_seq != 0:
        raise ValueError("X must hold n_seq sequences of equal length")
    desirable = np.asarray(desirable, dtype=bool)
    ref_logp = np.asarray(ref_logp, dtype=np.float64)
    valid = valid_mask(labels, W.shape[0], ignore_index)
    Z = logits(X, W)
    lse = row_logsumexp(Z)
    lp = log_probs(lse, target_logit(Z, labels, valid), valid)
    S, _ = sequence_sums(lp, valid, n_seq)
    r = S - ref_logp
    l, dl_dr = kto_sequence_terms(r, desirable, beta, z0, lambda_d, lambda_u)
    loss = float(l.sum() / n_seq)
    if not grads:
        return KTOResult(loss, S, r, None, None)
    G = dlogits_weighted(Z, lse, labels, kto_token_weights(dl_dr, valid, n_seq))
    return KTOResult(loss, S, r, grad_input(G, W), grad_weight(G, X))
