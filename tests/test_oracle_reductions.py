"""Pins of the oracle's other reductions (sum, per-token "none" with an
upstream gradient), its per-token log-probabilities and its weighted dlogits,
against things other than the oracle:

* torch's float64 ``cross_entropy(reduction="sum" / "none")`` with autograd
  (for "none", the backward of sum_i g_i l_i) and ``log_softmax``;
* central finite differences of L = sum_i g_i l_i written out directly with
  scipy's logsumexp;
* the mean reduction being the original definition.

``test_planted_mistakes_ex`` plants a mistake in one of the new steps at a
time and checks that some pin fails.
"""
import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
from oracle import flce_ref as om

II = -100


def _rand(N, H, V, seed, n_ign=2, ws=0.3):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((N, H))
    W = rng.standard_normal((V, H)) * ws
    y = rng.integers(0, V, size=N)
    y[rng.permutation(N)[:n_ign]] = II
    g = rng.standard_normal(N)
    return X, W, y, g


def _rel(a, b):
    a, b = np.asarray(a, float), np.asarray(b, float)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _torch_ref(X, W, y, reduction, g=None):
    import torch
    Xt = torch.tensor(X, dtype=torch.float64, requires_grad=True)
    Wt = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    yt = torch.tensor(y)
    Z = Xt @ Wt.T
    out = torch.nn.functional.cross_entropy(Z, yt, ignore_index=II, reduction=reduction)
    if reduction == "none":
        obj = (out * torch.tensor(g if g is not None else np.ones(len(y)))).sum()
        loss = float(out.sum())
        rl = out.detach().numpy()
    else:
        obj = out
        loss = out.item()
        rl = None
    obj.backward()
    lp = torch.log_softmax(Z.detach(), dim=1)
    valid = yt != II
    logprob = torch.where(valid, lp.gather(1, yt.clamp(min=0)[:, None])[:, 0],
                          torch.zeros(()))
    return loss, rl, logprob.numpy(), Xt.grad.numpy(), Wt.grad.numpy()


# ------------------------------------------------------------------ pins

def pin_mean_is_definition(fx):
    X, W, y, _ = _rand(9, 5, 13, 1)
    a = fx(X, W, y, II, "mean")
    b = om.flce(X, W, y, II)
    assert abs(a.loss - b.loss) <= 1e-12 * abs(b.loss)
    assert _rel(a.dX, b.dX) <= 1e-12 and _rel(a.dW, b.dW) <= 1e-12


def pin_torch_sum(fx):
    X, W, y, _ = _rand(11, 6, 17, 2)
    r = fx(X, W, y, II, "sum")
    loss, _, logprob, dX, dW = _torch_ref(X, W, y, "sum")
    assert abs(r.loss - loss) <= 1e-12 * abs(loss)
    assert _rel(r.dX, dX) <= 1e-10 and _rel(r.dW, dW) <= 1e-10
    assert _rel(r.logprob, logprob) <= 1e-12


def pin_torch_none(fx):
    X, W, y, g = _rand(12, 7, 19, 3, n_ign=3)
    r = fx(X, W, y, II, "none", grad_rows=g)
    loss, rl, logprob, dX, dW = _torch_ref(X, W, y, "none", g)
    assert _rel(r.row_loss, rl) <= 1e-12
    assert abs(r.loss - loss) <= 1e-12 * abs(loss)
    assert _rel(r.dX, dX) <= 1e-10 and _rel(r.dW, dW) <= 1e-10
    assert _rel(r.logprob, logprob) <= 1e-12


def pin_finite_differences_weighted(fx):
    """L(X, W) = sum_{valid i} g_i (logsumexp(z_i) - z_{i,y_i}), written out."""
    X, W, y, g = _rand(5, 4, 6, 4, n_ign=1)
    valid = y != II

    def L(X_, W_):
        Z = X_ @ W_.T
        l = logsumexp(Z, axis=1) - Z[np.arange(len(y)), np.where(valid, y, 0)]
        return float(np.sum(np.where(valid, g * l, 0.0)))

    r = fx(X, W, y, II, "none", grad_rows=g)
    h = 1e-5
    for A, grad in ((X, r.dX), (W, r.dW)):
        for idx in np.ndindex(A.shape):
            Ap, Am = A.copy(), A.copy()
            Ap[idx] += h
            Am[idx] -= h
            fd = (L(Ap, W) - L(Am, W)) / (2 * h) if A is X else (L(X, Ap) - L(X, Am)) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-7 * max(1.0, abs(fd)), (idx, fd, grad[idx])


def pin_sum_is_mean_times_n(fx):
    X, W, y, _ = _rand(10, 5, 11, 5, n_ign=4)
    s = fx(X, W, y, II, "sum")
    m = fx(X, W, y, II, "mean")
    nv = int((y != II).sum())
    assert abs(s.loss - nv * m.loss) <= 1e-12 * abs(s.loss)
    assert _rel(s.dW, nv * m.dW) <= 1e-12


PINS = [pin_mean_is_definition, pin_torch_sum, pin_torch_none,
        pin_finite_differences_weighted, pin_sum_is_mean_times_n]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin_ex(pin):
    pin(oracle.flce_ex)


def test_grad_rows_only_with_none():
    X, W, y, g = _rand(4, 3, 5, 6)
    with pytest.raises(ValueError):
        oracle.flce_ex(X, W, y, II, "sum", grad_rows=g)


# ------------------------------------------------------------------ planted mistakes

def _m_weights_keep_ignored(valid, n_valid, reduction, grad_rows=None):
    w = {"mean": np.full(valid.shape, 1.0 / max(n_valid, 1)), "sum": np.ones(valid.shape)}.get(
        reduction, np.ones(valid.shape) if grad_rows is None else np.asarray(grad_rows, float))
    return w


def _m_sum_normalised(valid, n_valid, reduction, grad_rows=None):
    w = np.ones(valid.shape) / max(n_valid, 1)
    if reduction == "none" and grad_rows is not None:
        w = np.asarray(grad_rows, float)
    return np.where(valid, w, 0.0)


def _m_none_ignores_grad_rows(valid, n_valid, reduction, grad_rows=None):
    w = np.full(valid.shape, 1.0 / max(n_valid, 1)) if reduction == "mean" else np.ones(valid.shape)
    return np.where(valid, w, 0.0)


def _m_weight_applied_twice(Z, lse, labels, weights, col_ids=None):
    P = np.exp(Z - lse[:, None])
    onehot = (labels[:, None] == np.arange(Z.shape[1])[None, :]).astype(float)
    return weights[:, None] ** 2 * (P - onehot)


def _m_weighted_no_onehot(Z, lse, labels, weights, col_ids=None):
    return weights[:, None] * np.exp(Z - lse[:, None])


def _m_logprob_sign(lse, zy, valid):
    return np.where(valid, lse - zy, 0.0)


def _m_logprob_unmasked(lse, zy, valid):
    return zy - lse


MISTAKES = [("token_weights", _m_weights_keep_ignored), ("token_weights", _m_sum_normalised),
            ("token_weights", _m_none_ignores_grad_rows),
            ("dlogits_weighted", _m_weight_applied_twice),
            ("dlogits_weighted", _m_weighted_no_onehot),
            ("log_probs", _m_logprob_sign), ("log_probs", _m_logprob_unmasked)]


@pytest.mark.parametrize("step,mistake", MISTAKES, ids=[m.__name__ for _, m in MISTAKES])
def test_planted_mistakes_ex(monkeypatch, step, mistake):
    monkeypatch.setattr(om, step, mistake)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(oracle.flce_ex)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {mistake.__name__}"


# ------------------------------------------------------------------ cross-entropy on given logits

def _torch_ce(Z, y, reduction, g=None):
    import torch
    Zt = torch.tensor(Z, dtype=torch.float64, requires_grad=True)
    out = torch.nn.functional.cross_entropy(Zt, torch.tensor(y), ignore_index=II,
                                            reduction=reduction)
    if reduction == "none":
        (out * torch.tensor(g if g is not None else np.ones(len(y)))).sum().backward()
        return float(out.sum()), out.detach().numpy(), Zt.grad.numpy()
    out.backward()
    return out.item(), None, Zt.grad.numpy()


@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_cross_entropy_against_torch(reduction):
    rng = np.random.default_rng(21)
    Z = rng.standard_normal((13, 29)) * 3.0
    y = rng.integers(0, 29, size=13)
    y[[2, 7]] = II
    g = rng.standard_normal(13) if reduction == "none" else None
    r = oracle.cross_entropy(Z, y, II, reduction, grad_rows=g)
    loss, rl, dZ = _torch_ce(Z, y, reduction, g)
    assert abs(r.loss - loss) <= 1e-12 * abs(loss)
    assert _rel(r.dZ, dZ) <= 1e-12
    if rl is not None:
        assert _rel(r.row_loss, rl) <= 1e-12


def test_cross_entropy_is_flce_on_logits():
    """Given Z = X W^T, the cross-entropy of Z has the loss of the fused
    definition and dX = dZ W, dW = dZ^T X."""
    X, W, y, g = _rand(8, 5, 11, 22)
    for red, gr in (("mean", None), ("none", g)):
        a = oracle.cross_entropy(X @ W.T, y, II, red, grad_rows=gr)
        b = oracle.flce_ex(X, W, y, II, red, grad_rows=gr)
        assert abs(a.loss - b.loss) <= 1e-12 * abs(b.loss)
        assert _rel(a.dZ @ W, b.dX) <= 1e-12 and _rel(a.dZ.T @ X, b.dW) <= 1e-12
