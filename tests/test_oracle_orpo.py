"""Pins of the oracle's odds-ratio preference loss (oracle.orpo) against
things other than the oracle:

* beta = 0 leaves the mean cross-entropy of the chosen half: torch's float64
  ``cross_entropy(ignore_index=-100)`` with autograd;
* a batch whose rejected sequences equal the chosen ones has log odds ratio 0,
  so L_OR = log 2 exactly, and the odds-ratio part of dW cancels;
* with V = 2 and one scored token per sequence, p / (1 - p) = exp(z_y -
  z_other), so the log odds are logit differences (closed form);
* the same loss built from torch float64 primitives (log_softmax, masked
  means, log1p, logsigmoid) with autograd pins the hand-derived gradient;
* central finite differences of the oracle's own forward pin its gradient to
  its loss;
* a pair with an empty sequence adds nothing to L_OR.

``test_planted_mistakes_orpo`` plants a mistake in one step at a time and
checks that some pin fails.
"""
import numpy as np
import pytest

import oracle
from oracle import flce_ref as om

II = -100


def _batch(B, T, H, V, seed, ws=0.5, prompt=1, pad=1):
    """2B sequences of T tokens, chosen first; the first `prompt` and last
    `pad` tokens of each sequence are not scored."""
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((2 * B * T, H))
    W = rng.standard_normal((V, H)) * ws
    y = rng.integers(0, V, size=(2 * B, T))
    y[:, :prompt] = II
    if pad:
        y[:, T - pad:] = II
    return X, W, y.reshape(-1)


def _rel(a, b):
    a, b = np.asarray(a, float), np.asarray(b, float)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _torch_orpo(X, W, y, B, beta):
    import torch
    Xt = torch.tensor(X, dtype=torch.float64, requires_grad=True)
    Wt = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    yt = torch.tensor(y)
    lp_all = torch.log_softmax(Xt @ Wt.T, dim=1)
    valid = yt != II
    lp = torch.where(valid, lp_all.gather(1, yt.clamp(min=0)[:, None])[:, 0], torch.zeros(()))
    lp = lp.view(2 * B, -1)
    v = valid.view(2 * B, -1).double()
    a = (lp * v).sum(1) / v.sum(1)
    lo = a - torch.log1p(-torch.exp(a))
    d = lo[:B] - lo[B:]
    or_loss = -torch.nn.functional.logsigmoid(d).mean()
    nll = -(lp[:B] * v[:B]).sum() / v[:B].sum()
    loss = nll + beta * or_loss
    loss.backward()
    return loss.item(), Xt.grad.numpy(), Wt.grad.numpy()


# ------------------------------------------------------------------ pins

def pin_beta0_is_chosen_ce(fx):
    import torch
    B, T = 3, 5
    X, W, y = _batch(B, T, 6, 11, 1)
    r = fx(X, W, y, B, II, beta=0.0)
    half = B * T
    Xt = torch.tensor(X[:half], dtype=torch.float64, requires_grad=True)
    Wt = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    out = torch.nn.functional.cross_entropy(Xt @ Wt.T, torch.tensor(y[:half]), ignore_index=II)
    out.backward()
    assert abs(r.loss - out.item()) <= 1e-12 * abs(out.item())
    assert _rel(r.dX[:half], Xt.grad.numpy()) <= 1e-10
    assert np.all(r.dX[half:] == 0.0)
    assert _rel(r.dW, Wt.grad.numpy()) <= 1e-10


def pin_identical_pairs(fx):
    B, T = 2, 6
    X, W, y = _batch(B, T, 5, 9, 2)
    half = B * T
    X[half:] = X[:half]
    y[half:] = y[:half]
    r = fx(X, W, y, B, II, beta=0.7)
    assert np.all(np.abs(r.log_odds_ratio) <= 1e-12)
    assert abs(r.or_loss - np.log(2.0)) <= 1e-12
    assert abs(r.loss - (r.nll + 0.7 * np.log(2.0))) <= 1e-12
    r0 = fx(X, W, y, B, II, beta=0.0)
    assert _rel(r.dW, r0.dW) <= 1e-10


def pin_two_classes_one_token(fx):
    """V = 2, T = 1: log odds of a sequence = z_y - z_other."""
    rng = np.random.default_rng(3)
    B, H = 4, 3
    X = rng.standard_normal((2 * B, H))
    W = rng.standard_normal((2, H))
    y = rng.integers(0, 2, size=2 * B)
    beta = 0.3
    z = np.array([[sum(X[i, k] * W[v, k] for k in range(H)) for v in range(2)]
                  for i in range(2 * B)])
    margin = z[np.arange(2 * B), y] - z[np.arange(2 * B), 1 - y]
    d = margin[:B] - margin[B:]
    or_loss = float(np.mean(np.log1p(np.exp(-d))))
    nll = float(np.mean(np.log1p(np.exp(-margin[:B]))))         # -log sigmoid(margin)
    r = fx(X, W, y, B, II, beta=beta)
    assert np.max(np.abs(r.log_odds_ratio - d)) <= 1e-10
    assert abs(r.or_loss - or_loss) <= 1e-12 * abs(or_loss)
    assert abs(r.loss - (nll + beta * or_loss)) <= 1e-12 * abs(r.loss)


def pin_torch_autograd(fx):
    B, T = 3, 7
    X, W, y = _batch(B, T, 5, 13, 4, prompt=2)
    loss, dX, dW = _torch_orpo(X, W, y, B, 0.25)
    r = fx(X, W, y, B, II, beta=0.25)
    assert abs(r.loss - loss) <= 1e-12 * abs(loss)
    assert _rel(r.dX, dX) <= 1e-10 and _rel(r.dW, dW) <= 1e-10


def pin_finite_differences(fx):
    B, T = 2, 3
    X, W, y = _batch(B, T, 3, 4, 5, prompt=1, pad=0)
    beta = 0.8
    r = fx(X, W, y, B, II, beta=beta)
    h = 1e-5

    def L(X_, W_):
        return fx(X_, W_, y, B, II, beta=beta, grads=False).loss

    for A, grad in ((X, r.dX), (W, r.dW)):
        for idx in np.ndindex(A.shape):
            Ap, Am = A.copy(), A.copy()
            Ap[idx] += h
            Am[idx] -= h
            fd = (L(Ap, W) - L(Am, W)) / (2 * h) if A is X else (L(X, Ap) - L(X, Am)) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-7 * max(1.0, abs(fd)), (idx, fd, grad[idx])


def pin_empty_pair(fx):
    B, T = 3, 5
    X, W, y = _batch(B, T, 4, 7, 6)
    y2 = y.reshape(2 * B, T).copy()
    y2[B + 1] = II                                   # rejected sequence of pair 1: empty
    r = fx(X, W, y2.reshape(-1), B, II, beta=0.5)
    assert r.log_odds_ratio[1] == 0.0
    keep = [0, 2]
    rows = np.concatenate([np.arange(s * T, (s + 1) * T) for s in keep + [B + k for k in keep]])
    r2 = fx(X[rows], W, y2.reshape(-1)[rows], 2, II, beta=0.5)
    # same pairs, same terms; L_OR's mean divides by the batch's pair count
    assert abs(r.or_loss * B - r2.or_loss * 2) <= 1e-12
    assert np.all(r.dX[(B + 1) * T:(B + 2) * T] == 0.0)


PINS = [pin_beta0_is_chosen_ce, pin_identical_pairs, pin_two_classes_one_token,
        pin_torch_autograd, pin_finite_differences, pin_empty_pair]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin_orpo(pin):
    pin(oracle.orpo)


def test_rows_form_matches_whole():
    B, T = 3, 6
    X, W, y = _batch(B, T, 5, 17, 8, prompt=2)
    r = oracle.orpo(X, W, y, B, II, beta=0.4)
    rows, vrows = np.array([0, 5, 17, 30]), np.array([1, 8, 16])
    q = oracle.orpo_rows(X, W, y, B, rows, vrows, II, beta=0.4, block=7)
    assert abs(q.loss - r.loss) <= 1e-13 * abs(r.loss) and abs(q.nll - r.nll) <= 1e-13 * r.nll
    assert _rel(q.log_odds_ratio, r.log_odds_ratio) <= 1e-12
    assert _rel(q.dX, r.dX[rows]) <= 1e-12 and _rel(q.dW, r.dW[vrows]) <= 1e-12


def test_layout_checked():
    X, W, y = _batch(2, 4, 3, 5, 7)
    with pytest.raises(ValueError):
        oracle.orpo(X[:-1], W, y[:-1], 2)


# ------------------------------------------------------------------ planted mistakes

def _m_sum_not_mean(lp, valid, n_seq):
    lp = lp.reshape(n_seq, -1)
    valid = valid.reshape(n_seq, -1)
    return np.where(valid, lp, 0.0).sum(axis=1), valid.sum(axis=1)


def _m_log_prob_not_odds(a):
    return a


def _m_or_sign(d, live):
    return np.where(live, np.logaddexp(0.0, d), 0.0)


def _m_weights_no_length(a_c, n_c, a_r, n_r, d, live, valid, n_pairs, n_chosen_valid, beta):
    return om_orig_weights(a_c, np.ones_like(n_c), a_r, np.ones_like(n_r), d, live, valid,
                           n_pairs, n_chosen_valid, beta)


def _m_weights_rejected_sign(a_c, n_c, a_r, n_r, d, live, valid, n_pairs, n_chosen_valid, beta):
    w = om_orig_weights(a_c, n_c, a_r, n_r, d, live, valid, n_pairs, n_chosen_valid, beta)
    half = w.size // 2
    w[half:] = -w[half:]
    return w


def _m_weights_no_nll(a_c, n_c, a_r, n_r, d, live, valid, n_pairs, n_chosen_valid, beta):
    return om_orig_weights(a_c, n_c, a_r, n_r, d, live, valid, n_pairs, 10 ** 12, beta)


om_orig_weights = om.orpo_token_weights

MISTAKES = [("sequence_logp", _m_sum_not_mean), ("log_odds", _m_log_prob_not_odds),
            ("odds_ratio_loss", _m_or_sign), ("orpo_token_weights", _m_weights_no_length),
            ("orpo_token_weights", _m_weights_rejected_sign),
            ("orpo_token_weights", _m_weights_no_nll)]


@pytest.mark.parametrize("step,mistake", MISTAKES, ids=[m.__name__ for _, m in MISTAKES])
def test_planted_mistakes_orpo(monkeypatch, step, mistake):
    monkeypatch.setattr(om, step, mistake)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(oracle.orpo)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {mistake.__name__}"
