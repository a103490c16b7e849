"""Pins of the oracle's unpaired preference loss (oracle.kto) against things
other than the oracle:

* references chosen so that every reward equals the reference point (r =
  z0) give sigmoid(0) = 1/2, so the loss is the mean of lambda / 2 (closed
  form), with the rewards computed independently by torch's log_softmax;
* with V = 2 and one scored token per sequence, log p(y) = -softplus(-m) for
  the logit margin m, so every reward and loss term is a closed form;
* a desirable sequence with reward r and an undesirable one with reward
  2 z0 - r contribute the same loss (lambda_d = lambda_u);
* the loss built from torch float64 primitives with autograd pins the
  hand-derived per-token weights, with z0 taking no gradient;
* central finite differences of the oracle's own forward.

``test_planted_mistakes_kto`` plants a mistake in one step at a time and
checks that some pin fails.
"""
import numpy as np
import pytest

import oracle
from oracle import flce_ref as om

II = -100


def _batch(S, T, H, V, seed, ws=0.5, prompt=1):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((S * T, H))
    W = rng.standard_normal((V, H)) * ws
    y = rng.integers(0, V, size=(S, T))
    y[:, :prompt] = II
    des = rng.random(S) < 0.5
    des[0], des[-1] = True, False
    ref = rng.standard_normal(S) * 2.0 - 3.0 * T
    return X, W, y.reshape(-1), des, ref


def _rel(a, b):
    a, b = np.asarray(a, float), np.asarray(b, float)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _torch_logp_sums(X, W, y, S):
    import torch
    lp_all = torch.log_softmax(torch.tensor(X) @ torch.tensor(W).T, dim=1).numpy()
    valid = y != II
    lp = np.where(valid, lp_all[np.arange(y.size), np.where(valid, y, 0)], 0.0)
    return lp.reshape(S, -1).sum(axis=1)


def _torch_kto(X, W, y, S, des, ref, beta, z0, ld, lu):
    import torch
    Xt = torch.tensor(X, dtype=torch.float64, requires_grad=True)
    Wt = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    yt = torch.tensor(y)
    lp_all = torch.log_softmax(Xt @ Wt.T, dim=1)
    valid = yt != II
    lp = torch.where(valid, lp_all.gather(1, yt.clamp(min=0)[:, None])[:, 0], torch.zeros(()))
    r = lp.view(S, -1).sum(1) - torch.tensor(ref)
    d = torch.tensor(des)
    z = torch.tensor(z0, dtype=torch.float64)          # a constant: no gradient
    l = torch.where(d, ld * (1 - torch.sigmoid(beta * (r - z))),
                    lu * (1 - torch.sigmoid(beta * (z - r))))
    loss = l.mean()
    loss.backward()
    return loss.item(), Xt.grad.numpy(), Wt.grad.numpy()


# ------------------------------------------------------------------ pins

def pin_rewards_at_reference_point(fx):
    S, T = 5, 4
    X, W, y, des, _ = _batch(S, T, 5, 9, 1)
    z0 = 0.37
    ref = _torch_logp_sums(X, W, y, S) - z0                  # r = z0 for every sequence
    r = fx(X, W, y, S, des, ref, II, beta=0.8, z0=z0, lambda_d=1.3, lambda_u=0.6)
    assert np.max(np.abs(r.reward - z0)) <= 1e-12
    want = float(np.mean(np.where(des, 1.3, 0.6)) / 2)
    assert abs(r.loss - want) <= 1e-12


def pin_two_classes_one_token(fx):
    rng = np.random.default_rng(2)
    S, H = 6, 3
    X = rng.standard_normal((S, H))
    W = rng.standard_normal((2, H))
    y = rng.integers(0, 2, size=S)
    des = np.array([True, False, True, True, False, False])
    ref = rng.standard_normal(S) - 1.0
    z = np.array([[sum(X[i, k] * W[v, k] for k in range(H)) for v in range(2)]
                  for i in range(S)])
    m = z[np.arange(S), y] - z[np.arange(S), 1 - y]
    rew = -np.log1p(np.exp(-m)) - ref
    beta, z0 = 0.9, 0.2
    u = np.where(des, beta * (rew - z0), beta * (z0 - rew))
    want = float(np.mean(1.0 - 1.0 / (1.0 + np.exp(-u))))
    r = fx(X, W, y, S, des, ref, II, beta=beta, z0=z0)
    assert np.max(np.abs(r.reward - rew)) <= 1e-12
    assert abs(r.loss - want) <= 1e-12 * want


def pin_mirror_symmetry(fx):
    S, T = 2, 5
    X, W, y, _, _ = _batch(S, T, 4, 7, 3)
    half = T
    X[half:] = X[:half]
    y[half:] = y[:half]
    s0 = _torch_logp_sums(X, W, y, S)[0]
    z0, r0 = 0.5, -1.7
    ref = np.array([s0 - r0, s0 - (2 * z0 - r0)])        # rewards r0 and 2 z0 - r0
    r = fx(X, W, y, S, np.array([True, False]), ref, II, beta=0.6, z0=z0)
    one = fx(X[:half], W, y[:half], 1, np.array([True]), ref[:1], II, beta=0.6, z0=z0)
    assert abs(r.loss - one.loss) <= 1e-12 * one.loss


def pin_torch_autograd(fx):
    S, T = 5, 6
    X, W, y, des, ref = _batch(S, T, 5, 13, 4, prompt=2)
    ref = _torch_logp_sums(X, W, y, S) + np.linspace(-3, 3, S)
    loss, dX, dW = _torch_kto(X, W, y, S, des, ref, 0.7, 0.3, 1.0, 1.5)
    r = fx(X, W, y, S, des, ref, II, beta=0.7, z0=0.3, lambda_d=1.0, lambda_u=1.5)
    assert abs(r.loss - loss) <= 1e-12 * abs(loss)
    assert _rel(r.dX, dX) <= 1e-10 and _rel(r.dW, dW) <= 1e-10


def pin_finite_differences(fx):
    S, T = 3, 3
    X, W, y, des, _ = _batch(S, T, 3, 4, 5)
    ref = _torch_logp_sums(X, W, y, S) + np.array([0.5, -0.4, 1.1])
    r = fx(X, W, y, S, des, ref, II, beta=1.2, z0=0.1)
    h = 1e-5

    def L(X_, W_):
        return fx(X_, W_, y, S, des, ref, II, beta=1.2, z0=0.1, grads=False).loss

    for A, grad in ((X, r.dX), (W, r.dW)):
        for idx in np.ndindex(A.shape):
            Ap, Am = A.copy(), A.copy()
            Ap[idx] += h
            Am[idx] -= h
            fd = (L(Ap, W) - L(Am, W)) / (2 * h) if A is X else (L(X, Ap) - L(X, Am)) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-7 * max(1.0, abs(fd)), (idx, fd, grad[idx])


PINS = [pin_rewards_at_reference_point, pin_two_classes_one_token, pin_mirror_symmetry,
        pin_torch_autograd, pin_finite_differences]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin_kto(pin):
    pin(oracle.kto)


# ------------------------------------------------------------------ planted mistakes

_orig_terms = om.kto_sequence_terms
_orig_weights = om.kto_token_weights


def _m_same_sign(r, desirable, beta, z0, lambda_d, lambda_u):
    return _orig_terms(r, np.ones_like(desirable), beta, z0, lambda_d, lambda_u)


def _m_swapped_lambdas(r, desirable, beta, z0, lambda_d, lambda_u):
    return _orig_terms(r, desirable, beta, z0, lambda_u, lambda_d)


def _m_z0_ignored(r, desirable, beta, z0, lambda_d, lambda_u):
    return _orig_terms(r, desirable, beta, 0.0, lambda_d, lambda_u)


def _m_weights_not_mean(dl_dr, valid, n_seq):
    return _orig_weights(dl_dr * n_seq, valid, n_seq)          # the sum, not the mean


MISTAKES = [("kto_sequence_terms", _m_same_sign), ("kto_sequence_terms", _m_swapped_lambdas),
            ("kto_sequence_terms", _m_z0_ignored), ("kto_token_weights", _m_weights_not_mean)]


@pytest.mark.parametrize("step,mistake", MISTAKES, ids=[m.__name__ for _, m in MISTAKES])
def test_planted_mistakes_kto(monkeypatch, step, mistake):
    monkeypatch.setattr(om, step, mistake)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(oracle.kto)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {mistake.__name__}"


# ------------------------------------------------------------------ reference point from a batch

def test_kto_reference_point_closed_form():
    """W = 0: every scored token has log p = -ln V, so S = -n ln V for a
    sequence of n scored tokens and z0 = max(0, mean(S - R)) is a closed form;
    a reference below the policy gives its mean gap, one above it gives 0."""
    S, T, H, V = 4, 6, 5, 9
    X, W, y, _, _ = _batch(S, T, H, V, seed=31, prompt=2)
    W = np.zeros_like(W)
    n = (y.reshape(S, T) != II).sum(axis=1)
    gap = np.array([1.0, 3.0, -0.5, 0.5])
    R = -n * np.log(V) - gap
    assert abs(oracle.kto_reference_point(X, W, y, S, R) - gap.mean()) <= 1e-12
    assert oracle.kto_reference_point(X, W, y, S, -n * np.log(V) + gap) == 0.0


def test_kto_reference_point_against_torch():
    """Random head: the mean policy-minus-reference gap with torch's
    log_softmax for the policy sums, clamped at 0; invariant to the order of
    the sequences."""
    S, T, H, V = 5, 7, 6, 11
    X, W, y, _, _ = _batch(S, T, H, V, seed=32)
    Sp = _torch_logp_sums(X, W, y, S)
    R = Sp - np.array([0.3, -0.1, 0.8, 0.2, 0.05])
    z = oracle.kto_reference_point(X, W, y, S, R)
    assert abs(z - 0.25) <= 1e-12
    perm = np.array([3, 0, 4, 1, 2])
    Xp = X.reshape(S, T, H)[perm].reshape(-1, H)
    yp = y.reshape(S, T)[perm].reshape(-1)
    assert abs(oracle.kto_reference_point(Xp, W, yp, S, R[perm]) - z) <= 1e-12
