"""Pins of the oracle's pairwise preference losses (oracle.preference: SimPO,
CPO, DPO; ORPO is pinned in test_oracle_orpo.py) against things other than
the oracle:

* identical chosen and rejected sequences give z = 0 (SimPO with gamma = 0,
  CPO, DPO with equal references), so the pair term is log 2; SimPO's margin
  alone then gives softplus(gamma) (closed forms);
* with V = 2 and one scored token per sequence, log p(y) = -softplus(-m) for
  the logit margin m, so every z is a closed form in the logits;
* DPO whose reference log-probabilities are the policy's own (computed with
  torch's log_softmax) has z = 0;
* CPO with beta = 0 is its NLL term alone: torch's cross_entropy of the
  chosen half with autograd;
* the losses built from torch float64 primitives with autograd pin the
  hand-derived per-token weights;
* central finite differences of the oracle's own forward;
* the "orpo" kind equals the separately pinned ORPO oracle.

``test_planted_mistakes_preference`` plants a mistake in one step at a time
and checks that some pin fails.
"""
import numpy as np
import pytest

import oracle
from oracle import flce_ref as om

II = -100
KINDS = ("simpo", "cpo", "dpo")
PARAMS = {"simpo": dict(beta=2.0, gamma=0.7, alpha=0.3), "cpo": dict(beta=0.4, alpha=1.0),
          "dpo": dict(beta=0.5, alpha=0.0)}


def _batch(B, T, H, V, seed, ws=0.5, prompt=1):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((2 * B * T, H))
    W = rng.standard_normal((V, H)) * ws
    y = rng.integers(0, V, size=(2 * B, T))
    y[:, :prompt] = II
    ref = rng.standard_normal((2, B)) * 3.0 - 10.0
    return X, W, y.reshape(-1), ref


def _rel(a, b):
    a, b = np.asarray(a, float), np.asarray(b, float)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _run(fx, kind, X, W, y, B, ref=None, grads=True, **kw):
    p = dict(PARAMS[kind])
    p.update(kw)
    rc, rr = (ref[0], ref[1]) if ref is not None else (None, None)
    if kind == "dpo" and ref is None:
        rc, rr = np.zeros(B), np.zeros(B)
    return fx(kind, X, W, y, B, II, ref_chosen=rc, ref_rejected=rr, grads=grads, **p)


def _torch_loss(kind, X, W, y, B, ref, beta, gamma=0.0, alpha=0.0):
    import torch
    Xt = torch.tensor(X, dtype=torch.float64, requires_grad=True)
    Wt = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    yt = torch.tensor(y)
    lp_all = torch.log_softmax(Xt @ Wt.T, dim=1)
    valid = yt != II
    lp = torch.where(valid, lp_all.gather(1, yt.clamp(min=0)[:, None])[:, 0], torch.zeros(()))
    lp = lp.view(2 * B, -1)
    v = valid.view(2 * B, -1).double()
    S = (lp * v).sum(1)
    n = v.sum(1)
    if kind == "simpo":
        z = beta * (S[:B] / n[:B] - S[B:] / n[B:]) - gamma
    elif kind == "cpo":
        z = beta * (S[:B] - S[B:])
    else:
        R = torch.tensor(ref, dtype=torch.float64)
        z = beta * ((S[:B] - R[0]) - (S[B:] - R[1]))
    nll = -(lp[:B] * v[:B]).sum() / v[:B].sum()
    loss = alpha * nll - torch.nn.functional.logsigmoid(z).mean()
    loss.backward()
    return loss.item(), Xt.grad.numpy(), Wt.grad.numpy(), lp.detach().numpy(), v.numpy()


# ------------------------------------------------------------------ pins

def pin_identical_pairs(fx):
    B, T = 2, 6
    X, W, y, ref = _batch(B, T, 5, 9, 1)
    half = B * T
    X[half:] = X[:half]
    y[half:] = y[:half]
    for kind in KINDS:
        same = np.stack([ref[0], ref[0]])
        r = _run(fx, kind, X, W, y, B, same, gamma=0.0) if kind == "simpo" else \
            _run(fx, kind, X, W, y, B, same)
        assert np.all(np.abs(r.pair_logit) <= 1e-12), kind
        assert abs(r.pair_loss - np.log(2.0)) <= 1e-12, kind
    r = _run(fx, "simpo", X, W, y, B, gamma=0.9)
    assert abs(r.pair_loss - np.log1p(np.exp(0.9))) <= 1e-12


def pin_two_classes_one_token(fx):
    rng = np.random.default_rng(2)
    B, H = 4, 3
    X = rng.standard_normal((2 * B, H))
    W = rng.standard_normal((2, H))
    y = rng.integers(0, 2, size=2 * B)
    ref = rng.standard_normal((2, B)) - 2.0
    z = np.array([[sum(X[i, k] * W[v, k] for k in range(H)) for v in range(2)]
                  for i in range(2 * B)])
    m = z[np.arange(2 * B), y] - z[np.arange(2 * B), 1 - y]
    lp = -np.log1p(np.exp(-m))                       # log sigmoid(m)
    want = {"simpo": 2.0 * (lp[:B] - lp[B:]) - 0.7, "cpo": 0.4 * (lp[:B] - lp[B:]),
            "dpo": 0.5 * ((lp[:B] - ref[0]) - (lp[B:] - ref[1]))}
    for kind in KINDS:
        r = _run(fx, kind, X, W, y, B, ref)
        assert np.max(np.abs(r.pair_logit - want[kind])) <= 1e-10, kind
        pl = float(np.mean(np.log1p(np.exp(-want[kind]))))
        assert abs(r.pair_loss - pl) <= 1e-12 * pl, kind


def pin_dpo_reference_is_policy(fx):
    import torch
    B, T = 3, 5
    X, W, y, _ = _batch(B, T, 4, 11, 3)
    lp_all = torch.log_softmax(torch.tensor(X) @ torch.tensor(W).T, dim=1).numpy()
    valid = y != II
    lp = np.where(valid, lp_all[np.arange(y.size), np.where(valid, y, 0)], 0.0)
    S = lp.reshape(2 * B, T).sum(axis=1)
    r = _run(fx, "dpo", X, W, y, B, np.stack([S[:B], S[B:]]))
    assert np.max(np.abs(r.pair_logit)) <= 1e-12
    assert abs(r.loss - np.log(2.0)) <= 1e-12


def pin_cpo_beta0_is_chosen_ce(fx):
    import torch
    B, T = 3, 5
    X, W, y, _ = _batch(B, T, 6, 10, 4)
    r = _run(fx, "cpo", X, W, y, B, beta=0.0, alpha=1.0)
    half = B * T
    Xt = torch.tensor(X[:half], dtype=torch.float64, requires_grad=True)
    Wt = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    out = torch.nn.functional.cross_entropy(Xt @ Wt.T, torch.tensor(y[:half]), ignore_index=II)
    out.backward()
    assert abs(r.loss - (out.item() + np.log(2.0))) <= 1e-12 * r.loss
    assert _rel(r.dX[:half], Xt.grad.numpy()) <= 1e-10 and np.all(r.dX[half:] == 0.0)
    assert _rel(r.dW, Wt.grad.numpy()) <= 1e-10


def pin_torch_autograd(fx):
    B, T = 3, 7
    X, W, y, ref = _batch(B, T, 5, 13, 5, prompt=2)
    for kind in KINDS:
        loss, dX, dW, lp, v = _torch_loss(kind, X, W, y, B, ref, **PARAMS[kind])
        r = _run(fx, kind, X, W, y, B, ref)
        assert abs(r.loss - loss) <= 1e-12 * abs(loss), kind
        assert _rel(r.dX, dX) <= 1e-10 and _rel(r.dW, dW) <= 1e-10, kind
        S = (lp * v).sum(1)
        u = S / v.sum(1) if kind == "simpo" else S
        assert _rel(r.chosen_logp, u[:B]) <= 1e-12 and _rel(r.rejected_logp, u[B:]) <= 1e-12


def pin_finite_differences(fx):
    B, T = 2, 3
    X, W, y, ref = _batch(B, T, 3, 4, 6)
    for kind in KINDS:
        r = _run(fx, kind, X, W, y, B, ref)
        h = 1e-5

        def L(X_, W_):
            return _run(fx, kind, X_, W_, y, B, ref, grads=False).loss

        for A, grad in ((X, r.dX), (W, r.dW)):
            for idx in np.ndindex(A.shape):
                Ap, Am = A.copy(), A.copy()
                Ap[idx] += h
                Am[idx] -= h
                fd = (L(Ap, W) - L(Am, W)) / (2 * h) if A is X else \
                    (L(X, Ap) - L(X, Am)) / (2 * h)
                assert abs(fd - grad[idx]) <= 1e-7 * max(1.0, abs(fd)), (kind, idx)


def pin_orpo_kind(fx):
    B, T = 3, 6
    X, W, y, _ = _batch(B, T, 5, 9, 7)
    a = oracle.orpo(X, W, y, B, II, beta=0.3)
    b = fx("orpo", X, W, y, B, II, beta=0.3, alpha=1.0)
    assert abs(a.loss - b.loss) <= 1e-13 * a.loss
    assert _rel(b.dX, a.dX) <= 1e-12 and _rel(b.dW, a.dW) <= 1e-12


PINS = [pin_identical_pairs, pin_two_classes_one_token, pin_dpo_reference_is_policy,
        pin_cpo_beta0_is_chosen_ce, pin_torch_autograd, pin_finite_differences, pin_orpo_kind]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin_preference(pin):
    pin(oracle.preference)


def test_dpo_needs_reference():
    X, W, y, _ = _batch(2, 4, 3, 5, 8)
    with pytest.raises(ValueError):
        oracle.preference("dpo", X, W, y, 2)
    with pytest.raises(ValueError):
        oracle.preference("kto", X, W, y, 2)


# ------------------------------------------------------------------ planted mistakes

_orig_logit = om.pair_logit
_orig_weights = om.preference_token_weights
_orig_sums = om.sequence_sums


def _m_simpo_sums(kind, S_c, n_c, S_r, n_r, beta, gamma, ref_c, ref_r):
    if kind == "simpo":
        return beta * (S_c - S_r) - gamma, np.full(S_c.shape, beta), np.full(S_c.shape, -beta)
    return _orig_logit(kind, S_c, n_c, S_r, n_r, beta, gamma, ref_c, ref_r)


def _m_dpo_ref_sign(kind, S_c, n_c, S_r, n_r, beta, gamma, ref_c, ref_r):
    return _orig_logit(kind, S_c, n_c, S_r, n_r, beta, gamma, -ref_c, -ref_r)


def _m_gamma_sign(kind, S_c, n_c, S_r, n_r, beta, gamma, ref_c, ref_r):
    return _orig_logit(kind, S_c, n_c, S_r, n_r, beta, -gamma, ref_c, ref_r)


def _m_weights_no_rejected(dz_c, dz_r, z, live, valid, n_pairs, n_chosen_valid, alpha, lam):
    return _orig_weights(dz_c, 0.0 * dz_r, z, live, valid, n_pairs, n_chosen_valid, alpha, lam)


def _m_weights_sigmoid_sign(dz_c, dz_r, z, live, valid, n_pairs, n_chosen_valid, alpha, lam):
    return _orig_weights(dz_c, dz_r, -z, live, valid, n_pairs, n_chosen_valid, alpha, lam)


def _m_sums_count_all(lp, valid, n_seq):
    S, n = _orig_sums(lp, valid, n_seq)
    return S, np.full(n.shape, valid.size // n_seq)


MISTAKES = [("pair_logit", _m_simpo_sums), ("pair_logit", _m_dpo_ref_sign),
            ("pair_logit", _m_gamma_sign), ("preference_token_weights", _m_weights_no_rejected),
            ("preference_token_weights", _m_weights_sigmoid_sign),
            ("sequence_sums", _m_sums_count_all)]


@pytest.mark.parametrize("step,mistake", MISTAKES, ids=[m.__name__ for _, m in MISTAKES])
def test_planted_mistakes_preference(monkeypatch, step, mistake):
    monkeypatch.setattr(om, step, mistake)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(oracle.preference)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {mistake.__name__}"
