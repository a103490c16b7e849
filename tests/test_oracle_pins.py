"""Pins of the fp64 oracle against things other than itself.

Each pin checks the oracle against the mathematics of mean cross-entropy over
CE(X W^T, y) (closed forms, invariants, finite differences), a pure-Python
brute force on tiny inputs, or torch's float64 cross_entropy with autograd.
``test_planted_mistakes`` then plants a plausible mistake in one oracle step
at a time and checks that at least one pin fails.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import flce_ref as om

II = -100


def _rand(N, H, V, seed, n_ign=1, xs=1.0, ws=0.3):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((N, H)) * xs
    W = rng.standard_normal((V, H)) * ws
    y = rng.integers(0, V, size=N)
    if n_ign:
        y[rng.permutation(N)[:n_ign]] = II
    return X, W, y


def _rel(a, b):
    a, b = np.asarray(a, float), np.asarray(b, float)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ------------------------------------------------------------------ pins
# Every pin takes the oracle entry point and raises AssertionError on failure.

def pin_w_zero(fl):
    """W = 0: every logit is 0, so loss = ln V, dX = 0 and
    dW_v = ((1/V) sum_valid x_i - sum_{valid, y_i = v} x_i) / N_valid."""
    X, _, y = _rand(9, 4, 6, 1, n_ign=2)
    W = np.zeros((6, 4))
    r = fl(X, W, y, II)
    assert abs(r.loss - math.log(6)) <= 1e-12 * math.log(6)
    assert np.all(r.dX == 0.0)
    valid = y != II
    nv = valid.sum()
    ref = np.empty((6, 4))
    for v in range(6):
        ref[v] = (X[valid].sum(0) / 6 - X[valid & (y == v)].sum(0)) / nv
    assert _rel(r.dW, ref) <= 1e-12


def pin_x_zero(fl):
    """X = 0: loss = ln V, dW = 0 and dX_i = ((1/V) sum_v w_v - w_{y_i}) / N_valid."""
    _, W, y = _rand(7, 3, 5, 2, n_ign=2)
    X = np.zeros((7, 3))
    r = fl(X, W, y, II)
    assert abs(r.loss - math.log(5)) <= 1e-12 * math.log(5)
    assert np.all(r.dW == 0.0)
    valid = y != II
    ref = np.zeros((7, 3))
    for i in np.flatnonzero(valid):
        ref[i] = (W.mean(0) - W[y[i]]) / valid.sum()
    assert _rel(r.dX, ref) <= 1e-12


def pin_row_sums(fl):
    """Each dlogits row sums to 0, hence sum_v dW[v, :] = 0."""
    X, W, y = _rand(30, 8, 40, 3, n_ign=4)
    r = fl(X, W, y, II)
    col = r.dW.sum(axis=0)
    assert np.max(np.abs(col)) <= 1e-12 * max(np.max(np.abs(r.dW)), 1e-300) * 40


def pin_ignored_rows(fl):
    """Ignored rows have exactly zero dX; deleting them leaves loss and dW."""
    X, W, y = _rand(20, 6, 11, 4, n_ign=6)
    r = fl(X, W, y, II)
    ign = y == II
    assert np.all(r.dX[ign] == 0.0)
    r2 = fl(X[~ign], W, y[~ign], II)
    assert abs(r.loss - r2.loss) <= 1e-12 * abs(r2.loss)
    assert _rel(r.dW, r2.dW) <= 1e-12
    assert _rel(r.dX[~ign], r2.dX) <= 1e-12


def pin_finite_differences(fl):
    """Central differences (h = 1e-5) of the loss agree with dX and dW."""
    X, W, y = _rand(6, 5, 7, 5, n_ign=1)
    r = fl(X, W, y, II)
    h = 1e-5
    for A, G in ((X, r.dX), (W, r.dW)):
        num = np.empty_like(A)
        for idx in np.ndindex(*A.shape):
            old = A[idx]
            A[idx] = old + h
            lp = fl(X, W, y, II).loss
            A[idx] = old - h
            lm = fl(X, W, y, II).loss
            A[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        assert _rel(G, num) <= 1e-7, _rel(G, num)


def pin_torch_cross_entropy(fl):
    """torch.nn.functional.cross_entropy(ignore_index=-100), float64 + autograd."""
    torch = pytest.importorskip("torch")
    X, W, y = _rand(512, 128, 256, 6, n_ign=51, ws=0.05)
    r = fl(X, W, y, II)
    Xt = torch.tensor(X, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    loss = torch.nn.functional.cross_entropy(Xt @ Wt.T, torch.tensor(y), ignore_index=II)
    loss.backward()
    assert abs(r.loss - loss.item()) <= 1e-12 * abs(loss.item())
    assert _rel(r.dX, Xt.grad.numpy()) <= 1e-12
    assert _rel(r.dW, Wt.grad.numpy()) <= 1e-12


def pin_shift_invariance(fl):
    """W -> W + 1 c^T shifts row i's logits by <x_i, c>: loss, dX, dW unchanged.
    A large c also checks the max-shifted log-sum-exp (logits near 1000)."""
    X, W, y = _rand(12, 5, 9, 7, n_ign=2)
    X[:, 0] = 1.0                                 # a constant feature
    r = fl(X, W, y, II)
    c = np.zeros(5)
    c[0] = 1000.0                                 # exp(1000) overflows fp64 unshifted
    r2 = fl(X, W + c[None, :], y, II)
    assert np.all(np.isfinite(r2.lse))
    assert abs(r.loss - r2.loss) <= 1e-12 * abs(r.loss) + 1e-10
    assert _rel(r2.dX, r.dX) <= 1e-9
    assert _rel(r2.dW, r.dW) <= 1e-9


def pin_permutations(fl):
    """Permuting the vocabulary (W rows and label ids together) permutes dW rows;
    permuting tokens permutes dX rows; the loss is unchanged by both."""
    X, W, y = _rand(10, 4, 8, 8, n_ign=2)
    r = fl(X, W, y, II)
    rng = np.random.default_rng(80)
    p = rng.permutation(8)                        # new id of old id v is inv[v]
    inv = np.argsort(p)
    y2 = np.where(y == II, II, inv[np.where(y == II, 0, y)])
    r2 = fl(X, W[p], y2, II)
    assert abs(r.loss - r2.loss) <= 1e-12 * abs(r.loss)
    assert _rel(r2.dW, r.dW[p]) <= 1e-12
    assert _rel(r2.dX, r.dX) <= 1e-12
    q = rng.permutation(10)
    r3 = fl(X[q], W, y[q], II)
    assert abs(r.loss - r3.loss) <= 1e-12 * abs(r.loss)
    assert _rel(r3.dX, r.dX[q]) <= 1e-12
    assert _rel(r3.dW, r.dW) <= 1e-12


def pin_two_classes(fl):
    """V = 2: the per-token loss is softplus(z_other - z_y)."""
    X, W, y = _rand(15, 3, 2, 9, n_ign=0)
    r = fl(X, W, y, II)
    Z = X @ W.T
    d = Z[np.arange(15), 1 - y] - Z[np.arange(15), y]
    ref = np.mean(np.logaddexp(0.0, d))
    assert abs(r.loss - ref) <= 1e-12 * abs(ref)


def _bruteforce(X, W, y, ii):
    """Pure-Python loops: loss, dX, dW from the definition, term by term."""
    N, H = len(X), len(X[0])
    V = len(W)
    nv = sum(1 for t in y if t != ii)
    loss = 0.0
    dX = [[0.0] * H for _ in range(N)]
    dW = [[0.0] * H for _ in range(V)]
    for i in range(N):
        if y[i] == ii:
            continue
        z = [sum(X[i][k] * W[v][k] for k in range(H)) for v in range(V)]
        m = max(z)
        s = sum(math.exp(t - m) for t in z)
        lse = m + math.log(s)
        loss += (lse - z[y[i]]) / nv
        for v in range(V):
            g = (math.exp(z[v] - lse) - (1.0 if v == y[i] else 0.0)) / nv
            for k in range(H):
                dX[i][k] += g * W[v][k]
                dW[v][k] += g * X[i][k]
    return loss, np.array(dX), np.array(dW)


def pin_bruteforce(fl):
    """Pure-Python triple loops on a tiny input."""
    X, W, y = _rand(5, 3, 4, 10, n_ign=1)
    r = fl(X, W, y, II)
    loss, dX, dW = _bruteforce(X.tolist(), W.tolist(), y.tolist(), II)
    assert abs(r.loss - loss) <= 1e-12 * abs(loss)
    assert _rel(r.dX, dX) <= 1e-12
    assert _rel(r.dW, dW) <= 1e-12


def pin_all_ignored(fl):
    """No valid token: loss 0 and zero gradients (the reading chosen for 0/0)."""
    X, W, _ = _rand(4, 3, 5, 11)
    y = np.full(4, II)
    r = fl(X, W, y, II)
    assert r.loss == 0.0 and np.all(r.dX == 0.0) and np.all(r.dW == 0.0)


def pin_ignore_index_in_range(fl):
    """ignore_index inside [0, V) ignores that class id: same as deleting the rows."""
    X, W, y = _rand(16, 4, 6, 12, n_ign=0)
    y[:5] = 3
    r = fl(X, W, y, 3)
    keep = y != 3
    r2 = fl(X[keep], W, y[keep], II)
    assert abs(r.loss - r2.loss) <= 1e-12 * abs(r2.loss)
    assert _rel(r.dW, r2.dW) <= 1e-12
    assert np.all(r.dX[~keep] == 0.0)


PINS = [pin_w_zero, pin_x_zero, pin_row_sums, pin_ignored_rows, pin_finite_differences,
        pin_torch_cross_entropy, pin_shift_invariance, pin_permutations, pin_two_classes,
        pin_bruteforce, pin_all_ignored, pin_ignore_index_in_range]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oracle.flce)


def test_invalid_label_raises():
    X, W, y = _rand(4, 3, 5, 13)
    y[2] = 5
    with pytest.raises(ValueError):
        oracle.flce(X, W, y, II)
    y[2] = -1
    with pytest.raises(ValueError):
        oracle.flce(X, W, y, II)


def test_expected_loss_at_init():
    """Statistical sanity of the workload recipe: with W ~ N(0, 0.02^2) and
    X ~ N(0, 1), logits are ~N(0, 0.02^2 H) so E[loss] ~ ln V + 0.02^2 H / 2."""
    import datagen
    inp = datagen.make(0)
    r = oracle.flce(inp.X_f64(), inp.W_f64(), inp.labels, II, grads=False)
    ref = math.log(256) + 0.02 ** 2 * 128 / 2
    assert abs(r.loss - ref) <= 0.01 * ref


# ------------------------------------------------------------------ planted mistakes

def _m_no_onehot(Z, lse, labels, valid, n_valid, col_ids=None):
    G = np.exp(Z - lse[:, None]) / max(n_valid, 1)
    G[~valid] = 0.0
    return G


def _m_norm_by_N(Z, lse, labels, valid, n_valid, col_ids=None):
    return _orig["dlogits"](Z, lse, labels, valid, n_valid, col_ids) * max(n_valid, 1) / Z.shape[0]


def _m_sign(Z, lse, labels, valid, n_valid, col_ids=None):
    return -_orig["dlogits"](Z, lse, labels, valid, n_valid, col_ids)


def _m_ignored_not_zeroed(Z, lse, labels, valid, n_valid, col_ids=None):
    return _orig["dlogits"](Z, lse, labels, np.ones_like(valid), n_valid, col_ids)


def _m_lse_drops_max(Z):
    m = Z.max(axis=1)
    return np.log(np.exp(Z - m[:, None]).sum(axis=1))


def _m_lse_unshifted(Z):
    with np.errstate(over="ignore"):
        return np.log(np.exp(Z).sum(axis=1))


def _m_target_off_by_one(Z, labels, valid):
    return _orig["target_logit"](Z, (labels + 1) % Z.shape[1], valid)


def _m_rowloss_unmasked(lse, zy, valid):
    return lse - zy


def _m_mean_over_N(row_loss, n_valid):
    return float(row_loss.sum() / row_loss.size)


def _m_dx_transposed_index(G, W):
    return np.roll(G, 1, axis=1) @ W


def _m_dw_wrong_rows(G, X):
    return G.T @ X[::-1]


def _m_logits_wrong_rows(X, W):
    return X @ W[::-1].T


def _m_valid_ignores_nothing_in_range(labels, V, ignore_index=II):
    labels = np.asarray(labels, dtype=np.int64)
    return labels >= 0


_orig = {n: getattr(om, n) for n in ("dlogits", "target_logit", "row_logsumexp",
                                     "row_losses", "mean_loss", "grad_input",
                                     "grad_weight", "logits", "valid_mask")}

MISTAKES = [
    ("dlogits", _m_no_onehot), ("dlogits", _m_norm_by_N), ("dlogits", _m_sign),
    ("dlogits", _m_ignored_not_zeroed), ("row_logsumexp", _m_lse_drops_max),
    ("row_logsumexp", _m_lse_unshifted), ("target_logit", _m_target_off_by_one),
    ("row_losses", _m_rowloss_unmasked), ("mean_loss", _m_mean_over_N),
    ("grad_input", _m_dx_transposed_index), ("grad_weight", _m_dw_wrong_rows),
    ("logits", _m_logits_wrong_rows), ("valid_mask", _m_valid_ignores_nothing_in_range),
]


@pytest.mark.parametrize("step,mistake", MISTAKES, ids=[m.__name__ for _, m in MISTAKES])
def test_planted_mistakes(monkeypatch, step, mistake):
    monkeypatch.setattr(om, step, mistake)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(oracle.flce)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {mistake.__name__}"


# ------------------------------------------------------------------ parts agree with the whole

def test_parts_equal_whole():
    X, W, y = _rand(37, 9, 53, 14, n_ign=5)
    r = oracle.flce(X, W, y, II)
    lse, rl, nv = oracle.forward_rows(X, W, y, block=8)
    assert nv == r.n_valid
    assert _rel(lse, r.lse) <= 1e-14 and _rel(rl, r.row_loss) <= 1e-14
    loss, lse2, _, _ = oracle.loss_blocked(X, W, y, block=5)
    assert abs(loss - r.loss) <= 1e-14 * abs(r.loss)
    rows = np.array([0, 3, 17, 36])
    assert _rel(oracle.dX_rows(X, W, y, rows), r.dX[rows]) <= 1e-13
    vrows = np.array([0, 1, 25, 52])
    assert _rel(oracle.dW_rows(X, W, y, lse, vrows), r.dW[vrows]) <= 1e-13
