"""GPU parity of libflce against the fp64 oracle at sizes the oracle finishes in
seconds: every output element compared, tile multiples and ragged tails,
several chunks, and the special cases of the loss."""
import math

import numpy as np
import pytest
import torch

import datagen
import linear_cross_entropy_04_amd as fl
import oracle
from _gpu_common import DEV, check_grad, check_loss, run_gpu, say, to_device

pytestmark = pytest.mark.gpu
II = -100


def _full_check(inp, chunk, ignore_index=II):
    kind = inp.wl.dtype
    say(f"case {inp.wl.name} N={inp.wl.N} H={inp.wl.H} V={inp.wl.V} {kind} seed={inp.seed} chunk={chunk}")
    g = run_gpu(inp, chunk, ignore_index)
    r = oracle.flce(inp.X_f64(), inp.W_f64(), inp.labels, ignore_index)
    check_loss(g["loss"], r.loss, kind)
    check_grad(g["dX"], r.dX, kind, "dX")
    check_grad(g["dW"], r.dW, kind, "dW")
    valid = inp.labels != ignore_index
    lse_tol = 1e-3 if kind == "bf16" else 1e-5
    assert np.max(np.abs(g["row_lse"] - r.lse) / np.abs(r.lse)) <= lse_tol
    assert np.all(g["row_loss"][~valid] == 0.0)
    assert np.max(np.abs(g["row_loss"] - r.row_loss)) <= lse_tol * np.max(np.abs(r.lse))
    assert np.all(g["dX"][~valid] == 0.0), "ignored rows must have exactly zero dX"
    return g, r


def test_tiny_fp32_workload():
    """The tiny all-fp32 workload: N=512, H=128, V=256, chunks of 128."""
    inp = datagen.make(0)
    _full_check(inp, 128)


def test_pages_api_example_shape():
    """nn.Linear(128, 256).weight, randn(4, 128) input, randint(256, (4,)) targets."""
    inp = datagen.make_custom(4, 128, 256, "bf16", seed=7, ignore_mode="none", w_std=0.05)
    _full_check(inp, 0)


@pytest.mark.parametrize("N,H,V,chunk", [
    (1000, 200, 1001, 384),     # no dimension a tile multiple; ragged last chunk
    (600, 512, 3000, 256),      # 12 vocabulary tiles, 3 chunks (last of 88 rows)
    (513, 256, 257, 512),       # one token past a tile; one vocab id past a tile
    (64, 64, 40000, 64),        # many vocabulary tiles, one small chunk
    (300, 1024, 700, 1000),     # one chunk (chunk > N), deep K
    (1500, 320, 1100, 512),     # dW old values added in the main loop (16 slices), V and H tails
    (2100, 512, 600, 1024),     # the same at 32 slices, V tail; last chunk of 52 rows
    (2100, 4096, 4452, 1024),   # 272 dW tiles inside V: resident workgroups chain tiles; V tail
    (1000, 256, 70000, 1000),   # 1092 forward tiles (more than one wave of 256 CUs); V and token tails
])
def test_bf16_ragged(N, H, V, chunk):
    inp = datagen.make_custom(N, H, V, "bf16", seed=N + V, ignore_frac=0.1)
    _full_check(inp, chunk)


def _random_shapes(count, seed):
    """Seeded shapes off every tile grid: N, V and the chunk anywhere in
    their ranges (chunk 0 lets the planner choose), H a multiple of 8 (the
    bf16 path's requirement)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        N = int(rng.integers(1, 1600))
        H = 8 * int(rng.integers(1, 97))
        V = int(rng.integers(1, 6000))
        chunk = int(rng.choice([0, int(rng.integers(1, N + 1)), int(rng.integers(1, 1100))]))
        out.append((N, H, V, chunk))
    return out


@pytest.mark.parametrize("N,H,V,chunk", _random_shapes(12, 20261203))
def test_bf16_random_shapes(N, H, V, chunk):
    inp = datagen.make_custom(N, H, V, "bf16", seed=N * 7 + V, ignore_frac=0.1)
    _full_check(inp, chunk)


@pytest.mark.parametrize("N,H,V,chunk", [(77, 33, 130, 32), (200, 64, 1000, 0)])
def test_fp32_ragged(N, H, V, chunk):
    inp = datagen.make_custom(N, H, V, "f32", seed=N, ignore_frac=0.1)
    _full_check(inp, chunk)


def test_bf16_rmsnorm_zipf_prefix():
    """The Qwen2-7B and long-context recipes at a small size."""
    inp = datagen.make_custom(700, 256, 5000, "bf16", seed=3, x_dist="rmsnorm",
                              label_dist="zipf", ignore_mode="prefix", ignore_frac=0.25)
    _full_check(inp, 256)


def test_label_extremes_and_ignore_in_range():
    inp = datagen.make_custom(300, 128, 777, "bf16", seed=11, ignore_frac=0.0)
    inp.labels[:100] = 0
    inp.labels[100:200] = 776
    _full_check(inp, 128)
    inp.labels[250:] = 5
    _full_check(inp, 128, ignore_index=5)


def test_all_ignored():
    inp = datagen.make_custom(100, 64, 500, "bf16", seed=2, ignore_frac=1.0)
    assert np.all(inp.labels == II)
    g = run_gpu(inp, 64)
    assert g["loss"] == 0.0
    assert np.all(g["dX"] == 0.0) and np.all(g["dW"] == 0.0)


def test_empty_input():
    inp = datagen.make_custom(0, 64, 500, "bf16", seed=2)
    g = run_gpu(inp, 0)
    assert g["loss"] == 0.0 and g["dX"].shape == (0, 64)
    assert np.all(g["dW"] == 0.0)


@pytest.mark.parametrize("ignored", [False, True])
def test_non_finite_input_propagates(ignored):
    """A NaN in one row of X is not checked and propagates as the oracle's
    plain definition does: a scored row makes the loss, its dX row and all of
    dW NaN; an ignored row leaves the loss and every dX row finite (its G row
    is exactly 0) and turns only dW's column of the NaN NaN (0 times NaN)."""
    import copy
    inp = copy.copy(datagen.make_custom(300, 64, 1000, "bf16", seed=5, ignore_frac=0.1))
    X = inp.X.copy()
    X[17, 5] = 0x7FC0                                  # bf16 quiet NaN
    inp.X = X
    labels = inp.labels.copy()
    labels[17] = II if ignored else 458
    say(f"case non-finite N=300 H=64 V=1000 bf16 seed=5 chunk=128 row 17 ignored={ignored}")
    g = run_gpu(inp, 128, labels=labels)
    r = oracle.flce(inp.X_f64(), inp.W_f64(), labels)
    finite_rows = np.ones(300, dtype=bool)
    if ignored:
        check_loss(g["loss"], r.loss, "bf16")
        assert np.all(g["dX"][17] == 0.0)
    else:
        assert math.isnan(g["loss"]) and math.isnan(r.loss)
        assert np.all(np.isnan(g["dX"][17]))
        finite_rows[17] = False
    assert np.all(np.isfinite(g["dX"][finite_rows]))
    check_grad(g["dX"][finite_rows], r.dX[finite_rows], "bf16", "dX (finite rows)")
    nan_cols = np.zeros(64, dtype=bool)
    nan_cols[5] = True
    if not ignored:
        nan_cols[:] = True
    assert np.array_equal(np.isnan(g["dW"]).all(axis=0), nan_cols)
    assert np.array_equal(np.isnan(r.dW).all(axis=0), nan_cols)
    if ignored:
        check_grad(g["dW"][:, ~nan_cols], r.dW[:, ~nan_cols], "bf16", "dW (finite columns)")


def test_invalid_label_reports_elabel():
    inp = datagen.make_custom(50, 64, 100, "bf16", seed=4)
    labels = inp.labels.copy()
    labels[7] = 100
    with pytest.raises(fl.FLCEError) as e:
        run_gpu(inp, 0, labels=labels)
    assert e.value.status == fl.FLCE_ELABEL
    labels[7] = -3
    with pytest.raises(fl.FLCEError) as e:
        run_gpu(inp, 0, labels=labels)
    assert e.value.status == fl.FLCE_ELABEL


def test_w_zero_closed_form():
    """W = 0: loss = ln V exactly, dX = 0 exactly, dW from its closed form."""
    inp = datagen.make_custom(400, 128, 3000, "bf16", seed=5, ignore_frac=0.1)
    inp.W[:] = 0
    g = run_gpu(inp, 128)
    assert abs(g["loss"] - math.log(3000)) <= 1e-6 * math.log(3000)
    assert np.all(g["dX"] == 0.0)
    X = inp.X_f64()
    valid = inp.labels != II
    nv = valid.sum()
    ref = np.tile(X[valid].sum(0) / 3000, (3000, 1))
    np.add.at(ref, inp.labels[valid], -X[valid])
    check_grad(g["dW"], ref / nv, "bf16", "dW (W=0)")


def test_x_zero_closed_form():
    """X = 0: loss = ln V, dW = 0 exactly, dX_i = (mean_v w_v - w_{y_i}) / N_valid."""
    inp = datagen.make_custom(300, 256, 1500, "bf16", seed=6, ignore_frac=0.1)
    inp.X[:] = 0
    g = run_gpu(inp, 256)
    assert abs(g["loss"] - math.log(1500)) <= 1e-6 * math.log(1500)
    assert np.all(g["dW"] == 0.0)
    W = inp.W_f64()
    valid = inp.labels != II
    ref = np.zeros((300, 256))
    ref[valid] = (W.mean(0)[None, :] - W[inp.labels[valid]]) / valid.sum()
    check_grad(g["dX"], ref, "bf16", "dX (X=0)")


def test_chunk_invariance_and_determinism():
    inp = datagen.make_custom(1100, 256, 2000, "bf16", seed=9, ignore_frac=0.05)
    r = oracle.flce(inp.X_f64(), inp.W_f64(), inp.labels)
    runs = {}
    for c in (128, 256, 1000, 2048):
        runs[c] = run_gpu(inp, c)
        check_loss(runs[c]["loss"], r.loss, "bf16")
        check_grad(runs[c]["dX"], r.dX, "bf16", f"dX chunk={c}")
        check_grad(runs[c]["dW"], r.dW, "bf16", f"dW chunk={c}")
    again = run_gpu(inp, 256)
    assert again["loss"] == runs[256]["loss"]
    assert torch.equal(again["dX_t"], runs[256]["dX_t"])
    assert torch.equal(again["dW_t"], runs[256]["dW_t"])


def test_fwd_only_matches():
    inp = datagen.make_custom(500, 128, 900, "bf16", seed=12)
    full = run_gpu(inp, 256)
    fwd = run_gpu(inp, 256, bwd=False)
    assert fwd["loss"] == full["loss"]
    assert np.array_equal(fwd["row_lse"], full["row_lse"])


def test_autograd_binding():
    inp = datagen.make_custom(256, 128, 1000, "bf16", seed=13)
    X, W, y = to_device(inp)
    r = oracle.flce(inp.X_f64(), inp.W_f64(), inp.labels)
    Xg = X.clone().requires_grad_(True)
    Wg = W.clone().requires_grad_(True)
    out = fl.loss(Wg, Xg, y)
    (3.0 * out).backward()
    check_loss(out.item(), r.loss, "bf16")
    check_grad(Xg.grad.double().cpu().numpy(), 3.0 * r.dX, "bf16", "autograd dX")
    check_grad(Wg.grad.double().cpu().numpy(), 3.0 * r.dW, "bf16", "autograd dW")
    mod = fl.FusedLinearCrossEntropyLoss()
    with torch.no_grad():
        assert abs(mod(W, X, y).item() - r.loss) <= 1e-3 * r.loss


def test_autograd_second_backward_refused():
    """The backward scales the gradients saved with the loss in place, so a
    second backward through a retained graph must fail loudly rather than
    return gradients scaled twice; a fresh loss differentiates again."""
    inp = datagen.make_custom(256, 128, 1000, "bf16", seed=14)
    X, W, y = to_device(inp)
    r = oracle.flce(inp.X_f64(), inp.W_f64(), inp.labels)
    Xg = X.clone().requires_grad_(True)
    Wg = W.clone().requires_grad_(True)
    out = fl.loss(Wg, Xg, y)
    (2.0 * out).backward(retain_graph=True)
    check_grad(Xg.grad.double().cpu().numpy(), 2.0 * r.dX, "bf16", "first backward dX")
    with pytest.raises(RuntimeError, match="already used"):
        out.backward()
    Xg.grad = None
    Wg.grad = None
    fl.loss(Wg, Xg, y).backward()
    check_grad(Xg.grad.double().cpu().numpy(), r.dX, "bf16", "fresh loss dX")
    check_grad(Wg.grad.double().cpu().numpy(), r.dW, "bf16", "fresh loss dW")
