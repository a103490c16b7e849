"""GPU parity of the pairwise preference losses SimPO, CPO and DPO
(flce_pair_fwd_bwd / flce_pair_fwd) against the fp64 oracle's preference:
every element at small sizes (bf16 and fp32, chunks of one or more pairs),
DPO with reference log-probabilities computed on the GPU from a reference
head (sequence_logps) against the oracle's, the autograd modules, and the
ORPO kind through the general entry point."""
import numpy as np
import pytest
import torch

import datagen
import linear_cross_entropy_04_amd as fl
import oracle
from _gpu_common import DEV, check_grad, check_loss, say, to_device

pytestmark = pytest.mark.gpu
II = -100
PARAMS = {"simpo": dict(beta=2.0, gamma=1.0, alpha=0.5), "cpo": dict(beta=0.1, gamma=0.0, alpha=1.0),
          "dpo": dict(beta=0.1, gamma=0.0, alpha=0.0), "orpo": dict(beta=0.2, gamma=0.0, alpha=1.0)}


def _ref_logps(B, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((2, B)) * 20.0 - 400.0).astype(np.float32)


def _run(kind, inp, B, chunk_pairs, ref=None, bwd=True):
    X, W, y = to_device(inp)
    N, H = X.shape
    V = W.shape[0]
    T = N // (2 * B)
    dt = fl.FLCE_BF16 if X.dtype == torch.bfloat16 else fl.FLCE_F32
    ws = torch.full((fl.flce_pair_workspace_bytes(B, T, H, V, dt, chunk_pairs),), 255,
                    dtype=torch.uint8, device=DEV)
    rc = rr = None
    if ref is not None:
        rc, rr = (torch.from_numpy(np.ascontiguousarray(r)).to(DEV) for r in ref)
    clp, rlp, z = (torch.full((B,), float("nan"), dtype=torch.float32, device=DEV)
                   for _ in range(3))
    p = PARAMS[kind]
    say(f"  gpu pair call: {kind} pairs={B} T={T} H={H} V={V} {'bf16' if dt else 'f32'} "
        f"chunk_pairs={chunk_pairs} {'fwd_bwd' if bwd else 'fwd'}")
    out = {}
    if bwd:
        dX = torch.full_like(X, float("nan"))
        dW = torch.full((V, H), float("nan"), dtype=torch.float32, device=DEV)
        out["loss"], out["nll"] = fl.flce_pair_fwd_bwd(kind, X, W, y, B, II, p["beta"], p["gamma"],
                                                       p["alpha"], chunk_pairs, dX, dW, ws, rc, rr,
                                                       clp, rlp, z)
        out["dX"], out["dW"] = dX.double().cpu().numpy(), dW.double().cpu().numpy()
    else:
        out["loss"], out["nll"] = fl.flce_pair_fwd(kind, X, W, y, B, II, p["beta"], p["gamma"],
                                                   p["alpha"], chunk_pairs, ws, rc, rr, clp, rlp,
                                                   z)
    torch.cuda.synchronize()
    out["clp"], out["rlp"], out["z"] = (t.double().cpu().numpy() for t in (clp, rlp, z))
    return out


def _oracle(kind, inp, B, ref=None, **kw):
    p = dict(PARAMS[kind])
    p.update(kw)
    rc, rr = (ref[0].astype(np.float64), ref[1].astype(np.float64)) if ref is not None else \
        (None, None)
    return oracle.preference(kind, inp.X_f64(), inp.W_f64(), inp.labels, B, II,
                             ref_chosen=rc, ref_rejected=rr, **p)


def _check(out, r, kind, dtype):
    check_loss(out["loss"], r.loss, dtype)
    check_loss(out["nll"], r.nll, dtype)
    tol = 2e-4 if dtype == "bf16" else 1e-5
    scale = max(np.max(np.abs(r.chosen_logp)), np.max(np.abs(r.rejected_logp)), 1.0)
    assert np.max(np.abs(out["clp"] - r.chosen_logp)) <= tol * scale
    assert np.max(np.abs(out["rlp"] - r.rejected_logp)) <= tol * scale
    zs = max(np.max(np.abs(r.pair_logit)), 1.0)
    assert np.max(np.abs(out["z"] - r.pair_logit)) <= 10 * tol * zs
    if "dX" in out:
        check_grad(out["dX"], r.dX, dtype, "dX")
        check_grad(out["dW"], r.dW, dtype, "dW")


CASES = [("bf16", 3, 77, 128, 1000, 2), ("bf16", 4, 96, 256, 3000, 1), ("f32", 3, 37, 64, 500, 2)]


@pytest.mark.parametrize("dtype,B,T,H,V,chunk_pairs", CASES)
@pytest.mark.parametrize("kind", ["simpo", "cpo", "dpo", "orpo"])
def test_pair_parity(kind, dtype, B, T, H, V, chunk_pairs):
    inp = datagen.make_pairs(B, T, H, V, dtype, seed=B * 100 + T + len(kind))
    ref = _ref_logps(B, T) if kind == "dpo" else None
    out = _run(kind, inp, B, chunk_pairs, ref)
    _check(out, _oracle(kind, inp, B, ref), kind, dtype)


def _random_pair_shapes(count, seed):
    """Seeded (kind, dtype, pairs, T, H, V, chunk_pairs): sequence lengths
    off the 256-row tile grid, so pairs straddle row tiles inside a chunk."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        B = int(rng.integers(1, 6))
        out.append((str(rng.choice(["simpo", "cpo", "dpo", "orpo"])), str(rng.choice(["bf16", "f32"])),
                    B, int(rng.integers(2, 300)), 8 * int(rng.integers(1, 49)),
                    int(rng.integers(2, 4000)), int(rng.integers(1, B + 1))))
    return out


@pytest.mark.parametrize("kind,dtype,B,T,H,V,chunk_pairs", _random_pair_shapes(8, 20261205))
def test_pair_random_shapes(kind, dtype, B, T, H, V, chunk_pairs):
    inp = datagen.make_pairs(B, T, H, V, dtype, seed=B * 1000 + T + V)
    ref = _ref_logps(B, T) if kind == "dpo" else None
    out = _run(kind, inp, B, chunk_pairs, ref)
    _check(out, _oracle(kind, inp, B, ref), kind, dtype)


def test_pair_forward_only():
    inp = datagen.make_pairs(3, 64, 128, 700, "bf16", seed=9)
    for kind in ("simpo", "cpo"):
        out = _run(kind, inp, 3, 1, bwd=False)
        _check(out, _oracle(kind, inp, 3), kind, "bf16")


def test_dpo_reference_from_head():
    """Reference log-probabilities from a second head through sequence_logps
    (its summed token log-probabilities on the GPU), then DPO."""
    B, T, H, V = 3, 48, 64, 400
    inp = datagen.make_pairs(B, T, H, V, "f32", seed=13)
    refw = datagen.make_pairs(B, T, H, V, "f32", seed=14).W
    X, W, y = to_device(inp)
    Wref = torch.from_numpy(refw).to(DEV)
    rc, rr = fl.sequence_logps(Wref, X, y.view(2 * B, T))
    ro = oracle.preference("cpo", inp.X_f64(), refw.astype(np.float64), inp.labels, B, II,
                           beta=0.0, grads=False)
    assert np.max(np.abs(rc.double().cpu().numpy() - ro.chosen_logp)) <= \
        1e-5 * np.max(np.abs(ro.chosen_logp))
    assert np.max(np.abs(rr.double().cpu().numpy() - ro.rejected_logp)) <= \
        1e-5 * np.max(np.abs(ro.rejected_logp))
    Xg = X.view(2 * B, T, H).clone().requires_grad_(True)
    Wg = W.clone().requires_grad_(True)
    loss = fl.FusedLinearDPOLoss(beta=0.1)(Wg, Xg, y.view(2 * B, T), ref_weight=Wref)
    loss.backward()
    r = oracle.preference("dpo", inp.X_f64(), inp.W_f64(), inp.labels, B, II, beta=0.1,
                          ref_chosen=ro.chosen_logp, ref_rejected=ro.rejected_logp)
    check_loss(float(loss), r.loss, "f32")
    check_grad(Xg.grad.reshape(-1, H).double().cpu().numpy(), r.dX, "f32", "dX")
    check_grad(Wg.grad.double().cpu().numpy(), r.dW, "f32", "dW")


@pytest.mark.parametrize("kind", ["simpo", "cpo"])
def test_pair_modules(kind):
    B, T, H, V = 2, 40, 64, 300
    inp = datagen.make_pairs(B, T, H, V, "f32", seed=17)
    X, W, y = to_device(inp)
    Xg = X.view(2 * B, T, H).clone().requires_grad_(True)
    Wg = W.clone().requires_grad_(True)
    mod = fl.FusedLinearSimPOLoss(beta=2.0, gamma=1.0, alpha=0.5) if kind == "simpo" else \
        fl.FusedLinearCPOLoss(beta=0.1, alpha=1.0)
    loss = mod(Wg, Xg, y.view(2 * B, T))
    (0.5 * loss).backward()
    r = _oracle(kind, inp, B)
    check_loss(float(loss), r.loss, "f32")
    check_grad(Xg.grad.reshape(-1, H).double().cpu().numpy(), 0.5 * r.dX, "f32", "dX")
    check_grad(Wg.grad.double().cpu().numpy(), 0.5 * r.dW, "f32", "dW")


def test_pair_degenerate_shapes():
    """T = 1 (one token per sequence), more pairs per chunk than pairs, and a
    batch with no scored token (every pair empty: loss 0, gradients 0)."""
    inp = datagen.make_pairs(5, 1, 64, 300, "f32", seed=81)
    inp.labels[:] = np.random.default_rng(1).integers(0, 300, inp.labels.size)
    for kind in ("orpo", "simpo", "cpo"):
        out = _run(kind, inp, 5, 9)
        _check(out, _oracle(kind, inp, 5), kind, "f32")
    empty = datagen.make_pairs(3, 16, 64, 300, "bf16", seed=82)
    empty.labels[:] = II
    out = _run("orpo", empty, 3, 2)
    r = _oracle("orpo", empty, 3)
    assert out["loss"] == 0.0 and r.loss == 0.0
    assert np.all(out["dX"] == 0.0) and np.all(out["dW"] == 0.0)
