"""GPU parity of the odds-ratio preference loss (flce_orpo_fwd_bwd /
flce_orpo_fwd) against the fp64 oracle's orpo: every element at small sizes
(bf16 and fp32, chunks of one or more pairs, ragged sequence lengths), the
special cases (an empty sequence, an invalid label), the autograd binding,
and at the Llama-3-8B head's size the exact loss with sampled dX and dW rows."""
import numpy as np
import pytest
import torch

import datagen
import linear_cross_entropy_04_amd as fl
import oracle
from _gpu_common import DEV, TOL, check_grad, check_loss, say, to_device

pytestmark = pytest.mark.gpu
II = -100


def _run(inp, B, beta, chunk_pairs, bwd=True, labels=None):
    X, W, y = to_device(inp)
    if labels is not None:
        y = torch.from_numpy(np.asarray(labels, dtype=np.int64)).to(DEV)
    N, H = X.shape
    V = W.shape[0]
    T = N // (2 * B)
    dt = fl.FLCE_BF16 if X.dtype == torch.bfloat16 else fl.FLCE_F32
    ws = torch.full((fl.flce_orpo_workspace_bytes(B, T, H, V, dt, chunk_pairs),), 255,
                    dtype=torch.uint8, device=DEV)
    clp, rlp, lor = (torch.full((B,), float("nan"), dtype=torch.float32, device=DEV)
                     for _ in range(3))
    say(f"  gpu orpo call: pairs={B} T={T} H={H} V={V} {'bf16' if dt else 'f32'} "
        f"chunk_pairs={chunk_pairs} beta={beta} {'fwd_bwd' if bwd else 'fwd'}")
    out = {}
    if bwd:
        dX = torch.full_like(X, float("nan"))
        dW = torch.full((V, H), float("nan"), dtype=torch.float32, device=DEV)
        out["loss"], out["nll"] = fl.flce_orpo_fwd_bwd(X, W, y, B, II, beta, chunk_pairs, dX, dW,
                                                       ws, clp, rlp, lor)
        out["dX_t"], out["dW_t"] = dX, dW
    else:
        out["loss"], out["nll"] = fl.flce_orpo_fwd(X, W, y, B, II, beta, chunk_pairs, ws, clp,
                                                   rlp, lor)
    torch.cuda.synchronize()
    out["clp"], out["rlp"], out["lor"] = (t.double().cpu().numpy() for t in (clp, rlp, lor))
    return out


def _check_pairs(out, r, kind):
    # the sequence log-probabilities come from fp32 accumulators on exact inputs
    scale = max(np.max(np.abs(r.chosen_logp)), np.max(np.abs(r.rejected_logp)), 1.0)
    tol = 2e-4 if kind == "bf16" else 1e-5
    assert np.max(np.abs(out["clp"] - r.chosen_logp)) <= tol * scale
    assert np.max(np.abs(out["rlp"] - r.rejected_logp)) <= tol * scale
    assert np.max(np.abs(out["lor"] - r.log_odds_ratio)) <= 10 * tol * scale


CASES = [("bf16", 3, 77, 128, 1000, 2), ("bf16", 4, 128, 256, 3000, 1),
         ("bf16", 5, 100, 192, 2049, 0), ("f32", 3, 37, 64, 500, 2), ("f32", 2, 50, 33, 130, 1)]


@pytest.mark.parametrize("kind,B,T,H,V,chunk_pairs", CASES)
def test_orpo_parity(kind, B, T, H, V, chunk_pairs):
    inp = datagen.make_pairs(B, T, H, V, kind, seed=B * 1000 + T)
    beta = 0.1
    out = _run(inp, B, beta, chunk_pairs)
    r = oracle.orpo(inp.X_f64(), inp.W_f64(), inp.labels, B, II, beta)
    check_loss(out["loss"], r.loss, kind)
    check_loss(out["nll"], r.nll, kind)
    _check_pairs(out, r, kind)
    check_grad(out["dX_t"].double().cpu().numpy(), r.dX, kind, "dX")
    check_grad(out["dW_t"].double().cpu().numpy(), r.dW, kind, "dW")
    dX = out["dX_t"].double().cpu().numpy()
    assert np.all(dX[inp.labels == II] == 0.0)


def test_orpo_large_beta_and_forward_only():
    inp = datagen.make_pairs(4, 64, 128, 777, "bf16", seed=31)
    r = oracle.orpo(inp.X_f64(), inp.W_f64(), inp.labels, 4, II, 2.5)
    out = _run(inp, 4, 2.5, 3)
    check_loss(out["loss"], r.loss, "bf16")
    check_grad(out["dW_t"].double().cpu().numpy(), r.dW, "bf16", "dW")
    fwd = _run(inp, 4, 2.5, 1, bwd=False)
    check_loss(fwd["loss"], r.loss, "bf16")
    _check_pairs(fwd, r, "bf16")


def test_orpo_empty_sequence_and_bad_label():
    B, T = 3, 40
    inp = datagen.make_pairs(B, T, 64, 300, "f32", seed=41)
    y = inp.labels.reshape(2 * B, T).copy()
    y[B + 1] = II                                    # pair 1's rejected sequence is empty
    r = oracle.orpo(inp.X_f64(), inp.W_f64(), y.reshape(-1), B, II, 0.2)
    out = _run(inp, B, 0.2, 2, labels=y.reshape(-1))
    check_loss(out["loss"], r.loss, "f32")
    assert out["lor"][1] == 0.0
    check_grad(out["dX_t"].double().cpu().numpy(), r.dX, "f32", "dX")
    check_grad(out["dW_t"].double().cpu().numpy(), r.dW, "f32", "dW")
    y[0, 5] = 300                                    # outside [0, V)
    with pytest.raises(fl.FLCEError) as e:
        _run(inp, B, 0.2, 2, labels=y.reshape(-1))
    assert e.value.status == fl.FLCE_ELABEL


def test_orpo_autograd():
    B, T, H, V = 3, 30, 64, 200
    inp = datagen.make_pairs(B, T, H, V, "f32", seed=51)
    X, W, y = to_device(inp)
    Xg = X.view(2 * B, T, H).clone().requires_grad_(True)
    Wg = W.clone().requires_grad_(True)
    loss = fl.FusedLinearORPOLoss(beta=0.3, chunk_pairs=2)(Wg, Xg, y.view(2 * B, T))
    (1.5 * loss).backward()
    r = oracle.orpo(inp.X_f64(), inp.W_f64(), inp.labels, B, II, 0.3)
    check_loss(float(loss), r.loss, "f32")
    check_grad(Xg.grad.reshape(-1, H).double().cpu().numpy(), 1.5 * r.dX, "f32", "dX")
    check_grad(Wg.grad.double().cpu().numpy(), 1.5 * r.dW, "f32", "dW")


def test_orpo_fullsize_llama_head():
    """8 pairs of 512-token sequences on the Llama-3-8B head (8192 rows, H =
    4096, V = 128256, bf16), one pair per chunk: the exact loss and the
    per-pair terms from every token, and sampled dX and dW rows."""
    B, T, H, V = 8, 512, 4096, 128256
    inp = datagen.make_pairs(B, T, H, V, "bf16", seed=2027)
    out = _run(inp, B, 0.1, 1)
    valid = np.flatnonzero(inp.labels != II)
    rows = datagen.sample_rows(2 * B * T, 12, 3, must=(int(valid[0]), int(valid[-1]),
                                                       B * T + int(valid[len(valid) // 2]) % (B * T)))
    vrows = datagen.sample_rows(V, 8, 4, must=(0, V - 1))
    X64, W64 = inp.X_f64(), inp.W_f64()
    r = oracle.orpo_rows(X64, W64, inp.labels, B, rows, vrows, II, 0.1, block=512)
    check_loss(out["loss"], r.loss, "bf16")
    check_loss(out["nll"], r.nll, "bf16")
    _check_pairs(out, r, "bf16")
    check_grad(out["dX_t"][torch.from_numpy(rows).to(DEV)].double().cpu().numpy(), r.dX, "bf16",
               "dX sampled rows")
    check_grad(out["dW_t"][torch.from_numpy(vrows).to(DEV)].double().cpu().numpy(), r.dW, "bf16",
               "dW sampled rows")
