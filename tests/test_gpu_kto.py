"""GPU parity of the unpaired preference loss KTO (flce_kto_fwd_bwd /
flce_kto_fwd) against the fp64 oracle's kto: every element at small sizes
(bf16 and fp32, chunks of one or more sequences, an odd sequence count), the
reference log-probabilities computed on the GPU from a reference head, the
autograd module, and at the Llama-3-8B head's size the exact loss with
sampled dX and dW rows (the oracle's row-block form of the same weights)."""
import numpy as np
import pytest
import torch

import datagen
import linear_cross_entropy_04_amd as fl
import oracle
from _gpu_common import DEV, check_grad, check_loss, say, to_device

pytestmark = pytest.mark.gpu
II = -100
P = dict(beta=0.1, z0=0.5, lambda_d=1.0, lambda_u=1.3)


def _run(inp, des, R, S, chunk_seqs, bwd=True, p=P):
    X, W, y = to_device(inp)
    N, H = X.shape
    V = W.shape[0]
    dt = fl.FLCE_BF16 if X.dtype == torch.bfloat16 else fl.FLCE_F32
    ws = torch.full((fl.flce_kto_workspace_bytes(S, N // S, H, V, dt, chunk_seqs),), 255,
                    dtype=torch.uint8, device=DEV)
    d = torch.from_numpy(des).to(DEV)
    r = torch.from_numpy(R).to(DEV)
    lp, rw = (torch.full((S,), float("nan"), dtype=torch.float32, device=DEV) for _ in range(2))
    say(f"  gpu kto call: seqs={S} T={N // S} H={H} V={V} {'bf16' if dt else 'f32'} "
        f"chunk_seqs={chunk_seqs} {'fwd_bwd' if bwd else 'fwd'}")
    out = {}
    if bwd:
        dX = torch.full_like(X, float("nan"))
        dW = torch.full((V, H), float("nan"), dtype=torch.float32, device=DEV)
        out["loss"] = fl.flce_kto_fwd_bwd(X, W, y, S, II, d, r, p["beta"], p["z0"], p["lambda_d"],
                                          p["lambda_u"], chunk_seqs, dX, dW, ws, lp, rw)
        out["dX_t"], out["dW_t"] = dX, dW
    else:
        out["loss"] = fl.flce_kto_fwd(X, W, y, S, II, d, r, p["beta"], p["z0"], p["lambda_d"],
                                      p["lambda_u"], chunk_seqs, ws, lp, rw)
    torch.cuda.synchronize()
    out["logp"], out["reward"] = lp.double().cpu().numpy(), rw.double().cpu().numpy()
    return out


def _check_seq(out, r, dtype):
    tol = 2e-4 if dtype == "bf16" else 1e-5
    scale = max(np.max(np.abs(r.logp)), 1.0)
    assert np.max(np.abs(out["logp"] - r.logp)) <= tol * scale
    assert np.max(np.abs(out["reward"] - r.reward)) <= tol * scale


CASES = [("bf16", 5, 77, 128, 1000, 2), ("bf16", 4, 128, 256, 3000, 1),
         ("bf16", 7, 64, 192, 2049, 0), ("f32", 5, 37, 64, 500, 3), ("f32", 3, 50, 33, 130, 1)]


@pytest.mark.parametrize("dtype,S,T,H,V,chunk_seqs", CASES)
def test_kto_parity(dtype, S, T, H, V, chunk_seqs):
    inp, des, R = datagen.make_unpaired(S, T, H, V, dtype, seed=S * 100 + T)
    out = _run(inp, des, R, S, chunk_seqs)
    r = oracle.kto(inp.X_f64(), inp.W_f64(), inp.labels, S, des.astype(bool), R.astype(np.float64),
                   II, **P)
    check_loss(out["loss"], r.loss, dtype)
    _check_seq(out, r, dtype)
    check_grad(out["dX_t"].double().cpu().numpy(), r.dX, dtype, "dX")
    check_grad(out["dW_t"].double().cpu().numpy(), r.dW, dtype, "dW")
    fwd = _run(inp, des, R, S, chunk_seqs, bwd=False)
    check_loss(fwd["loss"], r.loss, dtype)


def _random_kto_shapes(count, seed):
    """Seeded (dtype, sequences, T, H, V, chunk_seqs); chunk 0 lets the
    planner choose."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        S = int(rng.integers(1, 9))
        out.append((str(rng.choice(["bf16", "f32"])), S, int(rng.integers(2, 260)),
                    8 * int(rng.integers(1, 41)), int(rng.integers(2, 3500)),
                    int(rng.integers(0, S + 1))))
    return out


@pytest.mark.parametrize("dtype,S,T,H,V,chunk_seqs", _random_kto_shapes(6, 20261206))
def test_kto_random_shapes(dtype, S, T, H, V, chunk_seqs):
    inp, des, R = datagen.make_unpaired(S, T, H, V, dtype, seed=S * 1000 + T + V)
    out = _run(inp, des, R, S, chunk_seqs)
    r = oracle.kto(inp.X_f64(), inp.W_f64(), inp.labels, S, des.astype(bool), R.astype(np.float64),
                   II, **P)
    check_loss(out["loss"], r.loss, dtype)
    _check_seq(out, r, dtype)
    check_grad(out["dX_t"].double().cpu().numpy(), r.dX, dtype, "dX")
    check_grad(out["dW_t"].double().cpu().numpy(), r.dW, dtype, "dW")


def test_kto_module_with_reference_head():
    S, T, H, V = 5, 40, 64, 300
    inp, des, _ = datagen.make_unpaired(S, T, H, V, "f32", seed=61)
    refw = datagen.make_unpaired(S, T, H, V, "f32", seed=62)[0].W
    X, W, y = to_device(inp)
    Xg = X.view(S, T, H).clone().requires_grad_(True)
    Wg = W.clone().requires_grad_(True)
    loss = fl.FusedLinearKTOLoss(beta=0.3, lambda_u=1.5)(
        Wg, Xg, y.view(S, T), torch.from_numpy(des).to(DEV), z0=0.2,
        ref_weight=torch.from_numpy(refw).to(DEV))
    (2.0 * loss).backward()
    Rall = oracle.kto(inp.X_f64(), refw.astype(np.float64), inp.labels, S, des.astype(bool),
                      np.zeros(S), II, grads=False).logp      # the reference head's sums
    r = oracle.kto(inp.X_f64(), inp.W_f64(), inp.labels, S, des.astype(bool), Rall, II, beta=0.3,
                   z0=0.2, lambda_u=1.5)
    check_loss(float(loss), r.loss, "f32")
    check_grad(Xg.grad.reshape(-1, H).double().cpu().numpy(), 2.0 * r.dX, "f32", "dX")
    check_grad(Wg.grad.double().cpu().numpy(), 2.0 * r.dW, "f32", "dW")


def test_kto_fullsize_llama_head():
    """16 sequences of 512 tokens on the Llama-3-8B head (8192 rows, H = 4096,
    V = 128256, bf16), two sequences per chunk: the exact loss and every
    sequence's log-probability from all tokens, sampled dX and dW rows."""
    S, T, H, V = 16, 512, 4096, 128256
    inp, des, R = datagen.make_unpaired(S, T, H, V, "bf16", seed=2028)
    out = _run(inp, des, R, S, 2)
    X64, W64 = inp.X_f64(), inp.W_f64()
    lse, rl, _ = oracle.forward_rows(X64, W64, inp.labels, None, II, 512)
    valid = inp.labels != II
    lp = np.where(valid, -rl, 0.0)
    Sref = lp.reshape(S, T).sum(axis=1)
    assert np.max(np.abs(out["logp"] - Sref)) <= 2e-4 * np.max(np.abs(Sref))
    # the loss and weights from the oracle's steps on these log-probabilities
    from oracle import flce_ref as om
    l, dl_dr = om.kto_sequence_terms(Sref - R, des.astype(bool), P["beta"], P["z0"],
                                     P["lambda_d"], P["lambda_u"])
    check_loss(out["loss"], float(l.mean()), "bf16")
    w = om.kto_token_weights(dl_dr, valid, S)
    rows = datagen.sample_rows(S * T, 10, 5, must=(int(np.flatnonzero(valid)[0]),))
    vrows = datagen.sample_rows(V, 6, 6, must=(0, V - 1))
    Z = om.logits(X64[rows], W64)
    dX = om.grad_input(om.dlogits_weighted(Z, om.row_logsumexp(Z), inp.labels[rows], w[rows]),
                       W64)
    Zc = om.logits(X64, W64[vrows])
    dW = om.grad_weight(om.dlogits_weighted(Zc, lse, inp.labels, w, col_ids=vrows), X64)
    check_grad(out["dX_t"][torch.from_numpy(rows).to(DEV)].double().cpu().numpy(), dX, "bf16",
               "dX sampled rows")
    check_grad(out["dW_t"][torch.from_numpy(vrows).to(DEV)].double().cpu().numpy(), dW, "bf16",
               "dW sampled rows")


def test_kto_saturated_sigmoid():
    """Large |beta (r - z0)|: sigmoid(u) rounds to 1 in fp32, so the loss
    term and its derivative must come from sigmoid(-u) itself."""
    S, T, H, V = 6, 48, 64, 300
    inp, des, R = datagen.make_unpaired(S, T, H, V, "f32", seed=71)
    R = R + np.where(des == 1, -40.0, 40.0).astype(np.float32)    # u about +-40 beta
    p = dict(P, beta=1.0, z0=0.0)
    out = _run(inp, des, R, S, 2, p=p)
    r = oracle.kto(inp.X_f64(), inp.W_f64(), inp.labels, S, des.astype(bool),
                   R.astype(np.float64), II, **p)
    assert r.loss > 0.0
    check_loss(out["loss"], r.loss, "f32")
    check_grad(out["dW_t"].double().cpu().numpy(), r.dW, "f32", "dW")


def test_kto_degenerate_shapes():
    """One sequence, one token per sequence, more sequences per chunk than
    sequences, and a sequence with no scored token (its reward is -R)."""
    S, T, H, V = 3, 1, 64, 300
    inp, des, R = datagen.make_unpaired(S, T, H, V, "f32", seed=91)
    inp.labels[:] = np.random.default_rng(2).integers(0, V, S * T)
    inp.labels[1] = II
    out = _run(inp, des, R, S, 7)
    r = oracle.kto(inp.X_f64(), inp.W_f64(), inp.labels, S, des.astype(bool), R.astype(np.float64),
                   II, **P)
    check_loss(out["loss"], r.loss, "f32")
    _check_seq(out, r, "f32")
    check_grad(out["dW_t"].double().cpu().numpy(), r.dW, "f32", "dW")
    assert np.all(out["dX_t"][1].cpu().numpy() == 0.0)
    one, d1, R1 = datagen.make_unpaired(1, 40, H, V, "bf16", seed=92)
    o1 = _run(one, d1, R1, 1, 0)
    r1 = oracle.kto(one.X_f64(), one.W_f64(), one.labels, 1, d1.astype(bool), R1.astype(np.float64),
                    II, **P)
    check_loss(o1["loss"], r1.loss, "bf16")
    check_grad(o1["dW_t"].double().cpu().numpy(), r1.dW, "bf16", "dW")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_kto_reference_point(dtype):
    """z0 from a batch of completions (here the drawn sequences stand for
    mismatched ones): the reference sums sit a known gap below or above the
    oracle's policy sums, so z0 is the mean gap or, clamped, 0."""
    S, T, H, V = 6, 64, 128, 1000
    inp, _, _ = datagen.make_unpaired(S, T, H, V, dtype, seed=71)
    X, W, y = to_device(inp)
    Sp = oracle.kto(inp.X_f64(), inp.W_f64(), inp.labels, S, np.ones(S, bool), np.zeros(S),
                    II, grads=False).logp
    gap = np.array([0.5, 1.5, -0.25, 0.75, 0.0, 1.0])
    tol = (2e-4 if dtype == "bf16" else 1e-5) * max(np.max(np.abs(Sp)), 1.0)
    for R, want in ((Sp - gap, gap.mean()), (Sp + gap + 1.0, 0.0)):
        z = fl.kto_reference_point(W, X.view(S, T, H), y.view(S, T),
                                   torch.from_numpy(R.astype(np.float32)).to(DEV))
        say(f"    z0 = {z:.6f} (want {want:.6f})")
        assert abs(z - want) <= tol + 1e-6 * abs(want)
        assert z == max(0.0, z)
        # the C entry itself, with its per-sequence outputs S and S - R
        Rt = torch.from_numpy(R.astype(np.float32)).to(DEV)
        ws = torch.empty(fl.flce_kto_workspace_bytes(S, T, H, V, 1 if dtype == "bf16" else 0, 2),
                         dtype=torch.uint8, device=DEV)
        lp = torch.full((S,), float("nan"), dtype=torch.float32, device=DEV)
        rw = torch.full((S,), float("nan"), dtype=torch.float32, device=DEV)
        z2 = fl.flce_kto_reference_point(X, W, y, S, II, Rt, 2, ws, logp=lp, reward=rw)
        assert abs(z2 - want) <= tol + 1e-6 * abs(want)
        assert np.max(np.abs(lp.double().cpu().numpy() - Sp)) <= tol
        assert np.max(np.abs(rw.double().cpu().numpy() - (Sp - R))) <= tol
        # and against the oracle's own reference point
        zo = oracle.kto_reference_point(inp.X_f64(), inp.W_f64(), inp.labels, S, R, II)
        assert abs(z2 - zo) <= tol + 1e-6 * abs(zo)
