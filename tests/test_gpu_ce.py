"""GPU parity of cross-entropy on given logits (flce_ce_fwd_bwd / flce_ce_fwd)
against the fp64 oracle: every element at small sizes (vector and
one-element paths, all reductions, masked logits, the special cases), and
sampled rows plus the exact loss at the Llama-3-8B head's logits size."""
import numpy as np
import pytest
import torch

import datagen
import linear_cross_entropy_04_amd as fl
import oracle
from _gpu_common import DEV, TOL, check_grad, check_loss, say

pytestmark = pytest.mark.gpu
II = -100


def _logits(N, V, kind, seed, ignore_frac=0.1, want64=True):
    """Seeded logits (datagen.make_logits) and their exact fp64 values."""
    Zraw, y = datagen.make_logits(N, V, kind, seed=seed, ignore_frac=ignore_frac)
    if not want64:
        return Zraw, None, y
    Z = datagen.bf16_bits_to_f32(Zraw) if kind == "bf16" else Zraw
    return Zraw, Z.astype(np.float64), y


def _to_dev(Z, kind):
    if kind == "bf16":
        return torch.from_numpy(Z.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(Z).to(DEV)


def _run(Zraw, y, kind, reduction, grad_rows=None, grad=True):
    N, V = Zraw.shape
    L = _to_dev(Zraw, kind)
    yt = torch.from_numpy(y).to(DEV)
    ws = torch.full((fl.flce_ce_workspace_bytes(N),), 255, dtype=torch.uint8, device=DEV)
    rl = torch.full((N,), float("nan"), dtype=torch.float32, device=DEV)
    rs = torch.full((N,), float("nan"), dtype=torch.float32, device=DEV)
    lp = torch.full((N,), float("nan"), dtype=torch.float32, device=DEV)
    g = None if grad_rows is None else torch.from_numpy(grad_rows).to(DEV)
    say(f"  gpu ce call: N={N} V={V} {kind} reduction={reduction} grad={grad}")
    if grad:
        loss = fl.flce_ce_fwd_bwd(L, yt, II, ws, reduction=reduction, grad_rows=g, row_loss=rl,
                                  row_lse=rs, logprob=lp)
    else:
        loss = fl.flce_ce_fwd(L, yt, II, ws, reduction=reduction, row_loss=rl, row_lse=rs,
                              logprob=lp)
    torch.cuda.synchronize()
    return loss, L, rl.double().cpu().numpy(), rs.double().cpu().numpy(), lp.double().cpu().numpy()


def _random_ce_shapes(count, seed):
    """Seeded (kind, N, V): any row count and vocabulary size, including
    vocabularies shorter than one thread's vector and longer than a row's
    first pass holds in cache."""
    rng = np.random.default_rng(seed)
    return [(str(rng.choice(["bf16", "f32"])), int(rng.integers(1, 700)),
             int(rng.choice([rng.integers(1, 64), rng.integers(64, 9000), rng.integers(9000, 140000)])))
            for _ in range(count)]


@pytest.mark.parametrize("kind,N,V", _random_ce_shapes(8, 20261204))
def test_ce_random_shapes(kind, N, V):
    Zraw, Z, y = _logits(N, V, kind, seed=N * 11 + V)
    loss, L, rl, rs, lp = _run(Zraw, y, kind, "mean")
    r = oracle.cross_entropy(Z, y, II, "mean")
    check_loss(loss, r.loss, kind)
    check_grad(L.double().cpu().numpy(), r.dZ, kind, "dlogits")
    tol = 1e-3 if kind == "bf16" else 1e-5
    assert np.max(np.abs(rs - r.lse) / np.abs(r.lse)) <= tol


@pytest.mark.parametrize("kind,N,V", [("bf16", 300, 4096), ("bf16", 257, 1003),
                                      ("f32", 200, 1000), ("f32", 65, 999)])
@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_ce_parity(kind, N, V, reduction):
    Zraw, Z, y = _logits(N, V, kind, seed=N * 7 + V)
    gr = np.random.default_rng(3).standard_normal(N).astype(np.float32) \
        if reduction == "none" else None
    loss, L, rl, rs, lp = _run(Zraw, y, kind, reduction, gr)
    r = oracle.cross_entropy(Z, y, II, reduction,
                             grad_rows=None if gr is None else gr.astype(np.float64))
    check_loss(loss, r.loss, kind)
    check_grad(L.double().cpu().numpy(), r.dZ, kind, "dlogits")
    tol = 1e-3 if kind == "bf16" else 1e-5
    assert np.max(np.abs(rs - r.lse) / np.abs(r.lse)) <= tol
    assert np.max(np.abs(rl - r.row_loss)) <= tol * np.max(np.abs(r.lse))
    assert np.max(np.abs(lp - r.logprob)) <= tol * np.max(np.abs(r.lse))
    valid = y != II
    assert np.all(L.double().cpu().numpy()[~valid] == 0.0)


def test_ce_masked_logits():
    """-inf logits (masked classes) take no probability and get zero gradient."""
    Zraw, Z, y = _logits(128, 2048, "f32", seed=5)
    rng = np.random.default_rng(6)
    mask = rng.random(Z.shape) < 0.3
    mask[np.arange(128), np.where(y >= 0, y, 0)] = False       # never the target
    Zraw = Zraw.copy()
    Zraw[mask] = -np.inf
    Z = Zraw.astype(np.float64)
    loss, L, rl, _, _ = _run(Zraw, y, "f32", "mean")
    r = oracle.cross_entropy(Z, y, II, "mean")
    check_loss(loss, r.loss, "f32")
    G = L.double().cpu().numpy()
    check_grad(G, r.dZ, "f32", "dlogits")
    assert np.all(G[mask] == 0.0)


def test_ce_forward_only_leaves_logits():
    Zraw, Z, y = _logits(100, 3000, "bf16", seed=8)
    loss, L, _, _, _ = _run(Zraw, y, "bf16", "mean", grad=False)
    assert np.array_equal(L.view(torch.int16).cpu().numpy().view(np.uint16), Zraw)
    check_loss(loss, oracle.cross_entropy(Z, y, II, "mean", grads=False).loss, "bf16")


def test_ce_special_cases():
    # all ignored: loss 0, gradient 0
    Zraw, Z, y = _logits(64, 512, "bf16", seed=9)
    y[:] = II
    loss, L, _, _, _ = _run(Zraw, y, "bf16", "mean")
    assert loss == 0.0 and bool((L == 0).all())
    # invalid label
    Zraw, Z, y = _logits(64, 512, "bf16", seed=10)
    y[3] = 512
    with pytest.raises(fl.FLCEError) as e:
        _run(Zraw, y, "bf16", "mean")
    assert e.value.status == fl.FLCE_ELABEL
    # no tokens
    ws = torch.empty(fl.flce_ce_workspace_bytes(0), dtype=torch.uint8, device=DEV)
    L = torch.empty((0, 512), dtype=torch.bfloat16, device=DEV)
    assert fl.flce_ce_fwd_bwd(L, torch.empty(0, dtype=torch.int64, device=DEV), II, ws) == 0.0


@pytest.mark.parametrize("inplace", [True, False])
def test_ce_autograd(inplace):
    Zraw, Z, y = _logits(150, 777, "f32", seed=12)
    Lt = _to_dev(Zraw, "f32").requires_grad_(True)
    out = fl.cross_entropy(Lt, torch.from_numpy(y).to(DEV), reduction="sum", inplace=inplace)
    (0.5 * out).backward()
    r = oracle.cross_entropy(Z, y, II, "sum")
    check_loss(float(out), r.loss, "f32")
    check_grad(Lt.grad.double().cpu().numpy(), 0.5 * r.dZ, "f32", "dlogits")


def test_ce_fullsize_llama_head_logits():
    """N = 8192 tokens x V = 128256 bf16 logits: the exact loss (oracle over
    all rows in blocks) and sampled gradient rows."""
    N, V = 8192, 128256
    Zraw, _, y = _logits(N, V, "bf16", seed=2026, ignore_frac=0.05, want64=False)
    loss, L, rl, rs, _ = _run(Zraw, y, "bf16", "mean")
    Zf = datagen.bf16_bits_to_f32
    lse = np.empty(N)
    for s in range(0, N, 512):
        lse[s:s + 512] = oracle.cross_entropy(Zf(Zraw[s:s + 512]).astype(np.float64),
                                              y[s:s + 512], II, "sum", grads=False).lse
    valid = y != II
    zy = np.where(valid, Zf(Zraw[np.arange(N), np.where(valid, y, 0)]).astype(np.float64), 0.0)
    ref_loss = float(np.sum(np.where(valid, lse - zy, 0.0)) / valid.sum())
    check_loss(loss, ref_loss, "bf16")
    assert np.max(np.abs(rs - lse) / np.abs(lse)) <= 1e-3
    rows = datagen.sample_rows(N, 16, 77, must=(0, N - 1, int(np.flatnonzero(~valid)[0])))
    rr = oracle.cross_entropy(Zf(Zraw[rows]).astype(np.float64), y[rows], II, "sum")
    check_grad(L[torch.from_numpy(rows).to(DEV)].double().cpu().numpy(),
               rr.dZ / valid.sum(), "bf16", "dlogits sampled rows")
