"""Helpers shared by the GPU parity tests: upload, run through the C ABI, compare.

Tolerances (the contract of the loss): loss relative error <= 1e-3 and
max |gpu - ref| <= 2e-2 * max |ref| per gradient tensor for bf16 inputs with
fp32 accumulation; for the all-fp32 path, 1e-5 for both.
"""
import sys
import time

import numpy as np
import torch

import linear_cross_entropy_04_amd as fl

DEV = "cuda:0"
TOL = {"bf16": {"loss": 1e-3, "grad": 2e-2}, "f32": {"loss": 1e-5, "grad": 1e-5}}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(inp):
    if inp.wl.dtype == "bf16":
        X = torch.from_numpy(inp.X.view(np.int16)).to(DEV).view(torch.bfloat16)
        W = torch.from_numpy(inp.W.view(np.int16)).to(DEV).view(torch.bfloat16)
    else:
        X = torch.from_numpy(inp.X).to(DEV)
        W = torch.from_numpy(inp.W).to(DEV)
    y = torch.from_numpy(inp.labels).to(DEV)
    return X, W, y


def run_gpu(inp, chunk, ignore_index=-100, bwd=True, poison=True, labels=None, tensors=None,
            host_grads=True):
    """One flce_fwd_bwd (or flce_fwd) call; returns host float64 results."""
    X, W, y = tensors if tensors is not None else to_device(inp)
    if labels is not None:
        y = torch.from_numpy(np.asarray(labels, dtype=np.int64)).to(DEV)
    N, H = X.shape
    V = W.shape[0]
    dt = fl.FLCE_BF16 if X.dtype == torch.bfloat16 else fl.FLCE_F32
    ws = fl.workspace(N, H, V, dt, chunk, device=DEV)
    if poison:
        ws.fill_(255)                         # NaN patterns: unwritten scratch would show
    rl = torch.full((N,), float("nan"), dtype=torch.float32, device=DEV)
    rs = torch.full((N,), float("nan"), dtype=torch.float32, device=DEV)
    say(f"  gpu call: N={N} H={H} V={V} dtype={'bf16' if dt else 'f32'} chunk={chunk} "
        f"ignore_index={ignore_index} {'fwd_bwd' if bwd else 'fwd'}")
    t0 = time.time()
    if bwd:
        dX = torch.full_like(X, float("nan"))
        dW = torch.full((V, H), float("nan"), dtype=torch.float32, device=DEV)
        loss = fl.flce_fwd_bwd(X, W, y, ignore_index, chunk, dX, dW, ws, row_loss=rl, row_lse=rs)
    else:
        loss = fl.flce_fwd(X, W, y, ignore_index, chunk, ws, row_loss=rl, row_lse=rs)
    torch.cuda.synchronize()
    out = {"loss": loss, "row_loss": rl.double().cpu().numpy(), "row_lse": rs.double().cpu().numpy(),
           "seconds": time.time() - t0}
    if bwd:
        out["dX_t"] = dX
        out["dW_t"] = dW
        if host_grads:
            out["dX"] = dX.double().cpu().numpy()
            out["dW"] = dW.double().cpu().numpy()
    return out


def rel_max_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite values in GPU output"
    m = float(np.max(np.abs(ref))) if ref.size else 0.0
    e = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    return e / m if m > 0 else e


def check_loss(got, ref, kind):
    tol = TOL[kind]["loss"]
    if ref == 0.0:
        assert got == 0.0, got
    else:
        assert abs(got - ref) <= tol * abs(ref), (got, ref, abs(got - ref) / abs(ref))


def check_grad(got, ref, kind, name):
    e = rel_max_err(got, ref)
    say(f"    {name}: max|err|/max|ref| = {e:.3e}")
    assert e <= TOL[kind]["grad"], (name, e)
