"""The entry point that allocates nothing (flce_fwd_bwd_noalloc), through the
C ABI, against flce_fwd_bwd on the same inputs: two calls in a row, the
second on a smaller problem, each bitwise equal to the workspace entry
point's result with the same chunk; and a problem whose workspace exceeds the
library's scratch array is refused before any device work."""
import ctypes

import numpy as np
import pytest
import torch

import datagen
import linear_cross_entropy_04_amd as fl
from _gpu_common import DEV, check_grad, check_loss, say, to_device

pytestmark = pytest.mark.gpu


def _noalloc(X, W, y, chunk, dX, dW, rl, rs):
    N, H = X.shape
    V = W.shape[0]
    dt = fl.FLCE_BF16 if X.dtype == torch.bfloat16 else fl.FLCE_F32
    loss = ctypes.c_float(float("nan"))
    stream = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    st = fl._load().flce_fwd_bwd_noalloc(
        ctypes.c_void_p(X.data_ptr()), ctypes.c_void_p(W.data_ptr()), ctypes.c_void_p(y.data_ptr()),
        N, H, V, dt, -100, chunk, ctypes.byref(loss), ctypes.c_void_p(dX.data_ptr()),
        ctypes.c_void_p(dW.data_ptr()), ctypes.c_void_p(rl.data_ptr()),
        ctypes.c_void_p(rs.data_ptr()), stream)
    return st, loss.value


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_workspace_entry(dtype):
    import oracle
    cases = [(1000, 256, 5000, 256), (300, 128, 3000, 128)]      # the second call is smaller
    for N, H, V, chunk in cases:
        say(f"  noalloc case: N={N} H={H} V={V} dtype={dtype} chunk={chunk}")
        inp = datagen.make_custom(N, H, V, dtype, seed=N + V, ignore_frac=0.1)
        X, W, y = to_device(inp)
        ws = fl.workspace(N, H, V, fl.FLCE_BF16 if dtype == "bf16" else fl.FLCE_F32, chunk, device=DEV)
        dX0, dW0 = torch.empty_like(X), torch.empty((V, H), dtype=torch.float32, device=DEV)
        rl0 = torch.empty(N, dtype=torch.float32, device=DEV)
        rs0 = torch.empty(N, dtype=torch.float32, device=DEV)
        loss0 = fl.flce_fwd_bwd(X, W, y, -100, chunk, dX0, dW0, ws, row_loss=rl0, row_lse=rs0)
        dX1 = torch.full_like(X, float("nan"))
        dW1 = torch.full((V, H), float("nan"), dtype=torch.float32, device=DEV)
        rl1 = torch.full((N,), float("nan"), dtype=torch.float32, device=DEV)
        rs1 = torch.full((N,), float("nan"), dtype=torch.float32, device=DEV)
        st, loss1 = _noalloc(X, W, y, chunk, dX1, dW1, rl1, rs1)
        torch.cuda.synchronize()
        assert st == fl.FLCE_OK, fl.flce_status_string(st)
        assert loss1 == loss0
        assert torch.equal(dX1, dX0) and torch.equal(dW1, dW0)
        assert torch.equal(rl1, rl0) and torch.equal(rs1, rs0)
        # and both meet the oracle's bar
        r = oracle.flce(inp.X_f64(), inp.W_f64(), inp.labels)
        check_loss(loss1, r.loss, dtype)
        check_grad(dX1.double().cpu().numpy(), r.dX, dtype, "dX")
        check_grad(dW1.double().cpu().numpy(), r.dW, dtype, "dW")


def test_noalloc_refuses_oversized_workspace():
    # the Llama-3-8B head needs more than the static array at any chunk
    N, H, V = 8192, 4096, 128256
    assert fl.flce_workspace_bytes(N, H, V, fl.FLCE_BF16, 256) > fl.flce_noalloc_scratch_bytes()
    X = torch.zeros(N, H, dtype=torch.bfloat16, device=DEV)
    W = torch.zeros(V, H, dtype=torch.bfloat16, device=DEV)
    y = torch.zeros(N, dtype=torch.int64, device=DEV)
    dX = torch.empty_like(X)
    dW = torch.full((V, H), 7.0, dtype=torch.float32, device=DEV)
    rl = torch.empty(N, dtype=torch.float32, device=DEV)
    st, _ = _noalloc(X, W, y, 0, dX, dW, rl, rl)
    assert st == fl.FLCE_EWORKSPACE
    assert "exceeds the static scratch" in fl.flce_last_error()
    assert bool((dW == 7.0).all())                     # untouched
