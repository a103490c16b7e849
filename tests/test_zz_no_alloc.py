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


def test_noalloc_llama_head_and_refusal():
    # The Llama-3-8B head: with the chunk left to the library it plans the
    # largest chunk whose workspace fits the static array, and matches the
    # workspace entry point at that chunk bitwise; an explicit chunk whose
    # workspace exceeds the array is refused before any device work.
    N, H, V = 8192, 4096, 128256
    cap = fl.flce_noalloc_scratch_bytes()
    st, chunk, peak = fl.flce_plan(N, H, V, fl.FLCE_BF16, scratch_budget_bytes=cap)
    assert st == fl.FLCE_OK and peak <= cap
    assert fl.flce_workspace_bytes(N, H, V, fl.FLCE_BF16, 2 * chunk) > cap
    say(f"  noalloc case: N={N} H={H} V={V} bf16 chunk={chunk} (auto)")
    g = torch.Generator(device="cpu").manual_seed(7)
    X = (torch.randn(N, H, generator=g) * 0.5).to(torch.bfloat16).to(DEV)
    W = (torch.randn(V, H, generator=g) * 0.02).to(torch.bfloat16).to(DEV)
    y = torch.randint(0, V, (N,), generator=g).to(DEV)
    ws = fl.workspace(N, H, V, fl.FLCE_BF16, chunk, device=DEV)
    dX0, dW0 = torch.empty_like(X), torch.empty((V, H), dtype=torch.float32, device=DEV)
    rl0 = torch.empty(N, dtype=torch.float32, device=DEV)
    loss0 = fl.flce_fwd_bwd(X, W, y, -100, chunk, dX0, dW0, ws, row_loss=rl0, row_lse=None)
    del ws
    dX1 = torch.full_like(X, float("nan"))
    dW1 = torch.full((V, H), float("nan"), dtype=torch.float32, device=DEV)
    rl1 = torch.full((N,), float("nan"), dtype=torch.float32, device=DEV)
    rs1 = torch.empty(N, dtype=torch.float32, device=DEV)
    st, loss1 = _noalloc(X, W, y, 0, dX1, dW1, rl1, rs1)
    torch.cuda.synchronize()
    assert st == fl.FLCE_OK, fl.flce_status_string(st)
    assert loss1 == loss0
    assert torch.equal(dX1, dX0) and torch.equal(dW1, dW0) and torch.equal(rl1, rl0)
    del dX0, dW0, dX1

    big = 2 * chunk
    say(f"  noalloc refusal: chunk={big}")
    dX = torch.empty_like(X)
    dW1.fill_(7.0)
    st, _ = _noalloc(X, W, y, big, dX, dW1, rl1, rs1)
    assert st == fl.FLCE_EWORKSPACE
    assert "exceeds the static scratch" in fl.flce_last_error()
    torch.cuda.synchronize()
    assert bool((dW1 == 7.0).all())                    # untouched
