"""GPU test of the library's launch timing (flce_profile_*): with every class
selected each kernel class of a call reports its launches; with one class
selected only that class records events.  The results of the timed call are
checked against the fp64 oracle like any other call."""
import numpy as np
import pytest
import torch

import datagen
import linear_cross_entropy_04_amd as fl
import oracle
from _gpu_common import DEV, check_grad, check_loss, say, to_device

pytestmark = pytest.mark.gpu


def _call(X, W, y, N, H, V, chunk):
    ws = fl.workspace(N, H, V, fl.FLCE_BF16, chunk, device=DEV)
    dX = torch.empty_like(X)
    dW = torch.empty((V, H), dtype=torch.float32, device=DEV)
    loss = fl.flce_fwd_bwd(X, W, y, -100, chunk, dX, dW, ws)
    torch.cuda.synchronize()
    return loss, dX, dW


def test_profile_all_and_selected_classes():
    N, H, V, chunk = 600, 256, 3000, 256            # 3 chunks, the last one ragged
    inp = datagen.make_custom(N, H, V, "bf16", seed=77, ignore_frac=0.1)
    X, W, y = to_device(inp)
    r = oracle.flce(inp.X_f64(), inp.W_f64(), inp.labels)
    nchunks = -(-N // chunk)
    try:
        say(f"profile all classes: N={N} H={H} V={V} chunk={chunk}")
        fl.flce_profile_select(None)
        fl.flce_profile_enable(True)
        fl.flce_profile_read()
        loss, dX, dW = _call(X, W, y, N, H, V, chunk)
        prof = fl.flce_profile_read()
        check_loss(loss, r.loss, "bf16")
        check_grad(dX.double().cpu().numpy(), r.dX, "bf16", "dX")
        check_grad(dW.double().cpu().numpy(), r.dW, "bf16", "dW")
        for name in ("fwd_tile", "lse_combine", "dlogits", "dx_gemm", "pack_x"):
            assert prof[name][1] == nchunks, (name, prof[name])
        assert prof["label_check"][1] == 1 and prof["final"][1] == 1
        assert prof["dw_gemm"][1] >= nchunks
        for name, (ms, n) in prof.items():
            assert (n == 0 and ms == 0.0) or (n > 0 and ms > 0.0), (name, ms, n)

        say("profile dw_gemm only")
        fl.flce_profile_select(["dw_gemm"])
        fl.flce_profile_read()
        loss2, dX2, dW2 = _call(X, W, y, N, H, V, chunk)
        prof = fl.flce_profile_read()
        assert prof["dw_gemm"][1] >= nchunks and prof["dw_gemm"][0] > 0.0
        assert all(n == 0 for name, (ms, n) in prof.items() if name != "dw_gemm"), prof
        # the same call, bit for bit, whatever is timed
        assert loss2 == loss
        assert torch.equal(dX2.view(torch.int16), dX.view(torch.int16))
        assert torch.equal(dW2, dW)

        fl.flce_profile_enable(False)
        fl.flce_profile_read()
        _call(X, W, y, N, H, V, chunk)
        assert all(n == 0 for ms, n in fl.flce_profile_read().values())
    finally:
        fl.flce_profile_enable(False)
        fl.flce_profile_select(None)
