"""Calls that overlap in time: two host threads, each with its own stream,
workspace and outputs, run the fused loss at once (the binding's foreign
calls release the interpreter lock, and each call synchronises only its own
stream).  The header allows this for calls that do not share a workspace;
every output must equal, bit for bit, the same call made alone, and the
loss must still match the oracle."""
import threading

import numpy as np
import pytest
import torch

import datagen
import linear_cross_entropy_04_amd as fl
import oracle
from _gpu_common import DEV, check_loss, say, to_device

pytestmark = pytest.mark.gpu
II = -100


def _call(X, W, y, chunk, stream):
    N, H = X.shape
    V = W.shape[0]
    dt = fl.FLCE_BF16 if X.dtype == torch.bfloat16 else fl.FLCE_F32
    with torch.cuda.stream(stream):
        ws = fl.workspace(N, H, V, dt, chunk, device=DEV)
        dX = torch.empty_like(X)
        dW = torch.empty((V, H), dtype=torch.float32, device=DEV)
    stream.synchronize()
    loss = fl.flce_fwd_bwd(X, W, y, II, chunk, dX, dW, ws, stream=stream)
    return loss, dX, dW


def test_two_threads_two_streams():
    cases = [datagen.make_custom(1500, 512, 7000, "bf16", seed=81, ignore_frac=0.1),
             datagen.make_custom(900, 256, 12000, "bf16", seed=82, ignore_frac=0.1)]
    tensors = [to_device(inp) for inp in cases]
    chunks = [512, 256]
    streams = [torch.cuda.Stream(device=DEV) for _ in cases]
    alone = [_call(*t, c, s) for t, c, s in zip(tensors, chunks, streams)]
    torch.cuda.synchronize()
    for rep in range(3):
        results = [None, None]
        errors = []

        def work(i):
            try:
                results[i] = _call(*tensors[i], chunks[i], streams[i])
            except Exception as e:          # reported after the join
                errors.append(e)

        threads = [threading.Thread(target=work, args=(i,)) for i in range(2)]
        for t in threads:
            t.start()
        for t in threads:
            t.join(timeout=120)
        assert not any(t.is_alive() for t in threads), "a call did not return"
        assert not errors, errors
        torch.cuda.synchronize()
        for i in range(2):
            say(f"  repetition {rep} case {i}: loss {results[i][0]:.6f} alone {alone[i][0]:.6f}")
            assert results[i][0] == alone[i][0]
            assert torch.equal(results[i][1], alone[i][1])
            assert torch.equal(results[i][2], alone[i][2])
    for inp, (loss, _, _) in zip(cases, alone):
        r = oracle.flce(inp.X_f64(), inp.W_f64(), inp.labels, II)
        check_loss(loss, r.loss, "bf16")
