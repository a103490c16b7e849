"""GPU parity at one GPU's share of the Llama-3-8B head sharded over 8 GPUs
(the shapes bench.py --share measures): the token share (1024 tokens, the
whole head: one chunk) element by element against the oracle's full
definition, and the vocabulary share (8192 tokens against V/8 = 16032 rows,
labels reduced modulo the shard) with the exact loss and sampled rows.
The shares come from datagen.share_of."""
import numpy as np
import pytest
import torch

import datagen
import linear_cross_entropy_04_amd as fl
import oracle
from _gpu_common import DEV, check_grad, check_loss, run_gpu, say

pytestmark = pytest.mark.gpu


def test_token_share_full_parity():
    inp = datagen.share_of(datagen.make(1), "dp8")
    assert inp.wl.N == 1024 and inp.wl.V == 128256
    out = run_gpu(inp, 1024)
    r = oracle.flce(inp.X_f64(), inp.W_f64(), inp.labels)
    check_loss(out["loss"], r.loss, "bf16")
    check_grad(out["dX"], r.dX, "bf16", "dX")
    check_grad(out["dW"], r.dW, "bf16", "dW")


def test_vocab_share_sampled_parity():
    inp = datagen.share_of(datagen.make(1), "tp8")
    assert inp.wl.N == 8192 and inp.wl.V == 16032
    out = run_gpu(inp, 1024, host_grads=False)
    X64, W64 = inp.X_f64(), inp.W_f64()
    loss, lse, rl, nv = oracle.loss_blocked(X64, W64, inp.labels, block=1024)
    check_loss(out["loss"], loss, "bf16")
    assert np.max(np.abs(out["row_lse"] - lse)) <= 1e-3 * np.max(np.abs(lse))
    rows = datagen.sample_rows(8192, 16, 9, must=(0, 8191))
    vrows = datagen.sample_rows(16032, 16, 10, must=(0, 16031))
    check_grad(out["dX_t"][torch.from_numpy(rows).to(DEV)].double().cpu().numpy(),
               oracle.dX_rows(X64, W64, inp.labels, rows), "bf16", "dX sampled rows")
    check_grad(out["dW_t"][torch.from_numpy(vrows).to(DEV)].double().cpu().numpy(),
               oracle.dW_rows(X64, W64, inp.labels, lse, vrows), "bf16", "dW sampled rows")
