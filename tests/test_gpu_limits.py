"""GPU parity at the largest shapes the library accepts (V = 8,000,000 and
H = 2^20), with few tokens so that the fp64 oracle's full logits stay a few GB.

- V at its limit: 62,500 log-sum-exp partials per token, 31,250 vocabulary
  tiles per chunk, a dX split over millions of vocabulary rows, and about
  3.8 GiB of workspace (nearly all of it the chunk's bf16 logits, packed in
  row tiles of 256 tokens; W, 16 bytes per row, is read in place).
- H at its limit: one forward tile whose K loop runs 32,768 slices, dX over
  4,096 output tiles, dW over 8,192 column tiles of one vocabulary strip.
Both run two chunks, the second ragged.
"""
import numpy as np
import pytest
import torch

import datagen
import linear_cross_entropy_04_amd as fl
import oracle
from _gpu_common import check_grad, check_loss, run_gpu, say

II = -100
MAX_V = 8_000_000
MAX_H = 1 << 20


def _check(inp, chunk):
    say(f"case {inp.wl.name} N={inp.wl.N} H={inp.wl.H} V={inp.wl.V} seed={inp.seed} chunk={chunk}")
    need = fl.flce_workspace_bytes(inp.wl.N, inp.wl.H, inp.wl.V, fl.FLCE_BF16, chunk)
    say(f"    workspace {need / 2**30:.2f} GiB")
    g = run_gpu(inp, chunk, II)
    r = oracle.flce(inp.X_f64(), inp.W_f64(), inp.labels, II)
    check_loss(g["loss"], r.loss, "bf16")
    check_grad(g["dX"], r.dX, "bf16", "dX")
    check_grad(g["dW"], r.dW, "bf16", "dW")
    assert np.max(np.abs(g["row_lse"] - r.lse) / np.abs(r.lse)) <= 1e-3
    valid = inp.labels != II
    assert np.all(g["dX"][~valid] == 0.0)
    del g
    torch.cuda.empty_cache()


def test_limits_are_the_checked_ones():
    """One past each limit is refused before anything runs."""
    assert fl.flce_workspace_bytes(40, 8, MAX_V, fl.FLCE_BF16, 32) > 0
    assert fl.flce_workspace_bytes(40, 8, MAX_V + 1, fl.FLCE_BF16, 32) == 0
    assert fl.flce_workspace_bytes(40, MAX_H, 16, fl.FLCE_BF16, 32) > 0
    assert fl.flce_workspace_bytes(40, MAX_H + 8, 16, fl.FLCE_BF16, 32) == 0


@pytest.mark.gpu
def test_maximum_vocabulary():
    inp = datagen.make_custom(40, 8, MAX_V, "bf16", seed=41, ignore_frac=0.1, w_std=0.5)
    _check(inp, 32)


@pytest.mark.gpu
def test_maximum_hidden():
    inp = datagen.make_custom(40, MAX_H, 16, "bf16", seed=43, ignore_frac=0.1, w_std=0.002)
    _check(inp, 32)


@pytest.mark.gpu
@pytest.mark.parametrize("N,H,V,chunk", [(1, 8, 1, 0), (37, 8, 1, 16), (1, 8, 2, 1), (5, 8, 3, 2)])
def test_smallest_shapes(N, H, V, chunk):
    """The degenerate end: one class (softmax 1 everywhere, so loss, dX and
    dW are 0 up to fp32 rounding), the narrowest bf16 hidden size, a single
    token, and chunks of one or two tokens."""
    inp = datagen.make_custom(N, H, V, "bf16", seed=N * 10 + V, ignore_frac=0.0, w_std=0.5)
    say(f"case N={N} H={H} V={V} chunk={chunk}")
    g = run_gpu(inp, chunk, II)
    r = oracle.flce(inp.X_f64(), inp.W_f64(), inp.labels, II)
    if V == 1:
        # exact arithmetic gives 0; the log-sum-exp of one fp32 logit comes
        # out as z (1 + O(2^-24)) (exp2 of a fused z log2(e) - m log2(e)), so
        # the outputs are 0 up to a few fp32 roundings of the operands
        eps = 2.0 ** -20
        assert abs(g["loss"]) <= eps * max(np.max(np.abs(r.lse)), 1.0)
        assert np.max(np.abs(g["dX"])) <= eps * np.max(np.abs(inp.W_f64()))
        assert np.max(np.abs(g["dW"])) <= eps * np.max(np.abs(inp.X_f64()))
        assert np.allclose(g["row_lse"], r.lse, rtol=1e-3, atol=1e-3)
    else:
        check_loss(g["loss"], r.loss, "bf16")
        check_grad(g["dX"], r.dX, "bf16", "dX")
        check_grad(g["dW"], r.dW, "bf16", "dW")


@pytest.mark.gpu
@pytest.mark.timeout(600)
def test_weight_over_4_gib():
    """W of 4.4 GB (bf16, read in place by the forward and by dX) and dW of
    8.8 GB: the copies' buffer descriptors start at their slice and clamp
    their record counts, which differ for slices more than 4 GiB, between 2
    and 4 GiB, and less than 2 GiB from W's end.  Two chunks of 100 tokens.
    Checked against the fp64 oracle: the loss and every token's log-sum-exp
    over the whole vocabulary, sampled rows of dX and of dW (the latter at
    the vocabulary rows where the distance to W's end crosses 4 GiB and 2
    GiB)."""
    N, H, V, chunk = 200, 4096, 540_000, 100
    assert V * H * 2 > 4 << 30
    inp = datagen.make_custom(N, H, V, "bf16", seed=53, ignore_frac=0.1)
    say(f"case N={N} H={H} V={V} chunk={chunk}: W {V * H * 2 / 2**30:.2f} GiB")
    g = run_gpu(inp, chunk, II, poison=False, host_grads=False)
    X64, W64 = inp.X_f64(), inp.W_f64()
    loss, lse, rl, _ = oracle.loss_blocked(X64, W64, inp.labels, II, block=100)
    check_loss(g["loss"], loss, "bf16")
    assert np.max(np.abs(g["row_lse"] - lse) / np.abs(lse)) <= 1e-3
    assert np.max(np.abs(g["row_loss"] - rl)) <= 1e-3 * np.max(np.abs(lse))
    row_4g, row_2g = V - (4 << 30) // (2 * H), V - (2 << 30) // (2 * H)
    lab = inp.labels[inp.labels != II]
    vrows = datagen.sample_rows(V, 16, 59, must=(0, 1, row_4g - 1, row_4g, row_2g - 1, row_2g,
                                                 V - 1, int(lab[0]), int(lab[-1])))
    rows = datagen.sample_rows(N, 8, 61, must=(0, 99, 100, N - 1))
    dX_ref = oracle.dX_rows(X64, W64, inp.labels, rows, II)
    dW_ref = oracle.dW_rows(X64, W64, inp.labels, lse, vrows, II)
    dX_t, dW_t = g["dX_t"], g["dW_t"]
    check_grad(dX_t[torch.from_numpy(rows).to(dX_t.device)].double().cpu().numpy(), dX_ref, "bf16",
               "dX sampled rows")
    check_grad(dW_t[torch.from_numpy(vrows).to(dW_t.device)].double().cpu().numpy(), dW_ref, "bf16",
               "dW sampled rows")
    assert bool(torch.isfinite(dW_t).all()) and bool(torch.isfinite(dX_t.float()).all())
    del g, dX_t, dW_t
    torch.cuda.empty_cache()
