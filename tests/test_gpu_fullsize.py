"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times, on outputs the fp64 oracle can compute one by one:

* the mean loss and every token's log-sum-exp and loss (the oracle runs the
  full forward in row blocks, every row complete over the vocabulary);
* on the Llama-3-8B head, the headline workload, every element of dX and dW
  against the oracle's full fp64 computation (about 30 s of host BLAS and
  35 GB of host memory);
* on the other workloads, sampled rows of dX (each needs only its own logits
  row) and of dW (each needs one logits column over all tokens and the
  oracle's log-sum-exp of every token);
* ignored tokens' dX rows are exactly zero; sum_v dW[v, :] is ~0.

Workloads: Llama-3-8B head (8192 x 4096 x 128256, chunk 1024), Qwen2-7B head
(16384 x 3584 x 152064, chunk 2048), long-context Llama head (16384 tokens,
chunks 512 / 1024 / 4096), large-vocabulary head (8192 x 2304 x 256000, the
planned chunk and 2048).
"""
import time

import numpy as np
import pytest
import torch

import datagen
import oracle
from _gpu_common import check_grad, check_loss, run_gpu, say, to_device

pytestmark = pytest.mark.gpu

_INPUTS = {}
_ORACLE = {}


def _inputs(wid):
    if wid not in _INPUTS:
        _INPUTS.clear()
        _ORACLE.clear()
        t0 = time.time()
        _INPUTS[wid] = datagen.make(wid)
        say(f"workload {wid} {_INPUTS[wid].wl.name}: drawn in {time.time() - t0:.1f}s")
    return _INPUTS[wid]


# workloads whose dX and dW are compared element by element
FULL_GRADS = (1,)


def _oracle(wid):
    if wid in _ORACLE:
        return _ORACLE[wid]
    inp = _inputs(wid)
    X64, W64 = inp.X_f64(), inp.W_f64()
    if wid in FULL_GRADS:
        t0 = time.time()
        r = oracle.flce(X64, W64, inp.labels)
        say(f"  oracle loss, dX and dW over all {inp.wl.N} tokens: {time.time() - t0:.1f}s")
        _ORACLE[wid] = dict(loss=r.loss, lse=r.lse, row_loss=r.row_loss, dX=r.dX, dW=r.dW,
                            ign=np.flatnonzero(inp.labels == -100), full=True)
        return _ORACLE[wid]
    t0 = time.time()
    loss, lse, rl, nv = oracle.loss_blocked(X64, W64, inp.labels, block=512)
    say(f"  oracle forward over all {inp.wl.N} tokens: {time.time() - t0:.1f}s")
    N, V = inp.wl.N, inp.wl.V
    ign = np.flatnonzero(inp.labels == -100)
    rows = datagen.sample_rows(N, 12, 100 + wid, must=(0, N - 1) + tuple(ign[:2]))
    lab = inp.labels[inp.labels >= 0]
    vrows = datagen.sample_rows(V, 12, 200 + wid, must=(0, 1, V - 1, int(lab[0]), int(lab[-1])))
    t0 = time.time()
    dX = oracle.dX_rows(X64, W64, inp.labels, rows)
    dW = oracle.dW_rows(X64, W64, inp.labels, lse, vrows)
    say(f"  oracle sampled dX/dW rows: {time.time() - t0:.1f}s")
    _ORACLE[wid] = dict(loss=loss, lse=lse, row_loss=rl, rows=rows, vrows=vrows, dX=dX, dW=dW,
                        ign=ign, full=False)
    return _ORACLE[wid]


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("wid,chunk", [(1, 1024), (2, 2048), (3, 512), (3, 1024), (3, 4096),
                                       (4, 0), (4, 2048)])
def test_fullsize(wid, chunk):
    inp = _inputs(wid)
    say(f"full-size workload {wid} ({inp.wl.name}) chunk={chunk}")
    g = run_gpu(inp, chunk, poison=False, host_grads=False)
    say(f"  gpu call took {g['seconds']:.2f}s")
    ref = _oracle(wid)
    check_loss(g["loss"], ref["loss"], "bf16")
    assert np.max(np.abs(g["row_lse"] - ref["lse"]) / np.abs(ref["lse"])) <= 1e-3
    assert np.max(np.abs(g["row_loss"] - ref["row_loss"])) <= 1e-3 * np.max(np.abs(ref["lse"]))
    dX_t, dW_t = g["dX_t"], g["dW_t"]
    if ref["full"]:
        check_grad(dX_t.float().cpu().numpy(), ref["dX"], "bf16", "dX (every element)")
        check_grad(dW_t.cpu().numpy(), ref["dW"], "bf16", "dW (every element)")
    else:
        rows = torch.from_numpy(ref["rows"]).to(dX_t.device)
        vrows = torch.from_numpy(ref["vrows"]).to(dX_t.device)
        check_grad(dX_t[rows].double().cpu().numpy(), ref["dX"], "bf16", "dX sampled rows")
        check_grad(dW_t[vrows].double().cpu().numpy(), ref["dW"], "bf16", "dW sampled rows")
    ign = torch.from_numpy(ref["ign"]).to(dX_t.device)
    assert bool((dX_t[ign] == 0).all())
    assert bool(torch.isfinite(dW_t).all()) and bool(torch.isfinite(dX_t.float()).all())
    # Every dlogits row sums to 0, so the columns of dW sum to 0 up to the
    # rounding of G to bf16 (relative 2^-9 per element): a row's sum is then at
    # most 2^-9 sum_v |G| <= 2^-8 / N_valid, hence
    #   |sum_v dW[v, h]| <= 2^-8 / N_valid * sum_{valid t} |X[t, h]|
    # (plus fp32 accumulation, far below it).
    col = dW_t.double().sum(dim=0).abs().cpu().numpy()
    valid = inp.labels != -100
    bound = 2.0 ** -8 / valid.sum() * np.abs(inp.X_f64()[valid]).sum(axis=0)
    assert np.all(col <= bound + 1e-6 * dW_t.abs().max().item())
    del g
    torch.cuda.empty_cache()
