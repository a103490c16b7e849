"""GPU parity of libflce against the fp64 oracle where the logits are large.

The bf16 path keeps a chunk's logits in bf16 between the forward and the
dlogits rewrite.  Both cases below put logits where bf16's spacing is coarse
(0.5 to 2 near |z| = 100 .. 500), so a rewrite that exponentiated rounded
logits would miss the softmax by tens of percent; the library stores each
logit relative to its token's maximum over 128 vocabulary ids, and the
gradients must meet the usual bounds.
"""
import numpy as np
import pytest

import datagen
import oracle
from _gpu_common import check_grad, check_loss, run_gpu, say

pytestmark = pytest.mark.gpu
II = -100


def _check(inp, chunk, offset_col=None):
    """Loss, lse and gradients against the oracle.  offset_col: a hidden unit
    whose W column is one common value c0 for every vocabulary row (see
    test_common_offset); dX's column there is checked separately."""
    say(f"case {inp.wl.name} N={inp.wl.N} H={inp.wl.H} V={inp.wl.V} seed={inp.seed} chunk={chunk}")
    g = run_gpu(inp, chunk, II)
    r = oracle.flce(inp.X_f64(), inp.W_f64(), inp.labels, II)
    say(f"    logits: max |lse| = {np.max(np.abs(r.lse)):.1f}")
    check_loss(g["loss"], r.loss, "bf16")
    check_grad(g["dW"], r.dW, "bf16", "dW")
    assert np.max(np.abs(g["row_lse"] - r.lse) / np.abs(r.lse)) <= 1e-3
    valid = inp.labels != II
    assert np.all(g["dX"][~valid] == 0.0)
    if offset_col is None:
        check_grad(g["dX"], r.dX, "bf16", "dX")
    else:
        keep = np.arange(inp.wl.H) != offset_col
        check_grad(g["dX"][:, keep], r.dX[:, keep], "bf16", "dX (other columns)")
        # dX[:, col] = c0 * sum_v G_iv, zero in exact arithmetic; bf16 storage
        # of G (unit roundoff 2^-8) leaves at most c0 2^-8 sum_v |G_iv| per
        # row, and sum_v |G_iv| <= 2 / N_valid
        c0 = float(np.max(np.abs(inp.W_f64()[:, offset_col])))
        bound = c0 * 2.0 ** -8 * 2.0 / max(int(valid.sum()), 1)
        err = np.max(np.abs(g["dX"][:, offset_col] - r.dX[:, offset_col]))
        say(f"    dX column {offset_col}: max|err| = {err:.3e} (bound {bound:.3e})")
        assert err <= bound
    return r


@pytest.mark.parametrize("N,H,V,chunk", [(600, 512, 3000, 256), (333, 256, 1100, 128)])
def test_peaky_head(N, H, V, chunk):
    """W ~ N(0, 2^2): logits spread about 2 sqrt(H) (45 at H = 512), the top
    ones near 150-200, and the softmax of a token is close to one-hot."""
    inp = datagen.make_custom(N, H, V, "bf16", seed=N + 7, ignore_frac=0.1, w_std=2.0)
    r = _check(inp, chunk)
    assert np.max(r.lse) > 100.0


@pytest.mark.parametrize("N,H,V,chunk", [(600, 512, 3000, 256), (300, 128, 700, 1000)])
def test_common_offset(N, H, V, chunk):
    """Every token's logits share an offset of 400: hidden unit 0 of X is 8
    and column 0 of W is 50 (the drawn values, |w| << 0.125, round away), so
    z = 400 + (the other units' contribution, spread about 0.02 sqrt(H)).
    Only differences of logits enter the softmax; rounded to bf16 near 400
    (spacing 2) they would be lost.

    A linear head gives every token a common offset only through a column of
    W shared by all vocabulary rows, and then dX's column 0 is 50 sum_v G_iv,
    a sum that cancels exactly; there the bf16 rounding of G is amplified
    50 / 0.02 times against the other columns, whatever the logits' storage,
    so that column is held to the rounding bound instead."""
    inp = datagen.make_custom(N, H, V, "bf16", seed=N + 11, ignore_frac=0.1)
    X = datagen.bf16_bits_to_f32(inp.X).copy()
    W = datagen.bf16_bits_to_f32(inp.W).copy()
    X[:, 0] = 8.0
    W[:, 0] += 50.0
    inp.X = datagen.f32_to_bf16_bits(X)
    inp.W = datagen.f32_to_bf16_bits(W)
    assert np.all(datagen.bf16_bits_to_f32(inp.W)[:, 0] == 50.0)
    r = _check(inp, chunk, offset_col=0)
    assert np.min(r.lse) > 350.0
