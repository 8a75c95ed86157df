"""Pins of the oracle's process-pool unit driver (CPU).

``oracle.parallel.unit_step`` runs the oracle's row functions for one
(batch, KV head) unit on worker processes (row chunks of 256 per task, dk / dv
summed over per-worker slots).  Its results must equal what the whole-layer
oracle (``oracle.forward`` / ``oracle.backward``, themselves pinned by the
other oracle tests) gives for that unit, in every mode: the selection, both
streams, their log-sum-exps, delta and the gradients.  The unit's rows span
several chunks and a ragged tail, and the loss weights and the layer's element
count M are not the defaults, so a dropped chunk, a worker slot summed twice or
a loss normalised over the unit instead of the layer fails here.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import parallel
from oracle import DUAL_ACTIVE_FULL, DUAL_ACTIVE_SPARSE, FULL_ONLY, SPARSE_ONLY

B, HQ, HKV, N, D, BLOCK, K = 1, 4, 2, 600, 8, 8, 3
G = HQ // HKV
UNIT_C = 1                       # the second KV head: query heads 2 and 3
W_S, W_C = 0.7, 1.3


@pytest.fixture(scope="module")
def layer():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((B, HQ, N, D))
    k = rng.standard_normal((B, HKV, N, D))
    v = rng.standard_normal((B, HKV, N, D))
    g = rng.standard_normal((B, HQ, N, D))
    sel, _ = oracle.select_blocks(q, k, BLOCK, K, G)
    return q, k, v, g, sel


@pytest.mark.parametrize("mode", [DUAL_ACTIVE_FULL, DUAL_ACTIVE_SPARSE, FULL_ONLY, SPARSE_ONLY])
def test_unit_step_equals_whole_layer_oracle(layer, mode):
    q, k, v, g, sel = layer
    scale = 1.0 / math.sqrt(D)
    hs = slice(UNIT_C * G, (UNIT_C + 1) * G)
    fwd = oracle.forward(q, k, v, sel, BLOCK, scale, G, mode)
    dq, dk, dv = oracle.backward(q, k, v, sel, BLOCK, scale, G, mode, g, W_S, W_C, fwd=fwd)
    res = parallel.unit_step(q[0, hs], k[0, UNIT_C], v[0, UNIT_C], BLOCK, K, scale, mode, dout_u=g[0, hs],
                             w_sparsity=W_S, w_commit=W_C, M=q.size, workers=2)
    assert res["workers"] == 2
    if mode != FULL_ONLY:
        np.testing.assert_array_equal(res["sel"], sel[0, hs])
    for key in ("h_full", "lse_full", "h_sparse", "lse_sparse", "delta"):
        if key in fwd:
            np.testing.assert_allclose(res[key], fwd[key][0, hs], rtol=1e-12, atol=1e-12, err_msg=key)
        else:
            assert key not in res
    np.testing.assert_allclose(res["dq"], dq[0, hs], rtol=1e-10, atol=1e-12, err_msg="dq")
    np.testing.assert_allclose(res["dk"], dk[0, UNIT_C], rtol=1e-10, atol=1e-12, err_msg="dk")
    np.testing.assert_allclose(res["dv"], dv[0, UNIT_C], rtol=1e-10, atol=1e-12, err_msg="dv")


def test_unit_step_given_selection(layer):
    """With the selection passed in (as the GPU's is at full size) the unit's
    streams follow that selection, not the oracle's own."""
    q, k, v, g, sel = layer
    scale = 1.0 / math.sqrt(D)
    hs = slice(UNIT_C * G, (UNIT_C + 1) * G)
    other = sel.copy()
    other[..., 1:] = -1                 # the lowest selected block only
    fwd = oracle.forward(q, k, v, other, BLOCK, scale, G, DUAL_ACTIVE_SPARSE)
    res = parallel.unit_step(q[0, hs], k[0, UNIT_C], v[0, UNIT_C], BLOCK, K, scale, DUAL_ACTIVE_SPARSE,
                             sel_u=other[0, hs], backward=False, workers=2)
    assert "sel" not in res and "dq" not in res
    np.testing.assert_allclose(res["h_sparse"], fwd["h_sparse"][0, hs], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(res["delta"], fwd["delta"][0, hs], rtol=1e-12, atol=1e-12)
