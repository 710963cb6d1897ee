"""CPU pins of the fp64 attention-block oracle (oracle.block_attention,
block_forward, stack_forward): the attention part of a DiT block, T_l(x) =
f_l(A_l(x) + x) (ReHyAt §3.1, first display equation), with its input and
output projections.

* A block with full softmax attention equals torch's multi-head attention
  (torch.nn.functional.multi_head_attention_forward, fp64: the same packed
  q/k/v projection, 1/sqrt(d) scaling and output projection) plus the
  residual -- a library routine that shares nothing with the oracle.
* A hybrid block whose chunk spans the clip (T_c >= F: no linear set, §3.3)
  equals the same, for every feature map.
* With identity projections and zero biases the block is x plus the
  definition form on the heads of x (checks the split into heads and their
  concatenation).
* Row subsets equal the full output; a stack of dense blocks equals torch's
  attention applied block after block."""
import numpy as np
import pytest
import torch

from oracle import oracle as O

pytestmark = []


def _weights(rng, C, gain=1.0):
    return (rng.standard_normal((3 * C, C)) / np.sqrt(C), 0.1 * rng.standard_normal(3 * C),
            gain * rng.standard_normal((C, C)) / np.sqrt(C), 0.1 * rng.standard_normal(C))


def _torch_mha(x, w, heads):
    w_qkv, b_qkv, w_o, b_o = (torch.from_numpy(np.asarray(a, np.float64)) for a in w)
    xt = torch.from_numpy(x).transpose(0, 1)  # [N, B, C]
    C = xt.shape[-1]
    y, _ = torch.nn.functional.multi_head_attention_forward(
        xt, xt, xt, C, heads, w_qkv, b_qkv, None, None, False, 0.0, w_o, b_o, training=False,
        need_weights=False)
    return y.transpose(0, 1).numpy()


@pytest.mark.parametrize("B,F,HW,heads,d", [(1, 4, 6, 2, 8), (2, 3, 5, 4, 4)])
def test_dense_block_is_torch_mha(B, F, HW, heads, d):
    rng = np.random.default_rng(11 + B)
    C = heads * d
    x = rng.standard_normal((B, F * HW, C))
    w = _weights(rng, C)
    ref = x + _torch_mha(x, w, heads)
    got = O.block_forward(x, *w, heads, F, HW, hybrid=False)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("phi", ["elu1", "poly2", "none"])
def test_hybrid_block_one_chunk_is_torch_mha(phi):
    rng = np.random.default_rng(21)
    B, F, HW, heads, d = 1, 4, 5, 2, 8
    C = heads * d
    x = rng.standard_normal((B, F * HW, C))
    w = _weights(rng, C)
    ref = x + _torch_mha(x, w, heads)
    for Tc, To in ((F, 0), (F + 2, 1)):
        got = O.block_forward(x, *w, heads, F, HW, hybrid=True, chunk_frames=Tc, overlap_frames=To, phi=phi)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_identity_projections_give_definition_on_heads():
    rng = np.random.default_rng(31)
    B, F, HW, heads, d = 2, 5, 4, 3, 4
    C = heads * d
    x = rng.standard_normal((B, F * HW, C))
    eye = np.eye(C)
    w = (np.concatenate([eye, eye, eye]), np.zeros(3 * C), eye, np.zeros(C))
    xh = x.reshape(B, F * HW, heads, d).transpose(0, 2, 1, 3)
    y = O.definition(xh, xh / np.sqrt(d), xh, F, HW, 2, 1, "elu1")
    ref = x + y.transpose(0, 2, 1, 3).reshape(B, F * HW, C)
    got = O.block_forward(x, *w, heads, F, HW, hybrid=True, chunk_frames=2, overlap_frames=1, phi="elu1")
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-13)


def test_rows_subset_and_stack():
    rng = np.random.default_rng(41)
    B, F, HW, heads, d = 1, 6, 3, 2, 4
    C = heads * d
    x = rng.standard_normal((B, F * HW, C))
    w = _weights(rng, C)
    full = O.block_forward(x, *w, heads, F, HW, hybrid=True, chunk_frames=2, overlap_frames=1)
    rows = np.array([0, 5, 11, 17])
    part = O.block_forward(x, *w, heads, F, HW, hybrid=True, chunk_frames=2, overlap_frames=1, rows=rows)
    np.testing.assert_allclose(part, full[:, rows], rtol=0, atol=1e-13)
    ws = [_weights(rng, C, 0.5) for _ in range(3)]
    ref = x
    for wl in ws:
        ref = ref + _torch_mha(ref, wl, heads)
    got = O.stack_forward(x, ws, [False] * 3, heads, F, HW)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-11)
    # hybrid and dense blocks differ once a chunk has a linear set
    mixed = O.stack_forward(x, ws, [True, False, True], heads, F, HW, 2, 1, "elu1")
    assert np.abs(mixed - got).max() > 1e-3
