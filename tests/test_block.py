"""GPU parity of the attention blocks (rehyat_block_fwd, rehyat_stack_fwd)
against the fp64 block oracle on identical seeded inputs and weights.

A block is the attention part of a DiT block, T_l(x) = f_l(A_l(x) + x)
(ReHyAt §3.1, first display equation) with its bf16 MFMA projections; the
hybrid attention replaces full softmax attention in the converted blocks (15,
20 or 25 of 30 in Wan2.1 1.3B, §4.3).  The check is on A(x) = out - x at the
attention bar (rel-L2 <= 1e-2) and on out itself (max-abs <= 3e-2): q, k, v,
the attention output and out are bf16, so their roundings are the error
budget.  The output projection's gain (4 / sqrt(C) per weight) makes A(x)
about half the size of x, so that the rounding of the residual in out does not
dominate A's error, while out stays below 8 in magnitude (its bf16 rounding,
at most 2^-6, stays inside the max-abs bar)."""
import numpy as np
import pytest
import torch

import linear_attention_video_rehyat_amd as rh
from linear_attention_video_rehyat_amd import inputs
from oracle import oracle as O
from tests.parity_util import TOL_BF16_ABS, TOL_BF16_REL, rel_l2, sample_rows, sync, to64

pytestmark = pytest.mark.gpu


def _weights(seed_id, layer, C, gain):
    w = inputs.make_block_weights(seed_id, layer, C, gain)
    return rh.BlockWeights(*(t.cuda() for t in w)), w


def _check(out, x, ref_a, rows=None, what=""):
    o = to64(out) if rows is None else to64(out[:, torch.from_numpy(rows).cuda()])
    x64 = to64(x) if rows is None else to64(x[:, torch.from_numpy(rows)])
    r = rel_l2(o - x64, ref_a)
    a = float(np.abs(o - (x64 + ref_a)).max())
    assert r <= TOL_BF16_REL and a <= TOL_BF16_ABS, f"{what}: A(x) rel-L2 {r:.3e}, out max-abs {a:.3e}"
    return r, a


# the last geometry (width 128, head_dim 32) takes the projections' 128 x 128 tiles
# with 32-feature LDS stages; the others the 256 x 256 tiles with 64-feature stages
SMALL = [(1, 2, 128, 5, 40, 2, 1), (2, 4, 64, 4, 37, 1, 1), (1, 12, 128, 3, 50, 3, 1), (1, 4, 32, 3, 20, 1, 1)]


@pytest.mark.parametrize("geom", SMALL, ids=lambda g: "B{}H{}d{}F{}HW{}Tc{}To{}".format(*g))
@pytest.mark.parametrize("mode", ["elu1", "poly2", "dense"])
def test_block_small_every_element(geom, mode):
    B, H, d, F, HW, Tc, To = geom
    C = H * d
    x = inputs.make_block_input(900 + F, B, F * HW, C)
    wg, w = _weights(900 + F, 0, C, 4.0)
    hybrid = mode != "dense"
    phi = mode if hybrid else "none"
    out = rh.block_fwd(x.cuda(), wg, F, HW, H, hybrid, Tc, To, phi)
    sync()
    ref_a = O.block_attention(x, *w, H, F, HW, hybrid, Tc, To, phi)
    _check(out, x, ref_a, what=f"block {geom} {mode}")


@pytest.mark.parametrize("hybrid", [True, False])
def test_block_wan_shape_sampled(hybrid):
    """One Wan2.1-1.3B-shaped block: 21 x 1560 tokens, 12 heads of 128 (C =
    1536), T_c = 3, T_o = 1, elu+1 (or full softmax); every row of q, k, v
    formed in fp64, sampled output rows compared."""
    F, HW, H, d = 21, 1560, 12, 128
    C = H * d
    x = inputs.make_block_input(950, 1, F * HW, C)
    wg, w = _weights(950, 0, C, 4.0)
    out = rh.block_fwd(x.cuda(), wg, F, HW, H, hybrid, 3, 1, "elu1")
    sync()
    rows = sample_rows(F, HW, n_random=48, seed=9)
    ref_a = O.block_attention(x, *w, H, F, HW, hybrid, 3, 1, "elu1", rows=rows)
    _check(out, x, ref_a, rows, f"wan block hybrid={hybrid}")


def test_stack_mixed_blocks_every_element():
    """Four blocks, two hybrid and two with full softmax attention, against the
    fp64 stack."""
    B, H, d, F, HW, Tc, To = 1, 4, 64, 5, 30, 2, 1
    C = H * d
    x = inputs.make_block_input(960, B, F * HW, C)
    pairs = [_weights(960, l, C, 1.0) for l in range(4)]
    hyb = [True, False, True, False]
    out = rh.stack_fwd(x.cuda(), [p[0] for p in pairs], hyb, F, HW, H, Tc, To, "elu1")
    sync()
    ref = O.stack_forward(x, [p[1] for p in pairs], hyb, H, F, HW, Tc, To, "elu1")
    r = rel_l2(to64(out) - to64(x), ref - to64(x))
    assert r <= TOL_BF16_REL, f"stack: x_L - x rel-L2 {r:.3e}"
    assert np.abs(to64(out) - ref).max() <= TOL_BF16_ABS


def test_stack_equals_chain_of_blocks_bitwise():
    B, H, d, F, HW, Tc, To = 2, 2, 128, 4, 33, 1, 1
    C = H * d
    x = inputs.make_block_input(970, B, F * HW, C).cuda()
    ws = [_weights(970, l, C, 1.0)[0] for l in range(3)]
    hyb = [True, True, False]
    got = rh.stack_fwd(x, ws, hyb, F, HW, H, Tc, To, "poly2")
    y = x
    for w, hy in zip(ws, hyb):
        y = rh.block_fwd(y, w, F, HW, H, hy, Tc, To, "poly2")
    sync()
    assert torch.equal(got, y)


def test_converted_block_placement():
    """25 of 30 blocks converted (the pages' main configuration): the flags
    select the attention per block; a stack with every block dense equals one
    with no linear branch anywhere."""
    flags = inputs.converted_blocks(25)
    assert len(flags) == 30 and sum(flags) == 25 and flags[:25] == [True] * 25
    B, H, d, F, HW = 1, 2, 64, 4, 20
    C = H * d
    x = inputs.make_block_input(980, B, F * HW, C).cuda()
    ws = [_weights(980, l, C, 1.0)[0] for l in range(3)]
    dense = rh.stack_fwd(x, ws, [False] * 3, F, HW, H, 1, 1, "elu1")
    nolin = rh.stack_fwd(x, ws, [True] * 3, F, HW, H, F, 0, "none")
    sync()
    assert torch.equal(dense, nolin)
