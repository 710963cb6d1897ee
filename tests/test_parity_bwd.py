"""GPU parity of the backward (training direction, ReHyAt §3.4) against the
fp64 oracle.

rehyat_attn_fwd_lse returns the output and lse = ln(n^S + n^L) per query;
rehyat_attn_bwd returns dq, dk, dv of sum(dout * out), for the recurrent
(§3.3) and the bidirectional (§3.2 with overlap) partitions.  The oracle's gradients (oracle.backward) come from fp64 reverse
mode of the matrix form and are pinned on the CPU by central differences of the
definition form.  fp32 workloads: rel-L2 <= 1e-5 per gradient.  bf16 workloads:
rel-L2 <= 1e-2 per gradient and max-abs <= 3e-2 of the largest reference entry
(the output bar, stated relative to the gradient's scale, which is not O(1)).
"""
import numpy as np
import pytest
import torch

import linear_attention_video_rehyat_amd as rh
from linear_attention_video_rehyat_amd import inputs
from oracle import oracle as O
from tests.parity_util import gpu, rel_l2, sync, to64

pytestmark = pytest.mark.gpu


def _run(w, phi, Tc=None, To=None, causal=True):
    Tc = w.chunk_frames if Tc is None else Tc
    To = w.overlap_frames if To is None else To
    q, k, v = inputs.make_qkv(w)
    dy = inputs.make_dout(w)
    qg, kg, vg, dyg = gpu(q, k, v, dy)
    out, lse = rh.attn_fwd_lse(qg, kg, vg, w.frames, w.tokens_per_frame, Tc, To, phi, causal=causal)
    grads = rh.attn_bwd(qg, kg, vg, out, lse, dyg, w.frames, w.tokens_per_frame, Tc, To, phi, causal=causal)
    sync()
    ref = O.backward(to64(q), to64(k), to64(v), to64(dy), w.tokens_per_frame, Tc, To, phi, causal=causal)
    return (q, k, v, dy), out, lse, grads, ref, Tc, To


def _check(grads, ref, tol_rel, tol_abs, what):
    for name, g, r in zip(("dq", "dk", "dv"), grads, ref):
        got = to64(g)
        e = rel_l2(got, r)
        a = float(np.abs(got - r).max() / max(np.abs(r).max(), 1e-30))
        assert e <= tol_rel and a <= tol_abs, f"{what} {name}: rel-L2 {e:.3e}, max-abs/scale {a:.3e}"


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("phi", ["elu1", "poly2", "none"])
def test_tiny_f32(phi, causal):
    w = inputs.WORKLOADS["tiny_f4x8x8"]
    _, _, _, grads, ref, _, _ = _run(w, phi, causal=causal)
    _check(grads, ref, 1e-5, 1e-4, f"tiny fp32 {phi} causal={causal}")


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("Tc,To", [(1, 0), (2, 1), (3, 4), (2, 2), (3, 5)])
def test_f32_geometries(Tc, To, causal):
    w = inputs.custom(1, 2, 7, 23, 16, Tc, To, dtype="f32", seed_id=1100 + 10 * Tc + To)
    for phi in ("elu1", "poly2"):
        _, _, _, grads, ref, _, _ = _run(w, phi, causal=causal)
        _check(grads, ref, 1e-5, 1e-4, f"fp32 Tc{Tc} To{To} {phi} causal={causal}")


SMALL = [
    (1, 2, 6, 100, 128, 3, 1),
    (1, 1, 5, 97, 128, 1, 1),
    (1, 1, 7, 60, 128, 2, 3),     # T_o > T_c
    (2, 1, 6, 33, 64, 3, 0),
    (1, 2, 4, 45, 32, 1, 2),
    (1, 1, 3, 40, 128, 5, 1),     # one chunk: plain softmax attention
    (1, 2, 5, 128, 128, 1, 1),    # windows of whole key tiles: the last tile is a full one
]


@pytest.mark.parametrize("geom", SMALL, ids=lambda g: "B{}H{}F{}HW{}d{}Tc{}To{}".format(*g))
@pytest.mark.parametrize("phi", ["elu1", "poly2", "none"])
def test_bf16_small(geom, phi):
    B, H, F, HW, d, Tc, To = geom
    w = inputs.custom(B, H, F, HW, d, Tc, To, dtype="bf16", seed_id=1200 + F * 7 + d)
    _, _, _, grads, ref, _, _ = _run(w, phi)
    _check(grads, ref, 1e-2, 3e-2, f"bf16 {geom} {phi}")


@pytest.mark.parametrize("geom", SMALL + [(1, 1, 8, 50, 128, 2, 4), (1, 1, 9, 40, 64, 3, 5)],
                         ids=lambda g: "B{}H{}F{}HW{}d{}Tc{}To{}".format(*g))
@pytest.mark.parametrize("phi", ["elu1", "poly2"])
def test_bf16_small_bidirectional(geom, phi):
    B, H, F, HW, d, Tc, To = geom
    w = inputs.custom(B, H, F, HW, d, Tc, To, dtype="bf16", seed_id=1250 + F * 7 + d)
    _, _, _, grads, ref, _, _ = _run(w, phi, causal=False)
    _check(grads, ref, 1e-2, 3e-2, f"bf16 bidirectional {geom} {phi}")


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_lse_matches_oracle(dtype, causal):
    d = 16 if dtype == "f32" else 128
    w = inputs.custom(1, 2, 6, 50, d, 2, 1, dtype=dtype, seed_id=1300)
    q, k, v = inputs.make_qkv(w)
    out, lse = rh.attn_fwd_lse(*gpu(q, k, v), w.frames, w.tokens_per_frame, 2, 1, "elu1", causal=causal)
    y = rh.attn_fwd(*gpu(q, k, v), w.frames, w.tokens_per_frame, 2, 1, "elu1", causal=causal)
    sync()
    assert torch.equal(out, y)
    _, parts = O.definition(to64(q), to64(k), to64(v), w.frames, w.tokens_per_frame, 2, 1, "elu1", partials=True,
                            causal=causal)
    ref = np.log(np.exp(parts["m"]) * parts["nt"] + parts["nL"])
    np.testing.assert_allclose(to64(lse), ref, rtol=0, atol=1e-5 if dtype == "f32" else 2e-4)


def test_bf16_deterministic_and_dv_sum():
    """Bitwise repeatable; sum_j dv_j = sum_i dy_i (each output is a convex
    combination of values) at the Wan2.1-1.3B shape."""
    w = inputs.WORKLOADS["wan_21x30x52"]
    q, k, v = gpu(*inputs.make_qkv(w))
    dy = inputs.make_dout(w).cuda()
    out, lse = rh.attn_fwd_lse(q, k, v, w.frames, w.tokens_per_frame, 3, 1, "elu1")
    g1 = rh.attn_bwd(q, k, v, out, lse, dy, w.frames, w.tokens_per_frame, 3, 1, "elu1")
    g2 = rh.attn_bwd(q, k, v, out, lse, dy, w.frames, w.tokens_per_frame, 3, 1, "elu1")
    sync()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    for g in g1:
        assert torch.isfinite(g.float()).all()
    lhs = g1[2].double().sum(dim=2)
    rhs = dy.double().sum(dim=2)
    assert rel_l2(lhs.cpu().numpy(), rhs.cpu().numpy()) <= 1e-2


def test_bad_arguments():
    w = inputs.custom(1, 1, 4, 16, 32, 2, 1, dtype="bf16", seed_id=1400)
    q, k, v = gpu(*inputs.make_qkv(w))
    out, lse = rh.attn_fwd_lse(q, k, v, 4, 16, 2, 1, "elu1")
    with pytest.raises(rh.RehyatError):
        rh.attn_bwd(q, k, v, out, lse, out, 4, 16, 2, 1, "elu1", grads=(q, k, v))   # gradients alias inputs
    with pytest.raises(rh.RehyatError):
        rh.attn_bwd(q, k, v, out, lse[:, :, :-1].contiguous(), out, 4, 16, 2, 1, "elu1")


@pytest.mark.parametrize("causal", [True, False])
def test_wan_dq_sampled(causal):
    """Full Wan2.1-1.3B shape, in the configuration bench.py times: dq of
    seeded stratified rows (two per frame plus random ones, every chunk) against
    the oracle's per-row definition-form gradient.  The row sums D = dy . y come
    from the fp32 output (the bf16 output alone puts the bidirectional dq at
    the edge of the bar, see include/rehyat.h)."""
    from tests.parity_util import sample_rows
    w = inputs.WORKLOADS["wan_21x30x52"]
    q, k, v = inputs.make_qkv(w)
    dy = inputs.make_dout(w)
    qg, kg, vg, dyg = gpu(q, k, v, dy)
    out, lse, out32 = rh.attn_fwd_lse(qg, kg, vg, w.frames, w.tokens_per_frame, 3, 1, "elu1", causal=causal,
                                      out_f32=True)
    assert torch.equal(out32.to(torch.bfloat16), out)
    dq, _, _ = rh.attn_bwd(qg, kg, vg, out, lse, dyg, w.frames, w.tokens_per_frame, 3, 1, "elu1", causal=causal,
                           out_f32=out32)
    sync()
    rows = sample_rows(w.frames, w.tokens_per_frame, n_random=24, seed=31)
    ref = O.grad_q_rows(to64(q), to64(k), to64(v), to64(dy), w.frames, w.tokens_per_frame, 3, 1, rows, "elu1",
                        causal=causal)
    got = to64(dq[:, :, torch.from_numpy(rows).to("cuda")])
    e = rel_l2(got, ref)
    a = float(np.abs(got - ref).max() / np.abs(ref).max())
    assert e <= 1e-2 and a <= 3e-2, f"rel-L2 {e:.3e}, max-abs/scale {a:.3e}"
