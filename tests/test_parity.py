"""GPU parity of librehyat against the fp64 oracle on identical seeded inputs.

Every case calls the library through its C ABI (Python ctypes binding) and the
oracle's definition form (explicit per-query softmax / linear / ignored walk).
Small cases compare every output element; full-size workloads compare seeded
stratified row samples (first and last token of every frame plus random rows).
The softmax branch carries almost none of the normaliser after chunk 0 with
elu+1 features on these inputs, so branch partials and phi = NONE runs check it
separately.
"""
import numpy as np
import pytest
import torch

import linear_attention_video_rehyat_amd as rh
from linear_attention_video_rehyat_amd import inputs
from tests.parity_util import (check_bf16, check_f32, gpu, oracle_rows, per_chunk_rel, rel_l2,
                               sample_rows, sync, to64)

pytestmark = pytest.mark.gpu


def _fwd(w, phi, Tc=None, To=None):
    Tc = w.chunk_frames if Tc is None else Tc
    To = w.overlap_frames if To is None else To
    q, k, v = inputs.make_qkv(w)
    qg, kg, vg = gpu(q, k, v)
    y = rh.attn_fwd(qg, kg, vg, w.frames, w.tokens_per_frame, Tc, To, phi)
    sync()
    return (q, k, v), y, Tc, To


# ------------------------------------------------------------------ fp32

@pytest.mark.parametrize("phi", ["elu1", "poly2", "none"])
def test_tiny_f32_full(phi):
    """4 frames of 8x8 tokens, B1 H2 d16, T_c 1, T_o 1, fp32: every element."""
    w = inputs.WORKLOADS["tiny_f4x8x8"]
    (q, k, v), y, Tc, To = _fwd(w, phi)
    ref = oracle_rows(q, k, v, w.frames, w.tokens_per_frame, Tc, To, phi)
    check_f32(to64(y), ref, f"tiny fp32 {phi}")


@pytest.mark.parametrize("Tc,To", [(1, 0), (2, 1), (3, 5), (7, 0)])
@pytest.mark.parametrize("d", [16, 64, 128])
def test_f32_geometries(Tc, To, d):
    w = inputs.custom(1, 2, 7, 37, d, Tc, To, dtype="f32", seed_id=200 + d)
    for phi in ("elu1", "poly2"):
        (q, k, v), y, _, _ = _fwd(w, phi)
        ref = oracle_rows(q, k, v, w.frames, w.tokens_per_frame, Tc, To, phi)
        check_f32(to64(y), ref, f"fp32 d{d} Tc{Tc} To{To} {phi}")


# ------------------------------------------------------------------ bf16, small, every element

SMALL = [
    # (B, H, F, HW, d, Tc, To): several query tiles, ragged tails, T_o >= T_c, partial last chunk
    (1, 2, 7, 100, 128, 3, 1),
    (2, 1, 5, 97, 128, 1, 1),
    (1, 1, 9, 60, 128, 2, 3),
    (1, 2, 8, 33, 64, 3, 0),
    (1, 1, 6, 300, 128, 4, 2),
    (1, 3, 4, 45, 32, 1, 2),
    (1, 1, 3, 17, 128, 5, 1),     # one chunk longer than the clip: plain softmax
    (1, 2, 5, 128, 128, 1, 1),    # windows of whole key tiles: the last tile is a full one
]


@pytest.mark.parametrize("geom", SMALL, ids=lambda g: "B{}H{}F{}HW{}d{}Tc{}To{}".format(*g))
@pytest.mark.parametrize("phi", ["elu1", "poly2", "none"])
def test_bf16_small_full(geom, phi):
    B, H, F, HW, d, Tc, To = geom
    w = inputs.custom(B, H, F, HW, d, Tc, To, dtype="bf16", seed_id=300 + F * 7 + d)
    (q, k, v), y, _, _ = _fwd(w, phi)
    ref = oracle_rows(q, k, v, F, HW, Tc, To, phi)
    check_bf16(to64(y), ref, f"bf16 {geom} {phi}")


@pytest.mark.parametrize("phi", ["elu1", "poly2"])
def test_bf16_branch_partials_small(phi):
    """Each branch on its own: m, sum exp(s - m), a^S/n^S, a^L/n^L, n^L."""
    B, H, F, HW, d, Tc, To = 1, 2, 7, 100, 128, 3, 1
    w = inputs.custom(B, H, F, HW, d, Tc, To, dtype="bf16", seed_id=401)
    q, k, v = inputs.make_qkv(w)
    qg, kg, vg = gpu(q, k, v)
    p = rh.attn_fwd_partials(qg, kg, vg, F, HW, Tc, To, phi)
    sync()
    _, ref = oracle_rows(q, k, v, F, HW, Tc, To, phi, partials=True)
    np.testing.assert_allclose(to64(p["m"]), ref["m"], rtol=0, atol=1e-4)
    assert rel_l2(to64(p["nt"]), ref["nt"]) <= 1e-2
    assert rel_l2(to64(p["o_s"]), ref["oS"]) <= 1e-2
    lin = ref["nL"] > 0
    assert rel_l2(to64(p["n_l"])[lin], ref["nL"][lin]) <= 1e-5
    assert rel_l2(to64(p["o_l"])[lin], ref["oL"][lin]) <= 1e-2
    assert np.all(to64(p["n_l"])[~lin] == 0.0)


def test_bf16_deterministic():
    """No atomics anywhere: two runs give bitwise identical outputs."""
    w = inputs.custom(1, 2, 7, 100, 128, 3, 1, dtype="bf16", seed_id=402)
    q, k, v = gpu(*inputs.make_qkv(w))
    y1 = rh.attn_fwd(q, k, v, 7, 100, 3, 1, "elu1")
    y2 = rh.attn_fwd(q, k, v, 7, 100, 3, 1, "elu1")
    sync()
    assert torch.equal(y1, y2)


# ------------------------------------------------------------------ full-size workloads (sampled rows)

def _full_size(name, phi, Tc=None, To=None, n_random=96, check_chunks=True):
    w = inputs.WORKLOADS[name]
    (q, k, v), y, Tc, To = _fwd(w, phi, Tc, To)
    rows = sample_rows(w.frames, w.tokens_per_frame, n_random=n_random, seed=w.seed_id)
    ref = oracle_rows(q, k, v, w.frames, w.tokens_per_frame, Tc, To, phi, rows=rows)
    ys = to64(y[:, :, torch.from_numpy(rows).to("cuda")])
    r, a = check_bf16(ys, ref, f"{name} Tc{Tc} To{To} {phi}")
    chunks = per_chunk_rel(ys, ref, rows, w.tokens_per_frame, Tc)
    if check_chunks:
        worst = max(chunks.values())
        assert worst <= 1e-2, f"per-chunk rel-L2 {chunks}"
    return r, a, chunks


@pytest.mark.parametrize("phi", ["elu1", "none", "poly2"])
def test_wan_21x30x52(phi):
    _full_size("wan_21x30x52", phi)


@pytest.mark.parametrize("Tc", [1, 3, 7])
def test_wan_cfg_pair_chunk_sweep(Tc):
    _full_size("wan_cfg_21x30x52", "elu1", Tc=Tc)


def test_wan_cfg_pair_none():
    _full_size("wan_cfg_21x30x52", "none")


def test_dense_softmax_companion():
    """One chunk spanning all 21 frames with no linear branch: bidirectional softmax."""
    _full_size("wan_21x30x52", "none", Tc=21, To=0)


@pytest.mark.parametrize("phi", ["elu1", "none"])
def test_wan_outlier_21x45x80(phi):
    _full_size("wan_outlier_21x45x80", phi, n_random=64)


def test_wan_partials_sampled():
    """Branch partials at the full Wan shape, per chunk."""
    w = inputs.WORKLOADS["wan_21x30x52"]
    q, k, v = inputs.make_qkv(w)
    qg, kg, vg = gpu(q, k, v)
    p = rh.attn_fwd_partials(qg, kg, vg, w.frames, w.tokens_per_frame, 3, 1, "elu1")
    sync()
    rows = sample_rows(w.frames, w.tokens_per_frame, n_random=64, seed=7)
    _, ref = oracle_rows(q, k, v, w.frames, w.tokens_per_frame, 3, 1, "elu1", rows=rows,
                         partials=True)
    ridx = torch.from_numpy(rows).to("cuda")
    os_ = to64(p["o_s"][:, :, ridx])
    ol = to64(p["o_l"][:, :, ridx])
    chunk = (rows // w.tokens_per_frame) // 3
    for t in np.unique(chunk):
        sel = chunk == t
        assert rel_l2(os_[:, :, sel], ref["oS"][:, :, sel]) <= 1e-2, f"softmax branch chunk {t}"
        if t > 0:
            assert rel_l2(ol[:, :, sel], ref["oL"][:, :, sel]) <= 1e-2, f"linear branch chunk {t}"
    np.testing.assert_allclose(to64(p["m"][:, :, ridx]), ref["m"], rtol=0, atol=1e-3)
