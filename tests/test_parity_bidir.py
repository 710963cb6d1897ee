"""GPU parity of the bidirectional (non-causal) form against the fp64 oracle.

ReHyAt §3.2 with overlap: chunk t's softmax set is the same window as in the
recurrent form, and its linear set is every other key of the clip, the keys of
later chunks included.  The library calls go through the C ABI
(rehyat_attn_fwd_bidir, _f32, _partials); the oracle runs its definition form
with causal=False.  Small cases compare every element, full-size workloads
seeded stratified row samples, per chunk.
"""
import numpy as np
import pytest
import torch

import linear_attention_video_rehyat_amd as rh
from linear_attention_video_rehyat_amd import inputs
from tests.parity_util import (check_bf16, check_f32, gpu, oracle_rows, per_chunk_rel, rel_l2,
                               sample_rows, sync, to64)

pytestmark = pytest.mark.gpu


def _fwd(w, phi, Tc=None, To=None, causal=False):
    Tc = w.chunk_frames if Tc is None else Tc
    To = w.overlap_frames if To is None else To
    q, k, v = inputs.make_qkv(w)
    qg, kg, vg = gpu(q, k, v)
    y = rh.attn_fwd(qg, kg, vg, w.frames, w.tokens_per_frame, Tc, To, phi, causal=causal)
    sync()
    return (q, k, v), y, Tc, To


@pytest.mark.parametrize("phi", ["elu1", "poly2", "none"])
def test_tiny_f32_full(phi):
    w = inputs.WORKLOADS["tiny_f4x8x8"]
    (q, k, v), y, Tc, To = _fwd(w, phi)
    ref = oracle_rows(q, k, v, w.frames, w.tokens_per_frame, Tc, To, phi, causal=False)
    check_f32(to64(y), ref, f"tiny fp32 bidirectional {phi}")


@pytest.mark.parametrize("Tc,To", [(1, 0), (2, 1), (3, 5), (7, 0), (2, 4)])
@pytest.mark.parametrize("d", [16, 128])
def test_f32_geometries(Tc, To, d):
    w = inputs.custom(1, 2, 7, 37, d, Tc, To, dtype="f32", seed_id=600 + d)
    for phi in ("elu1", "poly2"):
        (q, k, v), y, _, _ = _fwd(w, phi)
        ref = oracle_rows(q, k, v, w.frames, w.tokens_per_frame, Tc, To, phi, causal=False)
        check_f32(to64(y), ref, f"fp32 bidirectional d{d} Tc{Tc} To{To} {phi}")


SMALL = [
    (1, 2, 7, 100, 128, 3, 1),
    (2, 1, 5, 97, 128, 1, 1),
    (1, 1, 9, 60, 128, 2, 3),     # T_o > T_c
    (1, 1, 8, 50, 128, 2, 4),     # T_o a multiple of T_c
    (1, 2, 8, 33, 64, 3, 0),
    (1, 3, 4, 45, 32, 1, 2),
    (1, 1, 3, 17, 128, 5, 1),     # one chunk: plain softmax
]


@pytest.mark.parametrize("geom", SMALL, ids=lambda g: "B{}H{}F{}HW{}d{}Tc{}To{}".format(*g))
@pytest.mark.parametrize("phi", ["elu1", "poly2"])
def test_bf16_small_full(geom, phi):
    B, H, F, HW, d, Tc, To = geom
    w = inputs.custom(B, H, F, HW, d, Tc, To, dtype="bf16", seed_id=700 + F * 7 + d)
    (q, k, v), y, _, _ = _fwd(w, phi)
    ref = oracle_rows(q, k, v, F, HW, Tc, To, phi, causal=False)
    check_bf16(to64(y), ref, f"bf16 bidirectional {geom} {phi}")


@pytest.mark.parametrize("phi", ["elu1", "poly2"])
def test_bf16_branch_partials_small(phi):
    """Each branch on its own; every chunk has a linear set (later chunks)."""
    B, H, F, HW, d, Tc, To = 1, 2, 7, 100, 128, 3, 1
    w = inputs.custom(B, H, F, HW, d, Tc, To, dtype="bf16", seed_id=801)
    q, k, v = inputs.make_qkv(w)
    qg, kg, vg = gpu(q, k, v)
    p = rh.attn_fwd_partials(qg, kg, vg, F, HW, Tc, To, phi, causal=False)
    sync()
    _, ref = oracle_rows(q, k, v, F, HW, Tc, To, phi, partials=True, causal=False)
    np.testing.assert_allclose(to64(p["m"]), ref["m"], rtol=0, atol=1e-4)
    assert rel_l2(to64(p["nt"]), ref["nt"]) <= 1e-2
    assert rel_l2(to64(p["o_s"]), ref["oS"]) <= 1e-2
    assert np.all(ref["nL"] > 0)
    assert rel_l2(to64(p["n_l"]), ref["nL"]) <= 1e-5
    assert rel_l2(to64(p["o_l"]), ref["oL"]) <= 1e-2


def test_no_linear_set_equals_recurrent_form():
    """Without a linear branch (phi = NONE), or with one chunk covering the clip,
    both forms are the same softmax over the same windows: bitwise equal."""
    w = inputs.custom(1, 2, 7, 100, 128, 3, 1, dtype="bf16", seed_id=802)
    q, k, v = gpu(*inputs.make_qkv(w))
    a = rh.attn_fwd(q, k, v, 7, 100, 3, 1, "none", causal=True)
    b = rh.attn_fwd(q, k, v, 7, 100, 3, 1, "none", causal=False)
    c = rh.attn_fwd(q, k, v, 7, 100, 7, 0, "elu1", causal=True)
    d = rh.attn_fwd(q, k, v, 7, 100, 7, 0, "elu1", causal=False)
    sync()
    assert torch.equal(a, b)
    assert torch.equal(c, d)


def test_last_chunk_matches_recurrent_form():
    """The last chunk has no later keys: its rows equal the recurrent form's up
    to the order of the fp32 sums (prefix of finer blocks)."""
    w = inputs.custom(1, 2, 7, 100, 128, 3, 1, dtype="bf16", seed_id=803)
    q, k, v = gpu(*inputs.make_qkv(w))
    a = rh.attn_fwd(q, k, v, 7, 100, 3, 1, "elu1", causal=True)
    b = rh.attn_fwd(q, k, v, 7, 100, 3, 1, "elu1", causal=False)
    sync()
    last = slice(6 * 100, 7 * 100)
    assert rel_l2(to64(b[:, :, last]), to64(a[:, :, last])) <= 2e-3
    assert rel_l2(to64(b[:, :, :600]), to64(a[:, :, :600])) > 1e-2  # earlier chunks see later keys


def test_bf16_deterministic():
    w = inputs.custom(1, 2, 7, 100, 128, 3, 1, dtype="bf16", seed_id=804)
    q, k, v = gpu(*inputs.make_qkv(w))
    y1 = rh.attn_fwd(q, k, v, 7, 100, 3, 1, "elu1", causal=False)
    y2 = rh.attn_fwd(q, k, v, 7, 100, 3, 1, "elu1", causal=False)
    sync()
    assert torch.equal(y1, y2)


def _full_size(name, phi, Tc=None, To=None, n_random=96):
    w = inputs.WORKLOADS[name]
    (q, k, v), y, Tc, To = _fwd(w, phi, Tc, To)
    rows = sample_rows(w.frames, w.tokens_per_frame, n_random=n_random, seed=w.seed_id + 17)
    ref = oracle_rows(q, k, v, w.frames, w.tokens_per_frame, Tc, To, phi, rows=rows, causal=False)
    ys = to64(y[:, :, torch.from_numpy(rows).to("cuda")])
    check_bf16(ys, ref, f"{name} bidirectional Tc{Tc} To{To} {phi}")
    chunks = per_chunk_rel(ys, ref, rows, w.tokens_per_frame, Tc)
    assert max(chunks.values()) <= 1e-2, f"per-chunk rel-L2 {chunks}"


@pytest.mark.parametrize("phi", ["elu1", "poly2"])
def test_wan_21x30x52(phi):
    _full_size("wan_21x30x52", phi)


@pytest.mark.parametrize("Tc", [1, 7])
def test_wan_cfg_pair_chunk_sweep(Tc):
    _full_size("wan_cfg_21x30x52", "elu1", Tc=Tc)


def test_wan_outlier_21x45x80():
    _full_size("wan_outlier_21x45x80", "elu1", n_random=64)


def test_wan_partials_sampled():
    """Branch partials at the full Wan shape, per chunk (chunk 0 included: its
    linear set is every later key)."""
    w = inputs.WORKLOADS["wan_21x30x52"]
    q, k, v = inputs.make_qkv(w)
    qg, kg, vg = gpu(q, k, v)
    p = rh.attn_fwd_partials(qg, kg, vg, w.frames, w.tokens_per_frame, 3, 1, "elu1", causal=False)
    sync()
    rows = sample_rows(w.frames, w.tokens_per_frame, n_random=64, seed=9)
    _, ref = oracle_rows(q, k, v, w.frames, w.tokens_per_frame, 3, 1, "elu1", rows=rows,
                         partials=True, causal=False)
    ridx = torch.from_numpy(rows).to("cuda")
    os_ = to64(p["o_s"][:, :, ridx])
    ol = to64(p["o_l"][:, :, ridx])
    chunk = (rows // w.tokens_per_frame) // 3
    for t in np.unique(chunk):
        sel = chunk == t
        assert rel_l2(os_[:, :, sel], ref["oS"][:, :, sel]) <= 1e-2, f"softmax branch chunk {t}"
        assert rel_l2(ol[:, :, sel], ref["oL"][:, :, sel]) <= 1e-2, f"linear branch chunk {t}"
