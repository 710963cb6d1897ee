"""GPU parity of the learned feature maps (two-layer MLP, degree 2) against the
fp64 oracle.

ReHyAt writes phi as the concatenation of powers of learned functions (§3.2,
the equation after the partitions) and makes them a two-layer MLP of degree 2
with separate maps for queries and keys (§4.3, appendix §7.1).  The library
evaluates the maps on MFMA (bf16) or the vector ALU (fp32) through
rehyat_feature_mlp / rehyat_attn_fwd_mlp / rehyat_attn_fwd_mlp_partials /
rehyat_attn_step_mlp; the oracle applies oracle.MlpFeatureMap in fp64 to the
same bf16 (or fp32) inputs and weights.  The weights are seeded synthetic draws
(no trained weights exist here); their pinned special cases (reductions to the
parameter-free maps) are covered by the CPU oracle tests.

The bf16 path rounds the hidden layer and phi to bf16 (a bf16 model's
activation precision), so its phi differs from the fp64 one by a few bf16 ulps;
the attention outputs keep the bf16 bar (rel-L2 <= 1e-2, max-abs <= 3e-2).
"""
import numpy as np
import pytest
import torch

import linear_attention_video_rehyat_amd as rh
from linear_attention_video_rehyat_amd import inputs
from oracle import oracle as O
from tests.parity_util import (check_bf16, check_f32, gpu, per_chunk_rel, rel_l2, sample_rows, sync,
                               to64)

pytestmark = pytest.mark.gpu


def _maps(w, hidden, seed_id=None):
    """(device MlpWeights pair, oracle MlpFeatureMap pair) of one workload."""
    seed_id = w.seed_id if seed_id is None else seed_id
    dev, orc = [], []
    for side, scale in ((0, 1.0), (1, w.key_scale)):
        w1, b1, w2, b2 = inputs.make_mlp_weights(seed_id, side, w.H, w.head_dim, hidden, w.dtype, scale)
        dt = w.torch_dtype
        dev.append(rh.MlpWeights(w1.to(dt).cuda(), b1.cuda(), w2.to(dt).cuda(), b2.cuda()))
        orc.append(O.MlpFeatureMap(w1.numpy(), b1.numpy(), w2.numpy(), b2.numpy()))
    return tuple(dev), tuple(orc)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("hidden", [32, 64, 128, 256])
def test_feature_map_kernel_bf16(d, hidden):
    """phi rows against the fp64 map, over a ragged row count (several 128-row
    blocks and a tail) and two heads with different weights."""
    w = inputs.custom(2, 2, 1, 300, d, 1, 0, dtype="bf16", seed_id=900 + d + hidden)
    q, _, _ = inputs.make_qkv(w)
    (wq, _), (oq, _) = _maps(w, hidden)
    phi = rh.feature_mlp(q.cuda(), wq)
    sync()
    ref = oq(to64(q))
    got = to64(phi)
    assert got.shape == ref.shape
    assert (got >= 0).all()
    r = rel_l2(got, ref)
    assert r <= 5e-3, f"rel-L2 {r:.3e}"
    err = np.abs(got - ref) / (1.0 + np.abs(ref))
    assert err.max() <= 3e-2, f"max scaled error {err.max():.3e}"


@pytest.mark.parametrize("d", [16, 128])
def test_feature_map_kernel_f32(d):
    w = inputs.custom(1, 3, 1, 77, d, 1, 0, dtype="f32", seed_id=950 + d)
    q, _, _ = inputs.make_qkv(w)
    (wq, _), (oq, _) = _maps(w, 64)
    phi = rh.feature_mlp(q.cuda(), wq)
    sync()
    check_f32(to64(phi), oq(to64(q)), f"fp32 feature map d{d}")


@pytest.mark.parametrize("causal", [True, False])
def test_tiny_f32_full(causal):
    w = inputs.WORKLOADS["tiny_f4x8x8"]
    q, k, v = inputs.make_qkv(w)
    dev, orc = _maps(w, 32)
    y = rh.attn_fwd(*gpu(q, k, v), w.frames, w.tokens_per_frame, w.chunk_frames, w.overlap_frames, dev,
                    causal=causal)
    sync()
    ref = O.definition(to64(q), to64(k), to64(v), w.frames, w.tokens_per_frame, w.chunk_frames,
                       w.overlap_frames, orc, causal=causal)
    check_f32(to64(y), ref, f"tiny fp32 learned map causal={causal}")


SMALL = [
    (1, 2, 7, 100, 128, 3, 1, 256),
    (2, 1, 5, 97, 128, 1, 1, 128),
    (1, 1, 9, 60, 128, 2, 3, 64),
    (1, 2, 8, 33, 64, 3, 0, 256),
    (1, 3, 4, 45, 32, 1, 2, 32),
]


@pytest.mark.parametrize("geom", SMALL, ids=lambda g: "B{}H{}F{}HW{}d{}Tc{}To{}hid{}".format(*g))
@pytest.mark.parametrize("causal", [True, False])
def test_bf16_small_full(geom, causal):
    B, H, F, HW, d, Tc, To, hidden = geom
    w = inputs.custom(B, H, F, HW, d, Tc, To, dtype="bf16", seed_id=960 + F * 7 + d)
    q, k, v = inputs.make_qkv(w)
    dev, orc = _maps(w, hidden)
    y = rh.attn_fwd(*gpu(q, k, v), F, HW, Tc, To, dev, causal=causal)
    sync()
    ref = O.definition(to64(q), to64(k), to64(v), F, HW, Tc, To, orc, causal=causal)
    check_bf16(to64(y), ref, f"bf16 learned map {geom} causal={causal}")


@pytest.mark.parametrize("causal", [True, False])
def test_bf16_branch_partials(causal):
    B, H, F, HW, d, Tc, To = 1, 2, 7, 100, 128, 3, 1
    w = inputs.custom(B, H, F, HW, d, Tc, To, dtype="bf16", seed_id=980)
    q, k, v = inputs.make_qkv(w)
    dev, orc = _maps(w, 256)
    p = rh.attn_fwd_partials(*gpu(q, k, v), F, HW, Tc, To, dev, causal=causal)
    sync()
    _, ref = O.definition(to64(q), to64(k), to64(v), F, HW, Tc, To, orc, partials=True, causal=causal)
    assert rel_l2(to64(p["o_s"]), ref["oS"]) <= 1e-2
    lin = ref["nL"] > 0
    assert lin.any()
    got_nl, got_ol = to64(p["n_l"]), to64(p["o_l"])
    assert rel_l2(got_nl[lin], ref["nL"][lin]) <= 1e-2
    assert rel_l2(got_ol[lin], ref["oL"][lin]) <= 1e-2
    assert np.all(got_nl[~lin] == 0)


def test_bf16_step_equals_fwd_bitwise():
    """The stream computes phi of each chunk's rows with the same kernel and
    carries phi(k) of the overlap frames: bitwise equal to the forward."""
    B, H, F, HW, d, Tc, To = 1, 2, 8, 70, 128, 3, 1
    w = inputs.custom(B, H, F, HW, d, Tc, To, dtype="bf16", seed_id=985)
    q, k, v = gpu(*inputs.make_qkv(w))
    dev, _ = _maps(w, 256)
    y_fwd = rh.attn_fwd(q, k, v, F, HW, Tc, To, dev)
    st = rh.StepState(B, H, HW, d, Tc, To, dev, dtype=q.dtype)
    outs = []
    for f in range(0, F, Tc):
        sl = slice(f * HW, min(f + Tc, F) * HW)
        outs.append(st.step(q[:, :, sl].contiguous(), k[:, :, sl].contiguous(), v[:, :, sl].contiguous()))
    sync()
    assert torch.equal(torch.cat(outs, dim=2), y_fwd)


def test_f32_step_matches_recurrent_oracle():
    w = inputs.custom(1, 2, 6, 20, 16, 2, 1, dtype="f32", seed_id=986)
    q, k, v = inputs.make_qkv(w)
    dev, orc = _maps(w, 64)
    st = rh.StepState(1, 2, 20, 16, 2, 1, dev, dtype=torch.float32)
    qg, kg, vg = gpu(q, k, v)
    outs = [st.step(qg[:, :, f * 20:(f + 2) * 20].contiguous(), kg[:, :, f * 20:(f + 2) * 20].contiguous(),
                    vg[:, :, f * 20:(f + 2) * 20].contiguous()) for f in range(0, 6, 2)]
    sync()
    ref = O.recurrent(to64(q), to64(k), to64(v), 6, 20, 2, 1, orc)
    check_f32(to64(torch.cat(outs, dim=2)), ref, "fp32 learned-map stream")


@pytest.mark.parametrize("causal", [True, False])
def test_wan_21x30x52_sampled(causal):
    """Full Wan2.1-1.3B shape (hidden 256: 2.37M map parameters per block),
    seeded stratified rows per chunk."""
    w = inputs.WORKLOADS["wan_21x30x52"]
    q, k, v = inputs.make_qkv(w)
    dev, orc = _maps(w, 256)
    y = rh.attn_fwd(*gpu(q, k, v), w.frames, w.tokens_per_frame, w.chunk_frames, w.overlap_frames, dev,
                    causal=causal)
    sync()
    rows = sample_rows(w.frames, w.tokens_per_frame, n_random=64, seed=23)
    ref = O.definition(to64(q), to64(k), to64(v), w.frames, w.tokens_per_frame, w.chunk_frames,
                       w.overlap_frames, orc, rows=rows, causal=causal)
    ys = to64(y[:, :, torch.from_numpy(rows).to("cuda")])
    check_bf16(ys, ref, f"wan learned map causal={causal}")
    chunks = per_chunk_rel(ys, ref, rows, w.tokens_per_frame, w.chunk_frames)
    assert max(chunks.values()) <= 1e-2, f"per-chunk rel-L2 {chunks}"


def test_bad_weights_rejected():
    w = inputs.custom(1, 2, 4, 40, 64, 2, 1, dtype="bf16", seed_id=990)
    q, k, v = gpu(*inputs.make_qkv(w))
    (wq, wk), _ = _maps(w, 64)
    (wq128, _), _ = _maps(w, 128)
    with pytest.raises(rh.RehyatError):
        rh.attn_fwd(q, k, v, 4, 40, 2, 1, (wq, wq128))     # different hidden widths
    with pytest.raises(rh.RehyatError):
        rh.attn_fwd(q, k, v, 4, 40, 2, 1, "mlp2")          # learned map without weights
    with pytest.raises(rh.RehyatError):
        rh.attn_fwd(q.float(), k.float(), v.float(), 4, 40, 2, 1, (wq, wk))  # dtype mismatch
