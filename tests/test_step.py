"""Streaming (chunk-wise RNN) path on the GPU: chunk-by-chunk calls of
rehyat_attn_step reproduce the whole-clip forward, match the oracle's recurrent
form, resume exactly from a saved state, and use memory that does not depend on
how many frames have been processed (ReHyAt §3.3 and §5.2: constant peak memory
in the recurrent form)."""
import numpy as np
import pytest
import torch

import linear_attention_video_rehyat_amd as rh
from linear_attention_video_rehyat_amd import inputs
from oracle import oracle as O
from tests.parity_util import check_bf16, check_f32, gpu, oracle_rows, rel_l2, sample_rows, sync, to64

pytestmark = pytest.mark.gpu


def _stream(q, k, v, HW, Tc, To, phi, frames_per_call=None):
    B, H, N, d = q.shape
    F = N // HW
    st = rh.StepState(B, H, HW, d, Tc, To, phi, dtype=q.dtype)
    outs = []
    f = 0
    while f < F:
        n = min(Tc, F - f)
        sl = slice(f * HW, (f + n) * HW)
        outs.append(st.step(q[:, :, sl].contiguous(), k[:, :, sl].contiguous(), v[:, :, sl].contiguous()))
        f += n
    return torch.cat(outs, dim=2), st


@pytest.mark.parametrize("geom", [(1, 2, 7, 100, 128, 3, 1), (1, 1, 9, 60, 128, 2, 3),
                                  (2, 1, 5, 97, 64, 1, 1), (1, 1, 8, 40, 128, 3, 0)],
                         ids=lambda g: "B{}H{}F{}HW{}d{}Tc{}To{}".format(*g))
@pytest.mark.parametrize("phi", ["elu1", "poly2", "none"])
def test_step_equals_fwd_bitwise(geom, phi):
    """Same rows, same tiles, same summation order: bitwise equal to the forward."""
    B, H, F, HW, d, Tc, To = geom
    w = inputs.custom(B, H, F, HW, d, Tc, To, dtype="bf16", seed_id=500 + F)
    q, k, v = gpu(*inputs.make_qkv(w))
    y_fwd = rh.attn_fwd(q, k, v, F, HW, Tc, To, phi)
    y_st, st = _stream(q, k, v, HW, Tc, To, phi)
    sync()
    assert st.frames_done == F
    assert torch.equal(y_st, y_fwd)


@pytest.mark.parametrize("phi", ["elu1", "poly2"])
def test_step_matches_recurrent_oracle(phi):
    B, H, F, HW, d, Tc, To = 1, 2, 8, 70, 128, 2, 1
    w = inputs.custom(B, H, F, HW, d, Tc, To, dtype="bf16", seed_id=510)
    q, k, v = inputs.make_qkv(w)
    y, _ = _stream(*gpu(q, k, v), HW, Tc, To, phi)
    sync()
    ref = O.recurrent(to64(q), to64(k), to64(v), F, HW, Tc, To, phi)
    check_bf16(to64(y), ref, f"stream {phi}")


@pytest.mark.parametrize("phi", ["elu1", "poly2", "none"])
def test_tiny_f32_stream(phi):
    w = inputs.WORKLOADS["tiny_f4x8x8"]
    q, k, v = inputs.make_qkv(w)
    y, _ = _stream(*gpu(q, k, v), w.tokens_per_frame, w.chunk_frames, w.overlap_frames, phi)
    sync()
    ref = O.recurrent(to64(q), to64(k), to64(v), w.frames, w.tokens_per_frame, w.chunk_frames,
                      w.overlap_frames, phi)
    check_f32(to64(y), ref, f"tiny fp32 stream {phi}")


def test_partial_last_chunk_and_end_of_stream():
    B, H, F, HW, d, Tc, To = 1, 1, 7, 50, 128, 3, 1
    w = inputs.custom(B, H, F, HW, d, Tc, To, dtype="bf16", seed_id=520)
    q, k, v = gpu(*inputs.make_qkv(w))
    y_st, st = _stream(q, k, v, HW, Tc, To, "elu1")
    y_fwd = rh.attn_fwd(q, k, v, F, HW, Tc, To, "elu1")
    sync()
    assert torch.equal(y_st, y_fwd)
    with pytest.raises(rh.RehyatError):
        st.step(q[:, :, :HW].contiguous(), k[:, :, :HW].contiguous(), v[:, :, :HW].contiguous())


def test_resume_from_saved_state():
    """The state buffer plus header is a checkpoint: restoring it continues exactly."""
    B, H, F, HW, d, Tc, To = 1, 2, 9, 64, 128, 3, 2
    w = inputs.custom(B, H, F, HW, d, Tc, To, dtype="bf16", seed_id=530)
    q, k, v = gpu(*inputs.make_qkv(w))
    ref, _ = _stream(q, k, v, HW, Tc, To, "elu1")
    st = rh.StepState(B, H, HW, d, Tc, To, "elu1")
    sl = lambda f0, f1: slice(f0 * HW, f1 * HW)
    outs = [st.step(q[:, :, sl(0, 3)].contiguous(), k[:, :, sl(0, 3)].contiguous(), v[:, :, sl(0, 3)].contiguous())]
    saved = st.save()
    st2 = rh.StepState(B, H, HW, d, Tc, To, "elu1")
    st2.restore(saved)
    for f0 in (3, 6):
        outs.append(st2.step(q[:, :, sl(f0, f0 + 3)].contiguous(), k[:, :, sl(f0, f0 + 3)].contiguous(),
                             v[:, :, sl(f0, f0 + 3)].contiguous()))
    sync()
    assert torch.equal(torch.cat(outs, dim=2), ref)


def test_constant_memory_long_stream():
    """Streaming 105 frames chunk by chunk allocates nothing beyond the fixed
    state buffer; the buffer size does not depend on the number of frames."""
    HW, d, Tc, To = 1560, 128, 3, 1
    st = rh.StepState(1, 12, HW, d, Tc, To, "elu1")
    gen = torch.Generator(device="cuda").manual_seed(5)
    shape = (1, 12, Tc * HW, d)
    q = torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16)
    k = (torch.randn(shape, generator=gen, device="cuda") / d ** 0.5).to(torch.bfloat16)
    v = torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16)
    out = torch.empty_like(q)
    sync()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    for _ in range(35):
        st.step(q, k, v, out=out)
    sync()
    assert torch.cuda.max_memory_allocated() == base
    assert st.frames_done == 105
    assert torch.isfinite(out.float()).all()
    st21 = rh.StepState(1, 12, HW, d, Tc, To, "elu1")
    assert st21.nbytes == st.nbytes


def test_long_105_frames_stream_vs_fwd_and_oracle():
    """105 latent frames of 1560 tokens, 35 steps of 3 frames: equals the
    whole-clip forward bitwise, and sampled rows match the oracle."""
    w = inputs.WORKLOADS["wan_long_105x30x52"]
    q, k, v = inputs.make_qkv(w)
    qg, kg, vg = gpu(q, k, v)
    y_st, st = _stream(qg, kg, vg, w.tokens_per_frame, w.chunk_frames, w.overlap_frames, "elu1")
    y_fwd = rh.attn_fwd(qg, kg, vg, w.frames, w.tokens_per_frame, w.chunk_frames, w.overlap_frames, "elu1")
    sync()
    assert torch.equal(y_st, y_fwd)
    del y_fwd
    rows = sample_rows(w.frames, w.tokens_per_frame, n_random=32, seed=4)
    rows = rows[rows >= 90 * w.tokens_per_frame]  # the last chunks carry the longest linear history
    rows = np.concatenate([sample_rows(3, w.tokens_per_frame, 8, 1), rows])
    ref = oracle_rows(q, k, v, w.frames, w.tokens_per_frame, w.chunk_frames, w.overlap_frames,
                      "elu1", rows=rows)
    ys = to64(y_st[:, :, torch.from_numpy(rows).to("cuda")])
    check_bf16(ys, ref, "long 105-frame stream")


def test_streams_on_two_user_streams_interleaved():
    """Two streams of steps queued alternately on two user streams (each with
    its own side stream for the fold, running concurrently): each equals its
    whole-clip forward bit for bit; releasing a stream's workspace (and side
    stream) in the middle of its stream changes nothing."""
    g = (1, 3, 10, 150, 128, 3, 1)
    B, H, F, HW, d, Tc, To = g
    clips = [gpu(*inputs.make_qkv(inputs.custom(*g, dtype="bf16", seed_id=s))) for s in (531, 532)]
    refs = [rh.attn_fwd(q, k, v, F, HW, Tc, To, "elu1") for q, k, v in clips]
    sync()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    states = [rh.StepState(B, H, HW, d, Tc, To, "elu1") for _ in clips]
    chunks = [[[t[:, :, f * HW:min(f + Tc, F) * HW].contiguous() for t in c] for f in range(0, F, Tc)] for c in clips]
    sync()
    outs = [[], []]
    for i in range(len(chunks[0])):
        for j in (0, 1):
            with torch.cuda.stream(streams[j]):
                outs[j].append(states[j].step(*chunks[j][i], stream=streams[j]))
        if i == 1:
            rh.workspace_release(streams[0])
    sync()
    for j in (0, 1):
        assert torch.equal(torch.cat(outs[j], dim=2), refs[j]), j
    rh.workspace_release(streams[1])


@pytest.mark.parametrize("phi", ["elu1", "poly2"])
def test_stream_fold_beside_a_nearly_full_local_launch(phi):
    """31 heads of 2048-token frames, one frame per step: each local launch has
    8 x 31 = 248 workgroups, so on 256 CUs the fold (62 sub-blocks) runs with a
    capped grid, its workgroups taking sub-blocks in turn and then making the
    overlap copy; the stream still equals the whole-clip forward bit for bit."""
    B, H, F, HW, d, Tc, To = 1, 31, 6, 2048, 128, 1, 1
    w = inputs.custom(B, H, F, HW, d, Tc, To, dtype="bf16", seed_id=540)
    q, k, v = gpu(*inputs.make_qkv(w))
    y_fwd = rh.attn_fwd(q, k, v, F, HW, Tc, To, phi)
    y_st, _ = _stream(q, k, v, HW, Tc, To, phi)
    sync()
    assert torch.equal(y_st, y_fwd)
