"""Failure paths and boundary hazards on the GPU (every kernel exits normally):

* guard canaries before and after `out`, the five partial buffers and the
  streaming state buffer catch writes outside them on ragged geometries
  (query tiles, key tiles and sub-blocks that end mid-tile);
* NaN propagation follows the partition exactly: a NaN key (or value) reaches
  the queries whose softmax or linear set holds it (ReHyAt §3.3 sets) -- every
  later chunk through the carried state -- and no other row changes;
* HIP failures forced at every HIP step of a call by the fault-injection hook
  return REHYAT_EHIP, and the library works normally afterwards;
* calls on two streams at once use separate workspace and give the same
  bits as each alone; releasing a stream's workspace changes nothing."""
import ctypes

import numpy as np
import pytest
import torch

import linear_attention_video_rehyat_amd as rh
from linear_attention_video_rehyat_amd import inputs
from oracle import oracle as O
from tests.parity_util import gpu, sync

pytestmark = pytest.mark.gpu

PAD = 4096
CANARY = 0xA5


class Guarded:
    """A device tensor with PAD canary bytes on each side."""

    def __init__(self, shape, dtype):
        self.nbytes = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.buf = torch.full((self.nbytes + 2 * PAD,), CANARY, dtype=torch.uint8, device="cuda")
        self.t = self.buf[PAD:PAD + self.nbytes].view(dtype).view(shape)

    def intact(self) -> bool:
        return bool((self.buf[:PAD] == CANARY).all() and (self.buf[PAD + self.nbytes:] == CANARY).all())


RAGGED = [(1, 2, 7, 100, 128, 3, 1), (2, 1, 5, 97, 128, 1, 1), (1, 3, 4, 45, 32, 1, 2), (1, 1, 9, 60, 64, 2, 3)]
GID = lambda g: "B{}H{}F{}HW{}d{}Tc{}To{}".format(*g)


@pytest.mark.parametrize("geom", RAGGED, ids=GID)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_canaries_forward_and_partials(geom, dtype):
    B, H, F, HW, d, Tc, To = geom
    w = inputs.custom(B, H, F, HW, d, Tc, To, dtype=dtype, seed_id=700 + F)
    q, k, v = gpu(*inputs.make_qkv(w))
    lib = rh.load_library()
    for phi in ("elu1", "poly2", "none"):
        out = Guarded(q.shape, q.dtype)
        for causal in (True, False):
            rh.attn_fwd(q, k, v, F, HW, Tc, To, phi, out=out.t, causal=causal)
            sync()
            assert out.intact(), f"write outside out ({phi}, causal={causal})"
        parts = [Guarded((B, H, w.N), torch.float32), Guarded((B, H, w.N), torch.float32),
                 Guarded(q.shape, torch.float32), Guarded(q.shape, torch.float32),
                 Guarded((B, H, w.N), torch.float32)]
        st = lib.rehyat_attn_fwd_partials(q.data_ptr(), k.data_ptr(), v.data_ptr(), rh._dtype_id(q),
                                          *[p.t.data_ptr() for p in parts], B, H, F, HW, d, Tc, To,
                                          rh.feature_map_id(phi), rh._stream_handle(None))
        assert st == 0, lib.rehyat_last_error()
        sync()
        assert all(p.intact() for p in parts), f"write outside a partial buffer ({phi})"


@pytest.mark.parametrize("geom", RAGGED, ids=GID)
def test_canaries_stream_state_and_outputs(geom):
    B, H, F, HW, d, Tc, To = geom
    w = inputs.custom(B, H, F, HW, d, Tc, To, dtype="bf16", seed_id=720 + F)
    q, k, v = gpu(*inputs.make_qkv(w))
    lib = rh.load_library()
    for phi in ("elu1", "poly2", "none"):
        fm = rh.feature_map_id(phi)
        need = lib.rehyat_step_state_bytes(B, H, HW, d, Tc, To, fm, rh.DTYPE_BF16)
        sbuf = Guarded((need,), torch.uint8)
        st = rh._StepStateC()
        assert lib.rehyat_step_state_init(ctypes.byref(st), sbuf.t.data_ptr(), need, B, H, HW, d, Tc, To, fm,
                                          rh.DTYPE_BF16) == 0
        ref = rh.attn_fwd(q, k, v, F, HW, Tc, To, phi)
        outs = []
        for f in range(0, F, Tc):
            n = min(Tc, F - f)
            sl = slice(f * HW, (f + n) * HW)
            o = Guarded((B, H, n * HW, d), torch.bfloat16)
            assert lib.rehyat_attn_step(ctypes.byref(st), q[:, :, sl].contiguous().data_ptr(),
                                        k[:, :, sl].contiguous().data_ptr(), v[:, :, sl].contiguous().data_ptr(),
                                        o.t.data_ptr(), n, rh._stream_handle(None)) == 0
            sync()
            assert o.intact(), f"write outside a step's out ({phi}, frame {f})"
            outs.append(o)
        assert sbuf.intact(), f"write outside the state buffer ({phi})"
        assert torch.equal(torch.cat([o.t for o in outs], dim=2), ref)


def _nan_rows(y):
    return torch.isnan(y.float()).any(dim=-1).cpu().numpy()


@pytest.mark.parametrize("phi", ["elu1", "none"])
@pytest.mark.parametrize("where", ["k", "v"])
@pytest.mark.parametrize("frame", [0, 2, 5])
def test_nan_propagates_along_the_partition(phi, where, frame):
    """A NaN in one key (or value) row: the rows whose softmax or linear set
    holds that key are NaN, every other row is bitwise what it was."""
    B, H, F, HW, d, Tc, To = 1, 2, 6, 40, 64, 2, 1
    w = inputs.custom(B, H, F, HW, d, Tc, To, dtype="bf16", seed_id=740)
    q, k, v = gpu(*inputs.make_qkv(w))
    clean = rh.attn_fwd(q, k, v, F, HW, Tc, To, phi)
    j = frame * HW + 7
    kk, vv = k.clone(), v.clone()
    (kk if where == "k" else vv)[0, 1, j, 3] = float("nan")
    y = rh.attn_fwd(q, kk, vv, F, HW, Tc, To, phi)
    sync()
    m_s, m_l = O.masks(w.N, HW, Tc, To, causal=True)
    expect = m_s[:, j] | (m_l[:, j] if phi != "none" else False)
    got = _nan_rows(y)
    assert not got[0, 0].any(), "the other head is untouched"
    np.testing.assert_array_equal(got[0, 1], expect)
    keep = torch.from_numpy(~expect).to("cuda")
    assert torch.equal(y[0, 1][keep], clean[0, 1][keep])
    assert torch.equal(y[0, 0], clean[0, 0])


def test_nan_query_poisons_only_its_row():
    B, H, F, HW, d, Tc, To = 1, 1, 6, 40, 128, 2, 1
    w = inputs.custom(B, H, F, HW, d, Tc, To, dtype="bf16", seed_id=741)
    q, k, v = gpu(*inputs.make_qkv(w))
    clean = rh.attn_fwd(q, k, v, F, HW, Tc, To, "elu1")
    qq = q.clone()
    qq[0, 0, 123, 5] = float("nan")
    y = rh.attn_fwd(qq, k, v, F, HW, Tc, To, "elu1")
    sync()
    rows = _nan_rows(y)[0, 0]
    assert rows[123] and rows.sum() == 1
    keep = torch.ones(w.N, dtype=torch.bool, device="cuda")
    keep[123] = False
    assert torch.equal(y[0, 0][keep], clean[0, 0][keep])


def _call_fwd(q, k, v, out, g, phi):
    lib = rh.load_library()
    B, H, F, HW, d, Tc, To = g
    return lib.rehyat_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, F, HW, d, Tc, To,
                               rh.feature_map_id(phi), rh._stream_handle(None))


@pytest.mark.parametrize("phi", ["elu1", "poly2", "none"])
def test_injected_hip_failure_at_every_step(phi):
    """Each HIP step of a forward failed in turn: REHYAT_EHIP with the step
    named, nothing queued after it; the next call runs normally."""
    g = (1, 2, 7, 100, 128, 3, 1)
    w = inputs.custom(*g, dtype="bf16", seed_id=760)
    q, k, v = gpu(*inputs.make_qkv(w))
    ref = rh.attn_fwd(q, k, v, *g[2:4], *g[5:7], phi)
    sync()
    lib = rh.load_library()
    out = torch.empty_like(q)
    assert _call_fwd(q, k, v, out, g, phi) == 0
    n_steps = rh.debug_hip_steps()
    assert n_steps >= (1 if phi == "none" else 4)
    for i in range(n_steps):
        rh.debug_inject_hip_error(i)
        st = _call_fwd(q, k, v, out, g, phi)
        assert st == 4 and f"HIP step {i}" in lib.rehyat_last_error().decode(), lib.rehyat_last_error()
        assert rh.debug_hip_steps() == i + 1
    sync()
    out.zero_()
    assert _call_fwd(q, k, v, out, g, phi) == 0
    sync()
    assert torch.equal(out, ref)


def test_injected_failure_backward_and_step():
    g = (1, 2, 7, 100, 128, 3, 1)
    B, H, F, HW, d, Tc, To = g
    w = inputs.custom(*g, dtype="bf16", seed_id=761)
    q, k, v = gpu(*inputs.make_qkv(w))
    dy = inputs.make_dout(w).cuda()
    out, lse = rh.attn_fwd_lse(q, k, v, F, HW, Tc, To, "elu1")
    ref = rh.attn_bwd(q, k, v, out, lse, dy, F, HW, Tc, To, "elu1")
    sync()
    rh.attn_bwd(q, k, v, out, lse, dy, F, HW, Tc, To, "elu1")
    n_steps = rh.debug_hip_steps()
    for i in range(n_steps):
        rh.debug_inject_hip_error(i)
        with pytest.raises(rh.RehyatError, match=f"HIP step {i}"):
            rh.attn_bwd(q, k, v, out, lse, dy, F, HW, Tc, To, "elu1")
    got = rh.attn_bwd(q, k, v, out, lse, dy, F, HW, Tc, To, "elu1")
    sync()
    assert all(torch.equal(a, b) for a, b in zip(got, ref))
    # a step that fails leaves the header unchanged; a fresh stream then matches the forward
    st = rh.StepState(B, H, HW, d, Tc, To, "elu1")
    rh.debug_inject_hip_error(0)
    with pytest.raises(rh.RehyatError, match="HIP step 0"):
        st.step(q[:, :, :Tc * HW].contiguous(), k[:, :, :Tc * HW].contiguous(), v[:, :, :Tc * HW].contiguous())
    assert st.frames_done == 0
    y_fwd = rh.attn_fwd(q, k, v, F, HW, Tc, To, "elu1")
    outs = []
    for f in range(0, F, Tc):
        sl = slice(f * HW, min(f + Tc, F) * HW)
        outs.append(st.step(q[:, :, sl].contiguous(), k[:, :, sl].contiguous(), v[:, :, sl].contiguous()))
    sync()
    assert torch.equal(torch.cat(outs, dim=2), y_fwd)


def test_injected_failure_at_every_step_of_a_streaming_step():
    """A streaming step failed at each of its HIP steps in turn (the fork, the
    local launch, the side stream's wait and launches, the join): REHYAT_EHIP
    with the header unchanged; restoring the checkpoint taken before it then
    continues the stream to the whole-clip forward's bits."""
    g = (1, 2, 10, 100, 128, 3, 1)
    B, H, F, HW, d, Tc, To = g
    w = inputs.custom(*g, dtype="bf16", seed_id=762)
    q, k, v = gpu(*inputs.make_qkv(w))
    y_fwd = rh.attn_fwd(q, k, v, F, HW, Tc, To, "elu1")
    chunks = []
    for f in range(0, F, Tc):
        sl = slice(f * HW, min(f + Tc, F) * HW)
        chunks.append([t[:, :, sl].contiguous() for t in (q, k, v)])
    st = rh.StepState(B, H, HW, d, Tc, To, "elu1")
    outs = [st.step(*chunks[0]), st.step(*chunks[1])]
    n_steps = rh.debug_hip_steps()
    assert n_steps >= 8  # fork, local launch, side wait, state, scan, copy, join record and wait
    sync()
    saved = st.save()
    for i in range(n_steps):
        rh.debug_inject_hip_error(i)
        with pytest.raises(rh.RehyatError, match=f"HIP step {i}"):
            st.step(*chunks[2])
        assert st.header() == saved[1]
        sync()
        st.restore(saved)
    for c in chunks[2:]:
        outs.append(st.step(*c))
    sync()
    assert torch.equal(torch.cat(outs, dim=2), y_fwd)


def test_two_streams_concurrently():
    """Two different clips on two streams at once: each stream has its own
    workspace, so each result equals its single-stream run bit for bit."""
    w = inputs.WORKLOADS["wan_21x30x52"]
    a = gpu(*inputs.make_qkv(w))
    b = gpu(*inputs.make_qkv(w.with_(seed_id=77)))
    F, HW, Tc, To = w.frames, w.tokens_per_frame, w.chunk_frames, w.overlap_frames
    ref_a = rh.attn_fwd(*a, F, HW, Tc, To, "elu1")
    ref_b = rh.attn_fwd(*b, F, HW, Tc, To, "elu1")
    sync()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    out_a = [torch.empty_like(a[0]) for _ in range(4)]
    out_b = [torch.empty_like(b[0]) for _ in range(4)]
    torch.cuda.current_stream().synchronize()
    for i in range(4):  # interleaved: both streams have work in flight at once
        rh.attn_fwd(*a, F, HW, Tc, To, "elu1", out=out_a[i], stream=s1)
        rh.attn_fwd(*b, F, HW, Tc, To, "elu1", out=out_b[i], stream=s2)
    s1.synchronize()
    s2.synchronize()
    for i in range(4):
        assert torch.equal(out_a[i], ref_a) and torch.equal(out_b[i], ref_b), i
    rh.workspace_release(s1)
    rh.workspace_release(s2)
    rh.workspace_release(None)
    again = rh.attn_fwd(*a, F, HW, Tc, To, "elu1", stream=s1)
    s1.synchronize()
    assert torch.equal(again, ref_a)
    rh.workspace_release(s1)
