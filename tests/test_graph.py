"""HIP graph capture of the library's calls (torch.cuda.graph on a stream of its
own): the whole-clip forward, the allocation-free forward and a whole stream of
streaming steps (its side stream joins the capture through the fork and join
events).  Each graph is replayed several times with other GPU work and
synchronisations in between, and every replay is compared bit for bit with the
eager result.  Nothing the library queues records a memset; the workspace and
the side stream are created by an eager call on the capture stream first."""
import pytest
import torch

import linear_attention_video_rehyat_amd as rh
from linear_attention_video_rehyat_amd import inputs
from tests.parity_util import gpu, sync

pytestmark = pytest.mark.gpu

G = (1, 3, 10, 150, 128, 3, 1)  # B, H, frames, tokens per frame, d, T_c, T_o


def _clip(seed):
    return gpu(*inputs.make_qkv(inputs.custom(*G, dtype="bf16", seed_id=seed)))


def _other_work(i):
    x = torch.randn(1 << 20, device="cuda") * (i + 1)
    return float(x.abs().max())


@pytest.mark.parametrize("phi", ["elu1", "none"])
def test_forward_graph_replays(phi):
    B, H, F, HW, d, Tc, To = G
    q, k, v = _clip(650)
    ref = rh.attn_fwd(q, k, v, F, HW, Tc, To, phi)
    out = torch.empty_like(q)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        rh.attn_fwd(q, k, v, F, HW, Tc, To, phi, out=out, stream=s)  # the stream's workspace
    sync()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        rh.attn_fwd(q, k, v, F, HW, Tc, To, phi, out=out, stream=s)
    for i in range(4):
        out.zero_()
        _other_work(i)
        g.replay()
        sync()
        assert torch.equal(out, ref), f"replay {i}"
    rh.workspace_release(s)


def test_noalloc_forward_graph_replays():
    B, H, F, HW, d, Tc, To = G
    q, k, v = _clip(651)
    ref = rh.attn_fwd(q, k, v, F, HW, Tc, To, "elu1")
    out = torch.empty_like(q)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        rh.attn_fwd_noalloc(q, k, v, F, HW, Tc, To, "elu1", out=out, stream=s)
    sync()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        rh.attn_fwd_noalloc(q, k, v, F, HW, Tc, To, "elu1", out=out, stream=s)
    for i in range(3):
        out.zero_()
        _other_work(i)
        g.replay()
        sync()
        assert torch.equal(out, ref), f"replay {i}"


def test_whole_stream_graph_replays():
    """A whole stream captured from a fresh state (whose buffer needs no
    initialisation) replays as the same stream again: every replay equals the
    whole-clip forward."""
    B, H, F, HW, d, Tc, To = G
    q, k, v = _clip(652)
    ref = rh.attn_fwd(q, k, v, F, HW, Tc, To, "elu1")
    chunks = [[t[:, :, f * HW:min(f + Tc, F) * HW].contiguous() for t in (q, k, v)] for f in range(0, F, Tc)]
    outs = [torch.empty_like(c[0]) for c in chunks]
    s = torch.cuda.Stream()
    warm = rh.StepState(B, H, HW, d, Tc, To, "elu1")
    with torch.cuda.stream(s):
        for c, o in zip(chunks, outs):
            warm.step(*c, out=o, stream=s)  # the side stream of s
    sync()
    assert torch.equal(torch.cat(outs, dim=2), ref)
    st = rh.StepState(B, H, HW, d, Tc, To, "elu1")
    sync()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for c, o in zip(chunks, outs):
            st.step(*c, out=o, stream=s)
    for i in range(3):
        for o in outs:
            o.zero_()
        _other_work(i)
        g.replay()
        sync()
        assert torch.equal(torch.cat(outs, dim=2), ref), f"replay {i}"
    rh.workspace_release(s)
