"""rehyat_attn_fwd_noalloc, the allocation-free forward: through the C ABI it
gives the bits of rehyat_attn_fwd on two calls in a row (the second on a
smaller clip, so stale contents of the shared fixed workspace would show), and
the device's free memory does not change across a call."""
import ctypes

import pytest
import torch

import linear_attention_video_rehyat_amd as rh
from linear_attention_video_rehyat_amd import inputs
from tests.parity_util import gpu, sync

pytestmark = pytest.mark.gpu


def _free_bytes():
    hip = ctypes.CDLL("libamdhip64.so")
    free, total = ctypes.c_size_t(), ctypes.c_size_t()
    assert hip.hipMemGetInfo(ctypes.byref(free), ctypes.byref(total)) == 0
    return free.value


@pytest.mark.parametrize("phi", ["elu1", "poly2", "none"])
def test_noalloc_matches_fwd_twice_second_smaller(phi):
    big = inputs.WORKLOADS["wan_21x30x52"]
    small = inputs.custom(1, 3, 7, 100, 128, 2, 1, dtype="bf16", seed_id=810)
    cases = []
    for w in (big, small):
        q, k, v = gpu(*inputs.make_qkv(w))
        geo = (w.frames, w.tokens_per_frame, w.chunk_frames, w.overlap_frames)
        cases.append(((q, k, v), geo, rh.attn_fwd(q, k, v, *geo, phi), torch.full_like(q, float("nan"))))
    # the fixed array exists once the library's code object is loaded on the
    # device; a first call makes sure it is before free memory is compared
    (q, k, v), geo, _, out = cases[1]
    rh.attn_fwd_noalloc(q, k, v, *geo, phi, out=out)
    sync()
    free0 = _free_bytes()
    for (q, k, v), geo, _, out in cases:  # back to back: big, then small
        rh.attn_fwd_noalloc(q, k, v, *geo, phi, out=out)
    sync()
    assert _free_bytes() == free0, "a call allocated device memory"
    for (_, _, ref, out), w in zip(cases, (big, small)):
        assert torch.equal(out, ref), (w.name, phi)


def test_noalloc_rejects_workspace_beyond_the_limit():
    """The 105-frame clip needs about 108 MB of workspace: REHYAT_ENOMEM with
    the limit named, nothing queued (checked before any HIP call)."""
    w = inputs.WORKLOADS["wan_long_105x30x52"]
    lib = rh.load_library()
    big = torch.empty(w.B, w.H, w.N, w.head_dim, dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(big)
    st = lib.rehyat_attn_fwd_noalloc(big.data_ptr(), big.data_ptr(), big.data_ptr(), out.data_ptr(), w.B, w.H,
                                     w.frames, w.tokens_per_frame, w.head_dim, 3, 1, 1, rh._stream_handle(None))
    assert st == 3 and "fixed scratch" in lib.rehyat_last_error().decode()
    assert lib.rehyat_noalloc_workspace_limit() == 64 << 20
