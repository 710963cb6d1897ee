"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/rehyat.h, and rejects invalid arguments on the host before
any GPU work (these calls never reach the HIP runtime)."""
import ctypes
import os
import re

import pytest

import linear_attention_video_rehyat_amd as rh

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rehyat.h")

pytestmark = pytest.mark.skipif(not os.path.exists(rh.library_path()),
                                reason="librehyat.so not built")

EINVAL, EUNSUPPORTED = 1, 2
FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(rehyat_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = rh.load_library()
    names = declared_functions()
    assert len(names) >= 9
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(rh.exported_symbols)


def test_status_strings_and_version():
    lib = rh.load_library()
    assert lib.rehyat_status_string(0) == b"ok"
    assert lib.rehyat_status_string(1) == b"invalid argument"
    assert lib.rehyat_status_string(99) == b"unknown status"
    assert lib.rehyat_version().startswith(b"librehyat")


def _fwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE * 4, B=1, H=1, F=4, HW=8, d=64, Tc=1, To=1, phi=1)
    a.update(kw)
    return lib.rehyat_attn_fwd(a["q"], a["k"], a["v"], a["out"], a["B"], a["H"], a["F"], a["HW"],
                               a["d"], a["Tc"], a["To"], a["phi"], None)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(B=0), EINVAL, "B and H"),
    (dict(H=-1), EINVAL, "B and H"),
    (dict(F=0), EINVAL, "frames"),
    (dict(HW=0), EINVAL, "frames"),
    (dict(Tc=0), EINVAL, "chunk_frames"),
    (dict(To=-1), EINVAL, "overlap_frames"),
    (dict(phi=7), EINVAL, "feature_map"),
    (dict(d=48), EUNSUPPORTED, "head_dim"),
    (dict(d=16), EUNSUPPORTED, "head_dim"),
    (dict(q=0), EINVAL, "null"),
    (dict(out=0), EINVAL, "null"),
    (dict(k=FAKE + 2), EINVAL, "aligned"),
    (dict(out=FAKE), EINVAL, "overlap"),
    (dict(F=1 << 20, HW=1 << 20), EINVAL, "too large"),
])
def test_fwd_validation(kw, code, needle):
    lib = rh.load_library()
    assert _fwd(lib, **kw) == code
    assert needle in lib.rehyat_last_error().decode()


def test_f32_head_dims():
    lib = rh.load_library()
    st = lib.rehyat_attn_fwd_f32(FAKE, FAKE, FAKE, FAKE * 4, 1, 1, 2, 4, 8, 1, 0, 1, None)
    assert st == EUNSUPPORTED


def test_partials_validation():
    lib = rh.load_library()
    st = lib.rehyat_attn_fwd_partials(FAKE, FAKE, FAKE, 1, None, None, None, None, None,
                                      1, 1, 4, 8, 64, 1, 1, 1, None)
    assert st == EINVAL and "no partial" in lib.rehyat_last_error().decode()
    st = lib.rehyat_attn_fwd_partials(FAKE, FAKE, FAKE, 5, FAKE, None, None, None, None,
                                      1, 1, 4, 8, 64, 1, 1, 1, None)
    assert st == EINVAL and "dtype" in lib.rehyat_last_error().decode()


def test_step_state_bytes_constant_in_video_length():
    """The streaming state is sized by the chunk geometry alone (constant memory)."""
    lib = rh.load_library()
    n = lib.rehyat_step_state_bytes(1, 12, 1560, 128, 3, 1, 1, 1)
    assert n > 0
    # holds S (d x D' + D' fp32), prepared hi/lo copies, two overlap slots of T_o frames
    assert n >= 12 * (128 * 128 + 128) * 4 + 2 * 2 * 12 * 1560 * 128 * 2
    assert lib.rehyat_step_state_bytes(0, 12, 1560, 128, 3, 1, 1, 1) == 0
    assert lib.rehyat_step_state_bytes(1, 12, 1560, 100, 3, 1, 1, 1) == 0
    # POLY2 doubles the feature dimension
    assert lib.rehyat_step_state_bytes(1, 12, 1560, 128, 3, 1, 2, 1) > n


def test_step_state_init_and_step_validation():
    lib = rh.load_library()
    st = rh._StepStateC()
    need = lib.rehyat_step_state_bytes(1, 2, 8, 64, 2, 1, 1, 1)
    assert lib.rehyat_step_state_init(ctypes.byref(st), FAKE, need - 1, 1, 2, 8, 64, 2, 1, 1, 1) == EINVAL
    assert "too small" in lib.rehyat_last_error().decode()
    assert lib.rehyat_step_state_init(ctypes.byref(st), FAKE + 8, need, 1, 2, 8, 64, 2, 1, 1, 1) == EINVAL
    assert lib.rehyat_step_state_init(ctypes.byref(st), FAKE, need, 1, 2, 8, 64, 2, 1, 1, 1) == 0
    assert st.frames_done == 0 and st.prev_frames == 0 and st.state_nonempty == 0
    # frames outside [1, chunk_frames] are rejected before any GPU work
    assert lib.rehyat_attn_step(ctypes.byref(st), FAKE, FAKE, FAKE, FAKE * 64, 3, None) == EINVAL
    assert lib.rehyat_attn_step(ctypes.byref(st), FAKE, FAKE, FAKE, FAKE * 64, 0, None) == EINVAL
    assert lib.rehyat_attn_step(ctypes.byref(st), 0, FAKE, FAKE, FAKE * 64, 1, None) == EINVAL
    # a stream that ended with a partial chunk takes no more chunks
    st.frames_done = 3
    assert lib.rehyat_attn_step(ctypes.byref(st), FAKE, FAKE, FAKE, FAKE * 64, 2, None) == EINVAL
    assert "partial" in lib.rehyat_last_error().decode()
    assert lib.rehyat_attn_step(None, FAKE, FAKE, FAKE, FAKE, 1, None) == EINVAL


def test_binding_fails_loudly_without_gpu_tensors():
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(rh.RehyatError):
        rh.attn_fwd(q, q, q, 1, 8, 1, 0)


def test_local_work_order_is_a_permutation(tmp_path):
    """The local kernel's workgroup -> work-item map (natural and longest-first
    order) is a bijection that keeps each XCD's share of items; host-side build
    of kernels.h with hipcc, run on the CPU."""
    import shutil
    import subprocess
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    src = os.path.join(ROOT, "tests", "native", "work_order_check.cpp")
    exe = str(tmp_path / "work_order_check")
    csrc = os.path.join(ROOT, "linear_attention_video_rehyat_amd", "csrc")
    build = subprocess.run([hipcc, "-O1", "-std=c++17", "-x", "hip", "--offload-arch=gfx950", f"-I{csrc}",
                            src, "-o", exe], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-2000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "0 violations" in run.stdout


def test_key_block_partition(tmp_path):
    """The key blocks of the state pass and the scan (kernels.h): each chunk's
    linear set is exactly the keys outside its softmax window, recurrent and
    bidirectional (ReHyAt §3.2, §3.3), assembled from whole blocks; sub-blocks
    cover every block's rows; the state kernel's workgroup decode visits every
    (block, sub-block) once.  Host-side build with hipcc, run on the CPU."""
    import shutil
    import subprocess
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    src = os.path.join(ROOT, "tests", "native", "block_partition_check.cpp")
    exe = str(tmp_path / "block_partition_check")
    csrc = os.path.join(ROOT, "linear_attention_video_rehyat_amd", "csrc")
    build = subprocess.run([hipcc, "-O1", "-std=c++17", "-x", "hip", "--offload-arch=gfx950", f"-I{csrc}",
                            src, "-o", exe], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-2000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert " 0 violations" in run.stdout


EHIP = 4


def test_row_extent_limit():
    """Rows of one (b, h) are addressed with 32-bit byte offsets: a clip whose
    rows reach 2^31 bytes is rejected on the host; one row less passes the
    checks (the armed fault-injection hook then stops the call at its first
    HIP step, so nothing reaches the runtime)."""
    lib = rh.load_library()
    # bf16, head_dim 128: 256 bytes per row, limit 2^23 rows
    assert _fwd(lib, F=8192, HW=1024, d=128) == EUNSUPPORTED
    assert "2^31" in lib.rehyat_last_error().decode()
    rh.debug_inject_hip_error(0)
    try:
        st = _fwd(lib, F=8191, HW=1024, d=128, out=FAKE * (1 << 16))
    finally:
        rh.debug_inject_hip_error(-1)
    assert st == EHIP and "injected" in lib.rehyat_last_error().decode()
    # fp32 at head_dim 64: 256 bytes per row as well
    assert lib.rehyat_attn_fwd_f32(FAKE, FAKE, FAKE, FAKE * (1 << 16), 1, 1, 8192, 1024, 64, 3, 1, 1,
                                   None) == EUNSUPPORTED
    # the learned maps' feature rows are twice as wide: the limit halves
    w = (ctypes.c_void_p * 4)()
    mlp = rh._MlpC(FAKE, FAKE, FAKE, FAKE, 256)
    st = lib.rehyat_attn_fwd_mlp(FAKE, FAKE, FAKE, FAKE * (1 << 16), 1, 1, 1, 4096, 1024, 128, 3, 1, 1,
                                 ctypes.byref(mlp), ctypes.byref(mlp), None)
    assert st == EUNSUPPORTED and "2^31" in lib.rehyat_last_error().decode()
    # the streaming state checks the same bound on its chunk geometry
    assert lib.rehyat_step_state_bytes(1, 1, 1 << 22, 128, 2, 1, 1, 1) == 0


@pytest.mark.parametrize("entry", ["fwd", "fwd_none", "bidir", "partials", "bwd", "step"])
def test_fault_injection_returns_ehip_before_any_hip_call(entry):
    """A HIP failure forced from the host: with the hook armed at step 0 a
    valid call stops at its first HIP step and reports REHYAT_EHIP with
    the hook named; nothing is queued, so this runs without a GPU."""
    lib = rh.load_library()
    base = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, out=FAKE * 4, B=1, H=1, F=4, HW=8, d=64, Tc=1, To=1)
    rh.debug_inject_hip_error(0)
    try:
        if entry == "fwd":
            st = _fwd(lib, **base)
        elif entry == "fwd_none":
            st = _fwd(lib, **base, phi=0)
        elif entry == "bidir":
            st = lib.rehyat_attn_fwd_bidir(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, 1, 1, 4, 8, 64, 1, 1, 1, None)
        elif entry == "partials":
            st = lib.rehyat_attn_fwd_partials(FAKE, FAKE * 2, FAKE * 3, 1, FAKE * 4, None, None, None, None,
                                              1, 1, 4, 8, 64, 1, 1, 1, None)
        elif entry == "bwd":
            p = [FAKE * (i + 1) * 4096 for i in range(10)]
            st = lib.rehyat_attn_bwd(p[0], p[1], p[2], p[3], None, p[4], p[5], p[6], p[7], p[8], 1,
                                     1, 1, 4, 8, 64, 1, 1, 1, 1, None)
        else:
            s = rh._StepStateC()
            need = lib.rehyat_step_state_bytes(1, 1, 8, 64, 1, 1, 1, 1)
            assert lib.rehyat_step_state_init(ctypes.byref(s), FAKE * 4096, need, 1, 1, 8, 64, 1, 1, 1, 1) == 0
            st = lib.rehyat_attn_step(ctypes.byref(s), FAKE, FAKE * 2, FAKE * 3, FAKE * 64, 1, None)
            # a failed step leaves the stream where it was
            assert s.frames_done == 0 and s.prev_frames == 0
    finally:
        rh.debug_inject_hip_error(-1)
    msg = lib.rehyat_last_error().decode()
    assert st == EHIP, (st, msg)
    assert "injected failure at HIP step 0" in msg
    assert rh.debug_hip_steps() == 1


def test_fault_injection_hook_is_one_shot_and_disarms():
    lib = rh.load_library()
    rh.debug_inject_hip_error(0)
    rh.debug_inject_hip_error(-1)
    # disarmed: a call that fails validation reports that, not an injected failure
    assert _fwd(lib, B=0) == EINVAL
    assert "B and H" in lib.rehyat_last_error().decode()


def test_noalloc_validation_and_limit():
    """The allocation-free forward validates like rehyat_attn_fwd and rejects
    a call whose workspace exceeds its fixed array before any HIP call."""
    lib = rh.load_library()
    assert lib.rehyat_noalloc_workspace_limit() == 64 << 20
    st = lib.rehyat_attn_fwd_noalloc(FAKE, FAKE, FAKE, FAKE * 4, 0, 1, 4, 8, 64, 1, 1, 1, None)
    assert st == EINVAL and "B and H" in lib.rehyat_last_error().decode()
    # 105 frames of 1560 tokens, 12 heads of 128, elu+1: ~108 MB of workspace
    big = 1 << 32
    st = lib.rehyat_attn_fwd_noalloc(big, big * 2, big * 3, big * 4, 1, 12, 105, 1560, 128, 3, 1, 1, None)
    assert st == 3 and "fixed scratch" in lib.rehyat_last_error().decode()
    # valid calls, stopped at their first HIP step (the workspace lookup, or
    # the launch when no chunk has a linear set and no workspace is needed)
    for phi in (1, 0):
        rh.debug_inject_hip_error(0)
        try:
            st = lib.rehyat_attn_fwd_noalloc(big, big * 2, big * 3, big * 4, 1, 12, 21, 1560, 128, 3, 1, phi, None)
        finally:
            rh.debug_inject_hip_error(-1)
        assert st == EHIP and "injected" in lib.rehyat_last_error().decode()
        assert rh.debug_hip_steps() == 1
