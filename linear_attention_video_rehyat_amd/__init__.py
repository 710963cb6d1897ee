"""Python binding of librehyat (ReHyAt recurrent hybrid attention forward, MI355X).

Argument marshalling only: torch supplies device memory and the stream; every
step of the computation runs in the HIP kernels of ``librehyat.so``.  The
library must be built first (``python -m linear_attention_video_rehyat_amd.build``);
calls raise :class:`RehyatError` if it is missing -- there is no fallback.

Method: "ReHyAt: Recurrent Hybrid Attention for Video Diffusion Transformers"
(arXiv 2601.04342): local softmax over each temporal chunk plus the T_o frames
before it, feature-mapped linear attention over every earlier key carried as a
chunk-wise RNN state, joint normalisation of the two branches (§3.1-§3.3).
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["RehyatError", "attn_fwd", "attn_fwd_partials", "attn_fwd_lse", "attn_bwd", "StepState",
           "feature_map_id", "MlpWeights", "feature_mlp", "library_path", "load_library", "exported_symbols",
           "workspace_release", "debug_inject_hip_error", "debug_hip_steps", "attn_fwd_noalloc",
           "BlockWeights", "block_fwd", "stack_fwd"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "librehyat.so")
_lib = None

FEATURE_MAPS = {"none": 0, "elu1": 1, "poly2": 2, "mlp2": 3}
DTYPE_F32, DTYPE_BF16 = 0, 1

# every entry point declared in include/rehyat.h
exported_symbols = (
    "rehyat_attn_fwd", "rehyat_attn_fwd_noalloc", "rehyat_noalloc_workspace_limit",
    "rehyat_attn_fwd_f32", "rehyat_attn_fwd_partials",
    "rehyat_attn_fwd_bidir", "rehyat_attn_fwd_bidir_f32", "rehyat_attn_fwd_bidir_partials",
    "rehyat_step_state_bytes", "rehyat_step_state_init", "rehyat_attn_step",
    "rehyat_feature_mlp", "rehyat_attn_fwd_mlp", "rehyat_attn_fwd_mlp_partials", "rehyat_attn_step_mlp",
    "rehyat_attn_fwd_lse", "rehyat_attn_bwd", "rehyat_block_fwd", "rehyat_stack_fwd",
    "rehyat_workspace_release", "rehyat_debug_inject_hip_error", "rehyat_debug_hip_steps",
    "rehyat_set_profile_events", "rehyat_status_string", "rehyat_last_error", "rehyat_version",
)


class RehyatError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class _StepStateC(ctypes.Structure):
    _fields_ = [
        ("buf", ctypes.c_void_p), ("bytes", ctypes.c_size_t),
        ("B", ctypes.c_int), ("H", ctypes.c_int), ("tokens_per_frame", ctypes.c_int),
        ("head_dim", ctypes.c_int), ("chunk_frames", ctypes.c_int), ("overlap_frames", ctypes.c_int),
        ("feature_map", ctypes.c_int), ("dtype", ctypes.c_int),
        ("prev_frames", ctypes.c_int), ("prev_slot", ctypes.c_int), ("state_nonempty", ctypes.c_int),
        ("frames_done", ctypes.c_longlong),
    ]


class _BlockWeightsC(ctypes.Structure):
    _fields_ = [("w_qkv", ctypes.c_void_p), ("b_qkv", ctypes.c_void_p), ("w_o", ctypes.c_void_p),
                ("b_o", ctypes.c_void_p)]


class _MlpC(ctypes.Structure):
    _fields_ = [("w1", ctypes.c_void_p), ("b1", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("b2", ctypes.c_void_p), ("hidden", ctypes.c_int)]


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load librehyat.so (raises RehyatError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RehyatError(-1, f"librehyat.so not found at {_LIB_PATH}; build it with "
                              "`python -m linear_attention_video_rehyat_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i, f_p = ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_float)
    sig_fwd = [vp, vp, vp, vp] + [i] * 8 + [vp]
    for name in ("rehyat_attn_fwd", "rehyat_attn_fwd_noalloc", "rehyat_attn_fwd_f32", "rehyat_attn_fwd_bidir",
                 "rehyat_attn_fwd_bidir_f32"):
        fn = getattr(lib, name)
        fn.argtypes, fn.restype = sig_fwd, i
    for name in ("rehyat_attn_fwd_partials", "rehyat_attn_fwd_bidir_partials"):
        fn = getattr(lib, name)
        fn.argtypes, fn.restype = [vp, vp, vp, i, vp, vp, vp, vp, vp] + [i] * 8 + [vp], i
    lib.rehyat_step_state_bytes.argtypes = [i] * 8
    lib.rehyat_step_state_bytes.restype = ctypes.c_size_t
    lib.rehyat_step_state_init.argtypes = [ctypes.POINTER(_StepStateC), vp, ctypes.c_size_t] + [i] * 8
    lib.rehyat_step_state_init.restype = i
    lib.rehyat_attn_step.argtypes = [ctypes.POINTER(_StepStateC), vp, vp, vp, vp, i, vp]
    lib.rehyat_attn_step.restype = i
    mp = ctypes.POINTER(_MlpC)
    lib.rehyat_feature_mlp.argtypes = [vp, vp, i, i, i, i, i, mp, vp]
    lib.rehyat_feature_mlp.restype = i
    lib.rehyat_attn_fwd_mlp.argtypes = [vp, vp, vp, vp] + [i] * 9 + [mp, mp, vp]
    lib.rehyat_attn_fwd_mlp.restype = i
    lib.rehyat_attn_fwd_mlp_partials.argtypes = [vp, vp, vp, i, vp, vp, vp, vp, vp] + [i] * 8 + [mp, mp, vp]
    lib.rehyat_attn_fwd_mlp_partials.restype = i
    lib.rehyat_attn_step_mlp.argtypes = [ctypes.POINTER(_StepStateC), vp, vp, vp, vp, i, mp, mp, vp]
    lib.rehyat_attn_step_mlp.restype = i
    lib.rehyat_attn_fwd_lse.argtypes = [vp] * 6 + [i] * 10 + [vp]
    lib.rehyat_attn_fwd_lse.restype = i
    bw = ctypes.POINTER(_BlockWeightsC)
    lib.rehyat_block_fwd.argtypes = [vp, vp, bw] + [i] * 9 + [vp]
    lib.rehyat_block_fwd.restype = i
    lib.rehyat_stack_fwd.argtypes = [vp, vp, bw, ctypes.POINTER(ctypes.c_int)] + [i] * 9 + [vp]
    lib.rehyat_stack_fwd.restype = i
    lib.rehyat_attn_bwd.argtypes = [vp] * 10 + [i] * 10 + [vp]
    lib.rehyat_attn_bwd.restype = i
    lib.rehyat_noalloc_workspace_limit.argtypes = []
    lib.rehyat_noalloc_workspace_limit.restype = ctypes.c_size_t
    lib.rehyat_workspace_release.argtypes = [vp]
    lib.rehyat_workspace_release.restype = i
    lib.rehyat_debug_inject_hip_error.argtypes = [i]
    lib.rehyat_debug_inject_hip_error.restype = None
    lib.rehyat_debug_hip_steps.argtypes = []
    lib.rehyat_debug_hip_steps.restype = i
    lib.rehyat_set_profile_events.argtypes = [ctypes.POINTER(ctypes.c_void_p), i]
    lib.rehyat_set_profile_events.restype = i
    lib.rehyat_status_string.argtypes = [i]
    lib.rehyat_status_string.restype = ctypes.c_char_p
    lib.rehyat_last_error.argtypes = []
    lib.rehyat_last_error.restype = ctypes.c_char_p
    lib.rehyat_version.argtypes = []
    lib.rehyat_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        lib = load_library()
        msg = f"{lib.rehyat_status_string(status).decode()}: {lib.rehyat_last_error().decode()}"
        raise RehyatError(status, msg)


def feature_map_id(fm) -> int:
    if isinstance(fm, str):
        return FEATURE_MAPS[fm.lower()]
    return int(fm)


def _torch():
    import torch
    return torch


def _stream_handle(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_id(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise RehyatError(2, f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _check_qkv(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise RehyatError(1, f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise RehyatError(1, f"{name} must be contiguous")
        if t.dim() != 4:
            raise RehyatError(1, f"{name} must be [B, H, N, head_dim]")
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise RehyatError(1, "q, k, v must have the same shape and dtype")


class MlpWeights:
    """Weights of one learned feature map (include/rehyat.h, rehyat_mlp_weights):
    w1 [H, hidden, d] and w2 [H, 2d, hidden] in the dtype of the calls they serve,
    b1 [H, hidden] and b2 [H, 2d] in float32, all contiguous on the GPU."""

    def __init__(self, w1, b1, w2, b2):
        torch = _torch()
        for name, t in (("w1", w1), ("b1", b1), ("w2", w2), ("b2", b2)):
            if not t.is_cuda or not t.is_contiguous():
                raise RehyatError(1, f"{name} must be a contiguous GPU tensor")
        if b1.dtype != torch.float32 or b2.dtype != torch.float32:
            raise RehyatError(1, "b1 and b2 must be float32")
        if w1.dim() != 3 or w2.dim() != 3 or w2.shape[2] != w1.shape[1] or w2.shape[1] != 2 * w1.shape[2]:
            raise RehyatError(1, "expected w1 [H, hidden, d] and w2 [H, 2d, hidden]")
        if tuple(b1.shape) != tuple(w1.shape[:2]) or tuple(b2.shape) != tuple(w2.shape[:2]):
            raise RehyatError(1, "expected b1 [H, hidden] and b2 [H, 2d]")
        self.w1, self.b1, self.w2, self.b2 = w1, b1, w2, b2
        self.hidden = int(w1.shape[1])
        self._c = _MlpC(w1.data_ptr(), b1.data_ptr(), w2.data_ptr(), b2.data_ptr(), self.hidden)

    def check(self, x):
        if self.w1.dtype != x.dtype or self.w1.shape[0] != x.shape[1] or self.w1.shape[2] != x.shape[3]:
            raise RehyatError(1, "feature-map weights do not match the inputs (dtype, H or head_dim)")
        return ctypes.byref(self._c)


def _mlp_pair(feature_map):
    """(phi_q, phi_k) if ``feature_map`` is a pair of MlpWeights, else None."""
    if isinstance(feature_map, (tuple, list)):
        if len(feature_map) != 2 or not all(isinstance(w, MlpWeights) for w in feature_map):
            raise RehyatError(1, "a learned feature map is a pair (phi_q, phi_k) of MlpWeights")
        return feature_map
    return None


def feature_mlp(x, weights, out=None, stream=None):
    """phi of every row of x [B, H, rows, d] with one learned map -> [B, H, rows, 2d]."""
    torch = _torch()
    lib = load_library()
    if not x.is_cuda or not x.is_contiguous() or x.dim() != 4:
        raise RehyatError(1, "x must be a contiguous [B, H, rows, d] GPU tensor")
    B, H, R, d = x.shape
    if out is None:
        out = torch.empty(B, H, R, 2 * d, dtype=x.dtype, device=x.device)
    _check(lib.rehyat_feature_mlp(x.data_ptr(), out.data_ptr(), _dtype_id(x), B, H, R, d, weights.check(x),
                                  _stream_handle(stream)))
    return out


def attn_fwd(q, k, v, frames, tokens_per_frame, chunk_frames, overlap_frames, feature_map="elu1",
             out=None, stream=None, causal=True):
    """Whole-clip hybrid attention forward.  q, k, v: [B, H, frames*tokens_per_frame, d]
    (bf16 or fp32, contiguous, on the GPU).  Returns ``out`` (allocated if None).
    causal=False selects the bidirectional form (keys of later chunks join the
    linear set).  ``feature_map`` is a name ("elu1", "poly2", "none") or a pair
    (phi_q, phi_k) of MlpWeights (the learned map)."""
    torch = _torch()
    lib = load_library()
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    if N != frames * tokens_per_frame:
        raise RehyatError(1, f"N={N} != frames*tokens_per_frame={frames * tokens_per_frame}")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or not out.is_cuda:
        raise RehyatError(1, "out must be a contiguous GPU tensor matching q")
    pair = _mlp_pair(feature_map)
    if pair is not None:
        _check(lib.rehyat_attn_fwd_mlp(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), _dtype_id(q),
                                       B, H, frames, tokens_per_frame, d, chunk_frames, overlap_frames,
                                       1 if causal else 0, pair[0].check(q), pair[1].check(k),
                                       _stream_handle(stream)))
        return out
    bf16 = _dtype_id(q) == DTYPE_BF16
    if causal:
        fn = lib.rehyat_attn_fwd if bf16 else lib.rehyat_attn_fwd_f32
    else:
        fn = lib.rehyat_attn_fwd_bidir if bf16 else lib.rehyat_attn_fwd_bidir_f32
    _check(fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, frames,
              tokens_per_frame, d, chunk_frames, overlap_frames, feature_map_id(feature_map),
              _stream_handle(stream)))
    return out


def attn_fwd_noalloc(q, k, v, frames, tokens_per_frame, chunk_frames, overlap_frames, feature_map="elu1",
                     out=None, stream=None):
    """rehyat_attn_fwd_noalloc: the bf16 recurrent forward with its workspace in
    the library's fixed per-device array (no device allocation by the library;
    ``out`` should be passed by callers that allocate nothing either)."""
    torch = _torch()
    lib = load_library()
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    if N != frames * tokens_per_frame:
        raise RehyatError(1, f"N={N} != frames*tokens_per_frame={frames * tokens_per_frame}")
    if q.dtype != torch.bfloat16:
        raise RehyatError(2, "rehyat_attn_fwd_noalloc takes bf16 tensors")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or not out.is_cuda:
        raise RehyatError(1, "out must be a contiguous GPU tensor matching q")
    _check(lib.rehyat_attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, frames,
                                       tokens_per_frame, d, chunk_frames, overlap_frames,
                                       feature_map_id(feature_map), _stream_handle(stream)))
    return out


def attn_fwd_partials(q, k, v, frames, tokens_per_frame, chunk_frames, overlap_frames,
                      feature_map="elu1", stream=None, causal=True):
    """Per-query partials of both branches (verification aid): dict with m, nt,
    o_s, o_l, n_l as fp32 tensors (see include/rehyat.h)."""
    torch = _torch()
    lib = load_library()
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    f32 = dict(dtype=torch.float32, device=q.device)
    parts = {"m": torch.empty(B, H, N, **f32), "nt": torch.empty(B, H, N, **f32),
             "o_s": torch.empty(B, H, N, d, **f32), "o_l": torch.empty(B, H, N, d, **f32),
             "n_l": torch.empty(B, H, N, **f32)}
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_id(q),
            parts["m"].data_ptr(), parts["nt"].data_ptr(), parts["o_s"].data_ptr(),
            parts["o_l"].data_ptr(), parts["n_l"].data_ptr(), B, H, frames, tokens_per_frame, d,
            chunk_frames, overlap_frames)
    pair = _mlp_pair(feature_map)
    if pair is not None:
        _check(lib.rehyat_attn_fwd_mlp_partials(*ptrs, 1 if causal else 0, pair[0].check(q), pair[1].check(k),
                                                _stream_handle(stream)))
        return parts
    fn = lib.rehyat_attn_fwd_partials if causal else lib.rehyat_attn_fwd_bidir_partials
    _check(fn(*ptrs, feature_map_id(feature_map), _stream_handle(stream)))
    return parts


def attn_fwd_lse(q, k, v, frames, tokens_per_frame, chunk_frames, overlap_frames, feature_map="elu1",
                 out=None, lse=None, stream=None, causal=True, out_f32=None):
    """Forward that also returns lse [B, H, N] fp32 = ln(n^S + n^L) per query,
    the normaliser the backward needs: (out, lse).  out_f32=True (or a float32
    tensor shaped like q) also keeps the bf16 call's output before rounding:
    (out, lse, out_f32)."""
    torch = _torch()
    lib = load_library()
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or not out.is_cuda:
        raise RehyatError(1, "out must be a contiguous GPU tensor matching q")
    if lse is None:
        lse = torch.empty(B, H, N, dtype=torch.float32, device=q.device)
    elif (tuple(lse.shape) != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous()
          or not lse.is_cuda):
        raise RehyatError(1, "lse must be a contiguous float32 [B, H, N] GPU tensor")
    want32 = out_f32 is not None and out_f32 is not False
    if out_f32 is True:
        out_f32 = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    _check(lib.rehyat_attn_fwd_lse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                   out_f32.data_ptr() if want32 else None, _dtype_id(q), B, H, frames,
                                   tokens_per_frame, d, chunk_frames, overlap_frames, feature_map_id(feature_map),
                                   1 if causal else 0, _stream_handle(stream)))
    return (out, lse, out_f32) if want32 else (out, lse)


def attn_bwd(q, k, v, out, lse, dout, frames, tokens_per_frame, chunk_frames, overlap_frames,
             feature_map="elu1", grads=None, stream=None, causal=True, out_f32=None):
    """Gradients (dq, dk, dv) of sum(dout * out) for the hybrid attention (the
    forward's partition), given its inputs, out and lse (attn_fwd_lse)."""
    torch = _torch()
    lib = load_library()
    _check_qkv(q, k, v)
    for name, t in (("out", out), ("dout", dout)):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous() or not t.is_cuda:
            raise RehyatError(1, f"{name} must match q")
    B, H, N, d = q.shape
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise RehyatError(1, "lse must be a contiguous float32 [B, H, N] tensor")
    dq, dk, dv = grads if grads is not None else (torch.empty_like(q), torch.empty_like(q), torch.empty_like(q))
    for t in (dq, dk, dv):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous() or not t.is_cuda:
            raise RehyatError(1, "gradients must be contiguous GPU tensors matching q")
    if out_f32 is not None and (out_f32.shape != q.shape or out_f32.dtype != torch.float32
                                or not out_f32.is_contiguous()):
        raise RehyatError(1, "out_f32 must be a contiguous float32 tensor shaped like q")
    _check(lib.rehyat_attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                               out_f32.data_ptr() if out_f32 is not None else None, lse.data_ptr(),
                               dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), _dtype_id(q),
                               B, H, frames, tokens_per_frame, d, chunk_frames, overlap_frames,
                               feature_map_id(feature_map), 1 if causal else 0, _stream_handle(stream)))
    return dq, dk, dv


def workspace_release(stream=None):
    """Wait for the stream's queued work and free its workspace arena."""
    _check(load_library().rehyat_workspace_release(_stream_handle(stream)))


def debug_inject_hip_error(step: int):
    """Test hook: the next call that reaches HIP step ``step`` fails there with
    REHYAT_EHIP without making that HIP call; a negative step disarms."""
    load_library().rehyat_debug_inject_hip_error(int(step))


def debug_hip_steps() -> int:
    """HIP steps (runtime calls and launches) of the last call on this thread."""
    return int(load_library().rehyat_debug_hip_steps())


class BlockWeights:
    """Projection weights of one attention block (include/rehyat.h,
    rehyat_block_weights): w_qkv [3C, C] and w_o [C, C] bf16 (out x in), b_qkv
    [3C] and b_o [C] float32, contiguous on the GPU."""

    def __init__(self, w_qkv, b_qkv, w_o, b_o):
        torch = _torch()
        for name, t in (("w_qkv", w_qkv), ("b_qkv", b_qkv), ("w_o", w_o), ("b_o", b_o)):
            if not t.is_cuda or not t.is_contiguous():
                raise RehyatError(1, f"{name} must be a contiguous GPU tensor")
        if w_qkv.dtype != torch.bfloat16 or w_o.dtype != torch.bfloat16:
            raise RehyatError(1, "w_qkv and w_o must be bfloat16")
        if b_qkv.dtype != torch.float32 or b_o.dtype != torch.float32:
            raise RehyatError(1, "b_qkv and b_o must be float32")
        C = w_o.shape[0]
        if (w_qkv.shape != (3 * C, C) or w_o.shape != (C, C) or tuple(b_qkv.shape) != (3 * C,)
                or tuple(b_o.shape) != (C,)):
            raise RehyatError(1, "expected w_qkv [3C, C], b_qkv [3C], w_o [C, C], b_o [C]")
        self.tensors = (w_qkv, b_qkv, w_o, b_o)
        self.C = C
        self._c = _BlockWeightsC(w_qkv.data_ptr(), b_qkv.data_ptr(), w_o.data_ptr(), b_o.data_ptr())


def _check_block_x(x, weights):
    torch = _torch()
    if not x.is_cuda or not x.is_contiguous() or x.dim() != 3 or x.dtype != torch.bfloat16:
        raise RehyatError(1, "x must be a contiguous bfloat16 [B, N, C] GPU tensor")
    if x.shape[2] != weights.C:
        raise RehyatError(1, f"x has {x.shape[2]} channels, the weights {weights.C}")


def block_fwd(x, weights, frames, tokens_per_frame, heads, hybrid=True, chunk_frames=3, overlap_frames=1,
              feature_map="elu1", out=None, stream=None):
    """One attention block, out = x + A(x) (rehyat_block_fwd): x [B, N, C] bf16,
    N = frames * tokens_per_frame, C = heads * head_dim; hybrid=False gives the
    block with full softmax attention."""
    torch = _torch()
    lib = load_library()
    _check_block_x(x, weights)
    B, N, C = x.shape
    if out is None:
        out = torch.empty_like(x)
    _check(lib.rehyat_block_fwd(x.data_ptr(), out.data_ptr(), ctypes.byref(weights._c), B, frames, tokens_per_frame,
                                heads, C // heads, 1 if hybrid else 0, chunk_frames, overlap_frames,
                                feature_map_id(feature_map), _stream_handle(stream)))
    return out


def stack_fwd(x, weights, hybrid, frames, tokens_per_frame, heads, chunk_frames=3, overlap_frames=1,
              feature_map="elu1", out=None, stream=None):
    """A stack of blocks (rehyat_stack_fwd): weights is a list of BlockWeights,
    hybrid a list of booleans of the same length (which blocks use the hybrid
    attention)."""
    torch = _torch()
    lib = load_library()
    if len(weights) != len(hybrid) or not weights:
        raise RehyatError(1, "weights and hybrid must be non-empty lists of the same length")
    for w in weights:
        _check_block_x(x, w)
    B, N, C = x.shape
    if out is None:
        out = torch.empty_like(x)
    arr = (_BlockWeightsC * len(weights))(*[w._c for w in weights])
    flags = (ctypes.c_int * len(hybrid))(*[1 if h else 0 for h in hybrid])
    _check(lib.rehyat_stack_fwd(x.data_ptr(), out.data_ptr(), arr, flags, len(weights), B, frames,
                                tokens_per_frame, heads, C // heads, chunk_frames, overlap_frames,
                                feature_map_id(feature_map), _stream_handle(stream)))
    return out


def set_profile_events(events):
    """Record 4 caller-owned hipEvent_t handles around the kernels of every
    forward call on this thread (see include/rehyat.h); None to stop."""
    lib = load_library()
    if events is None:
        _check(lib.rehyat_set_profile_events(None, 0))
        return
    arr = (ctypes.c_void_p * 4)(*[ctypes.c_void_p(int(e)) for e in events])
    _check(lib.rehyat_set_profile_events(arr, 4))


class StepState:
    """Streaming (chunk-wise RNN) state: a device buffer owned by this object
    plus the library's host header.  ``step`` attends one chunk of frames."""

    def __init__(self, B, H, tokens_per_frame, head_dim, chunk_frames, overlap_frames,
                 feature_map="elu1", dtype=None, device="cuda"):
        torch = _torch()
        lib = load_library()
        dtype = torch.bfloat16 if dtype is None else dtype
        self.dtype = dtype
        did = DTYPE_BF16 if dtype == torch.bfloat16 else DTYPE_F32
        self.mlp = _mlp_pair(feature_map)  # learned maps: passed again on every step
        fm = FEATURE_MAPS["mlp2"] if self.mlp is not None else feature_map_id(feature_map)
        nbytes = lib.rehyat_step_state_bytes(B, H, tokens_per_frame, head_dim, chunk_frames,
                                             overlap_frames, fm, did)
        if nbytes == 0:  # invalid geometry: let init report why
            probe = _StepStateC()
            _check(lib.rehyat_step_state_init(ctypes.byref(probe), None, 0, B, H, tokens_per_frame,
                                              head_dim, chunk_frames, overlap_frames, fm, did))
        self.buf = torch.empty(int(nbytes), dtype=torch.uint8, device=device)
        self._c = _StepStateC()
        _check(lib.rehyat_step_state_init(ctypes.byref(self._c), self.buf.data_ptr(), int(nbytes),
                                          B, H, tokens_per_frame, head_dim, chunk_frames,
                                          overlap_frames, fm, did))
        self.shape = (B, H, tokens_per_frame, head_dim)

    @property
    def nbytes(self) -> int:
        return int(self._c.bytes)

    @property
    def frames_done(self) -> int:
        return int(self._c.frames_done)

    def header(self) -> dict:
        return {name: getattr(self._c, name) for name, _ in _StepStateC._fields_ if name != "buf"}

    def step(self, q, k, v, out=None, stream=None):
        torch = _torch()
        lib = load_library()
        _check_qkv(q, k, v)
        if q.dtype != self.dtype:
            raise RehyatError(1, f"chunk dtype {q.dtype} != state dtype {self.dtype}")
        B, H, n, d = q.shape
        HW = self._c.tokens_per_frame
        if n % HW != 0:
            raise RehyatError(1, f"chunk rows {n} not a multiple of tokens_per_frame {HW}")
        if out is None:
            out = torch.empty_like(q)
        elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or not out.is_cuda:
            raise RehyatError(1, "out must be a contiguous GPU tensor matching the chunk")
        if self.mlp is not None:
            _check(lib.rehyat_attn_step_mlp(ctypes.byref(self._c), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                            out.data_ptr(), n // HW, self.mlp[0].check(q), self.mlp[1].check(k),
                                            _stream_handle(stream)))
            return out
        _check(lib.rehyat_attn_step(ctypes.byref(self._c), q.data_ptr(), k.data_ptr(),
                                    v.data_ptr(), out.data_ptr(), n // HW, _stream_handle(stream)))
        return out

    def save(self):
        """(host copy of the device buffer, header) -- a checkpoint of the stream."""
        return self.buf.cpu().clone(), self.header()

    def restore(self, saved):
        buf, header = saved
        self.buf.copy_(buf)
        for name, value in header.items():
            if name != "bytes":
                setattr(self._c, name, value)
