"""Plain fp64 CPU oracle for the ReHyAt hybrid attention forward.

TEST INFRASTRUCTURE ONLY.  This module is the correctness reference the GPU
library is checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code with the
GPU library and never imports it.

Source throughout: "ReHyAt: Recurrent Hybrid Attention for Video Diffusion
Transformers" (Ghafoorian & Habibian, arXiv 2601.04342), §3.1-§3.3.

Three independent forms of the same computation live here:

* :func:`definition` -- the fp64 C code in ``rehyat_oracle.c``: per query, an
  explicit walk over every key that classifies it as softmax / linear / ignored
  by the §3.3 partition, literal exponentials, joint normalisation (§3.2).
* :func:`brute_force` -- a numpy matrix form for tiny inputs: 0/1 masks built
  from the §3.3 set definitions written in token units, ``W = exp(QK^T)*M_S +
  (phi(Q) phi(K)^T)*M_L``, ``Y = W V / rowsum(W)``.
* :class:`RecurrentState` / :func:`recurrent` -- the chunk-wise RNN form the
  paper derives (ReHyAt page, Abstract and §3.3: processed chunk by chunk, the
  method's memory stays fixed as the video grows): chunks in order, carrying the linear sums (S, z) of
  §3.1 plus the keys/values of the last T_o frames (the next chunk's overlap).

Readings where the text is silent are listed in ``rehyat_oracle.c``'s header;
they apply here too.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

PHI_NONE, PHI_ELU1, PHI_POLY2, PHI_GIVEN = 0, 1, 2, 3
PHI_NAMES = {"none": PHI_NONE, "elu1": PHI_ELU1, "poly2": PHI_POLY2}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rehyat_oracle.c")
_LIB_PATH = os.path.join(_HERE, "librehyat_oracle.so")
_lib = None


def phi_kind(phi) -> int:
    """Kind of a feature-map argument: a name or code of a fixed map, or a pair
    (phi_q, phi_k) of callables (separate maps for queries and keys, such as two
    :class:`MlpFeatureMap` objects), which is PHI_GIVEN."""
    if isinstance(phi, (tuple, list)):
        return PHI_GIVEN
    if isinstance(phi, str):
        return PHI_NAMES[phi.lower()]
    return int(phi)


class MlpFeatureMap:
    """Learned polynomial feature map of ReHyAt.

    §3.2 (the equation after the partitions) writes phi as the concatenation of
    powers psi_p(x)^p, p = 1..P; §4.3 (model hyperparameters) and appendix §7.1
    make psi a two-layer MLP with degree 2, separate maps for keys and queries,
    about 2.4M parameters per converted block.  Readings where the pages are
    silent: the MLP is Linear -> ReLU -> Linear per head, with biases; its
    output of 2m values is split into psi_1 (first m) and psi_2 (last m); the
    degree-1 part is made non-negative (§3.1 requires phi >= 0) as 1 + elu, so

        hidden = relu(W1[h] x + b1[h]),  psi = W2[h] hidden + b2[h],
        phi(x) = [1 + elu(psi_1), psi_2 * psi_2]            (D' = 2m)

    W1: [H, hidden, d], b1: [H, hidden], W2: [H, 2m, hidden], b2: [H, 2m].
    With H = 12, d = 128, hidden = 256 and m = 128, the query and key maps of
    one block hold 12 * 2 * (256*128 + 256 + 256*256 + 256) = 2.37M parameters.
    """

    def __init__(self, w1, b1, w2, b2):
        self.w1, self.b1, self.w2, self.b2 = (_f64(a) for a in (w1, b1, w2, b2))
        H, hid, _ = self.w1.shape
        assert self.b1.shape == (H, hid)
        assert self.w2.shape[0] == H and self.w2.shape[2] == hid and self.w2.shape[1] % 2 == 0
        assert self.b2.shape == self.w2.shape[:2]

    @property
    def dim(self) -> int:
        return self.w2.shape[1]

    def __call__(self, x) -> np.ndarray:
        x = _f64(x)                                   # [B, H, N, d]
        assert x.shape[1] == self.w1.shape[0] and x.shape[-1] == self.w1.shape[2]
        hid = np.maximum(np.einsum("bhnd,hkd->bhnk", x, self.w1) + self.b1[None, :, None, :], 0.0)
        psi = np.einsum("bhnk,hmk->bhnm", hid, self.w2) + self.b2[None, :, None, :]
        m = psi.shape[-1] // 2
        p1, p2 = psi[..., :m], psi[..., m:]
        return np.concatenate([np.where(p1 > 0, p1 + 1.0, np.exp(np.minimum(p1, 0.0))), p2 * p2], axis=-1)


def feature_q(x, phi):
    """phi of query rows for any feature-map argument (see :func:`phi_kind`)."""
    return phi[0](x) if phi_kind(phi) == PHI_GIVEN else feature_map(x, phi)


def feature_k(x, phi):
    """phi of key rows for any feature-map argument (see :func:`phi_kind`)."""
    return phi[1](x) if phi_kind(phi) == PHI_GIVEN else feature_map(x, phi)


def features(q, k, phi):
    return feature_q(q, phi), feature_k(k, phi)


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (-O2, OpenMP, IEEE arithmetic: no fast-math)."""
    stale = (not os.path.exists(_LIB_PATH)
             or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC))
    if force or stale:
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                        "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        lp = ctypes.POINTER(ctypes.c_longlong)
        lib.rehyat_oracle_fwd.restype = ctypes.c_int
        lib.rehyat_oracle_fwd.argtypes = [dp, dp, dp, dp] + [ctypes.c_int] * 8 + [
            ctypes.c_double, ctypes.c_int, lp, ctypes.c_longlong, dp, dp, dp, dp, dp, ctypes.c_int,
            dp, dp, ctypes.c_int]
        lib.rehyat_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return _load().rehyat_oracle_max_threads()


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def definition(q, k, v, frames, tokens_per_frame, chunk_frames, overlap_frames, phi="elu1",
               scale=1.0, causal=True, rows=None, partials=False, nthreads=0):
    """Definition form (C, fp64).  q, k, v: [B, H, N, d], N = frames * tokens_per_frame.

    ``rows``: optional 1-D array of query indices (same for every (b, h)); the
    outputs then have that many rows.  Returns ``y`` or ``(y, parts)`` where
    ``parts`` has m, nt (= sum exp(s - m) over the softmax set), oS, oL, nL.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    assert k.shape == q.shape and v.shape == q.shape
    assert N == frames * tokens_per_frame
    kind = phi_kind(phi)
    fq = fk = None
    if kind == PHI_GIVEN:
        fq, fk = (np.ascontiguousarray(a) for a in features(q, k, phi))
        assert fq.shape == fk.shape and fq.shape[:3] == (B, H, N)
    if rows is not None:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        R = rows.shape[0]
    else:
        R = N
    y = np.empty((B, H, R, d), dtype=np.float64)
    parts = None
    if partials:
        parts = {"m": np.empty((B, H, R)), "nt": np.empty((B, H, R)),
                 "oS": np.empty((B, H, R, d)), "oL": np.empty((B, H, R, d)),
                 "nL": np.empty((B, H, R))}
    lib = _load()
    rows_p = rows.ctypes.data_as(ctypes.POINTER(ctypes.c_longlong)) if rows is not None else None
    st = lib.rehyat_oracle_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(y), B, H, frames, tokens_per_frame, d,
        chunk_frames, overlap_frames, kind, float(scale), 1 if causal else 0,
        rows_p, R,
        _ptr(parts["m"]) if parts else None, _ptr(parts["nt"]) if parts else None,
        _ptr(parts["oS"]) if parts else None, _ptr(parts["oL"]) if parts else None,
        _ptr(parts["nL"]) if parts else None, int(nthreads),
        _ptr(fq), _ptr(fk), fq.shape[-1] if fq is not None else 0)
    if st == 1:
        raise ValueError("oracle: invalid arguments")
    if st == 2:
        raise FloatingPointError("oracle: a sum is not finite (|score| too large for exp in fp64)")
    return (y, parts) if partials else y


# ---------------------------------------------------------------------------
# numpy forms
# ---------------------------------------------------------------------------

def feature_map(x: np.ndarray, phi) -> np.ndarray:
    """phi of §3.1/§3.2 on the last axis.  ELU1: 1 + elu(x) (alpha 1); POLY2:
    [1 + elu(x), x^2] (D' = 2d); NONE: an empty feature vector."""
    kind = phi_kind(phi)
    x = np.asarray(x, dtype=np.float64)
    if kind == PHI_NONE:
        return np.zeros(x.shape[:-1] + (0,))
    e = np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))
    if kind == PHI_ELU1:
        return e
    if kind == PHI_POLY2:
        return np.concatenate([e, x * x], axis=-1)
    raise ValueError(phi)


def masks(N, tokens_per_frame, chunk_frames, overlap_frames, causal=True):
    """0/1 key masks (M_S, M_L), [N, N], from the §3.3 sets written in tokens:
    N' = T_c HW, query i is in chunk t = floor(i / N'), T^S_t = {j : max(tN' -
    T_o HW, 0) <= j < (t+1)N'}, T^L_t = {j : j < max(tN' - T_o HW, 0)} (causal)
    or the complement of T^S_t (non-causal, §3.2)."""
    HW = tokens_per_frame
    n_chunk = chunk_frames * HW
    i = np.arange(N)
    t = i // n_chunk
    lo = np.maximum(t * n_chunk - overlap_frames * HW, 0)
    hi = (t + 1) * n_chunk
    j = np.arange(N)[None, :]
    m_s = (j >= lo[:, None]) & (j < hi[:, None])
    m_l = (j < lo[:, None]) if causal else ~m_s
    return m_s, m_l


def brute_force(q, k, v, tokens_per_frame, chunk_frames, overlap_frames, phi="elu1",
                scale=1.0, causal=True):
    """Matrix form for tiny inputs: Y = (exp(s QK^T) M_S + phi(Q)phi(K)^T M_L) V / rowsum."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    N = q.shape[-2]
    m_s, m_l = masks(N, tokens_per_frame, chunk_frames, overlap_frames, causal)
    s = scale * (q @ np.swapaxes(k, -1, -2))
    w = np.where(m_s, np.exp(np.where(m_s, s, 0.0)), 0.0)
    if phi_kind(phi) != PHI_NONE:
        fq, fk = features(q, k, phi)
        w = w + np.where(m_l, fq @ np.swapaxes(fk, -1, -2), 0.0)
    return (w @ v) / w.sum(axis=-1, keepdims=True)


class RecurrentState:
    """Chunk-wise RNN form (fp64): one chunk of T_c frames per :meth:`step`.

    Carried between steps: S = sum phi(k) v^T and z = sum phi(k) over every key
    that has left the softmax window (the cached sums of §3.1), the keys and
    values of the last min(T_o, frames so far) frames (the next chunk's overlap,
    §3.3), and the number of frames processed.  Its size does not depend on how
    many frames have been processed.
    """

    def __init__(self, B, H, tokens_per_frame, head_dim, chunk_frames, overlap_frames,
                 phi="elu1", scale=1.0):
        self.HW, self.d = tokens_per_frame, head_dim
        self.Tc, self.To = chunk_frames, overlap_frames
        self.phi, self.scale = (phi if phi_kind(phi) == PHI_GIVEN else phi_kind(phi)), scale
        Dp = feature_k(np.zeros((B, H, 1, head_dim)), self.phi).shape[-1]
        self.S = np.zeros((B, H, Dp, head_dim))
        self.z = np.zeros((B, H, Dp))
        self.k_prev = np.zeros((B, H, 0, head_dim))
        self.v_prev = np.zeros((B, H, 0, head_dim))
        self.frames_done = 0

    def carried_nbytes(self) -> int:
        """Bytes carried to the next step, at their maximum (T_o frames of K/V)."""
        B, H = self.S.shape[:2]
        return (self.S.nbytes + self.z.nbytes
                + 2 * B * H * self.To * self.HW * self.d * 8)

    def step(self, qc, kc, vc):
        """Attend one chunk; q/k/v chunks are [B, H, n_frames*HW, d]."""
        qc, kc, vc = _f64(qc), _f64(kc), _f64(vc)
        nf = qc.shape[-2] // self.HW
        assert qc.shape[-2] == nf * self.HW and nf >= 1
        # window = overlap frames carried from earlier chunks + this chunk
        kw = np.concatenate([self.k_prev, kc], axis=-2)
        vw = np.concatenate([self.v_prev, vc], axis=-2)
        e = np.exp(self.scale * (qc @ np.swapaxes(kw, -1, -2)))     # softmax set
        a_s = e @ vw
        n_s = e.sum(axis=-1)
        fq = feature_q(qc, self.phi)                                 # linear set
        a_l = fq @ self.S
        n_l = (fq * self.z[:, :, None, :]).sum(axis=-1)
        y = (a_s + a_l) / (n_s + n_l)[..., None]                     # joint normalisation
        # the next window starts T_o frames before the next chunk: keep the last
        # min(T_o, frames so far) frames, fold the rest of the window into (S, z)
        self.frames_done += nf
        keep = min(self.To, self.frames_done) * self.HW
        n_ev = kw.shape[-2] - keep
        if n_ev > 0:
            fk = feature_k(kw[:, :, :n_ev], self.phi)
            self.S = self.S + np.swapaxes(fk, -1, -2) @ vw[:, :, :n_ev]
            self.z = self.z + fk.sum(axis=-2)
        self.k_prev = kw[:, :, n_ev:]
        self.v_prev = vw[:, :, n_ev:]
        return y


def recurrent(q, k, v, frames, tokens_per_frame, chunk_frames, overlap_frames, phi="elu1",
              scale=1.0, return_state_sizes=False):
    """Whole clip through :class:`RecurrentState`, chunk by chunk."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    HW = tokens_per_frame
    assert N == frames * HW
    st = RecurrentState(B, H, HW, d, chunk_frames, overlap_frames, phi, scale)
    out = np.empty_like(q)
    sizes = []
    for f0 in range(0, frames, chunk_frames):
        f1 = min(f0 + chunk_frames, frames)
        sl = slice(f0 * HW, f1 * HW)
        out[:, :, sl] = st.step(q[:, :, sl], k[:, :, sl], v[:, :, sl])
        sizes.append(st.S.nbytes + st.z.nbytes + st.k_prev.nbytes + st.v_prev.nbytes)
    return (out, sizes, st) if return_state_sizes else out


# ---------------------------------------------------------------------------
# gradients (the training direction: distillation and fine-tuning, ReHyAt §3.4)
# ---------------------------------------------------------------------------

def _torch_feature(x, phi, side):
    """phi of §3.1/§3.2 on torch fp64 tensors (differentiable)."""
    import torch
    kind = phi_kind(phi)
    if kind == PHI_GIVEN:
        m = phi[side]
        h = torch.relu(torch.einsum("bhnd,hkd->bhnk", x, torch.from_numpy(m.w1))
                       + torch.from_numpy(m.b1)[None, :, None, :])
        psi = torch.einsum("bhnk,hmk->bhnm", h, torch.from_numpy(m.w2)) + torch.from_numpy(m.b2)[None, :, None, :]
        half = psi.shape[-1] // 2
        p1, p2 = psi[..., :half], psi[..., half:]
        return torch.cat([torch.where(p1 > 0, p1 + 1.0, torch.exp(torch.clamp(p1, max=0.0))), p2 * p2], dim=-1)
    e = torch.where(x > 0, x + 1.0, torch.exp(torch.clamp(x, max=0.0)))
    if kind == PHI_ELU1:
        return e
    if kind == PHI_POLY2:
        return torch.cat([e, x * x], dim=-1)
    raise ValueError(phi)


def backward(q, k, v, dy, tokens_per_frame, chunk_frames, overlap_frames, phi="elu1", scale=1.0,
             causal=True):
    """(dq, dk, dv) = gradients of sum(dy * y) for the hybrid output y, by
    reverse-mode differentiation (torch autograd, fp64, CPU) of the matrix form
    of :func:`brute_force`: W = exp(s QK^T) M_S + (phi(Q) phi(K)^T) M_L,
    Y = W V / rowsum(W).  Tiny and mid-size inputs (it builds N x N matrices)."""
    import torch
    Q, K, V = (torch.tensor(_f64(x), requires_grad=True) for x in (q, k, v))
    G = torch.tensor(_f64(dy))
    N = Q.shape[-2]
    m_s, m_l = (torch.from_numpy(m) for m in masks(N, tokens_per_frame, chunk_frames, overlap_frames, causal))
    s = scale * (Q @ K.transpose(-1, -2))
    w = torch.where(m_s, torch.exp(torch.where(m_s, s, torch.zeros_like(s))), torch.zeros_like(s))
    if phi_kind(phi) != PHI_NONE:
        lin = _torch_feature(Q, phi, 0) @ _torch_feature(K, phi, 1).transpose(-1, -2)
        w = w + torch.where(m_l, lin, torch.zeros_like(lin))
    y = (w @ V) / w.sum(dim=-1, keepdim=True)
    y.backward(G)
    return Q.grad.numpy(), K.grad.numpy(), V.grad.numpy()


def grad_q_rows(q, k, v, dy, frames, tokens_per_frame, chunk_frames, overlap_frames, rows, phi="elu1",
                causal=True):
    """dq for selected query rows, straight from the definition (no autograd):
    with the weights w_ij of §3.1-§3.3 (e^{q.k} on the softmax set, phi(q).phi(k)
    on the linear set), N_i = sum_j w_ij, y_i = sum_j w_ij v_j / N_i and
    g_ij = (dy_i . v_j - dy_i . y_i) / N_i,
        dq_i = sum_{softmax j} w_ij g_ij k_j + phi'(q_i) * sum_{linear j} g_ij phi(k_j)
    (phi' applied per feature: elu+1 -> 1 or e^x, the square -> 2x).  Each row
    costs O(N (d + D')): usable at full workload size on a sample of rows.
    Fixed feature maps only.  q, k, v, dy: [B, H, N, d]; returns [B, H, R, d]."""
    q, k, v, dy = _f64(q), _f64(k), _f64(v), _f64(dy)
    B, H, N, d = q.shape
    HW = tokens_per_frame
    kind = phi_kind(phi)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((B, H, rows.size, d))
    fk = feature_map(k, phi) if kind != PHI_NONE else None
    for b in range(B):
        for h in range(H):
            for r, i in enumerate(rows):
                t = (i // HW) // chunk_frames
                w0 = max(t * chunk_frames - overlap_frames, 0) * HW
                w1 = min((t + 1) * chunk_frames, frames) * HW
                soft = np.arange(w0, w1)
                lin = np.arange(0, w0) if causal else np.concatenate([np.arange(0, w0), np.arange(w1, N)])
                qi, gi = q[b, h, i], dy[b, h, i]
                ws = np.exp(k[b, h, soft] @ qi)
                if kind != PHI_NONE and lin.size:
                    fq = feature_map(qi[None], phi)[0]
                    wl = fk[b, h, lin] @ fq
                else:
                    wl = np.zeros(0)
                    lin = lin[:0]
                n = ws.sum() + wl.sum()
                y = (ws @ v[b, h, soft] + wl @ v[b, h, lin]) / n
                dd = gi @ y
                gs = (v[b, h, soft] @ gi - dd) / n
                dq = (ws * gs) @ k[b, h, soft]
                if lin.size:
                    gl = (v[b, h, lin] @ gi - dd) / n
                    dphi = gl @ fk[b, h, lin]
                    e = np.where(qi > 0, 1.0, np.exp(np.minimum(qi, 0.0)))
                    dq = dq + e * dphi[:d]
                    if kind == PHI_POLY2:
                        dq = dq + 2.0 * qi * dphi[d:]
                out[b, h, r] = dq
    return out


# ---------------------------------------------------------------------------
# attention blocks (ReHyAt §3.1, first display equation: T_l(x) = f_l(A_l(x) + x))
# ---------------------------------------------------------------------------

def block_attention(x, w_qkv, b_qkv, w_o, b_o, heads, frames, tokens_per_frame, hybrid=True, chunk_frames=3,
                    overlap_frames=1, phi="elu1", rows=None):
    """fp64 A(x) of one attention block, x [B, N, C] (C = heads d):
    q = x Wq^T + bq, k = (x Wk^T + bk)/sqrt(d), v = x Wv^T + bv (w_qkv rows: q, k,
    v), split into heads; y = the hybrid attention of the definition form
    (hybrid) or full softmax attention (one chunk over the clip, no linear
    set); A(x) = concat_heads(y) Wo^T + bo.  ``rows``: output token rows
    (every row of q, k, v is formed).  Returns [B, R, C]."""
    x = _f64(x)
    w_qkv, b_qkv, w_o, b_o = (_f64(a) for a in (w_qkv, b_qkv, w_o, b_o))
    B, N, C = x.shape
    d = C // heads
    assert heads * d == C and w_qkv.shape == (3 * C, C) and w_o.shape == (C, C)
    qkv = x @ w_qkv.T + b_qkv                                     # [B, N, 3C]

    def split(a):                                                 # [B, N, C] -> [B, H, N, d]
        return np.ascontiguousarray(a.reshape(B, N, heads, d).transpose(0, 2, 1, 3))

    q, k, v = split(qkv[..., :C]), split(qkv[..., C:2 * C]) / np.sqrt(d), split(qkv[..., 2 * C:])
    if hybrid:
        y = definition(q, k, v, frames, tokens_per_frame, chunk_frames, overlap_frames, phi, rows=rows)
    else:
        y = definition(q, k, v, frames, tokens_per_frame, frames, 0, "none", rows=rows)
    R = y.shape[2]
    y = y.transpose(0, 2, 1, 3).reshape(B, R, C)                  # concat heads
    return y @ w_o.T + b_o


def block_forward(x, w_qkv, b_qkv, w_o, b_o, heads, frames, tokens_per_frame, hybrid=True, chunk_frames=3,
                  overlap_frames=1, phi="elu1", rows=None):
    """fp64 x + A(x) (at ``rows`` if given)."""
    x = _f64(x)
    a = block_attention(x, w_qkv, b_qkv, w_o, b_o, heads, frames, tokens_per_frame, hybrid, chunk_frames,
                        overlap_frames, phi, rows)
    return (x if rows is None else x[:, np.asarray(rows)]) + a


def stack_forward(x, weights, hybrid, heads, frames, tokens_per_frame, chunk_frames=3, overlap_frames=1,
                  phi="elu1"):
    """fp64 stack x_{l+1} = x_l + A_l(x_l) over the blocks (f_l taken as the
    identity); weights: list of (w_qkv, b_qkv, w_o, b_o), hybrid: list of bools."""
    x = _f64(x)
    for w, hy in zip(weights, hybrid):
        x = block_forward(x, *w, heads, frames, tokens_per_frame, hy, chunk_frames, overlap_frames, phi)
    return x
