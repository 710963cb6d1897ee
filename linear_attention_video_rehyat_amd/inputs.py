"""Seeded synthetic q/k/v generators for the hybrid attention workloads.

This module holds no attention arithmetic: it only draws random tensors with
the shapes and value distributions of the workloads, so that the GPU library
and the CPU oracle can be handed the very same values.

Workload shapes follow the video geometry of "ReHyAt: Recurrent Hybrid
Attention for Video Diffusion Transformers" (§4.1 and §5.2): a 5 s, 81-frame
480x832 clip is a 21 x 30 x 52 latent (21 frames of 1560 tokens), the ablation
resolution 320x480 is 21 x 20 x 30.  Heads H = 12 and head_dim 128 are the
Wan2.1-1.3B attention shape.  Values are i.i.d. N(0, 1) for queries and values,
N(0, 1)/sqrt(head_dim) for keys (the softmax scale folded into the keys), drawn
in float32 with numpy's PCG64 and rounded to bfloat16 (round-to-nearest-even)
by torch where the workload is bf16.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    seed_id: int            # seeds are default_rng(1000*seed_id + s), s = 0/1/2/3 for q/k/v/outliers
    B: int
    H: int
    head_dim: int
    frames: int
    tokens_per_frame: int
    chunk_frames: int
    overlap_frames: int
    dtype: str              # "f32" or "bf16"
    key_scale: float = 1.0
    outlier_frac: float = 0.0   # fraction of key rows replaced by N(0, outlier_std^2), not scaled
    outlier_std: float = 0.0

    @property
    def N(self) -> int:
        return self.frames * self.tokens_per_frame

    @property
    def tokens(self) -> int:
        return self.B * self.N

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


_S128 = 1.0 / math.sqrt(128.0)

WORKLOADS = {
    # tiny fp32 check: 4 frames of 8x8 tokens
    "tiny_f4x8x8": Workload("tiny_f4x8x8", 1, 1, 2, 16, 4, 64, 1, 1, "f32"),
    # Wan2.1-1.3B attention at 480x832, 81 frames -> latent 21 x 30 x 52
    "wan_21x30x52": Workload("wan_21x30x52", 2, 1, 12, 128, 21, 1560, 3, 1, "bf16", _S128),
    # same with the CFG cond/uncond pair as B = 2 (chunk_frames swept by the caller)
    "wan_cfg_21x30x52": Workload("wan_cfg_21x30x52", 3, 2, 12, 128, 21, 1560, 3, 1, "bf16", _S128),
    # long video, 105 latent frames of 1560 tokens, processed chunk by chunk
    "wan_long_105x30x52": Workload("wan_long_105x30x52", 4, 1, 12, 128, 105, 1560, 3, 1, "bf16", _S128),
    # higher resolution 21 x 45 x 80 with 1% outlier key rows ~ N(0, 16)
    "wan_outlier_21x45x80": Workload("wan_outlier_21x45x80", 5, 1, 12, 128, 21, 3600, 3, 1, "bf16",
                                     _S128, 0.01, 4.0),
}


def _draw(seed: int, shape, scale: float = 1.0) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def make_qkv(w: Workload, device="cpu"):
    """(q, k, v) torch tensors [B, H, N, d] in the workload's dtype."""
    shape = (w.B, w.H, w.N, w.head_dim)
    base = 1000 * w.seed_id
    q = _draw(base + 0, shape)
    k = _draw(base + 1, shape, w.key_scale)
    v = _draw(base + 2, shape)
    if w.outlier_frac > 0.0:
        rng = np.random.Generator(np.random.PCG64(base + 3))
        rows = rng.random((w.B, w.H, w.N)) < w.outlier_frac
        vals = rng.standard_normal((int(rows.sum()), w.head_dim), dtype=np.float32)
        k[rows] = vals * np.float32(w.outlier_std)
    out = []
    for x in (q, k, v):
        t = torch.from_numpy(x).to(w.torch_dtype)
        out.append(t.to(device) if device != "cpu" else t)
    return tuple(out)


def make_dout(w: Workload, device="cpu"):
    """Seeded output gradient dy ~ N(0, 1) [B, H, N, d] in the workload dtype
    (seed default_rng(1000*seed_id + 5))."""
    x = _draw(1000 * w.seed_id + 5, (w.B, w.H, w.N, w.head_dim))
    t = torch.from_numpy(x).to(w.torch_dtype)
    return t.to(device) if device != "cpu" else t


def custom(B, H, frames, tokens_per_frame, head_dim, chunk_frames, overlap_frames,
           dtype="bf16", seed_id=100, key_scale=None) -> Workload:
    """An ad-hoc workload (tests: ragged tails, odd geometries)."""
    if key_scale is None:
        key_scale = 1.0 / math.sqrt(head_dim) if dtype == "bf16" else 1.0
    return Workload(f"custom_{B}x{H}x{frames}x{tokens_per_frame}x{head_dim}", seed_id, B, H,
                    head_dim, frames, tokens_per_frame, chunk_frames, overlap_frames, dtype,
                    key_scale)


def make_mlp_weights(seed_id: int, side: int, H: int, head_dim: int, hidden: int, dtype: str = "bf16",
                     input_scale: float = 1.0):
    """Seeded synthetic weights of one learned feature map (side 0: queries, 1:
    keys); there are no trained weights to load.  Returns float32 torch tensors
    (w1 [H, hidden, d] and w2 [H, 2d, hidden] rounded to the workload dtype and
    back, b1 [H, hidden], b2 [H, 2d]).  Scales keep the activations O(1):
    W1 ~ N(0, 1/(d s^2)) for inputs of rms s, b1 ~ N(0, 0.5^2), W2 ~ N(0,
    1/hidden), b2 ~ N(0, 0.1^2); seeds default_rng(1000*seed_id + 10 + 4*side + i)."""
    base = 1000 * seed_id + 10 + 4 * side
    w1 = _draw(base + 0, (H, hidden, head_dim), 1.0 / (math.sqrt(head_dim) * input_scale))
    b1 = _draw(base + 1, (H, hidden), 0.5)
    w2 = _draw(base + 2, (H, 2 * head_dim, hidden), 1.0 / math.sqrt(hidden))
    b2 = _draw(base + 3, (H, 2 * head_dim), 0.1)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    w1t = torch.from_numpy(w1).to(tdt).to(torch.float32)
    w2t = torch.from_numpy(w2).to(tdt).to(torch.float32)
    return w1t, torch.from_numpy(b1), w2t, torch.from_numpy(b2)


def make_block_input(seed_id: int, B: int, N: int, C: int, device="cpu"):
    """Seeded block input x ~ N(0, 1), [B, N, C] bf16 (seed default_rng(1000*seed_id + 6))."""
    x = _draw(1000 * seed_id + 6, (B, N, C))
    t = torch.from_numpy(x).to(torch.bfloat16)
    return t.to(device) if device != "cpu" else t


def make_block_weights(seed_id: int, layer: int, C: int, out_gain: float = 1.0):
    """Seeded synthetic projection weights of one attention block (there are no
    trained weights to load): w_qkv [3C, C] ~ N(0, 1/C) (so q, k, v of a unit-rms
    input are unit-rms), b_qkv [3C] ~ N(0, 0.1^2), w_o [C, C] ~ N(0, out_gain^2/C),
    b_o [C] ~ N(0, 0.1^2); the weights rounded to bf16 (returned as bf16), the
    biases float32.  Seeds default_rng(1000*seed_id + 100 + 4*layer + i)."""
    base = 1000 * seed_id + 100 + 4 * layer
    w_qkv = _draw(base + 0, (3 * C, C), 1.0 / math.sqrt(C))
    b_qkv = _draw(base + 1, (3 * C,), 0.1)
    w_o = _draw(base + 2, (C, C), out_gain / math.sqrt(C))
    b_o = _draw(base + 3, (C,), 0.1)
    return (torch.from_numpy(w_qkv).to(torch.bfloat16), torch.from_numpy(b_qkv),
            torch.from_numpy(w_o).to(torch.bfloat16), torch.from_numpy(b_o))


def converted_blocks(n_converted: int, n_blocks: int = 30):
    """Which of the n_blocks blocks use the hybrid attention: the first
    n_converted (the pages name how many blocks are converted, not which)."""
    return [i < n_converted for i in range(n_blocks)]
