"""Shared helpers of the GPU parity tests: run the library, run the oracle on the
same seeded inputs, compare with the stated tolerances."""
import numpy as np
import torch

from oracle import oracle as O

# tolerances: fp32 workloads rel-L2 <= 1e-5; bf16-in / fp32-accumulate workloads
# rel-L2 <= 1e-2 and max-abs <= 3e-2
TOL_F32_REL = 1e-5
TOL_BF16_REL = 1e-2
TOL_BF16_ABS = 3e-2


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.sqrt((b * b).sum())
    return float(np.sqrt(((a - b) ** 2).sum()) / max(den, 1e-300))


def to64(t) -> np.ndarray:
    return t.detach().to("cpu").double().numpy()


def sample_rows(frames, tokens_per_frame, n_random=128, seed=0):
    """First and last token of every frame plus seeded random rows (sorted, unique)."""
    HW = tokens_per_frame
    rows = set()
    for f in range(frames):
        rows.add(f * HW)
        rows.add(f * HW + HW - 1)
    rng = np.random.default_rng(seed)
    rows.update(rng.integers(0, frames * HW, size=n_random).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def per_chunk_rel(y, ref, rows, tokens_per_frame, chunk_frames):
    """rel-L2 per chunk over the given rows: {chunk: err}."""
    chunk = (rows // tokens_per_frame) // chunk_frames
    out = {}
    for t in np.unique(chunk):
        sel = chunk == t
        out[int(t)] = rel_l2(y[:, :, sel], ref[:, :, sel])
    return out


def check_bf16(y, ref, what=""):
    r = rel_l2(y, ref)
    a = float(np.abs(np.asarray(y, np.float64) - ref).max())
    assert r <= TOL_BF16_REL and a <= TOL_BF16_ABS, f"{what}: rel-L2 {r:.3e}, max-abs {a:.3e}"
    return r, a


def check_f32(y, ref, what=""):
    r = rel_l2(y, ref)
    assert r <= TOL_F32_REL, f"{what}: rel-L2 {r:.3e}"
    return r


def oracle_rows(q, k, v, frames, HW, Tc, To, phi, rows=None, partials=False, causal=True):
    return O.definition(to64(q), to64(k), to64(v), frames, HW, Tc, To, phi, rows=rows,
                        partials=partials, causal=causal)


def gpu(*ts):
    return [t.to("cuda") for t in ts]


def sync():
    torch.cuda.synchronize()
