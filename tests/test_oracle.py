"""Pins for the fp64 CPU oracle (no GPU).

Every check here ties the oracle to something other than itself: hand-worked
closed forms (tests/golden/closed_forms.json), textbook softmax attention
(torch's scaled_dot_product_attention in fp64) in the cases where the hybrid
reduces to it, an independent matrix form on tiny inputs, the chunk-wise RNN
form, and invariants that hold for any weights (convexity, permutation within
a frame, constant carried state).

Source: "ReHyAt: Recurrent Hybrid Attention for Video Diffusion Transformers"
(arXiv 2601.04342), §3.1-§3.3.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def rand_qkv(rng, B, H, N, d, kscale=1.0):
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d)) * kscale
    v = rng.standard_normal((B, H, N, d))
    return q, k, v


def rel(a, b):
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


# ---------------------------------------------------------------- closed forms

def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_closed_form_cases(case):
    """Hand-worked d = 1, HW = 1 cases (each derivation is in the fixture)."""
    F = case["frames"]
    shape = (1, 1, F, 1)
    q = np.array(case["q"], dtype=np.float64).reshape(shape)
    k = np.array(case["k"], dtype=np.float64).reshape(shape)
    v = np.array(case["v"], dtype=np.float64).reshape(shape)
    causal = case.get("causal", True)
    env = {"e": math.e, "exp": math.exp, "__builtins__": {}}
    expected = np.array([eval(s, env) for s in case["expected"]])  # noqa: S307 - fixed fixture text
    y = O.definition(q, k, v, F, 1, case["chunk_frames"], case["overlap_frames"], case["phi"],
                     causal=causal)
    np.testing.assert_allclose(y.reshape(-1), expected, rtol=1e-14, atol=1e-14)
    yb = O.brute_force(q, k, v, 1, case["chunk_frames"], case["overlap_frames"], case["phi"],
                       causal=causal)
    np.testing.assert_allclose(yb.reshape(-1), expected, rtol=1e-14, atol=1e-14)
    if causal:
        yr = O.recurrent(q, k, v, F, 1, case["chunk_frames"], case["overlap_frames"], case["phi"])
        np.testing.assert_allclose(yr.reshape(-1), expected, rtol=1e-14, atol=1e-14)


def test_feature_map_values():
    """phi = 1 + elu (§3.1): x + 1 for x > 0, exp(x) otherwise; POLY2 appends x^2."""
    x = np.array([[2.0, 0.0, -1.0, -3.5]])
    np.testing.assert_allclose(O.feature_map(x, "elu1"),
                               [[3.0, 1.0, math.exp(-1.0), math.exp(-3.5)]], rtol=1e-15)
    np.testing.assert_allclose(O.feature_map(x, "poly2"),
                               [[3.0, 1.0, math.exp(-1.0), math.exp(-3.5), 4.0, 0.0, 1.0, 12.25]],
                               rtol=1e-15)
    assert O.feature_map(x, "none").shape == (1, 0)
    # non-negative everywhere (§3.1 requirement)
    xs = np.linspace(-30, 30, 1001)[:, None]
    assert (O.feature_map(xs, "elu1") >= 0).all()


# ------------------------------------------------------ three forms agree

def _random_geometries(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        out.append(dict(F=int(rng.integers(1, 8)), HW=int(rng.choice([1, 3, 8])),
                        d=int(rng.choice([4, 16])), Tc=int(rng.integers(1, 5)),
                        To=int(rng.integers(0, 5)), phi=str(rng.choice(["elu1", "poly2", "none"])),
                        B=int(rng.integers(1, 3)), H=int(rng.integers(1, 3))))
    return out


@pytest.mark.parametrize("idx,g", list(enumerate(_random_geometries(60, 7))),
                         ids=lambda x: x if isinstance(x, int) else "F{F}HW{HW}d{d}Tc{Tc}To{To}{phi}".format(**x))
def test_definition_brute_recurrent_agree(idx, g):
    rng = np.random.default_rng(1000 + idx)
    N = g["F"] * g["HW"]
    q, k, v = rand_qkv(rng, g["B"], g["H"], N, g["d"], kscale=0.5)
    y = O.definition(q, k, v, g["F"], g["HW"], g["Tc"], g["To"], g["phi"])
    yb = O.brute_force(q, k, v, g["HW"], g["Tc"], g["To"], g["phi"])
    yr = O.recurrent(q, k, v, g["F"], g["HW"], g["Tc"], g["To"], g["phi"])
    assert rel(y, yb) <= 1e-12
    assert rel(yr, y) <= 1e-12
    # non-causal partition: definition vs matrix form
    ync = O.definition(q, k, v, g["F"], g["HW"], g["Tc"], g["To"], g["phi"], causal=False)
    ybnc = O.brute_force(q, k, v, g["HW"], g["Tc"], g["To"], g["phi"], causal=False)
    assert rel(ync, ybnc) <= 1e-12


def test_tiny_workload_three_forms():
    """The tiny 4-frame 8x8 workload: B1 H2 d16, T_c 1, T_o 1, every phi."""
    rng = np.random.default_rng(1)
    q, k, v = rand_qkv(rng, 1, 2, 256, 16)
    for phi in ("elu1", "poly2", "none"):
        y = O.definition(q, k, v, 4, 64, 1, 1, phi)
        assert rel(O.brute_force(q, k, v, 64, 1, 1, phi), y) <= 1e-12
        assert rel(O.recurrent(q, k, v, 4, 64, 1, 1, phi), y) <= 1e-12


# ----------------------------------------------- reductions to softmax attention

def _sdpa(q, k, v, mask=None, scale=1.0):
    t = [torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v)]
    m = None if mask is None else torch.from_numpy(mask)
    return torch.nn.functional.scaled_dot_product_attention(*t, attn_mask=m, scale=scale).numpy()


@pytest.mark.parametrize("phi", ["elu1", "poly2", "none"])
@pytest.mark.parametrize("scale", [1.0, 0.25])
def test_single_chunk_is_full_softmax(phi, scale):
    """T_c >= F: one chunk holds every frame, the linear set is empty (§3.3), so
    the hybrid is plain bidirectional softmax attention."""
    rng = np.random.default_rng(3)
    F, HW, d = 5, 6, 16
    q, k, v = rand_qkv(rng, 2, 3, F * HW, d)
    for Tc in (F, F + 3):
        y = O.definition(q, k, v, F, HW, Tc, 2, phi, scale=scale)
        assert rel(y, _sdpa(q, k, v, scale=scale)) <= 1e-12


def test_long_overlap_is_chunk_causal_softmax():
    """T_o >= F with phi = NONE: every window starts at frame 0, so query chunk t
    attends with softmax to all chunks <= t (chunk-causal softmax)."""
    rng = np.random.default_rng(4)
    F, HW, d, Tc = 7, 4, 8, 2
    q, k, v = rand_qkv(rng, 1, 2, F * HW, d)
    chunk = np.arange(F * HW) // (Tc * HW)
    mask = chunk[None, :] <= chunk[:, None]
    y = O.definition(q, k, v, F, HW, Tc, F + 1, "none")
    assert rel(y, _sdpa(q, k, v, mask)) <= 1e-12


def test_phi_none_is_banded_chunk_softmax():
    """phi = NONE leaves only the softmax window: chunk t and the T_o frames before it."""
    rng = np.random.default_rng(5)
    F, HW, d, Tc, To = 9, 3, 8, 2, 1
    q, k, v = rand_qkv(rng, 1, 1, F * HW, d)
    frame = np.arange(F * HW) // HW
    t = frame // Tc
    lo = np.maximum(t * Tc - To, 0)
    hi = np.minimum((t + 1) * Tc, F)
    mask = (frame[None, :] >= lo[:, None]) & (frame[None, :] < hi[:, None])
    y = O.definition(q, k, v, F, HW, Tc, To, "none")
    assert rel(y, _sdpa(q, k, v, mask)) <= 1e-12


def test_first_chunk_is_plain_softmax():
    """Chunk 0 has an empty linear set (§3.3): its rows are softmax over frames [0, T_c)."""
    rng = np.random.default_rng(6)
    F, HW, d, Tc = 6, 5, 16, 2
    q, k, v = rand_qkv(rng, 1, 2, F * HW, d)
    y = O.definition(q, k, v, F, HW, Tc, 1, "elu1")
    n0 = Tc * HW
    ref = _sdpa(q[:, :, :n0], k[:, :, :n0], v[:, :, :n0])
    assert rel(y[:, :, :n0], ref) <= 1e-12


# ------------------------------------------------------------- branch closed forms

def test_branch_partials_constant_keys():
    """With every key equal to c, each branch output is the plain mean of v over
    its key set, and m = q.c, nt = |softmax set|: pins the set boundaries."""
    rng = np.random.default_rng(8)
    F, HW, d, Tc, To = 7, 3, 4, 2, 1
    N = F * HW
    q = rng.standard_normal((1, 1, N, d))
    c = rng.standard_normal(d) * 0.3
    k = np.broadcast_to(c, (1, 1, N, d)).copy()
    v = rng.standard_normal((1, 1, N, d))
    y, p = O.definition(q, k, v, F, HW, Tc, To, "elu1", partials=True)
    for i in range(N):
        t = (i // HW) // Tc
        w0 = max(t * Tc - To, 0) * HW
        w1 = min((t + 1) * Tc, F) * HW
        np.testing.assert_allclose(p["oS"][0, 0, i], v[0, 0, w0:w1].mean(0), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(p["m"][0, 0, i], q[0, 0, i] @ c, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(p["nt"][0, 0, i], w1 - w0, rtol=1e-12)
        if w0 > 0:
            np.testing.assert_allclose(p["oL"][0, 0, i], v[0, 0, :w0].mean(0), rtol=1e-12, atol=1e-13)
        else:
            assert p["nL"][0, 0, i] == 0.0


def test_partials_recombine_to_output():
    """The joint normalisation written with the partials: y = (nt e^m oS + nL oL)/(nt e^m + nL)."""
    rng = np.random.default_rng(9)
    F, HW, d = 5, 4, 8
    q, k, v = rand_qkv(rng, 1, 2, F * HW, d, 0.5)
    for phi in ("elu1", "poly2"):
        y, p = O.definition(q, k, v, F, HW, 2, 1, phi, partials=True)
        ws = p["nt"] * np.exp(p["m"])
        yy = (ws[..., None] * p["oS"] + p["nL"][..., None] * p["oL"]) / (ws + p["nL"])[..., None]
        assert rel(yy, y) <= 1e-12


# ------------------------------------------------------------------- invariants

def test_convexity():
    """All weights are >= 0 and normalised: constant v gives constant y, and every
    output lies inside the range of v over the keys."""
    rng = np.random.default_rng(10)
    F, HW, d = 6, 4, 8
    q, k, _ = rand_qkv(rng, 1, 2, F * HW, d)
    v = np.full_like(q, 2.5)
    for phi in ("elu1", "poly2", "none"):
        y = O.definition(q, k, v, F, HW, 2, 1, phi)
        np.testing.assert_allclose(y, 2.5, rtol=1e-14)
    v = rng.standard_normal(q.shape)
    y = O.definition(q, k, v, F, HW, 2, 1, "elu1")
    assert (y <= v.max(axis=2, keepdims=True) + 1e-12).all()
    assert (y >= v.min(axis=2, keepdims=True) - 1e-12).all()


def test_permutation_within_frame():
    """The sets are defined by frames, so shuffling tokens inside each frame
    (the same way for q, k, v) shuffles the outputs the same way."""
    rng = np.random.default_rng(11)
    F, HW, d = 5, 6, 8
    N = F * HW
    q, k, v = rand_qkv(rng, 1, 1, N, d, 0.5)
    perm = np.concatenate([f * HW + rng.permutation(HW) for f in range(F)])
    y = O.definition(q, k, v, F, HW, 2, 1, "elu1")
    yp = O.definition(q[:, :, perm], k[:, :, perm], v[:, :, perm], F, HW, 2, 1, "elu1")
    assert rel(yp, y[:, :, perm]) <= 1e-12


def test_recurrent_state_constant_memory():
    """Chunk-wise RNN form: the carried state does not grow with video length."""
    rng = np.random.default_rng(12)
    HW, d = 4, 8
    sizes = {}
    for F in (6, 30):
        q, k, v = rand_qkv(rng, 1, 2, F * HW, d)
        _, sz, st = O.recurrent(q, k, v, F, HW, 3, 1, "elu1", return_state_sizes=True)
        sizes[F] = (max(sz), st.carried_nbytes())
    assert sizes[6] == sizes[30]


def test_query_subset_matches_full():
    rng = np.random.default_rng(13)
    F, HW, d = 6, 5, 8
    q, k, v = rand_qkv(rng, 2, 2, F * HW, d)
    rows = np.array([0, 7, 13, 29, 14])
    y = O.definition(q, k, v, F, HW, 2, 1, "poly2")
    ys = O.definition(q, k, v, F, HW, 2, 1, "poly2", rows=rows)
    np.testing.assert_array_equal(ys, y[:, :, rows])


def test_overflow_is_reported():
    """The literal exponential overflows fp64 past s ~ 709; the oracle says so."""
    q = np.full((1, 1, 2, 1), 30.0)
    k = np.full((1, 1, 2, 1), 30.0)
    v = np.ones((1, 1, 2, 1))
    with pytest.raises(FloatingPointError):
        O.definition(q, k, v, 2, 1, 1, 1, "elu1")


def test_bad_arguments():
    q = np.zeros((1, 1, 4, 2))
    with pytest.raises(ValueError):
        O.definition(q, q, q, 2, 2, 0, 0, "elu1")
    with pytest.raises(ValueError):
        O.definition(q, q, q, 2, 2, 1, -1, "elu1")


# ------------------------------------------------ learned (MLP) feature maps

def _reduction_weights(H, d, shift1=0.0, shift2=0.0, gain2=1.0):
    """MLP weights whose map has a closed form: W1 = [I; -I] (hidden = 2d, so
    relu splits x into its positive and negative parts), W2 = [[I, -I]; [g I, -g I]]
    (psi_1 = x + shift1, psi_2 = g x + shift2)."""
    I = np.eye(d)
    w1 = np.tile(np.concatenate([I, -I])[None], (H, 1, 1))
    b1 = np.zeros((H, 2 * d))
    w2 = np.tile(np.block([[I, -I], [gain2 * I, -gain2 * I]])[None], (H, 1, 1))
    b2 = np.tile(np.concatenate([np.full(d, shift1), np.full(d, shift2)])[None], (H, 1))
    return O.MlpFeatureMap(w1, b1, w2, b2)


def _closed(shift1=0.0, shift2=0.0, gain2=1.0):
    def phi(x):
        a = x + shift1
        b = gain2 * x + shift2
        return np.concatenate([np.where(a > 0, a + 1.0, np.exp(np.minimum(a, 0.0))), b * b], axis=-1)
    return phi


def test_mlp_map_reduces_to_poly2():
    """With W1 = [I; -I], W2 = [[I, -I]; [I, -I]] and zero biases, relu(x) - relu(-x)
    = x makes psi_1 = psi_2 = x, so the learned map is exactly [1 + elu(x), x^2]
    (the parameter-free degree-2 map) and every attention form agrees with it."""
    rng = np.random.default_rng(11)
    B, H, F, HW, d = 1, 2, 5, 3, 4
    q, k, v = rand_qkv(rng, B, H, F * HW, d)
    m = _reduction_weights(H, d)
    np.testing.assert_array_equal(m(q), O.feature_map(q, "poly2"))
    for causal in (True, False):
        ref = O.definition(q, k, v, F, HW, 2, 1, "poly2", causal=causal)
        assert rel(O.definition(q, k, v, F, HW, 2, 1, (m, m), causal=causal), ref) <= 1e-14
        assert rel(O.brute_force(q, k, v, HW, 2, 1, (m, m), causal=causal), ref) <= 1e-12
    assert rel(O.recurrent(q, k, v, F, HW, 2, 1, (m, m)), O.definition(q, k, v, F, HW, 2, 1, "poly2")) <= 1e-12


def test_mlp_zero_second_half_is_elu1():
    """psi_2 = 0 (zero lower half of W2 and b2) leaves [1 + elu(x), 0]: the zero
    features add nothing, so the hybrid equals the ELU1 one."""
    rng = np.random.default_rng(12)
    q, k, v = rand_qkv(rng, 2, 1, 12, 3)
    m = _reduction_weights(1, 3, gain2=0.0)
    for causal in (True, False):
        ref = O.definition(q, k, v, 4, 3, 1, 2, "elu1", causal=causal)
        assert rel(O.definition(q, k, v, 4, 3, 1, 2, (m, m), causal=causal), ref) <= 1e-14


def test_mlp_separate_query_and_key_maps():
    """Queries go through phi_q and keys through phi_k (§7.1: separate maps).  With
    shifted biases and a gain the two maps differ and have closed forms; swapping
    them changes the result."""
    rng = np.random.default_rng(13)
    B, H, F, HW, d = 1, 2, 6, 2, 3
    q, k, v = rand_qkv(rng, B, H, F * HW, d)
    mq = _reduction_weights(H, d, shift1=0.3, shift2=-0.5)
    mk = _reduction_weights(H, d, shift1=-0.7, shift2=0.25, gain2=2.0)
    cq, ck = _closed(0.3, -0.5), _closed(-0.7, 0.25, 2.0)
    np.testing.assert_allclose(mq(q), cq(q), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(mk(k), ck(k), rtol=1e-14, atol=1e-14)
    for causal in (True, False):
        want = O.brute_force(q, k, v, HW, 1, 1, (cq, ck), causal=causal)
        got = O.definition(q, k, v, F, HW, 1, 1, (mq, mk), causal=causal)
        assert rel(got, want) <= 1e-12
        swapped = O.definition(q, k, v, F, HW, 1, 1, (mk, mq), causal=causal)
        assert rel(swapped, want) > 1e-3
    assert rel(O.recurrent(q, k, v, F, HW, 1, 1, (mq, mk)), O.brute_force(q, k, v, HW, 1, 1, (cq, ck))) <= 1e-12


def test_mlp_map_random_weights_small_loops():
    """Random weights on a tiny case: the map against the two layers written as
    scalar loops over units (catches an index or transpose slip in the tensor form),
    and phi >= 0."""
    rng = np.random.default_rng(14)
    H, d, hid, m2 = 2, 3, 5, 4
    w1, b1 = rng.standard_normal((H, hid, d)), rng.standard_normal((H, hid))
    w2, b2 = rng.standard_normal((H, m2, hid)), rng.standard_normal((H, m2))
    x = rng.standard_normal((1, H, 4, d))
    got = O.MlpFeatureMap(w1, b1, w2, b2)(x)
    for h in range(H):
        for n in range(4):
            hidden = [max(sum(w1[h, a, c] * x[0, h, n, c] for c in range(d)) + b1[h, a], 0.0) for a in range(hid)]
            psi = [sum(w2[h, o, a] * hidden[a] for a in range(hid)) + b2[h, o] for o in range(m2)]
            want = [p + 1.0 if p > 0 else math.exp(p) for p in psi[:m2 // 2]] + [p * p for p in psi[m2 // 2:]]
            np.testing.assert_allclose(got[0, h, n], want, rtol=1e-13)
    assert (got >= 0).all()


# ------------------------------------------------------------------ gradients

@pytest.mark.parametrize("phi", ["elu1", "poly2", "none"])
@pytest.mark.parametrize("causal", [True, False])
def test_gradients_match_finite_differences(phi, causal):
    """Central differences of the C definition form (an implementation that
    shares nothing with the autograd matrix form) on every input coordinate of a
    tiny case."""
    rng = np.random.default_rng(21)
    B, H, F, HW, d, Tc, To = 1, 1, 4, 2, 3, 1, 1
    q, k, v = rand_qkv(rng, B, H, F * HW, d, kscale=0.7)
    dy = rng.standard_normal(q.shape)
    dq, dk, dv = O.backward(q, k, v, dy, HW, Tc, To, phi, causal=causal)
    eps = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [xp if a is x else a for a in (q, k, v)]
            args_m = [xm if a is x else a for a in (q, k, v)]
            yp = O.definition(*args_p, F, HW, Tc, To, phi, causal=causal)
            ym = O.definition(*args_m, F, HW, Tc, To, phi, causal=causal)
            num[idx] = ((yp - ym) * dy).sum() / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


def test_gradients_single_chunk_are_softmax_attention_gradients():
    """T_c >= F: the hybrid is softmax attention; its gradients are those of
    torch's scaled_dot_product_attention (fp64)."""
    rng = np.random.default_rng(22)
    q, k, v = rand_qkv(rng, 1, 2, 24, 8, kscale=0.5)
    dy = rng.standard_normal(q.shape)
    dq, dk, dv = O.backward(q, k, v, dy, 6, 4, 1, "elu1")
    t = [torch.tensor(x, requires_grad=True) for x in (q, k, v)]
    y = torch.nn.functional.scaled_dot_product_attention(*t, scale=1.0)
    y.backward(torch.from_numpy(dy))
    for a, b in zip((dq, dk, dv), t):
        np.testing.assert_allclose(a, b.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_gradient_of_v_sums_to_gradient_of_y():
    """Each output is a convex combination of values, so sum_j dv_j = sum_i dy_i."""
    rng = np.random.default_rng(23)
    q, k, v = rand_qkv(rng, 2, 1, 30, 4, kscale=0.5)
    dy = rng.standard_normal(q.shape)
    for phi in ("elu1", "poly2"):
        _, _, dv = O.backward(q, k, v, dy, 5, 2, 1, phi)
        np.testing.assert_allclose(dv.sum(axis=-2), dy.sum(axis=-2), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("phi", ["elu1", "poly2", "none"])
@pytest.mark.parametrize("causal", [True, False])
def test_grad_q_rows_matches_reverse_mode(phi, causal):
    """The per-row definition-form dq (usable at full size on sampled rows)
    equals the reverse-mode gradient of the matrix form."""
    rng = np.random.default_rng(24)
    F, HW = 6, 5
    q, k, v = rand_qkv(rng, 1, 2, F * HW, 4, kscale=0.6)
    dy = rng.standard_normal(q.shape)
    dq, _, _ = O.backward(q, k, v, dy, HW, 2, 1, phi, causal=causal)
    rows = np.array([0, 3, 7, 12, 18, 29])
    got = O.grad_q_rows(q, k, v, dy, F, HW, 2, 1, rows, phi, causal=causal)
    np.testing.assert_allclose(got, dq[:, :, rows], rtol=1e-10, atol=1e-12)
