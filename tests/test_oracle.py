"""Pins of the fp64 oracle against things other than itself.

Each test fixes a part of the oracle by something the recurrence's
mathematics determines independently: a hand-worked example, a brute-force
closed form, finite differences, a library autograd, split invariance and
special cases that reduce to textbook routines.  Shapes use d_k != d_v so
that a transposed operand cannot pass.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import twin

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_case(rng, B=1, H=2, T=7, dk=3, dv=5, decay="token", s_in=True, lo=0.6):
    q = rng.standard_normal((B, H, T, dk))
    k = rng.standard_normal((B, H, T, dk))
    v = rng.standard_normal((B, H, T, dv))
    if decay == "token":
        a = rng.uniform(lo, 1.0, (B, H, T))
    elif decay == "head":
        a = rng.uniform(lo, 1.0, (H,))
    else:
        a = None
    S_in = rng.standard_normal((B, H, dk, dv)) if s_in else None
    return q, k, v, a, S_in


def decay_full(a, B, H, T):
    if a is None:
        return np.ones((B, H, T))
    if a.ndim == 1:
        return np.broadcast_to(a[None, :, None], (B, H, T)).copy()
    return a


# ---------------------------------------------------------------- golden


def test_hand_worked_example():
    """Hand-derived d_k=2, d_v=1, T=3 example (binary fractions, exact)."""
    g = json.load(open(os.path.join(GOLDEN, "hand_worked_2x1.json")))
    inp, exp = g["inputs"], g["expected"]
    arr = lambda x: np.array(x, np.float64)[None, None]  # noqa: E731
    q, k, v, dO = arr(inp["q"]), arr(inp["k"]), arr(inp["v"]), arr(inp["dO"])
    a = np.array(inp["a"], np.float64)[None, None]
    S_in, dS_out = arr(inp["S_in"]), arr(inp["dS_out"])
    o, S_out = oracle.fwd(q, k, v, a, S_in)
    assert np.array_equal(o[0, 0], np.array(exp["o"]))
    assert np.array_equal(S_out[0, 0], np.array(exp["S_out"]))
    dq, dk, dv, dS_in, da = oracle.bwd(q, k, v, a, S_in, dO, dS_out, want_da=True)
    assert np.array_equal(dq[0, 0], np.array(exp["dq"]))
    assert np.array_equal(dk[0, 0], np.array(exp["dk"]))
    assert np.array_equal(dv[0, 0], np.array(exp["dv"]))
    assert np.array_equal(dS_in[0, 0], np.array(exp["dS_in"]))
    assert np.array_equal(da[0, 0], np.array(exp["da"]))


# ---------------------------------------------------------- closed form


def closed_form(q, k, v, a, S_in):
    """Brute force: o_t = sum_{s<=t} (prod_{r=s+1..t} a_r)(q_t.k_s) v_s
    + (prod_{r<=t} a_r) q_t S_in;  S_out = (prod a) S_in + sum_s (prod_{r>s} a_r) k_s^T v_s.
    Products are taken literally (no logs, no recurrence)."""
    B, H, T, dk = k.shape
    dv = v.shape[3]
    af = decay_full(a, B, H, T)
    o = np.zeros((B, H, T, dv))
    S_out = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            for t in range(T):
                acc = np.zeros(dv)
                for s in range(t + 1):
                    w = np.prod(af[b, h, s + 1:t + 1])
                    acc += w * np.dot(q[b, h, t], k[b, h, s]) * v[b, h, s]
                if S_in is not None:
                    acc += np.prod(af[b, h, :t + 1]) * (q[b, h, t] @ S_in[b, h])
                o[b, h, t] = acc
            S = np.zeros((dk, dv))
            if S_in is not None:
                S += np.prod(af[b, h]) * S_in[b, h]
            for s in range(T):
                S += np.prod(af[b, h, s + 1:]) * np.outer(k[b, h, s], v[b, h, s])
            S_out[b, h] = S
    return o, S_out


@pytest.mark.parametrize("decay", ["none", "head", "token"])
@pytest.mark.parametrize("T", [1, 5, 33])
def test_forward_matches_brute_force(decay, T):
    rng = np.random.default_rng(10 + T)
    q, k, v, a, S_in = rand_case(rng, B=2, H=2, T=T, dk=3, dv=4, decay=decay)
    o, S_out = oracle.fwd(q, k, v, a, S_in)
    o_ref, S_ref = closed_form(q, k, v, a, S_in)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S_out, S_ref, rtol=1e-12, atol=1e-12)


def test_forward_matches_brute_force_d64():
    rng = np.random.default_rng(3)
    q, k, v, a, S_in = rand_case(rng, B=1, H=1, T=64, dk=16, dv=24, decay="token", lo=0.9)
    o, S_out = oracle.fwd(q, k, v, a, S_in)
    o_ref, S_ref = closed_form(q, k, v, a, S_in)
    np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(S_out, S_ref, rtol=1e-11, atol=1e-11)


# ---------------------------------------------------------- numpy twin


@pytest.mark.parametrize("decay", ["none", "head", "token"])
def test_c_oracle_matches_numpy_twin(decay):
    rng = np.random.default_rng(7)
    q, k, v, a, S_in = rand_case(rng, B=2, H=3, T=40, dk=6, dv=5, decay=decay)
    dO = rng.standard_normal(v.shape)
    dS_out = rng.standard_normal(S_in.shape)
    o, S_out = oracle.fwd(q, k, v, a, S_in)
    o2, S2 = twin.fwd(q, k, v, a, S_in)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S_out, S2, rtol=1e-12, atol=1e-12)
    g1 = oracle.bwd(q, k, v, a, S_in, dO, dS_out)
    g2 = twin.bwd(q, k, v, a, S_in, dO, dS_out)
    for x, y in zip(g1, g2):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------ finite differences


def loss(q, k, v, a, S_in, dO, dS_out):
    o, S_out = oracle.fwd(q, k, v, a, S_in)
    return float(np.sum(dO * o) + np.sum(dS_out * S_out))


def test_backward_matches_finite_differences():
    """Central differences of L = <dO,o> + <dS_out,S_out> for every input.

    L is linear in each of q, k, v, S_in separately, so the central
    difference is exact up to rounding; in a it is a polynomial, with
    truncation error eps^2 f'''/6."""
    rng = np.random.default_rng(11)
    B, H, T, dk, dv = 1, 2, 9, 3, 4
    q, k, v, a, S_in = rand_case(rng, B, H, T, dk, dv, decay="token")
    dO = rng.standard_normal((B, H, T, dv))
    dS_out = rng.standard_normal((B, H, dk, dv))
    dq, dk_, dv_, dS_in, da = oracle.bwd(q, k, v, a, S_in, dO, dS_out, want_da=True)
    eps = 1e-6
    grads = {"q": (q, dq), "k": (k, dk_), "v": (v, dv_), "S_in": (S_in, dS_in), "a": (a, da)}
    for name, (x, gx) in grads.items():
        flat = x.reshape(-1)
        for idx in range(flat.size):
            old = flat[idx]
            flat[idx] = old + eps
            lp = loss(q, k, v, a, S_in, dO, dS_out)
            flat[idx] = old - eps
            lm = loss(q, k, v, a, S_in, dO, dS_out)
            flat[idx] = old
            fd = (lp - lm) / (2 * eps)
            an = gx.reshape(-1)[idx]
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, idx, fd, an)


def test_decay_gradient_identity():
    """The decay gradient the GPU path forms: with g_t = q_t.dq_t - k_t.dk_t,
    a_r da_r = sum_{t >= r} g_t + <dS_out, S_out>.  Checked on the oracle's
    own gradients (da pinned by finite differences above), per-token and
    per-head decay, with S_in and dS_out nonzero, and across a split where
    the later piece's sum becomes the earlier piece's carry."""
    rng = np.random.default_rng(21)
    B, H, T, dk, dv = 2, 3, 40, 4, 6
    for decay in ("token", "head"):
        q, k, v, a, S_in = rand_case(rng, B, H, T, dk, dv, decay=decay, lo=0.7)
        dO = rng.standard_normal((B, H, T, dv))
        dS_out = rng.standard_normal((B, H, dk, dv))
        dq, dk_, dv_, dS_in, da = oracle.bwd(q, k, v, a, S_in, dO, dS_out, want_da=True)
        _, S_out = oracle.fwd(q, k, v, a, S_in)
        g = np.sum(q * dq, -1) - np.sum(k * dk_, -1)
        carry = np.sum(dS_out * S_out, axis=(-2, -1))
        suffix = np.cumsum(g[..., ::-1], -1)[..., ::-1] + carry[..., None]
        af = decay_full(a, B, H, T)
        np.testing.assert_allclose(af * da, suffix, rtol=1e-10, atol=1e-10)
        # the carry entering a piece boundary is <dS, S> there
        cut = 17
        S_mid = oracle.fwd(q[:, :, :cut], k[:, :, :cut], v[:, :, :cut],
                           a if a.ndim == 1 else a[:, :, :cut], S_in)[1]
        dS_mid = oracle.bwd(q[:, :, cut:], k[:, :, cut:], v[:, :, cut:],
                            a if a.ndim == 1 else a[:, :, cut:], S_mid, dO[:, :, cut:], dS_out)[3]
        np.testing.assert_allclose(np.sum(dS_mid * S_mid, axis=(-2, -1)), suffix[:, :, cut],
                                   rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("decay", ["token", "head"])
def test_decay_gradient_across_checkpoint_blocks(decay):
    """The oracle's da rebuilds S_{t-1} from a checkpoint every 256 tokens.
    At T = 700 (two full blocks and a partial third) it is pinned two ways
    that do not use that code:
      * the suffix-sum identity a_r da_r = sum_{t >= r} g_t + <dS_out, S_out>,
        g_t = q_t.dq_t - k_t.dk_t (dq, dk come from the plain sweeps);
      * central differences of L in single a_t at the block edges.  L is
        affine in each single a_t (every path through the recurrence meets
        a_t once), so the central difference is exact up to rounding."""
    rng = np.random.default_rng(31)
    B, H, T, dk, dv = 1, 2, 700, 3, 4
    q, k, v, a, S_in = rand_case(rng, B, H, T, dk, dv, decay=decay, lo=0.985)
    dO = rng.standard_normal((B, H, T, dv))
    dS_out = rng.standard_normal((B, H, dk, dv))
    dq, dk_, dv_, dS_in, da = oracle.bwd(q, k, v, a, S_in, dO, dS_out, want_da=True)
    _, S_out = oracle.fwd(q, k, v, a, S_in)
    g = np.sum(q * dq, -1) - np.sum(k * dk_, -1)
    carry = np.sum(dS_out * S_out, axis=(-2, -1))
    suffix = np.cumsum(g[..., ::-1], -1)[..., ::-1] + carry[..., None]
    af = decay_full(a, B, H, T)
    scale = np.max(np.abs(suffix))
    np.testing.assert_allclose(af * da, suffix, rtol=1e-11, atol=1e-11 * scale)
    if decay != "token":
        return
    eps = 1e-5
    for t in (0, 255, 256, 257, 511, 512, 699):
        for h in range(H):
            old = a[0, h, t]
            a[0, h, t] = old + eps
            lp = loss(q, k, v, a, S_in, dO, dS_out)
            a[0, h, t] = old - eps
            lm = loss(q, k, v, a, S_in, dO, dS_out)
            a[0, h, t] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - da[0, h, t]) <= 1e-7 * max(1.0, abs(fd)), (t, h, fd, da[0, h, t])


# ------------------------------------------------------ torch autograd


def closed_form_torch(q, k, v, a, S_in):
    """Closed form with cumulative products, differentiated by torch."""
    P = torch.cumprod(a, dim=-1)                                  # [B,H,T]
    W = P[..., :, None] / P[..., None, :]                         # prod_{s<r<=t} a_r
    W = torch.tril(W)
    o = ((q @ k.transpose(-1, -2)) * W) @ v + P[..., None] * (q @ S_in)
    tail = P[..., -1:] / P                                        # prod_{r>s} a_r
    S_out = P[..., -1, None, None] * S_in + (k * tail[..., None]).transpose(-1, -2) @ v
    return o, S_out


def test_backward_matches_torch_autograd():
    rng = np.random.default_rng(5)
    B, H, T, dk, dv = 2, 2, 48, 5, 7
    q, k, v, a, S_in = rand_case(rng, B, H, T, dk, dv, decay="token", lo=0.8)
    dO = rng.standard_normal((B, H, T, dv))
    dS_out = rng.standard_normal((B, H, dk, dv))
    ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, a, S_in)]
    o, S_out = closed_form_torch(*ts)
    L = (o * torch.tensor(dO)).sum() + (S_out * torch.tensor(dS_out)).sum()
    L.backward()
    got = oracle.bwd(q, k, v, a, S_in, dO, dS_out, want_da=True)
    o_or, S_or = oracle.fwd(q, k, v, a, S_in)
    np.testing.assert_allclose(o_or, o.detach().numpy(), rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(S_or, S_out.detach().numpy(), rtol=1e-10, atol=1e-10)
    names = ["dq", "dk", "dv", "dS_in", "da"]
    order = [0, 1, 2, 4, 3]     # autograd leaves are (q,k,v,a,S_in)
    for name, g, li in zip(names, got, order):
        np.testing.assert_allclose(g, ts[li].grad.numpy(), rtol=1e-9, atol=1e-9, err_msg=name)


# ----------------------------------------------------- split invariance


def run_split(q, k, v, a, S_in, dO, dS_out, lengths):
    """Pieces in order with S carried; backward in reverse with dS carried."""
    B, H, T, dk = k.shape
    af = decay_full(a, B, H, T) if a is not None else None
    bounds = np.cumsum([0] + list(lengths))
    S = S_in
    S_starts, outs = [], []
    for i in range(len(lengths)):
        s0, s1 = bounds[i], bounds[i + 1]
        S_starts.append(S)
        ai = None if af is None else np.ascontiguousarray(af[:, :, s0:s1])
        o, S = oracle.fwd(q[:, :, s0:s1], k[:, :, s0:s1], v[:, :, s0:s1], ai, S)
        outs.append(o)
    S_out = S
    dS = dS_out
    grads = [None] * len(lengths)
    for i in reversed(range(len(lengths))):
        s0, s1 = bounds[i], bounds[i + 1]
        ai = None if af is None else np.ascontiguousarray(af[:, :, s0:s1])
        dq, dk_, dv_, dS = oracle.bwd(q[:, :, s0:s1], k[:, :, s0:s1], v[:, :, s0:s1], ai,
                                      S_starts[i], dO[:, :, s0:s1], dS)
        grads[i] = (dq, dk_, dv_)
    cat = lambda xs: np.concatenate(xs, axis=2)  # noqa: E731
    return (cat(outs), S_out, cat([g[0] for g in grads]), cat([g[1] for g in grads]),
            cat([g[2] for g in grads]), dS)


@pytest.mark.parametrize("split", ["uniform", "random", "ones"])
@pytest.mark.parametrize("decay", ["none", "head", "token"])
def test_split_invariance_is_bitwise(split, decay):
    rng = np.random.default_rng(21)
    B, H, T, dk, dv = 2, 2, 96, 4, 6
    q, k, v, a, S_in = rand_case(rng, B, H, T, dk, dv, decay=decay)
    dO = rng.standard_normal((B, H, T, dv))
    dS_out = rng.standard_normal((B, H, dk, dv))
    o, S_out = oracle.fwd(q, k, v, a, S_in)
    dq, dk_, dv_, dS_in = oracle.bwd(q, k, v, a, S_in, dO, dS_out)
    if split == "uniform":
        lengths = [24] * 4
    elif split == "random":
        cuts = np.sort(rng.choice(np.arange(1, T), size=6, replace=False))
        lengths = list(np.diff(np.concatenate([[0], cuts, [T]])))
    else:
        lengths = [1] * 5 + [T - 5]
    got = run_split(q, k, v, a, S_in, dO, dS_out, lengths)
    for x, y in zip(got, (o, S_out, dq, dk_, dv_, dS_in)):
        assert np.array_equal(x, y)


def test_interrupt_and_resume_from_boundary_state(tmp_path):
    """The boundary state is a complete checkpoint: serialise S after piece 2,
    reload it and finish; the result equals the uninterrupted run bitwise."""
    rng = np.random.default_rng(4)
    q, k, v, a, S_in = rand_case(rng, 1, 2, 80, 4, 3, decay="token")
    o_all, S_all = oracle.fwd(q, k, v, a, S_in)
    _, S_mid = oracle.fwd(q[:, :, :30], k[:, :, :30], v[:, :, :30],
                          np.ascontiguousarray(a[:, :, :30]), S_in)
    path = tmp_path / "S.npy"
    np.save(path, S_mid)
    S_back = np.load(path)
    o2, S2 = oracle.fwd(q[:, :, 30:], k[:, :, 30:], v[:, :, 30:],
                        np.ascontiguousarray(a[:, :, 30:]), S_back)
    assert np.array_equal(o2, o_all[:, :, 30:])
    assert np.array_equal(S2, S_all)


# --------------------------------------------------------- special cases


def test_no_decay_zero_state_is_cumsum():
    """a = 1, S_in = 0: S_t = sum_{s<=t} k_s^T v_s (causal linear attention)."""
    rng = np.random.default_rng(8)
    q, k, v, _, _ = rand_case(rng, 1, 2, 30, 4, 3, decay="none", s_in=False)
    o, S_out = oracle.fwd(q, k, v, None, None)
    outer = k[..., :, None] * v[..., None, :]          # [B,H,T,dk,dv]
    S_t = np.cumsum(outer, axis=2)
    np.testing.assert_allclose(S_out, S_t[:, :, -1], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o, np.einsum("bhti,bhtij->bhtj", q, S_t), rtol=1e-12, atol=1e-12)


def test_scalar_recurrence_closed_form():
    """d_k = d_v = 1: S_t = a_t S_{t-1} + k_t v_t solved by scipy's lfilter
    for constant a (a first-order IIR filter)."""
    from scipy.signal import lfilter
    rng = np.random.default_rng(9)
    T, a = 50, 0.9
    q, k, v = (rng.standard_normal((1, 1, T, 1)) for _ in range(3))
    S_in = np.array([[[[0.7]]]])
    o, S_out = oracle.fwd(q, k, v, np.array([a]), S_in)
    x = (k * v)[0, 0, :, 0]
    S_t, _ = lfilter([1.0], [1.0, -a], x, zi=[a * 0.7])
    np.testing.assert_allclose(o[0, 0, :, 0], q[0, 0, :, 0] * S_t, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S_out[0, 0, 0, 0], S_t[-1], rtol=1e-12)


def test_single_step():
    rng = np.random.default_rng(12)
    q, k, v, a, S_in = rand_case(rng, 1, 1, 1, 3, 2, decay="token")
    o, S_out = oracle.fwd(q, k, v, a, S_in)
    a1 = a[0, 0, 0]
    exp = a1 * q[0, 0, 0] @ S_in[0, 0] + np.dot(q[0, 0, 0], k[0, 0, 0]) * v[0, 0, 0]
    np.testing.assert_allclose(o[0, 0, 0], exp, rtol=1e-14)


def test_zero_keys_only_decay():
    rng = np.random.default_rng(13)
    q, k, v, a, S_in = rand_case(rng, 1, 2, 20, 3, 4, decay="token")
    k[:] = 0
    o, S_out = oracle.fwd(q, k, v, a, S_in)
    P = np.cumprod(a, axis=-1)
    np.testing.assert_allclose(S_out, P[..., -1, None, None] * S_in, rtol=1e-13)
    np.testing.assert_allclose(o, P[..., None] * (q @ S_in), rtol=1e-12, atol=1e-13)


def test_zero_upstream_gradient():
    """dO = 0: only dS_out drives the backward; G_t = (prod_{r>t} a_r) dS_out."""
    rng = np.random.default_rng(14)
    q, k, v, a, S_in = rand_case(rng, 1, 2, 16, 3, 4, decay="token")
    dO = np.zeros(v.shape)
    dS_out = rng.standard_normal(S_in.shape)
    dq, dk_, dv_, dS_in = oracle.bwd(q, k, v, a, S_in, dO, dS_out)
    P = np.cumprod(a, axis=-1)
    assert np.all(dq == 0)
    np.testing.assert_allclose(dS_in, P[..., -1, None, None] * dS_out, rtol=1e-13)
    tail = P[..., -1:] / P                       # prod_{r>t} a_r
    G = tail[..., None, None] * dS_out[:, :, None]
    np.testing.assert_allclose(dk_, np.einsum("bhtij,bhtj->bhti", G, v), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dv_, np.einsum("bhti,bhtij->bhtj", k, G), rtol=1e-12, atol=1e-13)


def test_linearity():
    rng = np.random.default_rng(15)
    q, k, v, a, S_in = rand_case(rng, 1, 2, 20, 3, 4, decay="head")
    o, S_out = oracle.fwd(q, k, v, a, S_in)
    o2, S2 = oracle.fwd(3.0 * q, k, v, a, S_in)
    np.testing.assert_allclose(o2, 3.0 * o, rtol=1e-13, atol=1e-14)
    assert np.array_equal(S2, S_out)
    o3, S3 = oracle.fwd(q, k, -2.0 * v, a, -2.0 * S_in)
    np.testing.assert_allclose(o3, -2.0 * o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(S3, -2.0 * S_out, rtol=1e-13, atol=1e-14)


def test_thread_count_does_not_change_bits():
    rng = np.random.default_rng(16)
    q, k, v, a, S_in = rand_case(rng, 2, 4, 50, 8, 8, decay="token")
    dO = rng.standard_normal(v.shape)
    r1 = oracle.bwd(q, k, v, a, S_in, dO, None, nthreads=1)
    r8 = oracle.bwd(q, k, v, a, S_in, dO, None, nthreads=8)
    for x, y in zip(r1, r8):
        assert np.array_equal(x, y)


def test_strided_views():
    """A piece passed as a strided view of a longer tensor gives the same bits
    as a contiguous copy (the oracle honours the strides it is handed)."""
    rng = np.random.default_rng(17)
    q, k, v, a, S_in = rand_case(rng, 2, 2, 64, 4, 4, decay="token")
    sl = slice(16, 48)
    o1, S1 = oracle.fwd(q[:, :, sl], k[:, :, sl], v[:, :, sl], np.ascontiguousarray(a[:, :, sl]), S_in)
    o2, S2 = oracle.fwd(*(np.ascontiguousarray(x[:, :, sl]) for x in (q, k, v)),
                        np.ascontiguousarray(a[:, :, sl]), S_in)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)
