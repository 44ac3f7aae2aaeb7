"""Pins of the fp64 delta-rule oracle against things other than itself.

The gated delta rule S_t = a_t (I - beta_t k_t^T k_t) S_{t-1} + beta_t k_t^T v_t,
o_t = q_t S_t is the recurrence of the Gated DeltaNet models StateFlow trains
(the gptget summary, "Experimental design").  Each test fixes part of the
oracle by something independent of its code: central finite differences of
the loss, torch autograd of a separately written recurrence, a chunkwise
closed form with a triangular solve, special cases with known answers
(beta = 0 is pure decay; a unit key written with beta = 1 is read back
exactly), and bitwise split invariance.  d_k != d_v throughout so that a
transposed operand cannot pass."""
import numpy as np
import pytest
import torch

import oracle


def case(rng, B=1, H=2, T=9, dk=3, dv=4, decay="token", lo=0.7, s_in=True, unit_k=True):
    q = rng.standard_normal((B, H, T, dk))
    k = rng.standard_normal((B, H, T, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, H, T, dv))
    beta = rng.uniform(0.1, 1.0, (B, H, T))
    if decay == "token":
        a = rng.uniform(lo, 1.0, (B, H, T))
    elif decay == "head":
        a = rng.uniform(lo, 1.0, (H,))
    else:
        a = None
    S_in = rng.standard_normal((B, H, dk, dv)) if s_in else None
    return q, k, v, beta, a, S_in


def loss(q, k, v, beta, a, S_in, dO, dS_out):
    o, S_out = oracle.delta_fwd(q, k, v, beta, a, S_in)
    return float(np.sum(dO * o) + np.sum(dS_out * S_out))


def full_decay(a, B, H, T):
    if a is None:
        return np.ones((B, H, T))
    if a.ndim == 1:
        return np.broadcast_to(a[None, :, None], (B, H, T)).copy()
    return a


@pytest.mark.parametrize("T", [9, 70])
def test_backward_matches_finite_differences(T):
    """Every input, central differences.  T = 70 crosses the oracle's
    64-token checkpoint block (its reverse sweep rebuilds S_{t-1} per block);
    there only entries at the block edges are probed."""
    rng = np.random.default_rng(41 + T)
    B, H, dk, dv = 1, 2, 3, 4
    q, k, v, beta, a, S_in = case(rng, B, H, T, dk, dv)
    dO = rng.standard_normal((B, H, T, dv))
    dS_out = rng.standard_normal((B, H, dk, dv))
    dq, dk_, dv_, dbeta, dS_in, da = oracle.delta_bwd(q, k, v, beta, a, S_in, dO, dS_out,
                                                       want_da=True)
    grads = {"q": (q, dq), "k": (k, dk_), "v": (v, dv_), "beta": (beta, dbeta), "a": (a, da),
             "S_in": (S_in, dS_in)}
    eps = 1e-6
    for name, (x, gx) in grads.items():
        flat = x.reshape(-1)
        idxs = range(flat.size)
        if T > 9:
            per_t = flat.size // (B * H * T) if name not in ("S_in",) else None
            if per_t:
                ts = (0, 62, 63, 64, 65, T - 1)
                idxs = [((bh * T) + t) * per_t + c for bh in range(B * H) for t in ts
                        for c in range(per_t)]
        for idx in idxs:
            old = flat[idx]
            flat[idx] = old + eps
            lp = loss(q, k, v, beta, a, S_in, dO, dS_out)
            flat[idx] = old - eps
            lm = loss(q, k, v, beta, a, S_in, dO, dS_out)
            flat[idx] = old
            fd = (lp - lm) / (2 * eps)
            an = gx.reshape(-1)[idx]
            assert abs(fd - an) <= 2e-7 * max(1.0, abs(an)), (name, idx, fd, an)


def recurrence_torch(q, k, v, beta, a, S_in):
    """The delta rule written directly as the matrix recurrence, in torch."""
    B, H, T, dk = k.shape
    eye = torch.eye(dk, dtype=torch.float64)
    S = S_in
    outs = []
    for t in range(T):
        kt = k[:, :, t]                                            # [B,H,dk]
        M = a[:, :, t, None, None] * (eye - beta[:, :, t, None, None] * kt[..., :, None] * kt[..., None, :])
        S = M @ S + beta[:, :, t, None, None] * kt[..., :, None] * v[:, :, t, None, :]
        outs.append((q[:, :, t, None, :] @ S)[:, :, 0])
    return torch.stack(outs, dim=2), S


def test_backward_matches_torch_autograd():
    rng = np.random.default_rng(43)
    B, H, T, dk, dv = 2, 2, 40, 5, 7
    q, k, v, beta, a, S_in = case(rng, B, H, T, dk, dv, lo=0.8)
    dO = rng.standard_normal((B, H, T, dv))
    dS_out = rng.standard_normal((B, H, dk, dv))
    ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, beta, a, S_in)]
    o, S_out = recurrence_torch(*ts)
    L = (o * torch.tensor(dO)).sum() + (S_out * torch.tensor(dS_out)).sum()
    L.backward()
    o_or, S_or = oracle.delta_fwd(q, k, v, beta, a, S_in)
    np.testing.assert_allclose(o_or, o.detach().numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(S_or, S_out.detach().numpy(), rtol=1e-11, atol=1e-11)
    got = oracle.delta_bwd(q, k, v, beta, a, S_in, dO, dS_out, want_da=True)
    names = ["dq", "dk", "dv", "dbeta", "dS_in", "da"]
    leaves = [0, 1, 2, 3, 5, 4]        # autograd leaves are (q, k, v, beta, a, S_in)
    for name, g, li in zip(names, got, leaves):
        np.testing.assert_allclose(g, ts[li].grad.numpy(), rtol=1e-9, atol=1e-9, err_msg=name)


def chunk_form(q, k, v, beta, a, S_in, C):
    """The delta rule chunk by chunk, without the token recurrence: with
    Gamma_i the chunk's cumulative decay up to token i, the new values
    U = (I + A)^{-1} diag(beta) (V - diag(Gamma) K S_0), A strictly lower
    triangular with A_ij = beta_i (Gamma_i / Gamma_j) k_i . k_j, then
    O = diag(Gamma) Q S_0 + [(Q K^T) .* D] U and
    S_C = Gamma_C S_0 + (K .* Gamma_C / Gamma)^T U, D_ij = Gamma_i / Gamma_j
    for j <= i.  Solved with numpy's triangular solve per chunk."""
    B, H, T, dk = k.shape
    dv = v.shape[3]
    af = full_decay(a, B, H, T)
    o = np.zeros((B, H, T, dv))
    S_out = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S_in is None else S_in[b, h].copy()
            for t0 in range(0, T, C):
                t1 = min(t0 + C, T)
                Q, K, V = q[b, h, t0:t1], k[b, h, t0:t1], v[b, h, t0:t1]
                bt = beta[b, h, t0:t1]
                g = np.cumprod(af[b, h, t0:t1])
                D = np.tril(g[:, None] / g[None, :])
                A = np.tril(bt[:, None] * D * (K @ K.T), -1)
                rhs = bt[:, None] * (V - g[:, None] * (K @ S))
                U = np.linalg.solve(np.eye(t1 - t0) + A, rhs)
                o[b, h, t0:t1] = g[:, None] * (Q @ S) + ((Q @ K.T) * D) @ U
                S = g[-1] * S + (K * (g[-1] / g)[:, None]).T @ U
            S_out[b, h] = S
    return o, S_out


@pytest.mark.parametrize("decay", ["token", "head", "none"])
def test_forward_matches_chunk_form(decay):
    rng = np.random.default_rng(44)
    q, k, v, beta, a, S_in = case(rng, 2, 2, 44, 6, 5, decay=decay)
    o, S_out = oracle.delta_fwd(q, k, v, beta, a, S_in)
    for C in (1, 8, 16):
        oc, Sc = chunk_form(q, k, v, beta, a, S_in, C)
        np.testing.assert_allclose(o, oc, rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(S_out, Sc, rtol=1e-11, atol=1e-11)


def test_zero_beta_is_pure_decay():
    rng = np.random.default_rng(45)
    q, k, v, beta, a, S_in = case(rng, 1, 2, 20, 3, 4)
    beta[:] = 0.0
    o, S_out = oracle.delta_fwd(q, k, v, beta, a, S_in)
    P = np.cumprod(a, axis=-1)
    np.testing.assert_allclose(S_out, P[..., -1, None, None] * S_in, rtol=1e-13)
    np.testing.assert_allclose(o, P[..., None] * (q @ S_in), rtol=1e-12, atol=1e-13)


def test_unit_key_with_unit_beta_overwrites_exactly():
    """With |k_t| = 1 and beta_t = 1 the update erases what the state held at
    k_t and writes v_t there: k_t S_t = v_t whatever came before."""
    rng = np.random.default_rng(46)
    B, H, T, dk, dv = 1, 2, 30, 4, 5
    q, k, v, beta, a, S_in = case(rng, B, H, T, dk, dv)
    hits = [3, 11, 12, 29]
    beta[:, :, hits] = 1.0
    q[:, :, hits] = k[:, :, hits]
    o, _ = oracle.delta_fwd(q, k, v, beta, a, S_in)
    np.testing.assert_allclose(o[:, :, hits], v[:, :, hits], rtol=1e-12, atol=1e-12)


def test_orthonormal_keys_do_not_interfere():
    """Orthonormal keys, beta = 1, no decay, S_in = 0: every write lands in a
    direction no other key reads, so the state is the plain outer-product
    sum of linear attention and each key reads back its own value."""
    rng = np.random.default_rng(47)
    dk, dv, T = 6, 3, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm[:T][None, None].copy()
    v = rng.standard_normal((1, 1, T, dv))
    beta = np.ones((1, 1, T))
    o, S_out = oracle.delta_fwd(k.copy(), k, v, beta, None, None)
    np.testing.assert_allclose(S_out[0, 0], k[0, 0].T @ v[0, 0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o, v, rtol=1e-12, atol=1e-12)


def run_split(q, k, v, beta, a, S_in, dO, dS_out, lengths):
    B, H, T, dk = k.shape
    af = full_decay(a, B, H, T) if a is not None else None
    bounds = np.cumsum([0] + list(lengths))
    S, starts, outs = S_in, [], []
    sl = lambda x, i: np.ascontiguousarray(x[:, :, bounds[i]:bounds[i + 1]])  # noqa: E731
    for i in range(len(lengths)):
        starts.append(S)
        o, S = oracle.delta_fwd(sl(q, i), sl(k, i), sl(v, i), sl(beta, i),
                                None if af is None else sl(af, i), S)
        outs.append(o)
    S_out, dS, grads = S, dS_out, [None] * len(lengths)
    for i in reversed(range(len(lengths))):
        dq, dk_, dv_, db, dS = oracle.delta_bwd(sl(q, i), sl(k, i), sl(v, i), sl(beta, i),
                                                None if af is None else sl(af, i), starts[i],
                                                sl(dO, i), dS)
        grads[i] = (dq, dk_, dv_, db)
    cat = lambda xs: np.concatenate(xs, axis=2)  # noqa: E731
    return (cat(outs), S_out, *(cat([g[j] for g in grads]) for j in range(4)), dS)


@pytest.mark.parametrize("lengths", [[48, 48], [1, 5, 90], [64, 20, 12]])
def test_split_invariance_is_bitwise(lengths):
    rng = np.random.default_rng(48)
    q, k, v, beta, a, S_in = case(rng, 2, 2, 96, 4, 6)
    dO = rng.standard_normal(v.shape)
    dS_out = rng.standard_normal(S_in.shape)
    o, S_out = oracle.delta_fwd(q, k, v, beta, a, S_in)
    dq, dk_, dv_, db, dS_in = oracle.delta_bwd(q, k, v, beta, a, S_in, dO, dS_out)
    got = run_split(q, k, v, beta, a, S_in, dO, dS_out, lengths)
    for x, y in zip(got, (o, S_out, dq, dk_, dv_, db, dS_in)):
        assert np.array_equal(x, y)


def test_thread_count_does_not_change_bits():
    rng = np.random.default_rng(49)
    q, k, v, beta, a, S_in = case(rng, 2, 4, 50, 8, 8)
    dO = rng.standard_normal(v.shape)
    r1 = oracle.delta_bwd(q, k, v, beta, a, S_in, dO, None, nthreads=1)
    r8 = oracle.delta_bwd(q, k, v, beta, a, S_in, dO, None, nthreads=8)
    for x, y in zip(r1, r8):
        assert np.array_equal(x, y)
