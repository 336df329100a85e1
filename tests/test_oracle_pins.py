"""Pins of the fp64 oracle against things other than itself.

Sources:
  [CB]  Inference Cookbook, "反向传播算法详解" (FlashAttention backward explained).
  [FA1] "解析 FlashAttention（3）：FlashAttention-v1 反向传播" (FlashAttention-v1 backward).

Pins used here:
  * the N=2, d=2 element-by-element chain rule of [FA1] section 2, typed out
    entry by entry (no matrix algebra), at seeded inputs;
  * central finite differences of L = <dO, O(Q, K, V)> through the oracle's
    forward only, for causal, softcap and GQA variants;
  * torch's fp64 autograd of scaled_dot_product_attention (a library routine);
  * identities the pages state or imply: [FA1] eq (3) = eq (6); rows of dZ sum
    to zero; <V, dV> = sum D; sum <Q, dQ> = <K, dK>;
  * closed forms: N = 1, Q = 0, the first causal row, a huge cap, GQA as MHA
    with repeated K/V.
"""
import math

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def rnd(rng, *shape, s=1.0):
    return rng.standard_normal(shape) * s


# ---------------------------------------------------------------- [FA1] N=2, d=2
def fa1_n2_d2_by_hand(q, k, v, dO, tau):
    """The scalar expansions of [FA1] 2.2-2.5, one entry at a time (1-based names)."""
    q11, q12, q21, q22 = q[0, 0], q[0, 1], q[1, 0], q[1, 1]
    k11, k12, k21, k22 = k[0, 0], k[0, 1], k[1, 0], k[1, 1]
    v11, v12, v21, v22 = v[0, 0], v[0, 1], v[1, 0], v[1, 1]
    dO11, dO12, dO21, dO22 = dO[0, 0], dO[0, 1], dO[1, 0], dO[1, 1]
    # [FA1] 2.5: S = tau Q K^T entry by entry
    S11 = tau * (q11 * k11 + q12 * k12)
    S12 = tau * (q11 * k21 + q12 * k22)
    S21 = tau * (q21 * k11 + q22 * k12)
    S22 = tau * (q21 * k21 + q22 * k22)
    # [FA1] 2.3: row softmax
    p11 = math.exp(S11) / (math.exp(S11) + math.exp(S12))
    p12 = math.exp(S12) / (math.exp(S11) + math.exp(S12))
    p21 = math.exp(S21) / (math.exp(S21) + math.exp(S22))
    p22 = math.exp(S22) / (math.exp(S21) + math.exp(S22))
    # [FA1] 2.2: O = P V entry by entry
    O11 = p11 * v11 + p12 * v21
    O12 = p11 * v12 + p12 * v22
    O21 = p21 * v11 + p22 * v21
    O22 = p21 * v12 + p22 * v22
    # [FA1] 2.2: dV entries (dL/dv_ab)
    dv11 = dO11 * p11 + dO21 * p21
    dv12 = dO12 * p11 + dO22 * p21
    dv21 = dO11 * p12 + dO21 * p22
    dv22 = dO12 * p12 + dO22 * p22
    # [FA1] 2.2 / 2.4: dP entries
    dp11 = dO11 * v11 + dO12 * v12
    dp12 = dO11 * v21 + dO12 * v22
    dp21 = dO21 * v11 + dO22 * v12
    dp22 = dO21 * v21 + dO22 * v22
    # [FA1] eq (3): D from P and dP; eq (6) (2.4): D from dO and O
    D1_p = p11 * dp11 + p12 * dp12
    D2_p = p21 * dp21 + p22 * dp22
    D1_o = dO11 * O11 + dO12 * O12
    D2_o = dO21 * O21 + dO22 * O22
    # [FA1] eq (4) per row: ds = p o (dp - D)
    ds11 = p11 * (dp11 - D1_p)
    ds12 = p12 * (dp12 - D1_p)
    ds21 = p21 * (dp21 - D2_p)
    ds22 = p22 * (dp22 - D2_p)
    # [FA1] 2.5: dL/dq_ab and dL/dk_ab
    dq11 = ds11 * tau * k11 + ds12 * tau * k21
    dq12 = ds11 * tau * k12 + ds12 * tau * k22
    dq21 = ds21 * tau * k11 + ds22 * tau * k21
    dq22 = ds21 * tau * k12 + ds22 * tau * k22
    dk11 = ds11 * tau * q11 + ds21 * tau * q21
    dk12 = ds11 * tau * q12 + ds21 * tau * q22
    dk21 = ds12 * tau * q11 + ds22 * tau * q21
    dk22 = ds12 * tau * q12 + ds22 * tau * q22
    return dict(
        O=np.array([[O11, O12], [O21, O22]]),
        D_p=np.array([D1_p, D2_p]),
        D_o=np.array([D1_o, D2_o]),
        dQ=np.array([[dq11, dq12], [dq21, dq22]]),
        dK=np.array([[dk11, dk12], [dk21, dk22]]),
        dV=np.array([[dv11, dv12], [dv21, dv22]]),
        P=np.array([[p11, p12], [p21, p22]]),
        dP=np.array([[dp11, dp12], [dp21, dp22]]),
        dS=np.array([[ds11, ds12], [ds21, ds22]]),
    )


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_fa1_n2_d2_hand_expansion(seed):
    rng = np.random.default_rng(seed)
    q, k, v, dO = (rnd(rng, 2, 2) for _ in range(4))
    tau = 0.7
    h = fa1_n2_d2_by_hand(q, k, v, dO, tau)
    # [FA1] 2.4: the two routes to D agree
    np.testing.assert_allclose(h["D_p"], h["D_o"], rtol=0, atol=1e-14)
    r = oracle.reference(q[None, None], k[None, None], v[None, None], dO[None, None], tau)
    for name in ("O", "dQ", "dK", "dV"):
        np.testing.assert_allclose(r[name][0, 0], h[name], rtol=0, atol=1e-14, err_msg=name)
    np.testing.assert_allclose(r["D"][0, 0], h["D_o"], rtol=0, atol=1e-14)


@pytest.mark.parametrize("seed", [0, 1])
def test_fa1_softmax_jacobian(seed):
    """[FA1] 2.3: ds = dp J with J = diag(p) - p^T p equals eq (4) p o (dp - D)."""
    rng = np.random.default_rng(seed)
    s = rnd(rng, 5)
    dp = rnd(rng, 5)
    p = np.exp(s - s.max())
    p /= p.sum()
    J = np.diag(p) - np.outer(p, p)
    # J against a finite-difference Jacobian of softmax itself
    eps = 1e-6
    Jfd = np.zeros((5, 5))
    for j in range(5):
        e = np.zeros(5)
        e[j] = eps
        sp, sm = s + e, s - e
        pp = np.exp(sp - sp.max()); pp /= pp.sum()
        pm = np.exp(sm - sm.max()); pm /= pm.sum()
        Jfd[:, j] = (pp - pm) / (2 * eps)
    np.testing.assert_allclose(J, Jfd, atol=1e-9)
    ds_j = dp @ J
    ds_4 = p * (dp - p @ dp)
    np.testing.assert_allclose(ds_j, ds_4, atol=1e-15)


# ---------------------------------------------------------------- finite differences
def _loss(Q, K, V, dO, tau, causal, softcap):
    O, _ = oracle.forward(Q, K, V, tau, causal, softcap)
    return float((dO * O).sum())


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("softcap", [0.0, 1.3])
@pytest.mark.parametrize("shape", [(1, 1, 1, 5, 3), (1, 4, 2, 4, 2), (2, 2, 1, 3, 4)])
def test_finite_differences(causal, softcap, shape):
    B, H, Hkv, N, d = shape
    rng = np.random.default_rng(100 + N + 7 * d + H)
    Q = rnd(rng, B, H, N, d, s=1.5)
    K = rnd(rng, B, Hkv, N, d, s=1.5)
    V = rnd(rng, B, Hkv, N, d)
    dO = rnd(rng, B, H, N, d)
    tau = 0.6
    O, LSE = oracle.forward(Q, K, V, tau, causal, softcap)
    dQ, dK, dV, _ = oracle.backward(Q, K, V, O, dO, LSE, tau, causal, softcap)
    h = 1e-6
    for X, G in ((Q, dQ), (K, dK), (V, dV)):
        fd = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            old = X[idx]
            X[idx] = old + h
            lp = _loss(Q, K, V, dO, tau, causal, softcap)
            X[idx] = old - h
            lm = _loss(Q, K, V, dO, tau, causal, softcap)
            X[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        scale = max(np.abs(G).max(), 1e-3)
        assert np.abs(fd - G).max() / scale < 1e-7


# ---------------------------------------------------------------- torch fp64 autograd
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 4, 2, 37, 16), (1, 3, 3, 64, 8), (1, 2, 1, 1, 4)])
def test_torch_sdpa_fp64(causal, shape):
    B, H, Hkv, N, d = shape
    g = torch.Generator().manual_seed(N * 31 + d)
    Q = torch.randn(B, H, N, d, generator=g, dtype=torch.float64)
    K = torch.randn(B, Hkv, N, d, generator=g, dtype=torch.float64)
    V = torch.randn(B, Hkv, N, d, generator=g, dtype=torch.float64)
    dO = torch.randn(B, H, N, d, generator=g, dtype=torch.float64)
    tau = 1.0 / math.sqrt(d)
    q, k, v = (t.clone().requires_grad_(True) for t in (Q, K, V))
    out = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, is_causal=causal, scale=tau, enable_gqa=(H != Hkv))
    out.backward(dO)
    r = oracle.reference(Q, K, V, dO, tau, causal)
    np.testing.assert_allclose(r["O"], out.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(r["dQ"], q.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(r["dK"], k.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(r["dV"], v.grad.numpy(), atol=1e-11)
    # LSE against torch.logsumexp of the masked scaled scores
    G = H // Hkv
    Kr = K.repeat_interleave(G, dim=1)
    Z = tau * Q @ Kr.transpose(-1, -2)
    if causal:
        Z = Z.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(r["LSE"], torch.logsumexp(Z, dim=-1).numpy(), atol=1e-12)


# ---------------------------------------------------------------- identities
def _random_case(seed, B=1, H=4, Hkv=2, N=19, d=8, s=1.0):
    rng = np.random.default_rng(seed)
    return (rnd(rng, B, H, N, d, s=s), rnd(rng, B, Hkv, N, d, s=s), rnd(rng, B, Hkv, N, d),
            rnd(rng, B, H, N, d))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("softcap", [0.0, 2.0])
def test_identities(causal, softcap):
    Q, K, V, dO = _random_case(11, s=1.3)
    tau = 0.4
    r = oracle.reference(Q, K, V, dO, tau, causal, softcap)
    B, H, N, d = Q.shape
    G = H // K.shape[1]
    # [FA1] eq (3) = eq (6): D_i = sum_j P_ij dP_ij, with P from torch.softmax
    for h in range(H):
        q, k, v, do = Q[0, h], K[0, h // G], V[0, h // G], dO[0, h]
        R = q @ k.T
        Zs = tau * (softcap * np.tanh(R / softcap) if softcap else R)
        if causal:
            Zs = np.where(np.triu(np.ones((N, N), bool), 1), -np.inf, Zs)
        P = torch.softmax(torch.from_numpy(Zs), dim=-1).numpy()
        dP = do @ v.T
        np.testing.assert_allclose((P * dP).sum(1), r["D"][0, h], atol=1e-12)
        # rows of dZ = P o (dP - D) sum to zero
        dZ = P * (dP - r["D"][0, h][:, None])
        np.testing.assert_allclose(dZ.sum(1), 0.0, atol=1e-12)
    for g in range(K.shape[1]):
        hs = range(g * G, (g + 1) * G)
        # <V_g, dV_g> = sum over the group's rows of D ([FA1] eqs (1), (6))
        assert abs((V[0, g] * r["dV"][0, g]).sum() - sum(r["D"][0, h].sum() for h in hs)) < 1e-10
        # column sums of dV equal the sum of dO rows (rows of P sum to 1)
        np.testing.assert_allclose(r["dV"][0, g].sum(0), sum(dO[0, h].sum(0) for h in hs), atol=1e-10)
        # sum_h <Q_h, dQ_h> = <K_g, dK_g>: both equal sum dR o R ([FA1] eqs (7), (8))
        lhs = sum((Q[0, h] * r["dQ"][0, h]).sum() for h in hs)
        assert abs(lhs - (K[0, g] * r["dK"][0, g]).sum()) < 1e-10
        if softcap == 0.0:
            # rows of dZ sum to 0 => keys' dK rows sum to 0
            np.testing.assert_allclose(r["dK"][0, g].sum(0), 0.0, atol=1e-10)


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("softcap", [0.0, 3.0])
def test_single_key(softcap):
    """N = 1: P = 1, O = V, dV = dO, dQ = dK = 0, LSE = Z."""
    Q, K, V, dO = _random_case(5, H=2, Hkv=1, N=1, d=6)
    tau = 0.3
    r = oracle.reference(Q, K, V, dO, tau, True, softcap)
    np.testing.assert_allclose(r["O"][0, 0], V[0, 0], atol=1e-15)
    np.testing.assert_allclose(r["dV"][0, 0], dO[0, 0] + dO[0, 1], atol=1e-15)
    assert np.abs(r["dQ"]).max() < 1e-15 and np.abs(r["dK"]).max() < 1e-15
    Rraw = (Q[0, 0, 0] * K[0, 0, 0]).sum()
    z = tau * (softcap * math.tanh(Rraw / softcap) if softcap else Rraw)
    assert abs(r["LSE"][0, 0, 0] - z) < 1e-14


def test_zero_queries_uniform():
    """Q = 0, no mask: P = 1/N, O_i = mean(V), dV_j = mean_i dO_i, dK = 0."""
    _, K, V, dO = _random_case(6, H=1, Hkv=1, N=7, d=5)
    Q = np.zeros((1, 1, 7, 5))
    r = oracle.reference(Q, K, V, dO, 0.9)
    np.testing.assert_allclose(r["O"][0, 0], np.tile(V[0, 0].mean(0), (7, 1)), atol=1e-14)
    np.testing.assert_allclose(r["dV"][0, 0], np.tile(dO[0, 0].mean(0), (7, 1)), atol=1e-14)
    assert np.abs(r["dK"]).max() < 1e-15
    np.testing.assert_allclose(r["LSE"][0, 0], math.log(7), atol=1e-14)
    # dQ_i = tau * sum_j (1/N)(dP_ij - D_i) K_j with dP = dO V^T
    dP = dO[0, 0] @ V[0, 0].T
    D = (dO[0, 0] * r["O"][0, 0]).sum(1)
    dQ = 0.9 * ((dP - D[:, None]) / 7) @ K[0, 0]
    np.testing.assert_allclose(r["dQ"][0, 0], dQ, atol=1e-13)


def test_first_causal_row():
    """Causal row 0 sees only key 0: O_0 = V_0, dQ_0 = 0."""
    Q, K, V, dO = _random_case(7, H=2, Hkv=2, N=9, d=4)
    r = oracle.reference(Q, K, V, dO, 0.5, True)
    np.testing.assert_allclose(r["O"][0, :, 0], V[0, :, 0], atol=1e-15)
    assert np.abs(r["dQ"][0, :, 0]).max() < 1e-15


def test_huge_cap_is_uncapped():
    Q, K, V, dO = _random_case(8)
    a = oracle.reference(Q, K, V, dO, 0.5, True, 1e12)
    b = oracle.reference(Q, K, V, dO, 0.5, True, 0.0)
    for n in ("O", "LSE", "dQ", "dK", "dV"):
        np.testing.assert_allclose(a[n], b[n], atol=1e-9)


def test_gqa_equals_repeated_mha():
    Q, K, V, dO = _random_case(9, H=6, Hkv=2, N=11)
    G = 3
    a = oracle.reference(Q, K, V, dO, 0.45, True, 2.5)
    Kr, Vr = np.repeat(K, G, axis=1), np.repeat(V, G, axis=1)
    b = oracle.reference(Q, Kr, Vr, dO, 0.45, True, 2.5)
    np.testing.assert_allclose(a["dQ"], b["dQ"], atol=1e-14)
    np.testing.assert_allclose(a["dK"], b["dK"].reshape(1, 2, G, 11, 8).sum(2), atol=1e-13)
    np.testing.assert_allclose(a["dV"], b["dV"].reshape(1, 2, G, 11, 8).sum(2), atol=1e-13)


def test_empty():
    z = np.zeros((1, 2, 0, 4))
    r = oracle.reference(z, z[:, :1], z[:, :1], z, 0.5, True)
    assert r["dQ"].shape == (1, 2, 0, 4) and r["dK"].shape == (1, 1, 0, 4)


# ---------------------------------------------------------------- row-sampled oracle
@pytest.mark.parametrize("causal,softcap", [(False, 0.0), (True, 0.0), (True, 1.7)])
def test_rows_match_full(causal, softcap):
    Q, K, V, dO = _random_case(10, H=1, Hkv=1, N=23, d=6, s=1.4)
    q, k, v, do = Q[0, 0], K[0, 0], V[0, 0], dO[0, 0]
    tau = 0.55
    O, L = oracle.forward_head(q, k, v, tau, causal, softcap)
    dq, dk, dv, D = oracle.backward_head(q, k, v, O, do, L, tau, causal, softcap)
    rows = np.array([0, 3, 22, 11])
    Or, Lr = oracle.forward_rows_head(q, k, v, rows, tau, causal, softcap)
    np.testing.assert_allclose(Or, O[rows], atol=1e-15)
    np.testing.assert_allclose(Lr, L[rows], atol=1e-15)
    dqr, Dr = oracle.backward_q_rows_head(q, k, v, O[rows], do[rows], L[rows], rows, tau, causal, softcap)
    np.testing.assert_allclose(dqr, dq[rows], atol=1e-14)
    np.testing.assert_allclose(Dr, D[rows], atol=1e-15)
    dkr, dvr = oracle.backward_kv_rows_head(q, k, v, O, do, L, rows, tau, causal, softcap)
    np.testing.assert_allclose(dkr, dk[rows], atol=1e-14)
    np.testing.assert_allclose(dvr, dv[rows], atol=1e-14)


def test_window_invariants():
    """A window at least N wide on both sides masks nothing; causal equals
    the window (-1, 0); a window only narrows what a query sees."""
    rng = np.random.default_rng(21)
    B, H, N, d = 1, 2, 9, 4
    Q, K, V, dO = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    plain = oracle.reference(Q, K, V, dO, 0.5, False, 0.0)
    wide = oracle.reference(Q, K, V, dO, 0.5, False, 0.0, (N, N))
    for n in ("O", "LSE", "dQ", "dK", "dV"):
        assert np.allclose(plain[n], wide[n], atol=1e-12), n
    causal = oracle.reference(Q, K, V, dO, 0.5, True, 0.0)
    band = oracle.reference(Q, K, V, dO, 0.5, False, 0.0, (-1, 0))
    for n in ("O", "LSE", "dQ", "dK", "dV"):
        assert np.allclose(causal[n], band[n], atol=1e-12), n
    # LSE is a log-sum-exp over the visible keys: a narrower window cannot raise it.
    narrow = oracle.reference(Q, K, V, dO, 0.5, True, 0.0, (2, -1))
    assert np.all(narrow["LSE"] <= causal["LSE"] + 1e-12)
