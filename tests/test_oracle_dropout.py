"""Pins of the oracle's dropout replay (oracle/philox.py and the dropout
terms of oracle/attention.py).

What fixes each part, independently of the oracle's own code:
  * the generator: PyTorch's header-only Philox4x32-10 engine (compiled with
    g++) for the 32-bit instance, numpy's Philox bit generator for the
    64-bit instance of the same round structure, and the closed forms of the
    Weyl key increments;
  * the element -> counter mapping and the keep rule u < t: the same engine,
    called with counters composed from the mapping's statement;
  * the scale 1/(1 - p): E[Z] = 1 and the keep fraction (binomial bounds),
    and E over seeds of the dropped output equals the undropped output;
  * the backward with dropout (the FlashAttention-v1 page, eqs (10)-(14)):
    torch fp64 autograd of the forward O = (softmax(Z) o M) V with the mask M
    held fixed, and the identity D_i = sum_j P_ij dP_ij of eq (13).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import philox
from tests._philox_ref import torch_philox_first_block

U64 = (1 << 64) - 1


# ---------------------------------------------------------------- generator

def test_philox4x32_matches_torch_engine():
    rng = np.random.default_rng(11)
    triples = [(0, 0, 0), (U64, U64, U64), (1, 0, 0), (0, 1, 0), (0, 0, 1), (0xDEADBEEF, 7, 1 << 40)]
    triples += [tuple(int(v) for v in rng.integers(0, U64, 3, dtype=np.uint64, endpoint=True)) for _ in range(40)]
    ref = torch_philox_first_block(triples)
    ctr = [[o & 0xFFFFFFFF, o >> 32, u & 0xFFFFFFFF, u >> 32] for s, u, o in triples]
    key = [[s & 0xFFFFFFFF, s >> 32] for s, u, o in triples]
    np.testing.assert_array_equal(philox.philox4x32(ctr, key), ref)


@pytest.mark.parametrize("key,counter", [((1, 2), (0, 0, 0, 0)), ((U64, 0), (U64, 5, 6, 7)),
                                         ((0x0123456789ABCDEF, 42), (3, U64, U64, 9))])
def test_philox4x64_round_structure_matches_numpy(key, counter):
    """numpy's Philox (4x64-10) advances the counter by one before each block."""
    g = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(counter, dtype=np.uint64))
    got = [int(v) for v in g.random_raw(8)]
    c = list(counter)
    for blk in range(2):
        # counter + 1 with carry through the four words
        for i in range(4):
            c[i] = (c[i] + 1) & U64
            if c[i] != 0:
                break
        assert philox.philox4x64(c, key) == got[4 * blk:4 * blk + 4]


def test_weyl_constants_closed_form():
    """Key increments: fractional parts of the golden ratio and sqrt(3) in fixed point."""
    for bits, (w0, w1) in ((32, philox.PHILOX_W32), (64, philox.PHILOX_W64)):
        one = 1 << bits
        assert (math.isqrt(5 << (2 * bits)) - one) // 2 == w0  # floor(2^bits (phi - 1))
        assert math.isqrt(3 << (2 * bits)) - one == w1  # floor(2^bits (sqrt 3 - 1))


# ------------------------------------------------------------- mask mapping

def test_dropout_bits_follow_the_stated_counter_mapping():
    """u(bh, q, k) = half (k & 1) of word (q & 3) of Philox(counter (k>>1, q>>2, bh, offset), key seed)."""
    rng = np.random.default_rng(5)
    seed, offset = 0x1234_5678_9ABC_DEF0, 77
    q = rng.integers(0, 1 << 20, 24)
    k = rng.integers(0, 1 << 20, 24)
    bh = rng.integers(0, 1 << 12, 24)
    # the engine's offset fills counter words 0-1, its subsequence words 2-3
    trip = [(seed, int(h) | (offset << 32), (int(kk) >> 1) | ((int(qq) >> 2) << 32)) for qq, kk, h in zip(q, k, bh)]
    words = torch_philox_first_block(trip)
    for n, (qq, kk, h) in enumerate(zip(q, k, bh)):
        want = (int(words[n, qq & 3]) >> (16 * (kk & 1))) & 0xFFFF
        assert int(philox.dropout_bits(seed, offset, int(h), [qq], [kk])[0, 0]) == want


def test_keep_rule_at_the_threshold():
    """Kept iff u < t: with t set to a value that occurs, that element is dropped; t + 1 keeps it."""
    seed, offset, bh = 99, 3, 5
    q, k = np.arange(8), np.arange(16)
    trip = [(seed, bh | (offset << 32), (kk >> 1) | ((qq >> 2) << 32)) for qq in q for kk in k]
    words = torch_philox_first_block(trip).reshape(8, 16, 4)
    u = np.array([[(int(words[qq, kk, qq & 3]) >> (16 * (kk & 1))) & 0xFFFF for kk in k] for qq in q])
    u0 = int(np.sort(u.ravel())[u.size // 2])  # a value that occurs
    for t in (u0, u0 + 1):
        p = 1.0 - t / 65536.0  # exact in float32: t / 65536 has at most 17 significant bits
        assert philox.keep_threshold(p) == t
        z = philox.dropout_multiplier(p, seed, offset, bh, q, k)
        np.testing.assert_array_equal(z > 0, u < t)
        assert np.all(z[z > 0] == 1.0 / (1.0 - np.float64(np.float32(p))))


def test_keep_threshold_values():
    assert philox.keep_threshold(0.0) == 65536
    assert philox.keep_threshold(0.5) == 32768
    assert philox.keep_threshold(np.float32(0.1)) == math.floor((1 - float(np.float32(0.1))) * 65536 + 0.5)
    for bad in (-0.1, 1.0, 1.5, float("nan")):
        with pytest.raises(ValueError):
            philox.keep_threshold(bad)


def test_sub_blocks_agree_with_the_full_matrix():
    full = philox.dropout_bits(7, 1, 3, np.arange(37), np.arange(53))
    rows, cols = np.array([36, 0, 5, 17]), np.array([52, 1, 2, 31, 30])
    np.testing.assert_array_equal(philox.dropout_bits(7, 1, 3, rows, cols), full[np.ix_(rows, cols)])


# -------------------------------------------------------------- statistics

@pytest.mark.parametrize("p", [0.1, 0.5, 0.875])
def test_mask_is_unbiased(p):
    """E[Z] = 1 and the keep fraction is t / 65536, within 5 binomial sigma."""
    n = 512
    z = philox.dropout_multiplier(p, 2024, 0, 1, np.arange(n), np.arange(n))
    keep = philox.keep_threshold(p) / 65536.0
    frac = (z > 0).mean()
    sigma = math.sqrt(keep * (1 - keep) / z.size)
    assert abs(frac - keep) < 5 * sigma
    assert abs(z.mean() - keep / (1 - float(np.float32(p)))) < 5 * sigma / (1 - p)
    assert abs(z.mean() - 1.0) < 5 * sigma / (1 - p) + 2e-5


def test_uniform_and_decorrelated():
    n = 256
    u = philox.dropout_bits(1, 0, 0, np.arange(n), np.arange(n)).astype(np.int64)
    hist = np.bincount(u.ravel() >> 12, minlength=16)
    expected = u.size / 16
    chi2 = ((hist - expected) ** 2 / expected).sum()
    assert chi2 < 50  # 15 degrees of freedom: P(chi2 > 50) ~ 1e-5
    for other in (philox.dropout_bits(2, 0, 0, np.arange(n), np.arange(n)),   # seed
                  philox.dropout_bits(1, 1, 0, np.arange(n), np.arange(n)),   # offset
                  philox.dropout_bits(1, 0, 1, np.arange(n), np.arange(n))):  # head
        assert (other.astype(np.int64) == u).mean() < 1e-3
    # neighbouring rows and columns of one block are not copies of each other
    assert (u[0::2] == u[1::2]).mean() < 1e-3 and (u[:, 0::2] == u[:, 1::2]).mean() < 1e-3


# ------------------------------------------------------------------- math

def _rnd(g, *shape, s=1.0):
    return torch.randn(*shape, generator=g, dtype=torch.float64) * s


def autograd_dropout(Q, K, V, dO, tau, causal, softcap, window, dropout):
    """fp64 autograd of O = (softmax(Z) o M) V with the mask M held fixed."""
    B, H, N, d = Q.shape
    G = H // K.shape[1]
    q, k, v = (t.clone().requires_grad_(True) for t in (Q, K, V))
    kk, vv = k.repeat_interleave(G, dim=1), v.repeat_interleave(G, dim=1)
    R = q @ kk.transpose(-1, -2)
    Z = tau * (softcap * torch.tanh(R / softcap) if softcap > 0 else R)
    i, j = torch.arange(N)[:, None], torch.arange(N)[None, :]
    vis = torch.ones(N, N, dtype=torch.bool)
    if causal:
        vis &= j <= i
    wl, wr = window
    if wl >= 0:
        vis &= j >= i - wl
    if wr >= 0:
        vis &= j <= i + wr
    P = torch.softmax(Z.masked_fill(~vis, -math.inf), dim=-1)
    p, seed, off = dropout
    M = torch.stack([torch.stack([torch.from_numpy(philox.dropout_multiplier(p, seed, off, b * H + h, np.arange(N),
                                                                             np.arange(N))) for h in range(H)])
                     for b in range(B)])
    O = (P * M) @ vv
    O.backward(dO)
    return O.detach(), q.grad, k.grad, v.grad


CASES = [  # causal, softcap, window, (B, H, H_kv, N, d), p
    (False, 0.0, (-1, -1), (1, 2, 2, 13, 4), 0.3),
    (True, 0.0, (-1, -1), (2, 4, 2, 11, 3), 0.5),
    (True, 1.4, (-1, -1), (1, 4, 1, 9, 5), 0.2),
    (False, 0.0, (3, 2), (1, 2, 1, 12, 4), 0.6),
    (True, 2.0, (4, -1), (1, 3, 3, 10, 2), 0.1),
]


@pytest.mark.parametrize("causal,softcap,window,shape,p", CASES)
def test_dropout_backward_matches_autograd(causal, softcap, window, shape, p):
    B, H, Hkv, N, d = shape
    g = torch.Generator().manual_seed(N)
    Q, K = _rnd(g, B, H, N, d, s=1.3), _rnd(g, B, Hkv, N, d, s=1.3)
    V, dO = _rnd(g, B, Hkv, N, d), _rnd(g, B, H, N, d)
    drop = (p, 0xABCDEF12345, 9)
    O, dq, dk, dv = autograd_dropout(Q, K, V, dO, 0.6, causal, softcap, window, drop)
    r = oracle.reference(Q, K, V, dO, 0.6, causal, softcap, window, drop)
    for name, want in (("O", O), ("dQ", dq), ("dK", dk), ("dV", dv)):
        np.testing.assert_allclose(r[name], want.numpy(), atol=1e-11, rtol=0, err_msg=name)


def test_dropout_D_is_rowsum_of_P_dP():
    """D_i = dO_i . O_i equals sum_j P_ij dP_ij with dP = (dO V^T) o Z (eqs (12), (13))."""
    rng = np.random.default_rng(8)
    N, d, tau, drop = 15, 6, 0.4, (0.4, 31, 2)
    q, k, v, do = (rng.standard_normal((N, d)) for _ in range(4))
    zf = oracle.head_dropout(drop, 0)
    o, lse = oracle.forward_head(q, k, v, tau, True, 0.0, None, zf)
    D = oracle.backward_head(q, k, v, o, do, lse, tau, True, 0.0, None, zf)[3]
    i = np.arange(N)
    P = np.where(i[None, :] <= i[:, None], np.exp(tau * q @ k.T - lse[:, None]), 0.0)
    dP = (do @ v.T) * zf(i, i)
    np.testing.assert_allclose(D, (P * dP).sum(axis=1), atol=1e-12)


def test_expected_output_is_undropped():
    """Averaged over seeds, the dropped output approaches the undropped one."""
    rng = np.random.default_rng(9)
    N, d, tau = 6, 3, 0.8
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    o_ref = oracle.forward_head(q, k, v, tau, False)[0]
    n = 3000
    acc = np.zeros_like(o_ref)
    sq = np.zeros_like(o_ref)
    for s in range(n):
        o = oracle.forward_head(q, k, v, tau, False, 0.0, None, oracle.head_dropout((0.5, s, 0), 0))[0]
        acc += o
        sq += o * o
    mean = acc / n
    se = np.sqrt(np.maximum(sq / n - mean * mean, 1e-30) / n)
    assert np.all(np.abs(mean - o_ref) < 5 * se)


def test_p0_is_no_dropout():
    rng = np.random.default_rng(10)
    Q, K, V, dO = (rng.standard_normal((1, 2, 7, 3)) for _ in range(4))
    a = oracle.reference(Q, K, V, dO, 0.5, True)
    b = oracle.reference(Q, K, V, dO, 0.5, True, dropout=(0.0, 5, 6))
    for n in a:
        np.testing.assert_array_equal(a[n], b[n])


@pytest.mark.parametrize("causal,softcap", [(False, 0.0), (True, 1.5)])
def test_dropout_rows_match_full(causal, softcap):
    rng = np.random.default_rng(12)
    N, d, tau = 21, 4, 0.5
    q, k, v, do = (rng.standard_normal((N, d)) for _ in range(4))
    zf = oracle.head_dropout((0.35, 4, 1), 2)
    o, lse = oracle.forward_head(q, k, v, tau, causal, softcap, None, zf)
    dq, dk, dv, D = oracle.backward_head(q, k, v, o, do, lse, tau, causal, softcap, None, zf)
    rows = np.array([20, 3, 0, 11])
    o_r, lse_r = oracle.forward_rows_head(q, k, v, rows, tau, causal, softcap, None, zf)
    np.testing.assert_allclose(o_r, o[rows], atol=1e-13)
    dq_r, D_r = oracle.backward_q_rows_head(q, k, v, o[rows], do[rows], lse[rows], rows, tau, causal, softcap, None, zf)
    np.testing.assert_allclose(dq_r, dq[rows], atol=1e-12)
    np.testing.assert_allclose(D_r, D[rows], atol=1e-12)
    cols = np.array([0, 19, 7])
    dk_c, dv_c = oracle.backward_kv_rows_head(q, k, v, o, do, lse, cols, tau, causal, softcap, None, zf)
    np.testing.assert_allclose(dk_c, dk[cols], atol=1e-12)
    np.testing.assert_allclose(dv_c, dv[cols], atol=1e-12)
