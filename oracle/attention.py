"""Plain fp64 CPU oracle of softmax attention, forward and backward.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path.  It
shares no code, header, table or helper with the HIP library.

Every step materialises the full N x N matrices of one head and follows the
definitions of the two source pages, cited as

  [CB]  Inference Cookbook, "反向传播算法详解" (FlashAttention backward pass
        explained), sections 1.2-2.3 (recompute P from LSE, the five gradients,
        the dPsum row dot product, the tanh softcap chain, dK scaled by the
        softmax scale, GQA head mapping in the epilogue section 8.5);
  [FA1] "解析 FlashAttention（3）：FlashAttention-v1 反向传播" (FlashAttention-v1
        backward), section 2 (the N=2, d=2 derivation) and equations (1)-(9).

Notation.  R = Q K^T are the raw scores ([CB] 1.1 calls them S).  With a tanh
softcap c > 0, T = tanh(R / c) and the capped score is c*T ([CB] 2.1 (3)).
Z = tau * (capped score) are the softmax logits ([FA1] 2.5 writes S = tau Q K^T
when there is no cap).  P = softmax(Z) row-wise, O = P V, LSE_i = ln sum_j
exp(Z_ij) ([CB] 1.2).  Causal masking sets Z_ij = -inf for key j > query i
(the diagonal is kept), after the cap ([CB] 5.2 step 3 applies the cap before
the mask).  A local (sliding-window) mask with window (wl, wr) also sets
Z_ij = -inf for j < i - wl (when wl >= 0) and for j > i + wr (when wr >= 0);
-1 leaves that side unbounded.

Readings taken where the pages are silent or ambiguous:
  * the cap applies to the unscaled scores R, and tau multiplies the capped
    value ([CB] 2.1 caps S_raw, and [CB] 1.1 defines S without the scale);
  * LSE is a natural logarithm;
  * the dPsum of [CB] 2.1 is D_i = sum_k dO_ik O_ik ([FA1] eq (6));
  * grouped-query attention: query head h reads key/value head h // G with
    G = H / H_kv, and dK, dV of a key/value head sum over its G query heads
    ([CB] 8.5);
  * the local mask: the backward-kernel page names a third masking phase for
    the query blocks at a local window's boundary but gives no formula; the
    window is read as the band i - wl <= j <= i + wr around the diagonal,
    combined with the causal mask when both are on;
  * dropout: [FA1] section 3.3 and the dropout lines of Algorithm 4 apply the
    replayed mask Z (elements 1/(1 - p) or 0) to P in the forward pass,
    O = (P o Z) V, and give dV = (P o Z)^T dO (eq (10)) and dP = (dO V^T) o Z
    (eq (12)); D = rowsum(dO o O) and dZ = P o (dP - D) are unchanged
    (eqs (13), (14)).  The pages fix no generator: oracle/philox.py states the
    Philox4x32-10 stream that is replayed.  LSE stays that of the undropped P.

Parity pins: tests/test_oracle_*.py (N=2, d=2 hand expansions of [FA1]
section 2, central finite differences of <dO, O>, invariants, closed forms,
torch fp64 autograd of scaled_dot_product_attention, hand-derived golden
fixtures under tests/golden/).
"""
from __future__ import annotations

import numpy as np

from . import philox

__all__ = [
    "forward",
    "forward_head",
    "backward",
    "backward_head",
    "forward_rows_head",
    "backward_q_rows_head",
    "backward_kv_rows_head",
    "reference",
    "head_dropout",
]


def _f64(x):
    """Exact upcast of a numpy array or CPU torch tensor to float64."""
    if hasattr(x, "detach"):  # torch tensor: upcast in torch, then hand to numpy
        import torch

        return x.detach().to(device="cpu", dtype=torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _visible(q_idx, k_idx, causal, window):
    """Boolean [len(q_idx), len(k_idx)]: key j is visible to query i."""
    i = q_idx[:, None]
    j = k_idx[None, :]
    ok = np.ones((q_idx.size, k_idx.size), dtype=bool)
    if causal:
        ok &= j <= i
    wl, wr = window if window is not None else (-1, -1)
    if wl >= 0:
        ok &= j >= i - wl
    if wr >= 0:
        ok &= j <= i + wr
    return ok


def _logits(q, k, q_idx, k_idx, tau, causal, softcap, window=None):
    """Logits Z (rows q_idx, columns k_idx) and T = tanh(R/c) (None if no cap).

    R = q K^T ([CB] 1.1); capped score c*tanh(R/c) ([CB] 2.1 (3));
    Z = tau * capped score; masked entries (causal: j > i; local window: outside
    i - wl <= j <= i + wr) are -inf ([FA1] section 4, the mask step of
    Algorithm 4 sets masked scores to -inf).
    """
    R = q @ k.T
    if softcap > 0.0:
        T = np.tanh(R / softcap)
        Z = tau * (softcap * T)
    else:
        T = None
        Z = tau * R
    if causal or (window is not None and tuple(window) != (-1, -1)):
        Z = np.where(_visible(q_idx, k_idx, causal, window), Z, -np.inf)
    return Z, T


def forward_rows_head(q, k, v, rows, tau, causal=False, softcap=0.0, window=None, zdrop=None):
    """O and LSE of the query rows `rows` of one head, straight from the definition.

    q: [N, d], k, v: [N, d].  P_i = softmax(Z_i) ([FA1] 1.1), O_i = P_i V,
    LSE_i = m_i + ln sum_j exp(Z_ij - m_i) with m_i = max_j Z_ij, which equals
    [FA1] eq (9)'s pair (m, l) through LSE = m + ln l, as [CB] 1.2 stores it.
    zdrop(rows, cols) -> dropout matrix Z, or None: O_i = (P_i o Z_i) V.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    rows = np.asarray(rows, dtype=np.int64)
    if rows.size == 0:
        return np.zeros((0, v.shape[1])), np.zeros((0,))
    Z, _ = _logits(q[rows], k, rows, np.arange(k.shape[0]), tau, causal, softcap, window)
    m = Z.max(axis=1)
    lse = m + np.log(np.exp(Z - m[:, None]).sum(axis=1))
    P = np.exp(Z - lse[:, None])
    if zdrop is not None:
        P = P * zdrop(rows, np.arange(k.shape[0]))
    return P @ v, lse


def forward_head(q, k, v, tau, causal=False, softcap=0.0, window=None, zdrop=None):
    """O [N, d] and LSE [N] of one head (all rows)."""
    n = _f64(q).shape[0]
    return forward_rows_head(q, k, v, np.arange(n), tau, causal, softcap, window, zdrop)


def backward_head(q, k, v, o, do, lse, tau, causal=False, softcap=0.0, window=None, zdrop=None):
    """dQ, dK, dV [N, d] and D [N] of one head from the saved forward tensors.

    Inputs are what [CB] 1.3 says the forward saves (Q, K, V, O, LSE) plus dO.
      P  = exp(Z - LSE)                 recomputed, [CB] 1.2
      dV = P^T dO                       [FA1] eq (1)
      dP = dO V^T                       [FA1] eq (2)
      D  = rowsum(dO o O)               [FA1] eq (6)
      dZ = P o (dP - D 1^T)             [FA1] eq (5)
      dR = tau dZ (1 - T^2) with cap, tau dZ without  ([CB] 2.1 (3); [FA1] 2.5)
      dQ = dR K,  dK = dR^T Q           [FA1] eqs (7), (8)
    With dropout (zdrop(rows, cols) -> Z): dV = (P o Z)^T dO ([FA1] eq (10))
    and dP = (dO V^T) o Z ([FA1] eq (12)).
    """
    q, k, v, o, do, lse = map(_f64, (q, k, v, o, do, lse))
    n = q.shape[0]
    if n == 0:
        z = np.zeros((0, q.shape[1]))
        return z, np.zeros_like(_f64(k)), np.zeros_like(_f64(v)), np.zeros((0,))
    idx = np.arange(n)
    Z, T = _logits(q, k, idx, np.arange(k.shape[0]), tau, causal, softcap, window)
    P = np.exp(Z - lse[:, None])
    del Z
    Zd = zdrop(idx, np.arange(k.shape[0])) if zdrop is not None else None
    dV = (P * Zd).T @ do if Zd is not None else P.T @ do
    dP = do @ v.T
    if Zd is not None:
        dP = dP * Zd
    D = (do * o).sum(axis=1)
    dZ = P * (dP - D[:, None])
    del P, dP
    if T is not None:
        dR = tau * dZ * (1.0 - T * T)
    else:
        dR = tau * dZ
    del dZ, T
    dQ = dR @ k
    dK = dR.T @ q
    return dQ, dK, dV, D


def backward_q_rows_head(q, k, v, o_rows, do_rows, lse_rows, rows, tau, causal=False, softcap=0.0, window=None,
                         zdrop=None):
    """dQ and D of the query rows `rows` of one head.

    Row i of dQ needs only row i of P, dP and D: dQ_i = sum_j dR_ij K_j
    ([FA1] eq (7) read row by row), with the same chain as `backward_head`.
    o_rows, do_rows, lse_rows hold the saved O, dO, LSE of those rows.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    o_rows, do_rows, lse_rows = _f64(o_rows), _f64(do_rows), _f64(lse_rows)
    rows = np.asarray(rows, dtype=np.int64)
    if rows.size == 0:
        return np.zeros((0, q.shape[1])), np.zeros((0,))
    Z, T = _logits(q[rows], k, rows, np.arange(k.shape[0]), tau, causal, softcap, window)
    P = np.exp(Z - lse_rows[:, None])
    dP = do_rows @ v.T
    if zdrop is not None:
        dP = dP * zdrop(rows, np.arange(k.shape[0]))
    D = (do_rows * o_rows).sum(axis=1)
    dZ = P * (dP - D[:, None])
    dR = tau * dZ * (1.0 - T * T) if T is not None else tau * dZ
    return dR @ k, D


def backward_kv_rows_head(q, k, v, o, do, lse, kv_rows, tau, causal=False, softcap=0.0, window=None, zdrop=None):
    """dK and dV of the key rows `kv_rows` contributed by one query head.

    Column j of P, dP and dZ over all query rows gives
    dV_j = sum_i P_ij dO_i ([FA1] eq (1)) and dK_j = sum_i dR_ij Q_i
    ([FA1] eq (8)).  Needs the saved O and LSE of every query row.
    """
    q, k, v, o, do, lse = map(_f64, (q, k, v, o, do, lse))
    cols = np.asarray(kv_rows, dtype=np.int64)
    if cols.size == 0:
        return np.zeros((0, k.shape[1])), np.zeros((0, v.shape[1]))
    Zc, Tc = _logits(q, k[cols], np.arange(q.shape[0]), cols, tau, causal, softcap, window)
    Pc = np.exp(Zc - lse[:, None])
    dPc = do @ v[cols].T
    Zd = zdrop(np.arange(q.shape[0]), cols) if zdrop is not None else None
    if Zd is not None:
        dPc = dPc * Zd
    D = (do * o).sum(axis=1)
    dZc = Pc * (dPc - D[:, None])
    dRc = tau * dZc * (1.0 - Tc * Tc) if Tc is not None else tau * dZc
    return dRc.T @ q, (Pc * Zd).T @ do if Zd is not None else Pc.T @ do


def head_dropout(dropout, bh):
    """zdrop(rows, cols) of query head bh (= b * H + h) for dropout = (p, seed, offset), or None.

    p = 0 turns dropout off."""
    if dropout is None or float(np.float32(dropout[0])) == 0.0:
        return None
    p, seed, offset = dropout
    return lambda rows, cols: philox.dropout_multiplier(p, seed, offset, bh, rows, cols)


def _group(H, H_kv):
    if H_kv <= 0 or H % H_kv != 0:
        raise ValueError(f"H={H} must be a positive multiple of H_kv={H_kv}")
    return H // H_kv


def forward(Q, K, V, tau, causal=False, softcap=0.0, window=None, dropout=None):
    """O [B,H,N,d] and LSE [B,H,N] for Q [B,H,N,d], K, V [B,H_kv,N,d].

    Query head h reads key/value head h // (H / H_kv) ([CB] 8.5).
    dropout = (p, seed, offset) replays the mask of oracle/philox.py.
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    B, H, N, d = Q.shape
    G = _group(H, K.shape[1])
    O = np.zeros((B, H, N, V.shape[3]))
    LSE = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            O[b, h], LSE[b, h] = forward_head(Q[b, h], K[b, h // G], V[b, h // G], tau, causal, softcap, window,
                                              head_dropout(dropout, b * H + h))
    return O, LSE


def backward(Q, K, V, O, dO, LSE, tau, causal=False, softcap=0.0, window=None, dropout=None):
    """dQ [B,H,N,d], dK, dV [B,H_kv,N,d], D [B,H,N] from the saved tensors.

    dK and dV of key/value head g sum the contributions of its G query heads
    ([CB] 8.5 accumulates the group before the final conversion).
    """
    Q, K, V, O, dO, LSE = map(_f64, (Q, K, V, O, dO, LSE))
    B, H, N, d = Q.shape
    G = _group(H, K.shape[1])
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    D = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            g = h // G
            dq, dk, dv, dd = backward_head(Q[b, h], K[b, g], V[b, g], O[b, h], dO[b, h], LSE[b, h],
                                           tau, causal, softcap, window, head_dropout(dropout, b * H + h))
            dQ[b, h] = dq
            dK[b, g] += dk
            dV[b, g] += dv
            D[b, h] = dd
    return dQ, dK, dV, D


def reference(Q, K, V, dO, tau, causal=False, softcap=0.0, window=None, dropout=None):
    """Forward then backward in fp64: dict with O, LSE, D, dQ, dK, dV.

    window = (wl, wr) adds the local mask (-1: that side unbounded);
    dropout = (p, seed, offset) applies the replayed dropout mask."""
    O, LSE = forward(Q, K, V, tau, causal, softcap, window, dropout)
    dQ, dK, dV, D = backward(Q, K, V, O, dO, LSE, tau, causal, softcap, window, dropout)
    return {"O": O, "LSE": LSE, "D": D, "dQ": dQ, "dK": dK, "dV": dV}
