"""The oracle's pins have teeth: plant plausible mistakes in a copy of the
oracle (on the CPU, in memory) and check that the pins reject every mutant.

Each mutant is the oracle source with one textual change (a dropped term, a
flipped sign, a transposed operand, a wrong index, a missing scale), executed
as a throw-away module.  The real oracle module is never modified.
"""
import math
import os
import types

import numpy as np
import pytest
import torch

from tests._philox_ref import torch_philox_first_block

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")
SRC_PATH = os.path.join(ORACLE_DIR, "attention.py")
PHILOX_PATH = os.path.join(ORACLE_DIR, "philox.py")

MUTATIONS = {
    "drop_D_term": ("dZ = P * (dP - D[:, None])", "dZ = P * dP"),
    "flip_D_sign": ("dZ = P * (dP - D[:, None])", "dZ = P * (dP + D[:, None])"),
    "untransposed_P_in_dV": ("else P.T @ do\n    dP = do", "else P @ do\n    dP = do"),
    "missing_tau_on_dR": ("        dR = tau * dZ\n", "        dR = dZ\n"),
    "softcap_derivative_sign": ("dR = tau * dZ * (1.0 - T * T)", "dR = tau * dZ * (1.0 + T * T)"),
    "mask_direction": ("ok &= j <= i\n", "ok &= j >= i\n"),
    "mask_drops_diagonal": ("ok &= j <= i\n", "ok &= j < i\n"),
    "window_left_off_by_one": ("ok &= j >= i - wl", "ok &= j > i - wl"),
    "window_right_mirrored": ("ok &= j <= i + wr", "ok &= j <= i - wr"),
    "lse_without_max": ("lse = m + np.log(", "lse = np.log("),
    "gqa_head_map": ("            g = h // G\n", "            g = h % K.shape[1]\n"),
    "dK_against_K": ("dK = dR.T @ q", "dK = dR.T @ k"),
    "dQ_against_Q": ("dQ = dR @ k", "dQ = dR @ q"),
    "D_from_dP": ("D = (do * o).sum(axis=1)\n    dZ", "D = dP.sum(axis=1)\n    dZ"),
    "cap_without_c": ("Z = tau * (softcap * T)", "Z = tau * T"),
    # dropout terms of the attention oracle
    "dropout_missing_in_dP": ("    if Zd is not None:\n        dP = dP * Zd\n", ""),
    "dropout_missing_in_dV": ("dV = (P * Zd).T @ do if Zd is not None else P.T @ do", "dV = P.T @ do"),
    "dropout_missing_in_O": ("P = P * zdrop(rows, np.arange(k.shape[0]))", "P = P"),
    "dropped_P_in_dS": ("dZ = P * (dP - D[:, None])\n    del P, dP",
                        "dZ = (P if Zd is None else P * Zd) * (dP - D[:, None])\n    del P, dP"),
    "dropout_kv_head_index": ("softcap, window, head_dropout(dropout, b * H + h))",
                              "softcap, window, head_dropout(dropout, b * H + g))"),
}

# Mistakes planted in the generator and the mask built from it (oracle/philox.py).
PHILOX_MUTATIONS = {
    "philox_word_mix": ("hi1 ^ x1 ^ k0", "hi1 ^ x3 ^ k0"),
    "philox_key_schedule": ("k0 = (k0 + w0) & mask", "k0 = (k0 + w1) & mask"),
    "philox_rounds": ("def philox4x32(counter, key, rounds=10)", "def philox4x32(counter, key, rounds=7)"),
    "philox_multiplier_swap": ("p0 = m0 * x0\n        p1 = m1 * x2", "p0 = m1 * x0\n        p1 = m0 * x2"),
    "mask_word_index": ("(q_idx & 3)[:, None]", "(q_idx & 1)[:, None]"),
    "mask_half": ("16 * (k_idx & 1)", "16 * (1 - (k_idx & 1))"),
    "mask_counter_order": ("ctr[..., 0] = kb[None, :]\n    ctr[..., 1] = qb[:, None]",
                           "ctr[..., 0] = qb[:, None]\n    ctr[..., 1] = kb[None, :]"),
    "keep_inclusive": ("u < np.uint64(t)", "u <= np.uint64(t)"),
    "scale_missing": ("1.0 / (1.0 - p), 0.0)", "1.0, 0.0)"),
    "threshold_truncates": ("(1.0 - p) * 65536.0 + 0.5", "(1.0 - p) * 65536.0"),
}


def _load(att_src, philox_src, tag):
    """Executes the two oracle sources as throw-away modules; the attention
    module gets the (possibly mutated) generator module as its `philox`."""
    ph = types.ModuleType("oracle_philox_" + tag)
    exec(compile(philox_src, PHILOX_PATH + ":" + tag, "exec"), ph.__dict__)
    mod = types.ModuleType("oracle_attention_" + tag)
    mod.__dict__["philox"] = ph
    assert att_src.count("from . import philox\n") == 1
    exec(compile(att_src.replace("from . import philox\n", ""), SRC_PATH + ":" + tag, "exec"), mod.__dict__)
    return mod


def mutant(name):
    att, ph = open(SRC_PATH).read(), open(PHILOX_PATH).read()
    if name in MUTATIONS:
        old, new = MUTATIONS[name]
        assert att.count(old) >= 1, f"mutation anchor for {name} not found"
        att = att.replace(old, new)
    else:
        old, new = PHILOX_MUTATIONS[name]
        assert ph.count(old) >= 1, f"mutation anchor for {name} not found"
        ph = ph.replace(old, new)
    return _load(att, ph, name)


def rnd(rng, *shape, s=1.0):
    return rng.standard_normal(shape) * s


def pin_finite_differences(mod):
    """Central differences of <dO, O> through mod.forward vs mod.backward."""
    for causal, softcap, (B, H, Hkv, N, d) in [(True, 1.3, (1, 4, 2, 4, 3)), (False, 0.0, (1, 2, 1, 5, 3))]:
        rng = np.random.default_rng(3)
        Q, K = rnd(rng, B, H, N, d, s=1.5), rnd(rng, B, Hkv, N, d, s=1.5)
        V, dO = rnd(rng, B, Hkv, N, d), rnd(rng, B, H, N, d)
        O, L = mod.forward(Q, K, V, 0.6, causal, softcap)
        grads = mod.backward(Q, K, V, O, dO, L, 0.6, causal, softcap)[:3]
        for X, G in zip((Q, K, V), grads):
            for idx in np.ndindex(X.shape):
                old = X[idx]
                X[idx] = old + 1e-6
                lp = float((dO * mod.forward(Q, K, V, 0.6, causal, softcap)[0]).sum())
                X[idx] = old - 1e-6
                lm = float((dO * mod.forward(Q, K, V, 0.6, causal, softcap)[0]).sum())
                X[idx] = old
                if abs((lp - lm) / 2e-6 - G[idx]) > 1e-6 * max(1.0, np.abs(G).max()):
                    return False
    return True


def pin_torch_sdpa(mod):
    """fp64 autograd of torch's scaled_dot_product_attention (causal GQA)."""
    B, H, Hkv, N, d = 1, 4, 2, 9, 8
    g = torch.Generator().manual_seed(1)
    Q, K, V, dO = (torch.randn(B, h, N, d, generator=g, dtype=torch.float64) for h in (H, Hkv, Hkv, H))
    tau = 1 / math.sqrt(d)
    q, k, v = (t.clone().requires_grad_(True) for t in (Q, K, V))
    out = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=tau, enable_gqa=True)
    out.backward(dO)
    r = mod.reference(Q, K, V, dO, tau, True)
    ok = np.allclose(r["O"], out.detach().numpy(), atol=1e-10)
    for n, t in (("dQ", q), ("dK", k), ("dV", v)):
        ok = ok and np.allclose(r[n], t.grad.numpy(), atol=1e-10)
    return bool(ok)


def pin_softcap_identity(mod):
    """With a cap: sum_h <Q_h, dQ_h> = <K_g, dK_g>, and the cap c=1e12 matches no cap."""
    rng = np.random.default_rng(4)
    Q, K, V, dO = rnd(rng, 1, 2, 7, 4, s=2.0), rnd(rng, 1, 1, 7, 4, s=2.0), rnd(rng, 1, 1, 7, 4), rnd(rng, 1, 2, 7, 4)
    r = mod.reference(Q, K, V, dO, 0.5, True, 1.1)
    ok = abs((Q * r["dQ"]).sum() - (K * r["dK"]).sum()) < 1e-10
    a = mod.reference(Q, K, V, dO, 0.5, True, 1e12)
    b = mod.reference(Q, K, V, dO, 0.5, True, 0.0)
    return bool(ok and all(np.allclose(a[n], b[n], atol=1e-8) for n in ("O", "dQ", "dK", "dV")))


def pin_window(mod):
    """Local window: fp64 autograd of torch's scaled_dot_product_attention with
    the band written out as a boolean mask, and window (0, 0) in closed form
    (each query sees only its own key: O = V, dQ = dK = 0, dV = dO)."""
    B, H, N, d = 1, 2, 11, 4
    g = torch.Generator().manual_seed(2)
    Q, K, V, dO = (torch.randn(B, H, N, d, generator=g, dtype=torch.float64) for _ in range(4))
    i = torch.arange(N)[:, None]
    j = torch.arange(N)[None, :]
    ok = True
    for causal, (wl, wr) in ((False, (3, 2)), (True, (4, -1)), (False, (-1, 1))):
        band = torch.ones(N, N, dtype=torch.bool)
        if causal:
            band &= j <= i
        if wl >= 0:
            band &= j >= i - wl
        if wr >= 0:
            band &= j <= i + wr
        q, k, v = (t.clone().requires_grad_(True) for t in (Q, K, V))
        out = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=band, scale=0.7)
        out.backward(dO)
        r = mod.reference(Q, K, V, dO, 0.7, causal, 0.0, (wl, wr))
        ok = ok and np.allclose(r["O"], out.detach().numpy(), atol=1e-10)
        for n, t in (("dQ", q), ("dK", k), ("dV", v)):
            ok = ok and np.allclose(r[n], t.grad.numpy(), atol=1e-10)
    r = mod.reference(Q, K, V, dO, 0.7, False, 0.0, (0, 0))
    ok = ok and np.allclose(r["O"], V.numpy(), atol=1e-12) and np.allclose(r["dV"], dO.numpy(), atol=1e-12)
    ok = ok and np.abs(r["dQ"]).max() < 1e-12 and np.abs(r["dK"]).max() < 1e-12
    return bool(ok)


def pin_dropout_generator(mod):
    """Mask bits against PyTorch's independent Philox4x32-10 engine, composed
    with the stated counter mapping; the keep rule u < t with t = round-half-up
    ((1 - p) 65536) at a p where the rounding matters; E[Z] = 1."""
    from fractions import Fraction

    ph = mod.philox
    seed, offset, bh = 0xFEEDFACE12345, 6, 3
    q, k = np.arange(12), np.arange(10)
    trip = [(seed, bh | (offset << 32), (kk >> 1) | ((qq >> 2) << 32)) for qq in q for kk in k]
    words = torch_philox_first_block(trip).reshape(12, 10, 4)
    u = np.array([[(int(words[qq, kk, qq & 3]) >> (16 * (kk & 1))) & 0xFFFF for kk in k] for qq in q])
    ok = np.array_equal(ph.dropout_bits(seed, offset, bh, q, k).astype(np.int64), u)
    # a p whose threshold rounds up, and one whose threshold is a value that occurs
    u0 = int(np.sort(u.ravel())[u.size // 2])  # a value that occurs
    for p in (float(np.float32(1.0 / 3.0)), 1.0 - u0 / 65536.0):
        t = int((1 - Fraction(p)) * 65536 + Fraction(1, 2))
        z = ph.dropout_multiplier(p, seed, offset, bh, q, k)
        ok = ok and ph.keep_threshold(p) == t and np.array_equal(z > 0, u < t)
        ok = ok and np.allclose(z[z > 0], 1.0 / (1.0 - p), rtol=1e-15)
    zz = ph.dropout_multiplier(0.5, 1, 0, 0, np.arange(256), np.arange(256))
    return bool(ok and abs(zz.mean() - 1.0) < 0.03)


def pin_dropout_autograd(mod):
    """fp64 autograd of O = (softmax(Z) o M) V, M from the module's own mask
    (causal GQA with a cap, and a local window)."""
    ok = True
    for causal, softcap, window, (B, H, Hkv, N, d) in ((True, 1.4, (-1, -1), (1, 4, 2, 9, 3)),
                                                         (False, 0.0, (3, 1), (1, 2, 1, 10, 4))):
        g = torch.Generator().manual_seed(N)
        Q, K = (torch.randn(B, h, N, d, generator=g, dtype=torch.float64) * 1.3 for h in (H, Hkv))
        V, dO = (torch.randn(B, h, N, d, generator=g, dtype=torch.float64) for h in (Hkv, H))
        drop = (0.4, 77, 1)
        q, k, v = (t.clone().requires_grad_(True) for t in (Q, K, V))
        G = H // Hkv
        kk, vv = k.repeat_interleave(G, dim=1), v.repeat_interleave(G, dim=1)
        R = q @ kk.transpose(-1, -2)
        Z = 0.6 * (softcap * torch.tanh(R / softcap) if softcap > 0 else R)
        i, j = torch.arange(N)[:, None], torch.arange(N)[None, :]
        vis = torch.ones(N, N, dtype=torch.bool)
        if causal:
            vis &= j <= i
        if window[0] >= 0:
            vis &= j >= i - window[0]
        if window[1] >= 0:
            vis &= j <= i + window[1]
        P = torch.softmax(Z.masked_fill(~vis, -math.inf), dim=-1)
        M = torch.tensor(np.stack([np.stack([mod.philox.dropout_multiplier(*drop, b * H + h, np.arange(N), np.arange(N))
                                             for h in range(H)]) for b in range(B)]))
        O = (P * M) @ vv
        O.backward(dO)
        r = mod.reference(Q, K, V, dO, 0.6, causal, softcap, window, drop)
        ok = ok and np.allclose(r["O"], O.detach().numpy(), atol=1e-11)
        for n, t in (("dQ", q), ("dK", k), ("dV", v)):
            ok = ok and np.allclose(r[n], t.grad.numpy(), atol=1e-11)
    return bool(ok)


PINS = (pin_finite_differences, pin_torch_sdpa, pin_softcap_identity, pin_window, pin_dropout_generator,
        pin_dropout_autograd)


def test_unmutated_source_passes_every_pin():
    mod = _load(open(SRC_PATH).read(), open(PHILOX_PATH).read(), "copy")
    assert all(p(mod) for p in PINS)


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("name", sorted(MUTATIONS) + sorted(PHILOX_MUTATIONS))
def test_mutant_is_caught(name):
    mod = mutant(name)
    caught = []
    for p in PINS:
        try:
            caught.append(not p(mod))
        except Exception:
            caught.append(True)
    assert any(caught), f"mutant {name} passed every pin"
