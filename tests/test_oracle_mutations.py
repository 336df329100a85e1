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

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "attention.py")

MUTATIONS = {
    "drop_D_term": ("dZ = P * (dP - D[:, None])", "dZ = P * dP"),
    "flip_D_sign": ("dZ = P * (dP - D[:, None])", "dZ = P * (dP + D[:, None])"),
    "untransposed_P_in_dV": ("dV = P.T @ do", "dV = P @ do"),
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
}


def mutant(name):
    src = open(SRC_PATH).read()
    old, new = MUTATIONS[name]
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mod = types.ModuleType("oracle_mutant_" + name)
    exec(compile(src.replace(old, new), SRC_PATH + ":" + name, "exec"), mod.__dict__)
    return mod


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


PINS = (pin_finite_differences, pin_torch_sdpa, pin_softcap_identity, pin_window)


def test_unmutated_source_passes_every_pin():
    mod = types.ModuleType("oracle_copy")
    exec(compile(open(SRC_PATH).read(), SRC_PATH, "exec"), mod.__dict__)
    assert all(p(mod) for p in PINS)


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutant_is_caught(name):
    mod = mutant(name)
    caught = []
    for p in PINS:
        try:
            caught.append(not p(mod))
        except Exception:
            caught.append(True)
    assert any(caught), f"mutant {name} passed every pin"
