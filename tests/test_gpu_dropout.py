"""Dropout replay through the C ABI against the fp64 oracle.

The oracle regenerates the mask from the same generator state with its own
Philox4x32-10 (oracle/philox.py); the kernels regenerate it on the device
(csrc/philox.h).  Values: max|GPU - oracle| / max|oracle| <= 1e-4 (fp32) and
<= 2e-2 (bf16) per output tensor.  Mask bits: exact, read off outputs whose
nonzero pattern is the mask (Q = 0, V and dO one-hot rows).
"""
import numpy as np
import pytest
import torch

import flashattention_backward_pass_amd as fab
import oracle
from flashattention_backward_pass_amd import workloads
from _parity import TOL, oracle_full, rel_err, run_gpu, to_np

pytestmark = pytest.mark.gpu

SEED = 0x0123_4567_89AB_CDEF

CASES = [
    # B, H, H_kv, N, d, dtype, causal, softcap, window, p
    (1, 2, 2, 128, 64, "fp32", False, 0.0, (-1, -1), 0.1),
    (2, 2, 1, 150, 128, "fp32", True, 5.0, (-1, -1), 0.3),
    (1, 2, 2, 100, 64, "fp32", False, 0.0, (20, 9), 0.5),
    (1, 4, 2, 300, 128, "bf16", True, 0.0, (-1, -1), 0.1),
    (2, 2, 2, 257, 64, "bf16", False, 0.0, (-1, -1), 0.5),
    (1, 2, 2, 384, 128, "bf16", False, 20.0, (-1, -1), 0.2),
    (1, 8, 2, 512, 128, "bf16", True, 0.0, (-1, -1), 0.15),  # grouped heads (head split)
    (1, 2, 1, 333, 64, "bf16", True, 0.0, (50, -1), 0.25),    # causal window, ragged
    (1, 2, 2, 256, 128, "bf16", False, 0.0, (-1, -1), 0.9),
    (1, 1, 1, 1, 128, "bf16", True, 0.0, (-1, -1), 0.5),      # one key
    (1, 4, 1, 5, 64, "bf16", False, 3.0, (2, 1), 0.3),        # tiny: every mask and the cap
    (2, 8, 2, 200, 64, "bf16", True, 10.0, (60, -1), 0.2),    # GQA d=64, cap, window
    (1, 2, 2, 64, 64, "fp32", True, 0.0, (-1, -1), 0.999),    # almost everything dropped
]


def _id(c):
    return (f"b{c[0]}h{c[1]}x{c[2]}N{c[3]}d{c[4]}{c[5]}{'c' if c[6] else ''}{'s' if c[7] else ''}"
            f"{'w%d_%d' % c[8] if c[8] != (-1, -1) else ''}p{c[9]}")


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_dropout_matches_oracle(case):
    B, H, Hkv, N, d, dt, causal, cap, win, p = case
    w = workloads.custom(B, H, Hkv, N, d, dt, causal, cap, seed=N + d + int(100 * p), name=_id(case), window=win,
                         dropout=(p, SEED + N, N % 7))
    x = workloads.make_inputs(w)
    got = run_gpu(w, x)
    ref = oracle_full(w, x)
    for n in ("O", "LSE", "D", "dQ", "dK", "dV"):
        e = rel_err(to_np(got[n]), ref[n])
        print(f"[{w.name}] {n}={e:.2e}", flush=True)
        assert e <= TOL[dt], f"{n}: {e:.3e}"


def _keep(p, seed, offset, B, H, N):
    """Oracle keep bits [B, H, N, N]."""
    return np.stack([np.stack([oracle.philox.dropout_multiplier(p, seed, offset, b * H + h, np.arange(N),
                                                                 np.arange(N)) > 0 for h in range(H)])
                     for b in range(B)])


@pytest.mark.parametrize("dt", ["fp32", "bf16"])
@pytest.mark.parametrize("N,causal", [(64, False), (128, False), (128, True)])
def test_mask_bits_exact(dt, N, causal):
    """Q = 0 makes P uniform over the visible keys; with V = I the forward's
    O_ij is Z_ij / n_i, and with dO = I the backward's dV_kj is P_jk Z_jk, so
    the nonzero patterns of O and dV are the mask and its transpose."""
    B, H, d = 2, 3, N
    p, seed, off = 0.3, SEED ^ N, 11
    dev = torch.device("cuda:0")
    tdt = torch.float32 if dt == "fp32" else torch.bfloat16
    g = torch.Generator().manual_seed(N)
    q = torch.zeros(B, H, N, d, dtype=tdt, device=dev)
    k = torch.randn(B, H, N, d, generator=g).to(tdt).to(dev)
    eye = torch.eye(N, dtype=tdt).expand(B, H, N, N).contiguous().to(dev)
    drop = (p, seed, off)
    o, lse = fab.attention_forward(q, k, eye, causal=causal, scale=0.125, dropout=drop)
    dq, dk, dv = fab.attention_backward(q, k, eye, o, eye, lse, causal=causal, scale=0.125, dropout=drop)
    torch.cuda.synchronize()
    keep = _keep(p, seed, off, B, H, N)
    vis = np.tril(np.ones((N, N), dtype=bool)) if causal else np.ones((N, N), dtype=bool)
    want = keep & vis
    np.testing.assert_array_equal(to_np(o) > 0, want)
    np.testing.assert_array_equal(to_np(dv) > 0, np.swapaxes(want, -1, -2))


def test_p0_is_bitwise_no_dropout():
    w0 = workloads.custom(1, 2, 2, 200, 128, "bf16", True, 0.0, seed=9, name="nodrop")
    w1 = workloads.custom(1, 2, 2, 200, 128, "bf16", True, 0.0, seed=9, name="p0", dropout=(0.0, 5, 6))
    x = workloads.make_inputs(w0)
    a, b = run_gpu(w0, x), run_gpu(w1, x)
    for n in ("O", "LSE", "D", "dQaccum", "dK", "dV"):
        assert torch.equal(a[n], b[n]), n


@pytest.mark.parametrize("dt", ["fp32", "bf16"])
def test_dropout_reproducible_and_seeded(dt):
    """The same state gives bitwise the same outputs; another offset another mask."""
    w = workloads.custom(1, 2, 1, 192, 64, dt, True, 0.0, seed=4, name="rep", dropout=(0.2, 77, 0))
    x = workloads.make_inputs(w)
    a = run_gpu(w, x, deterministic=True)
    b = run_gpu(w, x, deterministic=True)
    for n in ("O", "LSE", "D", "dQaccum", "dK", "dV"):
        assert torch.equal(a[n], b[n]), n
    w2 = workloads.custom(1, 2, 1, 192, 64, dt, True, 0.0, seed=4, name="rep2", dropout=(0.2, 77, 1))
    c = run_gpu(w2, x, deterministic=True)
    assert not torch.equal(a["O"], c["O"])


def test_long_sequence_sampled_rows():
    """N = 16384 causal, p = 0.1: O, LSE, D and dQ of sampled query rows of
    two heads, each computed row by row by the oracle."""
    w = workloads.WORKLOADS["bf16_dropout0.1_causal_b1h8_n16384_d128"]
    x = workloads.make_inputs(w)
    got = run_gpu(w, x)
    rows = np.array([0, 1, 127, 128, 4095, 8191, 8192, 12000, 16381, 16383])
    for h in (0, w.H - 1):
        q, k, v, do = x["Q"][0, h], x["K"][0, h // w.group], x["V"][0, h // w.group], x["dO"][0, h]
        zf = oracle.head_dropout(w.dropout, h)
        o_r, lse_r = oracle.forward_rows_head(q, k, v, rows, w.tau, w.causal, w.softcap, w.window, zf)
        dq_r, d_r = oracle.backward_q_rows_head(q, k, v, o_r, do[rows], lse_r, rows, w.tau, w.causal, w.softcap,
                                                w.window, zf)
        for n, ref in (("O", o_r), ("LSE", lse_r), ("D", d_r), ("dQ", dq_r)):
            e = rel_err(to_np(got[n][0, h])[rows], ref)
            print(f"[{w.name}] head {h} {n}={e:.2e}", flush=True)
            assert e <= TOL[w.dtype], n
