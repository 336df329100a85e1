"""Tensors past 2^31 elements: every kernel addresses with 64-bit offsets.

With B*H*N*d above 2^31 the rows of the last batch entries lie beyond any
32-bit element index (and, for the query heads, beyond 2^32 bytes).  Inputs
are drawn on the device from a seeded generator; the heads checked against
the fp64 oracle (first, middle and last batch entry) are copied back.  The
dropout generator's head word b*H + h runs past 2^14 here as well.
Tolerances as in the other parity tests.
"""
import numpy as np
import pytest
import torch

import flashattention_backward_pass_amd as fab
import oracle
from _parity import TOL, rel_err, to_np

pytestmark = pytest.mark.gpu

CASES = [
    # B, H, H_kv, N, d, dtype, causal, dropout
    (4100, 4, 2, 1040, 128, "bf16", True, (0.1, 0x0123_4567_89AB_CDEF, 3)),  # 2.18e9 elements, ragged N
    (44000, 4, 2, 96, 128, "fp32", False, None),                            # 2.16e9 elements, fp32 path
]


@pytest.mark.parametrize("case", CASES, ids=["bf16_b4100_n1040_dropout", "fp32_b44000_n96"])
def test_past_2_31_elements(case):
    B, H, Hkv, N, d, dt, causal, drop = case
    assert B * H * N * d > 2 ** 31
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    print(f"[large {dt}] B={B} H={H}/{Hkv} N={N} d={d}: {B * H * N * d / 2 ** 31:.3f} x 2^31 elements", flush=True)
    g = torch.Generator(device=dev).manual_seed(B + N)
    q = torch.randn(B, H, N, d, generator=g, device=dev, dtype=tdt)
    k = torch.randn(B, Hkv, N, d, generator=g, device=dev, dtype=tdt)
    v = torch.randn(B, Hkv, N, d, generator=g, device=dev, dtype=tdt)
    do = torch.randn(B, H, N, d, generator=g, device=dev, dtype=tdt)
    tau = d ** -0.5
    kw = dict(causal=causal, scale=tau, dropout=drop)
    o, lse = fab.attention_forward(q, k, v, **kw)
    dq, dk, dv = fab.attention_backward(q, k, v, o, do, lse, **kw)
    torch.cuda.synchronize()
    print(f"[large {dt}] kernels done", flush=True)
    G = H // Hkv
    for b in (0, B // 2, B - 1):
        for gk in range(Hkv):
            kb, vb = to_np(k[b, gk]), to_np(v[b, gk])
            dk_ref = dv_ref = 0.0
            for h in range(gk * G, (gk + 1) * G):
                qb, dob = to_np(q[b, h]), to_np(do[b, h])
                zf = oracle.head_dropout(drop, b * H + h)
                O, L = oracle.forward_head(qb, kb, vb, tau, causal, 0.0, None, zf)
                dq_r, dk_h, dv_h, _ = oracle.backward_head(qb, kb, vb, O, dob, L, tau, causal, 0.0, None, zf)
                dk_ref, dv_ref = dk_ref + dk_h, dv_ref + dv_h
                for n, got, ref in (("O", o, O), ("LSE", lse, L), ("dQ", dq, dq_r)):
                    e = rel_err(to_np(got[b, h]), ref)
                    assert e <= TOL[dt], f"batch {b} head {h} {n}: {e:.3e}"
            for n, got, ref in (("dK", dk, dk_ref), ("dV", dv, dv_ref)):
                e = rel_err(to_np(got[b, gk]), ref)
                assert e <= TOL[dt], f"batch {b} kv head {gk} {n}: {e:.3e}"
        print(f"[large {dt}] batch {b} matches the oracle", flush=True)
