"""attn_bwd_with_dq_noalloc: the backward step with the library's static
scratch array instead of caller buffers.  Its results must equal those of
attn_bwd_preprocess + attn_bwd_with_dq on the same inputs, bit for bit
(bf16; fp32 with the fixed summation order) or within the fp32 tolerance
(fp32 atomics), on two calls in a row, the second with a smaller problem
(the array keeps the previous call's contents)."""
import pytest
import torch

import flashattention_backward_pass_amd as fab
from flashattention_backward_pass_amd import workloads

pytestmark = pytest.mark.gpu

SEQUENCES = [
    # two calls in a row: (B, H, H_kv, N, d, dtype, causal, deterministic)
    [(1, 8, 2, 700, 128, "bf16", True, False), (1, 4, 1, 300, 128, "bf16", True, False)],     # head split
    [(2, 8, 8, 1024, 64, "bf16", True, False), (1, 2, 2, 200, 64, "bf16", False, False)],      # combined launch
    [(1, 4, 2, 300, 128, "fp32", True, True), (1, 2, 1, 130, 64, "fp32", False, True)],       # fp32, fixed order
    [(1, 2, 2, 257, 64, "fp32", True, False), (1, 1, 1, 100, 64, "fp32", True, False)],       # fp32 atomics
    [(1, 2, 1, 3000, 128, "bf16", True, False), (1, 2, 2, 4096, 64, "bf16", True, False)],    # split units
]


def _inputs(case, seed):
    B, H, Hkv, N, d, dt, causal, det = case
    w = workloads.custom(B, H, Hkv, N, d, dt, causal, 0.0, seed=seed, name="noalloc")
    x = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v, do = (x[n].to(dev) for n in ("Q", "K", "V", "dO"))
    o, lse = fab.attention_forward(q, k, v, causal=causal)
    return w, q, k, v, do, o, lse


def _reference(w, q, k, v, do, o, lse, det):
    B, H, N, d = q.shape
    D = torch.empty(B, H, N, device=q.device)
    acc = torch.empty(B, H, N, d, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fab.attn_bwd_preprocess(o, do, D, acc, H_kv=w.H_kv, causal=w.causal, scale=w.tau)
    fab.attn_bwd_with_dq(q, k, v, do, lse, D, acc, dq, dk, dv, causal=w.causal, scale=w.tau, deterministic=det)
    return dq, dk, dv


@pytest.mark.parametrize("seq", SEQUENCES, ids=["bf16_split", "bf16_combined", "fp32_det", "fp32_atomic",
                                                 "bf16_split_units"])
def test_noalloc_matches_attn_bwd_with_dq(seq):
    for n, case in enumerate(seq):
        det = case[7]
        w, q, k, v, do, o, lse = _inputs(case, seed=100 + n)
        dq, dk, dv = torch.full_like(q, float("nan")), torch.full_like(k, float("nan")), torch.full_like(v, float("nan"))
        fab.attn_bwd_with_dq_noalloc(q, k, v, o, do, lse, dq, dk, dv, causal=w.causal, scale=w.tau,
                                     deterministic=det)
        ref = _reference(w, q, k, v, do, o, lse, det)
        torch.cuda.synchronize()
        print(f"[{case}] {fab.attn_bwd_kernels(q, k, causal=w.causal, deterministic=det)}", flush=True)
        for name, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
            if w.dtype == "fp32" and not det and name == "dQ":
                err = float((got - want).abs().max() / want.abs().max())
                assert err <= 1e-5, f"call {n}: dQ differs by {err:.2e}"
            else:
                bits = torch.int16 if w.dtype == "bf16" else torch.int32
                assert torch.equal(got.view(bits), want.view(bits)), f"call {n}: {name} differs"

