"""attn_bwd_with_dq: dQ written by the backward itself.

bf16: the dQ work units round their sums to dQ directly, so the result must
be the same bits as attn_bwd followed by attn_bwd_dq_convert (the bf16 path
is reproducible), for each dispatch: the combined launch of small grids, the
two kernels one after the other, the grouped-head split (which keeps partial
sums in dQaccum), with soft cap, window and dropout.  fp32: attn_bwd then the
convert kernel inside the call, so dQ = fp32(scale * dQaccum) of the same
call, bit for bit (the atomic path's sums vary from run to run).  The dQ of
every case is also held to the oracle at the parity tolerance.

Where the combined launch splits its heaviest units in two (attn_bwd_kernels
returns "bwd_fused_kernel:split": dK/dV units of the first key blocks by query
range, dQ units of the last query blocks by key range), those rows add two
fp32 halves before rounding, a different fp32 summation order from attn_bwd's
single sum: dQ, dK and dV are held to the oracle at the parity tolerance, to
attn_bwd's within one bf16 step of the tensor's largest magnitude (a column
sum of dS can cancel, so the two fp32 sums need not round to neighbouring bf16
values elementwise), and to their own bits on a second call.
"""
import pytest
import torch

import flashattention_backward_pass_amd as fab
from flashattention_backward_pass_amd import workloads
from _parity import TOL, oracle_full, rel_err, run_gpu, to_np

pytestmark = pytest.mark.gpu

CASES = [
    # B, H, H_kv, N, d, dtype, causal, softcap, window, dropout, deterministic
    (1, 4, 4, 700, 128, "bf16", True, 0.0, (-1, -1), None, False),             # combined launch, ragged
    (4, 16, 16, 2200, 64, "bf16", True, 0.0, (-1, -1), None, False),           # two kernels (> 2048 workgroups at d = 64)
    (2, 16, 16, 2100, 128, "bf16", True, 0.0, (-1, -1), None, False),          # two kernels, d = 128, ragged
    (1, 20, 4, 700, 128, "bf16", True, 0.0, (-1, -1), None, False),            # head split, G = 5
    (1, 8, 2, 900, 128, "bf16", True, 0.0, (-1, -1), (0.2, 99, 4), False),     # head split, dropout
    (2, 4, 2, 333, 128, "bf16", False, 15.0, (40, 20), None, False),          # soft cap, window
    (1, 2, 2, 200, 64, "fp32", True, 0.0, (-1, -1), None, True),              # fp32, fixed order
    (1, 2, 1, 257, 128, "fp32", False, 5.0, (-1, -1), None, False),            # fp32, atomics
    (1, 2, 1, 3000, 128, "bf16", True, 0.0, (-1, -1), None, False),           # split dK/dV units, G = 2, ragged
    (1, 2, 2, 4096, 64, "bf16", True, 0.0, (-1, -1), None, False),            # split dK/dV and dQ units
    (1, 3, 3, 5000, 128, "bf16", True, 20.0, (-1, -1), (0.15, 5, 3), False),  # both, soft cap, dropout, ragged
]
IDS = ["bf16_combined", "bf16_two_kernels", "bf16_two_kernels_d128", "bf16_split_g5", "bf16_split_dropout",
       "bf16_softcap_window", "fp32_det", "fp32_atomic", "bf16_split_units_kv_gqa2", "bf16_split_units_d64",
       "bf16_split_units_cap_dropout"]
SPLIT_UNITS = {"bf16_split_units_kv_gqa2", "bf16_split_units_d64", "bf16_split_units_cap_dropout"}



@pytest.mark.parametrize("case,cid", list(zip(CASES, IDS)), ids=IDS)
def test_with_dq_matches_two_step(case, cid):
    B, H, Hkv, N, d, dt, causal, cap, win, drop, det = case
    w = workloads.custom(B, H, Hkv, N, d, dt, causal, cap, seed=N + H + d, name="with_dq", window=win,
                         dropout=drop)
    x = workloads.make_inputs(w)
    ref = run_gpu(w, x, deterministic=det)
    dev = torch.device("cuda:0")
    q, k, v, do = (x[n].to(dev) for n in ("Q", "K", "V", "dO"))
    o, lse = ref["O"], ref["LSE"]
    kw = dict(causal=causal, scale=w.tau, softcap=cap, window=win)
    D = torch.empty(B, H, N, device=dev, dtype=torch.float32)
    acc = torch.full((B, H, N, d), float("nan"), device=dev, dtype=torch.float32)
    dq = torch.full_like(q, float("nan"))
    dk, dv = torch.full_like(k, float("nan")), torch.full_like(v, float("nan"))
    plan = fab.attn_bwd_kernels(q, k, deterministic=det, dropout=drop, **kw)
    split = plan.endswith(":split")
    print(f"[{cid}] {plan}", flush=True)
    assert split == (cid in SPLIT_UNITS), plan
    fab.attn_bwd_preprocess(o, do, D, acc, H_kv=Hkv, **kw)
    fab.attn_bwd_with_dq(q, k, v, do, lse, D, acc, dq, dk, dv, deterministic=det, dropout=drop, **kw)
    torch.cuda.synchronize()
    bits = torch.int16 if dt == "bf16" else torch.int32
    if split:
        for n, got in (("dQ", dq), ("dK", dk), ("dV", dv)):
            e = rel_err(to_np(got), oracle_full(w, x)[n])
            e1 = rel_err(to_np(ref[n]), oracle_full(w, x)[n])
            diff = (got.float() - ref[n].float()).abs()
            top = ref[n].float().abs().max()
            step = torch.exp2(torch.floor(torch.log2(torch.maximum(got.float().abs(), ref[n].float().abs())
                                                      .clamp_min(1e-38))) - 7)
            print(f"[{cid}] {n} vs oracle {e:.2e} (attn_bwd {e1:.2e}); max |split - attn_bwd| / max|attn_bwd| "
                  f"{float(diff.max() / top):.2e}; {int((diff > step).sum())} of {diff.numel()} elements "
                  f"beyond one step of their own magnitude", flush=True)
            assert e <= TOL[dt], n
            assert float(diff.max()) <= float(top) * 2.0 ** -8, n
        again = [torch.full_like(t, float("nan")) for t in (dq, dk, dv)]
        fab.attn_bwd_with_dq(q, k, v, do, lse, D, acc, *again, deterministic=det, dropout=drop, **kw)
        torch.cuda.synchronize()
        for n, a, b in zip(("dQ", "dK", "dV"), again, (dq, dk, dv)):
            assert torch.equal(a.view(bits), b.view(bits)), f"{n} differs between two calls"
    elif dt == "bf16" or det:
        for n, got in (("dQ", dq), ("dK", dk), ("dV", dv)):
            assert torch.equal(got.view(bits), ref[n].view(bits)), n
    else:
        assert torch.equal(dq, acc * torch.tensor(w.tau, dtype=torch.float32, device=dev))
        for n, got in (("dK", dk), ("dV", dv)):
            assert torch.equal(got.view(bits), ref[n].view(bits)), n
    e = rel_err(to_np(dq), oracle_full(w, x)["dQ"])
    print(f"[{w.name} {dt}] dQ vs oracle {e:.2e}", flush=True)
    assert e <= TOL[dt]


def test_attention_backward_uses_one_bwd_call():
    """attention_backward (preprocess + attn_bwd_with_dq) against the oracle."""
    w = workloads.custom(2, 4, 2, 300, 128, "bf16", True, 0.0, seed=21, name="wrapper")
    x = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v, do = (x[n].to(dev) for n in ("Q", "K", "V", "dO"))
    o, lse = fab.attention_forward(q, k, v, causal=True)
    dq, dk, dv = fab.attention_backward(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    ref = oracle_full(w, x)
    for n, got in (("dQ", dq), ("dK", dk), ("dV", dv)):
        assert rel_err(to_np(got), ref[n]) <= TOL["bf16"], n
