"""Deterministic mode (attn_params.deterministic = 1) through the C ABI.

fp32: dK/dV without atomics plus a query-block-outer dQ kernel; checked
against the fp64 oracle (max|GPU - oracle| / max|oracle| <= 1e-4) and for
bitwise run-to-run equality.  bf16: the flag selects the same atomic-free
kernels, so the outputs must be bitwise equal to those of deterministic = 0.
"""
import pytest
import torch

from flashattention_backward_pass_amd import workloads
from _parity import TOL, oracle_full, rel_err, run_gpu, to_np

pytestmark = pytest.mark.gpu

FP32_CASES = [
    # B, H, H_kv, N, d, causal, softcap, sigma_qk
    (1, 2, 2, 257, 64, True, 0.0, 1.0),     # ragged, causal
    (1, 4, 2, 100, 128, True, 10.0, 1.5),   # ragged, causal, softcap, GQA
    (2, 2, 1, 96, 128, False, 0.0, 1.0),    # GQA, full tiles
]


def _ids(c):
    return f"B{c[0]}H{c[1]}x{c[2]}N{c[3]}d{c[4]}{'c' if c[5] else ''}{'s' if c[6] else ''}"


@pytest.mark.parametrize("case", FP32_CASES, ids=[_ids(c) for c in FP32_CASES])
def test_fp32_deterministic_matches_oracle(case):
    B, H, Hkv, N, d, causal, cap, s = case
    w = workloads.custom(B, H, Hkv, N, d, "fp32", causal, cap, sigma_qk=s, seed=7 * N + d, name=f"det{case}")
    x = workloads.make_inputs(w)
    got = run_gpu(w, x, deterministic=True)
    ref = oracle_full(w, x)
    for n in ("dQ", "dK", "dV"):
        e = rel_err(to_np(got[n]), ref[n])
        print(f"[{w.name}] {n}={e:.2e}", flush=True)
        assert e <= TOL["fp32"], f"{n}: {e:.3e}"


def test_fp32_workload_deterministic_bitwise_repeatable():
    w = workloads.WORKLOADS[workloads.WORKLOAD_ORDER[0]]
    x = workloads.make_inputs(w)
    a = run_gpu(w, x, deterministic=True)
    b = run_gpu(w, x, o=a["O"].cpu(), lse=a["LSE"].cpu(), deterministic=True)
    for n in ("dQaccum", "dK", "dV"):
        assert torch.equal(a[n], b[n]), n
    ref = oracle_full(w, x)
    for n in ("dQ", "dK", "dV"):
        assert rel_err(to_np(a[n]), ref[n]) <= TOL["fp32"], n


def test_fp32_deterministic_close_to_atomic():
    w = workloads.custom(1, 2, 2, 300, 128, "fp32", True, 0.0, seed=99, name="det-vs-atomic")
    x = workloads.make_inputs(w)
    a = run_gpu(w, x, deterministic=True)
    b = run_gpu(w, x, o=a["O"].cpu(), lse=a["LSE"].cpu(), deterministic=False)
    for n in ("dK", "dV"):
        assert torch.equal(a[n], b[n]), n  # the same kernel, same order
    e = rel_err(to_np(a["dQaccum"]), to_np(b["dQaccum"]))
    print(f"[det-vs-atomic] dQaccum {e:.2e}", flush=True)
    assert e <= 1e-5


@pytest.mark.parametrize("name", [workloads.WORKLOAD_ORDER[1], workloads.WORKLOAD_ORDER[2]])
def test_bf16_flag_is_bitwise_neutral(name):
    w = workloads.WORKLOADS[name]
    x = workloads.make_inputs(w)
    a = run_gpu(w, x, deterministic=False)
    b = run_gpu(w, x, o=a["O"].cpu(), lse=a["LSE"].cpu(), deterministic=True)
    for n in ("dQaccum", "dK", "dV"):
        assert torch.equal(a[n], b[n]), n
