"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerance (per output tensor, over the whole tensor): max|GPU - oracle| /
max|oracle| <= 1e-4 for fp32 inputs and <= 2e-2 for bf16 inputs.
"""
import numpy as np
import pytest
import torch

import flashattention_backward_pass_amd as fab
from flashattention_backward_pass_amd import workloads
import oracle
from _parity import TOL, oracle_full, oracle_kv_heads, rel_err, run_gpu, to_np

pytestmark = pytest.mark.gpu

SMALL = [
    # B, H, H_kv, N, d, dtype, causal, softcap, sigma_qk
    (1, 1, 1, 1, 128, "bf16", True, 0.0, 1.0),      # one key: dQ = dK = 0, dV = dO
    (1, 2, 1, 77, 64, "bf16", True, 0.0, 1.0),      # ragged, GQA
    (2, 3, 3, 200, 128, "bf16", False, 20.0, 1.5),  # ragged, softcap
    (1, 4, 2, 333, 128, "bf16", True, 15.0, 1.5),   # ragged, causal, softcap, GQA
    (1, 2, 2, 384, 64, "bf16", False, 0.0, 1.0),    # several full tiles
    (1, 8, 2, 256, 128, "bf16", True, 0.0, 1.0),    # GQA groups of 4
    # Grouped heads split over two workgroups per key block (G >= 4, few
    # units): odd groups give the two workgroups 2 + 3 and 3 + 4 heads.
    (1, 20, 4, 700, 128, "bf16", True, 0.0, 1.0),   # G = 5
    (1, 28, 4, 700, 128, "bf16", True, 0.0, 1.0),   # G = 7
    (2, 18, 2, 300, 64, "bf16", False, 10.0, 1.5),  # G = 9, soft cap, d = 64
    (1, 12, 4, 500, 128, "bf16", True, 0.0, 1.0),   # G = 3: no split
    (1, 2, 2, 257, 64, "fp32", True, 0.0, 1.0),
    (1, 2, 1, 130, 128, "fp32", False, 5.0, 1.5),
]


def _check(w, got, ref, names=("O", "LSE", "dQ", "dK", "dV"), tol=None):
    tol = tol if tol is not None else TOL[w.dtype]
    errs = {n: rel_err(to_np(got[n]), ref[n]) for n in names}
    print(f"[{w.name}] " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)
    for n, e in errs.items():
        assert e <= tol, f"{n}: {e:.3e} > {tol}"
    return errs


@pytest.mark.parametrize("case", SMALL, ids=[f"B{c[0]}H{c[1]}x{c[2]}N{c[3]}d{c[4]}{c[5]}{'c' if c[6] else ''}"
                                             f"{'s' if c[7] else ''}" for c in SMALL])
def test_small_shapes(case):
    B, H, Hkv, N, d, dt, causal, cap, s = case
    w = workloads.custom(B, H, Hkv, N, d, dt, causal, cap, sigma_qk=s, seed=N + 13 * d + H, name=f"small{case}")
    x = workloads.make_inputs(w)
    got = run_gpu(w, x)
    ref = oracle_full(w, x)
    _check(w, got, ref)
    if N == 1:
        assert np.abs(to_np(got["dQ"])).max() == 0.0 and np.abs(to_np(got["dK"])).max() == 0.0


@pytest.mark.parametrize("name", workloads.WORKLOAD_ORDER[:4])
@pytest.mark.parametrize("with_dq", [False, True], ids=["four_calls", "bench_step"])
def test_workload_full_oracle(name, with_dq):
    """The four smaller workloads, every output against the full oracle, both
    through the four-call interface and through the benchmarked step
    (attn_bwd_preprocess + attn_bwd_with_dq)."""
    w = workloads.WORKLOADS[name]
    x = workloads.make_inputs(w)
    got = run_gpu(w, x, with_dq=with_dq)
    ref = oracle_full(w, x)
    _check(w, got, ref, names=("O", "LSE", "D", "dQ", "dK", "dV"))


def test_long_sequence_all_heads_bench_step():
    """N = 16384, B = 1, H = 8, causal (the benchmarked workload) through the
    benchmarked step, attn_bwd_preprocess + attn_bwd_with_dq: O, LSE, D, dQ,
    dK and dV of all 8 heads against the full fp64 oracle, per head and over
    the whole tensor.  A second step on the same inputs must give the same
    bits (the bf16 path has no atomics and a fixed summation order)."""
    w = workloads.WORKLOADS[workloads.WORKLOAD_ORDER[4]]
    x = workloads.make_inputs(w)
    got = run_gpu(w, x, with_dq=True)
    again = run_gpu(w, x, o=got["O"], lse=got["LSE"], with_dq=True)
    for n in ("D", "dQ", "dK", "dV"):
        bits = torch.int16 if got[n].dtype == torch.bfloat16 else torch.int32
        assert torch.equal(got[n].view(bits), again[n].view(bits)), f"{n} differs between two steps"
    print(f"[{w.name}] two steps bitwise equal; oracle", flush=True)
    host = {n: to_np(got[n])[0] for n in ("O", "LSE", "D", "dQ", "dK", "dV")}
    del again
    ref = oracle_kv_heads(w, x, 0, range(w.H_kv), progress=True)
    for n in ("O", "LSE", "D", "dQ"):
        for h, r in ref[n].items():
            e = rel_err(host[n][h], r)
            print(f"[{w.name}] head {h} {n}={e:.2e}", flush=True)
            assert e <= TOL[w.dtype], (n, h)
        e = rel_err(host[n], np.stack([ref[n][h] for h in range(w.H)]))
        print(f"[{w.name}] all heads {n}={e:.2e}", flush=True)
        assert e <= TOL[w.dtype], n
    for n in ("dK", "dV"):
        for g, r in ref[n].items():
            e = rel_err(host[n][g], r)
            print(f"[{w.name}] kv head {g} {n}={e:.2e}", flush=True)
            assert e <= TOL[w.dtype], (n, g)
        e = rel_err(host[n], np.stack([ref[n][g] for g in range(w.H_kv)]))
        print(f"[{w.name}] all kv heads {n}={e:.2e}", flush=True)
        assert e <= TOL[w.dtype], n


@pytest.mark.parametrize("with_dq", [False, True], ids=["four_calls", "bench_step"])
def test_one_head_share_full_oracle(with_dq):
    """One head at N = 16384 (256 work units: the combined dK/dV + dQ launch at
    full length; given dQ, its 32 heaviest key blocks split by query range),
    every output against the oracle."""
    w = workloads.WORKLOADS["bf16_causal_b1h1_n16384_d128"]
    x = workloads.make_inputs(w)
    got = run_gpu(w, x, with_dq=with_dq)
    print(f"[{w.name}] kernels done; oracle", flush=True)
    ref = oracle_kv_heads(w, x, 0, [0])
    for n in ("O", "LSE", "D", "dQ", "dK", "dV"):
        e = rel_err(to_np(got[n][0, 0]), ref[n][0])
        print(f"[{w.name}] {n}={e:.2e}", flush=True)
        assert e <= TOL[w.dtype], n


@pytest.mark.parametrize("H,plan", [(8, "bwd_fused_kernel"), (16, "bwd_dkdv_kernel+bwd_dq_kernel")],
                         ids=["combined_2048", "standalone_4096"])
@pytest.mark.parametrize("cap,drop", [(0.0, None), (10.0, (0.1, 77, 2))], ids=["plain", "softcap_dropout"])
def test_many_units_d64(cap, drop, H, plan):
    """B=8 N=2048 d=64 causal at two workgroups per CU: H=8 gives 1024 dK/dV and
    1024 dQ work units, the largest grid the combined launch takes at d = 64;
    H=16 twice that, so the two kernels run one after the other.  Full oracle
    on the first and last heads."""
    w = workloads.custom(8, H, H, 2048, 64, "bf16", True, cap, seed=64, name=f"many_units_d64_h{H}", dropout=drop)
    x = workloads.make_inputs(w)
    assert fab.attn_bwd_kernels(x["Q"], x["K"], causal=True, softcap=cap, dropout=drop, with_dq=False) == plan
    got = run_gpu(w, x)
    for b, g in ((0, 0), (w.B - 1, w.H_kv - 1)):
        ref = oracle_kv_heads(w, x, b, [g])
        for n in ("O", "LSE", "dQ"):
            for h, r in ref[n].items():
                e = rel_err(to_np(got[n][b, h]), r)
                print(f"[{w.name}] b{b} head {h} {n}={e:.2e}", flush=True)
                assert e <= TOL[w.dtype], n
        for n in ("dK", "dV"):
            e = rel_err(to_np(got[n][b, g]), ref[n][g])
            print(f"[{w.name}] b{b} kv head {g} {n}={e:.2e}", flush=True)
            assert e <= TOL[w.dtype], n


def test_preprocess_matches_rowsum_of_same_inputs():
    """D from the GPU equals the fp64 row dot product of the very same O and dO."""
    w = workloads.WORKLOADS[workloads.WORKLOAD_ORDER[2]]
    x = workloads.make_inputs(w)
    got = run_gpu(w, x)
    o, do = to_np(got["O"]), x["dO"].double().numpy()
    ref = (o * do).sum(-1)
    e = np.abs(to_np(got["D"]) - ref).max() / np.abs(ref).max()
    print(f"preprocess D rel err {e:.2e}", flush=True)
    assert e < 1e-5
    # dQaccum was zeroed: its contents are exactly the kernel's sums (finite)
    assert torch.isfinite(got["dQaccum"]).all()


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_dq_convert_bit_exact(dtype):
    """dQ = round(scale * dQaccum) with one fp32 product then RNE to bf16."""
    w = workloads.custom(1, 4, 4, 300, 128, dtype, True, 0.0, seed=5)
    x = workloads.make_inputs(w)
    got = run_gpu(w, x)
    acc = got["dQaccum"].cpu()
    want = (acc * torch.tensor(w.tau, dtype=torch.float32)).to(w.torch_dtype)
    assert torch.equal(got["dQ"].cpu().view(torch.int16 if dtype == "bf16" else torch.int32),
                       want.view(torch.int16 if dtype == "bf16" else torch.int32))


@pytest.mark.parametrize("name", [workloads.WORKLOAD_ORDER[1], workloads.WORKLOAD_ORDER[2]])
def test_backward_on_oracle_forward(name):
    """Error-source isolation: the GPU backward fed the oracle's O (rounded to
    the dtype) and LSE (fp32)."""
    w = workloads.WORKLOADS[name]
    x = workloads.make_inputs(w)
    ref = oracle_full(w, x)
    o = torch.from_numpy(ref["O"]).to(w.torch_dtype)
    lse = torch.from_numpy(ref["LSE"]).float()
    got = run_gpu(w, x, o=o, lse=lse)
    _check(w, got, ref, names=("dQ", "dK", "dV"))


def test_poisoned_buffers():
    """NaN-filled D, dQaccum, dQ, dK, dV: preprocess must clear dQaccum and the
    epilogue must write every dK/dV row, including key blocks with no query rows."""
    w = workloads.custom(1, 4, 2, 333, 128, "bf16", True, 0.0, seed=3)
    x = workloads.make_inputs(w)
    got = run_gpu(w, x, poison=True)
    for n in ("D", "dQ", "dK", "dV"):
        assert torch.isfinite(got[n].float()).all(), n
    _check(w, got, oracle_full(w, x), names=("dQ", "dK", "dV"))


def test_full_scale_invariants():
    """Identities that hold at any size (evaluated in fp64 on the host):
    <V_g, dV_g> = sum over the group's rows of D, and
    sum_h <Q_h, dQ_h> = <K_g, dK_g>."""
    w = workloads.WORKLOADS[workloads.WORKLOAD_ORDER[3]]
    x = workloads.make_inputs(w)
    got = run_gpu(w, x)
    G = w.group
    Q, K, V = (x[n].double().numpy() for n in ("Q", "K", "V"))
    dQ, dK, dV, D = (to_np(got[n]) for n in ("dQ", "dK", "dV", "D"))
    for g in range(w.H_kv):
        hs = slice(g * G, (g + 1) * G)
        lhs, rhs = (V[0, g] * dV[0, g]).sum(), D[0, hs].sum()
        mag = np.abs(V[0, g] * dV[0, g]).sum()
        assert abs(lhs - rhs) / mag < 1e-2, (g, lhs, rhs)
        lhs, rhs = (Q[0, hs] * dQ[0, hs]).sum(), (K[0, g] * dK[0, g]).sum()
        mag = np.abs(K[0, g] * dK[0, g]).sum()
        assert abs(lhs - rhs) / mag < 1e-2, (g, lhs, rhs)


def test_fp32_atomic_run_to_run_spread():
    """fp32 with deterministic = 0 adds the dQ partials of each key block into
    dQaccum with fp32 atomics, so the order of the additions (and the low
    bits of dQ) may vary between runs: several results are correct.  Every
    run must be within the fp32 tolerance of the oracle; the spread between
    runs is reported and must stay at rounding level (1e-5 of max|dQaccum|)."""
    w = workloads.custom(1, 2, 2, 1024, 64, "fp32", True, 0.0, seed=11, name="fp32_atomic_spread")
    x = workloads.make_inputs(w)
    ref = oracle_full(w, x)
    runs = [run_gpu(w, x) for _ in range(4)]
    for r in runs:
        _check(w, r, ref, names=("dQ", "dK", "dV"))
    mag = float(runs[0]["dQaccum"].abs().max())
    spread = max(float((runs[0]["dQaccum"] - r["dQaccum"]).abs().max()) for r in runs[1:])
    differing = sum(int((runs[0]["dQaccum"] != r["dQaccum"]).sum()) for r in runs[1:])
    print(f"fp32 atomics: run-to-run max |dQaccum diff| = {spread:.3e} (max |dQaccum| {mag:.3e}), "
          f"{differing} differing elements over {len(runs) - 1} repeats", flush=True)
    assert spread <= 1e-5 * mag
