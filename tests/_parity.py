"""Helpers for the GPU parity tests: run the HIP path on a workload and
compare with the fp64 oracle.  Not collected by pytest (no test_ prefix)."""
import numpy as np
import torch

import flashattention_backward_pass_amd as fab
from flashattention_backward_pass_amd import workloads
import oracle

TOL = {"fp32": 1e-4, "bf16": 2e-2}


def rel_err(got, ref):
    """max |got - ref| / max |ref| over the whole tensor (0 when ref is all zero and got matches)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max() if ref.size else 0.0
    num = np.abs(got - ref).max() if ref.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)


def to_np(t):
    return t.detach().double().cpu().numpy()


def run_gpu(w, x, *, o=None, lse=None, poison=False, deterministic=False, with_dq=False):
    """Forward (unless o/lse given) then backward on cuda:0.  Returns a dict of
    device tensors.  with_dq=False: attn_bwd_preprocess, attn_bwd and
    attn_bwd_dq_convert (the four-call interface); with_dq=True:
    attn_bwd_preprocess and attn_bwd_with_dq, the step the benchmark times
    (dQaccum is then scratch and is not returned)."""
    dev = torch.device("cuda:0")
    q, k, v, do = (x[n].to(dev) for n in ("Q", "K", "V", "dO"))
    if o is None:
        o, lse = fab.attention_forward(q, k, v, causal=w.causal, scale=w.tau, softcap=w.softcap, window=w.window,
                                       dropout=w.dropout)
    else:
        o, lse = o.to(dev), lse.to(dev)
    B, H, N, d = q.shape
    D = torch.empty(B, H, N, device=dev, dtype=torch.float32)
    acc = torch.empty(B, H, N, d, device=dev, dtype=torch.float32)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if poison:
        for t in (D, acc, dq, dk, dv):
            t.fill_(float("nan"))
    fab.attn_bwd_preprocess(o, do, D, acc, H_kv=w.H_kv, causal=w.causal, scale=w.tau, softcap=w.softcap,
                            window=w.window)
    if with_dq:
        fab.attn_bwd_with_dq(q, k, v, do, lse, D, acc, dq, dk, dv, causal=w.causal, scale=w.tau,
                             softcap=w.softcap, deterministic=deterministic, window=w.window, dropout=w.dropout)
        torch.cuda.synchronize()
        return {"O": o, "LSE": lse, "D": D, "dQ": dq, "dK": dk, "dV": dv}
    fab.attn_bwd(q, k, v, do, lse, D, acc, dk, dv, causal=w.causal, scale=w.tau, softcap=w.softcap,
                 deterministic=deterministic, window=w.window, dropout=w.dropout)
    acc_copy = acc.clone()
    fab.attn_bwd_dq_convert(acc, dq, scale=w.tau)
    torch.cuda.synchronize()
    return {"O": o, "LSE": lse, "D": D, "dQaccum": acc_copy, "dQ": dq, "dK": dk, "dV": dv}


_ORACLE_CACHE = {}


def oracle_full(w, x):
    """The full oracle of a workload (inputs are the seeded ones of make_inputs(w));
    the last two workloads' results are kept, so tests that check two paths of
    one workload compute it once."""
    if w in _ORACLE_CACHE:
        return _ORACLE_CACHE[w]
    r = _oracle_full(w, x)
    while len(_ORACLE_CACHE) >= 2:
        _ORACLE_CACHE.pop(next(iter(_ORACLE_CACHE)))
    _ORACLE_CACHE[w] = r
    return r


def _oracle_full(w, x):
    return oracle.reference(x["Q"], x["K"], x["V"], x["dO"], w.tau, w.causal, w.softcap, w.window, w.dropout)


_KV_CACHE = {}


def oracle_kv_heads(w, x, b, kv_heads, progress=False):
    """Full per-head oracle for batch b and the given key/value heads (all their
    query heads); the last result is kept for a second path of the same heads."""
    key = (w, b, tuple(kv_heads))
    if key not in _KV_CACHE:
        _KV_CACHE.clear()
        _KV_CACHE[key] = _oracle_kv_heads(w, x, b, kv_heads, progress)
    return _KV_CACHE[key]


def _oracle_kv_heads(w, x, b, kv_heads, progress):
    G = w.group
    out = {"O": {}, "LSE": {}, "D": {}, "dQ": {}, "dK": {}, "dV": {}}
    for g in kv_heads:
        if progress:
            print(f"[{w.name}] oracle b{b} kv head {g}", flush=True)
        k, v = x["K"][b, g], x["V"][b, g]
        dk = dv = 0.0
        for h in range(g * G, (g + 1) * G):
            q, do = x["Q"][b, h], x["dO"][b, h]
            zf = oracle.head_dropout(w.dropout, b * w.H + h)
            O, L = oracle.forward_head(q, k, v, w.tau, w.causal, w.softcap, w.window, zf)
            dq, dk_h, dv_h, D = oracle.backward_head(q, k, v, O, do, L, w.tau, w.causal, w.softcap, w.window, zf)
            out["O"][h], out["LSE"][h], out["D"][h], out["dQ"][h] = O, L, D, dq
            dk = dk + dk_h
            dv = dv + dv_h
        out["dK"][g], out["dV"][g] = dk, dv
    return out
