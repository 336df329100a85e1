"""CPU-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments before any HIP call.

No test here launches a kernel: every call either fails validation or is an
empty problem (which enqueues nothing).
"""
import ctypes
import os
import re

import pytest

import flashattention_backward_pass_amd as fab

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fabwd.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fab.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    return fab.load_library()


def test_header_declares_the_entry_points():
    names = header_functions()
    for n in ("attn_fwd_stats", "attn_bwd_preprocess", "attn_bwd", "attn_bwd_dq_convert", "attn_status_str"):
        assert n in names


def test_library_exports_every_header_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), f"libfabwd.so does not export {name}"
    assert set(header_functions()) == set(fab.EXPORTS), "binding table out of sync with the header"


def test_status_strings(lib):
    for code in range(5):
        s = fab.status_str(code)
        assert s.startswith("ATTN_")
    assert "unknown" in fab.status_str(99)
    assert lib.attn_version().decode().startswith("fabwd")


def test_params_layout_matches_header():
    """The ctypes struct lists the header's fields, in order, with the same types."""
    import re
    text = open(HEADER).read()
    body = text[text.index("typedef struct attn_params {"):text.index("} attn_params;")]
    fields = []
    types = {"int32_t": ctypes.c_int32, "uint32_t": ctypes.c_uint32, "float": ctypes.c_float}
    for typ, names in re.findall(r"^\s*(u?int32_t|float)\s+([^;]+);", body, re.M):
        for n in names.split(","):
            fields.append((n.strip(), types[typ]))
    assert [(n, t) for n, t in fab.attn_params._fields_] == fields
    assert ctypes.sizeof(fab.attn_params) == 4 * len(fields)  # no padding


# Fake, 16-byte aligned, non-null device pointers: validation rejects the call
# before they could be used.
A = ctypes.c_void_p(0x10000)
MIS = ctypes.c_void_p(0x10008)
S = ctypes.c_void_p(0)


def call_all(lib, p, ptr=A):
    pp = ctypes.byref(p)
    return [
        lib.attn_fwd_stats(pp, ptr, ptr, ptr, ptr, ptr, S),
        lib.attn_bwd_preprocess(pp, ptr, ptr, ptr, ptr, S),
        lib.attn_bwd(pp, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, S),
        lib.attn_bwd_dq_convert(pp, ptr, ptr, S),
        lib.attn_bwd_with_dq(pp, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, S),
    ]


N_ENTRY = 5  # entry points that call_all exercises


BAD = [
    dict(H=0), dict(H_kv=0), dict(H=6, H_kv=4), dict(N=-1), dict(B=-2), dict(d=0), dict(dtype=2),
    dict(causal=2), dict(scale=0.0), dict(scale=-1.0), dict(scale=float("nan")), dict(scale=float("inf")),
    dict(softcap=-1.0), dict(softcap=float("inf")), dict(N=(1 << 24) + 1),
    dict(window_left=-2), dict(window_right=-3),
    dict(dropout_p=-0.1), dict(dropout_p=1.0), dict(dropout_p=1.5), dict(dropout_p=float("nan")),
    dict(dropout_p=float("inf")),
]


@pytest.mark.parametrize("bad", BAD, ids=[str(b) for b in BAD])
def test_invalid_arguments(lib, bad):
    kw = dict(B=1, H=4, H_kv=2, N=64, d=64, dtype=1, causal=0, scale=0.125, softcap=0.0, deterministic=0,
              window_left=-1, window_right=-1, dropout_p=0.0, rng_seed_lo=0, rng_seed_hi=0, rng_offset=0)
    kw.update(bad)
    p = fab.attn_params(**kw)
    assert call_all(lib, p) == [fab.ATTN_ERR_INVALID_ARG] * N_ENTRY


@pytest.mark.parametrize("d", [32, 96, 256])
def test_unsupported_head_dim(lib, d):
    assert call_all(lib, fab.make_params(1, 2, 2, 64, d, 1)) == [fab.ATTN_ERR_UNSUPPORTED] * N_ENTRY


@pytest.mark.parametrize("det", [2, -1])
def test_deterministic_flag_out_of_range(lib, det):
    assert call_all(lib, fab.make_params(1, 2, 2, 64, 64, 1, deterministic=det)) == [fab.ATTN_ERR_INVALID_ARG] * N_ENTRY


@pytest.mark.parametrize("dtype", [0, 1])
def test_deterministic_mode_accepted(lib, dtype):
    # An empty problem validates every argument but launches nothing.
    assert call_all(lib, fab.make_params(1, 2, 2, 0, 64, dtype, deterministic=1), ptr=None) == [fab.ATTN_OK] * N_ENTRY


def test_null_params(lib):
    assert lib.attn_bwd_dq_convert(None, A, A, S) == fab.ATTN_ERR_INVALID_ARG


def test_null_pointers(lib):
    assert call_all(lib, fab.make_params(1, 2, 2, 64, 64, 1), ptr=ctypes.c_void_p(0)) == \
        [fab.ATTN_ERR_INVALID_ARG] * N_ENTRY


def test_misaligned_pointers(lib):
    assert call_all(lib, fab.make_params(1, 2, 2, 64, 64, 1), ptr=MIS) == [fab.ATTN_ERR_MISALIGNED] * N_ENTRY


def test_too_many_elements(lib):
    assert call_all(lib, fab.make_params(1 << 12, 1 << 10, 1, 1 << 13, 128, 1)) == [fab.ATTN_ERR_INVALID_ARG] * N_ENTRY
    # B*H*N*d just above 2^36 is rejected; exactly 2^36 passes the size check, so
    # those calls fail on the (null or misaligned) pointers instead.
    over = fab.make_params(1, 1 << 9, 1 << 9, (1 << 20) + 1, 128, 1)
    assert call_all(lib, over) == [fab.ATTN_ERR_INVALID_ARG] * N_ENTRY
    at = fab.make_params(1, 1 << 9, 1 << 9, 1 << 20, 128, 1)
    assert call_all(lib, at, ptr=ctypes.c_void_p(0)) == [fab.ATTN_ERR_INVALID_ARG] * N_ENTRY  # null pointers
    assert call_all(lib, at, ptr=MIS) == [fab.ATTN_ERR_MISALIGNED] * N_ENTRY  # size accepted, pointer checked next


def test_grid_limits(lib):
    """Short sequences with very many heads: few elements, but a grid of
    2*B*H*ceil(N/128) workgroups of 256 work-items past 2^32 is rejected."""
    many = fab.make_params(1 << 22, 4, 4, 1, 64, 1)  # 2^30 elements, 2^33 work-items
    assert call_all(lib, many) == [fab.ATTN_ERR_INVALID_ARG] * N_ENTRY
    fits = fab.make_params(1 << 20, 4, 4, 1, 64, 1)  # 2^31 work-items: size accepted, pointers checked
    assert call_all(lib, fits, ptr=MIS) == [fab.ATTN_ERR_MISALIGNED] * N_ENTRY
    # fp32 puts B and H in the second and third grid dimensions
    assert call_all(lib, fab.make_params(65536, 1, 1, 16, 64, 0), ptr=MIS) == [fab.ATTN_ERR_INVALID_ARG] * N_ENTRY
    assert call_all(lib, fab.make_params(65535, 1, 1, 16, 64, 0), ptr=MIS) == [fab.ATTN_ERR_MISALIGNED] * N_ENTRY
    assert call_all(lib, fab.make_params(65536, 1, 1, 16, 64, 1), ptr=MIS) == [fab.ATTN_ERR_MISALIGNED] * N_ENTRY


@pytest.mark.parametrize("shape", [(0, 2, 2, 64), (1, 2, 2, 0)])
def test_empty_problems_are_ok_without_pointers(lib, shape):
    B, H, Hkv, N = shape
    assert call_all(lib, fab.make_params(B, H, Hkv, N, 128, 1, causal=1), ptr=ctypes.c_void_p(0)) == \
        [fab.ATTN_OK] * N_ENTRY


def test_binding_fails_loudly_without_library(tmp_path):
    saved = fab._lib
    try:
        fab._lib = None
        with pytest.raises(RuntimeError, match="not built"):
            fab.load_library(str(tmp_path / "missing.so"))
    finally:
        fab._lib = saved


def _bufs(B=1, H=4, Hkv=2, N=8, d=64):
    import torch
    bf, f32 = torch.bfloat16, torch.float32
    q = torch.zeros(B, H, N, d, dtype=bf)
    k = torch.zeros(B, Hkv, N, d, dtype=bf)
    return dict(q=q, k=k, v=k.clone(), o=q.clone(), do=q.clone(), lse=torch.zeros(B, H, N, dtype=f32),
                D=torch.zeros(B, H, N, dtype=f32), acc=torch.zeros(B, H, N, d, dtype=f32), dk=k.clone(),
                dv=k.clone(), dq=q.clone())


@pytest.mark.parametrize("bad", ["v", "do", "lse", "D", "acc", "dk", "dv"])
def test_binding_checks_every_buffer_of_attn_bwd(bad):
    """The C interface gets bare pointers: the binding rejects any buffer whose
    shape or dtype does not match the problem before the library is called."""
    import torch
    t = _bufs()
    wrong = dict(t)
    x = t[bad]
    wrong[bad] = torch.zeros(*x.shape[:-1], x.shape[-1] + 1, dtype=x.dtype)  # one element too many per row
    with pytest.raises(ValueError, match="shape"):
        fab.attn_bwd(wrong["q"], wrong["k"], wrong["v"], wrong["do"], wrong["lse"], wrong["D"], wrong["acc"],
                     wrong["dk"], wrong["dv"])
    wrong[bad] = x.to(torch.float16)
    with pytest.raises(TypeError, match="dtype"):
        fab.attn_bwd(wrong["q"], wrong["k"], wrong["v"], wrong["do"], wrong["lse"], wrong["D"], wrong["acc"],
                     wrong["dk"], wrong["dv"])


def test_binding_checks_buffers_of_the_other_entry_points():
    import torch
    t = _bufs()
    short = torch.zeros(1, 4, 7, dtype=torch.float32)
    with pytest.raises(ValueError, match="LSE"):
        fab.attn_fwd_stats(t["q"], t["k"], t["v"], t["o"], short)
    with pytest.raises(ValueError, match="D"):
        fab.attn_bwd_preprocess(t["o"], t["do"], short, t["acc"], H_kv=2)
    with pytest.raises(ValueError, match="dQaccum"):
        fab.attn_bwd_dq_convert(t["acc"][:, :, :7], t["dq"])
    with pytest.raises(ValueError, match="dQ"):
        fab.attn_bwd_with_dq(t["q"], t["k"], t["v"], t["do"], t["lse"], t["D"], t["acc"], t["dq"][:, :, :7],
                             t["dk"], t["dv"])


@pytest.mark.parametrize("window", [(0, 0), (5, -1), (-1, 3), (1 << 24, 7)])
def test_windows_accepted(lib, window):
    # Valid windows on an empty problem: every argument is checked, nothing runs.
    p = fab.make_params(1, 2, 2, 0, 64, 1, causal=1, window=window)
    assert call_all(lib, p, ptr=None) == [fab.ATTN_OK] * N_ENTRY


@pytest.mark.parametrize("p", [0.0, 0.1, 0.999])
def test_dropout_accepted(lib, p):
    params = fab.make_params(1, 2, 2, 0, 64, 1, dropout=(p, (1 << 64) - 1, (1 << 32) - 1))
    assert (params.rng_seed_lo, params.rng_seed_hi, params.rng_offset) == (0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF)
    assert call_all(lib, params, ptr=None) == [fab.ATTN_OK] * N_ENTRY


def test_dropout_seed_range():
    with pytest.raises(ValueError):
        fab.make_params(1, 2, 2, 8, 64, 1, dropout=(0.1, 1 << 64, 0))
    with pytest.raises(ValueError):
        fab.make_params(1, 2, 2, 8, 64, 1, dropout=(0.1, 0, 1 << 32))


def test_header_is_plain_c(tmp_path):
    """include/fabwd.h compiles as C99 with -pedantic (a C-ABI header: no C++ or torch types)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not installed")
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    src = tmp_path / "use_header.c"
    src.write_text('#include "fabwd.h"\nint main(void) { attn_params p; (void)p; return 0; }\n')
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", inc, str(src),
                        "-o", str(tmp_path / "use_header")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_bwd_kernels_query(lib):
    """attn_bwd_kernels names the kernels a call would launch (host logic only:
    it validates like the entry points and enqueues nothing)."""
    def plan(B, H, Hkv, N, d, dt, causal=0, det=0, with_dq=1):
        p = fab.make_params(B, H, Hkv, N, d, dt, causal, deterministic=det)
        return lib.attn_bwd_kernels(ctypes.byref(p), with_dq)
    assert plan(1, 3, 2, 100, 64, fab.ATTN_BF16) is None          # H % H_kv != 0
    assert plan(1, 2, 2, 100, 96, fab.ATTN_BF16) is None          # unsupported head dim
    assert plan(1, 2, 2, 100, 64, fab.ATTN_BF16, with_dq=2) is None
    assert plan(0, 2, 2, 100, 64, fab.ATTN_BF16) == b""
    assert plan(1, 2, 2, 100, 64, fab.ATTN_FP32, with_dq=0) == b"bwd_simple_kernel"
    assert plan(1, 2, 2, 100, 64, fab.ATTN_FP32) == b"bwd_simple_kernel+dq_convert_kernel"
    assert plan(1, 2, 2, 100, 64, fab.ATTN_FP32, det=1, with_dq=0) == b"bwd_simple_kernel+bwd_dq_simple_kernel"
    assert plan(1, 4, 4, 512, 128, fab.ATTN_BF16, 1) == b"bwd_fused_kernel"
    assert plan(1, 4, 4, 512, 128, fab.ATTN_BF16, 1, with_dq=0) == b"bwd_fused_kernel"
    # Given dQ, a combined launch whose heaviest causal units outweigh the
    # per-compute-unit average splits them; balanced grids do not.
    split = b"bwd_fused_kernel:split"
    assert plan(1, 1, 1, 16384, 128, fab.ATTN_BF16, 1) == split
    assert plan(1, 1, 1, 16384, 128, fab.ATTN_BF16, 1, with_dq=0) == b"bwd_fused_kernel"
    assert plan(1, 2, 1, 3000, 128, fab.ATTN_BF16, 1) == split
    assert plan(1, 1, 1, 16384, 128, fab.ATTN_BF16, 0) == b"bwd_fused_kernel"         # equal units
    assert plan(2, 16, 16, 1024, 64, fab.ATTN_BF16, 1) == b"bwd_fused_kernel"         # 2 units per compute unit
    assert plan(1, 16, 16, 1024, 128, fab.ATTN_BF16, 1) == b"bwd_fused_kernel"        # packing: too little to gain
    assert plan(2, 4, 4, 2500, 128, fab.ATTN_BF16, 1) == b"bwd_fused_kernel"          # packing: too little to gain
    assert plan(1, 4, 4, 2048, 128, fab.ATTN_BF16, 1) == split
    # The combined launch takes up to 2048 workgroups at d = 64, 1024 at d = 128.
    assert plan(8, 8, 8, 2048, 64, fab.ATTN_BF16, 1, with_dq=0) == b"bwd_fused_kernel"
    assert plan(8, 16, 16, 2048, 64, fab.ATTN_BF16, 1, with_dq=0) == b"bwd_dkdv_kernel+bwd_dq_kernel"
    assert plan(4, 16, 16, 2048, 128, fab.ATTN_BF16, 1, with_dq=0) == b"bwd_dkdv_kernel+bwd_dq_kernel"
    assert plan(1, 8, 8, 16384, 128, fab.ATTN_BF16, 1) == b"bwd_dkdv_kernel+bwd_dq_kernel"
    # Grouped heads with few units: the dK/dV work is split over two workgroups
    # per unit; given dQ the dQ kernel adds the partials, else a sum launch.
    assert plan(1, 32, 8, 1024, 128, fab.ATTN_BF16, 1) == b"bwd_dkdv_kernel+bwd_dq_kernel"
    assert plan(1, 32, 8, 1024, 128, fab.ATTN_BF16, 1, with_dq=0) == \
        b"bwd_dkdv_kernel+dkdv_split_sum_kernel+bwd_dq_kernel"
    assert plan(4, 16, 16, 4096, 64, fab.ATTN_BF16, 1, with_dq=0) == b"bwd_dkdv_kernel+bwd_dq_kernel"


def test_noalloc_rejects_oversized_scratch(lib):
    """attn_bwd_with_dq_noalloc keeps D and its scratch in a 2^24-float static
    array: a step that needs more (fp32: B*H*N*(d+1) floats) is refused before
    any device call; invalid parameters are refused as by the other calls."""
    ptr = ctypes.c_void_p(256)
    p = fab.make_params(1, 16, 16, 8192, 128, fab.ATTN_FP32, True)
    assert lib.attn_bwd_with_dq_noalloc(ctypes.byref(p), *(ptr,) * 9, None) == fab.ATTN_ERR_INVALID_ARG
    p = fab.make_params(1, 3, 2, 100, 64, fab.ATTN_BF16, True)
    assert lib.attn_bwd_with_dq_noalloc(ctypes.byref(p), *(ptr,) * 9, None) == fab.ATTN_ERR_INVALID_ARG
    p = fab.make_params(0, 2, 2, 100, 64, fab.ATTN_BF16, True)
    assert lib.attn_bwd_with_dq_noalloc(ctypes.byref(p), *(None,) * 9, None) == fab.ATTN_OK
