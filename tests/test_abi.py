"""CPU tests of the C ABI: the library loads, exports every declared symbol, and rejects bad
arguments with the documented status before any HIP call (so no GPU is needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "swattn.h")


def declared_functions():
    src = open(HEADER).read()
    return re.findall(r"^\s*(?:int|size_t|const char\*)\s+(attn_\w+)\s*\(", src, re.M)


@pytest.fixture(scope="module")
def lib():
    from causal_sliding_window_attn_amd import _lib

    if not os.path.exists(_lib.LIB_PATH):
        from causal_sliding_window_attn_amd import build

        build.build()
    return _lib.load()


def test_header_declares_the_entry_points():
    names = set(declared_functions())
    assert {"attn_fwd", "attn_bwd", "attn_bwd_dq", "attn_bwd_dkdv", "attn_decode", "attn_prefill",
            "attn_kv_append", "attn_decode_step", "attn_decode_step_noalloc", "attn_fwd_varlen", "attn_bwd_varlen",
            "attn_fwd_qknorm", "attn_bwd_qknorm", "attn_bwd_workspace_bytes",
            "attn_decode_workspace_bytes", "attn_decode_launches", "attn_last_error",
            "attn_abi_version"} == names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    from causal_sliding_window_attn_amd import _lib

    assert set(_lib.SIGNATURES) == set(declared_functions())


def test_nm_lists_only_c_symbols(lib):
    import subprocess

    from causal_sliding_window_attn_amd import _lib

    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for name in declared_functions():
        assert name in exported


def test_abi_version(lib):
    assert lib.attn_abi_version() == 6


P = 4096  # an aligned, non-null stand-in pointer: validation must fail before it is ever used


def err(lib):
    return lib.attn_last_error().decode()


@pytest.mark.parametrize("B,H,T,D,w,code", [
    (0, 1, 8, 128, 8, -1), (1, 0, 8, 128, 8, -1), (1, 1, 0, 128, 8, -1), (1, 1, 8, 128, 0, -1),
    (1, 1, 8, 96, 8, -2), (1, 1, 8, 32, 8, -2), (-3, 1, 8, 64, 8, -1), (1, 1, 8, 64, -5, -1),
    (70000, 1, 8, 64, 8, -1),
])
def test_fwd_rejects_bad_dims(lib, B, H, T, D, w, code):
    rc = lib.attn_fwd(P, P, P, P, None, B, H, T, D, w, 0, None)
    assert rc == code and err(lib)


def test_fwd_fp32_grid_limit(lib):
    # fp32 launches one workgroup per 32 queries: (T/32 + 1) * B * H must stay below 2^31, a
    # tighter bound than the bf16 kernels' (T/128 + 1) * B * H
    T = 1 << 24
    assert lib.attn_fwd(P, P, P, P, None, 1, 4096, T, 64, T, 1, None) == -1
    assert "fp32" in err(lib)
    assert lib.attn_fwd(P, P, P, P, None, 1, 4096, T, 64, T, 7, None) == -2  # dtype first


def test_fwd_rejects_bad_pointers_and_dtype(lib):
    assert lib.attn_fwd(None, P, P, P, None, 1, 1, 8, 64, 8, 0, None) == -1
    assert "q" in err(lib)
    assert lib.attn_fwd(P, P, P + 2, P, None, 1, 1, 8, 64, 8, 0, None) == -1
    assert "aligned" in err(lib)
    assert lib.attn_fwd(P, P, P, P, P + 4, 1, 1, 8, 64, 8, 0, None) == -1
    assert lib.attn_fwd(P, P, P, P, None, 1, 1, 8, 64, 8, 7, None) == -2


def test_bwd_validation(lib):
    need = lib.attn_bwd_workspace_bytes(2, 3, 100, 128)
    assert need >= 2 * 3 * 100 * 4 and need % 256 == 0
    assert lib.attn_bwd_workspace_bytes(0, 3, 100, 128) == 0
    args = [P] * 9
    assert lib.attn_bwd(*args, 2, 3, 100, 128, 8, 0, None, need, None) == -3
    assert lib.attn_bwd(*args, 2, 3, 100, 128, 8, 0, P, need - 1, None) == -3
    assert "workspace" in err(lib)
    assert lib.attn_bwd(*args, 2, 3, 100, 128, 8, 1, P, need, None) == -2  # fp32 backward
    bad = list(args)
    bad[5] = None  # dout
    assert lib.attn_bwd(*bad, 2, 3, 100, 128, 8, 0, P, need, None) == -1
    assert lib.attn_bwd(*args, 2, 3, 100, 100, 8, 0, P, need, None) == -2


def test_bwd_pass_validation(lib):
    need = lib.attn_bwd_workspace_bytes(2, 3, 100, 128)
    assert lib.attn_bwd_dq(P, P, P, P, P, P, P, 2, 3, 100, 128, 8, 0, P, need - 1, None) == -3
    assert lib.attn_bwd_dq(P, P, P, None, P, P, P, 2, 3, 100, 128, 8, 0, P, need, None) == -1
    assert lib.attn_bwd_dkdv(P, P, P, P, P, None, P, 2, 3, 100, 128, 8, 0, P, need, None) == -1
    assert lib.attn_bwd_dkdv(P, P, P, P, P, P, P, 2, 3, 100, 128, 8, 1, P, need, None) == -2
    assert lib.attn_bwd_dkdv(P, P, P, P, P, P, P, 2, 3, 0, 128, 8, 0, P, need, None) == -1


def test_prefill_append_decode_validation(lib):
    assert lib.attn_prefill(P, P, P, None, P, None, 2, 2, 16, 32, 128, 8, None) == -1
    assert lib.attn_prefill(P, P, P, P + 2, P, None, 2, 2, 16, 32, 128, 8, None) == -1
    assert lib.attn_prefill(P, P, P, P, P, None, 2, 2, 16, 0, 128, 8, None) == -1
    assert lib.attn_prefill(P, P, P, P, P, None, 2, 2, 16, 32, 64, 0, None) == -1
    assert lib.attn_kv_append(P, P, P, P, None, 2, 2, 32, 128, None) == -1
    assert lib.attn_kv_append(P, P, P, P, P, 2, 2, 32, 80, None) == -2
    need = lib.attn_decode_workspace_bytes(2, 2, 100, 128)
    assert need > 0
    assert lib.attn_decode(P, P, P, P, P, None, 2, 2, 100, 128, 8, P, need - 1, None) == -3
    assert lib.attn_decode(P, P, P, P, P, None, 2, 2, 100, 128, 8, None, need, None) == -3
    assert lib.attn_decode(P, P, P, P, P, None, 2, 2, 100, 128, 0, P, need, None) == -1
    assert lib.attn_decode(P, P, P, None, P, None, 2, 2, 100, 128, 8, P, need, None) == -1


def test_decode_schedule_rule(lib):
    # one launch unless fewer than 128 (sequence, head) pairs each see more than 2048 rows
    assert lib.attn_decode_launches(64, 15, 2048, 128, 1 << 30) == 1
    assert lib.attn_decode_launches(1, 15, 2048, 128, 1 << 30) == 1
    assert lib.attn_decode_launches(1, 15, 2049, 128, 1 << 30) == 2
    assert lib.attn_decode_launches(1, 15, 16384, 128, 2048) == 1
    assert lib.attn_decode_launches(8, 15, 16384, 64, 2049) == 2
    assert lib.attn_decode_launches(8, 16, 16384, 128, 1 << 30) == 1
    assert lib.attn_decode_launches(1, 15, 2049, 80, 1 << 30) == -2
    assert lib.attn_decode_launches(0, 15, 2049, 128, 1 << 30) == -1
    assert lib.attn_decode_launches(1, 15, 2049, 128, 0) == -1
    assert lib.attn_decode_launches(1, 15, 65535 * 64, 128, 1 << 30) == 2
    assert lib.attn_decode_launches(1, 15, 65535 * 64 + 1, 128, 1 << 30) == -1
    need = lib.attn_decode_workspace_bytes(1, 1, 65535 * 64 + 1, 128)
    assert lib.attn_decode(P, P, P, P, P, None, 1, 1, 65535 * 64 + 1, 128, 8, P, need, None) == -1


def test_decode_step_validation(lib):
    need = lib.attn_decode_workspace_bytes(2, 2, 100, 128)
    # q, knew, vnew, kcache, vcache, pos, o, lse, B, H, Lcap, D, window, ws, ws_bytes, stream
    ok = [P, P, P, P, P, P, P, None, 2, 2, 100, 128, 8, P, need, None]

    def call(**change):
        a = list(ok)
        for i, val in change.items():
            a[int(i[1:])] = val
        return lib.attn_decode_step(*a)

    assert call(a13=P, a14=need - 1) == -3
    assert call(a13=None) == -3
    assert "workspace" in err(lib)
    assert call(a12=0) == -1  # window
    assert call(a5=None) == -1 and "pos" in err(lib)
    assert call(a5=P + 2) == -1  # pos alignment
    assert call(a1=None) == -1 and "knew" in err(lib)
    assert call(a4=None) == -1 and "vcache" in err(lib)
    assert call(a7=P + 2) == -1  # lse alignment
    assert call(a11=80) == -2  # head dimension
    assert call(a10=0) == -1  # Lcap


def test_decode_step_noalloc_validation(lib):
    # q, knew, vnew, kcache, vcache, pos, o, lse, B, H, Lcap, D, window, stream
    ok = [P, P, P, P, P, P, P, None, 2, 2, 100, 128, 8, None]

    def call(**change):
        a = list(ok)
        for i, val in change.items():
            a[int(i[1:])] = val
        return lib.attn_decode_step_noalloc(*a)

    assert call(a12=0) == -1  # window
    assert call(a5=None) == -1 and "pos" in err(lib)
    assert call(a5=P + 2) == -1  # pos alignment
    assert call(a0=None) == -1 and "q" in err(lib)
    assert call(a6=None) == -1 and "o" in err(lib)
    assert call(a7=P + 2) == -1  # lse alignment
    assert call(a11=80) == -2  # head dimension
    assert call(a10=0) == -1  # Lcap
    assert call(a10=65535 * 64 + 1) == -1  # the split schedule's grid limit
    # the split schedule (few pairs, more than 2048 visible rows) whose partial results would
    # exceed the 32 MiB static scratch is refused before any HIP call
    assert lib.attn_decode_launches(4, 30, 70000, 128, 70000) == 2
    assert lib.attn_decode_workspace_bytes(4, 30, 70000, 128) > 32 << 20
    assert call(a8=4, a9=30, a10=70000, a12=70000) == -3
    assert "static scratch" in err(lib)


def test_varlen_validation(lib):
    # q, k, v, o, lse, cu, nseq, total, max_seqlen, H, D, window, stream
    ok = [P, P, P, P, None, P, 3, 100, 50, 2, 128, 8, None]

    def fwd(**change):
        a = list(ok)
        for i, val in change.items():
            a[int(i[1:])] = val
        return lib.attn_fwd_varlen(*a)

    assert fwd(a5=None) == -1 and "cu_seqlens" in err(lib)
    assert fwd(a5=P + 2) == -1
    assert fwd(a6=0) == -1  # nseq
    assert fwd(a7=0) == -1  # total
    assert fwd(a8=0) == -1  # max_seqlen
    assert fwd(a8=101) == -1 and "max_seqlen" in err(lib)
    assert fwd(a10=96) == -2  # head dimension
    assert fwd(a11=0) == -1  # window
    assert fwd(a0=None) == -1 and "q" in err(lib)
    assert fwd(a4=P + 4) == -1  # lse alignment
    need = lib.attn_bwd_workspace_bytes(1, 2, 100, 128)
    # q, k, v, o, lse, dout, dq, dk, dv, cu, nseq, total, max_seqlen, H, D, window, ws, ws_bytes
    bok = [P] * 10 + [3, 100, 50, 2, 128, 8, P, need, None]

    def bwd(**change):
        a = list(bok)
        for i, val in change.items():
            a[int(i[1:])] = val
        return lib.attn_bwd_varlen(*a)

    assert bwd(a17=need - 1) == -3 and "workspace" in err(lib)
    assert bwd(a16=None) == -3
    assert bwd(a4=None) == -1 and "lse" in err(lib)
    assert bwd(a9=None) == -1 and "cu_seqlens" in err(lib)
    assert bwd(a5=None) == -1 and "dout" in err(lib)
    assert bwd(a12=200) == -1


def test_qknorm_validation(lib):
    # q, k, v, qn, kn, rq, rk, o, lse, B, H, T, D, window, eps, stream
    ok = [P] * 8 + [None, 2, 3, 64, 128, 8, 1e-6, None]

    def fwd(**change):
        a = list(ok)
        for i, val in change.items():
            a[int(i[1:])] = val
        return lib.attn_fwd_qknorm(*a)

    assert fwd(a14=-1.0) == -1 and "eps" in err(lib)
    assert fwd(a14=float("nan")) == -1
    assert fwd(a3=None) == -1 and "qn" in err(lib)
    assert fwd(a6=None) == -1 and "rk" in err(lib)
    assert fwd(a12=80) == -2
    assert fwd(a13=0) == -1
    need = lib.attn_bwd_workspace_bytes(2, 3, 64, 128)
    # qn, kn, v, o, lse, dout, rq, rk, dq, dk, dv, B, H, T, D, window, ws, ws_bytes, stream
    bok = [P] * 11 + [2, 3, 64, 128, 8, P, need, None]

    def bwd(**change):
        a = list(bok)
        for i, val in change.items():
            a[int(i[1:])] = val
        return lib.attn_bwd_qknorm(*a)

    assert bwd(a6=None) == -1 and "rq" in err(lib)
    assert bwd(a7=P + 4) == -1
    assert bwd(a17=need - 1) == -3
    assert bwd(a5=None) == -1 and "dout" in err(lib)


def test_last_error_is_thread_local(lib):
    import threading

    lib.attn_fwd(None, P, P, P, None, 1, 1, 8, 64, 8, 0, None)
    here = err(lib)
    seen = []

    def other():
        seen.append(lib.attn_last_error().decode())

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert here and seen == [""]


def test_python_binding_rejects_host_tensors():
    import torch

    import causal_sliding_window_attn_amd as sw

    q = torch.zeros(1, 8, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sw.attn_fwd(q, q, q)
    with pytest.raises(ValueError):
        sw.attention(q, q, q, window=0)


def test_binding_exposes_c_names():
    import causal_sliding_window_attn_amd as sw

    for name in declared_functions():
        assert callable(getattr(sw, name)), name
