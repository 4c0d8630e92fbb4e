"""The C-ABI library on the CPU: it loads, exports every declared symbol,
plans splits, and rejects bad arguments before any HIP call.

Nothing here launches a kernel; the pointers passed are fake device
addresses that the host checks never dereference.
"""

import ctypes
import os
import re

import pytest

import decode_attention_06_amd as fd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fd.h")

FAKE = 0x10000          # 16-byte aligned non-null "device" address
MISALIGNED = 0x10002


@pytest.fixture(scope="module")
def lib():
    return fd.load()


def declared_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            text = open(os.path.join(ROOT, "include", h)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(fd_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 9
    for name in names:
        assert hasattr(lib, name), f"{name} declared in fd.h but not exported"
        assert name in fd.SIGNATURES, f"{name} has no ctypes signature in the binding"


def test_status_strings(lib):
    assert fd.status_name(fd.FD_OK) == "FD_OK"
    assert fd.status_name(fd.FD_ERR_WORKSPACE) == "FD_ERR_WORKSPACE"
    assert lib.fd_version() >= 100


# ---------------------------------------------------------------- planner

def test_plan_invalid_arguments():
    assert fd.plan_splits(0, 4, 4, 64, 512, fd.FD_F32, 256) == -1
    assert fd.plan_splits(1, 6, 4, 64, 512, fd.FD_F32, 256) == -1      # Hq % Hkv
    assert fd.plan_splits(1, 4, 4, 64, 0, fd.FD_F32, 256) == -1
    assert fd.plan_splits(1, 4, 4, 64, 512, 7, 256) == -1
    assert fd.plan_splits(1, 4, 4, 64, 512, fd.FD_F32, 0) == -1


def test_plan_full_gpu_needs_no_split():
    # batch x heads already covers every CU twice over: one piece, except
    # for several long sequences on the vector-ALU kernel (next test)
    assert fd.plan_splits(16, 32, 32, 128, 4096, fd.FD_BF16, 256) == 1
    assert fd.plan_splits(256, 16, 2, 128, 1 << 20, fd.FD_BF16, 256) == 1     # matrix-core kernel


def test_plan_balances_several_long_sequences():
    # lengths of several sequences may differ: long ones get four pieces each
    assert fd.plan_splits(16, 32, 32, 128, 65536, fd.FD_BF16, 256) == 4
    assert fd.plan_splits(64, 8, 8, 128, 1 << 20, fd.FD_BF16, 256) == 4
    assert fd.plan_splits(16, 32, 32, 128, 8192, fd.FD_BF16, 256) == 4
    assert fd.plan_splits(16, 32, 32, 128, 2048, fd.FD_BF16, 256) == 1       # short: the combine costs more
    assert fd.plan_splits(1, 32, 32, 128, 65536, fd.FD_BF16, 256) == 16      # one sequence: by CU count


def test_plan_long_single_sequence_splits_a_lot():
    s = fd.plan_splits(1, 16, 2, 128, 65536, fd.FD_BF16, 256)
    assert 128 <= s <= 512


def test_plan_short_history_limits_splitting():
    # pieces are never planned shorter than one workgroup step of the
    # kernel's rows (vector-ALU kernel: 128 rows for bf16 at D 128, fp32 at
    # D 64 and E4M3 with up to two query rows per unit; 64 with more)
    assert fd.plan_splits(1, 32, 32, 128, 512, fd.FD_BF16, 256) == 4
    assert fd.plan_splits(1, 32, 32, 128, 2048, fd.FD_BF16, 256) == 16
    assert fd.plan_splits(1, 4, 4, 64, 512, fd.FD_F32, 256) == 4
    assert fd.plan_splits(1, 8, 2, 64, 512, fd.FD_F32, 256) == 8        # 4 query rows per unit: 64-row steps
    assert fd.plan_splits(1, 4, 4, 64, 100, fd.FD_F32, 256) == 1
    assert fd.plan_splits(1, 4, 4, 64, 127, fd.FD_F32, 256) == 1
    assert fd.plan_splits(1, 4, 4, 64, 256, fd.FD_F32, 256) == 2


@pytest.mark.parametrize("L", [512, 2048, 8192, 32768, 65536, 1 << 20])
def test_plan_monotone_in_work_units(L):
    prev = None
    for B in (1, 2, 4, 8, 16, 32, 64, 128, 256):
        s = fd.plan_splits(B, 32, 32, 128, L, fd.FD_BF16, 256)
        assert 1 <= s <= fd.FD_MAX_SPLITS
        if prev is not None:
            assert s <= prev, "more independent units never asks for more pieces"
        prev = s


def test_plan_monotone_in_length():
    prev = 0
    for L in (256, 1024, 4096, 16384, 65536, 1 << 18):
        s = fd.plan_splits(1, 16, 2, 128, L, fd.FD_BF16, 256)
        assert s >= prev
        prev = s


# ---------------------------------------------------------- argument checks

def _decode(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, lens=None, B=1, Hq=4, Hkv=4, D=64, L=512, dtype=fd.FD_F32,
             n_splits=4, out=FAKE, out_dtype=fd.FD_F32, lse=None, scale=0.0, ws=FAKE, ws_bytes=0,
             stream=None)
    a.update(kw)
    return lib.fd_decode_attn(a["q"], a["k"], a["v"], a["lens"], a["B"], a["Hq"], a["Hkv"], a["D"], a["L"],
                              a["dtype"], a["n_splits"], a["out"], a["out_dtype"], a["lse"], a["scale"],
                              a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fd.FD_ERR_INVALID_ARG),
    (dict(k=None), fd.FD_ERR_INVALID_ARG),
    (dict(v=None), fd.FD_ERR_INVALID_ARG),
    (dict(out=None), fd.FD_ERR_INVALID_ARG),
    (dict(q=MISALIGNED), fd.FD_ERR_INVALID_ARG),
    (dict(k=MISALIGNED), fd.FD_ERR_INVALID_ARG),
    (dict(lens=0x10001), fd.FD_ERR_INVALID_ARG),
    (dict(B=0), fd.FD_ERR_INVALID_ARG),
    (dict(L=0), fd.FD_ERR_INVALID_ARG),
    (dict(L=(1 << 30) + 1), fd.FD_ERR_INVALID_ARG),
    (dict(Hq=6), fd.FD_ERR_UNSUPPORTED),
    (dict(D=96), fd.FD_ERR_UNSUPPORTED),
    (dict(D=256), fd.FD_ERR_UNSUPPORTED),
    (dict(dtype=5), fd.FD_ERR_UNSUPPORTED),
    (dict(out_dtype=3), fd.FD_ERR_UNSUPPORTED),
    (dict(n_splits=fd.FD_MAX_SPLITS + 1), fd.FD_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fd.FD_ERR_INVALID_ARG),
    (dict(ws=None), fd.FD_ERR_WORKSPACE),
    (dict(ws_bytes=100), fd.FD_ERR_WORKSPACE),
    (dict(ws=0x10008, ws_bytes=1 << 20), fd.FD_ERR_WORKSPACE),
])
def test_decode_rejects_before_any_hip_call(lib, kw, status):
    st = _decode(lib, **kw)
    assert st == status, (st, fd.load().fd_last_error_message())
    assert lib.fd_last_error_message().decode()


def _paged(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, lens=None, B=2, Hq=8, Hkv=2, D=128, ps=16, n_pages=64, mp=32,
             dtype=fd.FD_BF16, n_splits=4, out=FAKE, out_dtype=fd.FD_BF16, lse=None, scale=0.0, ws=FAKE,
             ws_bytes=0, stream=None)
    a.update(kw)
    return lib.fd_decode_attn_paged(a["q"], a["k"], a["v"], a["bt"], a["lens"], a["B"], a["Hq"], a["Hkv"], a["D"],
                                    a["ps"], a["n_pages"], a["mp"], a["dtype"], a["n_splits"], a["out"],
                                    a["out_dtype"], a["lse"], a["scale"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(bt=None), fd.FD_ERR_INVALID_ARG),
    (dict(bt=0x10002), fd.FD_ERR_INVALID_ARG),
    (dict(k=None), fd.FD_ERR_INVALID_ARG),
    (dict(v=MISALIGNED), fd.FD_ERR_INVALID_ARG),
    (dict(ps=8), fd.FD_ERR_UNSUPPORTED),
    (dict(ps=48), fd.FD_ERR_UNSUPPORTED),
    (dict(ps=1 << 21), fd.FD_ERR_UNSUPPORTED),
    (dict(n_pages=0), fd.FD_ERR_INVALID_ARG),
    (dict(n_pages=1 << 31), fd.FD_ERR_INVALID_ARG),
    (dict(mp=0), fd.FD_ERR_INVALID_ARG),
    (dict(mp=1 << 27, ps=16), fd.FD_ERR_INVALID_ARG),     # 2^31 rows per sequence
    (dict(D=96), fd.FD_ERR_UNSUPPORTED),
    (dict(Hq=7), fd.FD_ERR_UNSUPPORTED),
    (dict(q=None), fd.FD_ERR_INVALID_ARG),
    (dict(ws=None), fd.FD_ERR_WORKSPACE),
    (dict(ws_bytes=64), fd.FD_ERR_WORKSPACE),
])
def test_paged_rejects_before_any_hip_call(lib, kw, status):
    st = _paged(lib, **kw)
    assert st == status, (st, fd.load().fd_last_error_message())
    assert lib.fd_last_error_message().decode()


def _fp8(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ks=None, vs=None, lens=None, B=2, Hq=8, Hkv=2, D=128, L=512, n_splits=4,
             out=FAKE, out_dtype=fd.FD_BF16, lse=None, scale=0.0, ws=FAKE, ws_bytes=0, stream=None)
    a.update(kw)
    return lib.fd_decode_attn_fp8(a["q"], a["k"], a["v"], a["ks"], a["vs"], a["lens"], a["B"], a["Hq"], a["Hkv"],
                                  a["D"], a["L"], a["n_splits"], a["out"], a["out_dtype"], a["lse"], a["scale"],
                                  a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(k=None), fd.FD_ERR_INVALID_ARG),
    (dict(v=MISALIGNED), fd.FD_ERR_INVALID_ARG),
    (dict(ks=0x10002), fd.FD_ERR_INVALID_ARG),
    (dict(vs=0x10001), fd.FD_ERR_INVALID_ARG),
    (dict(D=96), fd.FD_ERR_UNSUPPORTED),
    (dict(Hq=6, Hkv=4), fd.FD_ERR_UNSUPPORTED),
    (dict(L=0), fd.FD_ERR_INVALID_ARG),
    (dict(out_dtype=2), fd.FD_ERR_UNSUPPORTED),
    (dict(ws=None), fd.FD_ERR_WORKSPACE),
    (dict(ws_bytes=16), fd.FD_ERR_WORKSPACE),
])
def test_fp8_rejects_before_any_hip_call(lib, kw, status):
    st = _fp8(lib, **kw)
    assert st == status, (st, fd.load().fd_last_error_message())
    assert lib.fd_last_error_message().decode()


def test_fp8_dtype_only_through_its_entry_point(lib):
    assert _decode(lib, dtype=fd.FD_FP8_E4M3, D=128, Hq=8, Hkv=2) == fd.FD_ERR_UNSUPPORTED
    assert _paged(lib, dtype=fd.FD_FP8_E4M3) == fd.FD_ERR_UNSUPPORTED
    assert lib.fd_decode_attn_partials(FAKE, FAKE, FAKE, None, 1, 8, 2, 128, 512, fd.FD_FP8_E4M3, 4, 0, FAKE,
                                       FAKE, 0.0, None) == fd.FD_ERR_UNSUPPORTED
    # planner and workspace size accept it (same partial layout as bf16)
    assert fd.plan_splits(1, 16, 2, 128, 65536, fd.FD_FP8_E4M3, 256) == fd.plan_splits(1, 16, 2, 128, 65536,
                                                                                       fd.FD_BF16, 256)
    n8, n16 = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert lib.fd_decode_attn_workspace_size(1, 16, 2, 128, 4096, fd.FD_FP8_E4M3, 8, ctypes.byref(n8)) == fd.FD_OK
    assert lib.fd_decode_attn_workspace_size(1, 16, 2, 128, 4096, fd.FD_BF16, 8, ctypes.byref(n16)) == fd.FD_OK
    assert n8.value == n16.value > 0


def test_prefill_rejects_before_any_hip_call(lib):
    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, lens=None, B=1, Hq=16, Hkv=2, D=128, L=1024, dtype=fd.FD_BF16, out=FAKE,
                 odt=fd.FD_BF16, lse=None, scale=0.0)
        a.update(kw)
        return lib.fd_prefill_attn(a["q"], a["k"], a["v"], a["lens"], a["B"], a["Hq"], a["Hkv"], a["D"], a["L"],
                                   a["dtype"], a["out"], a["odt"], a["lse"], a["scale"], None)
    assert call(dtype=fd.FD_F32) == fd.FD_ERR_UNSUPPORTED
    assert call(D=64) == fd.FD_ERR_UNSUPPORTED
    assert call(Hq=256, Hkv=1) == fd.FD_ERR_UNSUPPORTED
    assert call(Hq=6, Hkv=4) == fd.FD_ERR_UNSUPPORTED
    assert call(q=None) == fd.FD_ERR_INVALID_ARG
    assert call(k=MISALIGNED) == fd.FD_ERR_INVALID_ARG
    assert call(out=0x10001) == fd.FD_ERR_INVALID_ARG
    assert call(lens=0x10001) == fd.FD_ERR_INVALID_ARG
    assert call(L=0) == fd.FD_ERR_INVALID_ARG
    assert call(B=0) == fd.FD_ERR_INVALID_ARG
    assert call(scale=float("inf")) == fd.FD_ERR_INVALID_ARG
    assert call(odt=7) == fd.FD_ERR_UNSUPPORTED


def test_bifurcated_rejects_bad_arguments(lib):
    def call(**kw):
        a = dict(q=FAKE, kc=FAKE, vc=FAKE, kd=FAKE, vd=FAKE, dl=None, S=4, Hq=8, Hkv=2, D=128, Lc=64, Ld=8,
                 dtype=fd.FD_BF16, out=FAKE, odt=fd.FD_BF16, lse=None, scale=0.0, ws=FAKE, wsb=1 << 20)
        a.update(kw)
        return lib.fd_bifurcated_attn(a["q"], a["kc"], a["vc"], a["kd"], a["vd"], a["dl"], a["S"], a["Hq"],
                                      a["Hkv"], a["D"], a["Lc"], a["Ld"], a["dtype"], a["out"], a["odt"],
                                      a["lse"], a["scale"], a["ws"], a["wsb"], None)
    assert call(kc=None) == fd.FD_ERR_INVALID_ARG
    assert call(vd=MISALIGNED) == fd.FD_ERR_INVALID_ARG
    assert call(S=0) == fd.FD_ERR_INVALID_ARG
    assert call(Lc=0) == fd.FD_ERR_INVALID_ARG
    assert call(Ld=0) == fd.FD_ERR_INVALID_ARG
    assert call(Hkv=3) == fd.FD_ERR_UNSUPPORTED
    assert call(D=80) == fd.FD_ERR_UNSUPPORTED
    assert call(ws=None) == fd.FD_ERR_WORKSPACE
    assert call(dl=0x10003) == fd.FD_ERR_INVALID_ARG
    assert call(dtype=fd.FD_FP8_E4M3) == fd.FD_ERR_UNSUPPORTED


def test_combine_rejects_bad_arguments(lib):
    assert lib.fd_lse_combine(FAKE, FAKE, 0, 4, 64, FAKE, fd.FD_F32, None, None) == fd.FD_ERR_INVALID_ARG
    assert lib.fd_lse_combine(FAKE, FAKE, 4, 0, 64, FAKE, fd.FD_F32, None, None) == fd.FD_ERR_INVALID_ARG
    assert lib.fd_lse_combine(FAKE, FAKE, 4, 4, 513, FAKE, fd.FD_F32, None, None) == fd.FD_ERR_UNSUPPORTED
    assert lib.fd_lse_combine(None, FAKE, 4, 4, 64, FAKE, fd.FD_F32, None, None) == fd.FD_ERR_INVALID_ARG
    assert lib.fd_lse_combine(FAKE, FAKE, 4, 4, 64, 0x10001, fd.FD_F32, None, None) == fd.FD_ERR_INVALID_ARG


def test_workspace_size_is_pure_host_when_splits_forced(lib):
    n = ctypes.c_size_t(0)
    assert lib.fd_decode_attn_workspace_size(2, 8, 2, 128, 4096, fd.FD_BF16, 1, ctypes.byref(n)) == fd.FD_OK
    assert n.value == 0
    assert lib.fd_decode_attn_workspace_size(2, 8, 2, 128, 4096, fd.FD_BF16, 16, ctypes.byref(n)) == fd.FD_OK
    rows = 2 * 8
    assert n.value >= rows * 16 * (128 + 1) * 4
    assert lib.fd_decode_attn_workspace_size(2, 8, 2, 100, 4096, fd.FD_BF16, 16,
                                             ctypes.byref(n)) == fd.FD_ERR_UNSUPPORTED


def test_no_device_is_reported_not_fatal(lib):
    import torch

    if torch.cuda.is_available():
        pytest.skip("a device is visible")
    n = ctypes.c_int32(0)
    assert lib.fd_device_cu_count(ctypes.byref(n)) == fd.FD_ERR_HIP
    assert lib.fd_last_error_message().decode()
    # the planner path of the real call reports the same, without aborting
    assert _decode(lib, n_splits=0) == fd.FD_ERR_HIP


def test_piece_tile_rows():
    # matrix-core kernel: 4 waves of 32-row tiles
    assert fd.piece_tile_rows(16, 2, 128, fd.FD_BF16) == 128
    assert fd.piece_tile_rows(64, 2, 128, fd.FD_FP8_E4M3) == 128
    # vector-ALU kernel: 4 waves x (64 lanes / lanes per row) x loads in flight
    assert fd.piece_tile_rows(32, 32, 128, fd.FD_BF16) == 4 * 4 * 8     # 8 bf16 per lane, 16 lanes per row
    assert fd.piece_tile_rows(4, 4, 64, fd.FD_F32) == 4 * 4 * 8         # 4 fp32 per lane, 16 lanes per row
    assert fd.piece_tile_rows(8, 8, 64, fd.FD_BF16) == 4 * 8 * 8        # 8 lanes per row
    assert fd.piece_tile_rows(32, 32, 128, fd.FD_FP8_E4M3) == 4 * 8 * 4 # 16 codes per lane, half the loads
    assert fd.piece_tile_rows(12, 4, 128, fd.FD_BF16) == 4 * 4 * 8     # G 3: one query row per unit
    assert fd.piece_tile_rows(8, 2, 64, fd.FD_BF16) == 4 * 8 * 4        # 4 rows per unit: 4 loads in flight
    assert fd.piece_tile_rows(8, 1, 128, fd.FD_F32) == 4 * 2 * 4        # 32 lanes per row, 8 rows per unit
    for bad in [(0, 1, 128, fd.FD_BF16), (6, 4, 128, fd.FD_BF16), (8, 8, 96, fd.FD_BF16), (8, 8, 128, 7)]:
        assert fd.piece_tile_rows(*bad) == -1


def test_partials_reject_unknown_piece_layout(lib):
    for layout in (-1, 2):
        st = lib.fd_decode_attn_partials(FAKE, FAKE, FAKE, None, 1, 8, 2, 128, 512, fd.FD_BF16, 4, layout, FAKE,
                                         FAKE, 0.0, None)
        assert st == fd.FD_ERR_INVALID_ARG
        assert "piece_layout" in lib.fd_last_error_message().decode()


def test_noalloc_checks_before_any_hip_call(lib):
    def call(q=FAKE, B=1, n_splits=4, L=512):
        return lib.fd_decode_attn_noalloc(q, FAKE, FAKE, None, B, 4, 4, 64, L, fd.FD_F32, n_splits, FAKE,
                                          fd.FD_F32, None, 0.0, None)
    # partials beyond the fixed array: 1024 x 32 rows x 256 pieces x 65 floats
    assert lib.fd_decode_attn_noalloc(FAKE, FAKE, FAKE, None, 1024, 32, 32, 64, 4096, fd.FD_F32, 256, FAKE,
                                      fd.FD_F32, None, 0.0, None) == fd.FD_ERR_WORKSPACE
    assert "16777216" in lib.fd_last_error_message().decode()
    assert call(q=None) == fd.FD_ERR_INVALID_ARG
    assert call(q=MISALIGNED) == fd.FD_ERR_INVALID_ARG
    assert call(B=0) == fd.FD_ERR_INVALID_ARG
    assert call(n_splits=fd.FD_MAX_SPLITS + 1) == fd.FD_ERR_INVALID_ARG


def test_testing_entry_point_checks_before_any_hip_call(lib):
    def call(kernel, dtype=fd.FD_BF16, D=128, q=FAKE):
        return lib.fd_testing_decode_attn(q, FAKE, FAKE, None, None, None, 1, 8, 2, D, 512, dtype, 4, FAKE,
                                          fd.FD_F32, None, 0.0, FAKE, 0, None, kernel)
    assert call(3) == fd.FD_ERR_INVALID_ARG
    assert call(2, dtype=fd.FD_F32) == fd.FD_ERR_UNSUPPORTED        # matrix-core kernel: bf16 / E4M3 only
    assert call(2, D=64) == fd.FD_ERR_UNSUPPORTED
    assert call(1, q=None) == fd.FD_ERR_INVALID_ARG
    assert call(1) == fd.FD_ERR_WORKSPACE                           # 4 pieces need a workspace


def test_decode_grid_limit_is_checked(lib):
    # 2^22 sequences x 64 KV heads x 4 pieces = 2^30 work units: unsupported, before any launch
    B = 1 << 22
    assert _decode(lib, B=B, Hq=64, Hkv=64, n_splits=4, ws=FAKE, ws_bytes=1 << 62) == fd.FD_ERR_UNSUPPORTED
    assert "2^30" in lib.fd_last_error_message().decode()
    rc = lib.fd_decode_attn_partials(FAKE, FAKE, FAKE, None, B, 64, 64, 64, 512, fd.FD_F32, 4, 0, FAKE, FAKE,
                                     0.0, None)
    assert rc == fd.FD_ERR_UNSUPPORTED


def test_planner_ignores_the_environment(lib, monkeypatch):
    # the split count and the piece tile are functions of their arguments only
    before = (fd.plan_splits(1, 16, 2, 128, 65536, fd.FD_BF16, 256), fd.piece_tile_rows(16, 2, 128, fd.FD_BF16))
    monkeypatch.setenv("FD_PARTIAL_KERNEL", "valu")
    after = (fd.plan_splits(1, 16, 2, 128, 65536, fd.FD_BF16, 256), fd.piece_tile_rows(16, 2, 128, fd.FD_BF16))
    assert before == after == (128, 128)


def test_validation_switch(lib, monkeypatch):
    was = fd.validation_enabled()
    try:
        fd.set_validation(True)
        assert fd.validation_enabled()
        fd.set_validation(False)
        assert not fd.validation_enabled()
    finally:
        fd.set_validation(was)
