"""Python binding of libfd (MI355X decode attention): argument marshalling only.

Every step of the computation runs in the HIP kernels behind the C ABI in
include/fd.h.  PyTorch supplies device memory and the current stream; this
module checks tensor shapes, dtypes and placement, allocates the workspace
with torch, and calls the library through ctypes.  If libfd.so has not been
built the first call raises: there is no fallback implementation.
"""

import ctypes
import os

# FD_LIBRARY_PATH names another build of the same library (the sanitized
# build the CPU tests run under AddressSanitizer); default: the in-tree one.
LIB_PATH = os.environ.get("FD_LIBRARY_PATH") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib",
                                                             "libfd.so")

FD_OK, FD_ERR_INVALID_ARG, FD_ERR_UNSUPPORTED, FD_ERR_WORKSPACE, FD_ERR_HIP = range(5)
FD_F32, FD_BF16, FD_FP8_E4M3 = 0, 1, 2
FD_MAX_SPLITS = 4096
FD_NOALLOC_MAX_WORKSPACE = 16 << 20
FD_PIECES_CONTIGUOUS, FD_PIECES_INTERLEAVED = 0, 1
TESTING_KERNELS = {"auto": 0, "valu": 1, "mfma": 2}   # include/fd_testing.h

# Exported symbols and their ctypes signatures (mirrors include/fd.h).
_c_i32, _c_i64, _c_sz, _c_vp, _c_f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
SIGNATURES = {
    "fd_status_string": (ctypes.c_char_p, [_c_i32]),
    "fd_last_error_message": (ctypes.c_char_p, []),
    "fd_version": (_c_i32, []),
    "fd_plan_splits": (_c_i32, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _c_i32, _c_i32]),
    "fd_device_cu_count": (_c_i32, [ctypes.POINTER(_c_i32)]),
    "fd_decode_attn_workspace_size": (_c_i32, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _c_i32, _c_i32,
                                               ctypes.POINTER(_c_sz)]),
    "fd_decode_attn": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _c_i32,
                                _c_i32, _c_vp, _c_i32, _c_vp, _c_f32, _c_vp, _c_sz, _c_vp]),
    "fd_decode_attn_noalloc": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64,
                                        _c_i32, _c_i32, _c_vp, _c_i32, _c_vp, _c_f32, _c_vp]),
    "fd_decode_attn_fp8": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32,
                                    _c_i64, _c_i32, _c_vp, _c_i32, _c_vp, _c_f32, _c_vp, _c_sz, _c_vp]),
    "fd_decode_attn_paged": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32,
                                      _c_i32, _c_i64, _c_i32, _c_i32, _c_i32, _c_vp, _c_i32, _c_vp, _c_f32,
                                      _c_vp, _c_sz, _c_vp]),
    "fd_bifurcated_attn_workspace_size": (_c_i32, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _c_i64, _c_i32,
                                                   ctypes.POINTER(_c_sz)]),
    "fd_bifurcated_attn": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32,
                                    _c_i64, _c_i64, _c_i32, _c_vp, _c_i32, _c_vp, _c_f32, _c_vp, _c_sz, _c_vp]),
    "fd_prefill_attn": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _c_i32,
                                 _c_vp, _c_i32, _c_vp, _c_f32, _c_vp]),
    "fd_lse_combine": (_c_i32, [_c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_vp, _c_i32, _c_vp, _c_vp]),
    "fd_piece_tile_rows": (_c_i32, [_c_i32, _c_i32, _c_i32, _c_i32]),
    "fd_decode_attn_partials": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64,
                                         _c_i32, _c_i32, _c_i32, _c_vp, _c_vp, _c_f32, _c_vp]),
    "fd_read_probe": (_c_i32, [_c_vp, _c_sz, _c_vp, _c_vp]),
    "fd_testing_decode_attn": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32,
                                        _c_i64, _c_i32, _c_i32, _c_vp, _c_i32, _c_vp, _c_f32, _c_vp, _c_sz, _c_vp,
                                        _c_i32]),
}



class FdTensor(ctypes.Structure):
    """fd_tensor (include/fd.h): device pointer, fd_dtype, ndim, shape[4], stride[4] (elements)."""
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


_P_T = ctypes.POINTER(FdTensor)
SIGNATURES.update({
    "fd_set_validation": (_c_i32, [_c_i32]),
    "fd_validation_enabled": (_c_i32, []),
    "fd_decode_attn_strided": (_c_i32, [_P_T, _P_T, _P_T, _c_vp, _c_vp, _c_vp, _c_i32, _P_T, _c_vp, _c_f32, _c_vp,
                                        _c_sz, _c_vp]),
    "fd_bifurcated_attn_strided": (_c_i32, [_P_T, _P_T, _P_T, _P_T, _P_T, _c_vp, _P_T, _c_vp, _c_f32, _c_vp, _c_sz,
                                            _c_vp]),
    "fd_bifurcated_attn_paged": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32,
                                          _c_i32, _c_i64, _c_i32, _c_i64, _c_i32, _c_i32, _c_vp, _c_i32, _c_vp, _c_f32,
                                          _c_vp, _c_sz, _c_vp]),
})

_lib = None


class FdError(RuntimeError):
    """A non-OK fd_status, with the library's message."""

    def __init__(self, status, message):
        super().__init__(f"{status_name(status)}: {message}")
        self.status = status


def load(path=LIB_PATH):
    """Load libfd.so (once) and attach the ctypes signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing; build it with `python -m decode_attention_06_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_name(status):
    return load().fd_status_string(int(status)).decode()


def _check(status):
    if status != FD_OK:
        raise FdError(status, load().fd_last_error_message().decode())


def plan_splits(batch, q_heads, kv_heads, head_dim, max_len, dtype, n_cu):
    """fd_plan_splits: host-only split planner (-1 for invalid arguments)."""
    return load().fd_plan_splits(batch, q_heads, kv_heads, head_dim, max_len, dtype, n_cu)


def device_cu_count():
    n = _c_i32(0)
    _check(load().fd_device_cu_count(ctypes.byref(n)))
    return n.value


def _torch():
    import torch

    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return FD_F32
    if t.dtype == torch.bfloat16:
        return FD_BF16
    raise FdError(FD_ERR_UNSUPPORTED, f"dtype {t.dtype} not supported (float32 or bfloat16)")


def _dev_ptr(t, name):
    if not t.is_cuda:
        raise FdError(FD_ERR_INVALID_ARG, f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise FdError(FD_ERR_INVALID_ARG, f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _opt_ptr(t, name):
    return None if t is None else _dev_ptr(t, name)


def decode_workspace_size(batch, q_heads, kv_heads, head_dim, max_len, dtype, n_splits=0):
    n = _c_sz(0)
    _check(load().fd_decode_attn_workspace_size(batch, q_heads, kv_heads, head_dim, max_len, dtype,
                                                n_splits, ctypes.byref(n)))
    return n.value


def decode_attn(q, k, v, lens=None, n_splits=0, out=None, out_dtype=None, scale=0.0,
                return_lse=False, workspace=None, stream=None):
    """Split-KV decode attention (fd_decode_attn).

    q [B, Hq, D]; k, v [B, Hkv, Lmax, D] (same dtype: float32 or bfloat16);
    lens int32 [B] on the device or None.  Returns out [B, Hq, D] (dtype of q
    unless out/out_dtype say otherwise), and the natural-log lse [B, Hq]
    float32 when return_lse.
    """
    torch = _torch()
    lib = load()
    if q.dim() != 3 or k.dim() != 4 or v.shape != k.shape:
        raise FdError(FD_ERR_INVALID_ARG, "expected q [B,Hq,D] and k, v [B,Hkv,Lmax,D]")
    B, Hq, D = q.shape
    _, Hkv, Lmax, Dk = k.shape
    if k.shape[0] != B or Dk != D:
        raise FdError(FD_ERR_INVALID_ARG, f"k shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    dt = _dtype_code(q)
    if _dtype_code(k) != dt or _dtype_code(v) != dt:
        raise FdError(FD_ERR_UNSUPPORTED, "q, k and v must share one dtype")
    if lens is not None:
        if lens.dtype != torch.int32 or lens.shape != (B,):
            raise FdError(FD_ERR_INVALID_ARG, "lens must be int32 [B]")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype or q.dtype, device=q.device)
    if tuple(out.shape) != (B, Hq, D):
        raise FdError(FD_ERR_INVALID_ARG, "out must be [B, Hq, D]")
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if return_lse else None
    if workspace is None:
        nbytes = decode_workspace_size(B, Hq, Hkv, D, Lmax, dt, n_splits)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _check(lib.fd_decode_attn(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _opt_ptr(lens, "lens"),
                              B, Hq, Hkv, D, Lmax, dt, int(n_splits), _dev_ptr(out, "out"), _dtype_code(out),
                              _opt_ptr(lse, "lse"), float(scale), _dev_ptr(workspace, "workspace"),
                              workspace.numel() * workspace.element_size(), _stream(stream)))
    return (out, lse) if return_lse else out


def decode_attn_noalloc(q, k, v, lens=None, n_splits=0, out=None, out_dtype=None, scale=0.0,
                        return_lse=False, stream=None):
    """fd_decode_attn_noalloc: decode_attn with the partials in the library's
    fixed per-GPU array (no workspace); calls on one GPU must not overlap."""
    torch = _torch()
    lib = load()
    if q.dim() != 3 or k.dim() != 4 or v.shape != k.shape:
        raise FdError(FD_ERR_INVALID_ARG, "expected q [B,Hq,D] and k, v [B,Hkv,Lmax,D]")
    B, Hq, D = q.shape
    _, Hkv, Lmax, Dk = k.shape
    if k.shape[0] != B or Dk != D:
        raise FdError(FD_ERR_INVALID_ARG, f"k shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    dt = _dtype_code(q)
    if _dtype_code(k) != dt or _dtype_code(v) != dt:
        raise FdError(FD_ERR_UNSUPPORTED, "q, k and v must share one dtype")
    if lens is not None and (lens.dtype != torch.int32 or lens.shape != (B,)):
        raise FdError(FD_ERR_INVALID_ARG, "lens must be int32 [B]")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype or q.dtype, device=q.device)
    if tuple(out.shape) != (B, Hq, D):
        raise FdError(FD_ERR_INVALID_ARG, "out must be [B, Hq, D]")
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if return_lse else None
    _check(lib.fd_decode_attn_noalloc(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _opt_ptr(lens, "lens"),
                                      B, Hq, Hkv, D, Lmax, dt, int(n_splits), _dev_ptr(out, "out"),
                                      _dtype_code(out), _opt_ptr(lse, "lse"), float(scale), _stream(stream)))
    return (out, lse) if return_lse else out


def _fp8_codes(t, name):
    torch = _torch()
    if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise FdError(FD_ERR_UNSUPPORTED, f"{name} must hold E4M3 codes (uint8 or float8_e4m3fn)")
    return _dev_ptr(t, name)


def decode_attn_fp8(q, k, v, k_scale=None, v_scale=None, lens=None, n_splits=0, out=None, out_dtype=None,
                    scale=0.0, return_lse=False, workspace=None, stream=None):
    """Split-KV decode attention over an E4M3 KV cache (fd_decode_attn_fp8).

    q bf16 [B, Hq, D]; k, v [B, Hkv, Lmax, D] E4M3 codes (uint8 or
    float8_e4m3fn); k_scale, v_scale float32 [Hkv] on the device or None
    (= 1): cache value = code value * scale of its KV head.
    """
    torch = _torch()
    lib = load()
    if q.dim() != 3 or k.dim() != 4 or v.shape != k.shape:
        raise FdError(FD_ERR_INVALID_ARG, "expected q [B,Hq,D] and k, v [B,Hkv,Lmax,D]")
    B, Hq, D = q.shape
    _, Hkv, Lmax, Dk = k.shape
    if k.shape[0] != B or Dk != D:
        raise FdError(FD_ERR_INVALID_ARG, f"k shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    if q.dtype != torch.bfloat16:
        raise FdError(FD_ERR_UNSUPPORTED, "the query of an E4M3 cache is bf16")
    for sc, name in ((k_scale, "k_scale"), (v_scale, "v_scale")):
        if sc is not None and (sc.dtype != torch.float32 or tuple(sc.shape) != (Hkv,)):
            raise FdError(FD_ERR_INVALID_ARG, f"{name} must be float32 [Hkv]")
    if lens is not None and (lens.dtype != torch.int32 or lens.shape != (B,)):
        raise FdError(FD_ERR_INVALID_ARG, "lens must be int32 [B]")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype or q.dtype, device=q.device)
    if tuple(out.shape) != (B, Hq, D):
        raise FdError(FD_ERR_INVALID_ARG, "out must be [B, Hq, D]")
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if return_lse else None
    if workspace is None:
        nbytes = decode_workspace_size(B, Hq, Hkv, D, Lmax, FD_FP8_E4M3, n_splits)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _check(lib.fd_decode_attn_fp8(_dev_ptr(q, "q"), _fp8_codes(k, "k"), _fp8_codes(v, "v"),
                                  _opt_ptr(k_scale, "k_scale"), _opt_ptr(v_scale, "v_scale"), _opt_ptr(lens, "lens"),
                                  B, Hq, Hkv, D, Lmax, int(n_splits), _dev_ptr(out, "out"), _dtype_code(out),
                                  _opt_ptr(lse, "lse"), float(scale), _dev_ptr(workspace, "workspace"),
                                  workspace.numel() * workspace.element_size(), _stream(stream)))
    return (out, lse) if return_lse else out


def decode_attn_paged(q, k_pages, v_pages, block_table, lens=None, n_splits=0, out=None, out_dtype=None,
                      scale=0.0, return_lse=False, workspace=None, stream=None):
    """Split-KV decode attention over a paged KV cache (fd_decode_attn_paged).

    q [B, Hq, D]; k_pages, v_pages [num_pages, Hkv, page_size, D];
    block_table int32 [B, max_pages_per_seq] of page ids on the device; lens
    int32 [B] on the device or None (= max_pages_per_seq * page_size).
    """
    torch = _torch()
    lib = load()
    if q.dim() != 3 or k_pages.dim() != 4 or v_pages.shape != k_pages.shape or block_table.dim() != 2:
        raise FdError(FD_ERR_INVALID_ARG,
                      "expected q [B,Hq,D], k_pages, v_pages [pages,Hkv,page_size,D], block_table [B,max_pages]")
    B, Hq, D = q.shape
    n_pages, Hkv, page_size, Dk = k_pages.shape
    max_pages = block_table.shape[1]
    if Dk != D or block_table.shape[0] != B or block_table.dtype != torch.int32:
        raise FdError(FD_ERR_INVALID_ARG, "paged shapes do not match q, or block_table is not int32 [B, *]")
    dt = _dtype_code(q)
    if _dtype_code(k_pages) != dt or _dtype_code(v_pages) != dt:
        raise FdError(FD_ERR_UNSUPPORTED, "q, k and v must share one dtype")
    if lens is not None and (lens.dtype != torch.int32 or lens.shape != (B,)):
        raise FdError(FD_ERR_INVALID_ARG, "lens must be int32 [B]")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype or q.dtype, device=q.device)
    if tuple(out.shape) != (B, Hq, D):
        raise FdError(FD_ERR_INVALID_ARG, "out must be [B, Hq, D]")
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if return_lse else None
    if workspace is None:
        nbytes = decode_workspace_size(B, Hq, Hkv, D, max_pages * page_size, dt, n_splits)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _check(lib.fd_decode_attn_paged(_dev_ptr(q, "q"), _dev_ptr(k_pages, "k_pages"), _dev_ptr(v_pages, "v_pages"),
                                    _dev_ptr(block_table, "block_table"), _opt_ptr(lens, "lens"), B, Hq, Hkv, D,
                                    page_size, n_pages, max_pages, dt, int(n_splits), _dev_ptr(out, "out"),
                                    _dtype_code(out), _opt_ptr(lse, "lse"), float(scale),
                                    _dev_ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                                    _stream(stream)))
    return (out, lse) if return_lse else out


def bifurcated_workspace_size(samples, q_heads, kv_heads, head_dim, ctx_len, dec_max_len, dtype):
    n = _c_sz(0)
    _check(load().fd_bifurcated_attn_workspace_size(samples, q_heads, kv_heads, head_dim, ctx_len,
                                                    dec_max_len, dtype, ctypes.byref(n)))
    return n.value


def bifurcated_attn(q, k_ctx, v_ctx, k_dec, v_dec, dec_lens=None, out=None, out_dtype=None, scale=0.0,
                    return_lse=False, workspace=None, stream=None):
    """Bifurcated single-context batch-sampling attention (fd_bifurcated_attn).

    q [S, Hq, D]; k_ctx, v_ctx [Hkv, Lc, D]; k_dec, v_dec [S, Hkv, Ldmax, D];
    dec_lens int32 [S] (0..Ldmax) or None.
    """
    torch = _torch()
    lib = load()
    if q.dim() != 3 or k_ctx.dim() != 3 or k_dec.dim() != 4:
        raise FdError(FD_ERR_INVALID_ARG, "expected q [S,Hq,D], k_ctx [Hkv,Lc,D], k_dec [S,Hkv,Ldmax,D]")
    S, Hq, D = q.shape
    Hkv, Lc, _ = k_ctx.shape
    Ld = k_dec.shape[2]
    if (v_ctx.shape != k_ctx.shape or v_dec.shape != k_dec.shape or k_ctx.shape[2] != D
            or tuple(k_dec.shape) != (S, Hkv, Ld, D)):
        raise FdError(FD_ERR_INVALID_ARG, "bifurcated shapes do not match")
    dt = _dtype_code(q)
    for t in (k_ctx, v_ctx, k_dec, v_dec):
        if _dtype_code(t) != dt:
            raise FdError(FD_ERR_UNSUPPORTED, "all inputs must share one dtype")
    if dec_lens is not None and (dec_lens.dtype != torch.int32 or dec_lens.shape != (S,)):
        raise FdError(FD_ERR_INVALID_ARG, "dec_lens must be int32 [S]")
    if out is None:
        out = torch.empty((S, Hq, D), dtype=out_dtype or q.dtype, device=q.device)
    lse = torch.empty((S, Hq), dtype=torch.float32, device=q.device) if return_lse else None
    if workspace is None:
        nbytes = bifurcated_workspace_size(S, Hq, Hkv, D, Lc, Ld, dt)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _check(lib.fd_bifurcated_attn(_dev_ptr(q, "q"), _dev_ptr(k_ctx, "k_ctx"), _dev_ptr(v_ctx, "v_ctx"),
                                  _dev_ptr(k_dec, "k_dec"), _dev_ptr(v_dec, "v_dec"),
                                  _opt_ptr(dec_lens, "dec_lens"), S, Hq, Hkv, D, Lc, Ld, dt,
                                  _dev_ptr(out, "out"), _dtype_code(out), _opt_ptr(lse, "lse"),
                                  float(scale), _dev_ptr(workspace, "workspace"),
                                  workspace.numel() * workspace.element_size(), _stream(stream)))
    return (out, lse) if return_lse else out


def prefill_attn(q, k, v, lens=None, out=None, out_dtype=None, scale=0.0, return_lse=False, stream=None):
    """Causal prefill attention (fd_prefill_attn).

    q [B, Hq, Lmax, D]; k, v [B, Hkv, Lmax, D] (bf16, D 128); lens int32 [B]
    on the device or None.  Position p attends to cache rows [0, p].
    Returns out [B, Hq, Lmax, D] (positions past lens[b] untouched) and the
    natural-log lse [B, Hq, Lmax] when return_lse.
    """
    torch = _torch()
    lib = load()
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise FdError(FD_ERR_INVALID_ARG, "expected q [B,Hq,Lmax,D] and k, v [B,Hkv,Lmax,D]")
    B, Hq, Lmax, D = q.shape
    if k.shape[0] != B or k.shape[2] != Lmax or k.shape[3] != D:
        raise FdError(FD_ERR_INVALID_ARG, f"k shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    Hkv = k.shape[1]
    dt = _dtype_code(q)
    if _dtype_code(k) != dt or _dtype_code(v) != dt:
        raise FdError(FD_ERR_UNSUPPORTED, "q, k and v must share one dtype")
    if lens is not None and (lens.dtype != torch.int32 or lens.shape != (B,)):
        raise FdError(FD_ERR_INVALID_ARG, "lens must be int32 [B]")
    if out is None:
        out = torch.zeros((B, Hq, Lmax, D), dtype=out_dtype or q.dtype, device=q.device)
    if tuple(out.shape) != (B, Hq, Lmax, D):
        raise FdError(FD_ERR_INVALID_ARG, "out must be [B, Hq, Lmax, D]")
    lse = torch.full((B, Hq, Lmax), float("nan"), dtype=torch.float32, device=q.device) if return_lse else None
    _check(lib.fd_prefill_attn(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _opt_ptr(lens, "lens"), B, Hq,
                               Hkv, D, Lmax, dt, _dev_ptr(out, "out"), _dtype_code(out), _opt_ptr(lse, "lse"),
                               float(scale), _stream(stream)))
    return (out, lse) if return_lse else out


def lse_combine(o_part, lse_part, out=None, out_dtype=None, return_lse=False, stream=None):
    """fd_lse_combine: o_part [rows, P, D] fp32, lse_part [rows, P] fp32 -> out [rows, D]."""
    torch = _torch()
    lib = load()
    rows, P, D = o_part.shape
    if o_part.dtype != torch.float32 or lse_part.dtype != torch.float32 or tuple(lse_part.shape) != (rows, P):
        raise FdError(FD_ERR_INVALID_ARG, "o_part [rows,P,D] and lse_part [rows,P] must be float32")
    if out is None:
        out = torch.empty((rows, D), dtype=out_dtype or torch.float32, device=o_part.device)
    lse = torch.empty((rows,), dtype=torch.float32, device=o_part.device) if return_lse else None
    _check(lib.fd_lse_combine(_dev_ptr(o_part, "o_part"), _dev_ptr(lse_part, "lse_part"), rows, P, D,
                              _dev_ptr(out, "out"), _dtype_code(out), _opt_ptr(lse, "lse"), _stream(stream)))
    return (out, lse) if return_lse else out


def piece_tile_rows(q_heads, kv_heads, head_dim, dtype):
    """fd_piece_tile_rows: rows per tile of the interleaved piece layout (-1: invalid)."""
    return load().fd_piece_tile_rows(q_heads, kv_heads, head_dim, dtype)


def decode_attn_partials(q, k, v, n_splits, lens=None, o_part=None, lse_part=None, scale=0.0, stream=None,
                         layout=FD_PIECES_CONTIGUOUS):
    """fd_decode_attn_partials: per-piece outputs [B*Hq, n_splits, D] and lse [B*Hq, n_splits].
    layout: FD_PIECES_CONTIGUOUS (0) or FD_PIECES_INTERLEAVED (1)."""
    torch = _torch()
    lib = load()
    B, Hq, D = q.shape
    _, Hkv, Lmax, _ = k.shape
    dt = _dtype_code(q)
    rows = B * Hq
    if o_part is None:
        o_part = torch.empty((rows, n_splits, D), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((rows, n_splits), dtype=torch.float32, device=q.device)
    _check(lib.fd_decode_attn_partials(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                                       _opt_ptr(lens, "lens"), B, Hq, Hkv, D, Lmax, dt, int(n_splits),
                                       int(layout), _dev_ptr(o_part, "o_part"), _dev_ptr(lse_part, "lse_part"),
                                       float(scale), _stream(stream)))
    return o_part, lse_part


def testing_decode_attn(q, k, v, kernel, k_scale=None, v_scale=None, lens=None, n_splits=0, out=None,
                        out_dtype=None, scale=0.0, return_lse=False, stream=None):
    """fd_testing_decode_attn (test hook): decode attention on the named
    partial kernel ('auto', 'valu' or 'mfma').  k, v are bf16/fp32 like q,
    or E4M3 codes (uint8 / float8_e4m3fn) with a bf16 q and optional scales."""
    torch = _torch()
    lib = load()
    B, Hq, D = q.shape
    _, Hkv, Lmax, _ = k.shape
    fp8 = k.dtype in (torch.uint8, torch.float8_e4m3fn)
    dt = FD_FP8_E4M3 if fp8 else _dtype_code(q)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype or q.dtype, device=q.device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if return_lse else None
    nbytes = decode_workspace_size(B, Hq, Hkv, D, Lmax, dt, n_splits)
    workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    kp = _fp8_codes(k, "k") if fp8 else _dev_ptr(k, "k")
    vp = _fp8_codes(v, "v") if fp8 else _dev_ptr(v, "v")
    _check(lib.fd_testing_decode_attn(_dev_ptr(q, "q"), kp, vp, _opt_ptr(k_scale, "k_scale"),
                                      _opt_ptr(v_scale, "v_scale"), _opt_ptr(lens, "lens"), B, Hq, Hkv, D, Lmax, dt,
                                      int(n_splits), _dev_ptr(out, "out"), _dtype_code(out), _opt_ptr(lse, "lse"),
                                      float(scale), _dev_ptr(workspace, "workspace"), workspace.numel(),
                                      _stream(stream), TESTING_KERNELS[kernel]))
    return (out, lse) if return_lse else out


def _tensor_desc(t, name, dtype=None):
    """fd_tensor describing a device tensor of any strides (no copy)."""
    if not t.is_cuda:
        raise FdError(FD_ERR_INVALID_ARG, f"{name} must be a device tensor")
    d = FdTensor()
    d.data = t.data_ptr()
    d.dtype = _dtype_code(t) if dtype is None else dtype
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def decode_attn_strided(q, k, v, lens=None, n_splits=0, out=None, out_dtype=None, scale=0.0, k_scale=None,
                        v_scale=None, return_lse=False, workspace=None, stream=None):
    """fd_decode_attn_strided: q [B, Hq, D], k, v logical [B, Hkv, Lmax, D] and
    out [B, Hq, D] as views of any strides (last dimension contiguous), e.g.
    a token-major cache passed as kt.permute(0, 2, 1, 3).  k, v may be E4M3
    codes (uint8 / float8_e4m3fn) with a bf16 q and optional scales."""
    torch = _torch()
    lib = load()
    B, Hq, D = q.shape
    _, Hkv, Lmax, _ = k.shape
    fp8 = k.dtype in (torch.uint8, torch.float8_e4m3fn)
    dt = FD_FP8_E4M3 if fp8 else _dtype_code(k)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype or q.dtype, device=q.device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if return_lse else None
    if workspace is None:
        nbytes = decode_workspace_size(B, Hq, Hkv, D, Lmax, dt, n_splits)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    qd, kd, vd, od = (_tensor_desc(q, "q"), _tensor_desc(k, "k", dt), _tensor_desc(v, "v", dt),
                      _tensor_desc(out, "out"))
    _check(lib.fd_decode_attn_strided(ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(vd),
                                      _opt_ptr(k_scale, "k_scale"), _opt_ptr(v_scale, "v_scale"),
                                      _opt_ptr(lens, "lens"), int(n_splits), ctypes.byref(od), _opt_ptr(lse, "lse"),
                                      float(scale), _dev_ptr(workspace, "workspace"),
                                      workspace.numel() * workspace.element_size(), _stream(stream)))
    return (out, lse) if return_lse else out


def bifurcated_attn_strided(q, k_ctx, v_ctx, k_dec, v_dec, dec_lens=None, out=None, out_dtype=None, scale=0.0,
                            return_lse=False, workspace=None, stream=None):
    """fd_bifurcated_attn_strided: q [S, Hq, D], k_ctx, v_ctx logical [Hkv, Lc, D],
    k_dec, v_dec logical [S, Hkv, Ldmax, D], out [S, Hq, D], as views of any
    strides (last dimension contiguous)."""
    torch = _torch()
    lib = load()
    S, Hq, D = q.shape
    Hkv, Lc, _ = k_ctx.shape
    Ld = k_dec.shape[2]
    if out is None:
        out = torch.empty((S, Hq, D), dtype=out_dtype or q.dtype, device=q.device)
    lse = torch.empty((S, Hq), dtype=torch.float32, device=q.device) if return_lse else None
    if workspace is None:
        nbytes = bifurcated_workspace_size(S, Hq, Hkv, D, Lc, Ld, _dtype_code(q))
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    descs = [_tensor_desc(t, n) for t, n in ((q, "q"), (k_ctx, "k_ctx"), (v_ctx, "v_ctx"), (k_dec, "k_dec"),
                                              (v_dec, "v_dec"), (out, "out"))]
    qd, kcd, vcd, kdd, vdd, od = descs
    _check(lib.fd_bifurcated_attn_strided(ctypes.byref(qd), ctypes.byref(kcd), ctypes.byref(vcd), ctypes.byref(kdd),
                                          ctypes.byref(vdd), _opt_ptr(dec_lens, "dec_lens"), ctypes.byref(od),
                                          _opt_ptr(lse, "lse"), float(scale), _dev_ptr(workspace, "workspace"),
                                          workspace.numel() * workspace.element_size(), _stream(stream)))
    return (out, lse) if return_lse else out


def bifurcated_attn_paged(q, k_ctx, v_ctx, k_pages, v_pages, block_table, dec_lens=None, out=None, out_dtype=None,
                          scale=0.0, return_lse=False, workspace=None, stream=None):
    """fd_bifurcated_attn_paged: q [S, Hq, D]; k_ctx, v_ctx [Hkv, Lc, D] dense;
    the decode rows in k_pages, v_pages [num_pages, Hkv, page_size, D] found
    through block_table int32 [S, max_pages_per_seq]; dec_lens int32 [S]."""
    torch = _torch()
    lib = load()
    S, Hq, D = q.shape
    Hkv, Lc, _ = k_ctx.shape
    n_pages, _, page_size, _ = k_pages.shape
    max_pages = block_table.shape[1]
    if block_table.dtype != torch.int32 or tuple(block_table.shape[:1]) != (S,):
        raise FdError(FD_ERR_INVALID_ARG, "block_table must be int32 [S, max_pages_per_seq]")
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty((S, Hq, D), dtype=out_dtype or q.dtype, device=q.device)
    lse = torch.empty((S, Hq), dtype=torch.float32, device=q.device) if return_lse else None
    if workspace is None:
        nbytes = bifurcated_workspace_size(S, Hq, Hkv, D, Lc, max_pages * page_size, dt)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _check(lib.fd_bifurcated_attn_paged(_dev_ptr(q, "q"), _dev_ptr(k_ctx, "k_ctx"), _dev_ptr(v_ctx, "v_ctx"),
                                        _dev_ptr(k_pages, "k_pages"), _dev_ptr(v_pages, "v_pages"),
                                        _dev_ptr(block_table, "block_table"), _opt_ptr(dec_lens, "dec_lens"), S, Hq,
                                        Hkv, D, Lc, page_size, n_pages, max_pages, dt, _dev_ptr(out, "out"),
                                        _dtype_code(out), _opt_ptr(lse, "lse"), float(scale),
                                        _dev_ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                                        _stream(stream)))
    return (out, lse) if return_lse else out


def set_validation(on):
    """fd_set_validation: device-side checks of lens / block tables before each call."""
    _check(load().fd_set_validation(1 if on else 0))


def validation_enabled():
    return bool(load().fd_validation_enabled())


def read_probe(buf, sink, stream=None):
    """fd_read_probe: stream a device buffer once (HBM read-rate measurement)."""
    nbytes = buf.numel() * buf.element_size()
    _check(load().fd_read_probe(_dev_ptr(buf, "buf"), nbytes, _dev_ptr(sink, "sink"), _stream(stream)))
