"""Thin ctypes binding of libpoetx (include/poetx.h).

Argument marshalling only: every function takes torch tensors that already
live on the GPU (or None for optional arguments), passes their device pointers
and the current HIP stream to the library, and raises PoetxError on a non-zero
status.  No computation happens here and there is no fallback: if the shared
library is missing, load() raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpoetx.so")

POETX_OK, POETX_ERR_INVALID_ARG, POETX_ERR_SHAPE, POETX_ERR_UNSUPPORTED, POETX_ERR_WORKSPACE, POETX_ERR_HIP = range(6)
POETX_F32, POETX_BF16 = 0, 1
POETX_FAST, POETX_MEM, POETX_FOUR_PERM, POETX_WEIGHT_CENTRIC, POETX_MEM_Q8 = 0, 1, 2, 3, 4
POETX_GEMM_NT, POETX_GEMM_NN, POETX_GEMM_TN = 0, 1, 2

EXPORTS = [
    "poetx_version", "poetx_status_string", "poetx_last_hip_error",
    "poetx_skew_unpack", "poetx_skew_pack",
    "poetx_cnp_fwd_workspace_bytes", "poetx_cnp_fwd",
    "poetx_cnp_bwd_workspace_bytes", "poetx_cnp_bwd",
    "poetx_cnp_saved_bytes", "poetx_cnp_fwd_save", "poetx_cnp_bwd_saved",
    "poetx_permute", "poetx_prepermute",
    "poetx_check_perm_workspace_bytes", "poetx_check_perm",
    "poetx_linear_saved_bytes", "poetx_linear_fwd_workspace_bytes", "poetx_linear_fwd", "poetx_linear_fwd_noalloc",
    "poetx_linear_bwd_workspace_bytes", "poetx_linear_bwd",
    "poetx_group_saved_bytes", "poetx_group_fwd_workspace_bytes", "poetx_group_fwd",
    "poetx_group_bwd_workspace_bytes", "poetx_group_bwd",
    "poetx_merge_workspace_bytes", "poetx_merge",
    "poetx_qweight_bytes", "poetx_quantize_weight", "poetx_dequantize_weight",
    "poetx_gemm", "poetx_block_apply", "poetx_dense_fold_r", "poetx_block_grad_workspace_bytes", "poetx_block_grad",
    "poetx_adamw_step", "poetx_adamw_reset",
]


class PoetxError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str, hip: str):
        super().__init__(f"{fn} failed: {text} ({status}){': ' + hip if hip else ''}")
        self.status = status


class LinearDesc(C.Structure):
    _fields_ = [("T", C.c_int64), ("m", C.c_int64), ("n", C.c_int64), ("b", C.c_int64),
                ("k", C.c_int32), ("dtype", C.c_int32), ("variant", C.c_int32), ("reserved", C.c_int32)]


POETX_MAX_GROUP = 8


class GroupDesc(C.Structure):
    _fields_ = [("T", C.c_int64), ("n", C.c_int64), ("b", C.c_int64), ("k", C.c_int32), ("dtype", C.c_int32),
                ("variant", C.c_int32), ("count", C.c_int32), ("reserved", C.c_int32), ("pad", C.c_int32),
                ("m", C.c_int64 * POETX_MAX_GROUP)]


class AdamwParams(C.Structure):
    _fields_ = [("lr", C.c_double), ("gamma", C.c_double), ("beta1", C.c_double), ("beta2", C.c_double),
                ("eps", C.c_double), ("weight_decay", C.c_double)]


_lib: Optional[C.CDLL] = None
_VP, _I64, _I32, _SZ = C.c_void_p, C.c_int64, C.c_int, C.c_size_t
_DP = C.POINTER(LinearDesc)
_GP = C.POINTER(GroupDesc)

_SIGS = {
    "poetx_version": ([], C.c_char_p),
    "poetx_status_string": ([_I32], C.c_char_p),
    "poetx_last_hip_error": ([], C.c_char_p),
    "poetx_skew_unpack": ([_VP, _VP, _I32, _I64, _I64, _VP], _I32),
    "poetx_skew_pack": ([_VP, _VP, _I64, _I64, _VP], _I32),
    "poetx_cnp_fwd_workspace_bytes": ([_I64, _I64, _I32, _I32], _SZ),
    "poetx_cnp_fwd": ([_VP, _I64, _I64, _I32, _VP, _I32, _VP, _SZ, _VP], _I32),
    "poetx_cnp_bwd_workspace_bytes": ([_I64, _I64, _I32, _I32], _SZ),
    "poetx_cnp_bwd": ([_VP, _VP, _I64, _I64, _I32, _VP, _I32, _VP, _SZ, _VP], _I32),
    "poetx_cnp_saved_bytes": ([_I64, _I64, _I32, _I32], _SZ),
    "poetx_cnp_fwd_save": ([_VP, _I64, _I64, _I32, _VP, _I32, _VP, _SZ, _VP, _SZ, _VP], _I32),
    "poetx_cnp_bwd_saved": ([_VP, _VP, _I64, _I64, _I32, _VP, _I32, _VP, _SZ, _VP, _SZ, _VP], _I32),
    "poetx_permute": ([_VP, _VP, _I32, _I64, _I64, _VP, _VP, _I32, _VP], _I32),
    "poetx_prepermute": ([_VP, _VP, _I32, _I64, _I64, _VP, _VP, _VP], _I32),
    "poetx_check_perm_workspace_bytes": ([_I64], _SZ),
    "poetx_check_perm": ([_VP, _I64, _VP, _VP, _SZ, _VP], _I32),
    "poetx_linear_saved_bytes": ([_DP], _SZ),
    "poetx_linear_fwd_workspace_bytes": ([_DP], _SZ),
    "poetx_linear_fwd": ([_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP], _I32),
    "poetx_linear_fwd_noalloc": ([_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP], _I32),
    "poetx_linear_bwd_workspace_bytes": ([_DP], _SZ),
    "poetx_linear_bwd": ([_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP], _I32),
    "poetx_group_saved_bytes": ([_GP], _SZ),
    "poetx_group_fwd_workspace_bytes": ([_GP], _SZ),
    "poetx_group_fwd": ([_GP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP], _I32),
    "poetx_group_bwd_workspace_bytes": ([_GP], _SZ),
    "poetx_group_bwd": ([_GP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP], _I32),
    "poetx_merge_workspace_bytes": ([_DP], _SZ),
    "poetx_qweight_bytes": ([_I64, _I64], _SZ),
    "poetx_quantize_weight": ([_VP, _I32, _I64, _I64, _VP, _VP], _I32),
    "poetx_dequantize_weight": ([_VP, _I64, _I64, _VP, _VP], _I32),
    "poetx_merge": ([_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP], _I32),
    "poetx_gemm": ([_I32, _I32, _I32, _I64, _I64, _I64, _I64, _VP, _I64, _I64, _VP, _I64, _I64, _VP, _I64, _I64,
                    _VP], _I32),
    "poetx_block_apply": ([_I32, _I32, _I64, _I64, _I64, _VP, _VP, _VP, _VP], _I32),
    "poetx_dense_fold_r": ([_I32, _I64, _I64, _I64, _I64, _VP, _VP, _VP, _VP, _VP, _VP], _I32),
    "poetx_block_grad_workspace_bytes": ([_I64, _I64, _I64, _I32], _SZ),
    "poetx_block_grad": ([_I32, _I64, _I64, _I64, _VP, _VP, _VP, _VP, _SZ, _VP], _I32),
    "poetx_adamw_step": ([_VP, _VP, _VP, _VP, _I64, _I64, C.POINTER(AdamwParams), _VP], _I32),
    "poetx_adamw_reset": ([_VP, _VP, _I64, _VP], _I32),
}


def load(path: str = LIB_PATH) -> C.CDLL:
    """Load libpoetx.so (built in-tree by build.py); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libpoetx is not built ({path} missing); run orthogonal_equivalence_poet_amd.build.build()")
    lib = C.CDLL(path)
    for name, (args, res) in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return POETX_BF16
    if t.dtype == torch.float32:
        return POETX_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check(fn: str, status: int) -> None:
    if status != POETX_OK:
        lib = load()
        raise PoetxError(fn, status, lib.poetx_status_string(status).decode(),
                         lib.poetx_last_hip_error().decode())


def _ws(ws):
    return (None, 0) if ws is None else (ws.data_ptr(), ws.numel() * ws.element_size())


def desc(T, m, n, b, k, dtype, variant) -> LinearDesc:
    return LinearDesc(int(T), int(m), int(n), int(b), int(k), int(dtype), int(variant), 0)


def workspace(nbytes: int, device="cuda"):
    """A device byte buffer of nbytes (torch plumbing); None when nbytes is 0."""
    import torch
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device) if nbytes else None


# ---------------------------------------------------------------- entry points
def poetx_version() -> str:
    return load().poetx_version().decode()


def poetx_skew_unpack(q, Q, nblk, b, stream=None):
    _check("poetx_skew_unpack", load().poetx_skew_unpack(_ptr(q), _ptr(Q), _dtype_code(Q), nblk, b, _stream(stream)))


def poetx_skew_pack(dQ, dq, nblk, b, stream=None):
    _check("poetx_skew_pack", load().poetx_skew_pack(_ptr(dQ), _ptr(dq), nblk, b, _stream(stream)))


def poetx_cnp_fwd_workspace_bytes(nblk, b, k, G_dtype) -> int:
    return load().poetx_cnp_fwd_workspace_bytes(nblk, b, k, G_dtype)


def poetx_cnp_fwd(q, nblk, b, k, G, ws=None, stream=None):
    p, nbytes = _ws(ws)
    _check("poetx_cnp_fwd", load().poetx_cnp_fwd(_ptr(q), nblk, b, k, _ptr(G), _dtype_code(G), p, nbytes,
                                                 _stream(stream)))


def poetx_cnp_bwd_workspace_bytes(nblk, b, k, dtype) -> int:
    return load().poetx_cnp_bwd_workspace_bytes(nblk, b, k, dtype)


def poetx_cnp_bwd(q, dG, nblk, b, k, dq, dtype, ws=None, stream=None):
    p, nbytes = _ws(ws)
    _check("poetx_cnp_bwd", load().poetx_cnp_bwd(_ptr(q), _ptr(dG), nblk, b, k, _ptr(dq), dtype, p, nbytes,
                                                 _stream(stream)))


def poetx_cnp_saved_bytes(nblk, b, k, dtype) -> int:
    return load().poetx_cnp_saved_bytes(nblk, b, k, dtype)


def poetx_cnp_fwd_save(q, nblk, b, k, G, saved, ws=None, stream=None):
    p, nbytes = _ws(ws)
    sp, sbytes = _ws(saved)
    _check("poetx_cnp_fwd_save", load().poetx_cnp_fwd_save(_ptr(q), nblk, b, k, _ptr(G), _dtype_code(G), sp, sbytes,
                                                           p, nbytes, _stream(stream)))


def poetx_cnp_bwd_saved(q, dG, nblk, b, k, dq, dtype, saved, ws=None, stream=None):
    p, nbytes = _ws(ws)
    sp, sbytes = _ws(saved)
    _check("poetx_cnp_bwd_saved", load().poetx_cnp_bwd_saved(_ptr(q), _ptr(dG), nblk, b, k, _ptr(dq), dtype, sp,
                                                             sbytes, p, nbytes, _stream(stream)))


def poetx_permute(src, dst, rows, cols, row_idx=None, col_idx=None, scatter_cols=False, stream=None):
    _check("poetx_permute", load().poetx_permute(_ptr(src), _ptr(dst), _dtype_code(dst), rows, cols, _ptr(row_idx),
                                                 _ptr(col_idx), int(bool(scatter_cols)), _stream(stream)))


def poetx_prepermute(W0, Wt, m, n, pi_R, pi_P, stream=None):
    _check("poetx_prepermute", load().poetx_prepermute(_ptr(W0), _ptr(Wt), _dtype_code(Wt), m, n, _ptr(pi_R),
                                                       _ptr(pi_P), _stream(stream)))


def poetx_check_perm_workspace_bytes(length) -> int:
    return load().poetx_check_perm_workspace_bytes(length)


def poetx_check_perm(pi, length, ok, ws=None, stream=None):
    p, nbytes = _ws(ws)
    _check("poetx_check_perm", load().poetx_check_perm(_ptr(pi), length, _ptr(ok), p, nbytes, _stream(stream)))


def poetx_linear_saved_bytes(d: LinearDesc) -> int:
    return load().poetx_linear_saved_bytes(C.byref(d))


def poetx_linear_fwd_workspace_bytes(d: LinearDesc) -> int:
    return load().poetx_linear_fwd_workspace_bytes(C.byref(d))


def poetx_linear_fwd(d: LinearDesc, x, Wt, G_R, G_P, pi_R, pi_P, y, saved=None, ws=None, stream=None):
    p, nbytes = _ws(ws)
    _check("poetx_linear_fwd", load().poetx_linear_fwd(C.byref(d), _ptr(x), _ptr(Wt), _ptr(G_R), _ptr(G_P),
                                                       _ptr(pi_R), _ptr(pi_P), _ptr(y), _ptr(saved), p, nbytes,
                                                       _stream(stream)))


def group_desc(T, n, b, k, dtype, variant, ms) -> GroupDesc:
    ms = [int(v) for v in ms]
    if not 1 <= len(ms) <= POETX_MAX_GROUP:
        raise ValueError(f"a group holds 1 to {POETX_MAX_GROUP} linears, got {len(ms)}")
    m = (C.c_int64 * POETX_MAX_GROUP)(*(ms + [0] * (POETX_MAX_GROUP - len(ms))))
    return GroupDesc(int(T), int(n), int(b), int(k), int(dtype), int(variant), len(ms), 0, 0, m)


def poetx_group_saved_bytes(g: GroupDesc) -> int:
    return load().poetx_group_saved_bytes(C.byref(g))


def poetx_group_fwd_workspace_bytes(g: GroupDesc) -> int:
    return load().poetx_group_fwd_workspace_bytes(C.byref(g))


def poetx_linear_fwd_noalloc(d: LinearDesc, x, Wt, G_R, G_P, pi_R, pi_P, y, saved=None, stream=None):
    _check("poetx_linear_fwd_noalloc", load().poetx_linear_fwd_noalloc(C.byref(d), _ptr(x), _ptr(Wt), _ptr(G_R),
                                                                       _ptr(G_P), _ptr(pi_R), _ptr(pi_P), _ptr(y),
                                                                       _ptr(saved), _stream(stream)))


POETX_NOALLOC_SCRATCH_BYTES = 64 << 20


def poetx_group_fwd(g: GroupDesc, x, Wt, G_R, G_P, pi_R, pi_P, y, saved=None, ws=None, stream=None):
    p, nbytes = _ws(ws)
    _check("poetx_group_fwd", load().poetx_group_fwd(C.byref(g), _ptr(x), _ptr(Wt), _ptr(G_R), _ptr(G_P),
                                                     _ptr(pi_R), _ptr(pi_P), _ptr(y), _ptr(saved), p, nbytes,
                                                     _stream(stream)))


def poetx_group_bwd_workspace_bytes(g: GroupDesc) -> int:
    return load().poetx_group_bwd_workspace_bytes(C.byref(g))


def poetx_group_bwd(g: GroupDesc, dy, x, Wt, G_R, G_P, pi_R, pi_P, saved, dx, dG_R, dG_P, ws=None, stream=None):
    p, nbytes = _ws(ws)
    _check("poetx_group_bwd", load().poetx_group_bwd(C.byref(g), _ptr(dy), _ptr(x), _ptr(Wt), _ptr(G_R),
                                                     _ptr(G_P), _ptr(pi_R), _ptr(pi_P), _ptr(saved), _ptr(dx),
                                                     _ptr(dG_R), _ptr(dG_P), p, nbytes, _stream(stream)))


def poetx_linear_bwd_workspace_bytes(d: LinearDesc) -> int:
    return load().poetx_linear_bwd_workspace_bytes(C.byref(d))


def poetx_linear_bwd(d: LinearDesc, dy, x, Wt, G_R, G_P, pi_R, pi_P, saved, dx, dG_R, dG_P, ws=None,
                     stream=None):
    p, nbytes = _ws(ws)
    _check("poetx_linear_bwd", load().poetx_linear_bwd(C.byref(d), _ptr(dy), _ptr(x), _ptr(Wt), _ptr(G_R),
                                                       _ptr(G_P), _ptr(pi_R), _ptr(pi_P), _ptr(saved), _ptr(dx),
                                                       _ptr(dG_R), _ptr(dG_P), p, nbytes, _stream(stream)))


def poetx_merge_workspace_bytes(d: LinearDesc) -> int:
    return load().poetx_merge_workspace_bytes(C.byref(d))


def poetx_merge(d: LinearDesc, Wt, q_R, q_P, pi_R_old, pi_P_old, pi_R_new, pi_P_new, ws=None, stream=None):
    p, nbytes = _ws(ws)
    _check("poetx_merge", load().poetx_merge(C.byref(d), _ptr(Wt), _ptr(q_R), _ptr(q_P), _ptr(pi_R_old),
                                             _ptr(pi_P_old), _ptr(pi_R_new), _ptr(pi_P_new), p, nbytes,
                                             _stream(stream)))


def poetx_qweight_bytes(m, n) -> int:
    return load().poetx_qweight_bytes(m, n)


def poetx_quantize_weight(W, m, n, Wq, stream=None):
    _check("poetx_quantize_weight", load().poetx_quantize_weight(_ptr(W), _dtype_code(W), m, n, _ptr(Wq),
                                                                 _stream(stream)))


def poetx_dequantize_weight(Wq, m, n, W, stream=None):
    _check("poetx_dequantize_weight", load().poetx_dequantize_weight(_ptr(Wq), m, n, _ptr(W), _stream(stream)))


def poetx_gemm(layout, A, B, C, M, N, K, batch=1, lda=None, ldb=None, ldc=None, strideA=0, strideB=0, strideC=0,
               dense=False, stream=None):
    lda = lda if lda is not None else (K if layout != POETX_GEMM_TN else M)
    ldb = ldb if ldb is not None else (K if layout == POETX_GEMM_NT else N)
    ldc = ldc if ldc is not None else N
    _check("poetx_gemm", load().poetx_gemm(layout, _dtype_code(C), int(bool(dense)), M, N, K, batch, _ptr(A), lda,
                                           strideA, _ptr(B), ldb, strideB, _ptr(C), ldc, strideC, _stream(stream)))


def poetx_block_apply(inp, G, out, T, d, b, transpose_G=True, stream=None):
    _check("poetx_block_apply", load().poetx_block_apply(_dtype_code(out), int(bool(transpose_G)), T, d, b, _ptr(inp),
                                                         _ptr(G), _ptr(out), _stream(stream)))


def poetx_dense_fold_r(h1, Wt, G_R, z, T, m, n, b, h2=None, stream=None):
    _check("poetx_dense_fold_r", load().poetx_dense_fold_r(_dtype_code(z), T, m, n, b, _ptr(h1), _ptr(Wt), _ptr(G_R),
                                                           _ptr(h2), _ptr(z), _stream(stream)))


def poetx_block_grad_workspace_bytes(T, d, b, dtype) -> int:
    return load().poetx_block_grad_workspace_bytes(T, d, b, dtype)


def poetx_block_grad(A, B, dG, T, d, b, ws=None, stream=None):
    p, nbytes = _ws(ws)
    _check("poetx_block_grad", load().poetx_block_grad(_dtype_code(A), T, d, b, _ptr(A), _ptr(B), _ptr(dG), p,
                                                       nbytes, _stream(stream)))


def adamw_params(lr, gamma=0.5, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0) -> AdamwParams:
    return AdamwParams(lr, gamma, beta1, beta2, eps, weight_decay)


def poetx_adamw_step(q, dq, m, v, count, step, params: AdamwParams, stream=None):
    _check("poetx_adamw_step", load().poetx_adamw_step(_ptr(q), _ptr(dq), _ptr(m), _ptr(v), count, step,
                                                       C.byref(params), _stream(stream)))


def poetx_adamw_reset(m, v, count, stream=None):
    _check("poetx_adamw_reset", load().poetx_adamw_reset(_ptr(m), _ptr(v), count, _stream(stream)))
