"""Thin ctypes binding of libcsa.so with the same names as the C ABI (include/csa.h).

Argument marshalling only: torch tensors are passed as raw device pointers, the stream
is torch's current HIP stream.  Every computation runs in the library's HIP kernels;
there is no fallback.  If the library is missing, loading raises.
"""
import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcsa.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "csa.h")

CSA_OK, CSA_ERR_NULL, CSA_ERR_ARG, CSA_ERR_UNSUPPORTED, CSA_ERR_WORKSPACE, CSA_ERR_LAUNCH = (
    0, -1, -2, -3, -4, -5)
CSA_F32, CSA_BF16, CSA_FP8_E4M3 = 0, 1, 2
CSA_SPARSE, CSA_DENSE, CSA_WINDOW = 0, 1, 2
CSA_TEACHER_NONE, CSA_TEACHER_SELECTED, CSA_TEACHER_DENSE = 0, 1, 2
CSA_OP_ATTN_FWD, CSA_OP_ATTN_BWD, CSA_OP_INDEXER_KL, CSA_OP_INDEXER_KL_CACHED = 1, 2, 3, 4

_DT = {torch.float32: CSA_F32, torch.bfloat16: CSA_BF16, torch.uint8: CSA_FP8_E4M3}


class CsaParams(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "total_tokens", "max_seqlen", "ratio", "window", "topk", "topk_cap",
        "heads", "head_dim", "idx_heads", "idx_dim")] + [("scale", ctypes.c_float)] + [
        (n, ctypes.c_int32) for n in ("mode", "teacher", "dtype", "idx_dtype", "rope_dim")] + [
        ("rope_theta", ctypes.c_float)]


class CsaError(RuntimeError):
    def __init__(self, name, status, msg):
        super().__init__(f"{name} failed with status {status}: {msg}")
        self.status = status


_lib = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_F = ctypes.c_float
_PP = ctypes.POINTER(CsaParams)

_SIGS = {
    "csa_abi_version": ([], ctypes.c_int),
    "csa_status_string": ([_I32], ctypes.c_char_p),
    "csa_workspace_size": ([_PP, _I32, ctypes.POINTER(_SZ)], _I32),
    "csa_workspace_size_min": ([_PP, _I32, ctypes.POINTER(_SZ)], _I32),
    "csa_cmp_seqlens": ([_P, _I32, _I32, _P, _P], _I32),
    "csa_validate_metadata": ([_PP, _P, _P, _P], _I32),
    "csa_compress": ([_PP, _I32, _P, _I32, _P, _P, _P, _P], _I32),
    "csa_compress_bwd": ([_PP, _P, _I32, _P, _P, _P, _P], _I32),
    "csa_quantize_fp8": ([_P, _I32, _I64, _I32, _P, _P, _P], _I32),
    "csa_compress_learned": ([_PP, _I32, _P, _P, _P, _I32, _I32, _P, _P, _P, _P], _I32),
    "csa_compress_learned_bwd": ([_PP, _I32, _P, _P, _P, _P, _I32, _I32, _P, _P, _P, _P, _P, _P],
                                 _I32),
    "csa_index_scores": ([_PP, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _P], _I32),
    "csa_topk_select": ([_PP, _P, _I64, _P, _P, _P, _P], _I32),
    "csa_index_topk": ([_PP, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _I64, _P, _P], _I32),
    "csa_sparse_attn_fwd": ([_PP] + [_P] * 13 + [_SZ, _P], _I32),
    "csa_rope": ([_I32, _P, _P, _I64, _I32, _I32, _I32, _F, _I32, _I32, _P, _P], _I32),
    "csa_teacher_logits_stride": ([_PP], _I64),
    "csa_sparse_attn_bwd": ([_PP] + [_P] * 14 + [_P, _SZ, _P], _I32),
    "csa_sparse_attn_bwd_noalloc": ([_PP] + [_P] * 14 + [_P], _I32),
    "csa_indexer_kl": ([_PP, _P, _P, _P, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _F,
                        _P, _P, _P, _P, _P, _P, _SZ, _P], _I32),
}


def lib():
    """Load libcsa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "python -m long_context_compressed_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def header_functions():
    """Names of the functions include/csa.h declares."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:csa_status_t|int64_t|int|const char\*)\s+(csa_\w+)\s*\(",
                                 text, re.M)))


def make_params(**kw) -> CsaParams:
    p = CsaParams()
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a tensor or None")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(name, st):
    if st != CSA_OK:
        raise CsaError(name, st, lib().csa_status_string(st).decode())


def dtype_code(t: torch.Tensor) -> int:
    return _DT[t.dtype]


def csa_abi_version() -> int:
    return lib().csa_abi_version()


def csa_workspace_size(p: CsaParams, op: int) -> int:
    n = _SZ(0)
    _check("csa_workspace_size", lib().csa_workspace_size(ctypes.byref(p), op, ctypes.byref(n)))
    return n.value


def csa_workspace_size_min(p: CsaParams, op: int) -> int:
    n = _SZ(0)
    _check("csa_workspace_size_min",
           lib().csa_workspace_size_min(ctypes.byref(p), op, ctypes.byref(n)))
    return n.value


def csa_cmp_seqlens(cu_seqlens, batch, ratio, cu_cmp, stream=None):
    _check("csa_cmp_seqlens", lib().csa_cmp_seqlens(_ptr(cu_seqlens), batch, ratio, _ptr(cu_cmp),
                                                   _stream(stream)))


def csa_validate_metadata(p, cu_seqlens, status_dev, stream=None):
    _check("csa_validate_metadata", lib().csa_validate_metadata(
        ctypes.byref(p), _ptr(cu_seqlens), _ptr(status_dev), _stream(stream)))


def csa_compress(p, x, cu_seqlens, cu_cmp, x_cmp, stream=None):
    _check("csa_compress", lib().csa_compress(ctypes.byref(p), dtype_code(x), _ptr(x), x.shape[-1],
                                             _ptr(cu_seqlens), _ptr(cu_cmp), _ptr(x_cmp),
                                             _stream(stream)))


def csa_compress_bwd(p, d_x_cmp, cu_seqlens, cu_cmp, dx, stream=None):
    _check("csa_compress_bwd", lib().csa_compress_bwd(
        ctypes.byref(p), _ptr(d_x_cmp), d_x_cmp.shape[-1], _ptr(cu_seqlens), _ptr(cu_cmp),
        _ptr(dx), _stream(stream)))


def csa_compress_learned(p, x, score, bias, overlap, cu_seqlens, cu_cmp, x_cmp, stream=None):
    _check("csa_compress_learned", lib().csa_compress_learned(
        ctypes.byref(p), dtype_code(x), _ptr(x), _ptr(score), _ptr(bias), x.shape[-1],
        int(overlap), _ptr(cu_seqlens), _ptr(cu_cmp), _ptr(x_cmp), _stream(stream)))


def csa_compress_learned_bwd(p, x, score, bias, d_x_cmp, overlap, cu_seqlens, cu_cmp, dx,
                             dscore, dbias, stream=None):
    _check("csa_compress_learned_bwd", lib().csa_compress_learned_bwd(
        ctypes.byref(p), dtype_code(x), _ptr(x), _ptr(score), _ptr(bias), _ptr(d_x_cmp),
        x.shape[-1], int(overlap), _ptr(cu_seqlens), _ptr(cu_cmp), _ptr(dx), _ptr(dscore),
        _ptr(dbias), _stream(stream)))


def csa_quantize_fp8(x, codes, row_scale, stream=None):
    rows = x.numel() // x.shape[-1]
    _check("csa_quantize_fp8", lib().csa_quantize_fp8(_ptr(x), dtype_code(x), rows, x.shape[-1],
                                                     _ptr(codes), _ptr(row_scale),
                                                     _stream(stream)))


def csa_index_scores(p, qI, qI_scale, w, kI_cmp, kI_scale, cu_seqlens, cu_cmp, scores,
                     stream=None):
    _check("csa_index_scores", lib().csa_index_scores(
        ctypes.byref(p), _ptr(qI), _ptr(qI_scale), _ptr(w), _ptr(kI_cmp), _ptr(kI_scale),
        _ptr(cu_seqlens), _ptr(cu_cmp), _ptr(scores), scores.shape[-1], _stream(stream)))


def csa_topk_select(p, scores, cu_seqlens, cu_cmp, idx, stream=None):
    _check("csa_topk_select", lib().csa_topk_select(
        ctypes.byref(p), _ptr(scores), scores.shape[-1], _ptr(cu_seqlens), _ptr(cu_cmp),
        _ptr(idx), _stream(stream)))


def csa_index_topk(p, qI, qI_scale, w, kI_cmp, kI_scale, cu_seqlens, cu_cmp, idx,
                   scores=None, scores_mode=0, stream=None):
    """scores_mode 0: scores untouched; 1: the selected entries written; 2: every visible one."""
    _check("csa_index_topk", lib().csa_index_topk(
        ctypes.byref(p), _ptr(qI), _ptr(qI_scale), _ptr(w), _ptr(kI_cmp), _ptr(kI_scale),
        _ptr(cu_seqlens), _ptr(cu_cmp), scores_mode, _ptr(scores),
        scores.shape[-1] if scores is not None else 0, _ptr(idx), _stream(stream)))


def csa_sparse_attn_fwd(p, q, kv_cmp, kv, idx, sink, cu_seqlens, cu_cmp, out, lse, lse_cmp=None,
                        ws=None, stream=None, t_logits=None, out_rot=None):
    _check("csa_sparse_attn_fwd", lib().csa_sparse_attn_fwd(
        ctypes.byref(p), _ptr(q), _ptr(kv_cmp), _ptr(kv), _ptr(idx), _ptr(sink), _ptr(cu_seqlens),
        _ptr(cu_cmp), _ptr(out), _ptr(out_rot), _ptr(lse), _ptr(lse_cmp), _ptr(t_logits),
        _ptr(ws), _nbytes(ws), _stream(stream)))


def csa_rope(x, y, rope_dim, theta, inverse, batch, row_offsets, stream=None):
    """x, y: [rows, dim] or [rows, heads, dim] of one dtype; y may be x (in place)."""
    if y.shape != x.shape or y.dtype != x.dtype:
        raise ValueError("x and y must have the same shape and dtype")
    rows, dim = (x.shape[0], x.shape[-1]) if x.dim() >= 2 else (0, 0)
    heads = x.numel() // (rows * dim) if rows and dim else 1
    _check("csa_rope", lib().csa_rope(dtype_code(x), _ptr(x), _ptr(y), rows, heads, dim,
                                      int(rope_dim), float(theta), int(inverse), int(batch),
                                      _ptr(row_offsets), _stream(stream)))


def csa_teacher_logits_stride(p) -> int:
    return int(lib().csa_teacher_logits_stride(ctypes.byref(p)))


def csa_sparse_attn_bwd(p, q, kv_cmp, kv, idx, sink, cu_seqlens, cu_cmp, out, lse, d_out, dq,
                        dkv_cmp, dkv, dsink, ws=None, stream=None):
    _check("csa_sparse_attn_bwd", lib().csa_sparse_attn_bwd(
        ctypes.byref(p), _ptr(q), _ptr(kv_cmp), _ptr(kv), _ptr(idx), _ptr(sink), _ptr(cu_seqlens),
        _ptr(cu_cmp), _ptr(out), _ptr(lse), _ptr(d_out), _ptr(dq), _ptr(dkv_cmp), _ptr(dkv),
        _ptr(dsink), _ptr(ws), _nbytes(ws), _stream(stream)))


def csa_sparse_attn_bwd_noalloc(p, q, kv_cmp, kv, idx, sink, cu_seqlens, cu_cmp, out, lse,
                                d_out, dq, dkv_cmp, dkv, dsink, stream=None):
    _check("csa_sparse_attn_bwd_noalloc", lib().csa_sparse_attn_bwd_noalloc(
        ctypes.byref(p), _ptr(q), _ptr(kv_cmp), _ptr(kv), _ptr(idx), _ptr(sink), _ptr(cu_seqlens),
        _ptr(cu_cmp), _ptr(out), _ptr(lse), _ptr(d_out), _ptr(dq), _ptr(dkv_cmp), _ptr(dkv),
        _ptr(dsink), _stream(stream)))


def csa_indexer_kl(p, q, kv_cmp, scores, idx, qI, qI_scale, w, kI_cmp, kI_scale, cu_seqlens,
                   cu_cmp, grad_scale, kl, loss, dqI=None, dw=None, dkI_cmp=None, ws=None,
                   teacher_lse=None, stream=None, teacher_logits=None):
    _check("csa_indexer_kl", lib().csa_indexer_kl(
        ctypes.byref(p), _ptr(q), _ptr(kv_cmp), _ptr(scores),
        scores.shape[-1] if scores is not None else 0, _ptr(idx),
        _ptr(teacher_lse), _ptr(teacher_logits), _ptr(qI), _ptr(qI_scale), _ptr(w), _ptr(kI_cmp), _ptr(kI_scale), _ptr(cu_seqlens),
        _ptr(cu_cmp), float(grad_scale), _ptr(kl), _ptr(loss), _ptr(dqI), _ptr(dw), _ptr(dkI_cmp),
        _ptr(ws), _nbytes(ws), _stream(stream)))
