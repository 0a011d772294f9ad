"""Host-side checks of the C ABI: the library loads, exports every declared symbol,
and rejects invalid arguments before launching anything (no GPU needed)."""
import ctypes

import pytest

from long_context_compressed_amd import binding as B


@pytest.fixture(scope="module")
def lib():
    return B.lib()


def _params(**kw):
    base = dict(batch=1, total_tokens=256, max_seqlen=256, ratio=4, window=16, topk=16,
                topk_cap=64, heads=4, head_dim=64, idx_heads=2, idx_dim=32, scale=0.125,
                mode=B.CSA_SPARSE, teacher=B.CSA_TEACHER_DENSE, dtype=B.CSA_F32,
                idx_dtype=B.CSA_F32)
    base.update(kw)
    return B.make_params(**base)


def test_exports_every_declared_symbol(lib):
    names = B.header_functions()
    assert len(names) == 20
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(B._SIGS)


def test_version_and_status_strings(lib):
    assert lib.csa_abi_version() == 7
    for st in (0, -1, -2, -3, -4, -5):
        assert lib.csa_status_string(st)
    assert lib.csa_status_string(7) == b"unknown status"


def test_workspace_sizes(lib):
    p = _params()
    assert B.csa_workspace_size(p, B.CSA_OP_ATTN_BWD) == 0          # scalar path: none
    assert B.csa_workspace_size(p, B.CSA_OP_ATTN_FWD) == 0
    # bf16 H=64 D=512 backward: [scale*dS | P] (128 bf16) per (token, candidate slot) of a
    # token chunk, slots = k_cap + W rounded up to 64.  Top-k 1024 of at most 250 visible
    # rows: the rows' gradients are key-major products whose partial sums take at most
    # (250 // 128 + 1) * (1000 // 256 + 1) + (1000 + 127) // 128 + 2 items of 256 KiB
    big = _params(heads=64, head_dim=512, dtype=B.CSA_BF16, topk=1024, topk_cap=1024,
                  window=128, total_tokens=1000, max_seqlen=1000, batch=1)
    pds = 1000 * 1152 * 128 * 2
    items = 2 * (3 + 1) + (1000 + 127) // 128 + 2
    n = B.csa_workspace_size(big, B.CSA_OP_ATTN_BWD)
    assert pds + items * 2**18 <= n <= pds + items * (2**18 + 64) + 2**20
    # the backward also takes any workspace down to one chunk of 16 queries
    m = B.csa_workspace_size_min(big, B.CSA_OP_ATTN_BWD)
    items16 = 2 * (0 + 1) + (16 + 127) // 128 + 2
    assert 16 * 1152 * 256 + items16 * 2**18 <= m <= 16 * 1152 * 256 + items16 * (2**18 + 64) + 2**20
    # top-k 1024 of up to 25000 visible rows: one staged bf16 row gradient (512 values) per
    # (token, slot) besides [scale*dS | P], summed per row through a CSR
    sparse = _params(heads=64, head_dim=512, dtype=B.CSA_BF16, topk=1024, topk_cap=1024,
                     window=128, total_tokens=1000, max_seqlen=100000, batch=1)
    n = B.csa_workspace_size(sparse, B.CSA_OP_ATTN_BWD)
    assert 1000 * 1152 * (128 + 512) * 2 <= n <= 1000 * 1152 * (128 + 512) * 2 + 8 * 2**20
    m = B.csa_workspace_size_min(sparse, B.CSA_OP_ATTN_BWD)
    assert 16 * 1152 * (128 + 512) * 2 <= m <= 16 * 1152 * (128 + 512) * 2 + 2**20
    assert B.csa_workspace_size_min(p, B.CSA_OP_INDEXER_KL) == \
        B.csa_workspace_size(p, B.CSA_OP_INDEXER_KL)
    n = ctypes.c_size_t(0)
    assert lib.csa_workspace_size(ctypes.byref(p), 99, ctypes.byref(n)) == B.CSA_ERR_ARG
    assert lib.csa_workspace_size(None, 1, ctypes.byref(n)) == B.CSA_ERR_NULL


FAKE = 4096  # a non-null pointer value; every call below fails validation before any use


def test_compress_validation(lib):
    p = _params()
    f = lib.csa_compress
    assert f(ctypes.byref(p), 0, None, 64, FAKE, FAKE, FAKE, None) == B.CSA_ERR_NULL
    assert f(None, 0, FAKE, 64, FAKE, FAKE, FAKE, None) == B.CSA_ERR_NULL
    assert f(ctypes.byref(p), 0, FAKE, 4, FAKE, FAKE, FAKE, None) == B.CSA_ERR_ARG
    assert f(ctypes.byref(p), 0, FAKE, 60, FAKE, FAKE, FAKE, None) == B.CSA_ERR_UNSUPPORTED
    assert f(ctypes.byref(p), 2, FAKE, 64, FAKE, FAKE, FAKE, None) == B.CSA_ERR_UNSUPPORTED
    bad = _params(ratio=0)
    assert f(ctypes.byref(bad), 0, FAKE, 64, FAKE, FAKE, FAKE, None) == B.CSA_ERR_ARG
    bad = _params(batch=-1)
    assert f(ctypes.byref(bad), 0, FAKE, 64, FAKE, FAKE, FAKE, None) == B.CSA_ERR_ARG
    g = lib.csa_compress_bwd
    assert g(ctypes.byref(p), FAKE, 64, FAKE, FAKE, None, None) == B.CSA_ERR_NULL
    assert g(ctypes.byref(p), FAKE, 12, FAKE, FAKE, FAKE, None) == B.CSA_ERR_UNSUPPORTED


def test_learned_compressor_validation(lib):
    p = _params()
    f, g = lib.csa_compress_learned, lib.csa_compress_learned_bwd
    ok = [FAKE, FAKE, FAKE]                       # x, score, bias
    assert f(ctypes.byref(p), 0, FAKE, FAKE, None, 64, 1, FAKE, FAKE, FAKE, None) == B.CSA_ERR_NULL
    assert f(ctypes.byref(p), 0, *ok, 64, 2, FAKE, FAKE, FAKE, None) == B.CSA_ERR_ARG
    assert f(ctypes.byref(p), 0, *ok, 4, 1, FAKE, FAKE, FAKE, None) == B.CSA_ERR_ARG
    assert f(ctypes.byref(p), 0, *ok, 60, 1, FAKE, FAKE, FAKE, None) == B.CSA_ERR_UNSUPPORTED
    assert f(ctypes.byref(p), 2, *ok, 64, 1, FAKE, FAKE, FAKE, None) == B.CSA_ERR_UNSUPPORTED
    assert f(None, 0, *ok, 64, 1, FAKE, FAKE, FAKE, None) == B.CSA_ERR_NULL
    assert g(ctypes.byref(p), 0, *ok, FAKE, 64, 1, FAKE, FAKE, FAKE, FAKE, None,
             None) == B.CSA_ERR_NULL                                          # dbias
    assert g(ctypes.byref(p), 1, *ok, FAKE, 4096, 0, FAKE, FAKE, FAKE, FAKE, FAKE,
             None) == B.CSA_ERR_UNSUPPORTED


def test_cmp_seqlens_and_quantize_validation(lib):
    assert lib.csa_cmp_seqlens(None, 1, 4, FAKE, None) == B.CSA_ERR_NULL
    assert lib.csa_cmp_seqlens(FAKE, -1, 4, FAKE, None) == B.CSA_ERR_ARG
    assert lib.csa_cmp_seqlens(FAKE, 1, 0, FAKE, None) == B.CSA_ERR_ARG
    q = lib.csa_quantize_fp8
    assert q(None, 1, 10, 128, FAKE, FAKE, None) == B.CSA_ERR_NULL
    assert q(FAKE, 1, -1, 128, FAKE, FAKE, None) == B.CSA_ERR_ARG
    assert q(FAKE, 1, 10, 100, FAKE, FAKE, None) == B.CSA_ERR_UNSUPPORTED
    assert q(FAKE, 1, 10, 2048, FAKE, FAKE, None) == B.CSA_ERR_UNSUPPORTED
    assert q(FAKE, 2, 10, 128, FAKE, FAKE, None) == B.CSA_ERR_UNSUPPORTED
    v = lib.csa_validate_metadata
    assert v(None, FAKE, FAKE, None) == B.CSA_ERR_NULL


def test_scores_and_topk_validation(lib):
    p = _params()
    s = lib.csa_index_scores
    args = [FAKE, None, FAKE, FAKE, None, FAKE, FAKE, FAKE]
    assert s(ctypes.byref(p), *args[:7], None, 64, None) == B.CSA_ERR_NULL
    assert s(ctypes.byref(p), *args, 63, None) == B.CSA_ERR_ARG            # ld < n_cap = 64
    fp8 = _params(idx_dtype=B.CSA_FP8_E4M3)
    assert s(ctypes.byref(fp8), *args, 64, None) == B.CSA_ERR_NULL         # scales missing
    big = _params(idx_dim=512)
    assert s(ctypes.byref(big), *args, 64, None) == B.CSA_ERR_UNSUPPORTED
    odd = _params(idx_dim=36)
    assert s(ctypes.byref(odd), *args, 64, None) == B.CSA_ERR_UNSUPPORTED
    t = lib.csa_topk_select
    assert t(ctypes.byref(p), FAKE, 64, FAKE, FAKE, None, None) == B.CSA_ERR_NULL
    assert t(ctypes.byref(_params(topk_cap=48)), FAKE, 64, FAKE, FAKE, FAKE, None) == B.CSA_ERR_ARG
    assert t(ctypes.byref(_params(topk=0)), FAKE, 64, FAKE, FAKE, FAKE, None) == B.CSA_ERR_ARG
    assert t(ctypes.byref(_params(topk=100)), FAKE, 64, FAKE, FAKE, FAKE, None) == B.CSA_ERR_ARG
    assert t(ctypes.byref(p), FAKE, 10, FAKE, FAKE, FAKE, None) == B.CSA_ERR_ARG
    huge = _params(total_tokens=1 << 20, max_seqlen=1 << 20)
    assert t(ctypes.byref(huge), FAKE, 1 << 18, FAKE, FAKE, FAKE, None) == B.CSA_ERR_UNSUPPORTED


def test_fused_index_topk_validation(lib):
    f = lib.csa_index_topk
    big = dict(idx_heads=64, idx_dim=128, idx_dtype=B.CSA_BF16)
    p = _params(**big)
    ops = [FAKE, None, FAKE, FAKE, None, FAKE, FAKE]         # qI .. cu_cmp

    def call(pp, mode=0, scores=None, ld=0, idx=FAKE, ops=ops):
        return f(ctypes.byref(pp), *ops, mode, scores, ld, idx, None)

    assert call(p, idx=None) == B.CSA_ERR_NULL
    assert call(p, mode=3) == B.CSA_ERR_ARG
    assert call(p, mode=1) == B.CSA_ERR_NULL                   # scores wanted, none given
    assert call(p, mode=2, scores=FAKE, ld=63) == B.CSA_ERR_ARG  # ld < n_cap = 64
    assert call(_params(idx_dtype=B.CSA_FP8_E4M3, idx_heads=64, idx_dim=128)) == B.CSA_ERR_NULL
    assert call(_params(topk_cap=48, **big)) == B.CSA_ERR_ARG
    assert call(_params(topk=0, **big)) == B.CSA_ERR_ARG
    # shapes without a fused kernel: the separate score and top-k calls serve them
    assert call(_params()) == B.CSA_ERR_UNSUPPORTED                    # f32, 2 x 32 indexer
    assert call(_params(idx_heads=32, idx_dim=128, idx_dtype=B.CSA_BF16)) == B.CSA_ERR_UNSUPPORTED
    long_ = _params(total_tokens=1 << 18, max_seqlen=1 << 18, **big)  # 65536 visible > 32768
    assert call(long_) == B.CSA_ERR_UNSUPPORTED


def test_attention_validation(lib):
    p = _params()
    f = lib.csa_sparse_attn_fwd
    a = [FAKE] * 8 + [None, FAKE, FAKE, None]         # q .. out, out_rot, lse, lse_cmp, t_logits
    assert f(ctypes.byref(p), FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, None, FAKE, None,
             None, None, 0, None) == B.CSA_ERR_NULL                           # idx for sparse
    assert f(ctypes.byref(_params(window=0)), *a, None, 0, None) == B.CSA_ERR_ARG
    assert f(ctypes.byref(_params(scale=0.0)), *a, None, 0, None) == B.CSA_ERR_ARG
    assert f(ctypes.byref(_params(mode=3)), *a, None, 0, None) == B.CSA_ERR_ARG
    assert f(ctypes.byref(_params(head_dim=1024)), *a, None, 0, None) == B.CSA_ERR_UNSUPPORTED
    assert f(ctypes.byref(_params(dtype=B.CSA_FP8_E4M3)), *a, None, 0, None) == B.CSA_ERR_UNSUPPORTED
    assert f(ctypes.byref(_params(mode=B.CSA_DENSE)), FAKE, None, FAKE, None, None, FAKE, FAKE,
             FAKE, None, FAKE, None, None, None, 0, None) == B.CSA_ERR_NULL  # kv_cmp for dense
    # rotary band of the output rotation
    OTHER = 2 * FAKE
    rot = a[:8] + [OTHER] + a[9:]
    assert f(ctypes.byref(p), *rot, None, 0, None) == B.CSA_ERR_ARG          # rope_dim 0
    assert f(ctypes.byref(_params(rope_dim=8, rope_theta=1e4)), *a[:8], FAKE, *a[9:], None, 0,
             None) == B.CSA_ERR_ARG                                          # out_rot aliases out
    for bad in (dict(rope_dim=12, rope_theta=1e4), dict(rope_dim=72, rope_theta=1e4),
                dict(rope_dim=-8, rope_theta=1e4), dict(rope_dim=8, rope_theta=0.0),
                dict(rope_dim=8, rope_theta=float("inf"))):
        assert f(ctypes.byref(_params(**bad)), *a, None, 0, None) == B.CSA_ERR_ARG, bad
    b = lib.csa_sparse_attn_bwd
    args = [FAKE] * 14
    bf = _params(heads=64, head_dim=512, dtype=B.CSA_BF16)
    assert b(ctypes.byref(bf), *args, None, 0, None) == B.CSA_ERR_WORKSPACE
    assert b(ctypes.byref(bf), *args, FAKE, 100, None) == B.CSA_ERR_WORKSPACE
    args[11] = None                                                          # dq
    assert b(ctypes.byref(p), *args, FAKE, 1 << 20, None) == B.CSA_ERR_NULL


def test_indexer_kl_validation(lib):
    p = _params()
    f = lib.csa_indexer_kl

    def call(pp, idx=FAKE, grads=(FAKE, FAKE, FAKE), ld=64, gs=1.0, cache=None):
        return f(ctypes.byref(pp), FAKE, FAKE, FAKE, ld, idx, None, cache, FAKE, None, FAKE, FAKE,
                 None, FAKE, FAKE, gs, FAKE, FAKE, *grads, None, 0, None)

    assert call(_params(teacher=B.CSA_TEACHER_NONE)) == B.CSA_ERR_ARG
    assert call(_params(teacher=B.CSA_TEACHER_SELECTED), idx=None) == B.CSA_ERR_NULL
    assert call(p, grads=(FAKE, None, FAKE)) == B.CSA_ERR_NULL
    assert call(p, ld=10) == B.CSA_ERR_ARG
    assert call(p, gs=float("nan")) == B.CSA_ERR_ARG
    assert call(_params(heads=128)) == B.CSA_ERR_UNSUPPORTED
    assert call(_params(idx_dtype=B.CSA_FP8_E4M3)) == B.CSA_ERR_NULL


def test_teacher_logits_cache_contract(lib):
    stride = lib.csa_teacher_logits_stride
    stride.argtypes = [ctypes.POINTER(B.CsaParams)]
    stride.restype = ctypes.c_int64
    assert stride(ctypes.byref(_params(topk_cap=128))) == 128                 # sparse: topk_cap
    assert stride(ctypes.byref(_params(mode=B.CSA_DENSE, max_seqlen=260, ratio=4))) == 128
    assert stride(ctypes.byref(_params(mode=B.CSA_WINDOW))) == 0
    assert stride(ctypes.byref(_params(window=0))) == 0                      # invalid params
    f = lib.csa_indexer_kl

    def call(pp, cache):
        return f(ctypes.byref(pp), FAKE, FAKE, FAKE, 1 << 16, FAKE, None, cache, FAKE, None, FAKE,
                 FAKE, None, FAKE, FAKE, 1.0, FAKE, FAKE, None, None, None, None, 0, None)
    # the cache only stands in for the teacher when the candidate sets agree
    assert call(_params(teacher=B.CSA_TEACHER_SELECTED, mode=B.CSA_DENSE), FAKE) == B.CSA_ERR_ARG
    assert call(_params(teacher=B.CSA_TEACHER_DENSE, mode=B.CSA_SPARSE), FAKE) == B.CSA_ERR_ARG
    big = dict(heads=64, head_dim=512, idx_heads=64, idx_dim=128, dtype=B.CSA_BF16,
               idx_dtype=B.CSA_BF16, teacher=B.CSA_TEACHER_SELECTED, topk_cap=1024, topk=1024,
               total_tokens=65536, max_seqlen=16384)
    n = B.csa_workspace_size(_params(**big), B.CSA_OP_INDEXER_KL_CACHED)
    assert n >= 16384 * 1024 * 128 * 2                                       # bf16 staging


def test_rope_validation(lib):
    f = lib.csa_rope

    def call(dtype=B.CSA_BF16, x=FAKE, y=FAKE, rows=16, heads=2, dim=64, rope_dim=16,
             theta=1e4, inverse=0, batch=1, offs=FAKE):
        return f(dtype, x, y, rows, heads, dim, rope_dim, theta, inverse, batch, offs, None)

    assert call(x=None) == B.CSA_ERR_NULL
    assert call(y=None) == B.CSA_ERR_NULL
    assert call(offs=None) == B.CSA_ERR_NULL
    assert call(x=None, y=None, rows=0, dtype=B.CSA_FP8_E4M3) == B.CSA_ERR_UNSUPPORTED  # no rows
    assert call(dtype=B.CSA_FP8_E4M3) == B.CSA_ERR_UNSUPPORTED
    for bad in (dict(rows=-1), dict(rows=1 << 31), dict(heads=0), dict(dim=4), dict(dim=60),
                dict(rope_dim=0), dict(rope_dim=12), dict(rope_dim=72), dict(theta=0.0),
                dict(theta=float("nan")), dict(inverse=2), dict(batch=-1)):
        assert call(**bad) == B.CSA_ERR_ARG, bad
