"""Pins of the fp64 oracle against what the method and mathematics fix.

None of these re-types the oracle's formula: each compares it with a closed
form, a fixture, an invariant, a brute-force definition, an independent
formulation (dense boolean mask; torch autograd; finite differences) or a
library routine applied to a special case.
"""
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import csa_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(12345)


def _gold_lines(name):
    with open(os.path.join(GOLD, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


def _cu(lengths):
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    return cu


# --------------------------------------------------------------------------- metadata
def test_cmp_seqlens_golden():
    for ln in _gold_lines("cmp_seqlens.txt"):
        r, lens, want = [x.strip() for x in ln.split("|")]
        lens = [int(x) for x in lens.split()]
        got = O.cmp_seqlens(_cu(lens), int(r))
        assert got.tolist() == [int(x) for x in want.split()]


def test_visibility_golden_and_bruteforce():
    for ln in _gold_lines("visibility_r4.txt"):
        p, nv = (int(x) for x in ln.split())
        assert int(O.n_visible(p, 4)) == nv
    # brute force: group j visible iff all of its token positions are <= p
    for r in (1, 2, 4, 8, 128):
        for p in range(0, 600):
            brute = sum(1 for j in range(p + 2) if all(j * r + u <= p for u in range(r)))
            assert int(O.n_visible(p, r)) == brute


def test_cu_seqlens_guards():
    with pytest.raises(ValueError):
        O.sample_table([0, 5, 3])
    with pytest.raises(ValueError):
        O.sample_table([1, 5])
    with pytest.raises(ValueError):
        O.token_positions([0, 10], 8)


# --------------------------------------------------------------------------- compressor
def test_compress_closed_form_arange():
    lens = [9, 4, 13, 2]
    cu = _cu(lens)
    T, dim, r = int(cu[-1]) + 3, 5, 4
    x = np.arange(T)[:, None] * 10.0 + np.arange(dim)[None, :]
    got = O.compress(x, cu, r)
    cu_cmp = O.cmp_seqlens(cu, r)
    assert got.shape == (int(cu_cmp[-1]), dim)
    for b, (s, L) in enumerate(zip(cu[:-1], lens)):
        for j in range(L // r):
            # mean of 10*t + c over t = s+jr .. s+jr+r-1
            want = 10.0 * (s + j * r + (r - 1) / 2.0) + np.arange(dim)
            np.testing.assert_allclose(got[cu_cmp[b] + j], want, rtol=0, atol=1e-12)


def test_compress_tail_and_padding_ignored():
    lens = [10, 7]
    cu = _cu(lens)
    T = 20
    x = RNG.standard_normal((T, 6))
    base = O.compress(x, cu, 4)
    y = x.copy()
    y[8:10] = 99.0      # tail of sample 0 (10 mod 4 = 2 tokens)
    y[14:17] = -7.0     # tail of sample 1 (7 mod 4 = 3 tokens)
    y[17:] = np.nan     # capacity padding
    np.testing.assert_array_equal(O.compress(y, cu, 4), base)


def test_compress_adjoint():
    lens = [13, 4, 0, 9]
    cu = _cu(lens)
    T = 30
    for r in (4, 3):
        x = RNG.standard_normal((T, 7))
        cmp = O.compress(x, cu, r)
        y = RNG.standard_normal(cmp.shape)
        lhs = float((cmp * y).sum())
        rhs = float((x * O.compress_bwd(y, cu, r, T)).sum())
        assert abs(lhs - rhs) < 1e-12 * max(1.0, abs(lhs))


def test_compress_bwd_tails_zero():
    lens = [10, 7]
    cu = _cu(lens)
    d = np.ones((int(O.cmp_seqlens(cu, 4)[-1]), 3))
    dx = O.compress_bwd(d, cu, 4, 20)
    assert np.all(dx[0:8] == 0.25) and np.all(dx[8:10] == 0)
    assert np.all(dx[10:14] == 0.25) and np.all(dx[14:] == 0)


# --------------------------------------------------------------------------- indexer scores
def test_index_scores_scalar_loops():
    lens = [11, 6]
    cu = _cu(lens)
    T, HI, dI, r = 20, 3, 4, 2
    qI = RNG.standard_normal((T, HI, dI))
    w = RNG.standard_normal((T, HI))
    kI_tok = RNG.standard_normal((T, dI))
    kI = O.compress(kI_tok, cu, r)
    n_cap = max(lens) // r
    got = O.index_scores(qI, w, kI, cu, r, n_cap)
    cu_cmp = O.cmp_seqlens(cu, r)
    for b, (s, L) in enumerate(zip(cu[:-1], lens)):
        for p in range(L):
            t = s + p
            for j in range(n_cap):
                if (j + 1) * r - 1 <= p:
                    acc = 0.0
                    for h in range(HI):
                        z = 0.0
                        for d in range(dI):
                            z += qI[t, h, d] * kI[cu_cmp[b] + j, d]
                        acc += w[t, h] * (z if z > 0 else 0.0)
                    assert abs(got[t, j] - acc) < 1e-12
                else:
                    assert got[t, j] == -np.inf
    assert np.all(got[17:] == -np.inf)


def test_index_scores_reduces_to_dot():
    # one head, unit weight, positive operands: the score is the plain dot product
    cu = _cu([16])
    qI = np.abs(RNG.standard_normal((16, 1, 8)))
    kI_tok = np.abs(RNG.standard_normal((16, 8)))
    kI = O.compress(kI_tok, cu, 4)
    got = O.index_scores(qI, np.ones((16, 1)), kI, cu, 4, 4)
    for t in range(16):
        nv = (t + 1) // 4
        np.testing.assert_allclose(got[t, :nv], kI[:nv] @ qI[t, 0], rtol=1e-14)


# --------------------------------------------------------------------------- top-k
def _rank_select(s, k):
    """Brute-force definition: j is selected iff fewer than k entries beat it,
    where j' beats j when s[j'] > s[j], or s[j'] == s[j] and j' < j."""
    n = len(s)
    out = []
    for j in range(n):
        beats = sum(1 for jj in range(n) if s[jj] > s[j] or (s[jj] == s[j] and jj < j))
        if beats < k:
            out.append(j)
    return set(out)


def test_topk_bruteforce_with_ties_and_signed_zero():
    lens = [40, 23]
    cu = _cu(lens)
    T, r, k, k_cap = 70, 2, 5, 64
    n_cap = 20
    # quantized scores force many ties; include -0 and +0
    scores = np.round(RNG.standard_normal((T, n_cap)) * 2) / 2
    scores[scores == 0] = -0.0
    scores[::3, ::2] = 0.0
    idx = O.topk_select(scores, cu, r, k, k_cap, T)
    cu_cmp = O.cmp_seqlens(cu, r)
    for b, (s, L) in enumerate(zip(cu[:-1], lens)):
        for p in range(L):
            t = s + p
            nv = (p + 1) // r
            row = idx[t]
            sel = row[row >= 0]
            assert len(sel) == min(k, nv)
            assert np.all(row[len(sel):] == -1)
            local = set((sel - cu_cmp[b]).tolist())
            assert local == _rank_select(list(scores[t, :nv]), k)
    assert np.all(idx[63:] == -1)


def test_topk_invariants_and_library():
    cu = _cu([300])
    T, r, k = 300, 4, 16
    scores = RNG.standard_normal((T, 75)).astype(np.float32)
    idx = O.topk_select(scores, cu, r, k, 64, T)
    for t in range(T):
        nv = (t + 1) // r
        sel = idx[t][idx[t] >= 0]
        assert len(set(sel.tolist())) == len(sel) == min(k, nv)
        if nv > k:
            mask = np.zeros(nv, bool)
            mask[sel] = True
            assert scores[t, :nv][mask].min() >= scores[t, :nv][~mask].max()
            # library: a stable descending argsort of the same float32 bytes
            ref = np.argsort(-scores[t, :nv].astype(np.float64), kind="stable")[:k]
            assert set(ref.tolist()) == set(sel.tolist())


def test_topk_all_when_k_large():
    # dense mode == top-k with k >= n_cap: every visible row is selected
    cu = _cu([64, 37])
    scores = RNG.standard_normal((101, 16))
    idx = O.topk_select(scores, cu, 4, 16, 64, 101)
    cu_cmp = O.cmp_seqlens(cu, 4)
    for b, (s, L) in enumerate(zip(cu[:-1], [64, 37])):
        for p in range(L):
            sel = idx[s + p][idx[s + p] >= 0]
            assert sorted(sel.tolist()) == list(range(cu_cmp[b], cu_cmp[b] + (p + 1) // 4))


# --------------------------------------------------------------------------- attention
def _dense_mask_attention(q, kv_cmp, kv, idx, sink, cu, r, W, scale):
    """Independent formulation: one key set [kv_cmp; kv], a boolean mask, a full softmax
    (torch, float64, differentiable)."""
    T, H, D = q.shape
    Tc = kv_cmp.shape[0]
    keys = torch.cat([kv_cmp, kv], 0)                   # [Tc + T, D]
    mask = torch.zeros(T, Tc + T, dtype=torch.bool)
    cu_cmp = O.cmp_seqlens(cu, r)
    for b in range(len(cu) - 1):
        s, L = int(cu[b]), int(cu[b + 1] - cu[b])
        for p in range(L):
            t = s + p
            if idx is None:
                nv = (p + 1) // r
                mask[t, int(cu_cmp[b]):int(cu_cmp[b]) + nv] = True
            else:
                for g in idx[t]:
                    if g >= 0:
                        mask[t, int(g)] = True
            lo = max(0, p - W + 1)
            mask[t, Tc + s + lo: Tc + s + p + 1] = True
    logits = scale * torch.einsum("thd,nd->thn", q, keys)
    logits = logits.masked_fill(~mask[:, None, :], float("-inf"))
    if sink is not None:
        logits = torch.cat([logits, sink[None, :, None].expand(T, H, 1)], dim=2)
    lse = torch.logsumexp(logits, dim=2)
    P = torch.exp(logits - lse[..., None])
    if sink is not None:
        P = P[..., :-1]
    out = torch.einsum("thn,nd->thd", P, keys)
    return out, lse


def _small_case(lens, H=3, D=8, r=4, W=5, k=3, seed=0, T=None):
    rng = np.random.default_rng(seed)
    cu = _cu(lens)
    T = T or int(cu[-1])
    q = rng.standard_normal((T, H, D))
    kv = rng.standard_normal((T, D))
    kv_cmp = O.compress(kv, cu, r)
    n_cap = max(lens) // r
    scores = rng.standard_normal((T, n_cap))
    idx = O.topk_select(scores, cu, r, k, 64, T)
    return cu, q, kv, kv_cmp, idx, rng


@pytest.mark.parametrize("dense", [False, True])
@pytest.mark.parametrize("with_sink", [False, True])
def test_attn_fwd_equals_dense_mask(dense, with_sink):
    lens = [21, 9, 14]
    cu, q, kv, kv_cmp, idx, rng = _small_case(lens)
    sink = rng.standard_normal(3) if with_sink else None
    use_idx = None if dense else idx
    Ox, Lx = O.sparse_attn_fwd(q, kv_cmp, kv, use_idx, sink, cu, 4, 5, 0.3)
    Od, Ld = _dense_mask_attention(torch.tensor(q), torch.tensor(kv_cmp), torch.tensor(kv),
                                   use_idx, None if sink is None else torch.tensor(sink),
                                   cu, 4, 5, 0.3)
    np.testing.assert_allclose(Ox, Od.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(Lx, Ld.numpy(), rtol=0, atol=1e-12)


def test_attn_window_only_is_sliding_window_sdpa():
    # no compressed candidates (window-only layer): sliding-window causal MQA
    lens = [33]
    T, H, D, W = 33, 4, 16, 7
    rng = np.random.default_rng(3)
    q = rng.standard_normal((T, H, D))
    kv = rng.standard_normal((T, D))
    cu = _cu(lens)
    idx = np.full((T, 64), -1)
    Ox, Lx = O.sparse_attn_fwd(q, np.zeros((0, D)), kv, idx, None, cu, 4, W, 1 / np.sqrt(D))
    i = torch.arange(T)
    mask = (i[None, :] <= i[:, None]) & (i[None, :] > i[:, None] - W)
    qt = torch.tensor(q).permute(1, 0, 2)            # [H, T, D]
    kt = torch.tensor(kv)[None].expand(H, T, D)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, attn_mask=mask)
    np.testing.assert_allclose(Ox, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_attn_full_window_is_causal_attention():
    lens = [19, 12]
    H, D = 2, 8
    cu = _cu(lens)
    rng = np.random.default_rng(4)
    q = rng.standard_normal((31, H, D))
    kv = rng.standard_normal((31, D))
    idx = np.full((31, 64), -1)
    Ox, Lx = O.sparse_attn_fwd(q, np.zeros((0, D)), kv, idx, None, cu, 4, 1000, 1 / np.sqrt(D))
    for b in range(2):
        s, L = int(cu[b]), lens[b]
        qt = torch.tensor(q[s:s + L]).permute(1, 0, 2)
        kt = torch.tensor(kv[s:s + L])[None].expand(H, L, D)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, is_causal=True)
        np.testing.assert_allclose(Ox[s:s + L], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
        # LSE is the log-sum-exp of the causal logits
        for p in range(L):
            logits = q[s + p] @ kv[s:s + p + 1].T / np.sqrt(D)
            np.testing.assert_allclose(Lx[s + p], logsumexp(logits, axis=1), atol=1e-12)


def test_attn_sink_is_zero_valued_key():
    lens = [17]
    cu, q, kv, kv_cmp, idx, rng = _small_case(lens, seed=5)
    sink = rng.standard_normal(3)
    Os, Ls = O.sparse_attn_fwd(q, kv_cmp, kv, idx, sink, cu, 4, 5, 0.5)
    # append a virtual key with logit sink_h and value 0: emulate by a zero row whose
    # logit is forced, computed by hand per (t, h)
    for t in range(17):
        p = t
        cr = idx[t][idx[t] >= 0]
        wr = np.arange(max(0, p - 4), p + 1)
        X = np.concatenate([kv_cmp[cr], kv[wr]])
        for h in range(3):
            lg = np.concatenate([0.5 * X @ q[t, h], [sink[h]]])
            pr = np.exp(lg - lg.max())
            pr /= pr.sum()
            vals = np.concatenate([X, np.zeros((1, X.shape[1]))])
            np.testing.assert_allclose(Os[t, h], pr @ vals, atol=1e-12)
            np.testing.assert_allclose(Ls[t, h], logsumexp(lg), atol=1e-12)


def test_attn_bruteforce_softmax_tiny():
    # explicit scalar loops on a 2-sample pack
    lens = [6, 5]
    cu, q, kv, kv_cmp, idx, rng = _small_case(lens, H=2, D=3, r=2, W=2, k=1, seed=6)
    Ox, Lx = O.sparse_attn_fwd(q, kv_cmp, kv, idx, None, cu, 2, 2, 0.7)
    cu_cmp = O.cmp_seqlens(cu, 2)
    for b in range(2):
        s, L = int(cu[b]), lens[b]
        for p in range(L):
            t = s + p
            rows = [kv_cmp[g] for g in idx[t] if g >= 0]
            rows += [kv[s + u] for u in range(max(0, p - 1), p + 1)]
            for h in range(2):
                ls = [0.7 * sum(q[t, h, d] * x[d] for d in range(3)) for x in rows]
                mx = max(ls)
                ex = [np.exp(v - mx) for v in ls]
                den = sum(ex)
                for d in range(3):
                    want = sum(e * x[d] for e, x in zip(ex, rows)) / den
                    assert abs(Ox[t, h, d] - want) < 1e-13
                assert abs(Lx[t, h] - (mx + np.log(den))) < 1e-13
        assert all(cu_cmp[b] <= g < cu_cmp[b + 1] for g in idx[s:s + L].ravel() if g >= 0)


def test_attn_bwd_matches_autograd_dense_mask():
    lens = [21, 9, 14]
    cu, q, kv, kv_cmp, idx, rng = _small_case(lens, seed=7)
    sink = rng.standard_normal(3)
    dO = rng.standard_normal(q.shape)
    Ox, Lx = O.sparse_attn_fwd(q, kv_cmp, kv, idx, sink, cu, 4, 5, 0.3)
    dq, dkc, dkv, dsink = O.sparse_attn_bwd(q, kv_cmp, kv, idx, sink, cu, 4, 5, 0.3, Ox, Lx, dO)
    qt = torch.tensor(q, requires_grad=True)
    kct = torch.tensor(kv_cmp, requires_grad=True)
    kvt = torch.tensor(kv, requires_grad=True)
    st = torch.tensor(sink, requires_grad=True)
    out, _ = _dense_mask_attention(qt, kct, kvt, idx, st, cu, 4, 5, 0.3)
    (out * torch.tensor(dO)).sum().backward()
    np.testing.assert_allclose(dq, qt.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dkc, kct.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dkv, kvt.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dsink, st.grad.numpy(), atol=1e-11)


def test_attn_bwd_finite_differences():
    lens = [10, 7]
    cu, q, kv, kv_cmp, idx, rng = _small_case(lens, H=2, D=4, r=2, W=3, k=2, seed=8)
    sink = rng.standard_normal(2)
    dO = rng.standard_normal(q.shape)

    def f(q_, kc_, kv_, s_):
        o, _ = O.sparse_attn_fwd(q_, kc_, kv_, idx, s_, cu, 2, 3, 0.6)
        return float((o * dO).sum())

    Ox, Lx = O.sparse_attn_fwd(q, kv_cmp, kv, idx, sink, cu, 2, 3, 0.6)
    dq, dkc, dkv, dsink = O.sparse_attn_bwd(q, kv_cmp, kv, idx, sink, cu, 2, 3, 0.6, Ox, Lx, dO)
    eps = 1e-6
    for arr, grad, which in ((q, dq, 0), (kv_cmp, dkc, 1), (kv, dkv, 2), (sink, dsink, 3)):
        flat = arr.reshape(-1)
        for pos in np.random.default_rng(9).choice(flat.size, size=min(12, flat.size), replace=False):
            old = flat[pos]
            args = [q, kv_cmp, kv, sink]
            flat[pos] = old + eps
            fp = f(*args)
            flat[pos] = old - eps
            fm = f(*args)
            flat[pos] = old
            num = (fp - fm) / (2 * eps)
            assert abs(num - grad.reshape(-1)[pos]) <= 1e-7 * max(1.0, abs(num)), which


# --------------------------------------------------------------------------- indexer KL
def _kl_case(lens, H=3, D=6, HI=2, dI=4, r=2, k=3, seed=11, teacher="selected"):
    rng = np.random.default_rng(seed)
    cu = _cu(lens)
    T = int(cu[-1])
    q = rng.standard_normal((T, H, D))
    kv = rng.standard_normal((T, D))
    kv_cmp = O.compress(kv, cu, r)
    qI = rng.standard_normal((T, HI, dI))
    w = rng.standard_normal((T, HI))
    kI = O.compress(rng.standard_normal((T, dI)), cu, r)
    n_cap = max(lens) // r
    sc = O.index_scores(qI, w, kI, cu, r, n_cap)
    idx = O.topk_select(sc, cu, r, k, 64, T)
    return cu, q, kv_cmp, qI, w, kI, sc, idx


def test_kl_nonnegative_and_matches_torch_kl_div():
    cu, q, kc, qI, w, kI, sc, idx = _kl_case([17, 12])
    for teacher in ("selected", "dense"):
        kl, loss, *_ = O.indexer_kl(q, kc, sc, idx, qI, w, kI, cu, 2, 0.4, teacher)
        assert np.all(kl >= -1e-15)
        assert abs(loss - kl.sum()) < 1e-12
        cu_cmp = O.cmp_seqlens(cu, 2)
        bb, pp = O.token_positions(cu, q.shape[0])
        for t in range(q.shape[0]):
            nv = (pp[t] + 1) // 2
            if teacher == "dense":
                C = np.arange(nv)
            else:
                C = idx[t][idx[t] >= 0] - cu_cmp[bb[t]]
            if C.size == 0:
                assert kl[t] == 0
                continue
            a = torch.tensor(0.4 * q[t] @ kc[cu_cmp[bb[t]] + C].T)
            P = torch.softmax(a, dim=1).mean(0)
            logQ = torch.log_softmax(torch.tensor(sc[t, C]), dim=0)
            ref = torch.nn.functional.kl_div(logQ, P, reduction="sum")
            assert abs(kl[t] - ref.item()) < 1e-12


def test_kl_zero_when_student_equals_teacher():
    # H = H_I = 1, w = 1, qI = scale q, kI = kv_cmp, all-positive operands: relu is the
    # identity and the indexer logits equal the teacher logits, so every KL_t is 0
    rng = np.random.default_rng(13)
    cu = _cu([24, 13])
    T, D, r, scale = 37, 5, 4, 0.7
    q = np.abs(rng.standard_normal((T, 1, D)))
    kv = np.abs(rng.standard_normal((T, D)))
    kc = O.compress(kv, cu, r)
    qI = scale * q
    w = np.ones((T, 1))
    sc = O.index_scores(qI, w, kc, cu, r, 24 // r)
    idx = O.topk_select(sc, cu, r, 2, 64, T)
    for teacher in ("selected", "dense"):
        kl, loss, dqI, dw, dkI = O.indexer_kl(q, kc, sc, idx, qI, w, kc, cu, r, scale, teacher)
        assert np.all(np.abs(kl) < 1e-13)
        assert np.abs(dqI).max() < 1e-13 and np.abs(dw).max() < 1e-13 and np.abs(dkI).max() < 1e-13


def test_kl_single_candidate_is_zero_and_dense_equals_selected_when_k_covers():
    cu, q, kc, qI, w, kI, sc, idx = _kl_case([9], k=1)
    kl, *_ = O.indexer_kl(q, kc, sc, idx, qI, w, kI, cu, 2, 0.4, "selected")
    assert np.all(np.abs(kl) < 1e-14)
    cu, q, kc, qI, w, kI, sc, idx = _kl_case([19, 8], k=64)
    a = O.indexer_kl(q, kc, sc, idx, qI, w, kI, cu, 2, 0.4, "selected")
    b = O.indexer_kl(q, kc, sc, None, qI, w, kI, cu, 2, 0.4, "dense")
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, atol=1e-14)


def test_kl_grad_closed_form_and_finite_differences():
    lens = [15, 10]
    cu, q, kc, qI, w, kI, sc, idx = _kl_case(lens, seed=17)
    r, scale, gs = 2, 0.4, 0.75
    n_cap = max(lens) // r
    for teacher in ("selected", "dense"):
        kl, loss, dqI, dw, dkI = O.indexer_kl(q, kc, sc, idx, qI, w, kI, cu, r, scale, teacher, gs)

        def total(qI_, w_, kI_):
            s_ = O.index_scores(qI_, w_, kI_, cu, r, n_cap)
            return gs * O.indexer_kl(q, kc, s_, idx, qI_, w_, kI_, cu, r, scale, teacher)[1]

        eps = 1e-6
        pick = np.random.default_rng(19)
        for arr, grad in ((qI, dqI), (w, dw), (kI, dkI)):
            flat = arr.reshape(-1)
            for pos in pick.choice(flat.size, size=10, replace=False):
                old = flat[pos]
                flat[pos] = old + eps
                fp = total(qI, w, kI)
                flat[pos] = old - eps
                fm = total(qI, w, kI)
                flat[pos] = old
                num = (fp - fm) / (2 * eps)
                assert abs(num - grad.reshape(-1)[pos]) <= 1e-6 * max(1.0, abs(num))
    # closed form of the logit gradient: dKL_t/dI[t,j] = Q_t[j] - P_t[j]; sum_j of it is 0
    # so for H_I = 1, w = 1 and positive operands dw[t] = sum_j (Q-P) z_j  = <Q-P, I>
    rng = np.random.default_rng(23)
    T = 16
    cu1 = _cu([T])
    q1 = rng.standard_normal((T, 2, 3))
    kc1 = O.compress(rng.standard_normal((T, 3)), cu1, 2)
    qI1 = np.abs(rng.standard_normal((T, 1, 3)))
    kI1 = O.compress(np.abs(rng.standard_normal((T, 3))), cu1, 2)
    s1 = O.index_scores(qI1, np.ones((T, 1)), kI1, cu1, 2, 8)
    kl, loss, dqI, dw, dkI = O.indexer_kl(q1, kc1, s1, None, qI1, np.ones((T, 1)), kI1, cu1, 2,
                                          0.5, "dense")
    for t in range(T):
        nv = (t + 1) // 2
        if nv == 0:
            continue
        a = 0.5 * q1[t] @ kc1[:nv].T
        P = (np.exp(a - logsumexp(a, axis=1, keepdims=True))).mean(0)
        Q = np.exp(s1[t, :nv] - logsumexp(s1[t, :nv]))
        assert abs(dw[t, 0] - float((Q - P) @ s1[t, :nv])) < 1e-12


def test_kl_open_relu_bound_covers_mask_flips():
    """The undecided-ReLU bound: zero when no logit is within relu_eps of zero; with every
    mask open it dominates each gradient entry; and it covers the change that flipping one
    mask actually makes (that logit nudged across zero through its key row)."""
    lens = [15, 10]
    cu, q, kc, qI, w, kI, sc, idx = _kl_case(lens, seed=29)
    r, scale, gs = 2, 0.4, 0.75
    for teacher in ("selected", "dense"):
        base = O.indexer_kl(q, kc, sc, idx, qI, w, kI, cu, r, scale, teacher, gs)
        out = O.indexer_kl(q, kc, sc, idx, qI, w, kI, cu, r, scale, teacher, gs, relu_eps=0.0)
        for x, y in zip(base[2:5], out[2:5]):
            assert np.array_equal(x, y)
        assert all(not b.any() for b in out[5])
        full = O.indexer_kl(q, kc, sc, idx, qI, w, kI, cu, r, scale, teacher, gs, relu_eps=1.0)
        for grad, bound in zip(full[2:5], full[5]):
            assert np.all(np.abs(grad) <= bound + 1e-12)
    # one logit moved to +-tiny: both signs stay within the bound of either side
    t, h = 12, 1
    bb, pp = O.token_positions(cu, int(cu[-1]))
    row = int(O.cmp_seqlens(cu, r)[bb[t]]) + 1
    qI2 = qI.copy()
    zt = qI2[t, h] @ kI[row]
    qI2[t, h] -= (zt - 1e-12) * kI[row] / (kI[row] @ kI[row])
    pos = O.indexer_kl(q, kc, sc, idx, qI2, w, kI, cu, r, scale, "dense", gs, relu_eps=1e-6)
    qI2[t, h] -= 2e-12 * kI[row] / (kI[row] @ kI[row])
    neg = O.indexer_kl(q, kc, sc, idx, qI2, w, kI, cu, r, scale, "dense", gs, relu_eps=1e-6)
    for a_, b_, bound in zip(pos[2:5], neg[2:5], pos[5]):
        assert np.any(a_ != b_)
        assert np.all(np.abs(a_ - b_) <= bound + 1e-9)


# ------------------------------------------------------------------ learned compressor
def _learned_case(lens, dim=5, r=4, seed=31):
    rng = np.random.default_rng(seed)
    cu = _cu(lens)
    T = int(cu[-1])
    return cu, rng.standard_normal((T, dim)), rng.standard_normal((T, dim)), rng


def test_learned_compressor_reduces_to_mean_pool_and_window_mean():
    """Zero scores and positional parameter: non-overlapping groups are the mean-pool
    compressor; overlapping groups are the plain mean of their 8 (group 0: 4) tokens."""
    lens = [13, 9, 4, 3]
    cu, x, _, _ = _learned_case(lens)
    T, dim, r = x.shape[0], x.shape[1], 4
    z = np.zeros((T, dim))
    got = O.compress_learned(x, z, np.zeros((r, dim)), cu, r, overlap=False)
    assert np.allclose(got, O.compress(x, cu, r), rtol=0, atol=1e-14)
    got = O.compress_learned(x, z, np.zeros((2 * r, dim)), cu, r, overlap=True)
    rows = []
    for s, L in zip(cu[:-1], np.diff(cu)):
        for j in range(L // r):
            lo = s + max(0, j - 1) * r
            rows.append(x[lo: s + (j + 1) * r].mean(axis=0))
    assert np.allclose(got, np.array(rows), rtol=0, atol=1e-14)


def test_learned_compressor_limits_and_invariances():
    lens = [12, 8]
    cu, x, s, rng = _learned_case(lens, seed=37)
    T, dim, r = x.shape[0], x.shape[1], 4
    bias = rng.standard_normal((2 * r, dim))
    base = O.compress_learned(x, s, bias, cu, r, overlap=True)
    # a per-channel constant added to every score leaves every softmax unchanged
    shift = O.compress_learned(x, s + rng.standard_normal(dim), bias, cu, r, overlap=True)
    assert np.allclose(base, shift, rtol=0, atol=1e-12)
    # one dominant token per channel: the row is that token's value
    s2 = s.copy()
    s2[9] += 200.0      # token 9: in sample 0's group 2 (own) and nowhere else
    out = O.compress_learned(x, s2, bias, cu, r, overlap=True)
    assert np.allclose(out[2], x[9], rtol=0, atol=1e-12)
    # compression restarts per sample: sample 0's tokens do not reach sample 1's rows
    x3 = x.copy()
    x3[:12] = rng.standard_normal((12, dim))
    out3 = O.compress_learned(x3, s, bias, cu, r, overlap=True)
    n0 = 12 // r
    assert np.array_equal(out3[n0:], base[n0:])
    assert not np.allclose(out3[:n0], base[:n0])


def test_learned_compressor_adjoint_finite_differences():
    lens = [11, 9]
    for overlap in (True, False):
        cu, x, s, rng = _learned_case(lens, dim=3, seed=41)
        T, dim, r = x.shape[0], x.shape[1], 4
        bias = rng.standard_normal(((2 if overlap else 1) * r, dim))
        Tc = int(O.cmp_seqlens(cu, r)[-1])
        dc = rng.standard_normal((Tc, dim))
        dx, ds, db = O.compress_learned_bwd(x, s, bias, dc, cu, r, overlap, T)

        def f(x_, s_, b_):
            return float((O.compress_learned(x_, s_, b_, cu, r, overlap) * dc).sum())

        eps = 1e-6
        for arr, grad in ((x, dx), (s, ds), (bias, db)):
            flat = arr.reshape(-1)
            for pos in range(flat.size):
                old = flat[pos]
                flat[pos] = old + eps
                fp = f(x, s, bias)
                flat[pos] = old - eps
                fm = f(x, s, bias)
                flat[pos] = old
                assert abs((fp - fm) / (2 * eps) - grad.reshape(-1)[pos]) <= 1e-7, (overlap, pos)
        # tail tokens of a sample feed no group: zero gradient there
        assert not dx[8:11].any() and not ds[8:11].any()


# ------------------------------------------------------------------------------ RoPE
def test_rope_rotation_properties():
    """Inverse is the transpose, norms of every pair are kept, position 0 is the identity,
    and dot products of the rope band depend only on the relative position (the defining
    property of a rotary embedding); the nope channels are untouched."""
    rng = np.random.default_rng(61)
    dim, rd, theta = 24, 8, 10000.0
    x = rng.standard_normal((6, dim))
    pos = np.array([0, 1, 5, 37, 1000, 131071])
    y = O.rope(x, pos, rd, theta)
    assert np.allclose(O.rope(y, pos, rd, theta, inverse=True), x, rtol=0, atol=1e-12)
    assert np.array_equal(y[:, :dim - rd], x[:, :dim - rd])
    assert np.array_equal(y[0], x[0])
    pair = lambda a: a[:, dim - rd:].reshape(len(a), rd // 2, 2)      # noqa: E731
    assert np.allclose(np.linalg.norm(pair(y), axis=2), np.linalg.norm(pair(x), axis=2))
    q, k = rng.standard_normal(dim), rng.standard_normal(dim)
    dots = []
    for m, n in ((7, 3), (104, 100), (4, 0)):
        qm = O.rope(q[None], [m], rd, theta)[0, dim - rd:]
        kn = O.rope(k[None], [n], rd, theta)[0, dim - rd:]
        dots.append(qm @ kn)
    assert np.allclose(dots, dots[0], rtol=0, atol=1e-12)
    # closed form: pair 0 (frequency 1) at position 1 turns by one radian
    z = np.zeros((1, dim))
    z[0, dim - rd], z[0, dim - rd + 1] = 2.0, 3.0
    r1 = O.rope(z, [1], rd, theta)[0, dim - rd: dim - rd + 2]
    assert np.allclose(r1, [2 * np.cos(1.0) - 3 * np.sin(1.0), 2 * np.sin(1.0) + 3 * np.cos(1.0)])
    # pair 1 turns at theta^(-2/8) = 0.1 rad per position: one radian at position 10, while
    # pair 0 has turned 10 radians there
    z[0, dim - rd + 2], z[0, dim - rd + 3] = -1.0, 0.5
    r10 = O.rope(z, [10], rd, theta)[0, dim - rd:]
    c1, s1, c10, s10 = np.cos(1.0), np.sin(1.0), np.cos(10.0), np.sin(10.0)
    assert np.allclose(r10[:4], [2 * c10 - 3 * s10, 2 * s10 + 3 * c10, -c1 - 0.5 * s1, -s1 + 0.5 * c1])
    assert np.array_equal(r10[4:], np.zeros(rd - 4))


def test_rope_positions_restart_per_sample():
    cu = _cu([5, 3, 6])
    assert list(O.rope_positions(cu, 16)) == [0, 1, 2, 3, 4, 0, 1, 2, 0, 1, 2, 3, 4, 5, -1, -1]
    assert list(O.rope_positions(cu, 6, ratio=2)) == [0, 1, 0, 0, 1, 2]   # 2 + 1 + 3 rows
    assert list(O.rope_positions(cu, 7, ratio=2)) == [0, 1, 0, 0, 1, 2, -1]


# --------------------------------------------------------------------------- fp8
def test_e4m3_golden_codes():
    for ln in _gold_lines("e4m3_codes.txt"):
        v, c = ln.split()
        assert int(O.e4m3_encode(np.array([float(v)]))[0]) == int(c, 16), v


def test_e4m3_matches_torch_cast():
    x = np.concatenate([RNG.standard_normal(20000) * s for s in (1e-3, 0.05, 1, 30, 300)])
    x = np.concatenate([x, [0.0, -0.0, 448.0, -448.0, 447.9, 1e-9]])
    ref = torch.tensor(np.clip(x, -448, 448), dtype=torch.float32).to(torch.float8_e4m3fn)
    got = O.e4m3_encode(x.astype(np.float32))
    assert np.array_equal(got, ref.view(torch.uint8).numpy())
    np.testing.assert_array_equal(O.e4m3_decode(got), ref.to(torch.float64).numpy())


def test_quantize_rows_scale_and_roundtrip():
    x = (RNG.standard_normal((50, 128)) * np.logspace(-3, 2, 50)[:, None]).astype(np.float32)
    x[7] = 0
    codes, scale = O.quantize_fp8(x)
    assert scale[7] == 1.0
    amax = np.abs(x).max(axis=1)
    nz = amax > 0
    np.testing.assert_array_equal(scale[nz], (amax[nz] / np.float32(448)).astype(np.float32))
    deq = O.dequantize_fp8(codes, scale)
    # every row's largest magnitude maps to +-448 exactly; relative error within e4m3's
    # half-ulp (2^-4) for normal codes
    assert np.all(np.abs(O.e4m3_decode(codes)).max(axis=1)[nz] == 448.0)
    big = np.abs(x) > scale[:, None] * 2 ** -6
    assert np.all(np.abs(deq - x)[big] <= np.abs(x)[big] * 2 ** -4 * 1.0001)


# --------------------------------------------------------------------------- packing
@pytest.mark.parametrize("rope_dim", [0, 4])
def test_packing_invariance_whole_layer(rope_dim):
    """A packed run equals each sample run alone (THD vs single-sequence parity); with RoPE
    this pins the per-sample restart of the token and compressed positions."""
    from synth import configs
    cfg = configs.workload("tiny_csa_f32_L256", heads=2, head_dim=8, idx_heads=2, idx_dim=4,
                           window=5, topk=3, topk_cap=64, rope_dim=rope_dim, rope_theta=50.0)
    lens = [23, 17, 9]
    rng = np.random.default_rng(29)
    cu = _cu(lens)
    T = int(cu[-1])
    inp = dict(cu_seqlens=cu, max_seqlen=max(lens),
               q=rng.standard_normal((T, 2, 8)), kv=rng.standard_normal((T, 8)),
               qI=rng.standard_normal((T, 2, 4)), kI_tok=rng.standard_normal((T, 4)),
               w=rng.standard_normal((T, 2)), dO=rng.standard_normal((T, 2, 8)))
    packed = O.layer_step(inp, cfg)
    cu_cmp = O.cmp_seqlens(cu, 4)
    for b, L in enumerate(lens):
        s = int(cu[b])
        one = {k: (v[s:s + L] if isinstance(v, np.ndarray) and v.ndim > 1 else v)
               for k, v in inp.items()}
        one["cu_seqlens"] = _cu([L])
        one["max_seqlen"] = max(lens)     # same n_cap
        alone = O.layer_step(one, cfg)
        c0, c1 = int(cu_cmp[b]), int(cu_cmp[b + 1])
        for key in ("O", "LSE", "dq", "dqI", "dw", "kl") + (("O_rot",) if rope_dim else ()):
            np.testing.assert_allclose(packed[key][s:s + L], alone[key], atol=1e-12)
        for key in ("dkv", "dkI_tok"):
            np.testing.assert_allclose(packed[key][s:s + L], alone[key], atol=1e-12)
        for key in ("kv_cmp", "dkv_cmp", "dkI_cmp"):
            np.testing.assert_allclose(packed[key][c0:c1], alone[key], atol=1e-12)
        sel_p = packed["idx"][s:s + L]
        sel_a = alone["idx"]
        np.testing.assert_array_equal(np.where(sel_p >= 0, sel_p - c0, -1), sel_a)


def _rope_layer_case(seed=31):
    from synth import configs
    cfg = configs.workload("tiny_csa_f32_L256", heads=2, head_dim=8, idx_heads=2, idx_dim=6,
                           window=4, topk=3, topk_cap=64, teacher="dense", rope_dim=4,
                           rope_theta=30.0)
    lens = [14, 11]
    rng = np.random.default_rng(seed)
    cu = _cu(lens)
    T = int(cu[-1])
    inp = dict(cu_seqlens=cu, max_seqlen=max(lens),
               q=rng.standard_normal((T, 2, 8)), kv=rng.standard_normal((T, 8)),
               qI=rng.standard_normal((T, 2, 6)), kI_tok=rng.standard_normal((T, 6)),
               w=rng.standard_normal((T, 2)), dO=rng.standard_normal((T, 2, 8)))
    return cfg, inp


def test_rope_layer_gradients_finite_differences():
    """The rotated layer's gradients are those of the unrotated inputs: dq, dkv of
    sum(O_rot * dO) and dqI, dkI_tok of the loss match central differences (a rotation used
    where its inverse belongs, or a position from the wrong coordinate system, fails)."""
    cfg, inp = _rope_layer_case()
    res = O.layer_step(inp, cfg)
    assert not np.allclose(res["O_rot"], res["O"])
    eps = 1e-6
    pick = np.random.default_rng(5)

    def objective(key):
        out = O.layer_step(inp, cfg, backward=False)
        return float((out["O_rot"] * inp["dO"]).sum()) if key in ("q", "kv") else out["loss"]

    for key, gkey in (("q", "dq"), ("kv", "dkv"), ("qI", "dqI"), ("kI_tok", "dkI_tok")):
        flat = inp[key].reshape(-1)
        D = inp[key].shape[-1]
        # mostly rope-band channels (the last 4 of each row), a few nope ones
        band = [i for i in range(flat.size) if i % D >= D - 4]
        cand = np.concatenate([pick.choice(band, 10, replace=False),
                               pick.choice(flat.size, 4, replace=False)])
        for pos in cand:
            old = flat[pos]
            flat[pos] = old + eps
            fp = objective(key)
            flat[pos] = old - eps
            fm = objective(key)
            flat[pos] = old
            num = (fp - fm) / (2 * eps)
            got = res[gkey].reshape(-1)[pos]
            assert abs(num - got) <= 1e-6 * max(1.0, abs(num)), (key, pos, num, got)


def test_compressed_logits_normalize_to_compressed_lse_and_feed_the_teacher():
    # the cached-teacher path of the loss reads these logits: their log-sum-exp is the
    # attention's compressed-only normalizer (window 0, no sink), and the head-averaged
    # softmax of them reproduces the loss the oracle forms from q and kv_cmp
    cu, q, kc, qI, w, kI, sc, idx = _kl_case([17, 12])
    r, scale = 2, 0.4
    logits = O.compressed_logits(q, kc, idx, cu, r, scale)
    kv_raw = RNG.standard_normal((q.shape[0], q.shape[2]))
    rc = np.array([t for t, l in enumerate(logits) if l.shape[1] > 0])
    _, lse0 = O.sparse_attn_fwd(q, kc, kv_raw, idx[rc], None, cu, r, 0, scale, rows=rc)
    lse0 = dict(zip(rc.tolist(), lse0))
    kl, *_ = O.indexer_kl(q, kc, sc, idx, qI, w, kI, cu, r, scale, "selected")
    cu_cmp = O.cmp_seqlens(cu, r)
    bb, _ = O.token_positions(cu, q.shape[0])
    for t, l in enumerate(logits):
        if l.shape[1] == 0:
            assert kl[t] == 0
            continue
        assert np.allclose(logsumexp(l, axis=1), lse0[t], rtol=0, atol=1e-12)
        C = idx[t][idx[t] >= 0] - cu_cmp[bb[t]]
        P = torch.softmax(torch.tensor(l), dim=1).mean(0)
        logQ = torch.log_softmax(torch.tensor(sc[t, C]), dim=0)
        ref = torch.nn.functional.kl_div(logQ, P, reduction="sum").item()
        assert abs(kl[t] - ref) < 1e-12
    # dense order: visible rows 0 .. n_vis - 1
    dl = O.compressed_logits(q, kc, None, cu, r, scale)
    rd = np.array([t for t, l in enumerate(dl) if l.shape[1] > 0])
    _, lsed = O.sparse_attn_fwd(q, kc, kv_raw, None, None, cu, r, 0, scale, rows=rd)
    for i, t in enumerate(rd):
        assert np.allclose(logsumexp(dl[t], axis=1), lsed[i], rtol=0, atol=1e-12)


# --------------------------------------------------------------------------- storage rounding
def test_round_bf16_matches_torch_cast():
    """The oracle's bf16 rounding equals torch's float32 -> bfloat16 cast (round to nearest,
    ties to even), on wide magnitudes, exact halfway cases and subnormals."""
    x = np.concatenate([RNG.standard_normal(50000) * s for s in (1e-30, 1e-3, 1, 1e4, 1e30)])
    # halfway cases: bit 15 set and the lower 15 bits clear, both parities of bit 16
    u = RNG.integers(0x00800000, 0x7F000000, 4000, dtype=np.uint32) & np.uint32(0xFFFF0000)
    half = (u | np.uint32(0x8000)).view(np.float32).astype(np.float64)
    x = np.concatenate([x, half, -half, [0.0, -0.0, 1e-40, -3e-39]])
    ref = torch.tensor(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_bf16(x)
    np.testing.assert_array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))
    s = O.store(np.array([np.inf, -np.inf, 1.0 + 2 ** -9]), "bf16")
    assert np.isposinf(s[0]) and np.isneginf(s[1]) and s[2] == 1.0   # halfway to even


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_stored_chain_rounds_only_at_storage_points(dtype):
    """The layer chain with storage rounding: its compressed rows are the rounded compressor
    output; with float32 storage every result stays within float32 rounding of the float64
    chain; with bfloat16 storage within a few bf16 steps (an error dropped elsewhere, or a
    rounding applied to a step's arithmetic rather than to what it hands on, shows up)."""
    from synth import configs
    cfg = configs.workload("tiny_csa_f32_L256", heads=2, head_dim=8, idx_heads=2, idx_dim=4,
                           window=5, topk=3, topk_cap=64, teacher="selected", dtype=dtype,
                           idx_dtype=dtype)
    lens = [23, 17]
    rng = np.random.default_rng(41)
    cu = _cu(lens)
    T = int(cu[-1])
    rnd = (lambda a: O.store(a, dtype))
    inp = dict(cu_seqlens=cu, max_seqlen=max(lens),
               q=rnd(rng.standard_normal((T, 2, 8))), kv=rnd(rng.standard_normal((T, 8))),
               qI=rnd(rng.standard_normal((T, 2, 4))), kI_tok=rnd(rng.standard_normal((T, 4))),
               w=rng.standard_normal((T, 2)).astype(np.float32).astype(np.float64),
               dO=rnd(rng.standard_normal((T, 2, 8))))
    ref = O.layer_step(inp, cfg)
    st = O.layer_step(inp, cfg, stored=True)
    np.testing.assert_array_equal(st["kv_cmp"], O.store(O.compress(inp["kv"], cu, 4), dtype))
    np.testing.assert_array_equal(st["kI_cmp"], O.store(O.compress(inp["kI_tok"], cu, 4), dtype))
    fin = np.isfinite(ref["scores"])
    np.testing.assert_array_equal(np.isfinite(st["scores"]), fin)
    assert np.array_equal(st["scores"][fin], st["scores"][fin].astype(np.float32))
    np.testing.assert_array_equal(st["idx"], ref["idx"])   # no near-ties in this draw
    rel = 2.0 ** -20 if dtype == "f32" else 2.0 ** -6
    for key in ("O", "LSE", "kl", "dq", "dkv", "dqI", "dw", "dkI_tok"):
        a, b = st[key], ref[key]
        err = np.abs(a - b).max()
        assert err <= rel * np.abs(b).max(), (key, err, np.abs(b).max())
        if dtype == "bf16" and key in ("O", "dq", "dkv"):
            assert err > 0, key          # the rounding reached this output
