"""Pins of the fp64 oracle to things other than itself (CPU only).

* finite differences of the forward (coordinate-wise on the smallest cases, random
  directions on the others) for every mask type, GQA and ragged batches;
* torch's own fp64 scaled-dot-product attention and autograd where it applies (no mask,
  causal top-left via ``is_causal``, causal bottom-right via ``causal_lower_right``, banded
  windows built with ``torch.tril``/``torch.triu``);
* closed forms and exact identities;
* the row-sampled forms against the full backward;
* the split reduction against torch's bfloat16 rounding and a hand-checked ordering case;
* mutation tests: mistakes planted in a copy of the oracle must be caught by the pins.
"""

import inspect
import textwrap

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from torch.nn.attention.bias import causal_lower_right

import oracle
from oracle import attention as A

NONE, TL, BR, WIN = 0, 1, 2, 3
RNG = np.random.default_rng(12345)


def _rand(*shape):
    return RNG.standard_normal(shape)


def _loss(fwd, q, k, v, do, kw):
    o, _ = fwd(q, k, v, **kw)
    return float((o * do).sum())


def _fd_coordinate(fwd, q, k, v, do, kw, h=1e-6):
    grads = []
    for which in range(3):
        arrs = [q.copy(), k.copy(), v.copy()]
        x = arrs[which]
        g = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + h
            lp = _loss(fwd, *arrs, do, kw)
            x[idx] = old - h
            lm = _loss(fwd, *arrs, do, kw)
            x[idx] = old
            g[idx] = (lp - lm) / (2 * h)
        grads.append(g)
    return grads


def _fd_directional(fwd, bwd, q, k, v, do, kw, ndir=3, h=1e-5):
    """max relative error of <grad, U> against the central difference along U."""
    dq, dk, dv = bwd(q, k, v, do, **kw)
    worst = 0.0
    for which, g in enumerate((dq, dk, dv)):
        for _ in range(ndir):
            u = RNG.standard_normal(g.shape)
            arrs = [q, k, v]
            ap = list(arrs)
            am = list(arrs)
            ap[which] = arrs[which] + h * u
            am[which] = arrs[which] - h * u
            fd = (_loss(fwd, *ap, do, kw) - _loss(fwd, *am, do, kw)) / (2 * h)
            an = float((g * u).sum())
            worst = max(worst, abs(fd - an) / max(1e-3, abs(an)))
    return worst


CASES = [
    # (name, batch?, shapes...) batch mode: (B, Lq, Lk, Hq, Hkv, dqk, dv)
    ("none", dict(B=1, Lq=5, Lk=5, Hq=2, Hkv=1, dqk=4, dv=3, mask=NONE)),
    ("tl_rect", dict(B=2, Lq=5, Lk=8, Hq=2, Hkv=2, dqk=4, dv=4, mask=TL)),
    ("br_rect", dict(B=1, Lq=8, Lk=5, Hq=4, Hkv=2, dqk=4, dv=4, mask=BR)),
    ("br_tall_empty_rows", dict(B=1, Lq=8, Lk=3, Hq=1, Hkv=1, dqk=4, dv=4, mask=BR)),
    ("win_2_1", dict(B=1, Lq=8, Lk=8, Hq=2, Hkv=1, dqk=4, dv=4, mask=WIN, wl=2, wr=1)),
    ("win_1_0_rect", dict(B=1, Lq=5, Lk=8, Hq=2, Hkv=2, dqk=8, dv=4, mask=WIN, wl=1, wr=0)),
    ("win_left_unbounded", dict(B=1, Lq=6, Lk=6, Hq=1, Hkv=1, dqk=4, dv=4, mask=WIN, wl=-1, wr=2)),
]


def _batch_inputs(c):
    q = _rand(c["B"], c["Lq"], c["Hq"], c["dqk"])
    k = _rand(c["B"], c["Lk"], c["Hkv"], c["dqk"])
    v = _rand(c["B"], c["Lk"], c["Hkv"], c["dv"])
    do = _rand(c["B"], c["Lq"], c["Hq"], c["dv"])
    kw = dict(scale=0.7, mask_type=c["mask"], window_left=c.get("wl", -1), window_right=c.get("wr", -1))
    return q, k, v, do, kw


@pytest.mark.parametrize("name,c", CASES, ids=[n for n, _ in CASES])
def test_backward_matches_directional_finite_differences(name, c):
    q, k, v, do, kw = _batch_inputs(c)
    assert _fd_directional(A.forward, A.backward, q, k, v, do, kw) < 1e-6


@pytest.mark.parametrize("mask,wl,wr", [(NONE, -1, -1), (TL, -1, -1), (BR, -1, -1), (WIN, 1, 1)])
def test_backward_matches_coordinate_finite_differences(mask, wl, wr):
    q = _rand(1, 4, 2, 3)
    k = _rand(1, 5, 1, 3)
    v = _rand(1, 5, 1, 2)
    do = _rand(1, 4, 2, 2)
    kw = dict(scale=0.9, mask_type=mask, window_left=wl, window_right=wr)
    fd = _fd_coordinate(A.forward, q, k, v, do, kw)
    an = A.backward(q, k, v, do, **kw)
    for a, b in zip(an, fd):
        np.testing.assert_allclose(a, b, rtol=1e-6, atol=1e-8)


def test_ragged_finite_differences_and_independence():
    lq = [3, 5, 1, 0, 4]
    lk = [4, 5, 2, 3, 1]
    sq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    sk = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    hq, hkv, d = 4, 2, 4
    q, k, v, do = _rand(sq[-1], hq, d), _rand(sk[-1], hkv, d), _rand(sk[-1], hkv, d), _rand(sq[-1], hq, d)
    for mask in (NONE, TL, BR):
        kw = dict(scale=0.5, mask_type=mask, seqstart_q=sq, seqstart_k=sk)
        assert _fd_directional(A.forward, A.backward, q, k, v, do, kw) < 1e-6
        dq, dk, dv = A.backward(q, k, v, do, **kw)
        o, lse = A.forward(q, k, v, **kw)
        for b in range(len(lq)):
            a0, a1, b0, b1 = sq[b], sq[b + 1], sk[b], sk[b + 1]
            # each segment alone, as a batch of one
            kwb = dict(scale=0.5, mask_type=mask)
            dq1, dk1, dv1 = A.backward(q[None, a0:a1], k[None, b0:b1], v[None, b0:b1], do[None, a0:a1], **kwb)
            o1, lse1 = A.forward(q[None, a0:a1], k[None, b0:b1], v[None, b0:b1], **kwb)
            np.testing.assert_allclose(dq[a0:a1], dq1[0], atol=1e-12)
            np.testing.assert_allclose(dk[b0:b1], dk1[0], atol=1e-12)
            np.testing.assert_allclose(dv[b0:b1], dv1[0], atol=1e-12)
            np.testing.assert_allclose(o[a0:a1], o1[0], atol=1e-12)
            np.testing.assert_array_equal(lse[:, a0:a1], lse1[0])


def _torch_ref(q, k, v, do, scale, mask=None, causal=False):
    """torch fp64 SDPA + autograd in BSHD with contiguous GQA groups."""
    group = q.shape[2] // k.shape[2]
    tq = torch.tensor(q).transpose(1, 2).contiguous().requires_grad_(True)
    tk = torch.tensor(k).transpose(1, 2).contiguous().requires_grad_(True)
    tv = torch.tensor(v).transpose(1, 2).contiguous().requires_grad_(True)
    kk = tk.repeat_interleave(group, dim=1)
    vv = tv.repeat_interleave(group, dim=1)
    o = F.scaled_dot_product_attention(tq, kk, vv, attn_mask=mask, is_causal=causal, scale=scale)
    o.backward(torch.tensor(do).transpose(1, 2))
    t = lambda x: x.detach().transpose(1, 2).numpy()
    return t(o), t(tq.grad), t(tk.grad), t(tv.grad)


@pytest.mark.parametrize("mask", [NONE, TL, BR, WIN])
def test_against_torch_sdpa_fp64(mask):
    B, Lq, Lk, hq, hkv, d = 2, 37, 53 if mask != TL else 37, 4, 2, 16
    q, k, v, do = _rand(B, Lq, hq, d), _rand(B, Lk, hkv, d), _rand(B, Lk, hkv, d), _rand(B, Lq, hq, d)
    scale = 1 / np.sqrt(d)
    wl, wr = (7, 3) if mask == WIN else (-1, -1)
    if mask == NONE:
        ref = _torch_ref(q, k, v, do, scale)
    elif mask == TL:
        ref = _torch_ref(q, k, v, do, scale, causal=True)
    elif mask == BR:
        ref = _torch_ref(q, k, v, do, scale, mask=causal_lower_right(Lq, Lk))
    else:
        # band around the bottom-right diagonal, built with the library's tril/triu
        ones = torch.ones(Lq, Lk, dtype=torch.bool)
        dlt = Lk - Lq
        band = torch.triu(ones, diagonal=dlt - wl) & torch.tril(ones, diagonal=dlt + wr)
        ref = _torch_ref(q, k, v, do, scale, mask=band)
    kw = dict(scale=scale, mask_type=mask, window_left=wl, window_right=wr)
    o, _ = A.forward(q, k, v, **kw)
    grads = A.backward(q, k, v, do, **kw)
    np.testing.assert_allclose(o, ref[0], atol=1e-12)
    for a, b in zip(grads, ref[1:]):
        np.testing.assert_allclose(a, b, atol=1e-11)


def test_lse_against_library_logsumexp():
    q, k = _rand(1, 9, 2, 8), _rand(1, 11, 2, 8)
    v = _rand(1, 11, 2, 8)
    _, lse = A.forward(q, k, v, scale=0.3, mask_type=BR)
    s = torch.tensor(np.einsum("qhd,khd->hqk", q[0], k[0]) * 0.3)
    s = s.masked_fill(~causal_lower_right(9, 11)._materialize(), float("-inf"))
    np.testing.assert_allclose(lse[0], torch.logsumexp(s, dim=-1).numpy(), atol=1e-13)


def test_probability_rows_and_dv_is_pt_do():
    """With V = identity the forward returns P itself: rows sum to one (zero for a row with
    no allowed key) and dV equals P^T dO."""
    Lq, Lk, hq = 7, 4, 2
    q, k = _rand(1, Lq, hq, 5), _rand(1, Lk, 1, 5)
    eye = np.broadcast_to(np.eye(Lk)[None, :, None, :], (1, Lk, 1, Lk)).copy()
    do = _rand(1, Lq, hq, Lk)
    for mask in (NONE, TL, BR):
        p, _ = A.forward(q, k, eye, scale=0.8, mask_type=mask)
        rows = p.sum(axis=-1)
        ok = A.allowed(mask, -1, -1, Lq, Lk).any(axis=1)
        np.testing.assert_allclose(rows[0], np.where(ok, 1.0, 0.0)[:, None].repeat(hq, 1), atol=1e-14)
        v = _rand(1, Lk, 1, 3)
        do3 = _rand(1, Lq, hq, 3)
        _, _, dv = A.backward(q, k, v, do3, scale=0.8, mask_type=mask)
        pt_do = sum(p[0, :, h, :].T @ do3[0, :, h, :] for h in range(hq))
        np.testing.assert_allclose(dv[0, :, 0, :], pt_do, atol=1e-13)


@pytest.mark.parametrize("mask", [NONE, TL, BR])
def test_identities(mask):
    B, L, hq, hkv, d = 1, 23, 4, 2, 8
    q, k, v, do = _rand(B, L, hq, d), _rand(B, L + 3, hkv, d), _rand(B, L + 3, hkv, d), _rand(B, L, hq, d)
    kw = dict(scale=0.4, mask_type=mask)
    dq, dk, dv = A.backward(q, k, v, do, **kw)
    o, _ = A.forward(q, k, v, **kw)
    g = hq // hkv
    for kh in range(hkv):
        hs = range(kh * g, (kh + 1) * g)
        # each row of dS sums to zero  =>  sum_j dK_j = 0
        np.testing.assert_allclose(dk[0, :, kh, :].sum(axis=0), 0, atol=1e-12)
        # <dQ, Q> summed over the group == <dK, K>
        lhs = sum(float((dq[0, :, h, :] * q[0, :, h, :]).sum()) for h in hs)
        np.testing.assert_allclose(lhs, float((dk[0, :, kh, :] * k[0, :, kh, :]).sum()), rtol=1e-11, atol=1e-12)
        # <dV, V> == sum of D over the group's rows
        dsum = sum(float((do[0, :, h, :] * o[0, :, h, :]).sum()) for h in hs)
        np.testing.assert_allclose(float((dv[0, :, kh, :] * v[0, :, kh, :]).sum()), dsum, rtol=1e-11)


def test_gqa_equals_sum_of_per_head_mha():
    B, L, hq, hkv, d = 2, 13, 6, 2, 4
    q, k, v, do = _rand(B, L, hq, d), _rand(B, L, hkv, d), _rand(B, L, hkv, d), _rand(B, L, hq, d)
    dq, dk, dv = A.backward(q, k, v, do, scale=0.6, mask_type=TL)
    g = hq // hkv
    kx = np.repeat(k, g, axis=2)  # expanded K/V: one copy per query head
    vx = np.repeat(v, g, axis=2)
    dq1, dk1, dv1 = A.backward(q, kx, vx, do, scale=0.6, mask_type=TL)
    np.testing.assert_allclose(dq, dq1, atol=1e-13)
    np.testing.assert_allclose(dk, dk1.reshape(B, L, hkv, g, d).sum(axis=3), atol=1e-13)
    np.testing.assert_allclose(dv, dv1.reshape(B, L, hkv, g, d).sum(axis=3), atol=1e-13)


def test_closed_forms():
    # one key: P == 1, O == V_0, dQ == dK == 0, dV == sum_i dO_i
    q, k, v, do = _rand(1, 6, 2, 4), _rand(1, 1, 1, 4), _rand(1, 1, 1, 3), _rand(1, 6, 2, 3)
    o, _ = A.forward(q, k, v, scale=1.0)
    np.testing.assert_allclose(o, np.broadcast_to(v[:, :1], o.shape), atol=1e-15)
    dq, dk, dv = A.backward(q, k, v, do, scale=1.0)
    np.testing.assert_allclose(dq, 0, atol=1e-15)
    np.testing.assert_allclose(dk, 0, atol=1e-15)
    np.testing.assert_allclose(dv[0, 0, 0], do[0].sum(axis=(0, 1)), atol=1e-13)
    # Q == 0: uniform attention over the allowed keys
    L = 7
    q0 = np.zeros((1, L, 1, 4))
    k, v, do = _rand(1, L, 1, 4), _rand(1, L, 1, 3), _rand(1, L, 1, 3)
    o, lse = A.forward(q0, k, v, scale=1.0, mask_type=TL)
    for i in range(L):
        np.testing.assert_allclose(o[0, i, 0], v[0, :i + 1, 0].mean(axis=0), atol=1e-14)
        np.testing.assert_allclose(lse[0, 0, i], np.log(i + 1), atol=1e-14)
    dq, _, dv = A.backward(q0, k, v, do, scale=1.0, mask_type=TL)
    for i in range(L):
        n = i + 1
        dots = do[0, i, 0] @ v[0, :n, 0].T
        ds = (dots - dots.mean()) / n
        np.testing.assert_allclose(dq[0, i, 0], ds @ k[0, :n, 0], atol=1e-13)
    # dV_j = sum_{i >= j} dO_i / (i + 1) under uniform causal attention
    for j in range(L):
        np.testing.assert_allclose(dv[0, j, 0], sum(do[0, i, 0] / (i + 1) for i in range(j, L)), atol=1e-13)
    # causal top-left: row 0 sees only key 0, so its dQ is zero
    q, k, v, do = _rand(1, 5, 1, 4), _rand(1, 5, 1, 4), _rand(1, 5, 1, 4), _rand(1, 5, 1, 4)
    dq, _, _ = A.backward(q, k, v, do, scale=1.0, mask_type=TL)
    np.testing.assert_allclose(dq[0, 0], 0, atol=1e-15)


def test_empty_rows_and_segments():
    # bottom-right causal with Lq > Lk leaves the first Lq-Lk rows without keys
    q, k, v, do = _rand(1, 6, 1, 4), _rand(1, 2, 1, 4), _rand(1, 2, 1, 4), _rand(1, 6, 1, 4)
    o, lse = A.forward(q, k, v, scale=1.0, mask_type=BR)
    assert np.all(np.isneginf(lse[0, 0, :4])) and np.all(np.isfinite(lse[0, 0, 4:]))
    np.testing.assert_array_equal(o[0, :4], 0)
    dq, dk, dv = A.backward(q, k, v, do, scale=1.0, mask_type=BR)
    np.testing.assert_array_equal(dq[0, :4], 0)
    assert np.all(np.isfinite(dk)) and np.all(np.isfinite(dv))
    # a segment with no keys at all: every row is empty
    lq, lk = [2, 3], [0, 4]
    sq = np.array([0, 2, 5], np.int32)
    sk = np.array([0, 0, 4], np.int32)
    q, k, v, do = _rand(5, 2, 4), _rand(4, 1, 4), _rand(4, 1, 4), _rand(5, 2, 4)
    o, lse = A.forward(q, k, v, scale=1.0, seqstart_q=sq, seqstart_k=sk)
    assert np.all(np.isneginf(lse[:, :2])) and np.all(np.isfinite(lse[:, 2:]))
    np.testing.assert_array_equal(o[:2], 0)
    dq, dk, dv = A.backward(q, k, v, do, scale=1.0, seqstart_q=sq, seqstart_k=sk)
    np.testing.assert_array_equal(dq[:2], 0)
    dq1, dk1, dv1 = A.backward(q[None, 2:], k[None], v[None], do[None, 2:], scale=1.0)
    np.testing.assert_allclose(dq[2:], dq1[0], atol=1e-14)
    np.testing.assert_allclose(dk, dk1[0], atol=1e-14)
    # a window that excludes everything beyond the diagonal key
    assert A.allowed(WIN, 0, 0, 4, 4).sum() == 4


def test_mask_reductions():
    for lq, lk in [(5, 5), (4, 9), (9, 4), (1, 7), (7, 1)]:
        none = A.allowed(NONE, -1, -1, lq, lk)
        assert none.all()
        np.testing.assert_array_equal(A.allowed(WIN, -1, -1, lq, lk), none)
        np.testing.assert_array_equal(A.allowed(WIN, lq + lk, lq + lk, lq, lk), none)
        np.testing.assert_array_equal(A.allowed(WIN, -1, 0, lq, lk), A.allowed(BR, -1, -1, lq, lk))
        np.testing.assert_array_equal(A.allowed(BR, -1, -1, lq, lk),
                                      causal_lower_right(lq, lk)._materialize().numpy())
        tl = np.tril(np.ones((lq, lk), bool))
        np.testing.assert_array_equal(A.allowed(TL, -1, -1, lq, lk), tl)
        if lq == lk:
            np.testing.assert_array_equal(A.allowed(TL, -1, -1, lq, lk), A.allowed(BR, -1, -1, lq, lk))
        # windows grow monotonically with their bounds
        for wl in range(0, 4):
            for wr in range(0, 4):
                a = A.allowed(WIN, wl, wr, lq, lk)
                assert (a <= A.allowed(WIN, wl + 1, wr, lq, lk)).all()
                assert (a <= A.allowed(WIN, wl, wr + 1, lq, lk)).all()
                # each row is one contiguous run of at most wl + wr + 1 keys
                for row in a:
                    idx = np.flatnonzero(row)
                    assert len(idx) <= wl + wr + 1
                    if len(idx):
                        assert idx[-1] - idx[0] + 1 == len(idx)


def test_row_sampled_forms_match_full_backward():
    lens = [9, 14, 4]
    sq = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    hq, hkv, d = 4, 2, 8
    q, k, v, do = _rand(sq[-1], hq, d), _rand(sq[-1], hkv, d), _rand(sq[-1], hkv, d), _rand(sq[-1], hq, d)
    for mask, wl, wr in [(TL, -1, -1), (WIN, 3, 1), (NONE, -1, -1)]:
        kw = dict(scale=0.35, mask_type=mask, window_left=wl, window_right=wr, seqstart_q=sq, seqstart_k=sq)
        dq, dk, dv = A.backward(q, k, v, do, **kw)
        o, lse = A.forward(q, k, v, **kw)
        for b in range(len(lens)):
            st = A.row_statistics(q, k, v, do, segment=b, heads=range(hq), **kw)
            for h in range(hq):
                np.testing.assert_allclose(st[h][0], lse[h, sq[b]:sq[b + 1]], atol=1e-13)
                rows = np.arange(lens[b])
                np.testing.assert_allclose(
                    A.dq_rows(q, k, v, do, segment=b, head=h, rows=rows, stats=st[h], **kw),
                    dq[sq[b]:sq[b + 1], h], atol=1e-12)
            for g in range(hkv):
                rows = np.arange(lens[b])
                dk1, dv1 = A.dkdv_rows(q, k, v, do, segment=b, kv_head=g, rows=rows, stats=st, **kw)
                np.testing.assert_allclose(dk1, dk[sq[b]:sq[b + 1], g], atol=1e-12)
                np.testing.assert_allclose(dv1, dv[sq[b]:sq[b + 1], g], atol=1e-12)


def test_split_reduce_rounding_matches_torch_bfloat16():
    rng = np.random.default_rng(7)
    parts = (rng.standard_normal((5, 3, 64)) * np.exp(rng.uniform(-20, 20, (5, 3, 64)))).astype(np.float32)
    bits = A.dq_split_reduce(parts, 0.125)
    acc = np.zeros((3, 64), np.float32)
    for s in range(5):
        acc = acc + parts[s]
    ref = torch.tensor(acc * np.float32(0.125)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)
    # ties go to even
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)], np.float32)[None]
    np.testing.assert_array_equal(A.dq_split_reduce(x, 1.0), [0x3F80, 0x3F82, 0xBF80])


def test_split_reduce_order_is_ascending():
    # (1 + 2^-24) + 2^-24 == 1 in fp32 (ties to even), while 2^-24 + 2^-24 + 1 == 1 + 2^-23
    parts = np.array([[1.0], [2.0 ** -24], [2.0 ** -24]], np.float32)
    asc = A.dq_split_reduce(parts, 1.0)
    assert asc[0] == 0x3F80
    acc = A.dq_split_reduce(parts[::-1].copy(), 2.0 ** 7)  # 128 + 2^-16 rounds to 128 in bf16 too
    assert acc[0] == 0x4300
    assert A.dq_split_reduce(np.zeros((0, 4), np.float32), 1.0).tolist() == [0, 0, 0, 0]


# ---------------------------------------------------------------------------------------
# Mutation tests: plant plausible mistakes in a copy of the oracle; the pins must notice.
# ---------------------------------------------------------------------------------------

MUTATIONS = [
    ("dropped D term", "ds = p * (dp - d[:, None])", "ds = p * dp"),
    ("wrong sign of D", "ds = p * (dp - d[:, None])", "ds = p * (dp + d[:, None])"),
    ("missing dQ scale", "dqb[r0:r1, h, :] = scale * (ds @ kb[:, g, :])", "dqb[r0:r1, h, :] = ds @ kb[:, g, :]"),
    ("dK from P", "dkb[:, g, :] += scale * (ds.T @ qh)", "dkb[:, g, :] += scale * (p.T @ qh)"),
    ("dV wrong row index", "dvb[:, g, :] += (p * zf).T @ doh", "dvb[:, g, :] += (p * zf).T @ doh[::-1]"),
    ("GQA index", "g = h // group", "g = h % kb.shape[1]"),
]


def _mutated(fn, old, new):
    src = textwrap.dedent(inspect.getsource(fn))
    assert old in src
    src = src.replace(old, new)
    ns = dict(vars(A))
    exec(compile(src, "<mutant>", "exec"), ns)
    return ns[fn.__name__]


@pytest.mark.parametrize("label,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_backward_mistakes(label, old, new):
    bad = _mutated(A.backward, old, new)
    caught = False
    c = dict(B=1, Lq=6, Lk=6, Hq=4, Hkv=2, dqk=4, dv=4, mask=TL)
    q, k, v, do, kw = _batch_inputs(c)
    if _fd_directional(A.forward, bad, q, k, v, do, kw) > 1e-4:
        caught = True
    assert caught, label


def test_pins_catch_mask_misalignment():
    bad = _mutated(A.mask_geometry, "return len_k - len_q, -1, 0", "return len_q - len_k, -1, 0")
    assert not np.array_equal(
        np.array([[bad(BR, -1, -1, 3, 5)]]), np.array([[A.mask_geometry(BR, -1, -1, 3, 5)]]))
    # the library's lower-right causal mask disagrees with the mutant
    delta, _, _ = bad(BR, -1, -1, 3, 5)
    i = np.arange(3)[:, None]
    j = np.arange(5)[None, :]
    assert not np.array_equal(j <= i + delta, causal_lower_right(3, 5)._materialize().numpy())


def test_checker_catches_the_ragged_slot_zero_bug():
    """The pages' failure: every segment after the first read the first segment's dQ slot.
    A per-segment cosine check must flag it (the pages saw cosine 0.0036)."""
    lens = [100, 80, 76]
    sq = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q, k, v, do = _rand(256, 2, 8), _rand(256, 2, 8), _rand(256, 2, 8), _rand(256, 2, 8)
    dq, _, _ = A.backward(q, k, v, do, scale=0.35, mask_type=TL, seqstart_q=sq, seqstart_k=sq)
    bad = dq.copy()
    for b in range(1, 3):
        n = lens[b]
        bad[sq[b]:sq[b] + n] = dq[0:n]
    cos = []
    for b in range(3):
        x = bad[sq[b]:sq[b + 1]].ravel()
        y = dq[sq[b]:sq[b + 1]].ravel()
        cos.append(float(x @ y / np.linalg.norm(x) / np.linalg.norm(y)))
    assert cos[0] > 0.9999 and cos[1] < 0.5 and cos[2] < 0.5


def test_rowsum_product_is_the_row_dot():
    a, b = _rand(3, 5, 7), _rand(3, 5, 7)
    np.testing.assert_allclose(A.rowsum_product(a, b), np.einsum("ijk,ijk->ij", a, b), rtol=1e-14)
    # D equals <dO, O> with O from the forward, the identity the backward relies on
    q, k, v, do = _rand(1, 6, 2, 4), _rand(1, 6, 1, 4), _rand(1, 6, 1, 4), _rand(1, 6, 2, 4)
    o, _ = A.forward(q, k, v, scale=0.5)
    _, _, dv = A.backward(q, k, v, do, scale=0.5)
    np.testing.assert_allclose((dv * v).sum(), A.rowsum_product(do, o).sum(), rtol=1e-12)
