"""Pins of the oracle's additive bias and its gradient dbias (CPU only).

* central finite differences of the forward with respect to every bias entry, for the four
  bias shapes (1|B, 1|Hq, Sq, Sk), every mask type and GQA;
* torch's fp64 scaled-dot-product attention with the bias as a float ``attn_mask`` and
  autograd (which sums the gradient over broadcast dimensions by itself);
* identities: every row of dbias sums to 0; a bias that is constant along each row changes
  nothing; a broadcast bias's gradient is the sum of the full-shape gradients; a bias of
  -1e30 above the diagonal reproduces the causal mask, with dbias = 0 there;
* planted mistakes in a copy of the oracle are caught.
"""

import inspect
import textwrap

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention as A

NONE, TL, BR, WIN = 0, 1, 2, 3
RNG = np.random.default_rng(2468)
SHAPES = [(1, 1), (1, 4), (2, 1), (2, 4)]  # (bias_b, bias_h) with B = 2, Hq = 4: 11SS 1HSS B1SS BHSS


def _inputs(B=2, Lq=5, Lk=6, hq=4, hkv=2, d=4, bshape=(2, 4)):
    q = RNG.standard_normal((B, Lq, hq, d))
    k = RNG.standard_normal((B, Lk, hkv, d))
    v = RNG.standard_normal((B, Lk, hkv, d))
    do = RNG.standard_normal((B, Lq, hq, d))
    bias = RNG.standard_normal(bshape + (Lq, Lk))
    return q, k, v, do, bias


def _loss(q, k, v, do, bias, kw):
    o, _ = A.forward(q, k, v, bias=bias, **kw)
    return float((o * do).sum())


@pytest.mark.parametrize("bshape", SHAPES, ids=["11SS", "1HSS", "B1SS", "BHSS"])
@pytest.mark.parametrize("mask,wl,wr", [(NONE, -1, -1), (TL, -1, -1), (BR, -1, -1), (WIN, 1, 0)])
def test_dbias_matches_coordinate_finite_differences(bshape, mask, wl, wr):
    q, k, v, do, bias = _inputs(bshape=bshape)
    kw = dict(scale=0.6, mask_type=mask, window_left=wl, window_right=wr)
    *_, dbias = A.backward(q, k, v, do, bias=bias, **kw)
    h = 1e-6
    fd = np.zeros_like(bias)
    it = np.nditer(bias, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        bp = bias.copy()
        bm = bias.copy()
        bp[idx] += h
        bm[idx] -= h
        fd[idx] = (_loss(q, k, v, do, bp, kw) - _loss(q, k, v, do, bm, kw)) / (2 * h)
    np.testing.assert_allclose(dbias, fd, rtol=1e-6, atol=1e-8)


def test_qkv_gradients_with_bias_match_directional_finite_differences():
    q, k, v, do, bias = _inputs(bshape=(1, 4))
    kw = dict(scale=0.6, mask_type=BR)
    grads = A.backward(q, k, v, do, bias=bias, **kw)[:3]
    h = 1e-5
    for which, g in enumerate(grads):
        for _ in range(3):
            u = RNG.standard_normal(g.shape)
            ap = [q, k, v]
            am = [q, k, v]
            ap[which] = ap[which] + h * u
            am[which] = am[which] - h * u
            fd = (_loss(*ap, do, bias, kw) - _loss(*am, do, bias, kw)) / (2 * h)
            an = float((g * u).sum())
            assert abs(fd - an) <= 1e-6 * max(1e-3, abs(an))


def _torch_ref(q, k, v, do, bias, scale, allowed=None):
    group = q.shape[2] // k.shape[2]
    tq = torch.tensor(q).transpose(1, 2).contiguous().requires_grad_(True)
    tk = torch.tensor(k).transpose(1, 2).contiguous().requires_grad_(True)
    tv = torch.tensor(v).transpose(1, 2).contiguous().requires_grad_(True)
    tb = torch.tensor(bias).requires_grad_(True)
    m = tb
    if allowed is not None:
        m = tb + torch.where(torch.tensor(allowed), 0.0, -torch.inf).to(torch.float64)
    o = F.scaled_dot_product_attention(tq, tk.repeat_interleave(group, 1), tv.repeat_interleave(group, 1),
                                       attn_mask=m, scale=scale)
    o.backward(torch.tensor(do).transpose(1, 2))
    t = lambda x: x.detach().transpose(1, 2).numpy()
    return t(o), t(tq.grad), t(tk.grad), t(tv.grad), tb.grad.numpy()


@pytest.mark.parametrize("bshape", [(1, 1), (1, 8), (3, 1), (3, 8)], ids=["11SS", "1HSS", "B1SS", "BHSS"])
@pytest.mark.parametrize("mask", [NONE, TL, WIN])
def test_against_torch_sdpa_with_float_mask(bshape, mask):
    q, k, v, do, bias = _inputs(B=3, Lq=29, Lk=41, hq=8, hkv=2, d=16, bshape=bshape)
    wl, wr = (9, 2) if mask == WIN else (-1, -1)
    ok = A.allowed(mask, wl, wr, 29, 41)
    scale = 0.25
    ref = _torch_ref(q, k, v, do, bias, scale, None if mask == NONE else ok)
    kw = dict(scale=scale, mask_type=mask, window_left=wl, window_right=wr)
    o, _ = A.forward(q, k, v, bias=bias, **kw)
    got = A.backward(q, k, v, do, bias=bias, **kw)
    np.testing.assert_allclose(o, ref[0], atol=1e-12)
    for a, b in zip(got, ref[1:]):
        np.testing.assert_allclose(a, b, atol=1e-11)


def test_bias_identities():
    q, k, v, do, bias = _inputs(bshape=(2, 4))
    kw = dict(scale=0.6, mask_type=TL)
    dq, dk, dv, dbias = A.backward(q, k, v, do, bias=bias, **kw)
    # each row of dS sums to zero (P rows sum to 1, D = sum P dP)
    np.testing.assert_allclose(dbias.sum(axis=-1), 0.0, atol=1e-12)
    # softmax is shift invariant: a bias constant along each row changes nothing
    c = RNG.standard_normal((2, 4, 5, 1)) * np.ones((1, 1, 1, 6))
    ref = A.backward(q, k, v, do, **kw)
    got = A.backward(q, k, v, do, bias=c, **kw)
    for a, b in zip(got[:3], ref):
        np.testing.assert_allclose(a, b, atol=1e-12)
    # a broadcast bias's gradient is the full-shape gradient summed over the broadcast axes
    b11 = RNG.standard_normal((1, 1, 5, 6))
    full = A.backward(q, k, v, do, bias=np.broadcast_to(b11, (2, 4, 5, 6)).copy(), **kw)[3]
    np.testing.assert_allclose(A.backward(q, k, v, do, bias=b11, **kw)[3], full.sum(axis=(0, 1), keepdims=True),
                               atol=1e-12)


def test_large_negative_bias_is_the_causal_mask():
    q, k, v, do, _ = _inputs(Lq=5, Lk=7)
    ok = A.allowed(BR, -1, -1, 5, 7)
    bias = np.where(ok, 0.0, -1e30)[None, None]
    got = A.backward(q, k, v, do, bias=bias, scale=0.6, mask_type=NONE)
    ref = A.backward(q, k, v, do, scale=0.6, mask_type=BR)
    for a, b in zip(got[:3], ref):
        np.testing.assert_allclose(a, b, atol=1e-12)
    assert np.all(got[3][:, :, ~ok] == 0)
    o1, lse1 = A.forward(q, k, v, bias=bias, scale=0.6, mask_type=NONE)
    o2, lse2 = A.forward(q, k, v, scale=0.6, mask_type=BR)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(lse1, lse2, atol=1e-12)


BIAS_MUTATIONS = [
    ("dbias from P", "_bias_plane(dbias, b, h)[r0:r1] += ds", "_bias_plane(dbias, b, h)[r0:r1] += p"),
    ("bias scaled with the logits", "s = s + _bias_plane(bias, b, h)[r0:r1]",
     "s = s + scale * _bias_plane(bias, b, h)[r0:r1]"),
    ("bias head index", "return bias[b if bias.shape[0] > 1 else 0, h if bias.shape[1] > 1 else 0]",
     "return bias[b if bias.shape[0] > 1 else 0, 0]"),
]


@pytest.mark.parametrize("label,old,new", BIAS_MUTATIONS, ids=[m[0] for m in BIAS_MUTATIONS])
def test_pins_catch_planted_bias_mistakes(label, old, new):
    ns = dict(vars(A))
    for fn in (A._bias_plane, A.forward, A.backward):
        src = textwrap.dedent(inspect.getsource(fn))
        exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    q, k, v, do, bias = _inputs(B=2, Lq=9, Lk=11, hq=4, hkv=2, d=8, bshape=(2, 4))
    ref = _torch_ref(q, k, v, do, bias, 0.3)
    o, _ = ns["forward"](q, k, v, bias=bias, scale=0.3)
    got = ns["backward"](q, k, v, do, bias=bias, scale=0.3)
    close = np.allclose(o, ref[0], atol=1e-9) and all(
        np.allclose(a, b, atol=1e-9) for a, b in zip(got, ref[1:]))
    assert not close, label
