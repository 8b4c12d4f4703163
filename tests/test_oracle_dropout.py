"""Pins of the oracle's dropout (CPU only).

* The Philox implementation is written once for any word size.  At 64-bit words it must
  reproduce numpy's own Philox4x64-10 bit generator exactly, which pins the round function,
  the key schedule and the round count.  The 32-bit variant that the dropout uses differs
  only in its published constants (Salmon et al., SC 2011).
* The 32-bit variant is pinned to the published known-answer vectors of Philox4x32-10 that
  ship with the authors' Random123 library (Salmon et al., SC 2011), so a wrong multiplier,
  Weyl constant, word order or round count fails; planted swaps of the constants are caught.
* Its 32-bit output is checked statistically: byte histogram, keep rate, and independence of
  heads, batches and offsets.
* The backward with dropout is the gradient of the forward with dropout (central finite
  differences; the mask does not depend on Q, K, V).
* p = 0 is exactly no dropout.  The scaled mask has mean 1, so the forward averaged over seeds
  approaches the plain one.
* Planted mistakes in a copy of the oracle are caught.
"""

import inspect
import textwrap

import numpy as np
import pytest

from oracle import attention as A

NONE, TL, BR, WIN = 0, 1, 2, 3
RNG = np.random.default_rng(97531)


@pytest.mark.parametrize("key,counter", [((1, 2), (0, 0, 0, 0)),
                                         ((0xDEADBEEF, 0x12345), (5, 7, 9, 11)),
                                         ((2**64 - 1, 2**63 + 5), (2**64 - 2, 2**64 - 1, 3, 2**40))])
def test_philox_structure_matches_numpy_philox4x64(key, counter):
    g = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(counter, dtype=np.uint64))
    for step in range(1, 4):
        raw = [int(x) for x in g.random_raw(4)]
        # numpy advances the 256-bit counter before each block
        c = counter[0] + counter[1] * 2**64 + counter[2] * 2**128 + counter[3] * 2**192 + step
        ctr = [(c >> (64 * w)) & (2**64 - 1) for w in range(4)]
        got = [int(x) for x in A.philox(ctr, key, **A.PHILOX_4X64)]
        assert got == raw


# Philox4x32-10 known answers (Random123 known-answer vectors; Salmon, Moraes, Dror, Shaw,
# "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011): counter words c0..c3, key words
# k0, k1 -> output words.
PHILOX4X32_KAT = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF), (0xFFFFFFFF, 0xFFFFFFFF),
     (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("counter,key,expect", PHILOX4X32_KAT)
def test_philox4x32_matches_published_known_answers(counter, key, expect):
    got = tuple(int(x) for x in A.philox(counter, key, **A.PHILOX_4X32))
    assert got == expect


def _kat_ok(consts):
    return all(tuple(int(x) for x in A.philox(c, k, **consts)) == e for c, k, e in PHILOX4X32_KAT)


@pytest.mark.parametrize("label,consts", [
    ("multipliers swapped", dict(A.PHILOX_4X32, M=A.PHILOX_4X32["M"][::-1])),
    ("Weyl constants swapped", dict(A.PHILOX_4X32, W=A.PHILOX_4X32["W"][::-1])),
    ("first multiplier off by one", dict(A.PHILOX_4X32, M=(A.PHILOX_4X32["M"][0] ^ 1, A.PHILOX_4X32["M"][1]))),
    ("second Weyl constant off by one", dict(A.PHILOX_4X32, W=(A.PHILOX_4X32["W"][0], A.PHILOX_4X32["W"][1] ^ 1))),
    ("nine rounds", dict(A.PHILOX_4X32, rounds=9)),
])
def test_philox_known_answers_catch_planted_constant_mistakes(label, consts):
    assert _kat_ok(A.PHILOX_4X32)
    assert not _kat_ok(consts), label


def test_philox4x32_bytes_are_uniform_and_keep_rate_matches():
    rows, cols = np.arange(512), np.arange(512)
    for p in (0.1, 0.5):
        k = A.dropout_threshold(p)
        z = A.dropout_keep(2024, 7, 1, 3, 8, rows, cols, k)
        n = z.size
        rate = k / 256.0
        assert abs(z.mean() - rate) <= 5 * np.sqrt(rate * (1 - rate) / n)
    # byte histogram of 64K outputs: chi-square with 255 degrees of freedom
    out = A.philox((np.arange(16384), np.zeros(16384, np.int64), np.zeros(16384, np.int64),
                    np.zeros(16384, np.int64)), (99, 100), **A.PHILOX_4X32)
    words = np.concatenate([np.asarray(w, dtype=np.int64) for w in out])
    bytes_ = np.concatenate([(words >> (8 * s)) & 0xFF for s in range(4)])
    hist = np.bincount(bytes_, minlength=256)
    exp = bytes_.size / 256
    chi2 = ((hist - exp) ** 2 / exp).sum()
    assert 150 < chi2 < 380  # 255 dof: mean 255, sd 22.6


def test_masks_of_heads_batches_offsets_and_seeds_differ():
    k = A.dropout_threshold(0.5)
    base = A.dropout_keep(5, 0, 0, 0, 4, np.arange(64), np.arange(64), k)
    for args in ((5, 0, 0, 1), (5, 0, 1, 0), (5, 1, 0, 0), (6, 0, 0, 0)):
        seed, off, b, h = args
        other = A.dropout_keep(seed, off, b, h, 4, np.arange(64), np.arange(64), k)
        agree = (other == base).mean()
        assert 0.4 < agree < 0.6, args
    # positions: the mask of a sub-block equals that block of the full mask
    sub = A.dropout_keep(5, 0, 0, 0, 4, np.arange(13, 40), np.arange(7, 61), k)
    assert np.array_equal(sub, base[13:40, 7:61])


def _inputs(B=1, Lq=6, Lk=7, hq=2, hkv=1, d=4):
    return (RNG.standard_normal((B, Lq, hq, d)), RNG.standard_normal((B, Lk, hkv, d)),
            RNG.standard_normal((B, Lk, hkv, d)), RNG.standard_normal((B, Lq, hq, d)))


@pytest.mark.parametrize("mask", [NONE, TL, BR])
def test_dropout_backward_matches_finite_differences(mask):
    q, k, v, do = _inputs()
    kw = dict(scale=0.7, mask_type=mask, dropout=(0.3, 11, 2))
    grads = A.backward(q, k, v, do, **kw)
    h = 1e-6
    for which, g in enumerate(grads):
        fd = np.zeros_like(g)
        arrs = [q, k, v]
        it = np.nditer(arrs[which], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            ap = [a.copy() for a in arrs]
            am = [a.copy() for a in arrs]
            ap[which][idx] += h
            am[which][idx] -= h
            lp = float((A.forward(*ap, **kw)[0] * do).sum())
            lm = float((A.forward(*am, **kw)[0] * do).sum())
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8)


def test_dropout_with_bias_gradients_match_finite_differences():
    q, k, v, do = _inputs(B=2, hq=2, hkv=2)
    bias = RNG.standard_normal((1, 2, 6, 7))
    kw = dict(scale=0.5, mask_type=TL, dropout=(0.25, 3, 9), bias=bias)
    dbias = A.backward(q, k, v, do, **kw)[3]
    h = 1e-6
    fd = np.zeros_like(bias)
    it = np.nditer(bias, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        bp, bm = bias.copy(), bias.copy()
        bp[idx] += h
        bm[idx] -= h
        kwp = dict(kw, bias=bp)
        kwm = dict(kw, bias=bm)
        fd[idx] = (float((A.forward(q, k, v, **kwp)[0] * do).sum()) -
                   float((A.forward(q, k, v, **kwm)[0] * do).sum())) / (2 * h)
    np.testing.assert_allclose(dbias, fd, rtol=1e-6, atol=1e-8)


def test_zero_probability_is_no_dropout_and_mean_is_unbiased():
    q, k, v, do = _inputs(Lq=5, Lk=9)
    ref = A.backward(q, k, v, do, scale=0.6, mask_type=TL)
    got = A.backward(q, k, v, do, scale=0.6, mask_type=TL, dropout=(0.0, 1, 1))
    for a, b in zip(got, ref):
        np.testing.assert_array_equal(a, b)
    o_ref, lse_ref = A.forward(q, k, v, scale=0.6)
    acc = np.zeros_like(o_ref)
    n = 400
    for s in range(n):
        o, lse = A.forward(q, k, v, scale=0.6, dropout=(0.5, 1000 + s, 0))
        np.testing.assert_array_equal(lse, lse_ref)  # the softmax statistics ignore dropout
        acc += o
    # mean of Z*2 is 1: the average approaches the plain forward at the Monte Carlo rate
    assert np.abs(acc / n - o_ref).max() < 6 * np.abs(o_ref).max() / np.sqrt(n) + 0.05


DROP_MUTATIONS = [
    ("dP not masked", "dp = (doh @ vb[:, g, :].T) * zf", "dp = doh @ vb[:, g, :].T"),
    ("dV from the undropped P", "dvb[:, g, :] += (p * zf).T @ doh", "dvb[:, g, :] += p.T @ doh"),
    ("dS from the dropped P", "ds = p * (dp - d[:, None])", "ds = p * zf * (dp - d[:, None])"),
]


@pytest.mark.parametrize("label,old,new", DROP_MUTATIONS, ids=[m[0] for m in DROP_MUTATIONS])
def test_pins_catch_planted_dropout_mistakes(label, old, new):
    src = textwrap.dedent(inspect.getsource(A.backward))
    assert old in src
    ns = dict(vars(A))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    q, k, v, do = _inputs()
    kw = dict(scale=0.7, mask_type=TL, dropout=(0.3, 11, 2))
    bad = ns["backward"](q, k, v, do, **kw)
    u = [RNG.standard_normal(g.shape) for g in bad]
    h = 1e-5
    worst = 0.0
    for which in range(3):
        ap = [q, k, v]
        am = [q, k, v]
        ap[which] = ap[which] + h * u[which]
        am[which] = am[which] - h * u[which]
        fd = (float((A.forward(*ap, **kw)[0] * do).sum()) - float((A.forward(*am, **kw)[0] * do).sum())) / (2 * h)
        an = float((bad[which] * u[which]).sum())
        worst = max(worst, abs(fd - an) / max(1e-3, abs(an)))
    assert worst > 1e-4, label
