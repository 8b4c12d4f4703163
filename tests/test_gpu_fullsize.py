"""Parity at the largest workloads' full sizes (the 2x32x4096 causal headline and the
16384-token ones), in the launch configuration the benchmark times, on sampled output rows that
the oracle computes one by one (dQ rows per query, dK/dV rows per key).  The other graded
workloads are compared as whole tensors in test_gpu_fullsize_whole.py.

O and LSE (the backward's inputs) are computed by the oracle forward for the K/V groups whose
rows are checked; the other heads get O = 0 and LSE = +inf (their P is exactly 0), which the
kernels treat like any other input and which cannot reach the checked heads."""

import json
import os

import numpy as np
import pytest

import oracle
from attention_backward_fmha_amd import inputs as I
from gpu_common import TOL_COS, TOL_MAX, metrics

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _sample_rows(n, rng, k=40):
    fixed = [0, 1, 31, 32, 63, 64, 65, 127, 128, 129, n // 2, n - 2, n - 1]
    rows = {r for r in fixed if 0 <= r < n}
    rows |= set(rng.integers(0, n, size=min(k, n)).tolist()) if n else set()
    return np.array(sorted(rows), np.int64)


def _check(name, got, ref):
    assert np.all(np.isfinite(got)), name
    err, mref, cos = metrics(got, ref)
    assert err <= TOL_MAX * mref, "%s: max|err| %.3g > %.3g * %.3g" % (name, err, TOL_MAX, mref)
    assert cos >= TOL_COS, "%s: cosine %.6f" % (name, cos)


def _run(w, *, lens=None, deterministic, checks):
    """checks: list of (segment, kv_head) pairs whose query heads and keys are sampled."""
    import torch
    import attention_backward_fmha_amd as F
    Hq, Hkv, dqk, dv = w["Hq"], w["Hkv"], w["d_qk"], w["d_v"]
    grp = Hq // Hkv
    mask = w["mask"]
    wl, wr = w.get("window", (-1, -1))
    scale = 1.0 / np.sqrt(dqk)
    if lens is None:
        B, Sq, Sk = w["B"], w["Sq"], w["Sk"]
        shapes = [(B, Sq, Hq, dqk), (B, Sk, Hkv, dqk), (B, Sk, Hkv, dv), (B, Sq, Hq, dv)]
        sq = sk = None
    else:
        T = int(sum(lens))
        shapes = [(T, Hq, dqk), (T, Hkv, dqk), (T, Hkv, dv), (T, Hq, dv)]
        sq = sk = I.seqstart(lens)
    x = I.draw(w["seed"], shapes, w["sigmas"])
    # forward for the checked groups only
    o = np.zeros(shapes[3][:-1] + (dv,), np.float32)
    lse = np.full((shapes[0][0], Hq, shapes[0][1]) if lens is None else (Hq, shapes[0][0]), np.inf,
                  np.float32)
    stats = {}
    for (b, g) in checks:
        hs = list(range(g * grp, (g + 1) * grp))
        if lens is None:
            qb, kb, vb = x["q"][b:b + 1][:, :, hs], x["k"][b:b + 1][:, :, [g]], x["v"][b:b + 1][:, :, [g]]
            ob, lb = oracle.forward(qb, kb, vb, scale=scale, mask_type=mask, window_left=wl, window_right=wr)
            o[b][:, hs] = ob[0]
            lse[b][hs] = lb[0]
        else:
            s0, s1 = int(sq[b]), int(sq[b + 1])
            qb, kb, vb = x["q"][None, s0:s1][:, :, hs], x["k"][None, s0:s1][:, :, [g]], x["v"][None, s0:s1][:, :, [g]]
            ob, lb = oracle.forward(qb, kb, vb, scale=scale, mask_type=mask, window_left=wl, window_right=wr)
            o[s0:s1][:, hs] = ob[0]
            lse[hs, s0:s1] = lb[0]
        # (LSE, D) per query head from the same exact forward: D = rowsum(dO * O)
        dob = x["do"][b][:, hs] if lens is None else x["do"][int(sq[b]):int(sq[b + 1])][:, hs]
        dd = oracle.rowsum_product(dob, ob[0])  # [L, len(hs)]
        stats[(b, g)] = {h: (lb[0][i], dd[:, i]) for i, h in enumerate(hs)}
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).cuda()
    kw = {}
    if lens is not None:
        kw = dict(cu_seqlens_q=torch.from_numpy(sq).cuda(), cu_seqlens_k=torch.from_numpy(sk).cuda(),
                  cu_seqlens_q_host=sq, cu_seqlens_k_host=sk)
    dq, dk, dvv = F.bwd(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(I.round_bf16(o)),
                        torch.from_numpy(lse).cuda(), dev(x["do"]), scale=scale, mask_type=mask,
                        window=(wl, wr), deterministic=deterministic, **kw)
    torch.cuda.synchronize()
    dq, dk, dvv = (t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dvv))
    rng = np.random.default_rng(77)
    for (b, g) in checks:
        seg = lambda t: t[b] if lens is None else t[int(sq[b]):int(sq[b + 1])]
        lq = seg(x["q"]).shape[0]
        lk = seg(x["k"]).shape[0]
        for h in range(g * grp, (g + 1) * grp):
            rows = _sample_rows(lq, rng)
            ref = oracle.dq_rows(x["q"], x["k"], x["v"], x["do"], scale=scale, segment=b, head=h, rows=rows,
                                 stats=stats[(b, g)][h], mask_type=mask, window_left=wl, window_right=wr,
                                 seqstart_q=sq, seqstart_k=sk)
            _check("dq[b=%d,h=%d]" % (b, h), seg(dq)[rows, h], ref)
        keys = _sample_rows(lk, rng)
        rk, rv = oracle.dkdv_rows(x["q"], x["k"], x["v"], x["do"], scale=scale, segment=b, kv_head=g,
                                  rows=keys, stats=stats[(b, g)], mask_type=mask, window_left=wl,
                                  window_right=wr, seqstart_q=sq, seqstart_k=sk)
        _check("dk[b=%d,g=%d]" % (b, g), seg(dk)[keys, g], rk)
        _check("dv[b=%d,g=%d]" % (b, g), seg(dvv)[keys, g], rv)


@pytest.mark.parametrize("deterministic", [True, False], ids=["det", "atomic"])
def test_headline_2x32x4096_causal(deterministic):
    w = I.WORKLOADS["headline_2x32x4096_causal"]
    _run(w, deterministic=deterministic, checks=[(0, 0), (1, 31)])


@pytest.mark.parametrize("name", ["long_16384_causal_br", "long_16384_window_4096"])
def test_long_16384(name):
    w = I.WORKLOADS[name]
    _run(w, deterministic=True, checks=[(0, 5)])
