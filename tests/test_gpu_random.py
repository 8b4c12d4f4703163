"""Seeded random configurations against the oracle: layouts (batch, ragged, with empty and
one-token segments), every mask kind with random windows (including empty and one-key
windows), head dims, GQA ratios, the three dQ modes, bias shapes and dropout.  Each case is
small enough for the oracle; the parity bar is the usual one, per tensor and per segment,
except for a segment whose mask gives every row at most one allowed key.  There dQ and dK are
exactly 0, and the result must lie within the floor that the bf16 rounding of the O input
sets (gpu_common.single_key_floors)."""

import numpy as np
import pytest

from attention_backward_fmha_amd import inputs as I
from gpu_common import (assert_close, assert_vanishing, make_inputs, seq_offsets, single_key_floors,
                        to_dev_bf16, to_dev_f32)

pytestmark = pytest.mark.gpu
N_CASES = 40


def _case(i):
    rng = np.random.default_rng(7700 + i)
    dqk, dv = [(64, 64), (128, 128), (192, 128)][rng.integers(3)]
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2, 4]))
    mask = int(rng.integers(4))
    window = (-1, -1)
    if mask == 3:
        window = (int(rng.choice([-1, 0, 1, 7, 100])), int(rng.choice([-1, 0, 1, 33])))
    ragged = bool(rng.integers(2))
    mode = ["det", "atomic", "atomic16"][rng.integers(3)]
    if ragged:
        n = int(rng.integers(1, 5))
        lq = [int(rng.choice([0, 1, 2, 17, 63, 64, 65, 129, 200])) for _ in range(n)]
        lk = lq if rng.integers(2) else [int(rng.choice([1, 5, 64, 127, 128, 129, 250])) for _ in range(n)]
        shape = dict(lens_q=lq, lens_k=lk)
        bias = None
    else:
        B = int(rng.integers(1, 3))
        sq = int(rng.choice([1, 3, 64, 97, 130, 256]))
        sk = int(rng.choice([1, 5, 64, 100, 129, 300]))
        shape = dict(B=B, Sq=sq, Sk=sk)
        bias = None
        if rng.integers(3) == 0:
            bias = (int(rng.choice([1, B])), int(rng.choice([1, hq])))
    drop = (float(rng.choice([0.1, 0.5])), int(rng.integers(1 << 40)), int(rng.integers(1 << 20))) \
        if rng.integers(3) == 0 else None
    return dict(dqk=dqk, dv=dv, hq=hq, hkv=hkv, mask=mask, window=window, mode=mode, shape=shape,
                bias=bias, drop=drop, seed=7800 + i)


def _ids():
    out = []
    for i in range(N_CASES):
        c = _case(i)
        lay = "thd" if "lens_q" in c["shape"] else "bshd"
        out.append("%d-%s-d%d-m%d-%s%s%s" % (i, lay, c["dqk"], c["mask"], c["mode"],
                                            "-bias" if c["bias"] else "", "-drop" if c["drop"] else ""))
    return out


def _check_grads(got, ref, x, o, scale, c, sq, sk):
    """dQ, dK, dV per tensor and per segment (batch entries in batch mode); a segment with at
    most one allowed key per row is held to the bf16-O floor for dQ and dK."""
    import oracle
    group = c["hq"] // c["hkv"]
    if sq is None:
        B, Lq, Lk = x["q"].shape[0], x["q"].shape[1], x["k"].shape[1]
        segs = [((b, slice(None)), (b, slice(None))) for b in range(B)]
        lens = [(Lq, Lk)] * B
    else:
        segs = [(slice(int(sq[b]), int(sq[b + 1])), slice(int(sk[b]), int(sk[b + 1]))) for b in range(len(sq) - 1)]
        lens = [(int(sq[b + 1] - sq[b]), int(sk[b + 1] - sk[b])) for b in range(len(sq) - 1)]
    vanishing = []
    for (qs, ks), (lq, lk) in zip(segs, lens):
        ok = oracle.allowed(c["mask"], c["window"][0], c["window"][1], lq, lk)
        single = lq == 0 or lk == 0 or int(ok.sum(axis=1).max()) <= 1
        vanishing.append(single)
        xs = {"q": x["q"][qs], "k": x["k"][ks], "do": x["do"][qs]}
        if single:
            fq, fk = single_key_floors(xs, o[qs], scale, ok, group)
            assert_vanishing("dq%s" % (qs,), got[0][qs], fq)
            assert_vanishing("dk%s" % (ks,), got[1][ks], fk)
        else:
            if lq:
                assert_close("dq%s" % (qs,), got[0][qs], ref[0][qs])
            assert_close("dk%s" % (ks,), got[1][ks], ref[1][ks])
        if lk:
            assert_close("dv%s" % (ks,), got[2][ks], ref[2][ks])
    # whole tensors, over the segments that are not vanishing (those are checked above)
    keep = [i for i, v in enumerate(vanishing) if not v]
    if keep:
        for n, g, r, which in (("dq", got[0], ref[0], 0), ("dk", got[1], ref[1], 1)):
            gs = np.concatenate([g[segs[i][which]].ravel() for i in keep])
            rs = np.concatenate([r[segs[i][which]].ravel() for i in keep])
            assert_close(n, gs, rs)
    assert_close("dv", got[2], ref[2])


@pytest.mark.parametrize("i", range(N_CASES), ids=_ids())
def test_random_configuration(i):
    import torch
    import oracle
    import attention_backward_fmha_amd as F
    c = _case(i)
    sh = c["shape"]
    sq = sk = None
    if "lens_q" in sh:
        sq, sk = seq_offsets(sh["lens_q"]), seq_offsets(sh["lens_k"])
        x = make_inputs(c["seed"], lens_q=sh["lens_q"], lens_k=sh["lens_k"], Hq=c["hq"], Hkv=c["hkv"],
                        d_qk=c["dqk"], d_v=c["dv"])
    else:
        x = make_inputs(c["seed"], B=sh["B"], Sq=sh["Sq"], Sk=sh["Sk"], Hq=c["hq"], Hkv=c["hkv"],
                        d_qk=c["dqk"], d_v=c["dv"])
    bias = None
    if c["bias"]:
        rng = np.random.default_rng(c["seed"] + 1)
        bias = I.round_bf16(rng.standard_normal(c["bias"] + (sh["Sq"], sh["Sk"])).astype(np.float32))
    scale = 1.0 / np.sqrt(c["dqk"])
    okw = dict(scale=scale, mask_type=c["mask"], window_left=c["window"][0], window_right=c["window"][1],
               seqstart_q=sq, seqstart_k=sk)
    if bias is not None:
        okw["bias"] = bias
    if c["drop"]:
        okw["dropout"] = c["drop"]
    o, lse = oracle.forward(x["q"], x["k"], x["v"], **okw)
    ref = oracle.backward(x["q"], x["k"], x["v"], x["do"], **okw)

    kw = {}
    if sq is not None:
        kw = dict(cu_seqlens_q=torch.from_numpy(sq).cuda(), cu_seqlens_k=torch.from_numpy(sk).cuda(),
                  cu_seqlens_q_host=sq, cu_seqlens_k_host=sk)
    if bias is not None:
        kw["bias"] = to_dev_bf16(bias)
    if c["drop"]:
        kw.update(dropout_p=c["drop"][0], philox_seed=c["drop"][1], philox_offset=c["drop"][2])
    q, k, v, do = (to_dev_bf16(x[n]) for n in ("q", "k", "v", "do"))
    # device forward against the oracle forward
    o_dev, lse_dev = F.fwd(q, k, v, scale=scale, mask_type=c["mask"], window=c["window"], **kw)
    det, acc = {"det": (True, "fp32"), "atomic": (False, "fp32"), "atomic16": (False, "bf16")}[c["mode"]]
    out = F.bwd(q, k, v, to_dev_bf16(I.round_bf16(o.astype(np.float32))), to_dev_f32(lse.astype(np.float32)),
                do, scale=scale, mask_type=c["mask"], window=c["window"], deterministic=det,
                dq_acc_dtype=acc, bias_grad=bias is not None, **kw)
    torch.cuda.synchronize()
    got = [t.float().cpu().numpy().astype(np.float64) for t in out]
    _check_grads(got[:3], ref[:3], x, o, scale, c, sq, sk)
    if bias is not None:
        assert_close("dbias", got[3], ref[3])
    assert_close("o", o_dev.float().cpu().numpy().astype(np.float64), o)
    lse_d = lse_dev.cpu().numpy().astype(np.float64)
    fin = np.isfinite(lse)
    assert np.array_equal(np.isfinite(lse_d), fin)
    if fin.any():
        assert np.abs(lse_d[fin] - lse[fin]).max() <= 1e-3
