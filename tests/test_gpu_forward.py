"""GPU forward (fmha_fwd_run) against the oracle forward: O within the backward's tolerance per
tensor and per segment, LSE to 1e-3 absolute (natural log) with -inf exactly where a row has no
allowed key; and the device forward feeding the device backward."""

import json
import os

import numpy as np
import pytest

from attention_backward_fmha_amd import inputs as I
from gpu_common import assert_close, assert_grads_close, make_inputs, oracle_backward, oracle_forward, seq_offsets

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
NONE, TL, BR, WIN = 0, 1, 2, 3


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).cuda()


def _seqkw(sq, sk):
    import torch
    if sq is None:
        return {}
    return dict(cu_seqlens_q=torch.from_numpy(sq).cuda(), cu_seqlens_k=torch.from_numpy(sk).cuda(),
                cu_seqlens_q_host=sq, cu_seqlens_k_host=sk)


def _check_lse(got, ref, label):
    ninf = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), ninf), "%s: -inf rows differ" % label
    fin = ~ninf
    assert np.all(np.isfinite(got[fin])), label
    if fin.any():
        err = np.abs(got[fin] - ref[fin]).max()
        assert err <= 1e-3, "%s: max |lse err| %.3g" % (label, err)


def _run_fwd(x, *, scale, mask, window=(-1, -1), sq=None, sk=None):
    import torch
    import attention_backward_fmha_amd as F
    o, lse = F.fwd(_dev(x["q"]), _dev(x["k"]), _dev(x["v"]), scale=scale, mask_type=mask,
                   window=window, **_seqkw(sq, sk))
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _compare_fwd(x, *, scale, mask, window=(-1, -1), sq=None, sk=None):
    o_ref, lse_ref = oracle_forward(x, scale=scale, mask=mask, window=window, sq=sq, sk=sk)
    o, lse = _run_fwd(x, scale=scale, mask=mask, window=window, sq=sq, sk=sk)
    assert_close("o", o, o_ref)
    _check_lse(lse, lse_ref, "lse")
    if sq is not None:
        for b in range(len(sq) - 1):
            a0, a1 = int(sq[b]), int(sq[b + 1])
            if a1 > a0 and np.abs(o_ref[a0:a1]).max() > 0:
                assert_close("o[segment %d]" % b, o[a0:a1], o_ref[a0:a1])


CASES = [
    # id, batch shape or segment lengths, heads, dims, mask, window
    ("batch_causal_tl_d128", dict(B=2, Sq=300, Sk=300), (4, 4), (128, 128), TL, (-1, -1)),
    ("batch_causal_br_lq_gt_lk", dict(B=1, Sq=200, Sk=90), (2, 1), (128, 128), BR, (-1, -1)),
    ("batch_window_d64", dict(B=2, Sq=257, Sk=257), (4, 2), (64, 64), WIN, (40, 3)),
    ("batch_none_d192", dict(B=2, Sq=130, Sk=200), (2, 2), (192, 128), NONE, (-1, -1)),
    ("ragged_causal_gqa", dict(lens=[100, 80, 76, 200, 56]), (8, 2), (128, 128), TL, (-1, -1)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_forward_matches_oracle(case):
    _, shape, (hq, hkv), (dqk, dv), mask, window = case
    scale = 1.0 / np.sqrt(dqk)
    if "lens" in shape:
        lens = shape["lens"]
        sq = sk = seq_offsets(lens)
        x = make_inputs(6001, lens_q=lens, lens_k=lens, Hq=hq, Hkv=hkv, d_qk=dqk, d_v=dv)
    else:
        sq = sk = None
        x = make_inputs(6002, B=shape["B"], Sq=shape["Sq"], Sk=shape["Sk"], Hq=hq, Hkv=hkv, d_qk=dqk, d_v=dv)
    _compare_fwd(x, scale=scale, mask=mask, window=window, sq=sq, sk=sk)


def test_forward_mixed_8192_packing():
    """The mixed 8192-token packing of the Llama-3-8B-shaped GQA workload (32/8, d=128)."""
    lens = json.load(open(os.path.join(GOLDEN, "segments.json")))["mixed_8192"]
    sq = seq_offsets(lens)
    x = make_inputs(6003, lens_q=lens, lens_k=lens, Hq=32, Hkv=8, d_qk=128, d_v=128)
    _compare_fwd(x, scale=1 / np.sqrt(128), mask=TL, sq=sq, sk=sq)


def test_forward_padded_thd():
    """Padded slots: 103/77/61 tokens in 112/80/64-row slots; slot tails hold NaN."""
    import torch
    import attention_backward_fmha_amd as F
    lens = [103, 77, 61]
    sq = seq_offsets(lens)
    slots = np.array([0, 112, 192, 256], np.int32)
    x = make_inputs(6004, lens_q=lens, lens_k=lens, Hq=4, Hkv=2, d_qk=128, d_v=128)
    o_ref, lse_ref = oracle_forward(x, scale=0.088, mask=TL, sq=sq, sk=sq)
    rows = np.concatenate([np.arange(slots[b], slots[b] + n) for b, n in enumerate(lens)])

    def pad(a):
        out = np.full((256,) + a.shape[1:], np.nan, np.float32)
        out[rows] = a
        return _dev(out)

    sqd = torch.from_numpy(sq).cuda()
    o, lse = F.fwd(pad(x["q"]), pad(x["k"]), pad(x["v"]), scale=0.088, mask_type=TL,
                   cu_seqlens_q=sqd, cu_seqlens_k=sqd, cu_seqlens_q_host=sq, cu_seqlens_k_host=sq,
                   cu_seqlens_q_padded=torch.from_numpy(slots).cuda(),
                   cu_seqlens_k_padded=torch.from_numpy(slots).cuda(),
                   cu_seqlens_q_padded_host=slots, cu_seqlens_k_padded_host=slots)
    torch.cuda.synchronize()
    assert_close("o", o.float().cpu().numpy()[rows], o_ref)
    _check_lse(lse.cpu().numpy()[:, rows], lse_ref, "lse")


def test_forward_rows_without_keys():
    """Bottom-right causal with Lq > Lk and a one-sided window leave rows with no allowed key:
    LSE = -inf and O = 0 there."""
    x = make_inputs(6005, B=1, Sq=150, Sk=40, Hq=2, Hkv=2, d_qk=64, d_v=64)
    o_ref, lse_ref = oracle_forward(x, scale=0.125, mask=BR)
    assert np.isneginf(lse_ref).any()
    o, lse = _run_fwd(x, scale=0.125, mask=BR)
    _check_lse(lse, lse_ref, "lse")
    assert np.all(o[np.isneginf(lse_ref).transpose(0, 2, 1)] == 0)
    assert_close("o", o, o_ref)


@pytest.mark.parametrize("deterministic", [True, False], ids=["det", "atomic"])
def test_device_forward_then_backward(deterministic):
    """O and LSE from the device forward feed the device backward; gradients vs the oracle."""
    import torch
    import attention_backward_fmha_amd as F
    lens = [300, 77, 512]
    sq = seq_offsets(lens)
    x = make_inputs(6006, lens_q=lens, lens_k=lens, Hq=8, Hkv=2, d_qk=128, d_v=128)
    q, k, v, do = (_dev(x[n]) for n in ("q", "k", "v", "do"))
    kw = _seqkw(sq, sq)
    o, lse = F.fwd(q, k, v, scale=0.088, mask_type=TL, **kw)
    dq, dk, dv = F.bwd(q, k, v, o, lse, do, scale=0.088, mask_type=TL, deterministic=deterministic, **kw)
    torch.cuda.synchronize()
    got = tuple(t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv))
    ref = oracle_backward(x, scale=0.088, mask=TL, sq=sq, sk=sq)
    assert_grads_close(got, ref, sq, sq)
