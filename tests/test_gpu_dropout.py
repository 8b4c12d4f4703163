"""Dropout on the device (Philox4x32-10 keep mask from seed and offset, see include/fmha_bwd.h).

* The keep mask itself, bit for bit: with Q = K = 0 every probability is 1/Lk, so a one-hot V
  makes the forward's O[i, j] nonzero exactly where element (i, j) is kept, and a one-hot dO
  makes the backward's dV[j, i] nonzero exactly there; both are compared with the oracle's
  mask for several batches, heads, seeds and offsets.
* Forward and backward against the oracle with dropout, at the tolerance of the other parity
  tests: masks, GQA, head dims, ragged segments, the three dQ modes, and with a bias.
* The same seed and offset give the same bits; another offset gives another result."""

import numpy as np
import pytest

from attention_backward_fmha_amd import inputs as I
from gpu_common import assert_close, assert_grads_close, make_inputs, seq_offsets, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu
NONE, TL, BR, WIN = 0, 1, 2, 3


def _oracle_keep(p, seed, offset, b, h, hq, lq, lk):
    from oracle import attention as A
    k = A.dropout_threshold(p)
    return A.dropout_keep(seed, offset, b, h, hq, np.arange(lq), np.arange(lk), k)


@pytest.mark.parametrize("kernel", ["wide", "four_wave"])
@pytest.mark.parametrize("p,seed,offset", [(0.5, 1234, 0), (0.1, 2**40 + 17, 77), (0.9, 5, 2**31 + 3)])
def test_keep_mask_is_the_oracles_bit_for_bit(p, seed, offset, kernel):
    import torch
    import attention_backward_fmha_amd as F
    B, L, hq, d = 2, 100, 2, 128  # L <= d: one column of V (row of dO) per key (query)
    q = torch.zeros((B, L, hq, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, L, 1, d), dtype=torch.bfloat16, device="cuda")
    eye = torch.zeros((L, d), dtype=torch.bfloat16, device="cuda")
    eye[:, :L] = torch.eye(L, dtype=torch.bfloat16, device="cuda")
    v = eye[None, :, None, :].expand(B, L, 1, d).contiguous()
    kw = dict(scale=0.125, dropout_p=p, philox_seed=seed, philox_offset=offset)
    o, lse = F.fwd(q, k, v, **kw)
    do = eye[None, :, None, :].expand(B, L, hq, d).contiguous()
    tune = dict(kernel=F.KERNEL_WIDE if kernel == "wide" else F.KERNEL_FOUR_WAVE)
    _, _, dv = F.bwd(q, k, v, o, lse, do, tune=tune, **kw)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    dv = dv.float().cpu().numpy()
    for b in range(B):
        total = np.zeros((L, L), bool)
        for h in range(hq):
            ref = _oracle_keep(p, seed, offset, b, h, hq, L, L)
            got = o[b, :, h, :L] != 0
            assert np.array_equal(got, ref), (b, h)
            total |= ref
        # dV of the one K/V head sums the query heads' kept entries: nonzero where any is kept
        assert np.array_equal(dv[b, :, 0, :L].T != 0, total), b


def _run(x, o, lse, *, scale, mask, window=(-1, -1), sq=None, sk=None, deterministic=True,
         dq_acc_dtype="fp32", drop=(0.2, 42, 7), bias=None, tune=None):
    import torch
    import attention_backward_fmha_amd as F
    q, k, v, do = (to_dev_bf16(x[n]) for n in ("q", "k", "v", "do"))
    od = to_dev_bf16(I.round_bf16(o.astype(np.float32)))
    ld = to_dev_f32(lse.astype(np.float32))
    kw = {}
    if sq is not None:
        kw = dict(cu_seqlens_q=torch.from_numpy(sq).cuda(), cu_seqlens_k=torch.from_numpy(sk).cuda(),
                  cu_seqlens_q_host=sq, cu_seqlens_k_host=sk)
    if bias is not None:
        kw.update(bias=to_dev_bf16(bias), bias_grad=True)
    out = F.bwd(q, k, v, od, ld, do, scale=scale, mask_type=mask, window=window,
                deterministic=deterministic, dq_acc_dtype=dq_acc_dtype, dropout_p=drop[0],
                philox_seed=drop[1], philox_offset=drop[2], tune=tune, **kw)
    torch.cuda.synchronize()
    return tuple(t.float().cpu().numpy().astype(np.float64) for t in out)


CASES = [
    # id, shape, heads, dims, mask, window
    ("batch_causal_d128", dict(B=2, Sq=300, Sk=300), (4, 4), (128, 128), TL, (-1, -1)),
    ("batch_none_cross_d64", dict(B=1, Sq=130, Sk=333), (4, 2), (64, 64), NONE, (-1, -1)),
    ("batch_window_d192", dict(B=2, Sq=200, Sk=200), (2, 1), (192, 128), WIN, (40, 3)),
    ("ragged_causal_gqa", dict(lens=[100, 80, 76, 200, 56]), (8, 2), (128, 128), TL, (-1, -1)),
    ("ragged_br_lq_gt_lk", dict(lens_q=[150, 30], lens_k=[70, 90]), (2, 2), (128, 128), BR, (-1, -1)),
]


def _inputs(case, seed):
    _, shape, (hq, hkv), (dqk, dv), mask, window = case
    if "lens" in shape or "lens_q" in shape:
        lq = shape.get("lens_q", shape.get("lens"))
        lk = shape.get("lens_k", shape.get("lens"))
        sq, sk = seq_offsets(lq), seq_offsets(lk)
        x = make_inputs(seed, lens_q=lq, lens_k=lk, Hq=hq, Hkv=hkv, d_qk=dqk, d_v=dv)
    else:
        sq = sk = None
        x = make_inputs(seed, B=shape["B"], Sq=shape["Sq"], Sk=shape["Sk"], Hq=hq, Hkv=hkv,
                        d_qk=dqk, d_v=dv)
    return x, sq, sk, 1.0 / np.sqrt(dqk), mask, window


# d = 128 and 64 run the wide layout by default; the four-wave one is checked there as well
CASE_KERNELS = [(c, k) for c in CASES for k in (["auto", "four_wave"] if c[3][0] in (64, 128) else ["auto"])]


@pytest.mark.parametrize("mode", ["det", "atomic", "atomic16"])
@pytest.mark.parametrize("case,kernel", CASE_KERNELS, ids=["%s-%s" % (c[0], k) for c, k in CASE_KERNELS])
def test_backward_with_dropout_matches_oracle(case, kernel, mode):
    import oracle
    x, sq, sk, scale, mask, window = _inputs(case, 9101)
    drop = (0.2, 42, 7)
    kw = dict(scale=scale, mask_type=mask, window_left=window[0], window_right=window[1],
              seqstart_q=sq, seqstart_k=sk, dropout=drop)
    o, lse = oracle.forward(x["q"], x["k"], x["v"], **kw)
    ref = oracle.backward(x["q"], x["k"], x["v"], x["do"], **kw)
    det, acc = {"det": (True, "fp32"), "atomic": (False, "fp32"), "atomic16": (False, "bf16")}[mode]
    import attention_backward_fmha_amd as F
    got = _run(x, o, lse, scale=scale, mask=mask, window=window, sq=sq, sk=sk, deterministic=det,
               dq_acc_dtype=acc, drop=drop,
               tune=dict(kernel=F.KERNEL_FOUR_WAVE) if kernel == "four_wave" else None)
    assert_grads_close(got, ref, sq, sk)


WIDE_CASES = [c for c in CASES if c[3][0] in (64, 128)]


@pytest.mark.parametrize("case", WIDE_CASES, ids=[c[0] for c in WIDE_CASES])
def test_dropout_items_of_two_tiles_deterministic(case):
    """Deterministic items of two key tiles with dropout, wide layout: the second tile reads
    back the first one's dQ partial (a register load at d = 128, where the LDS slots of the
    read-back do not fit beside the dropout arrays; an LDS slot at d = 64)."""
    import oracle
    import attention_backward_fmha_amd as F
    x, sq, sk, scale, mask, window = _inputs(case, 9103)
    drop = (0.15, 7, 3)
    kw = dict(scale=scale, mask_type=mask, window_left=window[0], window_right=window[1],
              seqstart_q=sq, seqstart_k=sk, dropout=drop)
    o, lse = oracle.forward(x["q"], x["k"], x["v"], **kw)
    ref = oracle.backward(x["q"], x["k"], x["v"], x["do"], **kw)
    got = _run(x, o, lse, scale=scale, mask=mask, window=window, sq=sq, sk=sk, deterministic=True,
               dq_acc_dtype="fp32", drop=drop, tune=dict(kernel=F.KERNEL_WIDE, tiles_per_item=2))
    assert_grads_close(got, ref, sq, sk)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_forward_with_dropout_matches_oracle(case):
    import torch
    import oracle
    import attention_backward_fmha_amd as F
    x, sq, sk, scale, mask, window = _inputs(case, 9102)
    drop = (0.3, 2**33 + 9, 5)
    o_ref, lse_ref = oracle.forward(x["q"], x["k"], x["v"], scale=scale, mask_type=mask,
                                    window_left=window[0], window_right=window[1], seqstart_q=sq,
                                    seqstart_k=sk, dropout=drop)
    kw = {}
    if sq is not None:
        kw = dict(cu_seqlens_q=torch.from_numpy(sq).cuda(), cu_seqlens_k=torch.from_numpy(sk).cuda(),
                  cu_seqlens_q_host=sq, cu_seqlens_k_host=sk)
    o, lse = F.fwd(to_dev_bf16(x["q"]), to_dev_bf16(x["k"]), to_dev_bf16(x["v"]), scale=scale,
                   mask_type=mask, window=window, dropout_p=drop[0], philox_seed=drop[1],
                   philox_offset=drop[2], **kw)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy().astype(np.float64)
    assert_close("o", o, o_ref)
    if sq is not None:
        for b in range(len(sq) - 1):
            a0, a1 = int(sq[b]), int(sq[b + 1])
            if a1 > a0 and np.abs(o_ref[a0:a1]).max() > 0:
                assert_close("o[segment %d]" % b, o[a0:a1], o_ref[a0:a1])
    lse = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.abs(lse[fin] - lse_ref[fin]).max() <= 1e-3


def test_dropout_with_bias_matches_oracle():
    import oracle
    x = make_inputs(9103, B=2, Sq=257, Sk=257, Hq=4, Hkv=2, d_qk=128, d_v=128)
    rng = np.random.default_rng(9104)
    bias = I.round_bf16(rng.standard_normal((1, 4, 257, 257)).astype(np.float32))
    drop = (0.15, 99, 3)
    kw = dict(scale=1 / np.sqrt(128), mask_type=BR, bias=bias, dropout=drop)
    o, lse = oracle.forward(x["q"], x["k"], x["v"], **kw)
    ref = oracle.backward(x["q"], x["k"], x["v"], x["do"], **kw)
    got = _run(x, o, lse, scale=1 / np.sqrt(128), mask=BR, drop=drop, bias=bias)
    assert_grads_close(got[:3], ref[:3])
    assert_close("dbias", got[3], ref[3])


def test_same_seed_same_bits_other_offset_other_result():
    import oracle
    x, sq, sk, scale, mask, window = _inputs(CASES[3], 9105)
    kw = dict(scale=scale, mask_type=mask, seqstart_q=sq, seqstart_k=sk, dropout=(0.2, 42, 7))
    o, lse = oracle.forward(x["q"], x["k"], x["v"], **kw)
    a = _run(x, o, lse, scale=scale, mask=mask, sq=sq, sk=sk, drop=(0.2, 42, 7))
    b = _run(x, o, lse, scale=scale, mask=mask, sq=sq, sk=sk, drop=(0.2, 42, 7))
    c = _run(x, o, lse, scale=scale, mask=mask, sq=sq, sk=sk, drop=(0.2, 42, 8))
    for u, w in zip(a, b):
        assert np.array_equal(u, w)
    assert not np.array_equal(a[2], c[2])


def test_forward_with_bias_and_dropout_matches_oracle():
    import torch
    import oracle
    import attention_backward_fmha_amd as F
    x = make_inputs(9106, B=2, Sq=200, Sk=333, Hq=4, Hkv=2, d_qk=128, d_v=128)
    rng = np.random.default_rng(9107)
    bias = I.round_bf16(rng.standard_normal((2, 1, 200, 333)).astype(np.float32))
    drop = (0.25, 31337, 11)
    o_ref, lse_ref = oracle.forward(x["q"], x["k"], x["v"], scale=0.088, mask_type=BR, bias=bias,
                                    dropout=drop)
    o, lse = F.fwd(to_dev_bf16(x["q"]), to_dev_bf16(x["k"]), to_dev_bf16(x["v"]), scale=0.088,
                   mask_type=BR, bias=to_dev_bf16(bias), dropout_p=drop[0], philox_seed=drop[1],
                   philox_offset=drop[2])
    torch.cuda.synchronize()
    assert_close("o", o.float().cpu().numpy().astype(np.float64), o_ref)
    lse = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.abs(lse[fin] - lse_ref[fin]).max() <= 1e-3
