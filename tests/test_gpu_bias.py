"""Additive bias (batch mode; shapes 1|B x 1|Hq x Sq x Sk) on the device: forward (O, LSE) and
backward (dQ, dK, dV and dbias = the full-shape dS summed over the broadcast dimensions)
against the oracle, at the tolerance of the other parity tests; dbias is bit-identical from run
to run in every dQ mode (plain stores, then a fixed-order sum)."""

import numpy as np
import pytest

from attention_backward_fmha_amd import inputs as I
from gpu_common import assert_close, assert_grads_close, make_inputs, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu
NONE, TL, BR, WIN = 0, 1, 2, 3


def _bias(seed, shape, sigma=1.0):
    rng = np.random.default_rng(seed)
    return I.round_bf16((rng.standard_normal(shape) * sigma).astype(np.float32))


def _oracle(x, bias, **kw):
    import oracle
    o, lse = oracle.forward(x["q"], x["k"], x["v"], bias=bias, **kw)
    grads = oracle.backward(x["q"], x["k"], x["v"], x["do"], bias=bias, **kw)
    return o, lse, grads


def _run(x, o, lse, bias, *, scale, mask, window, deterministic=True, dq_acc_dtype="fp32", tune=None):
    import torch
    import attention_backward_fmha_amd as F
    q, k, v, do = (to_dev_bf16(x[n]) for n in ("q", "k", "v", "do"))
    od = to_dev_bf16(I.round_bf16(o.astype(np.float32)))
    ld = to_dev_f32(lse.astype(np.float32))
    bd = to_dev_bf16(bias)
    out = F.bwd(q, k, v, od, ld, do, scale=scale, mask_type=mask, window=window,
                deterministic=deterministic, dq_acc_dtype=dq_acc_dtype, bias=bd, bias_grad=True,
                tune=tune)
    torch.cuda.synchronize()
    return tuple(t.float().cpu().numpy().astype(np.float64) for t in out)


CASES = [
    # id, (B, Sq, Sk), (Hq, Hkv), (d_qk, d_v), bias (b, h), mask, window
    ("bhss_causal_d128", (2, 300, 300), (4, 4), (128, 128), (2, 4), TL, (-1, -1)),
    ("11ss_causal_gqa", (2, 257, 257), (8, 2), (128, 128), (1, 1), BR, (-1, -1)),
    ("1hss_none_cross_d64", (2, 130, 333), (4, 2), (64, 64), (1, 4), NONE, (-1, -1)),
    ("b1ss_window_d192", (3, 200, 200), (2, 1), (192, 128), (3, 1), WIN, (40, 3)),
    ("bhss_br_lq_gt_lk", (1, 150, 70), (2, 2), (128, 128), (1, 2), BR, (-1, -1)),
    # Sk a multiple of 8 with aligned rows: the main kernel stages the bias in 16-byte chunks
    ("bhss_causal_d128_sk8", (2, 200, 264), (4, 4), (128, 128), (2, 4), TL, (-1, -1)),
    ("11ss_br_gqa_sk8", (2, 256, 256), (8, 2), (128, 128), (1, 1), BR, (-1, -1)),
    ("1hss_none_d64_sk8", (2, 130, 320), (4, 2), (64, 64), (1, 4), NONE, (-1, -1)),
    ("b1ss_window_d128_sk8", (3, 150, 200), (2, 1), (128, 128), (3, 1), WIN, (40, 3)),
]


def _case_inputs(case, seed):
    _, (B, Sq, Sk), (hq, hkv), (dqk, dv), (bb, bh), mask, window = case
    x = make_inputs(seed, B=B, Sq=Sq, Sk=Sk, Hq=hq, Hkv=hkv, d_qk=dqk, d_v=dv)
    bias = _bias(seed + 1, (bb, bh, Sq, Sk))
    return x, bias, 1.0 / np.sqrt(dqk), mask, window


@pytest.mark.parametrize("mode", ["det", "atomic", "atomic16"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_with_bias_matches_oracle(case, mode):
    x, bias, scale, mask, window = _case_inputs(case, 9001)
    kw = dict(scale=scale, mask_type=mask, window_left=window[0], window_right=window[1])
    o, lse, ref = _oracle(x, bias, **kw)
    det, acc = {"det": (True, "fp32"), "atomic": (False, "fp32"), "atomic16": (False, "bf16")}[mode]
    got = _run(x, o, lse, bias, scale=scale, mask=mask, window=window, deterministic=det,
               dq_acc_dtype=acc)
    assert_grads_close(got[:3], ref[:3])
    assert_close("dbias", got[3], ref[3])
    for bb in range(bias.shape[0]):
        for hh in range(bias.shape[1]):
            if np.abs(ref[3][bb, hh]).max() > 0:
                assert_close("dbias[%d,%d]" % (bb, hh), got[3][bb, hh], ref[3][bb, hh])


@pytest.mark.parametrize("tile_m", [32, 64])
def test_staged_bias_at_both_block_heights(tile_m):
    """d_qk = 128 with 16-byte aligned bias rows and Sk % 8 == 0: the main kernel stages the
    bias through LDS at 32-row blocks and at the 64-row blocks the plan takes for it."""
    x, bias, scale, mask, window = _case_inputs(("bhss_sk8", (2, 200, 264), (4, 2), (128, 128), (2, 4), TL,
                                                 (-1, -1)), 9005)
    kw = dict(scale=scale, mask_type=mask, window_left=window[0], window_right=window[1])
    o, lse, ref = _oracle(x, bias, **kw)
    got = _run(x, o, lse, bias, scale=scale, mask=mask, window=window, tune={"tile_m": tile_m})
    assert_grads_close(got[:3], ref[:3])
    assert_close("dbias", got[3], ref[3])


def test_dbias_is_bit_identical_across_runs_and_modes():
    x, bias, scale, mask, window = _case_inputs(CASES[1], 9002)
    kw = dict(scale=scale, mask_type=mask, window_left=window[0], window_right=window[1])
    import oracle
    o, lse = oracle.forward(x["q"], x["k"], x["v"], bias=bias, **kw)
    first = _run(x, o, lse, bias, scale=scale, mask=mask, window=window)
    for det, acc in ((True, "fp32"), (True, "fp32"), (False, "fp32"), (False, "bf16")):
        again = _run(x, o, lse, bias, scale=scale, mask=mask, window=window, deterministic=det,
                     dq_acc_dtype=acc)
        assert np.array_equal(first[3], again[3])
        assert np.array_equal(first[1], again[1]) and np.array_equal(first[2], again[2])


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_forward_with_bias_matches_oracle(case):
    import torch
    import attention_backward_fmha_amd as F
    x, bias, scale, mask, window = _case_inputs(case, 9003)
    import oracle
    o_ref, lse_ref = oracle.forward(x["q"], x["k"], x["v"], bias=bias, scale=scale, mask_type=mask,
                                    window_left=window[0], window_right=window[1])
    o, lse = F.fwd(to_dev_bf16(x["q"]), to_dev_bf16(x["k"]), to_dev_bf16(x["v"]), scale=scale,
                   mask_type=mask, window=window, bias=to_dev_bf16(bias))
    torch.cuda.synchronize()
    assert_close("o", o.float().cpu().numpy().astype(np.float64), o_ref)
    lse = lse.cpu().numpy().astype(np.float64)
    ninf = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), ninf)
    if (~ninf).any():
        assert np.abs(lse[~ninf] - lse_ref[~ninf]).max() <= 1e-3


def test_device_forward_then_backward_with_bias():
    """O and LSE from the device forward (with the bias) feed the device backward."""
    import torch
    import attention_backward_fmha_amd as F
    x, bias, scale, mask, window = _case_inputs(CASES[0], 9004)
    q, k, v, do = (to_dev_bf16(x[n]) for n in ("q", "k", "v", "do"))
    bd = to_dev_bf16(bias)
    o, lse = F.fwd(q, k, v, scale=scale, mask_type=mask, bias=bd)
    out = F.bwd(q, k, v, o, lse, do, scale=scale, mask_type=mask, bias=bd, bias_grad=True)
    torch.cuda.synchronize()
    got = tuple(t.float().cpu().numpy().astype(np.float64) for t in out)
    _, _, ref = _oracle(x, bias, scale=scale, mask_type=mask)
    assert_grads_close(got[:3], ref[:3])
    assert_close("dbias", got[3], ref[3])
