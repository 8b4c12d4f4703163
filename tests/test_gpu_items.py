"""Deterministic work items of several key tiles (tiles_per_item forced to 2 and 4 through the
tune_tiles_per_item argument), in both main-kernel layouts and at d = 128 and 64: each item adds
its tiles' dQ contributions into one split, the later tiles reading back what the earlier ones
wrote (the wide layout loads that partial into LDS a step ahead).
Windows make consecutive tiles touch different query blocks, so blocks written by only some of
an item's tiles are covered."""

import numpy as np
import pytest

import attention_backward_fmha_amd as F

from gpu_common import assert_grads_close, make_inputs, oracle_backward, oracle_forward, run_gpu, seq_offsets

pytestmark = pytest.mark.gpu
NONE, TL, BR, WIN = 0, 1, 2, 3

CASES = [
    ("ragged_window", dict(lens=[700, 130, 1000]), (8, 2), WIN, (150, 0)),
    ("ragged_causal_gqa", dict(lens=[1000, 56, 613]), (8, 2), TL, (-1, -1)),
    ("batch_cross_none", dict(B=2, Sq=200, Sk=900), (4, 4), NONE, (-1, -1)),
    ("batch_window_two_sided", dict(B=1, Sq=1100, Sk=1100), (2, 1), WIN, (300, 200)),
]


KERNELS = [F.KERNEL_WIDE, F.KERNEL_FOUR_WAVE]


@pytest.mark.parametrize("dim", [128, 64])
@pytest.mark.parametrize("kernel", KERNELS, ids=["wide", "four_wave"])
@pytest.mark.parametrize("tpi", [2, 4])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_items_of_several_tiles(case, tpi, kernel, dim):
    tune = dict(tiles_per_item=tpi, kernel=kernel)
    _, shape, (hq, hkv), mask, window = case
    if "lens" in shape:
        lens = shape["lens"]
        sq = sk = seq_offsets(lens)
        x = make_inputs(7001, lens_q=lens, lens_k=lens, Hq=hq, Hkv=hkv, d_qk=dim, d_v=dim)
    else:
        sq = sk = None
        x = make_inputs(7002, B=shape["B"], Sq=shape["Sq"], Sk=shape["Sk"], Hq=hq, Hkv=hkv, d_qk=dim, d_v=dim)
    scale = 1.0 / np.sqrt(dim)
    o, lse = oracle_forward(x, scale=scale, mask=mask, window=window, sq=sq, sk=sk)
    ref = oracle_backward(x, scale=scale, mask=mask, window=window, sq=sq, sk=sk)
    got = run_gpu(x, o, lse, scale=scale, mask=mask, window=window, sq=sq, sk=sk, deterministic=True,
                  tune=tune)
    assert_grads_close(got, ref, sq, sk)


@pytest.mark.parametrize("kernel", KERNELS, ids=["wide", "four_wave"])
def test_items_of_four_tiles_are_bit_identical(kernel):
    tune = dict(tiles_per_item=4, kernel=kernel)
    lens = [700, 130, 1000]
    sq = seq_offsets(lens)
    x = make_inputs(7003, lens_q=lens, lens_k=lens, Hq=8, Hkv=2, d_qk=128, d_v=128)
    o, lse = oracle_forward(x, scale=0.088, mask=TL, sq=sq, sk=sq)
    first = run_gpu(x, o, lse, scale=0.088, mask=TL, sq=sq, sk=sq, deterministic=True, tune=tune)
    for _ in range(4):
        again = run_gpu(x, o, lse, scale=0.088, mask=TL, sq=sq, sk=sq, deterministic=True, tune=tune)
        for a, b in zip(first, again):
            assert np.array_equal(a, b)
