"""Deterministic work items of several key tiles (tiles_per_item forced to 2 and 4 through the
FMHA_BWD_TILES_PER_ITEM knob): each item adds its tiles' dQ contributions into one split, the
later tiles reading back what the earlier ones wrote.  Windows make consecutive tiles touch
different query blocks, so blocks written by only some of an item's tiles are covered."""

import numpy as np
import pytest

from gpu_common import assert_grads_close, make_inputs, oracle_backward, oracle_forward, run_gpu, seq_offsets

pytestmark = pytest.mark.gpu
NONE, TL, BR, WIN = 0, 1, 2, 3

CASES = [
    ("ragged_window", dict(lens=[700, 130, 1000]), (8, 2), WIN, (150, 0)),
    ("ragged_causal_gqa", dict(lens=[1000, 56, 613]), (8, 2), TL, (-1, -1)),
    ("batch_cross_none", dict(B=2, Sq=200, Sk=900), (4, 4), NONE, (-1, -1)),
    ("batch_window_two_sided", dict(B=1, Sq=1100, Sk=1100), (2, 1), WIN, (300, 200)),
]


@pytest.mark.parametrize("tpi", [2, 4])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_items_of_several_tiles(case, tpi, monkeypatch):
    monkeypatch.setenv("FMHA_BWD_TILES_PER_ITEM", str(tpi))
    _, shape, (hq, hkv), mask, window = case
    if "lens" in shape:
        lens = shape["lens"]
        sq = sk = seq_offsets(lens)
        x = make_inputs(7001, lens_q=lens, lens_k=lens, Hq=hq, Hkv=hkv, d_qk=128, d_v=128)
    else:
        sq = sk = None
        x = make_inputs(7002, B=shape["B"], Sq=shape["Sq"], Sk=shape["Sk"], Hq=hq, Hkv=hkv, d_qk=128, d_v=128)
    o, lse = oracle_forward(x, scale=0.088, mask=mask, window=window, sq=sq, sk=sk)
    ref = oracle_backward(x, scale=0.088, mask=mask, window=window, sq=sq, sk=sk)
    got = run_gpu(x, o, lse, scale=0.088, mask=mask, window=window, sq=sq, sk=sk, deterministic=True)
    assert_grads_close(got, ref, sq, sk)


def test_items_of_four_tiles_are_bit_identical(monkeypatch):
    monkeypatch.setenv("FMHA_BWD_TILES_PER_ITEM", "4")
    lens = [700, 130, 1000]
    sq = seq_offsets(lens)
    x = make_inputs(7003, lens_q=lens, lens_k=lens, Hq=8, Hkv=2, d_qk=128, d_v=128)
    o, lse = oracle_forward(x, scale=0.088, mask=TL, sq=sq, sk=sq)
    first = run_gpu(x, o, lse, scale=0.088, mask=TL, sq=sq, sk=sq, deterministic=True)
    for _ in range(4):
        again = run_gpu(x, o, lse, scale=0.088, mask=TL, sq=sq, sk=sq, deterministic=True)
        for a, b in zip(first, again):
            assert np.array_equal(a, b)
