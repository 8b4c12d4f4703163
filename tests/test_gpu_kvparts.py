"""Key tiles whose steps (query heads x query blocks) are split over several work groups
(FMHA_BWD_KV_PARTS forces the count; the plan uses parts when there are too few K/V heads and
tiles to fill the GPU).  Each part adds fp32 dK/dV partials and a final pass sums them in
ascending part order, so deterministic mode stays bit-reproducible."""

import numpy as np
import pytest

from gpu_common import assert_grads_close, make_inputs, oracle_backward, oracle_forward, run_gpu, seq_offsets

pytestmark = pytest.mark.gpu
NONE, TL, BR, WIN = 0, 1, 2, 3

CASES = [
    ("ragged_causal_gqa", dict(lens=[300, 77, 512]), (8, 2), (128, 128), TL, (-1, -1)),
    ("batch_window_d64", dict(B=2, Sq=257, Sk=257), (4, 2), (64, 64), WIN, (40, 3)),
    ("batch3_causal_d128", dict(B=3, Sq=200, Sk=200), (2, 1), (128, 128), BR, (-1, -1)),
    ("batch_cross_d192", dict(B=1, Sq=130, Sk=333), (4, 1), (192, 128), NONE, (-1, -1)),
    ("batch_br_lq_gt_lk", dict(B=1, Sq=300, Sk=90), (2, 2), (128, 128), BR, (-1, -1)),
]


def _inputs(case, seed):
    _, shape, (hq, hkv), (dqk, dv), mask, window = case
    if "lens" in shape:
        lens = shape["lens"]
        sq = sk = seq_offsets(lens)
        x = make_inputs(seed, lens_q=lens, lens_k=lens, Hq=hq, Hkv=hkv, d_qk=dqk, d_v=dv)
    else:
        sq = sk = None
        x = make_inputs(seed, B=shape["B"], Sq=shape["Sq"], Sk=shape["Sk"], Hq=hq, Hkv=hkv, d_qk=dqk, d_v=dv)
    return x, sq, sk, 1.0 / np.sqrt(dqk), mask, window


@pytest.mark.parametrize("mode", ["det", "atomic", "atomic16"])
@pytest.mark.parametrize("parts", [1, 3, 8])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_split_key_tiles_match_oracle(case, parts, mode, monkeypatch):
    monkeypatch.setenv("FMHA_BWD_KV_PARTS", str(parts))
    x, sq, sk, scale, mask, window = _inputs(case, 9401)
    o, lse = oracle_forward(x, scale=scale, mask=mask, window=window, sq=sq, sk=sk)
    ref = oracle_backward(x, scale=scale, mask=mask, window=window, sq=sq, sk=sk)
    det, acc = {"det": (True, "fp32"), "atomic": (False, "fp32"), "atomic16": (False, "bf16")}[mode]
    got = run_gpu(x, o, lse, scale=scale, mask=mask, window=window, sq=sq, sk=sk, deterministic=det,
                  dq_acc_dtype=acc)
    assert_grads_close(got, ref, sq, sk)


@pytest.mark.parametrize("tiles", [2, 4, 8])
@pytest.mark.parametrize("parts", [3, 8])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_parts_of_multi_tile_items_match_oracle(case, parts, tiles, monkeypatch):
    """Deterministic items of several key tiles, split into parts: a part adds its dQ partial
    of a later tile onto the split blocks it wrote for an earlier one."""
    monkeypatch.setenv("FMHA_BWD_KV_PARTS", str(parts))
    monkeypatch.setenv("FMHA_BWD_TILES_PER_ITEM", str(tiles))
    x, sq, sk, scale, mask, window = _inputs(case, 9403)
    o, lse = oracle_forward(x, scale=scale, mask=mask, window=window, sq=sq, sk=sk)
    ref = oracle_backward(x, scale=scale, mask=mask, window=window, sq=sq, sk=sk)
    got = run_gpu(x, o, lse, scale=scale, mask=mask, window=window, sq=sq, sk=sk)
    assert_grads_close(got, ref, sq, sk)


@pytest.mark.parametrize("tiles", ["1", "2"])
def test_split_key_tiles_are_bit_identical(tiles, monkeypatch):
    monkeypatch.setenv("FMHA_BWD_KV_PARTS", "5")
    monkeypatch.setenv("FMHA_BWD_TILES_PER_ITEM", tiles)
    x, sq, sk, scale, mask, window = _inputs(CASES[0], 9402)
    o, lse = oracle_forward(x, scale=scale, mask=mask, sq=sq, sk=sk)
    first = run_gpu(x, o, lse, scale=scale, mask=mask, sq=sq, sk=sk)
    for _ in range(4):
        again = run_gpu(x, o, lse, scale=scale, mask=mask, sq=sq, sk=sk)
        for a, b in zip(first, again):
            assert np.array_equal(a, b)
